"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Every head of the layer runs on the GPU and every head is checked against the oracle for
the reassign (assignments, sizes, counts, centroids, mean values, all keys). The forward of
every head is then teacher-forced with the oracle's refreshed cache, and the oracle checks
heads 0 and H-1 in full and 8 seeded query blocks (always the first and the ragged last) in
every other head. The oracle runs in CPU worker processes that regenerate each head from the
seeded generator. Nothing the GPU produced is fed to the oracle.
"""
import numpy as np
import pytest

import oracle as O
from datagen import get_config, make_layer
from parity_util import (OraclePool, check_forward, check_reassign_head, from_dev, rows_of,
                         say, store64, to_dev, torch_mod)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def lib():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_video_da_amd as S
    return S


@pytest.fixture(scope="module")
def pool():
    p = OraclePool()
    yield p
    p.close()


def _sample_qblocks(cfg, n, seed):
    rng = np.random.default_rng(seed)
    nb = cfg.num_blocks
    mid = [int(x) for x in rng.choice(np.arange(1, nb - 1), size=n - 2, replace=False)]
    return sorted({0, nb - 1, *mid})


def _step(lib, plan, cfg, L, mu0_stored, drift_steps, pool, qblocks, what, variance=False):
    """GPU reassign + forward on all heads against the oracle (all heads for the reassign;
    heads 0 and H-1 in full plus `qblocks` of every other head for the forward). Returns
    the oracle's refreshed caches (stored), the next step's cache."""
    torch = torch_mod()
    dt, H, N, B, C = cfg.dtype, cfg.heads, cfg.seq_len, cfg.block, cfg.clusters
    nb = cfg.num_blocks
    mask_h = (lambda h: L["mask"][0] if L["mask"].shape[0] == 1 else L["mask"][h])
    say(f"[case] {what}: H={H} N={N} C={C} S={cfg.kblock}")
    dev = {x: to_dev(L[x], dt) for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(mu0_stored, dt), variance=variance)
    torch.cuda.synchronize()
    refs = pool.reassign([(cfg, h, drift_steps, mu0_stored[h], mask_h(h)) for h in range(H)])
    got = {"assign": out["assign"].cpu().numpy(), "sizes": out["sizes"].cpu().numpy(),
           "counts": out["counts"].cpu().numpy()}
    moves = 0
    for h in range(H):
        g = {k: v[h] for k, v in got.items()}
        g["centroids"] = from_dev(out["centroids"][h], dt)
        g["mean_values"] = from_dev(out["mean_values"][h], dt)
        if variance:
            g["variance"] = out["variance"][h].cpu().numpy()
        r = check_reassign_head(O.to_f64(L["K"][h], dt), None, O.to_f64(mu0_stored[h], dt),
                                mask_h(h), B, dt, g, f"{what} head {h}", kblock=cfg.kblock,
                                ref=refs[h])
        moves += r["band_moves"]
    say(f"  reassign ok on all {H} heads ({moves} in-band moves)")
    # forward: every head teacher-forced with the oracle's refreshed cache
    mu1 = np.stack([store64(refs[h]["mu1"], dt) for h in range(H)])
    vb = np.stack([store64(refs[h]["vbar"], dt) for h in range(H)])
    cnt = np.stack([refs[h]["counts"].astype(np.int32) for h in range(H)])
    kv32 = np.stack([refs[h]["kvar"].astype(np.float32) for h in range(H)])
    o = plan.forward(dev["Q"], dev["K"], dev["V"], to_dev(mu1, dt), to_dev(vb, dt),
                     torch.from_numpy(cnt).cuda(),
                     variance=torch.from_numpy(kv32).cuda() if variance else None)
    torch.cuda.synchronize()
    full = {0, H - 1}
    tasks = []
    for h in range(H):
        if h in full:
            chunks = [list(range(s, min(nb, s + 128))) for s in range(0, nb, 128)]
        else:
            chunks = [qblocks]
        for qb in chunks:
            tasks.append((cfg, h, drift_steps, refs[h]["mu1"], refs[h]["vbar"], refs[h]["counts"],
                          mask_h(h), qb) + ((kv32[h].astype(np.float64),) if variance else ()))
    want = pool.forward(tasks)
    got_rows = []
    for t in tasks:
        rows = torch.from_numpy(rows_of(t[7], B, N)).cuda()
        got_rows.append(from_dev(o[t[1]][rows], dt))
    check_forward(np.concatenate(got_rows), np.concatenate(want), dt,
                  f"{what} forward ({len(full)} full heads + {len(qblocks)} blocks of {H - 2})")
    return mu1


@pytest.mark.parametrize("name", ["wan14b_bf16", "hunyuan13b_bf16", "hunyuan13b_budget_bf16",
                                  "hunyuan13b_sub32_bf16"])
def test_full_layer(lib, pool, name):
    cfg = get_config(name)
    L = make_layer(cfg, threads=16)
    plan = lib.Plan(cfg.heads, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters, L["mask"],
                    dtype=cfg.dtype, key_block=cfg.kblock)
    _step(lib, plan, cfg, L, L["cache_init"], 0, pool, _sample_qblocks(cfg, 8, 12), name)
    plan.close()


def test_full_layer_variance(lib, pool):
    """The 13B-class layer through da_reassign_var / da_forward_var."""
    cfg = get_config("hunyuan13b_bf16")
    L = make_layer(cfg, threads=16)
    plan = lib.Plan(cfg.heads, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters, L["mask"],
                    dtype=cfg.dtype)
    _step(lib, plan, cfg, L, L["cache_init"], 0, pool, _sample_qblocks(cfg, 8, 13),
          "hunyuan13b_bf16 var", variance=True)
    plan.close()


def test_long_sequence_layer(lib):
    """One head of about a million tokens (8055 query blocks, a ragged last block of 56): the
    plan's lists, the counting sort and the forward's grid at that length. The oracle assigns
    and refreshes every key, and takes the counts of 16 sampled query blocks (always the first
    and the ragged last) by the direct count; the GPU forward is then teacher-forced with the
    oracle's cache and those count rows (zeros elsewhere) and checked on the sampled blocks."""
    torch = torch_mod()
    cfg = get_config("long_video_bf16")
    dt, N, d, B, C = cfg.dtype, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters
    nb = cfg.num_blocks
    L = make_layer(cfg, threads=16)
    mask = L["mask"][0]
    say(f"[case] long sequence: N={N} nb={nb} C={C} exact={int(mask.sum())}")
    plan = lib.Plan(1, N, d, B, C, L["mask"], dtype=dt)
    dev = {x: to_dev(L[x], dt) for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(L["cache_init"], dt))
    torch.cuda.synchronize()
    qb = _sample_qblocks(cfg, 16, 17)
    K64 = O.to_f64(L["K"][0], dt)
    V64 = O.to_f64(L["V"][0], dt)
    mu0 = O.to_f64(L["cache_init"][0], dt)
    a, gap, d1, d2 = O.assign(K64, mu0)
    ref = O.refresh(K64, V64, a, mu0, mask[qb], B, dt)
    ref.update(assign=a, gap=gap, d1=d1, d2=d2)
    say("  oracle reassign done")
    gpu = {"assign": out["assign"][0].cpu().numpy(), "sizes": out["sizes"][0].cpu().numpy(),
           "counts": out["counts"][0].cpu().numpy()[qb],
           "centroids": from_dev(out["centroids"][0], dt),
           "mean_values": from_dev(out["mean_values"][0], dt)}
    r = check_reassign_head(K64, None, mu0, mask[qb], B, dt, gpu, "long sequence", ref=ref)
    say(f"  reassign ok ({r['band_moves']} in-band moves)")
    cnt = np.zeros((1, nb, C), np.int32)
    cnt[0, qb] = ref["counts"]
    o = plan.forward(dev["Q"], dev["K"], dev["V"], to_dev(store64(ref["mu1"], dt)[None], dt),
                     to_dev(store64(ref["vbar"], dt)[None], dt), torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    cnt64 = cnt[0].astype(np.int64)
    want, _ = O.forward(O.to_f64(L["Q"][0], dt), K64, V64, ref["mu1"], ref["vbar"], cnt64, mask,
                        B, qblocks=qb)
    rows = rows_of(qb, B, N)
    check_forward(from_dev(o[0][torch.from_numpy(rows).cuda()], dt), want[rows], dt,
                  f"long sequence forward ({len(qb)} blocks)")
    plan.close()

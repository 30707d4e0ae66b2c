"""Chained parity: the product chain (the GPU's reassign feeding the GPU's forward, and each
step's GPU cache feeding the next GPU step) against the oracle's own chain from the same
starting cache. Nothing the GPU produced is an oracle input: the two chains run side by side
and are compared step by step.

Where the chains' caches differ (the GPU rounds fp32 sums, the oracle exact means: at most one
bf16 step per element), an assignment is compared only where that difference cannot decide
it: with delta the largest distance between the two caches' centroids, a key whose oracle
squared distances satisfy D2 - D1 > 1e-4 D2 + 2 delta (sqrt(D1) + sqrt(D2)) + 2 delta^2 has the
same nearest centroid under both caches (each squared distance moves by at most
2 delta sqrt(D) + delta^2), and there the GPU must agree exactly. Sizes, counts and means are
compared exactly (means within one bf16 step) on every cluster no differing key touches.
The forward of each step is compared twice: teacher-forced with the oracle's cache at the bf16
tolerances, and as the product chain with the GPU's own cache. For the product chain the full
bf16 criterion (max-abs 2e-2, rel-L2 5e-3) applies to the heads whose chains have agreed on
every assignment so far (their caches differ by rounding only). Where some in-band key went to
a different, equally valid cluster, the two chains carry different valid caches from then on
(a key leaving a small cluster moves its mean value by O(1/size), and later steps reassign
from the moved centroids), so that head's product-chain output is not unique: it is checked
for validity instead (finite, and every output coordinate inside the range of the values it
averages), next to its teacher-forced comparison, which stays strict.
"""
import numpy as np
import pytest

import oracle as O
from datagen import drift_layer, get_config, make_layer
from parity_util import (OraclePool, bf16_ulp, check_forward, from_dev, rows_of, say,
                         store64, to_dev, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_video_da_amd as S
    return S


def _comparable(ref, delta):
    d1, d2 = ref["d1"], ref["d2"]
    margin = O.TIE_BAND * d2 + 2 * delta * (np.sqrt(d1) + np.sqrt(np.where(np.isfinite(d2), d2, 0)))
    return np.isinf(d2) | ((d2 - d1) > margin + 2 * delta * delta)


def _compare_step(gpu, ref, K64, mu0_orc64, delta, dtype, what):
    """One head: GPU step (from the GPU chain's cache) against the oracle step (from the
    oracle chain's cache). Returns the number of keys not compared."""
    a_gpu = gpu["assign"].astype(np.int64)
    a_ref = ref["assign"]
    comp = _comparable(ref, delta)
    bad = comp & (a_gpu != a_ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} assignments differ where the caches "
                           f"cannot decide them (first keys {np.nonzero(bad)[0][:8].tolist()})")
    diff = a_gpu != a_ref
    if delta == 0.0 and diff.any():   # same cache: in-band choices must be within the band
        ok = O.assignment_allowed(K64[diff], mu0_orc64, a_gpu[diff], ref["d1"][diff])
        assert ok.all(), f"{what}: in-band assignment not within the band"
    touched = np.zeros(len(ref["sizes"]), bool)
    touched[a_gpu[diff]] = True
    touched[a_ref[diff]] = True
    keep = ~touched
    np.testing.assert_array_equal(gpu["sizes"][keep], ref["sizes"][keep], err_msg=f"{what}: sizes")
    np.testing.assert_array_equal(gpu["counts"][:, keep], ref["counts"][:, keep],
                                  err_msg=f"{what}: counts")
    np.testing.assert_array_equal(gpu["counts"].sum(axis=1), ref["counts"].sum(axis=1),
                                  err_msg=f"{what}: keys outside the exact blocks")
    for name, exact, rounded in (("centroids", ref["mu1_exact"], ref["mu1"]),
                                 ("mean_values", ref["vbar_exact"], ref["vbar"])):
        # an empty cluster keeps its own chain's cache, which may differ by the chains' drift
        live = keep & (ref["sizes"] > 0)
        lim = (bf16_ulp(rounded[live]) + 1e-6) if dtype == "bf16" else \
            (1e-5 * np.sqrt(np.maximum(np.mean(exact[live] ** 2, axis=1, keepdims=True), 1e-6))
             + 1e-7)
        err = np.abs(gpu[name][live] - exact[live])
        assert np.all(err <= lim), f"{what}: {name} off by {float((err / lim).max()):.2f} x tol"
    return int((~comp).sum()), int(diff.sum())


def test_tiny_f32_chain_end_to_end(lib):
    """1 head, N=1024, d=64, fp32: GPU reassign -> GPU forward with the GPU's own cache and
    counts, against oracle reassign -> oracle forward from the same warmed cache, at the fp32
    tolerance (rel-L2 1e-5)."""
    torch = torch_mod()
    cfg = get_config("tiny_f32")
    L = make_layer(cfg)
    dt, H, N, d, B, C = cfg.dtype, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters
    mu0 = np.stack([O.lloyd_warmup(O.to_f64(L["K"][h], dt), O.to_f64(L["cache_init"][h], dt),
                                   10, dt) for h in range(H)]).astype(np.float32)
    L1 = drift_layer(cfg, L, 0)
    say(f"[case] tiny_f32 chain: N={N} C={C}")
    plan = lib.Plan(H, N, d, B, C, L1["mask"], dtype=dt)
    dev = {x: to_dev(L1[x], dt) for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(mu0, dt))
    o, lse = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                          out["counts"], lse=True)
    torch.cuda.synchronize()
    for h in range(H):
        K64, V64, Q64 = (O.to_f64(L1[x][h], dt) for x in ("K", "V", "Q"))
        mu64 = O.to_f64(mu0[h], dt)
        ref = O.reassign_step(K64, V64, mu64, L1["mask"][0], B, dt)
        gpu = {"assign": out["assign"][h].cpu().numpy(), "sizes": out["sizes"][h].cpu().numpy(),
               "counts": out["counts"][h].cpu().numpy(),
               "centroids": from_dev(out["centroids"][h], dt),
               "mean_values": from_dev(out["mean_values"][h], dt)}
        skipped, moved = _compare_step(gpu, ref, K64, mu64, 0.0, dt, f"tiny_f32 head {h}")
        assert moved == 0, "an in-band move would make the chained forward ill-posed"
        want, want_lse = O.forward(Q64, K64, V64, ref["mu1"], ref["vbar"], ref["counts"],
                                   L1["mask"][0], B)
        check_forward(from_dev(o[h], dt), want, dt, f"tiny_f32 chained forward head {h}")
        lg = lse[h].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(lg - want_lse) <= 1e-5 + 4.0 * 2.0 ** -24 * np.abs(want_lse))
    plan.close()


@pytest.fixture(scope="module")
def pool():
    p = OraclePool()
    yield p
    p.close()


def _sample_qblocks(nb, n, seed):
    rng = np.random.default_rng(seed)
    mid = [int(x) for x in rng.choice(np.arange(1, nb - 1), size=n - 2, replace=False)]
    return sorted({0, nb - 1, *mid})


@pytest.mark.slow
def test_extreme_cache_four_step_chain(lib, pool):
    """1% density, C = 512, 40 heads, N = 75600: four denoising steps (K and V drift each
    step). The GPU carries its own refreshed cache from step to step, the oracle its own;
    every head's reassign is compared on every step, the forward on heads 0 and H-1 in full
    and on 8 sampled query blocks of every other head."""
    torch = torch_mod()
    cfg = get_config("extreme_cache_bf16")
    dt, H, N, d, B, C = cfg.dtype, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters
    nb = cfg.num_blocks
    L = make_layer(cfg, threads=16)
    mask = L["mask"][0]
    plan = lib.Plan(H, N, d, B, C, L["mask"], dtype=dt)
    qblocks = _sample_qblocks(nb, 8, 22)
    mu_gpu = to_dev(L["cache_init"], dt)     # the GPU chain's cache (device)
    mu_orc = L["cache_init"].copy()          # the oracle chain's cache (stored bf16)
    Qd = to_dev(L["Q"], dt)
    diverged = np.zeros(H, bool)   # some assignment differed between the chains so far
    for step in range(cfg.steps):
        L = drift_layer(cfg, L, step, threads=16)
        say(f"[case] extreme-cache chain step {step}")
        Kd, Vd = to_dev(L["K"], dt), to_dev(L["V"], dt)
        out = plan.reassign(Kd, Vd, mu_gpu)
        torch.cuda.synchronize()
        refs = pool.reassign([(cfg, h, step + 1, mu_orc[h], mask) for h in range(H)])
        gpu_mu0 = from_dev(mu_gpu, dt)
        got = {"assign": out["assign"].cpu().numpy(), "sizes": out["sizes"].cpu().numpy(),
               "counts": out["counts"].cpu().numpy(),
               "centroids": from_dev(out["centroids"], dt),
               "mean_values": from_dev(out["mean_values"], dt)}
        skipped = moved = 0
        for h in range(H):
            mu0_64 = O.to_f64(mu_orc[h], dt)
            delta = float(np.sqrt(((gpu_mu0[h] - mu0_64) ** 2).sum(axis=1)).max())
            s_, m_ = _compare_step({k: v[h] for k, v in got.items()}, refs[h],
                                   O.to_f64(L["K"][h], dt), mu0_64, delta, dt,
                                   f"step {step} head {h}")
            skipped += s_
            moved += m_
            diverged[h] |= m_ > 0
        say(f"  reassign ok on all {H} heads ({skipped} keys left to the caches' difference, "
            f"{moved} assignments differ)")
        # forward: teacher-forced with the oracle chain's cache, and the GPU chain itself
        mu1 = np.stack([store64(refs[h]["mu1"], dt) for h in range(H)])
        vb = np.stack([store64(refs[h]["vbar"], dt) for h in range(H)])
        cnt = np.stack([refs[h]["counts"].astype(np.int32) for h in range(H)])
        o_tf = plan.forward(Qd, Kd, Vd, to_dev(mu1, dt), to_dev(vb, dt),
                            torch.from_numpy(cnt).cuda())
        o_ch = plan.forward(Qd, Kd, Vd, out["centroids"], out["mean_values"], out["counts"])
        torch.cuda.synchronize()
        tasks = []
        for h in range(H):
            chunks = ([list(range(s, min(nb, s + 128))) for s in range(0, nb, 128)]
                      if h in (0, H - 1) else [qblocks])
            for qb in chunks:
                tasks.append((cfg, h, step + 1, refs[h]["mu1"], refs[h]["vbar"],
                              refs[h]["counts"], mask, qb))
        want = pool.forward(tasks)
        for name, o in (("teacher-forced", o_tf), ("chained", o_ch)):
            rows = [from_dev(o[t[1]][torch.from_numpy(rows_of(t[7], B, N)).cuda()], dt)
                    for t in tasks]
            if name == "teacher-forced":
                check_forward(np.concatenate(rows), np.concatenate(want), dt,
                              f"step {step} {name} forward")
                continue
            agree = [i for i, t in enumerate(tasks) if not diverged[t[1]]]
            if agree:
                check_forward(np.concatenate([rows[i] for i in agree]),
                              np.concatenate([want[i] for i in agree]), dt,
                              f"step {step} chained forward, {H - int(diverged.sum())} heads "
                              f"whose chains agree")
            apart = [i for i, t in enumerate(tasks) if diverged[t[1]]]
            if apart:
                g = np.concatenate([rows[i] for i in apart])
                w = np.concatenate([want[i] for i in apart])
                r = float(np.linalg.norm(g - w) / np.linalg.norm(w))
                say(f"  step {step} chained forward, {int(diverged.sum())} heads whose chains "
                    f"moved apart: rel_l2={r:.3e} max_abs={float(np.abs(g - w).max()):.3e} "
                    f"(reported; validity checked)")
                assert np.all(np.isfinite(g))
                for i in apart:
                    h = tasks[i][1]
                    v = from_dev(Vd[h], dt)
                    vals = np.concatenate([v, from_dev(out["mean_values"][h], dt)])
                    lo, hi = vals.min(axis=0), vals.max(axis=0)
                    tol = 2.0 ** -8 * np.maximum(np.abs(lo), np.abs(hi))   # output rounding
                    assert np.all(rows[i] >= lo - tol) and np.all(rows[i] <= hi + tol), \
                        f"step {step} head {h}: chained output outside the value range"
        mu_gpu = out["centroids"].clone()
        mu_orc = mu1
        del Kd, Vd, out, o_tf, o_ch
    plan.close()

"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Stage-wise and teacher-forced in the oracle -> GPU direction only: the forward is fed the
oracle's refreshed cache, the reassign the seeded (or oracle-warmed) cache; nothing the
GPU produced is ever an oracle input. Sizes span several tiles with ragged tails.
"""
import numpy as np
import pytest

import oracle as O
from datagen import block_mask, get_config, make_layer, drift_layer
from parity_util import (check_forward, check_reassign_head, from_dev, say, store64,
                         to_dev, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_video_da_amd as S
    return S


def _layer64(L, dtype):
    return {x: np.stack([O.to_f64(L[x][i], dtype) for i in range(L[x].shape[0])])
            for x in ("Q", "K", "V")}


def _random_layer(seed, H, N, d, dtype, C, G=None, sigma=0.3):
    """Mixture-shaped Q/K, N(0,1) V, stored in dtype (for shapes the named configs lack)."""
    rng = np.random.default_rng(seed)
    G = G or max(2, C // 2)
    out = {}
    for x in ("Q", "K"):
        arr = []
        for h in range(H):
            cen = rng.standard_normal((G, d)).astype(np.float32)
            arr.append(cen[rng.integers(0, G, N)] + np.float32(sigma) *
                       rng.standard_normal((N, d)).astype(np.float32))
        out[x] = np.stack(arr)
    out["V"] = rng.standard_normal((H, N, d)).astype(np.float32)
    if dtype == "bf16":
        from datagen import f32_to_bf16_bits
        out = {k: f32_to_bf16_bits(v) for k, v in out.items()}
    cache = np.stack([out["K"][h][np.sort(rng.choice(N, C, replace=False))] for h in range(H)])
    return out, cache


def _run_case(lib, L, mu0_stored, mask, cfgd, what, check_reassign=True, heads=None,
              variance=False):
    """GPU reassign + forward vs the oracle on the given heads (default: all). With
    variance=True the variance entry points run (key variances checked, forward corrected)."""
    torch = torch_mod()
    H, N, d, B, C, dtype = (cfgd[k] for k in ("H", "N", "d", "B", "C", "dtype"))
    S = cfgd.get("S") or B
    scale = cfgd.get("scale", 0.0)
    heads = list(range(H)) if heads is None else heads
    say(f"[case] {what}: H={H} N={N} d={d} B={B} S={S} C={C} {dtype} exact={int(mask.sum())}")
    plan = lib.Plan(H, N, d, B, C, mask, dtype=dtype, key_block=S, scale=scale)
    dev = {x: to_dev(L[x], dtype) for x in ("Q", "K", "V")}
    mu0 = to_dev(mu0_stored, dtype)
    L64 = _layer64(L, dtype)
    mu0_64 = np.stack([O.to_f64(mu0_stored[h], dtype) for h in range(H)])
    mask_h = (lambda h: mask[0] if mask.shape[0] == 1 else mask[h])
    if check_reassign:
        out = plan.reassign(dev["K"], dev["V"], mu0, variance=variance)
        torch.cuda.synchronize()
        got = {"assign": out["assign"].cpu().numpy(), "sizes": out["sizes"].cpu().numpy(),
               "counts": out["counts"].cpu().numpy(),
               "centroids": from_dev(out["centroids"], dtype),
               "mean_values": from_dev(out["mean_values"], dtype)}
        if variance:
            got["variance"] = out["variance"].cpu().numpy()
        moves = 0
        for h in heads:
            r = check_reassign_head(L64["K"][h], L64["V"][h], mu0_64[h], mask_h(h), B, dtype,
                                    {k: v[h] for k, v in got.items()}, f"{what} head {h}",
                                    kblock=S)
            moves += r["band_moves"]
        say(f"  reassign ok ({len(heads)} heads, {moves} in-band moves)")
    # forward, teacher-forced with the oracle's refreshed cache
    caches = {h: O.reassign_step(L64["K"][h], L64["V"][h], mu0_64[h], mask_h(h), B, dtype,
                                 kblock=S)
              for h in heads}
    mu1 = np.zeros((H, C, d), np.float32 if dtype == "f32" else np.uint16)
    vb = np.zeros_like(mu1)
    cnt = np.zeros((H, plan.num_blocks, C), np.int32)
    kv32 = np.zeros((H, C), np.float32)
    for h in heads:
        mu1[h] = store64(caches[h]["mu1"], dtype)
        vb[h] = store64(caches[h]["vbar"], dtype)
        cnt[h] = caches[h]["counts"]
        kv32[h] = caches[h]["kvar"].astype(np.float32)
    o_dev, lse_dev = plan.forward(dev["Q"], dev["K"], dev["V"], to_dev(mu1, dtype),
                                  to_dev(vb, dtype), torch.from_numpy(cnt).cuda(), lse=True,
                                  variance=torch.from_numpy(kv32).cuda() if variance else None)
    torch.cuda.synchronize()
    o = from_dev(o_dev, dtype)
    lse = lse_dev.cpu().numpy().astype(np.float64)
    got_all, want_all, lg, lw = [], [], [], []
    for h in heads:
        ref_o, ref_lse = O.forward(L64["Q"][h], L64["K"][h], L64["V"][h], caches[h]["mu1"],
                                   caches[h]["vbar"], caches[h]["counts"], mask_h(h), B,
                                   kblock=S, scale=scale or None,
                                   kvar=kv32[h].astype(np.float64) if variance else None)
        got_all.append(o[h])
        want_all.append(ref_o)
        lg.append(lse[h])
        lw.append(ref_lse)
    check_forward(np.concatenate(got_all), np.concatenate(want_all), dtype, f"{what} forward")
    # lse tolerance (bf16): ln(1 + 2^-8) < 4e-3 bounds the change if every probability in
    # the row sum carried a full bf16 rounding error (8 significant bits, RNE); the kernel
    # sums fp32 probabilities and stays well inside it. fp32: 1e-5, plus 4 * 2^-24 |lse| for
    # the fp32 rounding of logit-sized quantities (the score sums, the max, the final sum),
    # which dominates once logits reach the hundreds
    lg, lw = np.concatenate(lg), np.concatenate(lw)
    lse_err = float(np.max(np.abs(lg - lw)))
    say(f"  {what} lse: max_abs={lse_err:.3e}")
    if dtype == "bf16":
        assert lse_err <= 4e-3, lse_err
    else:
        lim = 1e-5 + 4.0 * 2.0 ** -24 * np.abs(lw)
        assert np.all(np.abs(lg - lw) <= lim), lse_err
    plan.close()
    return o, caches


def _cfgd(cfg, H=None):
    return dict(H=H or cfg.heads, N=cfg.seq_len, d=cfg.head_dim, B=cfg.block, C=cfg.clusters,
                dtype=cfg.dtype, S=cfg.kblock)


# ----------------------------------------------------------------- named small configs
def test_tiny_f32_config(lib):
    """1 head, N=1024, d=64, fp32, 16 clusters, diagonal + 3 random blocks; the cache is
    warmed by 10 oracle Lloyd iterations on the pre-drift keys, then K drifts."""
    cfg = get_config("tiny_f32")
    L = make_layer(cfg)
    mu0 = np.stack([O.lloyd_warmup(O.to_f64(L["K"][h], "f32"), O.to_f64(L["cache_init"][h], "f32"),
                                   10, "f32") for h in range(cfg.heads)]).astype(np.float32)
    L1 = drift_layer(cfg, L, 0)
    _run_case(lib, L1, mu0, L["mask"], _cfgd(cfg), "tiny_f32")


def test_small_bf16_config(lib):
    """12 heads, N=4096, d=64, bf16, C=64, 25% 3D-local mask, oracle-warmed cache."""
    cfg = get_config("small_bf16")
    L = make_layer(cfg)
    mu0 = np.stack([store64(O.lloyd_warmup(O.to_f64(L["K"][h], "bf16"),
                                           O.to_f64(L["cache_init"][h], "bf16"), 10, "bf16"),
                            "bf16") for h in range(cfg.heads)])
    _run_case(lib, L, mu0, L["mask"], _cfgd(cfg), "small_bf16")


def test_small_budget_config(lib):
    """6 heads, N=8192, d=128, bf16, C=128, one mask per head with per-head and per-block
    exact budgets (3..39 of 64 key blocks): every head and query block checked, so a
    scheduling slip that skips or repeats work items shows up."""
    cfg = get_config("small_budget_bf16")
    L = make_layer(cfg)
    assert L["mask"].shape[0] == cfg.heads
    assert len(set(L["mask"].sum(axis=(1, 2)).tolist())) > 1   # budgets differ across heads
    _run_case(lib, L, L["cache_init"], L["mask"], _cfgd(cfg), "small_budget_bf16")


# ----------------------------------------------------------------- keys far from the origin
@pytest.mark.parametrize("name", ["offset_keys_bf16", "offset_keys_wide_bf16",
                                  "offset_keys_d64_bf16"])
def test_offset_keys_assignment_is_exact_outside_the_band(lib, name):
    """Tight clusters around centres shifted far from the origin (|k|^2 some 1e3-1e4 times
    the nearest squared distance): distances taken as |k|^2 + |mu|^2 - 2 k.mu in fp32 carry
    rounding errors that scale with |k|^2, not with the distances, so the assignment must
    still be bit-exact wherever the oracle's top-two gap is outside the band (resident
    table at d = 128 and d = 64, streamed table at C = 1024). Cache warmed by 3 oracle Lloyd
    iterations so many keys have a close second centroid."""
    cfg = get_config(name)
    L = make_layer(cfg)
    mu0 = np.stack([store64(O.lloyd_warmup(O.to_f64(L["K"][h], "bf16"),
                                           O.to_f64(L["cache_init"][h], "bf16"), 3, "bf16"),
                            "bf16") for h in range(cfg.heads)])
    _run_case(lib, L, mu0, L["mask"], _cfgd(cfg), name)


def test_duplicate_centroids_go_to_the_lowest_index(lib):
    """A cache holding some centroids twice (identical rows): every key nearest to such a
    centroid has an exact tie, and the assignment must take the lower index of the pair (the
    near-tie re-measurement breaks equal distances towards the lowest index). Resident table
    (C = 256) and streamed table (C = 1024), d = 128."""
    torch = torch_mod()
    for C in (256, 1024):
        L, cache = _random_layer(150 + C, 2, 6000, 128, "bf16", C, G=C // 4, sigma=0.2)
        dup = np.arange(C // 2, C, 3)          # higher index copies a lower one
        src = dup - C // 2
        cache[:, dup] = cache[:, src]
        nb = -(-6000 // 128)
        mask = np.zeros((1, nb, nb), np.uint8)
        np.fill_diagonal(mask[0], 1)
        say(f"[case] duplicate centroids: C={C}, {len(dup)} duplicated")
        plan = lib.Plan(2, 6000, 128, 128, C, mask, dtype="bf16")
        out = plan.reassign(to_dev(L["K"], "bf16"), to_dev(L["V"], "bf16"), to_dev(cache, "bf16"))
        torch.cuda.synchronize()
        a = out["assign"].cpu().numpy()
        hit = np.isin(a, dup)
        assert not hit.any(), f"C={C}: {int(hit.sum())} keys took the higher copy of a centroid"
        got = {"assign": a, "sizes": out["sizes"].cpu().numpy(),
               "counts": out["counts"].cpu().numpy(),
               "centroids": from_dev(out["centroids"], "bf16"),
               "mean_values": from_dev(out["mean_values"], "bf16")}
        for h in range(2):
            K64 = O.to_f64(L["K"][h], "bf16")
            used = np.isin(O.assign(K64, O.to_f64(cache[h], "bf16"))[0], src).sum()
            say(f"  head {h}: {int(used)} keys nearest to a duplicated centroid")
            check_reassign_head(K64, O.to_f64(L["V"][h], "bf16"), O.to_f64(cache[h], "bf16"),
                                mask[0], 128, "bf16", {k: v[h] for k, v in got.items()},
                                f"duplicates C={C} head {h}")
        plan.close()


@pytest.mark.parametrize("d,C", [(128, 256), (64, 512)])
def test_many_equal_centroids_take_the_exact_pass_over_the_half(lib, d, C):
    """Six identical copies of one centroid, all on one half-wave's side of the distance tiles
    (centroid index c with (c >> 2) & 1 == 0): a key nearest to them has more candidates than
    the near-tie pass keeps, so that lane re-measures every centroid of its half exactly. It
    must still take the lowest copy, and everything else must match the oracle. Resident table
    at d = 128 and d = 64."""
    torch = torch_mod()
    H, N = 2, 4000
    L, cache = _random_layer(700 + d, H, N, d, "bf16", C, G=C // 4, sigma=0.2)
    copies = np.array([8, 16, 24, 40, 48, 56])
    assert np.all(((copies >> 2) & 1) == 0)
    cache[:, copies[1:]] = cache[:, copies[:1]]
    nb = -(-N // 128)
    mask = np.zeros((1, nb, nb), np.uint8)
    np.fill_diagonal(mask[0], 1)
    say(f"[case] six equal centroids: d={d} C={C}")
    plan = lib.Plan(H, N, d, 128, C, mask, dtype="bf16")
    out = plan.reassign(to_dev(L["K"], "bf16"), to_dev(L["V"], "bf16"), to_dev(cache, "bf16"))
    torch.cuda.synchronize()
    a = out["assign"].cpu().numpy()
    hit = np.isin(a, copies[1:])
    assert not hit.any(), f"{int(hit.sum())} keys took a higher copy of the centroid"
    got = {"assign": a, "sizes": out["sizes"].cpu().numpy(),
           "counts": out["counts"].cpu().numpy(),
           "centroids": from_dev(out["centroids"], "bf16"),
           "mean_values": from_dev(out["mean_values"], "bf16")}
    for h in range(H):
        K64 = O.to_f64(L["K"][h], "bf16")
        n8 = int((O.assign(K64, O.to_f64(cache[h], "bf16"))[0] == copies[0]).sum())
        say(f"  head {h}: {n8} keys nearest to the repeated centroid")
        assert n8 > 0, "the case must exercise the repeated centroid"
        check_reassign_head(K64, O.to_f64(L["V"][h], "bf16"), O.to_f64(cache[h], "bf16"),
                            mask[0], 128, "bf16", {k: v[h] for k, v in got.items()},
                            f"six equal centroids d={d} head {h}")
    plan.close()


@pytest.mark.parametrize("C", [64, 1024])
def test_all_centroids_equal(lib, C):
    """Degenerate cache: every centroid the same row. Every key is an exact C-way tie, lists as
    a near tie and re-measures every centroid; all must go to cluster 0, which takes every key,
    while the other clusters stay empty (cached centroid kept, mean value zero, counts zero).
    Resident (C = 64) and streamed (C = 1024) tables."""
    torch = torch_mod()
    H, N, d = 2, 3000, 128
    L, cache = _random_layer(900 + C, H, N, d, "bf16", C)
    cache[:] = cache[:, :1]
    nb = -(-N // 128)
    mask = np.zeros((1, nb, nb), np.uint8)
    np.fill_diagonal(mask[0], 1)
    say(f"[case] all centroids equal: C={C}")
    plan = lib.Plan(H, N, d, 128, C, mask, dtype="bf16")
    out = plan.reassign(to_dev(L["K"], "bf16"), to_dev(L["V"], "bf16"), to_dev(cache, "bf16"))
    torch.cuda.synchronize()
    a = out["assign"].cpu().numpy()
    assert np.array_equal(a, np.zeros_like(a)), f"{int((a != 0).sum())} keys left cluster 0"
    got = {"assign": a, "sizes": out["sizes"].cpu().numpy(),
           "counts": out["counts"].cpu().numpy(),
           "centroids": from_dev(out["centroids"], "bf16"),
           "mean_values": from_dev(out["mean_values"], "bf16")}
    assert np.array_equal(got["sizes"][:, 0], np.full(H, N)) and not got["sizes"][:, 1:].any()
    for h in range(H):
        check_reassign_head(O.to_f64(L["K"][h], "bf16"), O.to_f64(L["V"][h], "bf16"),
                            O.to_f64(cache[h], "bf16"), mask[0], 128, "bf16",
                            {k: v[h] for k, v in got.items()}, f"all equal C={C} head {h}")
    plan.close()


# ----------------------------------------------------------------- ragged / edge shapes
@pytest.mark.parametrize("d,B,dtype,N", [(128, 128, "bf16", 1000), (128, 128, "bf16", 850),
                                         (64, 128, "bf16", 850), (128, 64, "bf16", 1000),
                                         (64, 64, "bf16", 1000), (64, 64, "bf16", 980),
                                         (128, 128, "f32", 1000), (64, 64, "f32", 1000)])
def test_ragged_shapes(lib, d, B, dtype, N):
    """Ragged last block (N = 1000, 980 or 850; 850 and 980 give an odd block count, so the
    last query-block pair has one block), C = 200 (ragged cluster tile), random 30% mask
    with one empty row and one full row, 2 heads with per-head masks."""
    H, C = 2, 200
    L, cache = _random_layer(100 + d + B, H, N, d, dtype, C)
    nb = -(-N // B)
    rng = np.random.default_rng(7)
    mask = (rng.random((H, nb, nb)) < 0.3).astype(np.uint8)
    mask[0, 1, :] = 0
    mask[1, 2, :] = 1
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype=dtype),
              f"ragged d{d} B{B} {dtype}")


@pytest.mark.parametrize("N,C,d", [(900, 20, 128), (2000, 300, 128), (4000, 2048, 128),
                                   (3000, 512, 128), (3000, 513, 128), (5000, 1024, 64),
                                   (5000, 1025, 64)])
def test_cluster_count_edges(lib, N, C, d):
    """bf16 cluster counts away from the tile sizes: fewer centroids than one 32-wide
    distance tile (C = 20), an odd number of 128-centroid staging chunks with a ragged last
    one (C = 300: 3 chunks), and many chunks with mostly tiny or empty clusters
    (C = 2048: 16 chunks, about 2 keys per cluster, many refresh segments); and both sides of
    the largest table the assignment keeps resident in LDS (128 KB of operands: C = 512 at
    d = 128, 1024 at d = 64), past which it streams the table in chunks."""
    H, B = 2, 128
    L, cache = _random_layer(300 + C, H, N, d, "bf16", C, G=max(2, C // 4))
    nb = -(-N // B)
    rng = np.random.default_rng(C)
    mask = (rng.random((1, nb, nb)) < 0.35).astype(np.uint8)
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype="bf16"),
              f"clusters C={C} N={N}")


@pytest.mark.parametrize("H,N,C", [(1, 200, 16), (7, 37000, 64)])
def test_assignment_work_split(lib, H, N, C):
    """The resident assignment splits H * ceil(N / 64) units of 64 keys over one workgroup
    per CU: far fewer units than workgroups (4 units, a ragged last one, most workgroups
    empty), and many units per workgroup with head boundaries inside workgroup ranges
    (7 heads of 579 units: about 16 units a workgroup on 256 CUs), where a workgroup reloads
    the centroid table of the next head. Every head's assignments, sizes, counts and cache
    against the oracle; the forward on a sparse mask (2 exact blocks per query block)."""
    d, B = 128, 128
    L, cache = _random_layer(1500 + H, H, N, d, "bf16", C, G=max(2, C // 4))
    nb = -(-N // B)
    rng = np.random.default_rng(H)
    mask = np.zeros((1, nb, nb), np.uint8)
    for b in range(nb):
        mask[0, b, rng.choice(nb, size=min(2, nb), replace=False)] = 1
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype="bf16"),
              f"assignment work split H={H} N={N}")


# ----------------------------------------------------------------- key blocks smaller than B
@pytest.mark.parametrize("name", ["small_sub32_bf16", "small_sub16_d64_bf16", "tiny_sub_f32"])
def test_key_block_configs(lib, name):
    """Exact key blocks of 32 or 16 keys packed into 128- or 64-row tiles: 3D-local masks
    at the finer granularity (d = 64 with 16-key blocks splits every fetch pass across
    four key blocks; N = 2700 and 1020 leave a partial last key block)."""
    cfg = get_config(name)
    L = make_layer(cfg)
    assert L["mask"].shape[1:] == (cfg.num_blocks, cfg.num_key_blocks)
    _run_case(lib, L, L["cache_init"], L["mask"], _cfgd(cfg), name)


@pytest.mark.parametrize("d,B,S,dtype,N", [
    (128, 128, 32, "bf16", 1000), (128, 128, 64, "bf16", 850), (128, 128, 16, "bf16", 1000),
    (64, 128, 32, "bf16", 850), (64, 128, 16, "bf16", 1000), (128, 64, 32, "bf16", 1000),
    (128, 64, 16, "bf16", 990), (64, 64, 32, "bf16", 980), (64, 64, 16, "bf16", 1000),
    (128, 128, 32, "f32", 1000), (64, 64, 16, "f32", 1000), (128, 128, 64, "f32", 850)])
def test_key_block_ragged(lib, d, B, S, dtype, N):
    """Random per-head key-block masks (25%) with the awkward rows: one query block keeps
    nothing, one keeps every key block, one keeps only the partial last key block, one keeps
    a single key block (a tile padded with unused copies), and the two query blocks of a
    pair keep disjoint sets (tiles of one user only, and mixed tiles at the seam). C = 200
    gives a ragged cluster tile."""
    H, C = 2, 200
    L, cache = _random_layer(500 + d + B + S, H, N, d, dtype, C)
    nb, nkb = -(-N // B), -(-N // S)
    rng = np.random.default_rng(S + B)
    mask = (rng.random((H, nb, nkb)) < 0.25).astype(np.uint8)
    mask[0, 1, :] = 0
    mask[1, 2, :] = 1
    mask[0, 3, :] = 0
    mask[0, 3, nkb - 1] = 1
    mask[1, 0, :] = 0
    mask[1, 0, 5] = 1
    mask[0, 4, :] = 0
    mask[0, 5, :] = 0
    mask[0, 4, : nkb // 2: 3] = 1
    mask[0, 5, nkb // 2:: 3] = 1
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype=dtype, S=S),
              f"key blocks d{d} B{B} S{S} {dtype} N{N}")


def test_key_block_plan_lists(lib):
    """A key-block plan reports its exact lists in key blocks of the plan's size."""
    cfg = get_config("small_sub32_bf16")
    mask = block_mask(cfg)
    plan = lib.Plan(2, cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters, mask,
                    key_block=cfg.kblock)
    rowptr, col = plan.exact_lists(0)
    for b in range(cfg.num_blocks):
        assert col[rowptr[b]:rowptr[b + 1]].tolist() == np.nonzero(mask[0, b])[0].tolist()
    assert plan.info()["exact_pairs"] == int(mask.sum())
    plan.close()


def test_all_key_blocks_exact_is_dense(lib):
    """Every 32-key block exact (N = 700: a partial last key block): dense attention."""
    torch = torch_mod()
    H, N, d, B, S, C = 1, 700, 128, 128, 32, 8
    L, cache = _random_layer(6, H, N, d, "bf16", C)
    mask = np.ones((1, -(-N // B), -(-N // S)), np.uint8)
    plan = lib.Plan(H, N, d, B, C, mask, key_block=S)
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(cache, "bf16"))
    assert int(out["counts"].abs().sum().item()) == 0
    o = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                     out["counts"])
    torch.cuda.synchronize()
    L64 = _layer64(L, "bf16")
    want = O.dense_attention(L64["Q"][0], L64["K"][0], L64["V"][0])
    check_forward(from_dev(o, "bf16")[0], want, "bf16", "all key blocks exact vs dense")
    plan.close()


@pytest.mark.parametrize("N,C,d,B,S,dtype", [
    (1, 1, 128, 128, None, "bf16"), (50, 3, 128, 128, None, "bf16"),
    (50, 3, 128, 128, 32, "bf16"), (129, 5, 128, 128, 16, "bf16"), (129, 5, 64, 64, 16, "bf16"),
    (1, 1, 64, 64, None, "f32"), (129, 5, 64, 64, None, "f32"), (70, 4, 64, 64, 16, "f32")])
def test_tiny_layers(lib, N, C, d, B, S, dtype):
    """Degenerate sizes: one token (one partial block, one cluster), fewer tokens than a
    block, one token past a full block; head 0 keeps a random half of the key blocks (at
    least the first), head 1 keeps none (pure compensation)."""
    H = 2
    L, cache = _random_layer(700 + N + C, H, N, d, dtype, C)
    S_ = S or B
    nb, nkb = -(-N // B), -(-N // S_)
    rng = np.random.default_rng(N + 3 * C)
    mask = (rng.random((H, nb, nkb)) < 0.5).astype(np.uint8)
    mask[0, 0, 0] = 1
    mask[1] = 0
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype=dtype, S=S),
              f"tiny N={N} C={C} d{d} B{B} S{S_} {dtype}")


@pytest.mark.parametrize("S", [None, 16])
def test_max_clusters(lib, S):
    """The largest cluster count the library accepts (C = 8192, 64 staging chunks in the
    assignment, 64 KB of LDS counts per pair with key blocks), about one key per cluster."""
    H, N, d, B, C = 1, 9000, 64, 64, 8192
    L, cache = _random_layer(800 + (S or 0), H, N, d, "bf16", C, G=C // 4)
    S_ = S or B
    nb, nkb = -(-N // B), -(-N // S_)
    mask = (np.random.default_rng(9).random((1, nb, nkb)) < 0.2).astype(np.uint8)
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype="bf16", S=S),
              f"max clusters C={C} S{S_}")


@pytest.mark.parametrize("dtype,scale", [("bf16", 0.05), ("bf16", 0.3), ("f32", 0.05)])
def test_custom_scale(lib, dtype, scale):
    """A softmax scale other than 1/sqrt(d) given in the descriptor."""
    H, N, d, B, C = 2, 700, 64, 64, 30
    L, cache = _random_layer(1000 + int(scale * 100), H, N, d, dtype, C)
    nb = -(-N // B)
    mask = (np.random.default_rng(13).random((1, nb, nb)) < 0.3).astype(np.uint8)
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype=dtype, scale=scale),
              f"scale {scale} {dtype}")


# ----------------------------------------------------------------- variance-corrected compensation
@pytest.mark.parametrize("name", ["small_bf16", "small_sub32_bf16", "tiny_f32", "tiny_sub_f32"])
def test_variance_correction_configs(lib, name):
    """da_reassign_var / da_forward_var on named layers (d = 64 and 128, key blocks of 128,
    64, 32 and 16, bf16 and fp32): key variances against the oracle's, corrected forward
    against the oracle's corrected forward."""
    cfg = get_config(name)
    L = make_layer(cfg)
    _run_case(lib, L, L["cache_init"], L["mask"], _cfgd(cfg), name + " var", variance=True)


@pytest.mark.parametrize("d,B,S,dtype,N", [(128, 128, 128, "bf16", 1000), (64, 128, 32, "bf16", 850),
                                           (128, 64, 64, "f32", 1000)])
def test_variance_correction_ragged(lib, d, B, S, dtype, N):
    """Ragged shapes with the variance entry points: random masks, C = 200."""
    H, C = 2, 200
    L, cache = _random_layer(900 + d + B + S, H, N, d, dtype, C, sigma=0.5)
    nb, nkb = -(-N // B), -(-N // S)
    mask = (np.random.default_rng(S + 7).random((H, nb, nkb)) < 0.3).astype(np.uint8)
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype=dtype, S=S),
              f"variance d{d} B{B} S{S} {dtype} N{N}", variance=True)


def test_zero_variance_equals_plain_forward(lib):
    """da_forward_var with all-zero variances reproduces da_forward bit for bit."""
    torch = torch_mod()
    H, N, d, B, C = 2, 900, 128, 128, 40
    L, cache = _random_layer(11, H, N, d, "bf16", C)
    nb = -(-N // B)
    mask = (np.random.default_rng(12).random((1, nb, nb)) < 0.4).astype(np.uint8)
    plan = lib.Plan(H, N, d, B, C, mask)
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(cache, "bf16"), variance=True)
    o1 = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                      out["counts"])
    o2 = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                      out["counts"], variance=torch.zeros((H, C), dtype=torch.float32,
                                                          device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    plan.close()


# ----------------------------------------------------------------- invariants on the GPU
def _dev_run(lib, L, cache, mask, H, N, d, B, C, counts=None, lse=True):
    torch = torch_mod()
    plan = lib.Plan(H, N, d, B, C, mask)
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(cache, "bf16"))
    cnt = out["counts"] if counts is None else counts
    o, l = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"], cnt,
                        lse=lse)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in out.items()}
    res["O"] = from_dev(o, "bf16")
    res["lse"] = l.cpu().numpy().astype(np.float64)
    plan.close()
    return res


def test_cluster_constant_layer_is_dense(lib):
    """Every key of a cluster equal to its centroid, every value of it equal: the compensation
    is exact, so any mask gives dense attention."""
    H, N, d, B, C = 2, 900, 128, 128, 12
    rng = np.random.default_rng(31)
    from datagen import f32_to_bf16_bits
    L = {}
    cache = []
    lab = rng.integers(0, C, (H, N))
    keys = rng.standard_normal((H, C, d)).astype(np.float32)
    vals = rng.standard_normal((H, C, d)).astype(np.float32)
    L["K"] = f32_to_bf16_bits(np.stack([keys[h][lab[h]] for h in range(H)]))
    L["V"] = f32_to_bf16_bits(np.stack([vals[h][lab[h]] for h in range(H)]))
    L["Q"] = f32_to_bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    cache = f32_to_bf16_bits(keys)
    nb = -(-N // B)
    mask = (rng.random((1, nb, nb)) < 0.3).astype(np.uint8)
    r = _dev_run(lib, L, cache, mask, H, N, d, B, C)
    L64 = _layer64(L, "bf16")
    for h in range(H):
        want = O.dense_attention(L64["Q"][h], L64["K"][h], L64["V"][h])
        check_forward(r["O"][h], want, "bf16", f"cluster-constant head {h} vs dense")


def test_convexity_and_lse_merge_on_gpu(lib):
    """Outputs lie within each dimension's value range; the exact-only and compensation-only
    forwards (counts zeroed; mask emptied) merged by their log-sum-exps give the full one."""
    torch = torch_mod()
    H, N, d, B, C = 2, 1000, 128, 128, 40
    L, cache = _random_layer(32, H, N, d, "bf16", C)
    nb = -(-N // B)
    mask = (np.random.default_rng(33).random((1, nb, nb)) < 0.35).astype(np.uint8)
    mask[0, :, 0] = 1                      # every block keeps one exact block (finite lse)
    full = _dev_run(lib, L, cache, mask, H, N, d, B, C)
    V64 = _layer64(L, "bf16")["V"]
    lo, hi = V64.min(axis=1, keepdims=True), V64.max(axis=1, keepdims=True)
    assert np.all(full["O"] >= lo - 2e-2) and np.all(full["O"] <= hi + 2e-2)
    zero = torch.zeros((H, nb, C), dtype=torch.int32, device="cuda")
    ex = _dev_run(lib, L, cache, mask, H, N, d, B, C, counts=zero)
    cp = _dev_run(lib, L, cache, np.zeros_like(mask), H, N, d, B, C,
                  counts=full["counts"].cuda())
    we = np.exp(ex["lse"] - full["lse"])
    wc = np.exp(cp["lse"] - full["lse"])
    assert np.max(np.abs(we + wc - 1.0)) < 1e-2
    merged = ex["O"] * we[..., None] + cp["O"] * wc[..., None]
    check_forward(merged.reshape(-1, d), full["O"].reshape(-1, d), "bf16", "lse merge")


def test_label_permutation_on_gpu(lib):
    """Reordering the cached centroids relabels the clusters: assignments, sizes, counts and
    means follow the permutation, and the output does not change."""
    H, N, d, B, C = 2, 1000, 128, 128, 40
    L, cache = _random_layer(34, H, N, d, "bf16", C)
    nb = -(-N // B)
    mask = (np.random.default_rng(35).random((1, nb, nb)) < 0.3).astype(np.uint8)
    perm = np.random.default_rng(36).permutation(C)
    a = _dev_run(lib, L, cache, mask, H, N, d, B, C)
    b = _dev_run(lib, L, np.ascontiguousarray(cache[:, perm]), mask, H, N, d, B, C)
    inv = np.argsort(perm)
    L64 = _layer64(L, "bf16")
    band = False
    for h in range(H):
        # key j assigned to cluster c in run a is assigned to inv[c] in run b, except where
        # the two nearest centroids sit inside the tie band (either choice is allowed there)
        gap = O.assign(L64["K"][h], O.to_f64(cache[h], "bf16"))[1]
        sure = gap >= O.TIE_BAND
        band |= bool((~sure).any())
        assert np.array_equal(inv[a["assign"][h].numpy()][sure], b["assign"][h].numpy()[sure])
    if not band:
        assert np.array_equal(a["sizes"].numpy()[:, perm], b["sizes"].numpy())
        assert np.array_equal(a["counts"].numpy()[:, :, perm], b["counts"].numpy())
        assert np.array_equal(a["centroids"].view(torch_mod().int16).numpy()[:, perm],
                              b["centroids"].view(torch_mod().int16).numpy())
    check_forward(b["O"].reshape(-1, d), a["O"].reshape(-1, d), "bf16", "permuted labels")


def test_all_blocks_exact_is_dense(lib):
    """Every block exact: the GPU output is dense attention (oracle's dense routine)."""
    torch = torch_mod()
    H, N, d, B, C = 1, 700, 128, 128, 8
    L, cache = _random_layer(5, H, N, d, "bf16", C)
    nb = -(-N // B)
    mask = np.ones((1, nb, nb), np.uint8)
    plan = lib.Plan(H, N, d, B, C, mask)
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(cache, "bf16"))
    assert int(out["counts"].abs().sum().item()) == 0
    o = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                     out["counts"])
    torch.cuda.synchronize()
    L64 = _layer64(L, "bf16")
    want = O.dense_attention(L64["Q"][0], L64["K"][0], L64["V"][0])
    check_forward(from_dev(o, "bf16")[0], want, "bf16", "all-exact vs dense")


def test_one_cluster_per_key_is_dense(lib):
    """C = N with the cache at the keys: any mask gives dense attention."""
    torch = torch_mod()
    H, N, d, B = 1, 300, 64, 64
    L, _ = _random_layer(6, H, N, d, "bf16", 4)
    nb = -(-N // B)
    mask = (np.random.default_rng(3).random((1, nb, nb)) < 0.4).astype(np.uint8)
    plan = lib.Plan(H, N, d, B, N, mask)
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], dev["K"].clone())
    o = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                     out["counts"])
    torch.cuda.synchronize()
    assert out["assign"].cpu().numpy().tolist() == [list(range(N))]
    L64 = _layer64(L, "bf16")
    want = O.dense_attention(L64["Q"][0], L64["K"][0], L64["V"][0])
    check_forward(from_dev(o, "bf16")[0], want, "bf16", "C=N vs dense")


def test_empty_mask_one_cluster_is_mean(lib):
    """No exact block, one cluster: every row is the mean of V (closed form)."""
    torch = torch_mod()
    H, N, d, B = 2, 520, 128, 128
    L, cache = _random_layer(8, H, N, d, "bf16", 1)
    nb = -(-N // B)
    plan = lib.Plan(H, N, d, B, 1, np.zeros((1, nb, nb), np.uint8))
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    out = plan.reassign(dev["K"], dev["V"], to_dev(cache, "bf16"))
    o = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"], out["mean_values"],
                     out["counts"])
    torch.cuda.synchronize()
    V64 = _layer64(L, "bf16")["V"]
    for h in range(H):
        want = np.broadcast_to(V64[h].mean(axis=0), (N, d))
        check_forward(from_dev(o, "bf16")[h], want, "bf16", f"empty mask C=1 head {h}")


def test_plan_exact_lists_match_mask(lib):
    cfg = get_config("wan14b_bf16")
    mask = block_mask(cfg)
    plan = lib.Plan(2, cfg.seq_len, 128, 128, 256, mask)
    rowptr, col = plan.exact_lists(0)
    nb = cfg.num_blocks
    assert rowptr[-1] == int(mask.sum())
    for b in range(nb):
        assert col[rowptr[b]:rowptr[b + 1]].tolist() == np.nonzero(mask[0, b])[0].tolist()
    info = plan.info()
    assert info["num_blocks"] == nb and info["exact_pairs"] == int(mask.sum())
    plan.close()


def test_entry_point_validation_on_device(lib):
    """Aliased cache buffers and misaligned pointers are rejected before any launch."""
    torch = torch_mod()
    H, N, d, B, C = 1, 256, 64, 64, 8
    plan = lib.Plan(H, N, d, B, C, np.ones((1, 4, 4), np.uint8))
    K = torch.zeros((H, N, d), dtype=torch.bfloat16, device="cuda")
    mu = torch.zeros((H, C, d), dtype=torch.bfloat16, device="cuda")
    outs = [torch.zeros((H, C, d), dtype=torch.bfloat16, device="cuda"),
            torch.zeros((H, N), dtype=torch.int32, device="cuda"),
            torch.zeros((H, C), dtype=torch.int32, device="cuda"),
            torch.zeros((H, 4, C), dtype=torch.int32, device="cuda")]
    st = lib.da_reassign(plan._h, K.data_ptr(), K.data_ptr(), mu.data_ptr(), mu.data_ptr(),
                         outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                         outs[3].data_ptr(), None)
    assert st == lib.DA_ERR_INVALID_ARGUMENT
    st = lib.da_forward(plan._h, K.data_ptr() + 2, K.data_ptr(), K.data_ptr(), mu.data_ptr(),
                        mu.data_ptr(), outs[3].data_ptr(), K.data_ptr(), None, None)
    assert st == lib.DA_ERR_INVALID_ARGUMENT
    st = lib.da_forward(plan._h, None, K.data_ptr(), K.data_ptr(), mu.data_ptr(),
                        mu.data_ptr(), outs[3].data_ptr(), K.data_ptr(), None, None)
    assert st == lib.DA_ERR_INVALID_ARGUMENT
    plan.close()


def test_side_stream_matches_current_stream(lib):
    """A plan driven on a side stream (the library checks that the stream belongs to the
    plan's device) gives bit-identical results to the same step on the current stream: every
    kernel is deterministic."""
    torch = torch_mod()
    H, N, d, B, C = 2, 1000, 128, 128, 40
    L, cache = _random_layer(31, H, N, d, "bf16", C)
    nb = -(-N // B)
    mask = (np.random.default_rng(31).random((1, nb, nb)) < 0.3).astype(np.uint8)
    plan = lib.Plan(H, N, d, B, C, mask)
    dev = {x: to_dev(L[x], "bf16") for x in ("Q", "K", "V")}
    mu0 = to_dev(cache, "bf16")

    def step(stream):
        out = plan.reassign(dev["K"], dev["V"], mu0, stream=stream)
        o, lse = plan.forward(dev["Q"], dev["K"], dev["V"], out["centroids"],
                              out["mean_values"], out["counts"], lse=True, stream=stream)
        return out, o, lse

    ref = step(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = step(side)
    side.synchronize()
    for k in ("centroids", "mean_values", "assign", "sizes", "counts"):
        assert torch.equal(ref[0][k], got[0][k]), k
    assert torch.equal(ref[1], got[1]) and torch.equal(ref[2], got[2])
    plan.close()


def test_layer_step_replays_in_a_hip_graph(lib):
    """The compute calls enqueue kernels only (no allocation, memset or synchronisation), so a
    layer step (reassign + forward) can be captured in a HIP graph. Every replay, with eager
    work and synchronisation between replays, is bit-identical to the eager step."""
    torch = torch_mod()
    H, N, d, B, C = 2, 1000, 128, 128, 40
    L, cache = _random_layer(41, H, N, d, "bf16", C)
    nb = -(-N // B)
    mask = (np.random.default_rng(41).random((1, nb, nb)) < 0.3).astype(np.uint8)
    plan = lib.Plan(H, N, d, B, C, mask)
    Q, K, V = (to_dev(L[x], "bf16") for x in ("Q", "K", "V"))
    mu0 = to_dev(cache, "bf16")
    out = plan.reassign(K, V, mu0)
    O = torch.empty_like(Q)

    def step(s=None):
        plan.reassign(K, V, mu0, out=out, stream=s)
        plan.forward(Q, K, V, out["centroids"], out["mean_values"], out["counts"], out=O,
                     stream=s)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    ref_o = O.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    for r in range(3):
        for v in out.values():
            v.zero_()
        O.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], out[k]), (r, k)
        assert torch.equal(ref_o, O), r
        step()
        torch.cuda.synchronize()
    del graph
    plan.close()


@pytest.mark.parametrize("d,B,S,dtype", [(128, 128, 128, "bf16"), (64, 64, 16, "bf16"),
                                         (128, 128, 32, "bf16"), (64, 64, 64, "f32")])
def test_wide_logit_range_moves_the_reference_max(lib, d, B, S, dtype):
    """Logits spanning about 80 log2 units, growing along the sequence (key rows scaled by
    1 + 3 j/N, queries by 4): the forward's lazily moved reference max has to move on many
    chunks, and probabilities up to the rescale limit occur, exact and cluster tiles alike."""
    H, N, C = 2, 1000, 40
    rng = np.random.default_rng(61 + d + S)
    G = 8
    L = {}
    for x in ("Q", "K"):
        arr = []
        for h in range(H):
            cen = rng.standard_normal((G, d)).astype(np.float32)
            arr.append(cen[rng.integers(0, G, N)] + np.float32(0.3) *
                       rng.standard_normal((N, d)).astype(np.float32))
        L[x] = np.stack(arr)
    L["Q"] *= np.float32(4.0)
    L["K"] *= (1.0 + 3.0 * np.arange(N, dtype=np.float32) / N)[None, :, None]
    L["V"] = rng.standard_normal((H, N, d)).astype(np.float32)
    if dtype == "bf16":
        from datagen import f32_to_bf16_bits
        L = {k: f32_to_bf16_bits(v) for k, v in L.items()}
    cache = np.stack([L["K"][h][np.sort(rng.choice(N, C, replace=False))] for h in range(H)])
    nb, nkb = -(-N // B), -(-N // S)
    mask = (rng.random((H, nb, nkb)) < 0.3).astype(np.uint8)
    mask[0, 1, :] = 0
    _run_case(lib, L, cache, mask, dict(H=H, N=N, d=d, B=B, C=C, dtype=dtype, S=S),
              f"wide logits d{d} B{B} S{S} {dtype}")


def test_plan_as_context_manager_and_after_close(lib):
    """`with Plan(...)` releases the plan on exit; a closed plan's calls raise (the library
    rejects the null handle before enqueuing anything)."""
    torch = torch_mod()
    H, N, d, B, C = 1, 300, 64, 64, 8
    L, cache = _random_layer(51, H, N, d, "bf16", C)
    mask = np.ones((1, 5, 5), np.uint8)
    K = to_dev(L["K"], "bf16")
    with lib.Plan(H, N, d, B, C, mask) as plan:
        out = plan.reassign(K, K, to_dev(cache, "bf16"))
        torch.cuda.synchronize()
        assert int(out["sizes"].sum().item()) == H * N
    assert plan._h is None
    with pytest.raises(lib.DAError):
        plan.reassign(K, K, to_dev(cache, "bf16"))
    plan.close()   # a second close is a no-op

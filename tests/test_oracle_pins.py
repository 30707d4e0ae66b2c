"""Pins of the fp64 oracle against things other than itself: a hand-derived worked
example, closed forms, special cases that reduce to plain attention or to library
routines, brute force on tiny inputs, and invariants of the definitions.

Each pin is chosen so that a plausible slip (a dropped compensation term, ln swapped for
log2 or for the raw count, an off-by-one block index, transposed operands, means over
the wrong key set, a wrong empty-cluster rule) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from datagen import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, n, d, scale=1.0):
    return np.random.default_rng(seed).standard_normal((n, d)) * scale


def _mask(seed, nb, density):
    rng = np.random.default_rng(seed)
    m = (rng.random((nb, nb)) < density).astype(np.uint8)
    return m


# ----------------------------------------------------------------- hand-worked example
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    e = g["expected"]
    B, scale = g["block"], g["scale"]
    mask = np.array(g["mask"], np.uint8)
    K = np.log(np.array(g["x_of_keys"], float))[:, None]
    Q = np.array(g["q"], float)[:, None]
    V = np.array(g["v"], float)[:, None]
    mu0 = np.array(g["mu0"], float)[:, None]
    st = O.reassign_step(K, V, mu0, mask, B, "f64")
    assert st["assign"].tolist() == e["assign"]
    assert st["sizes"].tolist() == e["sizes"]
    np.testing.assert_allclose(np.exp(st["mu1"][:2, 0]), e["mu1_as_exp"], rtol=1e-13)
    assert st["mu1"][2, 0] == e["mu1_empty"]
    np.testing.assert_allclose(st["vbar"][:, 0], e["vbar"], rtol=0, atol=1e-14)
    assert st["counts"].tolist() == e["counts"]
    out, lse = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B, scale=scale)
    want = np.array(e["out_num"], float) / np.array(e["out_den"], float)
    np.testing.assert_allclose(out[:, 0], want, rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.array(e["lse_exp"], float)), rtol=1e-13)
    dense = O.dense_attention(Q, K, V, scale=scale)
    assert dense[0, 0] == pytest.approx(e["dense_token0_num"] / e["dense_token0_den"], rel=1e-13)
    sub = O.forward_substituted(Q, K, V, st["assign"], st["mu1"], st["vbar"], mask, B,
                                scale=scale)
    np.testing.assert_allclose(sub[:, 0], want, rtol=1e-13)


# ----------------------------------------------------------------- storage rounding
def test_bf16_rounding_closed_forms():
    one = 1.0
    cases = {
        one + 2 ** -8: one,                         # tie -> even (mantissa 0)
        one + 3 * 2 ** -8: one + 2 ** -6,           # tie -> even (mantissa 2)
        one + 2 ** -8 + 2 ** -20: one + 2 ** -7,    # just above the tie
        -(2.0 + 2 ** -7): -2.0,                     # tie at exponent 1 -> even
        3.0e38 * 2: math.inf,                       # overflow
        0.0: 0.0,
    }
    for x, want in cases.items():
        assert O.storage_round(np.array([x]), "bf16")[0] == want, x


def test_bf16_rounding_matches_bit_rounding():
    x = np.random.default_rng(5).standard_normal(200000).astype(np.float32) * 7
    want = bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(O.storage_round(x.astype(np.float64), "bf16"), want)
    np.testing.assert_array_equal(O.to_f64(f32_to_bf16_bits(x), "bf16"), want)


# ----------------------------------------------------------------- P1, P2, P3, P5
def test_all_blocks_exact_is_dense():
    """P1: with every block exact no key is left over (n = 0) and the result is dense
    softmax attention (ragged tail: N = 200, B = 64)."""
    n, d, B, C = 200, 16, 64, 7
    Q, K, V = _rand(1, n, d), _rand(2, n, d), _rand(3, n, d)
    nb = -(-n // B)
    mask = np.ones((nb, nb), np.uint8)
    st = O.reassign_step(K, V, K[:C].copy(), mask, B, "f64")
    assert st["counts"].sum() == 0
    out, _ = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B)
    np.testing.assert_allclose(out, O.dense_attention(Q, K, V), rtol=1e-12, atol=1e-13)


def test_one_cluster_per_key_is_dense():
    """P2: C = N with the cache at the keys themselves: each key is its own cluster, the
    refreshed centroid/mean are that key/value, counts are 0/1, and any mask gives
    dense attention."""
    n, d, B = 150, 8, 32
    Q, K, V = _rand(4, n, d), _rand(5, n, d), _rand(6, n, d)
    nb = -(-n // B)
    mask = _mask(7, nb, 0.3)
    st = O.reassign_step(K, V, K.copy(), mask, B, "f64")
    assert st["assign"].tolist() == list(range(n))
    assert set(np.unique(st["counts"]).tolist()) <= {0, 1}
    out, _ = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B)
    np.testing.assert_allclose(out, O.dense_attention(Q, K, V), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cluster_constant_keys_and_values_is_dense(seed):
    """P3: if every key and value equals its cluster's centroid and mean value, the
    compensation with ln-count weights reproduces dense attention exactly for any mask
    (a count off by one, or log2 for ln, breaks it)."""
    rng = np.random.default_rng(seed)
    n, d, B, C = 300, 8, 64, 5
    mu = rng.standard_normal((C, d))
    vb = rng.standard_normal((C, d))
    a = rng.integers(0, C, n)
    K, V = mu[a], vb[a]
    Q = rng.standard_normal((n, d)) * 2
    nb = -(-n // B)
    mask = _mask(seed + 10, nb, 0.25)
    counts = O.qblock_counts_direct(a, mask, B, C)
    out, _ = O.forward(Q, K, V, mu, vb, counts, mask, B)
    np.testing.assert_allclose(out, O.dense_attention(Q, K, V), rtol=1e-11, atol=1e-12)


def test_empty_mask_single_cluster_is_mean_value():
    """P5: no exact block and one cluster: every output row is the mean of all values."""
    n, d, B = 130, 6, 32
    Q, K, V = _rand(8, n, d), _rand(9, n, d), _rand(10, n, d)
    nb = -(-n // B)
    mask = np.zeros((nb, nb), np.uint8)
    st = O.reassign_step(K, V, K[:1].copy(), mask, B, "f64")
    out, lse = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B)
    np.testing.assert_allclose(out, np.broadcast_to(V.mean(axis=0), out.shape), rtol=1e-12)
    np.testing.assert_allclose(
        lse, O.default_scale(d) * (Q @ K.mean(axis=0)) + math.log(n), rtol=1e-12)


# ----------------------------------------------------------------- P4, P6, P7
def _small_case(seed, n=260, d=16, B=64, C=9, density=0.3):
    Q, K, V = _rand(seed, n, d), _rand(seed + 1, n, d), _rand(seed + 2, n, d)
    nb = -(-n // B)
    mask = _mask(seed + 3, nb, density)
    st = O.reassign_step(K, V, K[::max(1, n // C)][:C].copy(), mask, B, "f64")
    return Q, K, V, mask, B, st


def test_convexity():
    """P4: weights are positive and sum to one, so every output coordinate lies between
    the smallest and largest value coordinate."""
    Q, K, V, mask, B, st = _small_case(20)
    out, _ = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B)
    assert np.all(out <= V.max(axis=0) + 1e-12)
    assert np.all(out >= V.min(axis=0) - 1e-12)


def test_split_merge_by_lse():
    """P6: exact-only and compensation-only results merged by their log-sum-exps equal
    the one-softmax result."""
    Q, K, V, mask, B, st = _small_case(30)
    mu, vb, cnt = st["mu1"], st["vbar"], st["counts"]
    full, lse = O.forward(Q, K, V, mu, vb, cnt, mask, B)
    ex, lse_e = O.forward(Q, K, V, mu, vb, np.zeros_like(cnt), mask, B)
    cp, lse_c = O.forward(Q, K, V, mu, vb, cnt, np.zeros_like(mask), B)
    # rows whose block has no exact key block get lse_e = -inf (no logits); handle that
    we = np.where(np.isfinite(lse_e), np.exp(lse_e - lse), 0.0)
    wc = np.exp(lse_c - lse)
    merged = np.nan_to_num(ex) * we[:, None] + cp * wc[:, None]
    np.testing.assert_allclose(we + wc, 1.0, rtol=1e-12)
    np.testing.assert_allclose(merged, full, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", [40, 41])
def test_matches_key_substitution_brute_force(seed):
    """P7: the count-weighted cluster logits equal attention over all N keys with every
    non-exact key replaced by its cluster's centroid and mean value."""
    Q, K, V, mask, B, st = _small_case(seed, n=150, d=8, B=32, C=6)
    out, _ = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B)
    sub = O.forward_substituted(Q, K, V, st["assign"], st["mu1"], st["vbar"], mask, B)
    np.testing.assert_allclose(out, sub, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- P8, P9, P10
def test_count_invariants():
    """P8: sum_c N_c = N; sum_c n[b][c] = N minus the valid keys in b's exact blocks;
    0 <= n <= N_c; n = N_c minus a per-block histogram over the exact blocks (counted
    here key by key); the unrounded centroid is the mean of its keys."""
    Q, K, V, mask, B, st = _small_case(50, n=333, C=11)
    n = K.shape[0]
    a, sizes, cnt = st["assign"], st["sizes"], st["counts"]
    nb = mask.shape[0]
    assert sizes.sum() == n
    hist = np.zeros((nb, len(sizes)), np.int64)
    for j in range(n):
        hist[j // B, a[j]] += 1
    for b in range(nb):
        valid_exact = sum(min(n, (kb + 1) * B) - kb * B for kb in range(nb) if mask[b, kb])
        assert cnt[b].sum() == n - valid_exact
        np.testing.assert_array_equal(cnt[b], sizes - hist[mask[b] != 0].sum(axis=0))
    assert np.all(cnt >= 0) and np.all(cnt <= sizes[None, :])
    for c in range(len(sizes)):
        if sizes[c]:
            np.testing.assert_allclose((K[a == c] - st["mu1_exact"][c]).sum(axis=0), 0,
                                       atol=1e-12)


def test_lloyd_monotone_and_fixed_point():
    """P9: for fixed keys, J(a1, mu1) <= J(a1, mu0) <= J(a0, mu0); a converged cache
    reassigns every key to the same cluster and leaves the centroids unchanged."""
    rng = np.random.default_rng(60)
    K = rng.standard_normal((400, 8))
    mu0 = K[rng.choice(400, 12, replace=False)] + 0.3
    a_prev = O.assign(K, mu0 + 0.2)[0]
    st = O.reassign_step(K, K, mu0, np.zeros((7, 7), np.uint8), 64, "f64")
    j_prev = O.objective(K, mu0, a_prev)
    j0 = O.objective(K, mu0, st["assign"])
    j1 = O.objective(K, st["mu1"], st["assign"])
    assert j1 <= j0 + 1e-12 and j0 <= j_prev + 1e-12
    mu = O.lloyd_warmup(K, mu0, 60, "f64")
    st2 = O.reassign_step(K, K, mu, np.zeros((7, 7), np.uint8), 64, "f64")
    np.testing.assert_array_equal(st2["assign"], O.assign(K, mu)[0])
    np.testing.assert_allclose(st2["mu1"], mu, atol=1e-13)


def test_label_permutation():
    """P10: renumbering the clusters permutes assignments and leaves the output unchanged."""
    Q, K, V, mask, B, st = _small_case(70, C=8)
    perm = np.random.default_rng(71).permutation(8)
    mu0 = K[::260 // 8][:8].copy()
    st1 = O.reassign_step(K, V, mu0, mask, B, "f64")
    st2 = O.reassign_step(K, V, mu0[perm], mask, B, "f64")
    inv = np.argsort(perm)
    np.testing.assert_array_equal(st2["assign"], inv[st1["assign"]])
    o1, _ = O.forward(Q, K, V, st1["mu1"], st1["vbar"], st1["counts"], mask, B)
    o2, _ = O.forward(Q, K, V, st2["mu1"], st2["vbar"], st2["counts"], mask, B)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- P11, ties, libraries
def test_well_separated_mixture_recovers_labels():
    rng = np.random.default_rng(80)
    G, d = 16, 32
    centres = rng.standard_normal((G, d)) * 4
    lab = rng.integers(0, G, 2000)
    K = centres[lab] + 0.05 * rng.standard_normal((2000, d))
    a, gap, _, _ = O.assign(K, centres)
    np.testing.assert_array_equal(a, lab)
    assert gap.min() > 0.5


def test_ties_go_to_lowest_index_and_are_flagged():
    K = np.array([[0.0, 0.0], [1.0, 1.0], [2.0, 0.0]])
    mu = np.array([[1.0, 0.0], [5.0, 5.0], [1.0, 0.0], [0.0, 1.0]])   # 0 and 2 identical
    a, gap, d1, d2 = O.assign(K, mu)
    assert a.tolist() == [0, 0, 0]
    assert gap[0] == 0 and gap[2] == 0           # exact ties
    assert d1.tolist() == [1.0, 1.0, 1.0]
    ok = O.assignment_allowed(K, mu, np.array([2, 3, 2]), d1)
    assert ok.tolist() == [True, True, True]      # key 1: mu_3 also at distance 1
    assert not O.assignment_allowed(K, mu, np.array([1, 1, 1]), d1).any()


def test_assignment_matches_scipy_vq():
    vq = pytest.importorskip("scipy.cluster.vq")
    rng = np.random.default_rng(90)
    K = rng.standard_normal((3000, 16))
    mu = rng.standard_normal((40, 16))
    code, dist = vq.vq(K, mu)
    a, gap, d1, _ = O.assign(K, mu)
    np.testing.assert_array_equal(a, code)
    np.testing.assert_allclose(np.sqrt(d1), dist, rtol=1e-12)


def test_dense_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    Q, K, V = _rand(100, 97, 24), _rand(101, 97, 24), _rand(102, 97, 24)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None])[0]
    np.testing.assert_allclose(O.dense_attention(Q, K, V), want.numpy(), rtol=1e-12,
                               atol=1e-13)


def test_bf16_cache_refresh_rounds_means():
    """The refreshed cache is the unrounded mean rounded once to bf16."""
    rng = np.random.default_rng(110)
    K = O.storage_round(rng.standard_normal((500, 16)), "bf16")
    mu0 = K[:10].copy()
    st = O.reassign_step(K, K, mu0, np.zeros((8, 8), np.uint8), 64, "bf16")
    np.testing.assert_array_equal(st["mu1"], O.storage_round(st["mu1_exact"], "bf16"))
    assert np.max(np.abs(st["mu1"] - st["mu1_exact"]) / np.maximum(
        np.abs(st["mu1_exact"]), 1e-30)) <= 2 ** -8


# ----------------------------------------------------------------- key blocks finer than query blocks
def test_hand_worked_key_blocks():
    """Exact keys chosen one at a time (key block S = 1 inside query blocks of 2): counts
    and outputs against closed forms worked on paper."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_key_blocks.json")))
    e = g["expected"]
    B, S, scale = g["block"], g["key_block"], g["scale"]
    mask = np.array(g["mask"], np.uint8)
    K = np.log(np.array(g["x_of_keys"], float))[:, None]
    Q = np.array(g["q"], float)[:, None]
    V = np.array(g["v"], float)[:, None]
    mu0 = np.array(g["mu0"], float)[:, None]
    st = O.reassign_step(K, V, mu0, mask, B, "f64", kblock=S)
    assert st["counts"].tolist() == e["counts"]
    out, lse = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B, scale=scale,
                         kblock=S)
    den = np.array(e["out_den"], float)
    np.testing.assert_allclose(out[:, 0], np.array(e["out_num"], float) / den, rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(den), rtol=1e-13)
    sub = O.forward_substituted(Q, K, V, st["assign"], st["mu1"], st["vbar"], mask, B,
                                scale=scale, kblock=S)
    np.testing.assert_allclose(sub[:, 0], np.array(e["out_num"], float) / den, rtol=1e-13)


def _expand(mask, factor, n_keys_blocks):
    """Block mask [nb][nb] -> the same exact key set at key blocks `factor` times finer."""
    return np.repeat(mask, factor, axis=1)[:, :n_keys_blocks]


@pytest.mark.parametrize("S", [16, 32])
def test_expanded_mask_is_the_block_mask(S):
    """A key-block mask that keeps exactly the keys of a query-sized block mask gives the
    same counts and the same forward, to the last bit (same exact key set, same order)."""
    n, d, B, C = 300, 16, 64, 7
    Q, K, V = _rand(60, n, d), _rand(61, n, d), _rand(62, n, d)
    nb = -(-n // B)
    m = _mask(63, nb, 0.4)
    ms = _expand(m, B // S, -(-n // S))
    mu0 = K[::40][:C].copy()
    st = O.reassign_step(K, V, mu0, m, B, "f64")
    ss = O.reassign_step(K, V, mu0, ms, B, "f64", kblock=S)
    np.testing.assert_array_equal(st["counts"], ss["counts"])
    o1, l1 = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], m, B)
    o2, l2 = O.forward(Q, K, V, ss["mu1"], ss["vbar"], ss["counts"], ms, B, kblock=S)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("seed", [70, 71])
def test_key_blocks_match_substitution_brute_force(seed):
    """Key blocks of 8 inside query blocks of 32, ragged at both granularities (N = 150):
    the count-weighted forward equals attention over all keys with every key outside the
    exact key blocks replaced by its cluster's centroid and mean value."""
    n, d, B, S, C = 150, 8, 32, 8, 6
    Q, K, V = _rand(seed, n, d), _rand(seed + 1, n, d), _rand(seed + 2, n, d)
    nb, nkb = -(-n // B), -(-n // S)
    mask = (np.random.default_rng(seed + 3).random((nb, nkb)) < 0.3).astype(np.uint8)
    st = O.reassign_step(K, V, K[::25][:C].copy(), mask, B, "f64", kblock=S)
    out, _ = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B, kblock=S)
    sub = O.forward_substituted(Q, K, V, st["assign"], st["mu1"], st["vbar"], mask, B,
                                kblock=S)
    np.testing.assert_allclose(out, sub, rtol=1e-12, atol=1e-13)


def test_key_block_count_invariants():
    """Counts at key-block granularity: sum_c n[b][c] is N minus the valid keys of b's
    exact key blocks (the last one ragged), and n = N_c minus a key-by-key histogram."""
    n, d, B, S, C = 333, 8, 64, 16, 11
    K, V = _rand(80, n, d), _rand(81, n, d)
    nb, nkb = -(-n // B), -(-n // S)
    mask = (np.random.default_rng(82).random((nb, nkb)) < 0.35).astype(np.uint8)
    mask[:, nkb - 1] = 1                      # every query block keeps the ragged key block
    st = O.reassign_step(K, V, K[::30][:C].copy(), mask, B, "f64", kblock=S)
    a, sizes, cnt = st["assign"], st["sizes"], st["counts"]
    for b in range(nb):
        valid = sum(min(n, (kb + 1) * S) - kb * S for kb in range(nkb) if mask[b, kb])
        assert cnt[b].sum() == n - valid
        inside = np.zeros(C, np.int64)
        for j in range(n):
            if mask[b, j // S]:
                inside[a[j]] += 1
        np.testing.assert_array_equal(cnt[b], sizes - inside)


# ----------------------------------------------------------------- variance-corrected compensation
def _one_cluster_lse(Q, K, kvar):
    """lse of the forward with no exact block and every key in one cluster (centroid = mean)."""
    n, d = K.shape
    a = np.zeros(n, np.int64)
    mu = K.mean(axis=0, keepdims=True)
    counts = np.full((1, 1), n, np.int64)
    mask = np.zeros((1, 1), np.uint8)
    V = np.zeros_like(K)
    _, lse = O.forward(Q, K, V, mu, np.zeros((1, d)), counts, mask, n, kvar=kvar)
    return lse


def test_variance_correction_is_second_order_exact():
    """Keys mu +- delta e_i (2d keys): the sum of exp(s q.k) is exp(s q.mu) sum_i 2 cosh(s delta
    q_i). The plain representative misses it at order delta^2; with kvar = delta^2 / d the
    correction leaves an order-delta^4 residual (halving delta divides it by 16)."""
    d = 6
    rng = np.random.default_rng(90)
    q = rng.standard_normal((1, d)) * 2.0
    mu = rng.standard_normal(d)
    s = O.default_scale(d)
    errs_plain, errs_corr = [], []
    for delta in (0.4, 0.2, 0.1):
        K = np.concatenate([mu + delta * np.eye(d), mu - delta * np.eye(d)])
        exact = s * q[0] @ mu + np.log(np.sum(2 * np.cosh(s * delta * q[0])))
        kv = O.key_variance(K, np.zeros(2 * d, np.int64), K.mean(axis=0, keepdims=True))
        assert kv[0] == pytest.approx(delta * delta / d, rel=1e-12)
        errs_plain.append(abs(_one_cluster_lse(q, K, None)[0] - exact))
        errs_corr.append(abs(_one_cluster_lse(q, K, kv)[0] - exact))
    for e0, e1 in zip(errs_plain, errs_plain[1:]):
        assert 3.5 < e0 / e1 < 4.5          # delta^2
    for e0, e1 in zip(errs_corr, errs_corr[1:]):
        assert 14.0 < e0 / e1 < 18.0        # delta^4
    assert errs_corr[-1] < 1e-3 * errs_plain[-1]


def test_variance_correction_matches_gaussian_keys():
    """Isotropic Gaussian keys k = mu + sigma z: log of the mean of exp(s q.k) is
    s q.mu + s^2 sigma^2 |q|^2 / 2; the corrected compensation reproduces it within the
    sampling error while the plain one is off by that term."""
    d, n, sigma = 8, 400_000, 0.5
    rng = np.random.default_rng(91)
    mu = rng.standard_normal(d)
    K = mu + sigma * rng.standard_normal((n, d))
    q = np.full((1, d), 1.5)
    s = O.default_scale(d)
    kv = O.key_variance(K, np.zeros(n, np.int64), K.mean(axis=0, keepdims=True))
    assert kv[0] == pytest.approx(sigma * sigma, rel=1e-2)
    logits = s * K @ q[0]
    m = logits.max()
    exact = m + np.log(np.exp(logits - m).sum())
    term = 0.5 * s * s * sigma * sigma * float(q[0] @ q[0])
    plain = _one_cluster_lse(q, K, None)[0]
    corr = _one_cluster_lse(q, K, kv)[0]
    assert abs(corr - exact) < 0.02 * term
    assert abs((exact - plain) - term) < 0.02 * term


def test_zero_variance_is_the_plain_forward():
    Q, K, V, mask, B, st = _small_case(92)
    o1, l1 = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B)
    o2, l2 = O.forward(Q, K, V, st["mu1"], st["vbar"], st["counts"], mask, B,
                       kvar=np.zeros(st["mu1"].shape[0]))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert np.all(st["kvar"] >= 0)


# ----------------------------------------------------------------- tie band and key variance
def _frac(x):
    from fractions import Fraction
    if isinstance(x, list):
        return Fraction(int(x[0]), int(x[1]))
    return Fraction(x)


def test_near_tie_gaps_are_the_hand_derived_fractions():
    """Relative top-two gaps (D2 - D1) / D2 of hand-placed near ties (about 6e-5, 2.4e-4, just
    under 1e-4, 9e-5): exact fractions, so a gap measured against D1, a dropped square or a
    swapped pair changes them."""
    g = json.load(open(os.path.join(GOLDEN, "near_ties_and_key_variance.json")))["near_ties"]
    e = g["expected"]
    K = np.array(g["keys"], float)[:, None]
    mu = np.array([float(_frac(c)) for c in g["centroids"]])[:, None]
    a, gap, d1, d2 = O.assign(K, mu)
    assert a.tolist() == e["assign"]
    assert d1.tolist() == [float(e["d1"])] * len(K)
    np.testing.assert_allclose(d2, [float(_frac(x)) for x in e["d2"]], rtol=1e-15)
    np.testing.assert_allclose(gap, [float(_frac(x)) for x in e["gap"]], rtol=1e-12)
    # the parity rule excuses a mismatch only inside the band
    assert (gap < O.TIE_BAND).tolist() == e["inside_band"]


def test_tie_band_membership_is_measured_against_the_candidate_distance():
    """assignment_allowed accepts a centroid whose squared distance exceeds the minimum by
    0.90e-4 of itself and by 0.99994e-4 of itself (more than 1e-4 of the minimum: a band
    measured against D1 would reject it), and rejects ones at 1.10e-4 and 2.4e-4."""
    g = json.load(open(os.path.join(GOLDEN, "near_ties_and_key_variance.json")))["near_ties"]
    K = np.array(g["keys"], float)[:, None]
    mu = np.array([float(_frac(c)) for c in g["centroids"]])[:, None]
    _, _, d1, _ = O.assign(K, mu)
    for key, c, want in g["expected"]["allowed_tests"]:
        got = O.assignment_allowed(K[key:key + 1], mu, np.array([c]), d1[key:key + 1])
        assert bool(got[0]) is want, (key, c)
    # the minimum itself is always allowed
    assert O.assignment_allowed(K, mu, np.array(g["expected"]["assign"]), d1).all()


def test_key_variance_is_centred_on_the_new_mean():
    """kvar of a cluster whose mean (2, 2/3) is not its cached centroid (2, 1): 7/9 around the
    mean (5/6 around the cached centroid would be wrong); a single-key cluster and an empty
    one have zero variance, and the empty one keeps its cached centroid."""
    from fractions import Fraction
    g = json.load(open(os.path.join(GOLDEN, "near_ties_and_key_variance.json")))["variance"]
    e = g["expected"]
    K = np.array(g["keys"], float)
    mu0 = np.array(g["mu0"], float)
    st = O.reassign_step(K, np.zeros_like(K), mu0, np.zeros((1, 1), np.uint8), 4, "f64")
    assert st["assign"].tolist() == e["assign"]
    assert st["sizes"].tolist() == e["sizes"]
    want_mu = np.array([[float(Fraction(x)) for x in row] for row in e["mu1"]])
    np.testing.assert_allclose(st["mu1_exact"], want_mu, rtol=1e-15)
    np.testing.assert_allclose(st["kvar"], [float(Fraction(x)) for x in e["kvar"]], rtol=1e-14,
                               atol=0)

"""fp64 reference definitions (test infrastructure only; see the package docstring).

Notation (one attention head at a time):
  N tokens, head dim d, query block size B, nb = ceil(N / B) query blocks,
  key block size S (`kblock`, default S = B), nkb = ceil(N / S) key blocks, blk(j) = j // S,
  C clusters, mask[b][kb] != 0 when key block kb is computed exactly for query block b
  (mask is nb x nkb), E_b = {kb : mask[b][kb] != 0}, scale = 1 / sqrt(d) unless given.

Key blocks smaller than the query block (S = B/2, B/4, ...) are the finer exact granularity
of the Accurate Block Attention (AB-Attention) abstract, whose kernel packs key/value blocks
smaller than a tile into full tensor-core tiles. Nothing else changes: every key outside
E_b's key blocks is compensated by its cluster, so the counts n[b][c] are taken over keys,
whatever the key block size.

Every array handed in is already the exact value of the stored tensor (bf16 or fp32)
widened to float64; `to_f64` does that widening for the storage formats used here.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

# Relative top-two gap below which two centroids count as tied (squared distances).
TIE_BAND = 1e-4


def default_scale(d: int) -> float:
    """Softmax temperature of standard scaled dot-product attention, 1/sqrt(d)."""
    return 1.0 / math.sqrt(d)


# ----------------------------------------------------------------------------- storage
def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements: bf16 bit patterns (uint16) or float32."""
    if dtype == "bf16":
        bits = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f64"):
        return np.asarray(stored, dtype=np.float64)
    raise ValueError(dtype)


def storage_round(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the cache storage format (nearest, ties to even) and
    return them as float64. bf16 keeps 8 significant bits with float32's exponent range;
    'f64' means no rounding (used by hand-worked examples).

    The cache (centroid keys and mean values) is held in the plan's element type, so
    the next step's distances use exactly the stored values."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                      # |x| in [2^(e-1), 2^e)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))  # 8 significant bits; bf16 subnormal step
    r = np.rint(x[nz] / ulp) * ulp               # np.rint: round half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.sign(r) * np.inf, r)   # past bf16's range
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


# ----------------------------------------------------------------------------- assignment
def _sqdist_exact(k: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """sum_i (k_i - mu_i)^2, row by row, in difference form (k and mu have <= 24-bit
    significands, so differences and squares are exact in float64)."""
    diff = k - mu
    return np.einsum("ij,ij->i", diff, diff)


def assign(K: np.ndarray, mu: np.ndarray, chunk: int = 8192
           ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Nearest cached centroid of every key (the reassignment of the Reassign Cache
    sentence of the DecoupAttn abstract; Lloyd's nearest-codeword step).

    Returns (a, gap, d1, d2): a[j] = lowest c attaining min_c ||k_j - mu_c||^2,
    d1/d2 = smallest and second-smallest squared distances (with multiplicity), and
    gap = (d2 - d1) / d2 (0 when both are 0).

    Candidates are screened with the expanded form ||k||^2 - 2 k.mu + ||mu||^2, then
    every centroid that could be first or second is re-measured in difference form, so
    d1, d2 and the tie-break are exact up to the final float64 rounding of a sum."""
    K = np.asarray(K, np.float64)
    mu = np.asarray(mu, np.float64)
    n, c = K.shape[0], mu.shape[0]
    a = np.empty(n, np.int64)
    d1 = np.empty(n)
    d2 = np.full(n, np.inf)
    mu2 = np.einsum("ij,ij->i", mu, mu)
    for s in range(0, n, chunk):
        k = K[s:s + chunk]
        k2 = np.einsum("ij,ij->i", k, k)
        dexp = k2[:, None] - 2.0 * (k @ mu.T) + mu2[None, :]
        tol = 1e-12 * (k2 + mu2.max()) + 1e-300
        if c == 1:
            rows, cols = np.arange(len(k)), np.zeros(len(k), np.int64)
        else:
            e2 = np.partition(dexp, 1, axis=1)[:, 1]
            rows, cols = np.nonzero(dexp <= (e2 + tol)[:, None])
        dx = _sqdist_exact(k[rows], mu[cols])
        order = np.lexsort((cols, dx, rows))          # by row, then distance, then index
        rows, cols, dx = rows[order], cols[order], dx[order]
        first = np.ones(len(rows), bool)
        first[1:] = rows[1:] != rows[:-1]
        fi = np.nonzero(first)[0]
        a[s + rows[fi]] = cols[fi]
        d1[s + rows[fi]] = dx[fi]
        second = fi + 1
        ok = second < len(rows)
        ok[ok] = rows[second[ok]] == rows[fi[ok]]
        d2[s + rows[fi[ok]]] = dx[second[ok]]
    with np.errstate(invalid="ignore", divide="ignore"):
        gap = np.where(d2 > 0, (d2 - d1) / d2, 0.0)
    gap[~np.isfinite(d2)] = np.inf                    # a single centroid: never tied
    return a, gap, d1, d2


def assignment_allowed(K: np.ndarray, mu: np.ndarray, a_test: np.ndarray,
                       d1: np.ndarray) -> np.ndarray:
    """Whether each a_test[j] is within the tie band: D(a_test) - D_min <= 1e-4 D(a_test)."""
    K = np.asarray(K, np.float64)
    d = _sqdist_exact(K, np.asarray(mu, np.float64)[np.asarray(a_test, np.int64)])
    return (d - d1) <= TIE_BAND * d


# ----------------------------------------------------------------------------- refresh
def qblock_counts_direct(a: np.ndarray, mask: np.ndarray, block: int, clusters: int,
                         kblock: Optional[int] = None) -> np.ndarray:
    """n[b][c] = number of keys j with a_j = c whose key block is NOT exact for query block b.

    These are the keys that cluster c stands in for when query block b is attended (the
    exact blocks stay fixed while every other key is compensated, per the abstract).
    Key j lies in key block j // S (S = kblock, default the query block size B)."""
    n_tok = len(a)
    nb = mask.shape[0]
    blk = np.arange(n_tok) // (block if kblock is None else kblock)
    out = np.zeros((nb, clusters), np.int64)
    for b in range(nb):
        outside = mask[b][blk] == 0
        out[b] = np.bincount(a[outside], minlength=clusters)
    return out


def key_variance(K: np.ndarray, a: np.ndarray, mu1_exact: np.ndarray) -> np.ndarray:
    """Isotropic spread of each cluster's keys around their mean:
    kvar[c] = (1 / (N_c d)) sum_{j : a_j = c} ||k_j - mu_c||^2 (0 for an empty cluster).

    The second moment a variance-based correction of the cluster representative's weight
    needs (ESTRA abstract, the sentence on the variance-based correction; the pages give no
    formula, see `forward`)."""
    K = np.asarray(K, np.float64)
    c, d = mu1_exact.shape
    sq = np.zeros(c)
    np.add.at(sq, a, ((K - mu1_exact[a]) ** 2).sum(axis=1))
    n = np.bincount(a, minlength=c)
    out = np.zeros(c)
    has = n > 0
    out[has] = sq[has] / (n[has] * d)
    return out


def refresh(K: np.ndarray, V: np.ndarray, a: np.ndarray, mu0: np.ndarray,
            mask: np.ndarray, block: int, dtype: str, kblock: Optional[int] = None
            ) -> Dict[str, np.ndarray]:
    """Refresh of the compensation after reassignment (Reassign Cache sentence).

    sizes[c] = #{j : a_j = c}
    mu1[c]   = mean of the keys assigned to c, or the cached mu0[c] if none are
    vbar[c]  = mean of the values of those keys, or 0 if none are
    counts   = qblock_counts_direct(a, mask)
    Both means are returned unrounded (mu1_exact, vbar_exact) and rounded to the cache
    storage format (mu1, vbar), which is what the next step and the forward consume."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    mu0 = np.asarray(mu0, np.float64)
    c, d = mu0.shape
    sizes = np.bincount(a, minlength=c).astype(np.int64)
    ksum = np.zeros((c, d))
    vsum = np.zeros((c, d))
    np.add.at(ksum, a, K)
    np.add.at(vsum, a, V)
    has = sizes > 0
    mu1 = mu0.copy()
    mu1[has] = ksum[has] / sizes[has, None]
    vbar = np.zeros((c, d))
    vbar[has] = vsum[has] / sizes[has, None]
    return {
        "sizes": sizes,
        "mu1_exact": mu1,
        "vbar_exact": vbar,
        "mu1": storage_round(mu1, dtype),
        "vbar": storage_round(vbar, dtype),
        "counts": qblock_counts_direct(a, mask, block, c, kblock),
        "kvar": key_variance(K, a, mu1),
    }


def reassign_step(K: np.ndarray, V: np.ndarray, mu0: np.ndarray, mask: np.ndarray,
                  block: int, dtype: str, kblock: Optional[int] = None
                  ) -> Dict[str, np.ndarray]:
    """One Reassign Cache step: assign every key to the cached centroids, then refresh."""
    a, gap, d1, d2 = assign(K, mu0)
    out = refresh(K, V, a, mu0, mask, block, dtype, kblock)
    out.update(assign=a, gap=gap, d1=d1, d2=d2)
    return out


# ----------------------------------------------------------------------------- forward
def _exact_keys(mask_row: np.ndarray, block: int, n_tok: int) -> np.ndarray:
    kbs = np.nonzero(mask_row)[0]
    if len(kbs) == 0:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(kb * block, min(n_tok, (kb + 1) * block))
                           for kb in kbs]).astype(np.int64)


def forward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mu: np.ndarray, vbar: np.ndarray,
            counts: np.ndarray, mask: np.ndarray, block: int, scale: Optional[float] = None,
            qblocks: Optional[Sequence[int]] = None, kblock: Optional[int] = None,
            kvar: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decoupled sparse attention output of one head (abstract: exact attention on a few
    position-fixed blocks, semantic clusters compensating every other key, one softmax).

    For query i in block b:
      exact logits   s_j = scale * q_i . k_j            for every key j in E_b's key blocks
      cluster logits t_c = scale * q_i . mu_c + ln n[b][c]   for every c with n[b][c] > 0
      o_i   = (sum_j e^{s_j - m} v_j + sum_c e^{t_c - m} vbar_c) / (sum of the same weights)
      lse_i = m + ln(sum of weights), m = the largest logit.
    The ln-count bias gives cluster c the weight of its n[b][c] stand-in keys.

    With `kvar` (per-cluster key variance, `key_variance`), each cluster logit gains
      + 0.5 * scale^2 * kvar[c] * ||q_i||^2,
    the second-order correction of the representative's weight: for keys spread around mu_c
    with covariance kvar[c] * I, the mean of exp(scale q.k) over them is
    exp(scale q.mu_c + 0.5 scale^2 q^T Sigma q) exactly for Gaussian keys and to second
    order otherwise (Jensen: the plain representative underweights a spread cluster). This
    is the reading taken for the variance-based correction the ESTRA abstract names without
    a formula.

    Returns (O [N][d], lse [N]); rows of query blocks not in `qblocks` are NaN."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    mu, vbar = np.asarray(mu, np.float64), np.asarray(vbar, np.float64)
    n_tok, d = Q.shape
    nb = mask.shape[0]
    scale = default_scale(d) if scale is None else scale
    O = np.full((n_tok, d), np.nan)
    lse = np.full(n_tok, np.nan)
    for b in (range(nb) if qblocks is None else qblocks):
        rows = slice(b * block, min(n_tok, (b + 1) * block))
        q = Q[rows]
        ex = _exact_keys(mask[b], block if kblock is None else kblock, n_tok)
        cs = np.nonzero(counts[b] > 0)[0]
        comp = scale * (q @ mu[cs].T) + np.log(counts[b, cs].astype(np.float64))[None, :]
        if kvar is not None:
            qq = (q * q).sum(axis=1)
            comp = comp + 0.5 * scale * scale * qq[:, None] * np.asarray(kvar, np.float64)[cs][None, :]
        logits = np.concatenate([scale * (q @ K[ex].T), comp], axis=1)
        vals = np.concatenate([V[ex], vbar[cs]], axis=0)
        m = logits.max(axis=1, keepdims=True)
        w = np.exp(logits - m)
        tot = w.sum(axis=1)
        O[rows] = (w @ vals) / tot[:, None]
        lse[rows] = m[:, 0] + np.log(tot)
    return O, lse


def forward_substituted(Q: np.ndarray, K: np.ndarray, V: np.ndarray, a: np.ndarray,
                        mu: np.ndarray, vbar: np.ndarray, mask: np.ndarray, block: int,
                        scale: Optional[float] = None, kblock: Optional[int] = None
                        ) -> np.ndarray:
    """Brute force for tiny inputs: for query block b, every key outside E_b's key blocks is
    replaced by its cluster's centroid key and mean value, then plain softmax attention
    runs over all N (substituted) keys. Same quantity as `forward`, built per key."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    mu, vbar = np.asarray(mu, np.float64), np.asarray(vbar, np.float64)
    n_tok, d = Q.shape
    scale = default_scale(d) if scale is None else scale
    O = np.empty((n_tok, d))
    kb_size = block if kblock is None else kblock
    for i in range(n_tok):
        b = i // block
        Kt = np.empty_like(K)
        Vt = np.empty_like(V)
        for j in range(n_tok):
            if mask[b][j // kb_size]:
                Kt[j], Vt[j] = K[j], V[j]
            else:
                Kt[j], Vt[j] = mu[a[j]], vbar[a[j]]
        s = scale * (Kt @ Q[i])
        w = np.exp(s - s.max())
        O[i] = (w @ Vt) / w.sum()
    return O


def dense_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                    scale: Optional[float] = None) -> np.ndarray:
    """softmax(scale Q K^T) V, the full attention the method approximates."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    scale = default_scale(Q.shape[1]) if scale is None else scale
    s = scale * (Q @ K.T)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ V) / w.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------- Lloyd
def objective(K: np.ndarray, mu: np.ndarray, a: np.ndarray) -> float:
    """Lloyd's quantisation error: sum_j ||k_j - mu_{a_j}||^2."""
    return float(_sqdist_exact(np.asarray(K, np.float64),
                               np.asarray(mu, np.float64)[a]).sum())


def lloyd_warmup(K: np.ndarray, mu_init: np.ndarray, iters: int, dtype: str) -> np.ndarray:
    """`iters` Lloyd iterations (assign, then move every non-empty centroid to the mean of
    its keys, rounded to the cache format). Stands in for the offline calibration that
    produces the cached centroids; returns the cache in float64."""
    mu = storage_round(np.asarray(mu_init, np.float64), dtype)
    K = np.asarray(K, np.float64)
    for _ in range(iters):
        a = assign(K, mu)[0]
        sizes = np.bincount(a, minlength=mu.shape[0])
        ksum = np.zeros_like(mu)
        np.add.at(ksum, a, K)
        has = sizes > 0
        new = mu.copy()
        new[has] = ksum[has] / sizes[has, None]
        mu = storage_round(new, dtype)
    return mu

"""Shared helpers for the GPU parity tests: moving seeded inputs to the device, running
the oracle per head, and the comparison rules.

Tolerances (floating point):
  forward, bf16 inputs: max-abs <= 2e-2 and rel-L2 <= 5e-3 over all compared rows
  forward, fp32 inputs: rel-L2 <= 1e-5
  refreshed cache, bf16: |gpu - exact mean| <= 1 bf16 ulp of the oracle's rounded value + 1e-6
  refreshed cache, fp32: |gpu - exact mean| <= 1e-5 * rms of the cluster's member keys
Integer results (assignments outside the tie band, sizes, counts) must match exactly.
"""
from __future__ import annotations

import sys
from typing import Dict, Iterable, List, Optional

import numpy as np

import oracle as O
from datagen import bf16_bits_to_f32, f32_to_bf16_bits

FWD_TOL = {"bf16": dict(max_abs=2e-2, rel_l2=5e-3), "f32": dict(max_abs=None, rel_l2=1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(stored: np.ndarray, dtype: str):
    """Stored numpy array (uint16 bf16 bits or float32) -> device tensor of that dtype."""
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(stored, np.uint16).view(np.int16))
        return t.cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(stored, np.float32)).cuda()


def from_dev(t, dtype: str) -> np.ndarray:
    """Device tensor -> exact float64 values."""
    torch = torch_mod()
    if dtype == "bf16":
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def store64(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values that are exactly representable in `dtype` -> stored numpy array."""
    x32 = np.asarray(x64, np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def check_forward(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    tol = FWD_TOL[dtype]
    r = rel_l2(got, want)
    m = float(np.max(np.abs(got - want))) if got.size else 0.0
    say(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= tol["rel_l2"], f"{what}: rel-L2 {r:.3e} > {tol['rel_l2']}"
    if tol["max_abs"] is not None:
        assert m <= tol["max_abs"], f"{what}: max-abs {m:.3e} > {tol['max_abs']}"
    return r, m


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (np.maximum(e, -126) - 7), 2.0 ** -133)


def check_reassign_head(K64, V64, mu0_64, mask, block, dtype, gpu: Dict[str, np.ndarray],
                        what: str, kblock: Optional[int] = None,
                        ref: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, int]:
    """Compare one head's GPU reassign outputs with the oracle's (same inputs).

    Assignments: identical wherever the oracle's top-two gap is >= 1e-4 (relative);
    inside the band the GPU's choice must be within 1e-4 of the minimum. Sizes, counts
    and means are compared exactly/within tolerance on every cluster that no
    band-disagreeing key touches; touched clusters get the sum and bound checks. `ref` is the
    oracle's step when it was computed elsewhere (see `OraclePool`)."""
    if ref is None:
        ref = O.reassign_step(K64, V64, mu0_64, mask, block, dtype, kblock=kblock)
    a_gpu = gpu["assign"].astype(np.int64)
    a_ref = ref["assign"]
    diff = a_gpu != a_ref
    outside = ref["gap"] >= O.TIE_BAND
    bad = diff & outside
    assert not bad.any(), (f"{what}: {int(bad.sum())} assignments differ outside the tie band "
                           f"(first keys {np.nonzero(bad)[0][:8].tolist()})")
    if diff.any():
        ok = O.assignment_allowed(K64[diff], mu0_64, a_gpu[diff], ref["d1"][diff])
        assert ok.all(), f"{what}: in-band assignment not within the band"
    touched = np.zeros(mu0_64.shape[0], bool)
    touched[a_gpu[diff]] = True
    touched[a_ref[diff]] = True
    keep = ~touched
    sizes = gpu["sizes"].astype(np.int64)
    assert sizes.sum() == K64.shape[0]
    np.testing.assert_array_equal(sizes[keep], ref["sizes"][keep], err_msg=f"{what}: sizes")
    np.testing.assert_array_equal(sizes, np.bincount(a_gpu, minlength=len(sizes)),
                                  err_msg=f"{what}: sizes vs own assignments")
    cnt = gpu["counts"].astype(np.int64)
    np.testing.assert_array_equal(cnt[:, keep], ref["counts"][:, keep], err_msg=f"{what}: counts")
    moved = np.bincount(a_gpu[diff], minlength=len(sizes)) + np.bincount(
        a_ref[diff], minlength=len(sizes))
    assert np.all(np.abs(cnt - ref["counts"]) <= moved[None, :]), f"{what}: counts bound"
    assert np.all(cnt >= 0) and np.all(cnt <= sizes[None, :]), f"{what}: counts range"
    np.testing.assert_array_equal(cnt.sum(axis=1), ref["counts"].sum(axis=1),
                                  err_msg=f"{what}: keys outside exact blocks per query block")
    for name, exact, rounded in (("centroids", ref["mu1_exact"], ref["mu1"]),
                                 ("mean_values", ref["vbar_exact"], ref["vbar"])):
        g = gpu[name][keep]
        e = exact[keep]
        if dtype == "bf16":
            lim = bf16_ulp(rounded[keep]) + 1e-6
        else:
            rms = np.sqrt(np.maximum(np.mean(e ** 2, axis=1, keepdims=True), 1e-30))
            lim = 1e-5 * np.maximum(rms, 1e-3) + 1e-7
        err = np.abs(g - e)
        assert np.all(err <= lim), f"{what}: {name} off by {float((err / lim).max()):.2f} x tol"
    if "variance" in gpu:
        # fp32 sum of squared norms minus the squared fp32 mean: the error scales with the
        # clusters' mean squared key element, sum ||k||^2 / (n d) = kvar + ||mean||^2 / d
        ms = ref["kvar"] + (ref["mu1_exact"] ** 2).sum(axis=1) / ref["mu1_exact"].shape[1]
        lim = 3e-5 * ms[keep] + 1e-9
        err = np.abs(gpu["variance"].astype(np.float64)[keep] - ref["kvar"][keep])
        assert np.all(err <= lim), f"{what}: variance off by {float((err / lim).max()):.2f} x tol"
        assert np.all(gpu["variance"] >= 0), f"{what}: negative variance"
    return {"band_moves": int(diff.sum()), "keys": int(K64.shape[0]), "ref": ref}


def oracle_forward_heads(L64: Dict[str, np.ndarray], caches: Dict[int, Dict[str, np.ndarray]],
                         mask: np.ndarray, block: int, heads: Iterable[int],
                         qblocks: Optional[Dict[int, List[int]]] = None,
                         kblock: Optional[int] = None):
    """Oracle outputs for selected heads (and optionally selected query blocks)."""
    out = {}
    for h in heads:
        c = caches[h]
        mh = mask[0] if mask.shape[0] == 1 else mask[h]
        qb = None if qblocks is None else qblocks[h]
        out[h] = O.forward(L64["Q"][h], L64["K"][h], L64["V"][h], c["mu1"], c["vbar"],
                           c["counts"], mh, block, qblocks=qb, kblock=kblock)
    return out


def rows_of(qblocks: List[int], block: int, n: int) -> np.ndarray:
    return np.concatenate([np.arange(b * block, min(n, (b + 1) * block)) for b in qblocks])


# ----------------------------------------------------------------------------- oracle pool
# Full-size layers have tens of heads: the oracle runs them in CPU worker processes (spawned,
# one BLAS thread each; they never touch the GPU) while the test process drives the GPU.
# A worker regenerates its head from the seeded generator (and its drift steps) instead of
# receiving the tensors, so only caches, counts and masks cross the process boundary.
_REF_KEYS = ("assign", "gap", "d1", "d2", "sizes", "counts", "mu1", "vbar", "mu1_exact",
             "vbar_exact", "kvar")
_HEAD_CACHE = {}


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _head(cfg, head: int, drift_steps: int):
    """Stored Q, K, V of one head after `drift_steps` drift steps (as drift_layer makes them)."""
    key = (cfg, head, drift_steps)
    if key not in _HEAD_CACHE:
        from datagen.video_layers import apply_drift, head_tensors
        t = head_tensors(cfg, head)
        for step in range(drift_steps):
            for which, on in (("K", cfg.drift_k), ("V", cfg.drift_v)):
                if on:
                    t[which] = apply_drift(cfg, t[which], head, step, which)
        _HEAD_CACHE.clear()
        _HEAD_CACHE[key] = t
    return _HEAD_CACHE[key]


def _reassign_task(args):
    cfg, head, drift_steps, mu0, mask = args
    t = _head(cfg, head, drift_steps)
    dt = cfg.dtype
    ref = O.reassign_step(O.to_f64(t["K"], dt), O.to_f64(t["V"], dt), O.to_f64(mu0, dt), mask,
                          cfg.block, dt, kblock=cfg.kblock)
    return {k: ref[k] for k in _REF_KEYS}


def _forward_task(args):
    cfg, head, drift_steps, mu1, vbar, counts, mask, qblocks = args[:8]
    kvar = args[8] if len(args) > 8 else None
    t = _head(cfg, head, drift_steps)
    dt = cfg.dtype
    o, _ = O.forward(O.to_f64(t["Q"], dt), O.to_f64(t["K"], dt), O.to_f64(t["V"], dt), mu1, vbar,
                     counts, mask, cfg.block, qblocks=qblocks, kblock=cfg.kblock, kvar=kvar)
    return o[rows_of(qblocks, cfg.block, cfg.seq_len)]


class OraclePool:
    """Oracle steps of many heads of a generated layer, in parallel CPU processes."""

    def __init__(self, workers: Optional[int] = None):
        import multiprocessing as mp
        import os
        from concurrent.futures import ProcessPoolExecutor
        n = workers or max(1, min(12, (os.cpu_count() or 2) - 2))
        self.ex = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                                      initializer=_one_blas_thread)

    def reassign(self, tasks):
        """tasks: (cfg, head, drift_steps, mu0 stored [C][d], mask [nb][nkb]) each."""
        return list(self.ex.map(_reassign_task, tasks))

    def forward(self, tasks):
        """tasks: (cfg, head, drift_steps, mu1, vbar (float64), counts, mask, qblocks[, kvar])
        each; returns the oracle's output rows of each task's query blocks."""
        return list(self.ex.map(_forward_task, tasks))

    def close(self):
        self.ex.shutdown()

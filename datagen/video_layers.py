"""Synthetic video-DiT attention layers (Q, K, V, block masks, drift, cache seeds).

Token t of a T x Hs x Ws latent lives in frame-major raster order:
frame f = t // (Hs*Ws), row r = (t // Ws) % Hs, column w = t % Ws.

Per head, G mixture centres are drawn from N(0, I_d); every token draws a component
uniformly, and K_t = centre + sigma * N(0, I), Q_t likewise with its own component and
noise draws (K and Q share the head's centres); V ~ N(0, I). Values are produced in
float32 and stored in the layer's dtype (bf16 by round-to-nearest-even, or float32).

Optional shared offset (`key_offset` s, 0 in every named workload): every mixture centre
gains s in every dimension, so Q and K sit far from the origin (|k|^2 about d (1 + s^2))
while their spread stays sigma. It draws nothing, so the offset layer's noise is the plain
layer's; it exercises distance arithmetic whose rounding grows with |k|^2 rather than with
the distances themselves.

Every random stream is seeded with numpy's SeedSequence over the tuple
(config id, head, stream, step), so any single head can be regenerated on its own.
Streams: 0 centres, 1 K components, 2 K noise, 3 Q components, 4 Q noise, 5 V,
6 K drift, 7 V drift, 8 mask, 9 cache seed.

The mask is a plan input: position-fixed exact key blocks per query block. Three kinds:
  * "random": the diagonal block plus (k - 1) distinct seeded other blocks per row;
  * "local": the k key blocks nearest in a 3D sense, distance^2 between the query block's
    centre and the key block's centre (S*df)^2 + dr^2 + dw^2 with S = Hs / 4, ties to the
    smaller block index; optionally every key block holding a token of frame 0 is kept
    first ("first-frame" blocks). Key blocks may be smaller than query blocks
    (`key_block`); k then counts key blocks of that size. With `local_rule="reach"` the
    distance of a key block is instead that from its centre to the nearest token of the
    query block (the keys within reach of some query, not of the block's centre: for key
    blocks shorter than the query block the centre rule keeps a ball that misses the keys
    near the query block's ends);
  * "local_budget": the same nearest-block rule with a budget k[h][b] per head and query
    block (one mask per head). Budgets are k times a head factor and a block factor, each
    log-uniform in [1/2, 2] and seeded per head, rescaled so their mean over the layer is
    k, rounded and clipped to [1, nb]: the shape of a per-head, per-block budget allocation
    such as the pages' Distortion Budget produces, with synthetic numbers.

Nothing here computes attention, distances to centroids, cluster means or counts.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional

import numpy as np

STREAM_CENTRES, STREAM_KCOMP, STREAM_KNOISE, STREAM_QCOMP, STREAM_QNOISE = 0, 1, 2, 3, 4
STREAM_V, STREAM_KDRIFT, STREAM_VDRIFT, STREAM_MASK, STREAM_CACHE = 5, 6, 7, 8, 9


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    heads: int
    frames: int
    height: int
    width: int
    head_dim: int
    block: int
    clusters: int
    mask_kind: str          # "random" | "local" | "local_budget"
    blocks_per_row: int     # k = |E_b| (the mean budget for "local_budget")
    first_frame: bool       # force blocks holding frame-0 tokens (local masks only)
    mixture: int            # G
    sigma: float
    dtype: str              # "bf16" | "f32"
    steps: int              # denoising steps with drift (0 = no drift)
    drift_k: bool
    drift_v: bool
    drift_sigma: float = 0.05
    description: str = ""
    key_block: int = 0      # exact key block size (0: the query block size)
    key_offset: float = 0.0     # added to every coordinate of every mixture centre
    local_rule: str = "centre"  # key block distance for "local" masks: "centre" | "reach"

    @property
    def seq_len(self) -> int:
        return self.frames * self.height * self.width

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def kblock(self) -> int:
        return self.key_block or self.block

    @property
    def num_key_blocks(self) -> int:
        return -(-self.seq_len // self.kblock)

    @property
    def local_scale(self) -> float:
        return self.height / 4.0

    def with_heads(self, heads: int) -> "LayerConfig":
        return dataclasses.replace(self, heads=heads)


CONFIGS: Dict[str, LayerConfig] = {
    "tiny_f32": LayerConfig(
        "tiny_f32", 1, heads=1, frames=4, height=16, width=16, head_dim=64, block=64,
        clusters=16, mask_kind="random", blocks_per_row=4, first_frame=False, mixture=16,
        sigma=0.3, dtype="f32", steps=1, drift_k=True, drift_v=False,
        description="1 head, N=1024 (4x16x16), d=64, block 64, C=16, diagonal + 3 random "
                    "blocks, one reassign step after K drift"),
    "small_bf16": LayerConfig(
        "small_bf16", 2, heads=12, frames=4, height=32, width=32, head_dim=64, block=64,
        clusters=64, mask_kind="local", blocks_per_row=16, first_frame=False, mixture=64,
        sigma=0.3, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        description="12 heads, N=4096 (4x32x32), d=64, block 64, C=64, 25% 3D-local mask"),
    "wan14b_bf16": LayerConfig(
        "wan14b_bf16", 3, heads=40, frames=21, height=45, width=80, head_dim=128, block=128,
        clusters=256, mask_kind="local", blocks_per_row=59, first_frame=True, mixture=256,
        sigma=0.25, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        description="40 heads, N=75600 (21x45x80), d=128, block 128, C=256, 10% 3D-local "
                    "+ first-frame mask"),
    "hunyuan13b_bf16": LayerConfig(
        "hunyuan13b_bf16", 4, heads=24, frames=33, height=45, width=80, head_dim=128,
        block=128, clusters=512, mask_kind="local", blocks_per_row=46, first_frame=False,
        mixture=256, sigma=0.25, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        description="24 heads, N=118800 (33x45x80), d=128, block 128, C=512, 5% 3D-local "
                    "mask"),
    "small_budget_bf16": LayerConfig(
        "small_budget_bf16", 6, heads=6, frames=8, height=32, width=32, head_dim=128,
        block=128, clusters=128, mask_kind="local_budget", blocks_per_row=12,
        first_frame=False, mixture=64, sigma=0.3, dtype="bf16", steps=0, drift_k=False,
        drift_v=False,
        description="6 heads, N=8192 (8x32x32), d=128, block 128, C=128, per-head and "
                    "per-block budgets around 12 of 64 key blocks (3D-local)"),
    "hunyuan13b_budget_bf16": LayerConfig(
        "hunyuan13b_budget_bf16", 7, heads=24, frames=33, height=45, width=80, head_dim=128,
        block=128, clusters=512, mask_kind="local_budget", blocks_per_row=46,
        first_frame=False, mixture=256, sigma=0.25, dtype="bf16", steps=0, drift_k=False,
        drift_v=False,
        description="13B-class layer with per-head and per-block budgets averaging 46 of "
                    "929 key blocks (5% density), one 3D-local mask per head"),
    "small_sub32_bf16": LayerConfig(
        "small_sub32_bf16", 8, heads=4, frames=8, height=32, width=32, head_dim=128,
        block=128, clusters=128, mask_kind="local", blocks_per_row=48, first_frame=False,
        mixture=64, sigma=0.3, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_block=32,
        local_rule="reach",
        description="4 heads, N=8192 (8x32x32), d=128, query blocks of 128, exact key blocks "
                    "of 32: the 48 nearest to some token of each query block (18.75%, "
                    "3D-local)"),
    "small_sub16_d64_bf16": LayerConfig(
        "small_sub16_d64_bf16", 9, heads=3, frames=3, height=30, width=30, head_dim=64,
        block=128, clusters=64, mask_kind="local", blocks_per_row=48, first_frame=True,
        mixture=64, sigma=0.3, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_block=16,
        description="3 heads, N=2700 (3x30x30, ragged at both block sizes), d=64, query "
                    "blocks of 128, exact key blocks of 16: first frame + nearest, 48 per "
                    "query block"),
    "tiny_sub_f32": LayerConfig(
        "tiny_sub_f32", 10, heads=1, frames=4, height=15, width=17, head_dim=64, block=64,
        clusters=16, mask_kind="local", blocks_per_row=16, first_frame=False, mixture=16,
        sigma=0.3, dtype="f32", steps=0, drift_k=False, drift_v=False, key_block=16,
        description="1 head, N=1020 (4x15x17), d=64, query blocks of 64, exact key blocks of "
                    "16 (16 nearest per query block), fp32"),
    "hunyuan13b_sub32_bf16": LayerConfig(
        "hunyuan13b_sub32_bf16", 11, heads=24, frames=33, height=45, width=80, head_dim=128,
        block=128, clusters=512, mask_kind="local", blocks_per_row=184, first_frame=False,
        mixture=256, sigma=0.25, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_block=32,
        local_rule="reach",
        description="13B-class layer with exact key blocks of 32 keys: the 184 nearest to "
                    "some token of each query block of 128, the same 5% of keys as 46 "
                    "blocks of 128"),
    "hunyuan13b_sub64_bf16": LayerConfig(
        "hunyuan13b_sub64_bf16", 12, heads=24, frames=33, height=45, width=80, head_dim=128,
        block=128, clusters=512, mask_kind="local", blocks_per_row=92, first_frame=False,
        mixture=256, sigma=0.25, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_block=64,
        local_rule="reach",
        description="13B-class layer with exact key blocks of 64 keys: the 92 nearest to "
                    "some token of each query block of 128 (5% of keys)"),
    "long_video_bf16": LayerConfig(
        "long_video_bf16", 13, heads=1, frames=129, height=72, width=111, head_dim=128,
        block=128, clusters=512, mask_kind="local", blocks_per_row=46, first_frame=False,
        mixture=256, sigma=0.25, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        description="1 head, N=1030968 (129x72x111, a ragged last block of 56), d=128, "
                    "block 128, C=512, 46 3D-local blocks per query block (0.57%)"),
    "extreme_cache_bf16": LayerConfig(
        "extreme_cache_bf16", 5, heads=40, frames=21, height=45, width=80, head_dim=128,
        block=128, clusters=512, mask_kind="local", blocks_per_row=6, first_frame=False,
        mixture=256, sigma=0.25, dtype="bf16", steps=4, drift_k=True, drift_v=True,
        description="40 heads, N=75600, d=128, C=512, 1% 3D-local mask, 4 steps of K,V "
                    "drift with reassign + forward"),
    "offset_keys_bf16": LayerConfig(
        "offset_keys_bf16", 14, heads=4, frames=8, height=32, width=32, head_dim=128,
        block=128, clusters=512, mask_kind="local", blocks_per_row=12, first_frame=False,
        mixture=256, sigma=0.05, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_offset=3.0,
        description="4 heads, N=8192 (8x32x32), d=128, C=512: tight clusters (spread 0.05) "
                    "around centres shifted by 3 in every coordinate, so |k|^2 is about "
                    "1300 against nearest squared distances about 0.6"),
    "offset_keys_wide_bf16": LayerConfig(
        "offset_keys_wide_bf16", 15, heads=2, frames=8, height=32, width=32, head_dim=128,
        block=128, clusters=1024, mask_kind="local", blocks_per_row=12, first_frame=False,
        mixture=512, sigma=0.02, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_offset=8.0,
        description="2 heads, N=8192, d=128, C=1024 (more centroids than fit in LDS at "
                    "once): spread 0.02 around centres shifted by 8 (|k|^2 about 8300)"),
    "offset_keys_d64_bf16": LayerConfig(
        "offset_keys_d64_bf16", 16, heads=3, frames=4, height=32, width=32, head_dim=64,
        block=64, clusters=256, mask_kind="local", blocks_per_row=16, first_frame=False,
        mixture=128, sigma=0.03, dtype="bf16", steps=0, drift_k=False, drift_v=False,
        key_offset=4.0,
        description="3 heads, N=4096, d=64, C=256: spread 0.03 around centres shifted by 4"),
}

def get_config(name: str) -> LayerConfig:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {', '.join(CONFIGS)}")
    return CONFIGS[name]


def _rng(cfg: LayerConfig, head: int, stream: int, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.cfg_id, head, stream, step])


# ---------------------------------------------------------------- storage helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly equal float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _store(cfg: LayerConfig, x32: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x32) if cfg.dtype == "bf16" else np.ascontiguousarray(
        x32, dtype=np.float32)


def to_f32(cfg: LayerConfig, stored: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(stored) if cfg.dtype == "bf16" else np.asarray(stored, np.float32)


# ---------------------------------------------------------------- tensors
def head_tensors(cfg: LayerConfig, head: int) -> Dict[str, np.ndarray]:
    """Q, K, V of one head, [N][d] in the storage dtype (uint16 bf16 bits or float32)."""
    n, d, g = cfg.seq_len, cfg.head_dim, cfg.mixture
    sig = np.float32(cfg.sigma)
    centres = _rng(cfg, head, STREAM_CENTRES).standard_normal((g, d), dtype=np.float32)
    if cfg.key_offset:
        centres += np.float32(cfg.key_offset)
    kc = _rng(cfg, head, STREAM_KCOMP).integers(0, g, size=n)
    k = centres[kc] + sig * _rng(cfg, head, STREAM_KNOISE).standard_normal((n, d), dtype=np.float32)
    qc = _rng(cfg, head, STREAM_QCOMP).integers(0, g, size=n)
    q = centres[qc] + sig * _rng(cfg, head, STREAM_QNOISE).standard_normal((n, d), dtype=np.float32)
    v = _rng(cfg, head, STREAM_V).standard_normal((n, d), dtype=np.float32)
    return {"Q": _store(cfg, q), "K": _store(cfg, k), "V": _store(cfg, v),
            "k_component": kc.astype(np.int64)}


def drift_noise(cfg: LayerConfig, head: int, step: int, which: str) -> np.ndarray:
    """The float32 N(0, drift_sigma^2) increment applied to K or V at a denoising step."""
    stream = STREAM_KDRIFT if which == "K" else STREAM_VDRIFT
    e = _rng(cfg, head, stream, step + 1).standard_normal(
        (cfg.seq_len, cfg.head_dim), dtype=np.float32)
    return np.float32(cfg.drift_sigma) * e


def apply_drift(cfg: LayerConfig, stored: np.ndarray, head: int, step: int,
                which: str) -> np.ndarray:
    """Stored tensor of one head after one drift step (added in float32, re-stored)."""
    return _store(cfg, to_f32(cfg, stored) + drift_noise(cfg, head, step, which))


# ---------------------------------------------------------------- masks
def _token_coords(cfg: LayerConfig) -> np.ndarray:
    """(frame, row, column) of every token, float64 [N][3]."""
    n, hw, w = cfg.seq_len, cfg.height * cfg.width, cfg.width
    t = np.arange(n, dtype=np.int64)
    return np.stack([t // hw, (t // w) % cfg.height, t % w], axis=1).astype(np.float64)


def _block_centres(cfg: LayerConfig, size: Optional[int] = None) -> np.ndarray:
    """Mean (frame, row, column) of the tokens of each block of `size` tokens."""
    n = cfg.seq_len
    b = cfg.block if size is None else size
    coords = _token_coords(cfg)
    nb = -(-n // b)
    cen = np.zeros((nb, 3))
    for kb in range(nb):
        cen[kb] = coords[kb * b:min(n, (kb + 1) * b)].mean(axis=0)
    return cen


def budgets(cfg: LayerConfig) -> np.ndarray:
    """int [H][nb] exact-block budgets of a "local_budget" layer (see the module notes)."""
    nb, k = cfg.num_blocks, cfg.blocks_per_row
    f = np.empty((cfg.heads, nb))
    for h in range(cfg.heads):
        rng = _rng(cfg, h, STREAM_MASK)
        head = np.exp(rng.uniform(-math.log(2.0), math.log(2.0)))
        f[h] = head * np.exp(rng.uniform(-math.log(2.0), math.log(2.0), size=nb))
    f *= k / f.mean()
    return np.clip(np.rint(f), 1, nb).astype(np.int64)


def _local_orders(cfg: LayerConfig) -> np.ndarray:
    """[nb][nb] key blocks of each query block by 3D distance, ties to the smaller index."""
    nb = cfg.num_blocks
    cen = _block_centres(cfg)
    s = cfg.local_scale
    idx = np.arange(nb)
    out = np.empty((nb, nb), dtype=np.int64)
    for b in range(nb):
        diff = cen - cen[b]
        dist2 = (s * diff[:, 0]) ** 2 + diff[:, 1] ** 2 + diff[:, 2] ** 2
        out[b] = np.lexsort((idx, dist2))
    return out


def block_mask(cfg: LayerConfig) -> np.ndarray:
    """uint8 [1][nb][nkb] (or [H][nb][nb] for per-head budgets); nonzero = key block computed
    exactly for that query block."""
    nb, k = cfg.num_blocks, cfg.blocks_per_row
    if cfg.kblock != cfg.block and cfg.mask_kind != "local":
        raise ValueError("key blocks smaller than query blocks need a local mask")
    if not 1 <= k <= cfg.num_key_blocks:
        raise ValueError("blocks_per_row out of range")
    if cfg.mask_kind == "local_budget":
        kk = budgets(cfg)
        order = _local_orders(cfg)
        mask = np.zeros((cfg.heads, nb, nb), dtype=np.uint8)
        for h in range(cfg.heads):
            for b in range(nb):
                mask[h, b, order[b, : kk[h, b]]] = 1
        return mask
    mask = np.zeros((nb, nb), dtype=np.uint8)
    if cfg.mask_kind == "random":
        rng = _rng(cfg, 0, STREAM_MASK)
        for b in range(nb):
            others = np.array([x for x in range(nb) if x != b])
            pick = rng.choice(others, size=k - 1, replace=False)
            mask[b, b] = 1
            mask[b, pick] = 1
        return mask[None]
    if cfg.mask_kind != "local":
        raise ValueError(cfg.mask_kind)
    if cfg.local_rule not in ("centre", "reach"):
        raise ValueError(cfg.local_rule)
    nkb = cfg.num_key_blocks
    mask = np.zeros((nb, nkb), dtype=np.uint8)
    cen_q = _block_centres(cfg)
    cen = _block_centres(cfg, cfg.kblock)
    s = cfg.local_scale
    scaled = np.array([s, 1.0, 1.0])
    tok = _token_coords(cfg) * scaled
    forced = np.zeros(nkb, dtype=bool)
    if cfg.first_frame:
        hw = cfg.height * cfg.width
        forced[: (min(hw, cfg.seq_len) - 1) // cfg.kblock + 1] = True
    idx = np.arange(nkb)
    for b in range(nb):
        if cfg.local_rule == "centre":
            diff = cen - cen_q[b]
            dist2 = (s * diff[:, 0]) ** 2 + diff[:, 1] ** 2 + diff[:, 2] ** 2
        else:
            q = tok[b * cfg.block:min(cfg.seq_len, (b + 1) * cfg.block)]
            kc = cen * scaled
            d2 = ((kc[None, :, :] - q[:, None, :]) ** 2).sum(axis=2)
            dist2 = d2.min(axis=0)
        order = np.lexsort((idx, dist2))          # by distance, then by block index
        chosen = list(idx[forced][:k])
        for kb in order:
            if len(chosen) >= k:
                break
            if not forced[kb]:
                chosen.append(kb)
        mask[b, chosen] = 1
    return mask[None]


# ---------------------------------------------------------------- cache seeds
def cache_init_indices(cfg: LayerConfig, head: int) -> np.ndarray:
    """C distinct token indices (ascending) whose keys seed the head's centroid cache."""
    rng = _rng(cfg, head, STREAM_CACHE)
    return np.sort(rng.choice(cfg.seq_len, size=cfg.clusters, replace=False)).astype(np.int64)


def cache_init(cfg: LayerConfig, k_stored: np.ndarray, head: int) -> np.ndarray:
    """Seed centroids of one head: rows of the (stored) keys at cache_init_indices."""
    return np.ascontiguousarray(k_stored[cache_init_indices(cfg, head)])


# ---------------------------------------------------------------- whole layers
def make_layer(cfg: LayerConfig, heads: Optional[Iterable[int]] = None,
               threads: int = 8) -> Dict[str, np.ndarray]:
    """Q, K, V [H'][N][d] (storage dtype), mask [1][nb][nb], seed centroids [H'][C][d].

    `heads` selects a subset (default: all heads); each head is generated independently.
    """
    hs = list(range(cfg.heads)) if heads is None else list(heads)
    n, d = cfg.seq_len, cfg.head_dim
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    out = {x: np.empty((len(hs), n, d), dtype=st) for x in ("Q", "K", "V")}
    comp = np.empty((len(hs), n), dtype=np.int64)
    cache = np.empty((len(hs), cfg.clusters, d), dtype=st)

    def one(i_h):
        i, h = i_h
        t = head_tensors(cfg, h)
        for x in ("Q", "K", "V"):
            out[x][i] = t[x]
        comp[i] = t["k_component"]
        cache[i] = cache_init(cfg, t["K"], h)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, enumerate(hs)))
    out["mask"] = block_mask(cfg)
    out["cache_init"] = cache
    out["k_component"] = comp
    out["heads"] = np.array(hs, dtype=np.int64)
    return out


def drift_layer(cfg: LayerConfig, layer: Dict[str, np.ndarray], step: int,
                threads: int = 8) -> Dict[str, np.ndarray]:
    """A copy of `layer` with K (and/or V, per the config) drifted for denoising `step`."""
    new = dict(layer)
    for which, on in (("K", cfg.drift_k), ("V", cfg.drift_v)):
        if not on:
            continue
        arr = np.empty_like(layer[which])

        def one(i_h, which=which, arr=arr):
            i, h = i_h
            arr[i] = apply_drift(cfg, layer[which][i], int(h), step, which)

        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(one, enumerate(layer["heads"])))
        new[which] = arr
    return new

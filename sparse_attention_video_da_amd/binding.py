"""ctypes binding of libdecoupattn.so (argument marshalling only).

The C functions keep their names (da_plan_create, da_reassign, da_forward, ...). `Plan`
wraps a plan handle and takes device tensors from PyTorch, which is used only to own
device memory and to name the current HIP stream; every step of the computation runs in
the library's HIP kernels. There is no fallback: if the library is missing, importing
this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libdecoupattn.so")

DA_OK, DA_ERR_INVALID_ARGUMENT, DA_ERR_UNSUPPORTED, DA_ERR_OUT_OF_MEMORY, DA_ERR_DEVICE = range(5)
DA_DTYPE_F32, DA_DTYPE_BF16 = 0, 1
DTYPES = {"f32": DA_DTYPE_F32, "bf16": DA_DTYPE_BF16}

EXPORTED = ("da_plan_create", "da_plan_destroy", "da_reassign", "da_forward", "da_reassign_var",
            "da_forward_var", "da_reassign_noalloc", "da_plan_info", "da_plan_exact_lists",
            "da_validate_desc", "da_status_str", "da_version")


class da_desc(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("clusters", ctypes.c_int32), ("mask_heads", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("key_block", ctypes.c_int32)]


class DAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {da_status_str(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python sparse_attention_video_da_amd/build.py`"
            " (there is no non-HIP fallback)")
    # PyTorch ships its own HIP runtime under the same soname as the system one this library
    # links. Loading PyTorch first makes the library bind to that one runtime, so the device
    # pointers and stream handles PyTorch hands over belong to the runtime that uses them;
    # loading the library first would bring up a second runtime that PyTorch's cannot share
    # the device with.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    sig = {
        "da_plan_create": ([ctypes.POINTER(da_desc), u8p, ctypes.POINTER(vp)], ctypes.c_int),
        "da_plan_destroy": ([vp], ctypes.c_int),
        "da_reassign": ([vp] + [vp] * 9, ctypes.c_int),
        "da_forward": ([vp] + [vp] * 9, ctypes.c_int),
        "da_reassign_var": ([vp] + [vp] * 10, ctypes.c_int),
        "da_reassign_noalloc": ([vp] + [vp] * 9, ctypes.c_int),
        "da_forward_var": ([vp] + [vp] * 10, ctypes.c_int),
        "da_plan_info": ([vp, i32p, i64p, i64p], ctypes.c_int),
        "da_plan_exact_lists": ([vp, ctypes.c_int32, i32p, i32p], ctypes.c_int),
        "da_validate_desc": ([ctypes.POINTER(da_desc), u8p], ctypes.c_int),
        "da_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "da_version": ([], ctypes.c_int32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    return lib


_lib = _load()


# ------------------------------------------------------------------------ raw C calls
def da_status_str(status: int) -> str:
    return _lib.da_status_str(int(status)).decode()


def da_version() -> int:
    return int(_lib.da_version())


def make_desc(heads: int, seq_len: int, head_dim: int, block: int, clusters: int,
              dtype: str = "bf16", mask_heads: int = 1, scale: float = 0.0,
              key_block: int = 0) -> da_desc:
    return da_desc(heads, seq_len, head_dim, block, clusters, mask_heads,
                   DTYPES.get(dtype, dtype) if isinstance(dtype, str) else int(dtype), scale,
                   key_block)


def _mask_ptr(mask: Optional[np.ndarray]):
    if mask is None:
        return None, None
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    return m, m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def da_validate_desc(desc: Optional[da_desc], mask: Optional[np.ndarray]) -> int:
    m, mp = _mask_ptr(mask)
    return int(_lib.da_validate_desc(ctypes.byref(desc) if desc is not None else None, mp))


def da_plan_create(desc: da_desc, mask: np.ndarray):
    """Returns (status, handle)."""
    m, mp = _mask_ptr(mask)
    h = ctypes.c_void_p()
    st = _lib.da_plan_create(ctypes.byref(desc), mp, ctypes.byref(h))
    return int(st), h


def da_plan_destroy(handle) -> int:
    return int(_lib.da_plan_destroy(handle))


def da_reassign(handle, K, V, centroids_in, centroids_out, mean_values_out, assign_out,
                cluster_sizes_out, qblock_counts_out, stream) -> int:
    return int(_lib.da_reassign(handle, K, V, centroids_in, centroids_out, mean_values_out,
                                assign_out, cluster_sizes_out, qblock_counts_out, stream))


def da_reassign_noalloc(handle, K, V, centroids_in, centroids_out, mean_values_out, assign_out,
                        cluster_sizes_out, qblock_counts_out, stream) -> int:
    return int(_lib.da_reassign_noalloc(handle, K, V, centroids_in, centroids_out,
                                        mean_values_out, assign_out, cluster_sizes_out,
                                        qblock_counts_out, stream))


def da_forward(handle, Q, K, V, centroids, mean_values, qblock_counts, O, lse_out,
               stream) -> int:
    return int(_lib.da_forward(handle, Q, K, V, centroids, mean_values, qblock_counts, O,
                               lse_out, stream))


def da_reassign_var(handle, K, V, centroids_in, centroids_out, mean_values_out, assign_out,
                    cluster_sizes_out, qblock_counts_out, key_variance_out, stream) -> int:
    return int(_lib.da_reassign_var(handle, K, V, centroids_in, centroids_out, mean_values_out,
                                    assign_out, cluster_sizes_out, qblock_counts_out,
                                    key_variance_out, stream))


def da_forward_var(handle, Q, K, V, centroids, mean_values, qblock_counts, key_variance, O,
                   lse_out, stream) -> int:
    return int(_lib.da_forward_var(handle, Q, K, V, centroids, mean_values, qblock_counts,
                                   key_variance, O, lse_out, stream))


# ------------------------------------------------------------------------ torch wrapper
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Plan:
    """A compiled plan: fixed exact key blocks per query block plus device workspace.

    `mask` is [mask_heads][nb][nkb] (or [nb][nkb]) with nb = ceil(N / block) query blocks
    and nkb = ceil(N / key_block) key blocks; key_block None or 0 means key_block = block."""

    def __init__(self, heads: int, seq_len: int, head_dim: int, block: int, clusters: int,
                 mask: np.ndarray, dtype: str = "bf16", scale: float = 0.0,
                 key_block: Optional[int] = None):
        mask = np.asarray(mask, dtype=np.uint8)
        if mask.ndim == 2:
            mask = mask[None]
        kblock = int(key_block or 0)
        self.desc = make_desc(heads, seq_len, head_dim, block, clusters, dtype,
                              mask_heads=mask.shape[0], scale=scale, key_block=kblock)
        nb = -(-seq_len // block)
        nkb = -(-seq_len // (kblock or block))
        if mask.shape[1:] != (nb, nkb):
            raise ValueError(f"mask must be [mask_heads][{nb}][{nkb}], got {mask.shape}")
        st, h = da_plan_create(self.desc, mask)
        if st != DA_OK:
            raise DAError(st, "da_plan_create")
        self._h = h
        self.heads, self.seq_len, self.head_dim = heads, seq_len, head_dim
        self.block, self.clusters, self.dtype, self.num_blocks = block, clusters, dtype, nb
        self.key_block, self.num_key_blocks = kblock or block, nkb

    # -- introspection
    def info(self) -> Dict[str, int]:
        nb, pairs, ws = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        st = _lib.da_plan_info(self._h, ctypes.byref(nb), ctypes.byref(pairs), ctypes.byref(ws))
        if st != DA_OK:
            raise DAError(st, "da_plan_info")
        return {"num_blocks": nb.value, "exact_pairs": pairs.value, "workspace_bytes": ws.value}

    def exact_lists(self, mh: int = 0):
        nb = self.num_blocks
        rowptr = np.zeros(nb + 1, np.int32)
        st = _lib.da_plan_exact_lists(self._h, mh, rowptr.ctypes.data_as(
            ctypes.POINTER(ctypes.c_int32)), None)
        if st != DA_OK:
            raise DAError(st, "da_plan_exact_lists")
        col = np.zeros(max(1, int(rowptr[-1])), np.int32)
        _lib.da_plan_exact_lists(self._h, mh, None, col.ctypes.data_as(
            ctypes.POINTER(ctypes.c_int32)))
        return rowptr, col[:int(rowptr[-1])]

    def close(self):
        if getattr(self, "_h", None):
            da_plan_destroy(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- tensor checks (marshalling)
    def _tdtype(self):
        torch = _torch()
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def _check(self, name, t, shape, dtype=None):
        torch = _torch()
        dtype = self._tdtype() if dtype is None else dtype
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name} is on {t.device}, but the current device is "
                             f"cuda:{torch.cuda.current_device()} (the plan's device)")
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                             f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")

    def _stream(self, stream):
        torch = _torch()
        s = torch.cuda.current_stream() if stream is None else stream
        return ctypes.c_void_p(s.cuda_stream)

    def reassign(self, K, V, centroids_in, out: Optional[Dict] = None, stream=None,
                 variance: bool = False, noalloc: bool = False):
        """One Reassign Cache step. Returns dict(centroids, mean_values, assign, sizes, counts),
        plus `variance` ([H][C] float32 key variance, da_reassign_var) when variance=True.
        noalloc=True runs da_reassign_noalloc (the library's static scratch instead of the
        plan's workspace; pass `out` to allocate nothing on this side either)."""
        torch = _torch()
        H, N, d, C, nb = self.heads, self.seq_len, self.head_dim, self.clusters, self.num_blocks
        self._check("K", K, (H, N, d))
        self._check("V", V, (H, N, d))
        self._check("centroids_in", centroids_in, (H, C, d))
        dev = K.device
        if out is None:
            out = {
                "centroids": torch.empty((H, C, d), dtype=self._tdtype(), device=dev),
                "mean_values": torch.empty((H, C, d), dtype=self._tdtype(), device=dev),
                "assign": torch.empty((H, N), dtype=torch.int32, device=dev),
                "sizes": torch.empty((H, C), dtype=torch.int32, device=dev),
                "counts": torch.empty((H, nb, C), dtype=torch.int32, device=dev),
            }
            if variance:
                out["variance"] = torch.empty((H, C), dtype=torch.float32, device=dev)
        else:
            self._check("centroids_out", out["centroids"], (H, C, d))
            self._check("mean_values_out", out["mean_values"], (H, C, d))
            self._check("assign_out", out["assign"], (H, N), torch.int32)
            self._check("sizes_out", out["sizes"], (H, C), torch.int32)
            self._check("counts_out", out["counts"], (H, nb, C), torch.int32)
            if variance:
                self._check("variance_out", out["variance"], (H, C), torch.float32)
        args = (self._h, _ptr(K), _ptr(V), _ptr(centroids_in), _ptr(out["centroids"]),
                _ptr(out["mean_values"]), _ptr(out["assign"]), _ptr(out["sizes"]),
                _ptr(out["counts"]))
        if variance and noalloc:
            raise ValueError("the variance outputs have no allocation-free entry point")
        if variance:
            st = da_reassign_var(*args, _ptr(out["variance"]), self._stream(stream))
            name = "da_reassign_var"
        elif noalloc:
            st = da_reassign_noalloc(*args, self._stream(stream))
            name = "da_reassign_noalloc"
        else:
            st = da_reassign(*args, self._stream(stream))
            name = "da_reassign"
        if st != DA_OK:
            raise DAError(st, name)
        return out

    def forward(self, Q, K, V, centroids, mean_values, counts, out=None, lse=False,
                stream=None, variance=None):
        """Decoupled sparse attention. Returns O, or (O, lse) when lse=True. With `variance`
        ([H][C] float32 key variance) the cluster logits are variance-corrected
        (da_forward_var)."""
        torch = _torch()
        H, N, d, C, nb = self.heads, self.seq_len, self.head_dim, self.clusters, self.num_blocks
        for name, t in (("Q", Q), ("K", K), ("V", V)):
            self._check(name, t, (H, N, d))
        self._check("centroids", centroids, (H, C, d))
        self._check("mean_values", mean_values, (H, C, d))
        self._check("counts", counts, (H, nb, C), torch.int32)
        if out is None:
            out = torch.empty((H, N, d), dtype=self._tdtype(), device=Q.device)
        else:
            self._check("O", out, (H, N, d))
        lse_t = None
        if lse is True:
            lse_t = torch.empty((H, N), dtype=torch.float32, device=Q.device)
        elif lse is not False and lse is not None:
            self._check("lse", lse, (H, N), torch.float32)
            lse_t = lse
        if variance is not None:
            self._check("variance", variance, (H, C), torch.float32)
            st = da_forward_var(self._h, _ptr(Q), _ptr(K), _ptr(V), _ptr(centroids),
                                _ptr(mean_values), _ptr(counts), _ptr(variance), _ptr(out),
                                _ptr(lse_t), self._stream(stream))
        else:
            st = da_forward(self._h, _ptr(Q), _ptr(K), _ptr(V), _ptr(centroids),
                            _ptr(mean_values), _ptr(counts), _ptr(out), _ptr(lse_t),
                            self._stream(stream))
        if st != DA_OK:
            raise DAError(st, "da_forward_var" if variance is not None else "da_forward")
        return (out, lse_t) if lse_t is not None else out

"""Host logic of plan compilation (csrc/plan_lists.cpp, the code da_plan_create runs), built
with g++ for the CPU and checked against invariants of the plan format on random masks:
every exact (query block, key block) pair appears once with the right use bit, tiles of
several key blocks serve one set of users and walk ascending, padding carries no use bit,
the partial-key-block flag marks exactly the last key block when it runs past N, and the
XCD work split covers every item in eight contiguous, balanced ranges."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_video_da_amd", "csrc")
IDX, U0, U1, PART = 0x0FFFFFFF, 28, 29, 30


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("plan") / "probe.so")
    subprocess.run([gxx, "-O2", "-std=c++17", "-shared", "-fPIC", f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "native", "plan_lists_probe.cpp"),
                    os.path.join(CSRC, "plan_lists.cpp"), "-o", out], check=True)
    lib = ctypes.CDLL(out)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.probe_plan_lists.argtypes = [ctypes.POINTER(ctypes.c_ubyte)] + [ctypes.c_int] * 6 + \
        [ip] * 5 + [ctypes.POINTER(ctypes.c_longlong)]

    def run(mask, heads, N, B, S, C):
        mask = np.ascontiguousarray(mask, np.uint8)
        sizes = (ctypes.c_longlong * 6)()
        mp = mask.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte))
        lib.probe_plan_lists(mp, mask.shape[0], heads, N, B, S, C, None, None, None, None, None,
                             sizes)
        arrs = [np.zeros(max(1, sizes[i]), np.int32) for i in range(4)]
        xs = np.zeros(9, np.int32)
        ptr = lambda a: a.ctypes.data_as(ip)
        lib.probe_plan_lists(mp, mask.shape[0], heads, N, B, S, C, *(ptr(a) for a in arrs),
                             ptr(xs), sizes)
        rowptr, col, prowptr, pcol = (a[:sizes[i]] for i, a in enumerate(arrs))
        return rowptr, col, prowptr, pcol, int(sizes[4]), xs, int(sizes[5])
    return run


CASES = [  # (heads, mask_heads, N, B, S, C, density)
    (3, 1, 1000, 128, 128, 200, 0.3), (2, 2, 850, 128, 32, 100, 0.25),
    (2, 2, 1000, 128, 16, 64, 0.15), (4, 1, 2700, 128, 64, 512, 0.4),
    (2, 2, 980, 64, 32, 50, 0.3), (1, 1, 129, 64, 16, 5, 0.5), (5, 5, 4096, 64, 64, 64, 0.05),
    (2, 1, 1, 128, 32, 1, 1.0),
]


@pytest.mark.parametrize("heads,mh,N,B,S,C,density", CASES)
def test_plan_lists_invariants(probe, heads, mh, N, B, S, C, density):
    nb, nkb, G = -(-N // B), -(-N // S), B // S
    rng = np.random.default_rng(N + 7 * S + mh)
    mask = (rng.random((mh, nb, nkb)) < density).astype(np.uint8)
    if nb > 2:
        mask[0, 1, :] = 0                  # an empty row
        mask[0, 2, :] = 1                  # a full row
    rowptr, col, prowptr, pcol, npairs, xs, xmax = probe(mask, heads, N, B, S, C)
    assert npairs == (nb + 1) // 2
    # exact lists: ascending key blocks of every row
    for m in range(mh):
        for b in range(nb):
            got = col[rowptr[m * (nb + 1) + b]:rowptr[m * (nb + 1) + b + 1]]
            assert got.tolist() == np.nonzero(mask[m, b])[0].tolist()
    partial = N % S != 0
    for m in range(mh):
        for pr in range(npairs):
            lst = pcol[prowptr[m * (npairs + 1) + pr]:prowptr[m * (npairs + 1) + pr + 1]]
            assert len(lst) % G == 0
            kb = lst & IDX
            use = (lst >> U0) & 3
            assert np.all(kb < nkb)
            assert np.all(((lst >> PART) & 1) == ((kb == nkb - 1) & partial))
            for half in (0, 1):
                b = 2 * pr + half
                mine = np.sort(kb[(use >> half) & 1 == 1])
                want = np.nonzero(mask[m, b])[0] if b < nb else np.zeros(0, np.int64)
                assert mine.tolist() == want.tolist()          # each exact pair once
            if G == 1:
                assert np.all(use != 0) and np.all(np.diff(kb) > 0)
                continue
            tiles = lst.reshape(-1, G)
            firsts = []
            for t in tiles:
                u = (t >> U0) & 3
                real = u != 0
                assert real[0] and len(set(u[real].tolist())) == 1   # one set of users
                nreal = int(real.sum())
                assert np.all(real[:nreal]) and not np.any(real[nreal:])   # pads at the end
                assert np.all((t[nreal:] & IDX) == (t[nreal - 1] & IDX))   # pads copy the last
                assert np.all(np.diff(t[:nreal] & IDX) > 0)
                firsts.append(int(t[0] & IDX))
            assert firsts == sorted(firsts)                    # tiles walk ascending
    # XCD split: contiguous ranges over all items, balanced by tile count
    items = heads * npairs
    assert xs[0] == 0 and xs[8] == items and np.all(np.diff(xs) >= 0)
    assert xmax == int(np.diff(xs).max())
    ctiles = -(-C // B)
    work = []
    for i in range(items):
        h, pr = divmod(i, npairs)
        m = 0 if mh == 1 else h
        n = prowptr[m * (npairs + 1) + pr + 1] - prowptr[m * (npairs + 1) + pr]
        work.append(n // G + ctiles + 1)
    work = np.array(work)
    per = [int(work[xs[x]:xs[x + 1]].sum()) for x in range(8)]
    assert sum(per) == work.sum()
    assert max(per) <= work.sum() / 8 + work.max() + 1

"""da_reassign_noalloc (the static-scratch variant of da_reassign) against da_reassign through the
C ABI: calls in a row on the same device, each followed by a smaller layer (other H, N, d, C;
resident and streamed centroid tables), replays of a captured HIP graph with other calls rewriting the scratch between them, and a
plan whose workspace exceeds the static scratch rejected before anything runs. The two entry
points share their kernels, so every output must be identical bit for bit."""
import ctypes

import numpy as np
import pytest

from parity_util import say, to_dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_video_da_amd as S
    return S


def _layer(seed, H, N, d, C, G):
    rng = np.random.default_rng(seed)
    from datagen import f32_to_bf16_bits
    cen = rng.standard_normal((G, d)).astype(np.float32)
    K = cen[rng.integers(0, G, (H, N))] + np.float32(0.25) * rng.standard_normal((H, N, d)).astype(np.float32)
    V = rng.standard_normal((H, N, d)).astype(np.float32)
    Kb, Vb = f32_to_bf16_bits(K), f32_to_bf16_bits(V)
    cache = np.stack([Kb[h][np.sort(rng.choice(N, C, replace=False))] for h in range(H)])
    return Kb, Vb, cache


def _outputs(lib, plan, H, N, d, C):
    torch = torch_mod()
    nb = plan.num_blocks
    return {"centroids": torch.empty((H, C, d), dtype=torch.bfloat16, device="cuda"),
            "mean_values": torch.empty((H, C, d), dtype=torch.bfloat16, device="cuda"),
            "assign": torch.full((H, N), -7, dtype=torch.int32, device="cuda"),
            "sizes": torch.full((H, C), -7, dtype=torch.int32, device="cuda"),
            "counts": torch.full((H, nb, C), -7, dtype=torch.int32, device="cuda")}


@pytest.mark.parametrize("order", ["noalloc_first", "plan_first"])
def test_noalloc_matches_reassign_on_two_calls(lib, order):
    torch = torch_mod()
    # resident table, then a smaller layer; then a streamed table (C beyond the LDS-resident
    # limit) and a smaller one again
    cases = [(4, 9000, 128, 128, 512, 7), (2, 2500, 64, 64, 100, 8),
             (2, 6000, 128, 128, 1536, 9), (1, 1800, 128, 64, 40, 10)]
    for i, (H, N, d, B, C, seed) in enumerate(cases):
        Kb, Vb, cache = _layer(seed, H, N, d, C, G=C // 2)
        nb = -(-N // B)
        rng = np.random.default_rng(seed + 100)
        mask = (rng.random((1, nb, nb)) < 0.2).astype(np.uint8)
        np.fill_diagonal(mask[0], 1)
        say(f"[case] no-alloc call {i}: H={H} N={N} d={d} C={C} ({order})")
        plan = lib.Plan(H, N, d, B, C, mask, dtype="bf16")
        K, V, mu = to_dev(Kb, "bf16"), to_dev(Vb, "bf16"), to_dev(cache, "bf16")
        a, b = _outputs(lib, plan, H, N, d, C), _outputs(lib, plan, H, N, d, C)
        if order == "noalloc_first":
            plan.reassign(K, V, mu, out=b, noalloc=True)
            plan.reassign(K, V, mu, out=a)
        else:
            plan.reassign(K, V, mu, out=a)
            plan.reassign(K, V, mu, out=b, noalloc=True)
        torch.cuda.synchronize()
        for k in a:
            x, y = a[k], b[k]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), f"call {i}: {k} differs between the entry points"
        assert int(a["assign"].min()) >= 0 and int(a["counts"].min()) >= 0
        plan.close()


def test_noalloc_replays_in_a_hip_graph(lib):
    """The callers da_reassign_noalloc is for include code under HIP graph capture: capture it
    on a side stream, then replay it three times with eager calls between the replays that
    rewrite the shared scratch (an allocation-free call on another, larger layer, and
    da_reassign on the captured layer). Every replay must equal the eager call bit for bit."""
    torch = torch_mod()
    H, N, d, B, C = 3, 5000, 128, 128, 256
    Kb, Vb, cache = _layer(31, H, N, d, C, G=C // 2)
    nb = -(-N // B)
    mask = (np.random.default_rng(131).random((1, nb, nb)) < 0.2).astype(np.uint8)
    np.fill_diagonal(mask[0], 1)
    plan = lib.Plan(H, N, d, B, C, mask, dtype="bf16")
    K, V, mu = to_dev(Kb, "bf16"), to_dev(Vb, "bf16"), to_dev(cache, "bf16")
    # the other layer whose eager calls overwrite the scratch between replays
    H2, N2, d2, C2 = 2, 9000, 64, 512
    K2b, V2b, cache2 = _layer(32, H2, N2, d2, C2, G=C2 // 2)
    nb2 = -(-N2 // 64)
    mask2 = np.zeros((1, nb2, nb2), np.uint8)
    np.fill_diagonal(mask2[0], 1)
    plan2 = lib.Plan(H2, N2, d2, 64, C2, mask2, dtype="bf16")
    K2, V2, mu2 = to_dev(K2b, "bf16"), to_dev(V2b, "bf16"), to_dev(cache2, "bf16")
    out2 = _outputs(lib, plan2, H2, N2, d2, C2)

    ref = _outputs(lib, plan, H, N, d, C)
    plan.reassign(K, V, mu, out=ref, noalloc=True)
    torch.cuda.synchronize()
    out = _outputs(lib, plan, H, N, d, C)
    eager = _outputs(lib, plan, H, N, d, C)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.reassign(K, V, mu, out=out, stream=side, noalloc=True)
    side.synchronize()
    say("[case] no-alloc reassign captured in a HIP graph")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        plan.reassign(K, V, mu, out=out, stream=side, noalloc=True)
    torch.cuda.synchronize()
    for r in range(3):
        plan2.reassign(K2, V2, mu2, out=out2, noalloc=True)   # rewrites the shared scratch
        plan.reassign(K, V, mu, out=eager)
        for v in out.values():
            v.fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            x, y, z = ref[k], out[k], eager[k]
            if x.dtype == torch.bfloat16:
                x, y, z = x.view(torch.int16), y.view(torch.int16), z.view(torch.int16)
            assert torch.equal(x, y), f"replay {r}: {k} differs from the eager call"
            assert torch.equal(x, z), f"replay {r}: {k} differs between the entry points"
    del graph
    plan2.close()
    plan.close()


def test_noalloc_rejects_a_workspace_beyond_the_scratch(lib):
    torch = torch_mod()
    H, N, d, B, C = 2, 65536, 64, 64, 8192     # workspace about 2 * 1024 * 8192 * 5 B = 84 MB
    mask = np.zeros((1, N // B, N // B), np.uint8)
    np.fill_diagonal(mask[0], 1)
    plan = lib.Plan(H, N, d, B, C, mask, dtype="bf16")
    K = torch.zeros((H, N, d), dtype=torch.bfloat16, device="cuda")
    mu = torch.zeros((H, C, d), dtype=torch.bfloat16, device="cuda")
    out = _outputs(lib, plan, H, N, d, C)
    st = lib.da_reassign_noalloc(plan._h, K.data_ptr(), K.data_ptr(), mu.data_ptr(),
                                 out["centroids"].data_ptr(), out["mean_values"].data_ptr(),
                                 out["assign"].data_ptr(), out["sizes"].data_ptr(),
                                 out["counts"].data_ptr(),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == lib.DA_ERR_UNSUPPORTED
    assert int(out["assign"].min()) == -7 and int(out["assign"].max()) == -7   # nothing ran
    plan.close()

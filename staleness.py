"""How stale does the Reassign Cache get? A measurement over S denoising steps.

Each step drifts K (and V, per the workload) by N(0, 0.05^2) and runs one `da_reassign`
from the previous step's centroids: one Lloyd iteration per step, the cache the method
carries. Beside it, a fresh clustering of the same drifted keys: 10 `da_reassign`
iterations from seeds taken at the workload's seed token indices of the drifted keys. For
both caches the step reports

  * the clustering objective J = sum_j |k_j - mu_{a_j}|^2 after the step's refresh, and
  * the forward's relative L2 distance to dense softmax attention, next to the same
    distance for exact blocks alone (every cluster count zero, no compensation).

Dense attention is the library's own forward on a plan whose mask keeps every block exact.
Everything runs through the C ABI on one GPU; the host only reduces the reported numbers.

    python staleness.py [--config extreme_cache_bf16] [--steps 8] [--heads 4]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="extreme_cache_bf16")
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--heads", type=int, default=4, help="first heads of the layer to use")
    ap.add_argument("--fresh-iters", type=int, default=10)
    args = ap.parse_args(argv)

    import torch
    from datagen import cache_init, drift_layer, get_config, make_layer
    import sparse_attention_video_da_amd as S

    cfg = get_config(args.config)
    heads = list(range(min(args.heads, cfg.heads)))
    H, N, d, B, C = len(heads), cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters
    nb = cfg.num_blocks
    if cfg.dtype != "bf16":
        raise SystemExit("the staleness measurement is written for bf16 layers")
    drift_cfg = cfg if (cfg.drift_k or cfg.drift_v) else dataclasses.replace(
        cfg, drift_k=True, drift_v=True)
    print(f"[staleness] {cfg.name}: heads {heads}, N={N}, C={C}, {args.steps} steps",
          file=sys.stderr, flush=True)
    L = make_layer(cfg, heads=heads, threads=16)
    mask = L["mask"][:1] if L["mask"].shape[0] == 1 else L["mask"][heads]

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    plan = S.Plan(H, N, d, B, C, mask, dtype="bf16")
    dense = S.Plan(H, N, d, B, C, np.ones((1, nb, nb), np.uint8), dtype="bf16")
    zeros = torch.zeros((H, nb, C), dtype=torch.int32, device="cuda")
    seeds = dev(L["cache_init"])

    def lloyd(K, V, mu, iters):
        out = None
        for _ in range(iters):
            out = plan.reassign(K, V, mu)
            mu = out["centroids"]
        return out

    def objective(K, out):
        k = K.float()
        mu = out["centroids"].float()
        a = out["assign"].long()
        diff = k - torch.gather(mu, 1, a[..., None].expand(-1, -1, d))
        return float((diff * diff).sum())

    def rel(o, ref):
        return float(torch.linalg.vector_norm((o.float() - ref.float()).flatten()) /
                     torch.linalg.vector_norm(ref.float().flatten()))

    K, V, Q = dev(L["K"]), dev(L["V"]), dev(L["Q"])
    cache = lloyd(K, V, seeds, args.fresh_iters)["centroids"].clone()
    rows = []
    t0 = time.time()
    for step in range(args.steps):
        L = drift_layer(drift_cfg, L, step, threads=16)
        K, V = dev(L["K"]), dev(L["V"])
        stale = plan.reassign(K, V, cache)
        stale = {k: v.clone() for k, v in stale.items()}
        # a fresh clustering seeds from the drifted keys at the workload's seed indices
        fresh_seeds = dev(np.stack([cache_init(cfg, L["K"][i], h) for i, h in enumerate(heads)]))
        fresh = lloyd(K, V, fresh_seeds, args.fresh_iters)
        fresh = {k: v.clone() for k, v in fresh.items()}
        o_dense = dense.forward(Q, K, V, stale["centroids"], stale["mean_values"], zeros)
        o_exact = plan.forward(Q, K, V, stale["centroids"], stale["mean_values"], zeros)
        o_stale = plan.forward(Q, K, V, stale["centroids"], stale["mean_values"], stale["counts"])
        o_fresh = plan.forward(Q, K, V, fresh["centroids"], fresh["mean_values"], fresh["counts"])
        torch.cuda.synchronize()
        row = {"step": step + 1,
               "J_cache_over_fresh": objective(K, stale) / objective(K, fresh),
               "err_cache": rel(o_stale, o_dense), "err_fresh": rel(o_fresh, o_dense),
               "err_exact_only": rel(o_exact, o_dense)}
        rows.append(row)
        print(f"[staleness] step {step + 1}: J cache/fresh {row['J_cache_over_fresh']:.4f}, "
              f"rel-L2 to dense: cache {row['err_cache']:.4f}, fresh {row['err_fresh']:.4f}, "
              f"exact only {row['err_exact_only']:.4f}", file=sys.stderr, flush=True)
        cache = stale["centroids"]
    print(json.dumps({"workload": cfg.name, "heads": heads, "steps": args.steps,
                      "fresh_iters": args.fresh_iters, "seconds": round(time.time() - t0, 1),
                      "rows": rows}))
    plan.close()
    dense.close()


if __name__ == "__main__":
    main()

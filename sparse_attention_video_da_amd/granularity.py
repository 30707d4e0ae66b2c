"""Accuracy of the exact key block size at a fixed budget of exact keys.

For one layer (Q, K, V and the seeded cache of a 3D-local workload) and each key block size
S, the mask keeps the k*B/S nearest key blocks of S keys per query block of B (by default
nearest to any token of the query block, the generator's "reach" rule): the same
number of exact keys as k blocks of B, chosen at a finer granularity (the Accurate Block
Attention (AB-Attention) abstract packs key/value blocks smaller than a tile into full
tensor-core tiles to refine the selection). The cache is 10 `da_reassign` Lloyd iterations
from the seeds, refreshed per mask (the counts depend on it). Reported per S: the forward's
relative L2 distance to dense softmax attention with cluster compensation and with the
exact blocks alone (every count zero), and with the variance-corrected compensation
(`da_reassign_var` / `da_forward_var`). Dense attention is the library's forward on a plan
whose mask keeps every block exact. Everything runs through the C ABI on one GPU; the host
only reduces the reported numbers.

`--locality a` adds the generator's positional term (Q and K gain a * phi(x), a Gaussian
kernel of 3D distance with length `--locality-len`): without it the synthetic logits do
not depend on position at all, and no choice of position-fixed blocks can matter.

    python -m sparse_attention_video_da_amd.granularity [--config hunyuan13b_bf16]
        [--heads 3] [--key-blocks 128 64 32 16] [--locality 12] [--locality-len 6]
        [--rule reach|centre]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="hunyuan13b_bf16")
    ap.add_argument("--heads", type=int, default=3, help="first heads of the layer to use")
    ap.add_argument("--key-blocks", type=int, nargs="+", default=[128, 64, 32, 16])
    ap.add_argument("--iters", type=int, default=10)
    ap.add_argument("--locality", type=float, default=0.0)
    ap.add_argument("--locality-len", type=float, default=6.0)
    ap.add_argument("--rule", default="reach", choices=["centre", "reach"],
                    help="key block distance of the local masks (see datagen)")
    args = ap.parse_args(argv)

    import torch
    from datagen import block_mask, get_config, make_layer
    import sparse_attention_video_da_amd as S

    cfg = dataclasses.replace(get_config(args.config), locality=args.locality,
                              locality_len=args.locality_len, local_rule=args.rule)
    if cfg.mask_kind != "local" or cfg.kblock != cfg.block or cfg.dtype != "bf16":
        raise SystemExit("needs a bf16 layer with a local mask of query-sized key blocks")
    heads = list(range(min(args.heads, cfg.heads)))
    H, N, d, B, C = len(heads), cfg.seq_len, cfg.head_dim, cfg.block, cfg.clusters
    nb = cfg.num_blocks
    print(f"[granularity] {cfg.name}: heads {heads}, N={N}, B={B}, {cfg.blocks_per_row} blocks "
          f"of {B} exact per query block, locality {cfg.locality} (length "
          f"{cfg.locality_len}), {cfg.local_rule} rule", file=sys.stderr, flush=True)
    L = make_layer(cfg, heads=heads, threads=16)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)

    Q, K, V = dev(L["Q"]), dev(L["K"]), dev(L["V"])
    seeds = dev(L["cache_init"])
    zeros = torch.zeros((H, nb, C), dtype=torch.int32, device="cuda")

    def rel(o, ref):
        return float(torch.linalg.vector_norm((o.float() - ref.float()).flatten()) /
                     torch.linalg.vector_norm(ref.float().flatten()))

    dense = S.Plan(H, N, d, B, C, np.ones((1, nb, nb), np.uint8), dtype="bf16")
    rows = []
    o_dense = None
    t0 = time.time()
    for kb in args.key_blocks:
        if B % kb:
            raise SystemExit(f"key block {kb} does not divide the query block {B}")
        kcfg = dataclasses.replace(cfg, key_block=kb, blocks_per_row=cfg.blocks_per_row * B // kb)
        mask = block_mask(kcfg)
        plan = S.Plan(H, N, d, B, C, mask, dtype="bf16", key_block=kb)
        mu = seeds
        for _ in range(args.iters):
            out = plan.reassign(K, V, mu, variance=True)
            mu = out["centroids"]
        if o_dense is None:
            o_dense = dense.forward(Q, K, V, out["centroids"], out["mean_values"], zeros)
        o_comp = plan.forward(Q, K, V, out["centroids"], out["mean_values"], out["counts"])
        o_exact = plan.forward(Q, K, V, out["centroids"], out["mean_values"], zeros)
        o_var = plan.forward(Q, K, V, out["centroids"], out["mean_values"], out["counts"],
                             variance=out["variance"])
        torch.cuda.synchronize()
        row = {"key_block": kb, "exact_blocks_per_row": kcfg.blocks_per_row,
               "exact_key_fraction": round(float(mask.sum()) * kb / (nb * N), 5),
               "err_compensated": rel(o_comp, o_dense), "err_exact_only": rel(o_exact, o_dense),
               "err_variance_corrected": rel(o_var, o_dense)}
        rows.append(row)
        print(f"[granularity] S={kb}: rel-L2 to dense {row['err_compensated']:.4f}, "
              f"variance-corrected {row['err_variance_corrected']:.4f} "
              f"(exact blocks alone {row['err_exact_only']:.4f})", file=sys.stderr, flush=True)
        plan.close()
    dense.close()
    print(json.dumps({"workload": cfg.name, "heads": heads, "iters": args.iters,
                      "locality": cfg.locality, "locality_len": cfg.locality_len,
                      "rule": cfg.local_rule,
                      "seconds": round(time.time() - t0, 1), "rows": rows}))


if __name__ == "__main__":
    main()

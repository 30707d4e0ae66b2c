"""Plain fp64 CPU oracle for decoupled sparse attention with a reassigned cluster cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
package: only the tests, the package smoke check and the benchmark's CPU-baseline leg use
it. It shares no code with the HIP library (no kernels, headers, helpers or tables); the
only thing both sides consume is the seeded input generator in `datagen`, which holds
none of the method's arithmetic.

Source of every definition: the DecoupAttn abstract ("DecoupAttn: Decoupled Sparse
Attention for Training-Free Acceleration of Video Diffusion", arXiv 2611.05917, Abstract),
and Lloyd, "Least squares quantization in PCM" (listed on that paper page under the works
it builds on). Each function names the sentence of the abstract it follows. Exact key
blocks smaller than the query blocks (the optional `kblock`) follow the kernel sentence of
the Accurate Block Attention (AB-Attention) abstract.

Pinning status: every public function is pinned by tests that do not retype it (closed
forms, a hand-derived worked example, brute force, invariants and library special cases).
Unpinned by the pages (a reading, not a derivation): whether the compensation centroid and
mean value are global per cluster or restricted to keys outside the exact blocks; this
oracle uses global per-cluster means (parity unpinned on that reading). The optional
variance correction (`kvar` in `forward`, `key_variance`) is named by the ESTRA abstract
without a formula: the second-order correction with an isotropic per-cluster variance is
this oracle's reading; its arithmetic is pinned to closed forms and sampling, but that the
pages mean exactly this is unpinned.
"""
from .decoupattn_oracle import (  # noqa: F401
    TIE_BAND,
    storage_round,
    to_f64,
    assign,
    assignment_allowed,
    refresh,
    qblock_counts_direct,
    key_variance,
    forward,
    forward_substituted,
    dense_attention,
    objective,
    lloyd_warmup,
    reassign_step,
    default_scale,
)

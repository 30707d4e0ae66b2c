/*
 * decoupattn.h — C ABI of the MI355X (gfx950) decoupled sparse attention library.
 *
 * The method (DecoupAttn: Decoupled Sparse Attention for Training-Free Acceleration of
 * Video Diffusion, arXiv 2611.05917, Abstract): for every query block, attention is
 * computed exactly on a few key blocks chosen once offline by position; every other key
 * is compensated by its semantic cluster (centroid key, mean value, and a logit bias of
 * ln n where n is how many of the cluster's keys lie outside the exact blocks), and both
 * parts are merged in one softmax. Each denoising step first reassigns the drifted keys
 * to the cached centroids and refreshes the centroids, mean values and counts while the
 * exact blocks stay fixed (the abstract's Reassign Cache). The assignment is Lloyd's
 * nearest-centroid step (Lloyd, Least squares quantization in PCM).
 *
 * Conventions shared by every entry point
 *   - Tensors are caller-owned device buffers (hipMalloc'd or framework allocations),
 *     passed as plain pointers, row-major and contiguous, batch folded into heads:
 *       Q, K, V, O           [H][N][d]   elements of the plan dtype
 *       centroids, means     [H][C][d]   elements of the plan dtype (the cluster cache)
 *       assign               [H][N]      int32
 *       cluster_sizes        [H][C]      int32
 *       qblock_counts        [H][nb][C]  int32, nb = ceil(N / block)
 *       block mask (host)    [mask_heads][nb][nkb] uint8, nkb = ceil(N / key_block)
 *       lse                  [H][N]      float (natural-log log-sum-exp of each row)
 *     N need not be a multiple of the block size; exactly N rows are read and written.
 *   - Device pointers to element tensors must be 16-byte aligned; int32/float outputs
 *     4-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Compute entry
 *     points only enqueue work on it: they never allocate, free or synchronise.
 *   - Every argument is validated before anything is enqueued; on any error nothing is
 *     enqueued and no output is touched. Asynchronous device faults surface at the
 *     caller's next synchronisation. The library never prints and never throws.
 *   - A plan owns a device workspace; one plan must not be used by two streams at once.
 *     Distinct plans are independent.
 *   - A plan belongs to the device that was current when it was created: compute entry
 *     points must be called with that device current, and a non-NULL stream must be one of
 *     its streams (checked; INVALID_ARGUMENT otherwise).
 */
#ifndef DECOUPATTN_H
#define DECOUPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define DA_API __attribute__((visibility("default")))
#else
#define DA_API
#endif

typedef enum {
  DA_OK = 0,
  DA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, inconsistent sizes, aliasing */
  DA_ERR_UNSUPPORTED = 2,      /* a size or dtype outside the compiled kernel set      */
  DA_ERR_OUT_OF_MEMORY = 3,    /* device allocation for the plan failed                 */
  DA_ERR_DEVICE = 4            /* no usable device, or a HIP call/launch failed         */
} da_status;

typedef enum { DA_DTYPE_F32 = 0, DA_DTYPE_BF16 = 1 } da_dtype;

/* Shape of one attention layer.
 *   heads       H >= 1
 *   seq_len     N >= 1 tokens per head, with N * d * (element bytes) < 2^31 (one head's Q, K,
 *               V or O addressed with 32-bit byte offsets)
 *   head_dim    d in {64, 128}
 *   block       B in {64, 128}: query block size of the mask (and the tile height)
 *   clusters    C, 1 <= C <= N and C <= 8192
 *   mask_heads  1 (one mask shared by all heads) or H (one mask per head)
 *   dtype       element type of Q, K, V, O and the cluster cache (da_dtype)
 *   scale       softmax scale; 0 selects 1/sqrt(d). Must be finite and >= 0.
 *   key_block   S, the size of the exact key blocks; 0 selects S = B. S in {16, 32, 64,
 *               128} with S <= B. With S < B the forward packs B/S exact key blocks of a
 *               query block into each B-row tile (Accurate Block Attention (AB-Attention),
 *               Abstract: key/value blocks smaller than a tile gathered into full
 *               tensor-core tiles), so exact keys are chosen at the finer granularity for
 *               the matrix-core cost of B-row tiles. */
typedef struct {
  int32_t heads;
  int32_t seq_len;
  int32_t head_dim;
  int32_t block;
  int32_t clusters;
  int32_t mask_heads;
  int32_t dtype;
  float scale;
  int32_t key_block;
} da_desc;

typedef struct da_plan_s* da_plan;

/* Compile a plan from a position-fixed block mask (abstract: the exact blocks are fixed
 * once offline by position; one plan is compiled offline and reused every step).
 *   desc             layer shape (copied).
 *   block_mask_host  HOST array uint8 [mask_heads][nb][nkb]; nonzero at [h][b][kb] means
 *                    key block kb (keys kb*S .. min(N, (kb+1)*S) - 1) is attended exactly
 *                    by query block b. Any pattern is legal, including rows with no exact
 *                    block. Copied; not retained.
 *   out              receives the plan handle (set to NULL on error).
 * Builds the per-query-block exact lists (sorted key-block indices), uploads them and
 * allocates the reassignment workspace. This is the only call that allocates device
 * memory or synchronises. Errors: INVALID_ARGUMENT, UNSUPPORTED, OUT_OF_MEMORY, DEVICE. */
DA_API da_status da_plan_create(const da_desc* desc, const uint8_t* block_mask_host,
                                da_plan* out);

/* Release a plan and its device memory (synchronises the plan's device first; the caller's
 * current device is left as it was). NULL is a no-op. */
DA_API da_status da_plan_destroy(da_plan plan);

/* Reassign Cache step (abstract: each step reassigns drifted keys to the cached
 * centroids and refreshes the compensation; the exact blocks stay fixed).
 *   K, V               [H][N][d] current keys and values (device).
 *   centroids_in       [H][C][d] cached centroids mu0 (device, read only; must not
 *                      overlap any output).
 *   centroids_out      [H][C][d] refreshed centroids: mean of the keys assigned to each
 *                      cluster, rounded to the dtype; a cluster with no key keeps mu0.
 *   mean_values_out    [H][C][d] mean of the values of each cluster's keys (0 if none).
 *   assign_out         [H][N] a_j = argmin_c ||k_j - mu0_c||^2 (squared Euclidean on the
 *                      stored values). fp32 plans: differences squared and summed in fp32,
 *                      equal sums go to the lowest c. bf16 plans: distances from the bf16
 *                      matrix cores with fp32 accumulation (their error grows with
 *                      |k|^2 + |mu|^2, not with the distance); a key whose two nearest
 *                      computed distances lie within 2^-15 (|k|^2 + max |mu|^2), plus 2^-16
 *                      of the smaller, of each other is re-measured as an fp32 sum of squared
 *                      differences against every centroid whose computed distance is within
 *                      that bound of its smallest (no other can be its nearest), equal sums
 *                      going to the lowest c. Either way the chosen centroid is the nearest unless
 *                      the two nearest lie within a relative 1e-4 of each other (then any of
 *                      them may be chosen).
 *   cluster_sizes_out  [H][C] number of keys per cluster.
 *   qblock_counts_out  [H][nb][C] n[b][c]: keys of cluster c outside query block b's
 *                      exact key blocks (counted key by key, whatever the key block size).
 * All outputs are written in full. Errors: INVALID_ARGUMENT, DEVICE. */
DA_API da_status da_reassign(da_plan plan, const void* K, const void* V,
                             const void* centroids_in, void* centroids_out,
                             void* mean_values_out, int32_t* assign_out,
                             int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                             void* stream);

/* da_reassign for callers that cannot allocate or may not touch the plan's workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * computation, arguments, outputs and errors as da_reassign, with its scratch (histograms,
 * the cluster-sorted key order, partial sums, distance operands, the near-tie list) taken
 * from a static device array of 64 MiB that the library holds on every device it runs on
 * until the process ends, instead of the plan's workspace. Nothing is allocated, freed or
 * synchronised. A plan whose reassignment workspace exceeds 64 MiB is rejected with
 * DA_ERR_UNSUPPORTED before anything is enqueued (the workspace takes about
 * H * (nb * C * 5 + N * 12 + (N / 256 + C) * (8 d + 4) + C * (2 d + 20)) bytes).
 * All calls on one device share that array: calls whose executions overlap on a device
 * (two streams, or two host threads) race and give undefined results; calls ordered on
 * one stream are safe, and each call rewrites everything it reads from the array. */
DA_API da_status da_reassign_noalloc(da_plan plan, const void* K, const void* V,
                                     const void* centroids_in, void* centroids_out,
                                     void* mean_values_out, int32_t* assign_out,
                                     int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                                     void* stream);

/* Decoupled sparse attention forward (abstract: exact attention on the fixed blocks,
 * cluster compensation of every other key, one fused kernel).
 *   Q, K, V        [H][N][d] (device).
 *   centroids      [H][C][d] compensation centroid keys mu.
 *   mean_values    [H][C][d] compensation mean values vbar.
 *   qblock_counts  [H][nb][C] n[b][c] >= 0; clusters with n = 0 are skipped.
 *   O              [H][N][d] output: for query i of block b,
 *                  softmax over { scale q_i.k_j : j in the exact blocks of b } united with
 *                  { scale q_i.mu_c + ln n[b][c] : n[b][c] > 0 }, applied to the matching
 *                  values v_j and vbar_c. fp32 softmax and accumulation.
 *   lse_out        [H][N] float, natural log of each row's softmax denominator
 *                  (including the row max); may be NULL.
 * Errors: INVALID_ARGUMENT, DEVICE. */
DA_API da_status da_forward(da_plan plan, const void* Q, const void* K, const void* V,
                            const void* centroids, const void* mean_values,
                            const int32_t* qblock_counts, void* O, float* lse_out,
                            void* stream);

/* Variance-corrected compensation (optional; the ESTRA page, "Extreme Sparsity Through
 * Refined Attention", zhuanzhiai paper page, Abstract: a variance-based correction refines
 * the attention weights of the cluster representatives; the page gives no formula, and the
 * second-order correction below is this library's reading of it).
 *
 * da_reassign_var: da_reassign plus
 *   key_variance_out  [H][C] float (4-byte aligned, device): kvar_c, the mean over the
 *                     cluster's keys and the d dimensions of (k_j - mean_c)^2 (fp32, from the
 *                     unrounded mean); 0 for an empty cluster. Must not overlap centroids_in.
 * da_forward_var: da_forward where every cluster logit gains
 *                 0.5 * scale^2 * key_variance[c] * ||q_i||^2
 *   key_variance      [H][C] float (device), kvar >= 0 (for instance da_reassign_var's).
 *                     With all zeros the result equals da_forward's.
 * For keys spread around the centroid with covariance kvar * I the mean of exp(scale q.k)
 * over them is exp(scale q.mean + 0.5 scale^2 kvar ||q||^2) (exact for Gaussian keys, to
 * second order otherwise), so the corrected representative carries the cluster's weight
 * instead of underestimating it (Jensen). Errors: as da_reassign / da_forward, and
 * INVALID_ARGUMENT for a NULL or misaligned variance pointer. */
DA_API da_status da_reassign_var(da_plan plan, const void* K, const void* V,
                                 const void* centroids_in, void* centroids_out,
                                 void* mean_values_out, int32_t* assign_out,
                                 int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                                 float* key_variance_out, void* stream);
DA_API da_status da_forward_var(da_plan plan, const void* Q, const void* K, const void* V,
                                const void* centroids, const void* mean_values,
                                const int32_t* qblock_counts, const float* key_variance,
                                void* O, float* lse_out, void* stream);

/* Plan introspection (host-side values; no device work).
 *   num_blocks       nb = ceil(N / block)
 *   exact_pairs      total number of (query block, exact key block) pairs over mask heads
 *                    (key blocks of the plan's key block size)
 *   workspace_bytes  device bytes the plan owns (exact lists + reassignment workspace) */
DA_API da_status da_plan_info(da_plan plan, int32_t* num_blocks, int64_t* exact_pairs,
                              int64_t* workspace_bytes);

/* Copy of the plan's exact lists for mask head mh: rowptr[nb+1] and col[rowptr[nb]]
 * (sorted key-block indices, in key blocks of the plan's key block size, per query block).
 * Either output may be NULL to skip it. */
DA_API da_status da_plan_exact_lists(da_plan plan, int32_t mh, int32_t* rowptr,
                                     int32_t* col);

/* Validate a descriptor and mask without touching any device (same checks as
 * da_plan_create). Returns DA_OK when da_plan_create would accept them. */
DA_API da_status da_validate_desc(const da_desc* desc, const uint8_t* block_mask_host);

/* Static, human-readable name of a status code ("unknown status" for other values). */
DA_API const char* da_status_str(da_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
DA_API int32_t da_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECOUPATTN_H */

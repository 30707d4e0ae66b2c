// C ABI of the decoupled sparse attention library: argument validation, plan compilation
// (mask -> per-query-block exact lists, device workspace) and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <utility>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/decoupattn.h"
#include "da_internal.h"
#include "plan_lists.h"

namespace da {
hipError_t prepare_forward_kernels();
hipError_t prepare_reassign_kernels();
}  // namespace da

struct da_plan_s {
  da_desc desc;
  int32_t nb;
  int32_t kblock;               // exact key block size S
  int32_t nkb;                  // ceil(N / S)
  float scale;
  std::vector<int32_t> rowptr;  // [mask_heads][nb + 1], absolute offsets into col
  std::vector<int32_t> col;
  // query-block pairs (2p, 2p+1): union of both exact lists in the da::kEnt* entry format
  // (ascending when S = B; grouped by user and padded to a multiple of B/S when S < B)
  std::vector<int32_t> prowptr;  // [mask_heads][npairs + 1]
  std::vector<int32_t> pcol;
  int32_t npairs = 0;
  // bf16 forward schedule: work items (head, pair) in natural order split into 8
  // contiguous ranges of about equal work, range x for XCD x
  int32_t xstart[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  int32_t xmax = 0;
  int32_t* d_rowptr = nullptr;
  int32_t* d_col = nullptr;
  int32_t* d_prowptr = nullptr;
  int32_t* d_pcol = nullptr;
  void* d_ws = nullptr;          // reassignment workspace (layout: workspace_layout)
  int64_t bytes = 0;
  int32_t ncu = 0;   // compute units of the plan's device
  int device = 0;
};

namespace {

constexpr int32_t kMaxClusters = 8192;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(const da_desc& d) { return d.dtype == DA_DTYPE_BF16 ? 2 : 4; }

int32_t key_block_of(const da_desc& d) { return d.key_block > 0 ? d.key_block : d.block; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

da_status check_desc(const da_desc* d) {
  if (d == nullptr) return DA_ERR_INVALID_ARGUMENT;
  if (d->heads < 1 || d->seq_len < 1 || d->clusters < 1 || d->head_dim < 1 || d->block < 1)
    return DA_ERR_INVALID_ARGUMENT;
  if (d->clusters > d->seq_len) return DA_ERR_INVALID_ARGUMENT;
  if (d->mask_heads != 1 && d->mask_heads != d->heads) return DA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(d->scale) || d->scale < 0.f) return DA_ERR_INVALID_ARGUMENT;
  if (d->dtype != DA_DTYPE_F32 && d->dtype != DA_DTYPE_BF16) return DA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return DA_ERR_UNSUPPORTED;
  if (d->block != 64 && d->block != 128) return DA_ERR_UNSUPPORTED;
  if (d->clusters > kMaxClusters) return DA_ERR_UNSUPPORTED;
  if (d->key_block < 0) return DA_ERR_INVALID_ARGUMENT;
  const int32_t S = key_block_of(*d);
  if ((S != 16 && S != 32 && S != 64 && S != 128) || S > d->block) return DA_ERR_UNSUPPORTED;
  // int32 byte offsets within one head's [N][d] tensor (the kernels' buffer resources and
  // row offsets), int32 indexing of [H][nb][C] counts and of the mask
  const int64_t nb = (d->seq_len + d->block - 1) / d->block;
  const int64_t nkb = (d->seq_len + S - 1) / S;
  const int64_t es = d->dtype == DA_DTYPE_BF16 ? 2 : 4;
  if ((int64_t)d->seq_len * d->head_dim * es > INT32_MAX || nb * d->clusters > INT32_MAX ||
      nb * nkb * d->mask_heads > INT32_MAX || (int64_t)d->heads * d->seq_len > INT32_MAX)
    return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

void destroy_device(da_plan_s* p) {
  void* bufs[] = {p->d_rowptr, p->d_col, p->d_prowptr, p->d_pcol, p->d_ws};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  p->d_rowptr = p->d_col = p->d_prowptr = p->d_pcol = nullptr;
  p->d_ws = nullptr;
}

// Reassignment workspace of a layer shape, carved from one device buffer (each part 256-byte
// aligned): byte histograms [H][nb][C], column offsets [H][nb][C], cluster starts [H][C], the
// sorted order [H][N], the bf16 distance operands [H][C][d + 8], fp32 partial sums
// [H][ceil(N/256) + C][2][d] and squared norms [H][ceil(N/256) + C], the near-tie list.
struct WorkspaceLayout {
  size_t hist, off, start, perm, cop, part, psq, fix, total;
};

WorkspaceLayout workspace_layout(const da_desc& d, int32_t nb) {
  const size_t H = d.heads, N = d.seq_len, C = d.clusters, D = d.head_dim;
  const size_t nseg = (N + 255) / 256;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at += (bytes + 255) / 256 * 256;
    return o;
  };
  WorkspaceLayout w;
  w.hist = take(H * nb * C);
  w.off = take(H * nb * C * 4);
  w.start = take(H * C * 4);
  w.perm = take(H * N * 4);
  w.cop = take(H * C * (D + 8) * 2);
  w.part = take(H * (nseg + C) * 2 * D * 4);
  w.psq = take(H * (nseg + C) * 4);
  w.fix = take((da::fix_list_offset((int)H) + 2 * H * N) * 4);
  w.total = at;
  return w;
}

// Kernel attributes (dynamic LDS limits) are set once per device, on first use.
std::mutex g_prep_mu;
std::vector<int> g_prepared;

hipError_t prepare_device(int dev) {
  std::lock_guard<std::mutex> lock(g_prep_mu);
  for (int x : g_prepared)
    if (x == dev) return hipSuccess;
  hipError_t e = da::prepare_forward_kernels();
  if (e == hipSuccess) e = da::prepare_reassign_kernels();
  if (e == hipSuccess) e = da::scratch_setup(dev);
  if (e == hipSuccess) g_prepared.push_back(dev);
  return e;
}

// A plan's lists and workspace live on the device that was current at its creation: compute
// calls must run with that device current and, when a stream is given, on one of its streams.
da_status check_device(const da_plan_s* p, void* stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DA_ERR_DEVICE;
  if (dev != p->device) return DA_ERR_INVALID_ARGUMENT;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return DA_ERR_INVALID_ARGUMENT;
    }
    if (sdev != p->device) return DA_ERR_INVALID_ARGUMENT;
  }
  return DA_OK;
}

}  // namespace

extern "C" {

DA_API const char* da_status_str(da_status s) {
  switch (s) {
    case DA_OK: return "DA_OK";
    case DA_ERR_INVALID_ARGUMENT: return "DA_ERR_INVALID_ARGUMENT: invalid argument";
    case DA_ERR_UNSUPPORTED: return "DA_ERR_UNSUPPORTED: unsupported size or dtype";
    case DA_ERR_OUT_OF_MEMORY: return "DA_ERR_OUT_OF_MEMORY: device allocation failed";
    case DA_ERR_DEVICE: return "DA_ERR_DEVICE: HIP device or launch error";
  }
  return "unknown status";
}

DA_API int32_t da_version(void) { return 102; }

DA_API da_status da_validate_desc(const da_desc* desc, const uint8_t* mask) {
  const da_status st = check_desc(desc);
  if (st != DA_OK) return st;
  if (mask == nullptr) return DA_ERR_INVALID_ARGUMENT;
  return DA_OK;
}

DA_API da_status da_plan_create(const da_desc* desc, const uint8_t* mask, da_plan* out) {
  if (out == nullptr) return DA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const da_status st = da_validate_desc(desc, mask);
  if (st != DA_OK) return st;

  da_plan_s* p = new (std::nothrow) da_plan_s();
  if (p == nullptr) return DA_ERR_OUT_OF_MEMORY;
  p->desc = *desc;
  const int32_t nb = (desc->seq_len + desc->block - 1) / desc->block;
  const int32_t S = key_block_of(*desc);
  const int32_t nkb = (desc->seq_len + S - 1) / S;
  p->nb = nb;
  p->kblock = S;
  p->nkb = nkb;
  p->scale = desc->scale > 0.f ? desc->scale : 1.0f / std::sqrt((float)desc->head_dim);
  {
    da::PlanLists lists;
    da::build_plan_lists(mask, desc->mask_heads, desc->heads, desc->seq_len, desc->block, S,
                         desc->clusters, lists);
    p->rowptr = std::move(lists.rowptr);
    p->col = std::move(lists.col);
    p->prowptr = std::move(lists.prowptr);
    p->pcol = std::move(lists.pcol);
    p->npairs = lists.npairs;
    for (int x = 0; x < 9; ++x) p->xstart[x] = lists.xstart[x];
    p->xmax = lists.xmax;
  }

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1 || hipGetDevice(&p->device) != hipSuccess) {
    delete p;
    return DA_ERR_DEVICE;
  }
  if (prepare_device(p->device) != hipSuccess ||
      hipDeviceGetAttribute(&p->ncu, hipDeviceAttributeMultiprocessorCount, p->device) !=
          hipSuccess ||
      p->ncu < 1) {
    (void)hipGetLastError();
    delete p;
    return DA_ERR_DEVICE;
  }

  const size_t n_rowptr = p->rowptr.size(), n_col = std::max<size_t>(1, p->col.size());
  const size_t n_prowptr = p->prowptr.size(), n_pcol = std::max<size_t>(1, p->pcol.size());
  struct Alloc { void** ptr; size_t bytes; } allocs[] = {
      {reinterpret_cast<void**>(&p->d_rowptr), n_rowptr * 4},
      {reinterpret_cast<void**>(&p->d_col), n_col * 4},
      {reinterpret_cast<void**>(&p->d_prowptr), n_prowptr * 4},
      {reinterpret_cast<void**>(&p->d_pcol), n_pcol * 4},
      {&p->d_ws, workspace_layout(*desc, nb).total}};
  for (const Alloc& a : allocs) {
    if (hipMalloc(a.ptr, a.bytes) != hipSuccess) {
      (void)hipGetLastError();
      destroy_device(p);
      delete p;
      return DA_ERR_OUT_OF_MEMORY;
    }
    p->bytes += (int64_t)a.bytes;
  }
  if (hipMemcpy(p->d_rowptr, p->rowptr.data(), n_rowptr * sizeof(int32_t),
                hipMemcpyHostToDevice) != hipSuccess ||
      (!p->col.empty() && hipMemcpy(p->d_col, p->col.data(), p->col.size() * sizeof(int32_t),
                                    hipMemcpyHostToDevice) != hipSuccess) ||
      hipMemcpy(p->d_prowptr, p->prowptr.data(), n_prowptr * sizeof(int32_t),
                hipMemcpyHostToDevice) != hipSuccess ||
      (!p->pcol.empty() && hipMemcpy(p->d_pcol, p->pcol.data(), p->pcol.size() * sizeof(int32_t),
                                     hipMemcpyHostToDevice) != hipSuccess)) {
    destroy_device(p);
    delete p;
    return DA_ERR_DEVICE;
  }
  *out = p;
  return DA_OK;
}

DA_API da_status da_plan_destroy(da_plan p) {
  if (p == nullptr) return DA_OK;
  // synchronise and free on the plan's device, leaving the caller's current device as it was
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  const bool switched = have_cur && cur != p->device && hipSetDevice(p->device) == hipSuccess;
  (void)hipDeviceSynchronize();
  destroy_device(p);
  if (switched) (void)hipSetDevice(cur);
  delete p;
  return DA_OK;
}

DA_API da_status da_plan_info(da_plan p, int32_t* num_blocks, int64_t* exact_pairs,
                              int64_t* workspace_bytes) {
  if (p == nullptr) return DA_ERR_INVALID_ARGUMENT;
  if (num_blocks) *num_blocks = p->nb;
  if (exact_pairs) *exact_pairs = (int64_t)p->col.size();
  if (workspace_bytes) *workspace_bytes = p->bytes;
  return DA_OK;
}

DA_API da_status da_plan_exact_lists(da_plan p, int32_t mh, int32_t* rowptr, int32_t* col) {
  if (p == nullptr || mh < 0 || mh >= p->desc.mask_heads) return DA_ERR_INVALID_ARGUMENT;
  const size_t base = (size_t)mh * (p->nb + 1);
  const int32_t first = p->rowptr[base];
  if (rowptr)
    for (int32_t b = 0; b <= p->nb; ++b) rowptr[b] = p->rowptr[base + b] - first;
  if (col)
    for (int32_t i = first; i < p->rowptr[base + p->nb]; ++i) col[i - first] = p->col[i];
  return DA_OK;
}

}  // extern "C"

namespace {

// The reassignment runs in the plan's workspace, or (use_scratch) in the library's static
// scratch of the plan's device, which must hold the plan's workspace layout.
da_status reassign_impl(da_plan p, const void* K, const void* V, const void* centroids_in,
                        void* centroids_out, void* mean_values_out, int32_t* assign_out,
                        int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                        float* key_variance_out, bool want_variance, bool use_scratch,
                        void* stream) {
  if (p == nullptr || K == nullptr || V == nullptr || centroids_in == nullptr ||
      centroids_out == nullptr || mean_values_out == nullptr || assign_out == nullptr ||
      cluster_sizes_out == nullptr || qblock_counts_out == nullptr ||
      (want_variance && key_variance_out == nullptr))
    return DA_ERR_INVALID_ARGUMENT;
  if (const da_status ds = check_device(p, stream); ds != DA_OK) return ds;
  const da_desc& d = p->desc;
  const size_t es = elem_size(d);
  const size_t cache_bytes = (size_t)d.heads * d.clusters * d.head_dim * es;
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(centroids_in, 16) ||
      !aligned(centroids_out, 16) || !aligned(mean_values_out, 16) || !aligned(assign_out, 4) ||
      !aligned(cluster_sizes_out, 4) || !aligned(qblock_counts_out, 4) ||
      (want_variance && !aligned(key_variance_out, 4)))
    return DA_ERR_INVALID_ARGUMENT;
  const size_t H = d.heads, N = d.seq_len, C = d.clusters;
  const void* outs[] = {centroids_out, mean_values_out, assign_out, cluster_sizes_out,
                        qblock_counts_out, key_variance_out};
  const size_t out_bytes[] = {cache_bytes, cache_bytes, H * N * 4, H * C * 4,
                              H * (size_t)p->nb * C * 4, want_variance ? H * C * 4 : 0};
  for (int i = 0; i < 6; ++i)
    if (out_bytes[i] && overlap(centroids_in, cache_bytes, outs[i], out_bytes[i]))
      return DA_ERR_INVALID_ARGUMENT;
  const WorkspaceLayout wl = workspace_layout(d, p->nb);
  char* ws = static_cast<char*>(p->d_ws);
  if (use_scratch) {
    void* sp = nullptr;
    if (wl.total > da::kScratchBytes) return DA_ERR_UNSUPPORTED;
    if (da::scratch_address(p->device, &sp) != hipSuccess || sp == nullptr) return DA_ERR_DEVICE;
    ws = static_cast<char*>(sp);
  }
  da::ReassignArgs a{};
  a.K = K;
  a.V = V;
  a.mu_in = centroids_in;
  a.mu_out = centroids_out;
  a.vbar_out = mean_values_out;
  a.assign = assign_out;
  a.sizes = cluster_sizes_out;
  a.counts = qblock_counts_out;
  a.rowptr = p->d_rowptr;
  a.col = p->d_col;
  a.prowptr = p->d_prowptr;
  a.pcol = p->d_pcol;
  a.npairs = p->npairs;
  a.hist = reinterpret_cast<uint8_t*>(ws + wl.hist);
  a.off = reinterpret_cast<int32_t*>(ws + wl.off);
  a.start = reinterpret_cast<int32_t*>(ws + wl.start);
  a.perm = reinterpret_cast<int32_t*>(ws + wl.perm);
  a.cop = reinterpret_cast<uint16_t*>(ws + wl.cop);
  a.part = reinterpret_cast<float*>(ws + wl.part);
  a.psq = reinterpret_cast<float*>(ws + wl.psq);
  a.kvar = want_variance ? key_variance_out : nullptr;
  a.fix = reinterpret_cast<int32_t*>(ws + wl.fix);
  a.H = d.heads;
  a.N = d.seq_len;
  a.C = d.clusters;
  a.nb = p->nb;
  a.block = d.block;
  a.mask_heads = d.mask_heads;
  a.kblock = p->kblock;
  a.ncu = p->ncu;
  const hipError_t e = da::launch_reassign(a, d.head_dim, d.dtype == DA_DTYPE_BF16,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_DEVICE;
}

da_status forward_impl(da_plan p, const void* Q, const void* K, const void* V,
                       const void* centroids, const void* mean_values,
                       const int32_t* qblock_counts, const float* key_variance,
                       bool want_variance, void* O, float* lse_out, void* stream) {
  if (p == nullptr || Q == nullptr || K == nullptr || V == nullptr || centroids == nullptr ||
      mean_values == nullptr || qblock_counts == nullptr || O == nullptr ||
      (want_variance && key_variance == nullptr))
    return DA_ERR_INVALID_ARGUMENT;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(centroids, 16) ||
      !aligned(mean_values, 16) || !aligned(O, 16) || !aligned(qblock_counts, 4) ||
      (lse_out != nullptr && !aligned(lse_out, 4)) ||
      (want_variance && !aligned(key_variance, 4)))
    return DA_ERR_INVALID_ARGUMENT;
  if (const da_status ds = check_device(p, stream); ds != DA_OK) return ds;
  const da_desc& d = p->desc;
  da::FwdArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.mu = centroids;
  a.vbar = mean_values;
  a.counts = qblock_counts;
  a.rowptr = p->d_rowptr;
  a.col = p->d_col;
  a.prowptr = p->d_prowptr;
  a.pcol = p->d_pcol;
  a.npairs = p->npairs;
  for (int x = 0; x < 9; ++x) a.xstart[x] = p->xstart[x];
  a.xmax = p->xmax;
  a.O = O;
  a.lse = lse_out;
  a.H = d.heads;
  a.N = d.seq_len;
  a.C = d.clusters;
  a.nb = p->nb;
  a.mask_heads = d.mask_heads;
  a.kblock = p->kblock;
  a.scale_log2e = p->scale * 1.4426950408889634f;
  a.kvar = want_variance ? key_variance : nullptr;
  const hipError_t e = da::launch_forward(a, d.head_dim, d.block, p->kblock,
                                          d.dtype == DA_DTYPE_BF16,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DA_OK : DA_ERR_DEVICE;
}

}  // namespace

extern "C" {

DA_API da_status da_reassign(da_plan p, const void* K, const void* V, const void* centroids_in,
                             void* centroids_out, void* mean_values_out, int32_t* assign_out,
                             int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                             void* stream) {
  return reassign_impl(p, K, V, centroids_in, centroids_out, mean_values_out, assign_out,
                       cluster_sizes_out, qblock_counts_out, nullptr, false, false, stream);
}

DA_API da_status da_reassign_noalloc(da_plan p, const void* K, const void* V,
                                     const void* centroids_in, void* centroids_out,
                                     void* mean_values_out, int32_t* assign_out,
                                     int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                                     void* stream) {
  return reassign_impl(p, K, V, centroids_in, centroids_out, mean_values_out, assign_out,
                       cluster_sizes_out, qblock_counts_out, nullptr, false, true, stream);
}

DA_API da_status da_reassign_var(da_plan p, const void* K, const void* V,
                                 const void* centroids_in, void* centroids_out,
                                 void* mean_values_out, int32_t* assign_out,
                                 int32_t* cluster_sizes_out, int32_t* qblock_counts_out,
                                 float* key_variance_out, void* stream) {
  return reassign_impl(p, K, V, centroids_in, centroids_out, mean_values_out, assign_out,
                       cluster_sizes_out, qblock_counts_out, key_variance_out, true, false,
                       stream);
}

DA_API da_status da_forward(da_plan p, const void* Q, const void* K, const void* V,
                            const void* centroids, const void* mean_values,
                            const int32_t* qblock_counts, void* O, float* lse_out,
                            void* stream) {
  return forward_impl(p, Q, K, V, centroids, mean_values, qblock_counts, nullptr, false, O,
                      lse_out, stream);
}

DA_API da_status da_forward_var(da_plan p, const void* Q, const void* K, const void* V,
                                const void* centroids, const void* mean_values,
                                const int32_t* qblock_counts, const float* key_variance,
                                void* O, float* lse_out, void* stream) {
  return forward_impl(p, Q, K, V, centroids, mean_values, qblock_counts, key_variance, true, O,
                      lse_out, stream);
}

}  // extern "C"

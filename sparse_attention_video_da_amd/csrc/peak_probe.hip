// Measured peaks of the two rooflines the library is held against on gfx950: the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16 issued back to back from independent accumulators) and HBM
// (a streaming read and a streaming copy). A measurement tool, built as its own library (libdapeak.so) and used by
// the benchmark only; not part of the attention ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Each wave runs `iters` rounds of 8 independent 32x32x16 MFMA chains (32768 flop each).
__global__ void __launch_bounds__(256) mfma_peak_kernel(float* out, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(l + e));
    b[e] = (__bf16)(0.002f * (float)(l - e));
  }
  f32x16 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the chains live
}

// dst[i] = src[i] over n 16-byte words (n a multiple of 4 * the grid's threads), grid-stride,
// four loads in flight per thread before the four stores.
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i + 3 * stride < n;
       i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
}

// Streaming read of n 16-byte words (same layout as the copy), folded into one word a thread.
__global__ void __launch_bounds__(256) read_kernel(const u32x4* __restrict__ src, size_t n,
                                                   uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i + 3 * stride < n;
       i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" __attribute__((visibility("default")))
int dapeak_mfma_bf16(int workgroups, int iters, float* out_dev, float* ms, double* flop) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, 0, out_dev, 16);
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, 0, out_dev, iters);
  (void)hipEventRecord(e1, 0);
  const int rc = hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess ? 0 : 1;
  (void)hipEventElapsedTime(ms, e0, e1);
  *flop = (double)workgroups * 4 * iters * 8 * 32768.0;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

extern "C" __attribute__((visibility("default")))
int dapeak_read(const void* src_dev, size_t bytes, int workgroups, int reps, uint32_t* out_dev,
                float* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(read_kernel, dim3(workgroups), dim3(256), 0, 0,
                     static_cast<const u32x4*>(src_dev), n, out_dev);
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(read_kernel, dim3(workgroups), dim3(256), 0, 0,
                       static_cast<const u32x4*>(src_dev), n, out_dev);
  (void)hipEventRecord(e1, 0);
  const int rc = hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess ? 0 : 1;
  (void)hipEventElapsedTime(ms, e0, e1);
  *ms /= (float)reps;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

extern "C" __attribute__((visibility("default")))
int dapeak_copy(const void* src_dev, void* dst_dev, size_t bytes, int workgroups, int reps,
                float* ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(copy_kernel, dim3(workgroups), dim3(256), 0, 0,
                     static_cast<const u32x4*>(src_dev), static_cast<u32x4*>(dst_dev), n);
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(copy_kernel, dim3(workgroups), dim3(256), 0, 0,
                       static_cast<const u32x4*>(src_dev), static_cast<u32x4*>(dst_dev), n);
  (void)hipEventRecord(e1, 0);
  const int rc = hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess ? 0 : 1;
  (void)hipEventElapsedTime(ms, e0, e1);
  *ms /= (float)reps;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

// Reassign Cache for gfx950: nearest-centroid assignment of every key, then the refresh
// of the cluster cache (centroid keys, mean values, sizes) and of the per-query-block
// counts n[b][c] (keys of cluster c outside query block b's exact key blocks).
//
// Kernel sequence per call (one stream, no host synchronisation):
//   1. assign        MFMA distance product against LDS-staged centroid chunks, per-lane
//                    running argmin (ties to the lowest index), written as int32.
//   2. block_hist    per key block, an LDS-atomic histogram of its keys' clusters.
//   3. col_scan      per cluster, exclusive prefix of the histograms over key blocks
//                    (where each block's keys start inside the cluster) and the sizes.
//   4. starts        per head, exclusive prefix of the sizes over clusters.
//   5. scatter       key index -> slot start[c] + off[kb][c] + rank within the block, so
//                    every cluster's keys sit contiguously in ascending key order.
//   6. cluster_sum   one wave per cluster sums its keys and values in that fixed order
//                    (fp32, deterministic), divides, rounds to the cache dtype.
//   7. counts        n[b][c] = size[c] - sum over b's exact blocks of hist[kb][c].
#include "da_device.h"
#include "da_internal.h"

namespace da {

constexpr float kPosInf = __builtin_inff();

// ----------------------------------------------------------------------------- 1. assign
// bf16: 4 waves x 64 keys per workgroup (2 key tiles of 32 per wave, two waves per SIMD so
// one wave's argmin VALU work overlaps the other's MFMAs). Centroids are staged CH at a
// time in swizzled LDS together with their squared norms; the score tile D^T = mu * K^T
// gives each lane one key and 16 centroids per 32-centroid tile, so the argmin stays in
// registers, and every centroid operand read from LDS feeds 2 MFMAs.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
assign_bf16_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ mu,
                   int32_t* __restrict__ assign, int N, int C) {
  constexpr int CH = 256;
  constexpr int DS = D / 16;
  constexpr int NCH = D / 8;
  constexpr int PER_T = CH * NCH / 256;
  constexpr int KTW = 2;           // key tiles (of 32) per wave
  __shared__ __attribute__((aligned(16))) char mu_lds[CH * D * 2];
  __shared__ __attribute__((aligned(16))) float norm_lds[CH];

  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int key0 = blockIdx.x * (4 * 32 * KTW) + w * (32 * KTW) + l32;
  const uint16_t* Kh = K + (size_t)h * N * D;
  const uint16_t* Mh = mu + (size_t)h * C * D;

  bf16x8 kreg[KTW][DS];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int key = key0 + 32 * kt;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      kreg[kt][s] = key < N ? *reinterpret_cast<const bf16x8*>(Kh + (size_t)key * D + 16 * s + 8 * hl)
                            : bf16x8{};
  }

  float best[KTW];
  int bidx[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    best[kt] = kPosInf;
    bidx[kt] = 0;
  }
  for (int c0 = 0; c0 < C; c0 += CH) {
    const int valid = min(CH, C - c0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = i * 256 + tid;
      const int row = idx / NCH;
      const int ch = idx - row * NCH;
      bf16x8 v = bf16x8{};
      if (row < valid) v = *reinterpret_cast<const bf16x8*>(Mh + (size_t)(c0 + row) * D + ch * 8);
      *reinterpret_cast<bf16x8*>(mu_lds + swz_byte<D>(row, ch)) = v;
    }
    __syncthreads();
    {
      float nrm = 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const bf16x8 v = lds_read_b128(mu_lds, swz_byte<D>(tid, ch));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)v[e];
          nrm = fmaf(x, x, nrm);
        }
      }
      norm_lds[tid] = tid < valid ? nrm : kPosInf;
    }
    __syncthreads();
    const int ntile = (valid + 31) / 32;
    for (int ct = 0; ct < ntile; ++ct) {
      f32x16 acc[KTW];
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) acc[kt] = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 a = lds_read_b128(mu_lds, swz_byte<D>(32 * ct + l32, 2 * s + hl));
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) acc[kt] = mfma32x32x16(a, kreg[kt][s], acc[kt]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 nv = *reinterpret_cast<const f32x4*>(norm_lds + 32 * ct + 8 * i + 4 * hl);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = c0 + 32 * ct + 8 * i + 4 * hl + j;
#pragma unroll
          for (int kt = 0; kt < KTW; ++kt) {
            const float dist = fmaf(-2.f, acc[kt][4 * i + j], nv[j]);
            if (dist < best[kt]) {   // ascending c per lane: ties keep the lower index
              best[kt] = dist;
              bidx[kt] = c;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const float ob = xor32(best[kt]);
    const int oi = __shfl_xor(bidx[kt], 32, 64);
    int bi = bidx[kt];
    if (ob < best[kt] || (ob == best[kt] && oi < bi)) bi = oi;
    const int key = key0 + 32 * kt;
    if (hl == 0 && key < N) assign[(size_t)h * N + key] = bi;
  }
}

// fp32: one key per thread, distances in difference form sum (k - mu)^2 in fp32 against
// LDS-staged centroid chunks (the fp32 layer is small; this keeps full fp32 accuracy).
template <int D>
__global__ void __launch_bounds__(256)
assign_f32_kernel(const float* __restrict__ K, const float* __restrict__ mu,
                  int32_t* __restrict__ assign, int N, int C) {
  constexpr int CH = 64;
  __shared__ float mu_lds[CH * D];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int key = blockIdx.x * 256 + tid;
  const float* Kh = K + (size_t)h * N * D;
  const float* Mh = mu + (size_t)h * C * D;
  float kreg[D];
#pragma unroll
  for (int e = 0; e < D; ++e) kreg[e] = key < N ? Kh[(size_t)key * D + e] : 0.f;
  float best = kPosInf;
  int bidx = 0;
  for (int c0 = 0; c0 < C; c0 += CH) {
    const int valid = min(CH, C - c0);
    __syncthreads();
    for (int i = tid; i < valid * D; i += 256) mu_lds[i] = Mh[(size_t)c0 * D + i];
    __syncthreads();
    for (int c = 0; c < valid; ++c) {
      float dist = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        const float df = kreg[e] - mu_lds[c * D + e];
        dist = fmaf(df, df, dist);
      }
      if (dist < best) {
        best = dist;
        bidx = c0 + c;
      }
    }
  }
  if (key < N) assign[(size_t)h * N + key] = bidx;
}

// ----------------------------------------------------------------------------- 2. hist
__global__ void __launch_bounds__(256)
block_hist_kernel(const int32_t* __restrict__ assign, uint8_t* __restrict__ hist, int N, int C,
                  int nb, int block) {
  extern __shared__ int32_t hist_lds[];
  const int h = blockIdx.y, kb = blockIdx.x, tid = threadIdx.x;
  for (int c = tid; c < C; c += 256) hist_lds[c] = 0;
  __syncthreads();
  const int j = kb * block + tid;
  if (tid < block && j < N) atomicAdd(&hist_lds[assign[(size_t)h * N + j]], 1);
  __syncthreads();
  uint8_t* dst = hist + ((size_t)h * nb + kb) * C;   // a block holds <= 128 keys
  for (int c = tid; c < C; c += 256) dst[c] = (uint8_t)hist_lds[c];
}

// ----------------------------------------------------------------------------- 3. col scan
// 16 waves split the key blocks; lane = cluster. Two passes over the histograms.
__global__ void __launch_bounds__(1024)
col_scan_kernel(const uint8_t* __restrict__ hist, int32_t* __restrict__ off,
                int32_t* __restrict__ sizes, int C, int nb) {
  __shared__ int32_t part[16][64];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int span = (nb + 15) / 16;
  const int kb0 = min(nb, w * span), kb1 = min(nb, kb0 + span);
  const uint8_t* col = hist + (size_t)h * nb * C + c;
  int s = 0;
  if (c < C)
    for (int kb = kb0; kb < kb1; ++kb) s += col[(size_t)kb * C];
  part[w][lane] = s;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pre += i < w ? part[i][lane] : 0;
    tot += part[i][lane];
  }
  if (c < C) {
    int32_t* ocol = off + (size_t)h * nb * C + c;
    int run = pre;
    for (int kb = kb0; kb < kb1; ++kb) {
      ocol[(size_t)kb * C] = run;
      run += col[(size_t)kb * C];
    }
    if (w == 0) sizes[(size_t)h * C + c] = tot;
  }
}

// ----------------------------------------------------------------------------- 4. starts
__global__ void __launch_bounds__(1024)
starts_kernel(const int32_t* __restrict__ sizes, int32_t* __restrict__ start, int C) {
  __shared__ int32_t buf[1024];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int per = (C + 1023) / 1024;
  const int c0 = min(C, tid * per), c1 = min(C, c0 + per);
  const int32_t* sz = sizes + (size_t)h * C;
  int s = 0;
  for (int c = c0; c < c1; ++c) s += sz[c];
  buf[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive Hillis-Steele scan
    const int v = tid >= d ? buf[tid - d] : 0;
    __syncthreads();
    buf[tid] += v;
    __syncthreads();
  }
  int run = buf[tid] - s;
  int32_t* st = start + (size_t)h * C;
  for (int c = c0; c < c1; ++c) {
    st[c] = run;
    run += sz[c];
  }
}

// ----------------------------------------------------------------------------- 5. scatter
__global__ void __launch_bounds__(256)
scatter_kernel(const int32_t* __restrict__ assign, const int32_t* __restrict__ off,
               const int32_t* __restrict__ start, int32_t* __restrict__ perm, int N, int C,
               int nb, int block) {
  __shared__ int32_t a_lds[256];
  const int h = blockIdx.y, kb = blockIdx.x, tid = threadIdx.x;
  const int j = kb * block + tid;
  const int c = (tid < block && j < N) ? assign[(size_t)h * N + j] : -1;
  a_lds[tid] = c;
  __syncthreads();
  if (c >= 0) {
    int r = 0;
    for (int t = 0; t < tid; ++t) r += a_lds[t] == c;
    const int pos = start[(size_t)h * C + c] + off[((size_t)h * nb + kb) * C + c] + r;
    perm[(size_t)h * N + pos] = j;
  }
}

// ----------------------------------------------------------------------------- 6. sums
// One wave per cluster; each lane owns D/64 consecutive dims. Keys are visited in the
// scattered (ascending) order, 8 rows in flight.
template <int D, bool BF16>
__global__ void __launch_bounds__(256)
cluster_sum_kernel(const void* __restrict__ Kv, const void* __restrict__ Vv,
                   const void* __restrict__ mu_in, void* __restrict__ mu_out,
                   void* __restrict__ vbar_out, const int32_t* __restrict__ sizes,
                   const int32_t* __restrict__ start, const int32_t* __restrict__ perm, int N,
                   int C) {
  constexpr int EPL = D / 64;
  constexpr int U = 16;
  const int h = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + w;
  if (c >= C) return;
  const int cnt = sizes[(size_t)h * C + c];
  const int32_t* pl = perm + (size_t)h * N + start[(size_t)h * C + c];
  float ks[EPL], vs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ks[e] = vs[e] = 0.f;

  auto load_row = [&](const void* base, int j, float* out) {
    if constexpr (BF16) {
      const uint16_t* r = static_cast<const uint16_t*>(base) + ((size_t)h * N + j) * D + lane * EPL;
      if constexpr (EPL == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(r);
        out[0] = __uint_as_float(u << 16);
        out[1] = __uint_as_float(u & 0xffff0000u);
      } else {
        out[0] = bf16_to_f32(r[0]);
      }
    } else {
      const float* r = static_cast<const float*>(base) + ((size_t)h * N + j) * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) out[e] = r[e];
    }
  };

  int i = 0;
  for (; i + U <= cnt; i += U) {
    float kr[U][EPL], vr[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = pl[i + u];
      load_row(Kv, j, kr[u]);
      load_row(Vv, j, vr[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ks[e] += kr[u][e];
        vs[e] += vr[u][e];
      }
  }
  for (; i < cnt; ++i) {
    float kr[EPL], vr[EPL];
    const int j = pl[i];
    load_row(Kv, j, kr);
    load_row(Vv, j, vr);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      ks[e] += kr[e];
      vs[e] += vr[e];
    }
  }
  const size_t o = ((size_t)h * C + c) * D + lane * EPL;
  const float fc = (float)cnt;
  if constexpr (BF16) {
    uint16_t* mo = static_cast<uint16_t*>(mu_out) + o;
    uint16_t* vo = static_cast<uint16_t*>(vbar_out) + o;
    const uint16_t* mi = static_cast<const uint16_t*>(mu_in) + o;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mo[e] = cnt > 0 ? f32_to_bf16_rne(ks[e] / fc) : mi[e];
      vo[e] = cnt > 0 ? f32_to_bf16_rne(vs[e] / fc) : (uint16_t)0;
    }
  } else {
    float* mo = static_cast<float*>(mu_out) + o;
    float* vo = static_cast<float*>(vbar_out) + o;
    const float* mi = static_cast<const float*>(mu_in) + o;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mo[e] = cnt > 0 ? ks[e] / fc : mi[e];
      vo[e] = cnt > 0 ? vs[e] / fc : 0.f;
    }
  }
}

// ----------------------------------------------------------------------------- 7. counts
// n[b][c] = size[c] - sum over b's exact blocks of hist[kb][c]; 4 clusters per thread from
// the byte histograms (one head's histograms stay resident in L2 across its query blocks).
__global__ void __launch_bounds__(256)
counts_kernel(const uint8_t* __restrict__ hist, const int32_t* __restrict__ sizes,
              const int32_t* __restrict__ rowptr, const int32_t* __restrict__ col,
              int32_t* __restrict__ counts, int C, int nb, int mask_heads) {
  const int h = blockIdx.y, b = blockIdx.x;
  const int mh = mask_heads == 1 ? 0 : h;
  const int e0 = rowptr[mh * (nb + 1) + b], e1 = rowptr[mh * (nb + 1) + b + 1];
  const uint8_t* hh = hist + (size_t)h * nb * C;
  int32_t* dst = counts + ((size_t)h * nb + b) * C;
  const int32_t* sz = sizes + (size_t)h * C;
  if ((C & 3) == 0) {
    for (int c = 4 * threadIdx.x; c < C; c += 4 * 256) {
      int n0 = sz[c], n1 = sz[c + 1], n2 = sz[c + 2], n3 = sz[c + 3];
      for (int e = e0; e < e1; ++e) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(hh + (size_t)col[e] * C + c);
        n0 -= v & 0xff;
        n1 -= (v >> 8) & 0xff;
        n2 -= (v >> 16) & 0xff;
        n3 -= v >> 24;
      }
      *reinterpret_cast<int4*>(dst + c) = make_int4(n0, n1, n2, n3);
    }
  } else {
    for (int c = threadIdx.x; c < C; c += 256) {
      int n = sz[c];
      for (int e = e0; e < e1; ++e) n -= hh[(size_t)col[e] * C + c];
      dst[c] = n;
    }
  }
}

// ----------------------------------------------------------------------------- launch
template <int D>
static hipError_t launch_reassign_t(const ReassignArgs& a, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((assign_bf16_kernel<D>), dim3((a.N + 255) / 256, a.H), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.mu_in),
                       a.assign, a.N, a.C);
  else
    hipLaunchKernelGGL((assign_f32_kernel<D>), dim3((a.N + 255) / 256, a.H), dim3(256), 0, s,
                       static_cast<const float*>(a.K), static_cast<const float*>(a.mu_in),
                       a.assign, a.N, a.C);
  hipLaunchKernelGGL(block_hist_kernel, dim3(a.nb, a.H), dim3(256), a.C * sizeof(int32_t), s,
                     a.assign, a.hist, a.N, a.C, a.nb, a.block);
  hipLaunchKernelGGL(col_scan_kernel, dim3((a.C + 63) / 64, a.H), dim3(1024), 0, s, a.hist,
                     a.off, a.sizes, a.C, a.nb);
  hipLaunchKernelGGL(starts_kernel, dim3(a.H), dim3(1024), 0, s, a.sizes, a.start, a.C);
  hipLaunchKernelGGL(scatter_kernel, dim3(a.nb, a.H), dim3(256), 0, s, a.assign, a.off,
                     a.start, a.perm, a.N, a.C, a.nb, a.block);
  if (bf16)
    hipLaunchKernelGGL((cluster_sum_kernel<D, true>), dim3((a.C + 3) / 4, a.H), dim3(256), 0, s,
                       a.K, a.V, a.mu_in, a.mu_out, a.vbar_out, a.sizes, a.start, a.perm, a.N,
                       a.C);
  else
    hipLaunchKernelGGL((cluster_sum_kernel<D, false>), dim3((a.C + 3) / 4, a.H), dim3(256), 0,
                       s, a.K, a.V, a.mu_in, a.mu_out, a.vbar_out, a.sizes, a.start, a.perm,
                       a.N, a.C);
  hipLaunchKernelGGL(counts_kernel, dim3(a.nb, a.H), dim3(256), 0, s, a.hist, a.sizes,
                     a.rowptr, a.col, a.counts, a.C, a.nb, a.mask_heads);
  return hipGetLastError();
}

hipError_t launch_reassign(const ReassignArgs& a, int head_dim, bool bf16, hipStream_t s) {
  if (head_dim == 64) return launch_reassign_t<64>(a, bf16, s);
  if (head_dim == 128) return launch_reassign_t<128>(a, bf16, s);
  return hipErrorInvalidValue;
}

hipError_t prepare_reassign_kernels() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&block_hist_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(8192 * sizeof(int32_t)));
}

}  // namespace da

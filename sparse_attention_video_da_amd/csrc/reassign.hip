// Reassign Cache for gfx950: nearest-centroid assignment of every key, then the refresh
// of the cluster cache (centroid keys, mean values, sizes) and of the per-query-block
// counts n[b][c] (keys of cluster c outside query block b's exact key blocks).
//
// Kernel sequence per call (one stream, no host synchronisation):
//   0. operands      (bf16) per centroid: -2 mu and the split |mu|^2 row for the MFMA;
//                    clears the per-head near-tie counters.
//   1. assign        MFMA distance product against centroid operands in LDS (bf16: the
//                    whole table of a head resident when it fits in 128 KB, with a
//                    persistent grid; streamed in chunks otherwise), per-lane running top
//                    two, the nearest written as int32; keys whose top two are too close for
//                    the expanded-form arithmetic go to a per-head near-tie list (fp32:
//                    difference form, lowest index on ties). The resident form also writes
//                    each key block's cluster histogram.
//   1b. near ties    (bf16) the listed keys re-measured in difference form against every
//                    centroid that could be their nearest; lowest index on equal distances;
//                    a moved key's histogram counters are patched.
//   2. block_hist    (streamed and fp32 assignments) per key block, an LDS-atomic
//                    histogram of its keys' clusters.
//   3. col_scan      per cluster, exclusive prefix of the histograms over key blocks
//                    (where each block's keys start inside the cluster) and the sizes.
//   4. starts        per head, exclusive prefix of the sizes over clusters.
//   5. scatter       key index -> slot start[c] + off[kb][c] + rank within the block, so
//                    every cluster's keys sit contiguously in ascending key order.
//   6. sums          fixed-size segments of the sorted order give fp32 partial sums per
//                    cluster run, then one wave per cluster adds its partials in order,
//                    divides and rounds to the cache dtype (deterministic throughout); with
//                    the key variance requested, the squared key norms ride along and the
//                    finish writes each cluster's isotropic key variance.
//   7. counts        n[b][c] = size[c] - sum over b's exact blocks of hist[kb][c], per pair
//                    (with key blocks smaller than the query blocks: size[c] minus the
//                    exact keys of cluster c, read from the assignments).
#include <mutex>
#include <utility>
#include <vector>

#include "da_device.h"
#include "da_internal.h"

namespace da {

constexpr float kPosInf = __builtin_inff();
#ifndef ASG_WAVES
#define ASG_WAVES 4
#endif
#ifndef ASG_CH
#define ASG_CH 128
#endif
// VALU instructions scheduled beside each group of the assignment's pipelined MFMAs
#ifndef ASG_NV
#define ASG_NV 12
#endif

// ----------------------------------------------------------------------------- 1. assign
// bf16 distances come straight out of the MFMA. Per centroid, a pre-pass writes the product
// operands: -2 mu (exact in bf16) and an 8-element row [h, m, l, 1, 1, 1, 0, 0] whose three
// bf16 parts h + m + l carry |mu|^2 (fp32, about 24 bits). Each key gets the matching row
// [1, 1, 1, h', m', l', 0, 0] for |k|^2, so one extra 16-deep MFMA step (of D/16 + 1) leaves
// the squared distance |k|^2 + |mu|^2 - 2 k.mu in the accumulator.
// |mu|^2 is summed in fp64 (the squares of bf16 values are exact there, the sum nearly so),
// so the three parts carry it to about 2^-24 relative. The kernel also clears the
// per-head counters of the near-tie lists that the assignment fills.
template <int D>
__global__ void __launch_bounds__(256)
centroid_operands_kernel(const uint16_t* __restrict__ mu, uint16_t* __restrict__ mup,
                         uint16_t* __restrict__ aug, int32_t* __restrict__ fix_count, int C) {
  const int h = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c == 0) fix_count[h] = 0;
  if (c >= C) return;
  const size_t row = (size_t)h * C + c;
  const uint16_t* src = mu + row * D;
  uint16_t* dst = mup + row * D;
  double nrm = 0.0;
#pragma unroll
  for (int ch = 0; ch < D / 8; ++ch) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * ch);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = bf16_to_f32((uint16_t)(wv[q] & 0xffffu));
      const float hi = bf16_to_f32((uint16_t)(wv[q] >> 16));
      nrm = fma((double)lo, (double)lo, nrm);
      nrm = fma((double)hi, (double)hi, nrm);
      // -2x is exact in bf16 (finite inputs): flip the sign, double through fp32
      o[q] = (uint32_t)f32_to_bf16_rne(-2.f * lo) | ((uint32_t)f32_to_bf16_rne(-2.f * hi) << 16);
    }
    *reinterpret_cast<uint4*>(dst + 8 * ch) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  // three bf16 parts of the fp64 norm (each part rounds the remainder left by the previous)
  const uint16_t n0 = f32_to_bf16_rne((float)nrm);
  const double r1 = nrm - (double)bf16_to_f32(n0);
  const uint16_t n1 = f32_to_bf16_rne((float)r1);
  const uint16_t n2 = f32_to_bf16_rne((float)(r1 - (double)bf16_to_f32(n1)));
  constexpr uint16_t kOne = 0x3f80;
  *reinterpret_cast<uint4*>(aug + row * 8) =
      make_uint4((uint32_t)n0 | ((uint32_t)n1 << 16), (uint32_t)n2 | ((uint32_t)kOne << 16),
                 (uint32_t)kOne | ((uint32_t)kOne << 16), 0u);
}

__device__ __forceinline__ int min3i(int a, int b, int c) { return min(a, min(b, c)); }
// median of three (compiled to one v_med3_i32)
__device__ __forceinline__ int med3i(int a, int b, int c) { return max(min(a, b), min(max(a, b), c)); }

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xf) | (0x7 << 4) | (0xf << 8) | ((n >> 4) << 14); }

// One wave's share of the bf16 assignment: 2 key tiles of 32 keys. The score tile
// D^T = mu * K^T gives each lane one key and 16 centroids per 32-centroid tile; the lane
// packs a 5-bit tile-local index into the low mantissa bits of each distance (a change
// below 2^-18 relative, far inside the 1e-4 tie band) and keeps the integer minimum with
// three-way mins. Distances are non-negative up to rounding; a slightly negative one (a key
// equal to a centroid) orders below every positive one as an integer, which is the right
// winner.
constexpr int kAsgKtw = 2;

// |k|^2 of a lane's half row (D/2 bf16 values) by packed bf16 dot products, four partial
// sums. Its rounding shifts every distance of the key alike, so it moves neither the nearest
// centroid nor the top-two gap; the assignment and the near-tie pass must take it the same
// way, since the pass compares its distances with the assignment's.
template <int D>
__device__ __forceinline__ float half_row_sq_norm(const bf16x8 (&row)[D / 16]) {
  float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 x = {row[s][2 * e], row[s][2 * e + 1]};
      part[e] = __builtin_amdgcn_fdot2_f32_bf16(x, x, part[e], false);
    }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// This lane's keys: the B operand of D^T = mu K^T (dims 16s + 8hl .. +7), and the
// augmented row for |k|^2 on the lower half (zero on the upper half, so whatever the
// centroid side holds in dims 8..15 of that step contributes nothing). The loads go through
// a buffer resource over the head's keys (32-bit offsets; keys at or past N read as zero).
template <int D>
__device__ __forceinline__ void assign_load_keys(__amdgpu_buffer_rsrc_t rK, int key0, int hl,
                                                 bf16x8 (&kreg)[kAsgKtw][D / 16],
                                                 bf16x8 (&kaug)[kAsgKtw],
                                                 float (&knorm)[kAsgKtw]) {
  constexpr int DS = D / 16;
#pragma unroll
  for (int kt = 0; kt < kAsgKtw; ++kt) {
    const int key = key0 + 32 * kt;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      kreg[kt][s] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rK, (key * D + 16 * s + 8 * hl) * 2, 0, 0));
    const float ps = half_row_sq_norm<D>(kreg[kt]);
    const float nk = ps + xor32(ps);
    knorm[kt] = nk;
    const __bf16 n0 = (__bf16)nk;
    const float r1 = nk - (float)n0;
    const __bf16 n1 = (__bf16)r1;
    const __bf16 n2 = (__bf16)(r1 - (float)n1);
    const __bf16 one = (__bf16)1.f, zero = (__bf16)0.f;
    kaug[kt] = hl == 0 ? bf16x8{one, one, one, n0, n1, n2, zero, zero} : bf16x8{};
  }
}

// Running top two (packed) of this wave's keys over one 32-centroid distance tile starting at
// centroid cbase; centroids at or past `limit` (a ragged last tile) are excluded. Accumulator r
// of a lane holds centroid cbase + 8(r/4) + 4hl + r%4: its distance with the tile-local index
// 8(r/4) + r%4 packed into the 5 low mantissa bits.
__device__ __forceinline__ void tile_top2(const f32x16 (&acc)[kAsgKtw], int cbase, bool ragged,
                                          int limit, int hl, int (&bestp)[kAsgKtw],
                                          int (&bbase)[kAsgKtw], int (&secp)[kAsgKtw]) {
#pragma unroll
  for (int kt = 0; kt < kAsgKtw; ++kt) {
    int pk[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pk[r] = (int)((__float_as_uint(acc[kt][r]) & ~0x1fu) | (uint32_t)(8 * (r >> 2) + (r & 3)));
      if (ragged && cbase + 8 * (r >> 2) + 4 * hl + (r & 3) >= limit) pk[r] = 0x7fffffff;
    }
    // smallest and second smallest of the 16 by a network of 3-way mins and medians: the
    // median of three is their second smallest; five groups of three plus pk[15] give six
    // minima, whose own top two (two more groups of three) and the groups' seconds give the
    // tile's second (the smaller of the minima's second and the winning group's second,
    // which is the smallest group second that can matter)
    int gm[5], gs[5];
#pragma unroll
    for (int g = 0; g < 5; ++g) {
      gm[g] = min3i(pk[3 * g], pk[3 * g + 1], pk[3 * g + 2]);
      gs[g] = med3i(pk[3 * g], pk[3 * g + 1], pk[3 * g + 2]);
    }
    const int a1 = min3i(gm[0], gm[1], gm[2]), a2 = med3i(gm[0], gm[1], gm[2]);
    const int c1 = min3i(gm[3], gm[4], pk[15]), c2 = med3i(gm[3], gm[4], pk[15]);
    const int m = min(a1, c1);
    const int sv = min(min3i(max(a1, c1), a2, c2), min3i(min3i(gs[0], gs[1], gs[2]), gs[3], gs[4]));
    // running top two over the tiles: the second is the smaller of the larger of the two
    // minima and the two seconds
    secp[kt] = min(max(bestp[kt], m), min(secp[kt], sv));
    if (m < bestp[kt]) {
      bestp[kt] = m;
      bbase[kt] = cbase;
    }
  }
}

// Distance tiles of this wave's keys against the centroid rows of an LDS table (-2 mu rows
// swizzled, then the augmented rows): D/16 + 1 MFMAs per key tile.
template <int D>
struct AsgTiles {
  static constexpr int DS = D / 16;
  const char* ms;
  const char* as;
  int l32, hl;
  const bf16x8 (&kreg)[kAsgKtw][D / 16];
  const bf16x8 (&kaug)[kAsgKtw];
  __device__ __forceinline__ void load_ops(int ct, bf16x8 (&o)[DS + 1]) const {
#pragma unroll
    for (int s = 0; s < DS; ++s) o[s] = lds_read_b128(ms, swz_byte<D>(32 * ct + l32, 2 * s + hl));
    o[DS] = lds_read_b128(as, (32 * ct + l32) * 16);
  }
  __device__ __forceinline__ void mfma_ops(const bf16x8 (&o)[DS + 1],
                                           f32x16 (&acc)[kAsgKtw]) const {
#pragma unroll
    for (int kt = 0; kt < kAsgKtw; ++kt) acc[kt] = f32x16{};
#pragma unroll
    for (int s = 0; s <= DS; ++s)
#pragma unroll
      for (int kt = 0; kt < kAsgKtw; ++kt)
        acc[kt] = mfma32x32x16(o[s], s < DS ? kreg[kt][s] : kaug[kt], acc[kt]);
  }
  __device__ __forceinline__ void tile(int ct, f32x16 (&acc)[kAsgKtw]) const {
    bf16x8 o[DS + 1];
    load_ops(ct, o);
    mfma_ops(o, acc);
  }
};

// Scheduling groups beside one tile's MFMAs: KTW MFMAs, one LDS operand read and ASG_NV VALU
// instructions per k-step, so the next tile's products run beside this tile's argmin.
template <int D>
__device__ __forceinline__ void asg_sched_groups() {
#pragma unroll
  for (int g = 0; g < D / 16 + 1; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, kAsgKtw, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, ASG_NV, 0);
  }
}

// Running top two of this wave's keys over one LDS chunk of centroid operands: rows
// c0 .. c0 + valid - 1 (valid <= CH), stored as the staging below lays them out.
template <int D, int CH>
__device__ __forceinline__ void assign_chunk(const char* ms, const char* as, int c0, int valid,
                                             int l32, int hl,
                                             const bf16x8 (&kreg)[kAsgKtw][D / 16],
                                             const bf16x8 (&kaug)[kAsgKtw],
                                             int (&bestp)[kAsgKtw], int (&bbase)[kAsgKtw],
                                             int (&secp)[kAsgKtw]) {
  constexpr int DS = D / 16;
  constexpr int KTW = kAsgKtw;
  const AsgTiles<D> T{ms, as, l32, hl, kreg, kaug};
  constexpr int NT = CH / 32;
  if (valid == CH) {
    // full chunk, software-pipelined: the MFMAs of tile t+1 run beside the argmin of t,
    // and the centroid operands of tile t+2 are read meanwhile into the register set
    // tile t has just released
    f32x16 acc[2][KTW];
    bf16x8 ops[2][DS + 1];
    T.load_ops(0, ops[0]);
    if (NT > 1) T.load_ops(1, ops[1]);
    T.mfma_ops(ops[0], acc[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t + 1 < NT) T.mfma_ops(ops[(t + 1) & 1], acc[(t + 1) & 1]);
      if (t + 2 < NT) T.load_ops(t + 2, ops[t & 1]);
      tile_top2(acc[t & 1], c0 + 32 * t, false, 0, hl, bestp, bbase, secp);
      if (t + 1 < NT) asg_sched_groups<D>();
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    const int ntile = (valid + 31) / 32;
    for (int ct = 0; ct < ntile; ++ct) {
      f32x16 acc[KTW];
      T.tile(ct, acc);
      tile_top2(acc, c0 + 32 * ct, 32 * ct + 32 > valid, c0 + valid, hl, bestp, bbase, secp);
    }
  }
}

// Running top two over a whole resident table of C centroids (rows contiguous in LDS): one
// software pipeline across an even number of full 32-centroid tiles (no restart at chunk
// edges), then an odd last full tile and the ragged tile of C % 32 centroids one at a time.
template <int D>
__device__ __forceinline__ void assign_table(const char* ms, const char* as, int C, int l32,
                                             int hl, const bf16x8 (&kreg)[kAsgKtw][D / 16],
                                             const bf16x8 (&kaug)[kAsgKtw],
                                             int (&bestp)[kAsgKtw], int (&bbase)[kAsgKtw],
                                             int (&secp)[kAsgKtw]) {
  constexpr int DS = D / 16;
  constexpr int KTW = kAsgKtw;
  const AsgTiles<D> T{ms, as, l32, hl, kreg, kaug};
  const int ntp = (C >> 5) & ~1;   // full tiles taken in pairs
  if (ntp > 0) {
    f32x16 acc[2][KTW];
    bf16x8 ops[2][DS + 1];
    T.load_ops(0, ops[0]);
    T.load_ops(1, ops[1]);
    T.mfma_ops(ops[0], acc[0]);
    __builtin_amdgcn_sched_barrier(0);
    // steady state, two tiles a trip: the argmin of tile t beside the MFMAs of tile t+1,
    // while tile t+2's operands load into the registers tile t's MFMAs have released
    for (int t = 0; t + 2 < ntp; t += 2) {
      T.mfma_ops(ops[1], acc[1]);
      T.load_ops(t + 2, ops[0]);
      tile_top2(acc[0], 32 * t, false, 0, hl, bestp, bbase, secp);
      asg_sched_groups<D>();
      __builtin_amdgcn_sched_barrier(0);
      T.mfma_ops(ops[0], acc[0]);
      T.load_ops(t + 3, ops[1]);
      tile_top2(acc[1], 32 * t + 32, false, 0, hl, bestp, bbase, secp);
      asg_sched_groups<D>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the last pair: tile ntp-1's MFMAs beside tile ntp-2's argmin, then its own argmin
    T.mfma_ops(ops[1], acc[1]);
    tile_top2(acc[0], 32 * (ntp - 2), false, 0, hl, bestp, bbase, secp);
    asg_sched_groups<D>();
    __builtin_amdgcn_sched_barrier(0);
    tile_top2(acc[1], 32 * (ntp - 1), false, 0, hl, bestp, bbase, secp);
  }
  for (int ct = ntp; ct < (C + 31) / 32; ++ct) {   // an odd full tile, the ragged tile
    f32x16 acc[KTW];
    T.tile(ct, acc);
    tile_top2(acc, 32 * ct, 32 * ct + 32 > C, C, hl, bestp, bbase, secp);
  }
}

// Near ties. The squared distance |k|^2 + |mu|^2 - 2 k.mu leaves the MFMA with a rounding error
// that scales with |k|^2 + |mu|^2, not with the distance: keys far from the origin with a close
// second centroid can come out in the wrong order. An in-bounds check of the bf16 MFMA on
// gfx950 shows exact products aligned to the largest of the 17 terms (16 products and the
// accumulator) and kept down to 2^-24 of its leading power of two (a term one binade lower is
// dropped), then one round-to-nearest-even. Each 16-deep step is therefore off by less than
// 17 truncations and a rounding, 18 * 2^-24 of its largest term, and every term here is at
// most |k|^2 + |mu|^2. Over D/16 + 1 <= 9 steps, with |mu|^2 carried to 2^-24 and the packed
// index below 2^-18 of the value, every computed distance is within
//   E = kTieErr * (|k|^2 + max_c |mu_c|^2)  (+ 2^-18 of itself)
// of the true one, with kTieErr = 2^-16 (162 * 2^-24 < 2^-16 by a factor of 1.6). A key whose
// two smallest computed distances are further apart than 2E (+ the packing slack) has the
// true nearest centroid; any other key is listed with its smallest computed distance, and a
// second kernel re-measures it: every centroid whose computed distance lies within 2E of that
// smallest is a candidate (no other can be the nearest), and each candidate's distance is
// taken again as an fp32 sum of squared differences (error below 1e-5 of the distance).
constexpr float kTieErr = 1.0f / 65536.f;   // 2^-16

// Upper limit of the computed distance of any centroid that could be the nearest of a listed
// key: its smallest packed distance (low index bits cleared), plus 2E, plus the packing slack.
__device__ __forceinline__ float near_tie_limit(int b1, float knorm, float mu2max) {
  const float q1 = __int_as_float(b1 & ~0x1f);
  return q1 + 2.f * kTieErr * (knorm + mu2max) + 0x1p-16f * fabsf(q1);
}

// Merge the two half-waves' top two of each key (ties to the lower centroid), store the
// nearest and append keys whose top two are too close to tell apart to the head's near-tie
// list, entries (key, smallest packed distance).
__device__ __forceinline__ void assign_store(const int (&bestp)[kAsgKtw],
                                             const int (&bbase)[kAsgKtw],
                                             const int (&secp)[kAsgKtw],
                                             const float (&knorm)[kAsgKtw], float mu2max,
                                             int hl, int key0, int N,
                                             int32_t* __restrict__ assign_h,
                                             int32_t* __restrict__ fix_count_h,
                                             int2* __restrict__ fix_list_h,
                                             uint32_t* hist_lds) {
#pragma unroll
  for (int kt = 0; kt < kAsgKtw; ++kt) {
    const int mv = bestp[kt] & ~0x1f;
    const int mc = bbase[kt] + (bestp[kt] & 0x1f) + 4 * hl;
    const int ov = __shfl_xor(mv, 32, 64);
    const int oc = __shfl_xor(mc, 32, 64);
    const int bi = (ov < mv || (ov == mv && oc < mc)) ? oc : mc;
    // top two over both halves: min of the larger best and the smaller second
    const int ob = __shfl_xor(bestp[kt], 32, 64);
    const int os = __shfl_xor(secp[kt], 32, 64);
    const int b1 = min(bestp[kt], ob);
    const int b2 = min(max(bestp[kt], ob), min(secp[kt], os));
    const int key = key0 + 32 * kt;
    // every other centroid's computed distance is at least the second's (low bits cleared):
    // past the limit, none of them can be the nearest
    const bool near = hl == 0 && key < N && b2 != 0x7fffffff &&
                      !(__int_as_float(b2 & ~0x1f) > near_tie_limit(b1, knorm[kt], mu2max));
    if (hl == 0 && key < N) {
      assign_h[key] = bi;
      // the block's cluster histogram (16-bit counters, two to a word)
      if (hist_lds != nullptr) atomicAdd(&hist_lds[bi >> 1], 1u << (16 * (bi & 1)));
    }
    // wave-compacted append: one counter update per wave
    const uint64_t ball = __builtin_amdgcn_ballot_w64(near);
    if (ball != 0) {
      const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      int base = 0;
      if (lane == 0) base = atomicAdd(fix_count_h, (int)__builtin_popcountll(ball));
      base = __shfl(base, 0, 64);
      if (near) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0u));
        fix_list_h[base + below] = make_int2(key, b1);
      }
    }
  }
}

// Largest |mu|^2 over centroid rows [0, rows) of an LDS block of augmented rows (the three
// bf16 parts of each norm lead the row), wave-wide.
__device__ __forceinline__ float aug_norm_max(const char* as, int rows, int lane) {
  float m = 0.f;
  for (int r = lane; r < rows; r += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(as + r * 16);
    const float n = bf16_to_f32((uint16_t)(v.x & 0xffffu)) + bf16_to_f32((uint16_t)(v.x >> 16)) +
                    bf16_to_f32((uint16_t)(v.y & 0xffffu));
    m = fmaxf(m, n);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// Stage centroid rows c0 .. c0 + CH - 1 of one head (rows past C re-read row C - 1; their
// distances are masked) into an LDS chunk: the -2 mu operands swizzled by row, and the
// augmented rows, by direct buffer loads. The threads of the workgroup share the work.
template <int D, int CH, int THREADS>
__device__ __forceinline__ void assign_stage(__amdgpu_buffer_rsrc_t rM, __amdgpu_buffer_rsrc_t rA,
                                             int c0, int C, int tid, int w, char* ms, char* as) {
  constexpr int NCH = D / 8;
  constexpr int PER_T = CH * NCH / THREADS;
  static_assert(PER_T * THREADS == CH * NCH, "chunk must split evenly");
  const int valid = min(CH, C - c0);
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    const int slot = i * THREADS + tid;
    const int row = slot / NCH;
    const int pc = slot - row * NCH;
    const int off = (c0 + min(row, valid - 1)) * (D * 2) + ((pc ^ swz_key<D>(row)) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rM, (__attribute__((address_space(3))) void*)(ms + (i * THREADS + w * 64) * 16), 16,
        off, 0, 0, 0);
  }
  static_assert(CH % 64 == 0 && CH <= THREADS, "augmented rows: one load per thread");
  if (tid < CH)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rA, (__attribute__((address_space(3))) void*)(as + w * 64 * 16), 16,
        (c0 + min(tid, valid - 1)) * 16, 0, 0, 0);
}

// Streaming form, any C: WAVES waves x 64 keys per workgroup (4 waves, two workgroups per
// CU, by default). Centroid chunks of CH (128 by default) stream into two swizzled LDS
// buffers by direct buffer loads, each waited for on its own.
template <int D, int WAVES, int CH>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
assign_bf16_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ mup,
                   const uint16_t* __restrict__ aug, int32_t* __restrict__ assign,
                   int32_t* __restrict__ fix_count, int2* __restrict__ fix_list, int N,
                   int C) {
  constexpr int DS = D / 16;
  constexpr int NCH = D / 8;
  constexpr int THREADS = WAVES * 64;
  constexpr int KTW = kAsgKtw;
  constexpr int KEYS = (THREADS / 64) * 32 * KTW;
  constexpr int PER_T = CH * NCH / THREADS;
  __shared__ __attribute__((aligned(256))) char mu_s0[CH * D * 2];
  __shared__ __attribute__((aligned(256))) char mu_s1[CH * D * 2];
  __shared__ __attribute__((aligned(16))) char aug_s0[CH * 16];
  __shared__ __attribute__((aligned(16))) char aug_s1[CH * 16];

  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int key0 = blockIdx.x * KEYS + w * (32 * KTW) + l32;
  const uint16_t* Kh = K + (size_t)h * N * D;
  const __amdgpu_buffer_rsrc_t rM = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(mup + (size_t)h * C * D), (short)0, C * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(aug + (size_t)h * C * 8), (short)0, C * 16, kBufferWord3);
  const int nchunks = (C + CH - 1) / CH;

  bf16x8 kreg[KTW][DS];
  bf16x8 kaug[KTW];
  float knorm[KTW];
  const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kh, (short)0, N * D * 2, kBufferWord3);
  assign_load_keys<D>(rK, key0, hl, kreg, kaug, knorm);

  // The centroid chunks are staged after the key loads are issued, so waiting for a chunk
  // (vmcnt counts in issue order) never waits for more than the loads issued after it.
  assign_stage<D, CH, THREADS>(rM, rA, 0, C, tid, w, mu_s0, aug_s0);
  if (nchunks > 1) assign_stage<D, CH, THREADS>(rM, rA, CH, C, tid, w, mu_s1, aug_s1);

  int bestp[KTW], bbase[KTW], secp[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    bestp[kt] = secp[kt] = 0x7fffffff;
    bbase[kt] = 0;
  }
  float mu2max = 0.f;   // largest |mu|^2 of the chunks seen (for the near-tie bound)
  auto compute = [&](int ci, const char* ms, const char* as) {
    mu2max = fmaxf(mu2max, aug_norm_max(as, min(CH, C - ci * CH), lane));
    assign_chunk<D, CH>(ms, as, ci * CH, min(CH, C - ci * CH), l32, hl, kreg, kaug, bestp, bbase,
                        secp);
  };
  // Chunk ci sits in buffer ci % 2. Before computing it, each thread waits only until its
  // loads of chunk ci are done (the next chunk's may still be in flight), then the
  // workgroup meets; once every wave is done with a buffer, chunk ci + 2 streams into it.
  auto wait_chunk = [&](bool next_in_flight) {
    if (next_in_flight) {
      if (w * 64 < CH) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_T + 1));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_T));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();
  };
  for (int ci = 0; ci < nchunks; ci += 2) {
    wait_chunk(ci + 1 < nchunks);
    compute(ci, mu_s0, aug_s0);
    if (ci + 1 < nchunks) {
      __builtin_amdgcn_s_barrier();   // every wave is done with buffer 0
      if (ci + 2 < nchunks) assign_stage<D, CH, THREADS>(rM, rA, (ci + 2) * CH, C, tid, w, mu_s0, aug_s0);
      wait_chunk(ci + 2 < nchunks);
      compute(ci + 1, mu_s1, aug_s1);
      if (ci + 3 < nchunks) {
        __builtin_amdgcn_s_barrier();   // every wave is done with buffer 1
        assign_stage<D, CH, THREADS>(rM, rA, (ci + 3) * CH, C, tid, w, mu_s1, aug_s1);
      }
    }
  }
  assign_store(bestp, bbase, secp, knorm, mu2max, hl, key0, N, assign + (size_t)h * N,
               fix_count + h, fix_list + (size_t)h * N, nullptr);
}

// Resident form, C <= kAsgResidentRows<D> (512 at d = 128, 1024 at d = 64): the whole table
// of one head stays in LDS (128 KB of operands plus the augmented rows) and the keys stream
// past it. One workgroup of WAVES waves per CU, a persistent grid: workgroup g takes units
// [g U / G, (g+1) U / G) of the U = H * nb key blocks in (head, block) order, reloading the
// table where its range enters the next head; between reloads every wave walks its own
// blocks (u = first + w, + WAVES, ...) with no barrier, so one wave's key loads hide behind
// the others' MFMAs. A wave assigns a block's keys 64 at a time and counts them per cluster
// in its own LDS histogram (16-bit counters, LDS atomics), then stores the block's byte
// histogram row for the refresh (the near-tie pass corrects it where it moves a key).
template <int D>
constexpr int kAsgResidentRows = 65536 / D;   // 128 KB of bf16 operands
template <int D, int WAVES, int BLK>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
assign_resident_bf16_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ mup,
                            const uint16_t* __restrict__ aug, int32_t* __restrict__ assign,
                            uint8_t* __restrict__ hist, int32_t* __restrict__ fix_count,
                            int2* __restrict__ fix_list, int H, int N, int C, int nb) {
  constexpr int DS = D / 16;
  constexpr int CH = 128;
  constexpr int ROWS = kAsgResidentRows<D>;
  constexpr int THREADS = WAVES * 64;
  constexpr int KTW = kAsgKtw;
  static_assert(ROWS % CH == 0, "whole chunks");
  __shared__ __attribute__((aligned(256))) char mu_s[ROWS * D * 2];
  __shared__ __attribute__((aligned(16))) char aug_s[ROWS * 16];
  __shared__ uint32_t hist_s[WAVES * ROWS / 2];   // per wave: C 16-bit counters

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int nchunks = (C + CH - 1) / CH;
  const long long U = (long long)H * nb;
  const int G = gridDim.x;
  int u = (int)(U * blockIdx.x / G);
  const int u_end = (int)(U * (blockIdx.x + 1) / G);
  uint32_t* hs = hist_s + w * (ROWS / 2);
  while (u < u_end) {
    const int h = u / nb;
    const int seg_end = min(u_end, (h + 1) * nb);
    const __amdgpu_buffer_rsrc_t rM = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(mup + (size_t)h * C * D), (short)0, C * D * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(aug + (size_t)h * C * 8), (short)0, C * 16, kBufferWord3);
    __builtin_amdgcn_s_barrier();   // every wave is done with the previous head's table
    for (int ci = 0; ci < nchunks; ++ci)
      assign_stage<D, CH, THREADS>(rM, rA, ci * CH, C, tid, w, mu_s + ci * CH * D * 2,
                                   aug_s + ci * CH * 16);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    const float mu2max = aug_norm_max(aug_s, C, lane);   // for the near-tie bound
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(K + (size_t)h * N * D), (short)0, N * D * 2, kBufferWord3);
    for (int v = u + w; v < seg_end; v += WAVES) {
      const int kb = v - h * nb;
      for (int i = lane; i < (C + 1) / 2; i += 64) hs[i] = 0u;
#pragma unroll 1
      for (int sub = 0; sub < BLK; sub += 64) {
        const int key0 = kb * BLK + sub + l32;
        bf16x8 kreg[KTW][DS];
        bf16x8 kaug[KTW];
        float knorm[KTW];
        assign_load_keys<D>(rK, key0, hl, kreg, kaug, knorm);
        int bestp[KTW], bbase[KTW], secp[KTW];
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) {
          bestp[kt] = secp[kt] = 0x7fffffff;
          bbase[kt] = 0;
        }
        assign_table<D>(mu_s, aug_s, C, l32, hl, kreg, kaug, bestp, bbase, secp);
        assign_store(bestp, bbase, secp, knorm, mu2max, hl, key0, N, assign + (size_t)h * N,
                     fix_count + h, fix_list + (size_t)h * N, hs);
      }
      uint8_t* row = hist + ((size_t)h * nb + kb) * C;
      for (int c = lane; c < C; c += 64) row[c] = (uint8_t)(hs[c >> 1] >> (16 * (c & 1)));
    }
    u = seg_end;
  }
}

// Exact squared distance of a full key row (in registers) to centroid c of an LDS table of -2 mu rows
// (swizzled as assign_stage stores them): sum over dims of (k + m/2)^2 = (k - mu)^2 in fp32.
// Each difference of two bf16 values is exact, and a sum of D non-negative terms keeps its
// relative error below D * 2^-24 (under 1e-5 of the distance, far inside the 1e-4 band).
template <int D>
__device__ __forceinline__ float exact_sqdist(const uint4 (&kf)[D / 8], const char* ms, int c) {
  float acc = 0.f;
#pragma unroll
  for (int ch = 0; ch < D / 8; ++ch) {
    const uint4 mv = *reinterpret_cast<const uint4*>(ms + swz_byte<D>(c, ch));
    const uint32_t kw[4] = {kf[ch].x, kf[ch].y, kf[ch].z, kf[ch].w};
    const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float d0 = __uint_as_float(kw[q] << 16) + 0.5f * __uint_as_float(mw[q] << 16);
      const float d1 = __uint_as_float(kw[q] & 0xffff0000u) + 0.5f * __uint_as_float(mw[q] & 0xffff0000u);
      acc = fmaf(d0, d0, acc);
      acc = fmaf(d1, d1, acc);
    }
  }
  return acc;
}

// Near-tie re-measurement with the head's table resident in LDS (C <= kAsgResidentRows<D>).
// The listed keys of each head, 64 to a wave, go through the same matrix-core distances as
// the assignment; every centroid whose distance is within the key's candidate limit
// (near_tie_limit of its listed smallest) is re-measured exactly, the smallest exact distance
// wins, ties to the lowest index. Persistent grid over the units of 64 listed keys of all
// heads, table reloaded where a workgroup's range enters the next head.
template <int D, int WAVES>
__global__ void __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
near_tie_resident_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ mup,
                         const uint16_t* __restrict__ aug, const int32_t* __restrict__ fix_count,
                         const int2* __restrict__ fix_list, int32_t* __restrict__ assign,
                         uint8_t* __restrict__ hist, int H, int N, int C, int nb, int block) {
  constexpr int DS = D / 16;
  constexpr int CH = 128;
  constexpr int ROWS = kAsgResidentRows<D>;
  constexpr int THREADS = WAVES * 64;
  constexpr int KTW = kAsgKtw;
  __shared__ __attribute__((aligned(256))) char mu_s[ROWS * D * 2];
  __shared__ __attribute__((aligned(16))) char aug_s[ROWS * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int nchunks = (C + CH - 1) / CH;
  long long U = 0;   // units of 64 listed keys, over all heads
  for (int h = 0; h < H; ++h) U += (__builtin_amdgcn_readfirstlane(fix_count[h]) + 63) / 64;
  const int G = gridDim.x;
  long long u = U * blockIdx.x / G;
  const long long u_end = U * (blockIdx.x + 1) / G;
  int h = 0;
  long long hbase = 0;   // first unit of head h
  while (u < u_end) {
    int nh = __builtin_amdgcn_readfirstlane(fix_count[h]);
    while (u >= hbase + (nh + 63) / 64) {   // the head holding unit u
      hbase += (nh + 63) / 64;
      ++h;
      nh = __builtin_amdgcn_readfirstlane(fix_count[h]);
    }
    const long long seg_end = min(u_end, hbase + (nh + 63) / 64);
    const __amdgpu_buffer_rsrc_t rM = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(mup + (size_t)h * C * D), (short)0, C * D * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(aug + (size_t)h * C * 8), (short)0, C * 16, kBufferWord3);
    __builtin_amdgcn_s_barrier();   // every wave is done with the previous head's table
    for (int ci = 0; ci < nchunks; ++ci)
      assign_stage<D, CH, THREADS>(rM, rA, ci * CH, C, tid, w, mu_s + ci * CH * D * 2,
                                   aug_s + ci * CH * 16);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    const float mu2max = aug_norm_max(aug_s, C, lane);
    const uint16_t* Kh = K + (size_t)h * N * D;
    const int2* lh = fix_list + (size_t)h * N;
    for (long long v = u + w; v < seg_end; v += WAVES) {
      const int e0 = (int)(v - hbase) * 64;
      int key[KTW], b1[KTW];
      bf16x8 kreg[KTW][DS];
      bf16x8 kaug[KTW];
      float knorm[KTW], lim[KTW], bd[KTW];
      int bc[KTW];
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        const int e = e0 + 32 * kt + l32;
        const int2 ent = e < nh ? lh[e] : make_int2(-1, 0);
        key[kt] = ent.x;
        b1[kt] = ent.y;
#pragma unroll
        for (int s_ = 0; s_ < DS; ++s_)
          kreg[kt][s_] = key[kt] >= 0
              ? *reinterpret_cast<const bf16x8*>(Kh + (size_t)key[kt] * D + 16 * s_ + 8 * hl)
              : bf16x8{};
        const float ps = half_row_sq_norm<D>(kreg[kt]);
        const float nk = ps + xor32(ps);
        knorm[kt] = nk;
        const __bf16 n0 = (__bf16)nk;
        const float r1 = nk - (float)n0;
        const __bf16 n1 = (__bf16)r1;
        const __bf16 n2 = (__bf16)(r1 - (float)n1);
        const __bf16 one = (__bf16)1.f, zero = (__bf16)0.f;
        kaug[kt] = hl == 0 ? bf16x8{one, one, one, n0, n1, n2, zero, zero} : bf16x8{};
        lim[kt] = near_tie_limit(b1[kt], nk, mu2max);
        bd[kt] = kPosInf;
        bc[kt] = 0x7fffffff;
      }
      // phase 1: the matrix-core distances, collecting each lane's candidates (up to four;
      // more mark the key for an exact pass over every centroid)
      int cs[KTW][4], ncand[KTW];
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        ncand[kt] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) cs[kt][j] = 0;
      }
      for (int ct = 0; ct < (C + 31) / 32; ++ct) {
        f32x16 acc[KTW];
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) acc[kt] = f32x16{};
#pragma unroll
        for (int s_ = 0; s_ < DS; ++s_) {
          const bf16x8 a = lds_read_b128(mu_s, swz_byte<D>(32 * ct + l32, 2 * s_ + hl));
#pragma unroll
          for (int kt = 0; kt < KTW; ++kt) acc[kt] = mfma32x32x16(a, kreg[kt][s_], acc[kt]);
        }
        const bf16x8 a = lds_read_b128(aug_s, (32 * ct + l32) * 16);
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) acc[kt] = mfma32x32x16(a, kaug[kt], acc[kt]);
#pragma unroll
        for (int kt = 0; kt < KTW; ++kt) {
          uint32_t cand = 0;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * ct + 8 * (r >> 2) + 4 * hl + (r & 3);
            cand |= (key[kt] >= 0 && c < C && acc[kt][r] <= lim[kt]) ? (1u << r) : 0u;
          }
          while (cand != 0) {   // rare: only centroids near the nearest of a listed key
            const int r = __builtin_ctz(cand);
            cand &= cand - 1;
            const int c = 32 * ct + 8 * (r >> 2) + 4 * hl + (r & 3);
            const int n = ncand[kt];
            cs[kt][0] = n == 0 ? c : cs[kt][0];
            cs[kt][1] = n == 1 ? c : cs[kt][1];
            cs[kt][2] = n == 2 ? c : cs[kt][2];
            cs[kt][3] = n == 3 ? c : cs[kt][3];
            ncand[kt] = min(n + 1, 5);
          }
        }
      }
      // phase 2: exact distances from the full key row (in registers) and the LDS table
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        if (key[kt] < 0 || ncand[kt] == 0) continue;
        uint4 kf[D / 8];
        const uint4* kr = reinterpret_cast<const uint4*>(Kh + (size_t)key[kt] * D);
#pragma unroll
        for (int ch = 0; ch < D / 8; ++ch) kf[ch] = kr[ch];
        const int n = ncand[kt];
        const int ncheck = n <= 4 ? n : C;   // more than four: every centroid of this half
        for (int j = 0; j < ncheck; ++j) {
          int c;
          if (n <= 4) c = j == 0 ? cs[kt][0] : j == 1 ? cs[kt][1] : j == 2 ? cs[kt][2] : cs[kt][3];
          else c = j;
          if (n > 4 && (((c >> 2) & 1) != hl)) continue;   // the other half's centroids
          const float dx = exact_sqdist<D>(kf, mu_s, c);
          if (dx < bd[kt] || (dx == bd[kt] && c < bc[kt])) {
            bd[kt] = dx;
            bc[kt] = c;
          }
        }
      }
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        const float od = __shfl_xor(bd[kt], 32, 64);
        const int oc = __shfl_xor(bc[kt], 32, 64);
        const int best = (od < bd[kt] || (od == bd[kt] && oc < bc[kt])) ? oc : bc[kt];
        // The key's own nearest computed distance is always within its limit, so a candidate
        // exists; only non-finite inputs (NaN distances compare false) can leave none, and then
        // the provisional assignment stands.
        if (hl == 0 && key[kt] >= 0 && best >= 0 && best < C) {
          int32_t* ap = assign + (size_t)h * N + key[kt];
          const int old = *ap;
          if (old != best) {
            // move the key between the byte counters of its block's histogram row: the old
            // counter holds it (no borrow), the new one stays below 256 (no carry)
            const size_t rb = ((size_t)h * nb + key[kt] / block) * C;
            const size_t ob = rb + old, nbt = rb + best;
            atomicAdd(reinterpret_cast<uint32_t*>(hist + (ob & ~(size_t)3)),
                      0u - (1u << (8 * (ob & 3))));
            atomicAdd(reinterpret_cast<uint32_t*>(hist + (nbt & ~(size_t)3)),
                      1u << (8 * (nbt & 3)));
            *ap = best;
          }
        }
      }
    }
    u = seg_end;
  }
}

// Near-tie re-measurement when the table does not fit in LDS (C > kAsgResidentRows<D>): every
// listed key against every centroid of its head, exactly (exact_sqdist's arithmetic with the
// centroid rows read from global memory); ties to the lowest index. One wave per listed key,
// lane l taking centroids l, l + 64, ...; a fixed grid walks the lists of all heads.
template <int D>
__global__ void __launch_bounds__(256)
near_tie_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ mu,
                const int32_t* __restrict__ fix_count, const int2* __restrict__ fix_list,
                int32_t* __restrict__ assign, int H, int N, int C) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  int total = 0;
  for (int h = 0; h < H; ++h) total += fix_count[h];
  for (int i = blockIdx.x * 4 + (threadIdx.x >> 6); i < total; i += nw) {
    int h = 0, e = i;
    while (e >= fix_count[h]) e -= fix_count[h++];
    const int key = fix_list[(size_t)h * N + e].x;
    const uint4* kr = reinterpret_cast<const uint4*>(K + ((size_t)h * N + key) * D);
    uint4 kw[D / 8];
#pragma unroll
    for (int ch = 0; ch < D / 8; ++ch) kw[ch] = kr[ch];
    float best = kPosInf;
    int bc = 0;
    for (int c = lane; c < C; c += 64) {
      const uint4* mr = reinterpret_cast<const uint4*>(mu + ((size_t)h * C + c) * D);
      float acc = 0.f;
#pragma unroll
      for (int ch = 0; ch < D / 8; ++ch) {
        const uint4 mv = mr[ch];
        const uint32_t kv[4] = {kw[ch].x, kw[ch].y, kw[ch].z, kw[ch].w};
        const uint32_t mw[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float d0 = __uint_as_float(kv[q] << 16) - __uint_as_float(mw[q] << 16);
          const float d1 = __uint_as_float(kv[q] & 0xffff0000u) - __uint_as_float(mw[q] & 0xffff0000u);
          acc = fmaf(d0, d0, acc);
          acc = fmaf(d1, d1, acc);
        }
      }
      if (acc < best) {   // centroids ascend within a lane: the first of equals is kept
        best = acc;
        bc = c;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ob = __shfl_xor(best, o, 64);
      const int oc = __shfl_xor(bc, o, 64);
      if (ob < best || (ob == best && oc < bc)) {
        best = ob;
        bc = oc;
      }
    }
    if (lane == 0) assign[(size_t)h * N + key] = bc;
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
// 16 waves split the key blocks; lane = cluster. Two passes over the histograms, each with 8
// rows' bytes in flight (the rows are independent loads; one at a time would leave every
// wave waiting on the memory latency once per block).
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
  constexpr int U = 8;
  int s = 0;
  if (c < C) {
    int kb = kb0;
    for (; kb + U <= kb1; kb += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = col[(size_t)(kb + u) * C];
#pragma unroll
      for (int u = 0; u < U; ++u) s += v[u];
    }
    for (; kb < kb1; ++kb) s += col[(size_t)kb * C];
  }
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
    int kb = kb0;
    for (; kb + U <= kb1; kb += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = col[(size_t)(kb + u) * C];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ocol[(size_t)(kb + u) * C] = run;
        run += v[u];
      }
    }
    for (; kb < kb1; ++kb) {
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
// One workgroup of `block` threads (64 or 128) per query block; a key's slot is its cluster's
// start, plus the block's offset in that cluster, plus its rank among the block's earlier keys
// of the cluster, so the sorted order is ascending key order within each cluster.
__global__ void __launch_bounds__(128)
scatter_kernel(const int32_t* __restrict__ assign, const int32_t* __restrict__ off,
               const int32_t* __restrict__ start, int32_t* __restrict__ perm, int N, int C,
               int nb, int block) {
  __shared__ int4 a_lds[32];   // the block's assignments (at most 128), four to an entry
  const int h = blockIdx.y, kb = blockIdx.x, tid = threadIdx.x;
  const int j = kb * block + tid;
  const int c = (tid < block && j < N) ? assign[(size_t)h * N + j] : -1;
  reinterpret_cast<int32_t*>(a_lds)[tid] = c;
  __syncthreads();
  if (c >= 0) {
    // rank among the block's earlier keys of the same cluster: whole entries, then the rest
    int r = 0;
    for (int t4 = 0; t4 < (tid >> 2); ++t4) {
      const int4 v = a_lds[t4];
      r += (v.x == c) + (v.y == c) + (v.z == c) + (v.w == c);
    }
    for (int t = tid & ~3; t < tid; ++t) r += reinterpret_cast<const int32_t*>(a_lds)[t] == c;
    const int pos = start[(size_t)h * C + c] + off[((size_t)h * nb + kb) * C + c] + r;
    perm[(size_t)h * N + pos] = j;
  }
}

// ----------------------------------------------------------------------------- 6. sums
// Two phases with balanced work whatever the cluster sizes. Phase 1: wave s sums the keys
// and values at sorted positions [s*SEG, (s+1)*SEG) (clusters are contiguous there, in
// ascending key order), writing one fp32 partial per cluster run it meets into slot s + c:
// unique, because a cluster that reaches segment s+1 ends before cluster c+1 starts. Phase 2:
// one wave per cluster adds its partials in segment order, divides and rounds. Every sum
// runs in a fixed order, so results are bit-reproducible. Each lane owns D/64 dims.
constexpr int kSeg = 256;
#ifndef SEG_U
#define SEG_U 16
#endif

// Wave-wide sum (all 64 lanes receive it).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// With VAR, each partial also carries the sum of the squared norms of its keys (one float per
// slot in psq), from which the finish derives the clusters' key variance.
template <int D, bool BF16, bool VAR>
__global__ void __launch_bounds__(256)
segment_sum_kernel(const void* __restrict__ Kv, const void* __restrict__ Vv,
                   const int32_t* __restrict__ sizes, const int32_t* __restrict__ start,
                   const int32_t* __restrict__ perm, float* __restrict__ part,
                   float* __restrict__ psq, int N, int C, int nseg) {
  constexpr int EPL = D / 64;
  constexpr int U = SEG_U;
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int sgi = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sgi >= nseg) return;
  const int p0 = sgi * kSeg, p1 = min(N, p0 + kSeg);
  const int32_t* st = start + (size_t)h * C;
  const int32_t* sz = sizes + (size_t)h * C;
  const int32_t* pl = perm + (size_t)h * N;
  // cluster holding position p0: the last c with start[c] <= p0 (it is non-empty)
  int lo = 0, hi = C - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  int cend = st[c] + sz[c];
  float ks[EPL], vs[EPL];
  float qs = 0.f;   // this lane's share of the squared key norms (VAR)
#pragma unroll
  for (int e = 0; e < EPL; ++e) ks[e] = vs[e] = 0.f;
  float* ph = part + (size_t)h * (nseg + C) * 2 * D;
  auto flush = [&]() {
    float* o = ph + (size_t)(sgi + c) * 2 * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      o[e] = ks[e];
      o[D + e] = vs[e];
      ks[e] = vs[e] = 0.f;
    }
    if constexpr (VAR) {
      const float t = wave_sum(qs);
      if (lane == 0) psq[(size_t)h * (nseg + C) + sgi + c] = t;
      qs = 0.f;
    }
  };
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
  for (int i = p0; i < p1; i += U) {
    const int n = min(U, p1 - i);
    float kr[U][EPL], vr[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = pl[i + min(u, n - 1)];
      load_row(Kv, j, kr[u]);
      load_row(Vv, j, vr[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < n) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          ks[e] += kr[u][e];
          vs[e] += vr[u][e];
          if constexpr (VAR) qs = fmaf(kr[u][e], kr[u][e], qs);
        }
        if (i + u + 1 == cend) {   // this cluster's run ends here
          flush();
          while (c + 1 < C && st[c + 1] + sz[c + 1] <= i + u + 1) ++c;   // skip empty ones
          ++c;
          cend = c < C ? st[c] + sz[c] : N;
        }
      }
    }
  }
  if (c < C && st[c] < p1 && p1 < cend) flush();   // a run continuing into the next segment
}

// With VAR, also the isotropic key variance of each cluster,
// kvar = max(0, sum ||k||^2 / n - ||mean||^2) / D (fp32, from the unrounded mean; 0 if empty).
template <int D, bool BF16, bool VAR>
__global__ void __launch_bounds__(256)
cluster_finish_kernel(const float* __restrict__ part, const float* __restrict__ psq,
                      const void* __restrict__ mu_in, void* __restrict__ mu_out,
                      void* __restrict__ vbar_out, float* __restrict__ kvar_out,
                      const int32_t* __restrict__ sizes, const int32_t* __restrict__ start,
                      int C, int nseg) {
  constexpr int EPL = D / 64;
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= C) return;
  const int cnt = sizes[(size_t)h * C + c];
  float ks[EPL], vs[EPL];
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ks[e] = vs[e] = 0.f;
  if (cnt > 0) {
    const int p0 = start[(size_t)h * C + c];
    const int s0 = p0 / kSeg, s1 = (p0 + cnt - 1) / kSeg;
    const float* ph = part + (size_t)h * (nseg + C) * 2 * D + lane * EPL;
    for (int sg = s0; sg <= s1; ++sg) {
      const float* q = ph + (size_t)(sg + c) * 2 * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ks[e] += q[e];
        vs[e] += q[D + e];
      }
      if constexpr (VAR) sq += psq[(size_t)h * (nseg + C) + sg + c];
    }
  }
  const size_t o = ((size_t)h * C + c) * D + lane * EPL;
  const float fc = (float)cnt;
  if constexpr (VAR) {
    float m2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float m = cnt > 0 ? ks[e] / fc : 0.f;
      m2 = fmaf(m, m, m2);
    }
    m2 = wave_sum(m2);
    if (lane == 0)
      kvar_out[(size_t)h * C + c] = cnt > 0 ? fmaxf(0.f, sq / fc - m2) / (float)D : 0.f;
  }
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
// n[b][c] = size[c] - sum over b's exact blocks of hist[kb][c], for the two query blocks of
// a pair at once: the pair's union list (entries kb | in 2p << 28 | in 2p+1 << 29) reads each
// shared key block's byte histogram once. Each thread owns 2 clusters of both blocks.
__global__ void __launch_bounds__(256)
counts_kernel(const uint8_t* __restrict__ hist, const int32_t* __restrict__ sizes,
              const int32_t* __restrict__ prowptr, const int32_t* __restrict__ pcol,
              int32_t* __restrict__ counts, int C, int nb, int npairs, int mask_heads) {
  const int h = blockIdx.y, pr = blockIdx.x;
  const int b0 = 2 * pr;
  const bool has1 = b0 + 1 < nb;
  const int mh = mask_heads == 1 ? 0 : h;
  const int e0 = prowptr[mh * (npairs + 1) + pr], e1 = prowptr[mh * (npairs + 1) + pr + 1];
  const uint8_t* hh = hist + (size_t)h * nb * C;
  int32_t* dst0 = counts + ((size_t)h * nb + b0) * C;
  int32_t* dst1 = dst0 + C;
  const int32_t* sz = sizes + (size_t)h * C;
  if ((C & 1) == 0) {
    for (int c = 2 * threadIdx.x; c < C; c += 2 * 256) {
      int a0 = sz[c], a1 = sz[c + 1];
      int c0 = a0, c1 = a1;
      // 8 list entries (wave-uniform) and their histogram rows in flight at a time
      constexpr int U = 8;
      int e = e0;
      for (; e + U <= e1; e += U) {
        int ent[U];
        uint32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ent[u] = pcol[e + u];
#pragma unroll
        for (int u = 0; u < U; ++u)
          v[u] = *reinterpret_cast<const uint16_t*>(hh + (size_t)(ent[u] & 0x0fffffff) * C + c);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int lo = v[u] & 0xff, hi = v[u] >> 8;
          const int f0 = (ent[u] >> 28) & 1, f1 = (ent[u] >> 29) & 1;
          a0 -= f0 * lo; a1 -= f0 * hi;
          c0 -= f1 * lo; c1 -= f1 * hi;
        }
      }
      for (; e < e1; ++e) {
        const int ent = pcol[e];
        const uint32_t v = *reinterpret_cast<const uint16_t*>(hh + (size_t)(ent & 0x0fffffff) * C + c);
        const int lo = v & 0xff, hi = v >> 8;
        if (ent & (1 << 28)) { a0 -= lo; a1 -= hi; }
        if (ent & (1 << 29)) { c0 -= lo; c1 -= hi; }
      }
      *reinterpret_cast<int2*>(dst0 + c) = make_int2(a0, a1);
      if (has1) *reinterpret_cast<int2*>(dst1 + c) = make_int2(c0, c1);
    }
  } else {
    for (int c = threadIdx.x; c < C; c += 256) {
      int a0 = sz[c], c0 = sz[c];
      for (int e = e0; e < e1; ++e) {
        const int ent = pcol[e];
        const int v = hh[(size_t)(ent & 0x0fffffff) * C + c];
        if (ent & (1 << 28)) a0 -= v;
        if (ent & (1 << 29)) c0 -= v;
      }
      dst0[c] = a0;
      if (has1) dst1[c] = c0;
    }
  }
}

// The same counts with 8 clusters a lane (C a multiple of 8): one wave per (pair, slab of 512
// clusters) walks the pair's union list, reading 8 histogram bytes of each entry's row with
// one load (a wave reads 512 consecutive bytes) and adding them into the counters of the users
// of that entry (wave-uniform branches on the entry's user bits).
__global__ void __launch_bounds__(256)
counts8_kernel(const uint8_t* __restrict__ hist, const int32_t* __restrict__ sizes,
               const int32_t* __restrict__ prowptr, const int32_t* __restrict__ pcol,
               int32_t* __restrict__ counts, int C, int nb, int npairs, int mask_heads,
               int nslab, int items) {
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= items) return;
  const int lane = threadIdx.x & 63;
  const int slab = item % nslab;
  const int pr = (item / nslab) % npairs;
  const int h = item / (nslab * npairs);
  const int c = slab * 512 + lane * 8;
  const int b0 = 2 * pr;
  const bool has1 = b0 + 1 < nb;
  const int mh = mask_heads == 1 ? 0 : h;
  const int e0 = sload(prowptr, mh * (npairs + 1) + pr);
  const int e1 = sload(prowptr, mh * (npairs + 1) + pr + 1);
  if (c >= C) return;
  const uint8_t* hh = hist + (size_t)h * nb * C + c;
  int both[8], only0[8], only1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) both[j] = only0[j] = only1[j] = 0;
  auto add = [](int (&acc)[8], uint2 v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += (v.x >> (8 * j)) & 0xff;
      acc[4 + j] += (v.y >> (8 * j)) & 0xff;
    }
  };
  constexpr int U = 8;   // entries (and their rows) in flight
  int e = e0;
  for (; e + U <= e1; e += U) {
    int ent[U];
    uint2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ent[u] = sload(pcol, e + u);
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = *reinterpret_cast<const uint2*>(hh + (size_t)(ent[u] & kEntIndex) * C);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int use = (ent[u] >> kEntUse0) & 3;
      if (use == 3) add(both, v[u]);
      else if (use == 1) add(only0, v[u]);
      else if (use == 2) add(only1, v[u]);
    }
  }
  for (; e < e1; ++e) {
    const int ent = sload(pcol, e);
    const uint2 v = *reinterpret_cast<const uint2*>(hh + (size_t)(ent & kEntIndex) * C);
    const int use = (ent >> kEntUse0) & 3;
    if (use == 3) add(both, v);
    else if (use == 1) add(only0, v);
    else if (use == 2) add(only1, v);
  }
  const int4 sa = *reinterpret_cast<const int4*>(sizes + (size_t)h * C + c);
  const int4 sb = *reinterpret_cast<const int4*>(sizes + (size_t)h * C + c + 4);
  const int sz[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
  int32_t* dst0 = counts + ((size_t)h * nb + b0) * C + c;
  int n0[8], n1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    n0[j] = sz[j] - both[j] - only0[j];
    n1[j] = sz[j] - both[j] - only1[j];
  }
  *reinterpret_cast<int4*>(dst0) = make_int4(n0[0], n0[1], n0[2], n0[3]);
  *reinterpret_cast<int4*>(dst0 + 4) = make_int4(n0[4], n0[5], n0[6], n0[7]);
  if (has1) {
    *reinterpret_cast<int4*>(dst0 + C) = make_int4(n1[0], n1[1], n1[2], n1[3]);
    *reinterpret_cast<int4*>(dst0 + C + 4) = make_int4(n1[4], n1[5], n1[6], n1[7]);
  }
}

// Counts when the exact key blocks (S keys) are smaller than the query blocks: per pair,
// n[b][c] starts from size[c] in LDS and every key of the union list's key blocks takes one
// off the rows of the query blocks that keep it, read straight from the assignments (4 bytes
// a key, where histograms of S-key blocks would cost C bytes per block). Integer LDS
// atomics, so the result does not depend on their order. 256/S list entries per pass, U
// passes in flight.
__global__ void __launch_bounds__(256)
counts_keys_kernel(const int32_t* __restrict__ assign, const int32_t* __restrict__ sizes,
                   const int32_t* __restrict__ prowptr, const int32_t* __restrict__ pcol,
                   int32_t* __restrict__ counts, int N, int C, int nb, int npairs,
                   int mask_heads, int S) {
  extern __shared__ int32_t cnt_lds[];   // [2][C]
  const int h = blockIdx.y, pr = blockIdx.x, tid = threadIdx.x;
  const int b0 = 2 * pr;
  const bool has1 = b0 + 1 < nb;
  const int mh = mask_heads == 1 ? 0 : h;
  const int e0 = prowptr[mh * (npairs + 1) + pr], e1 = prowptr[mh * (npairs + 1) + pr + 1];
  const int32_t* sz = sizes + (size_t)h * C;
  for (int c = tid; c < C; c += 256) {
    const int v = sz[c];
    cnt_lds[c] = v;
    cnt_lds[C + c] = v;
  }
  __syncthreads();
  const int32_t* ah = assign + (size_t)h * N;
  const int per = 256 / S;
  const int sub = tid / S, r = tid % S;
  constexpr int U = 4;
  for (int e = e0 + sub; e < e1; e += U * per) {
    int ent[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ent[u] = e + u * per < e1 ? pcol[e + u * per] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = (ent[u] & kEntIndex) * S + r;
      const bool used = (ent[u] >> kEntUse0) & 3;
      c[u] = (used && key < N) ? ah[key] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c[u] < 0) continue;
      if ((ent[u] >> kEntUse0) & 1) atomicSub(&cnt_lds[c[u]], 1);
      if ((ent[u] >> kEntUse1) & 1) atomicSub(&cnt_lds[C + c[u]], 1);
    }
  }
  __syncthreads();
  int32_t* dst = counts + ((size_t)h * nb + b0) * C;
  for (int c = tid; c < C; c += 256) {
    dst[c] = cnt_lds[c];
    if (has1) dst[C + c] = cnt_lds[C + c];
  }
}

// ----------------------------------------------------------------------------- scratch
// Workspace of da_reassign_noalloc, for callers that cannot allocate: a file-scope device
// array that every GPU running the library holds until the process ends. Host code never
// passes its name to a kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, and that pointer is what the
// kernels receive. Every call on one device shares the array; calls that overlap on a
// device race.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<std::pair<int, void*>> g_scratch_ptr;   // (device, device address)
}  // namespace

hipError_t scratch_setup(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (const auto& e : g_scratch_ptr)
    if (e.first == device) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (err != hipSuccess) return err;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr.emplace_back(device, ptr);
  return hipSuccess;
}

hipError_t scratch_address(int device, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (const auto& e : g_scratch_ptr)
    if (e.first == device) {
      *out = e.second;
      return hipSuccess;
    }
  *out = nullptr;
  return hipErrorNotReady;
}

// ----------------------------------------------------------------------------- launch
template <int D, bool BF16, bool VAR>
static void launch_sums(const ReassignArgs& a, int nseg, hipStream_t s) {
  hipLaunchKernelGGL((segment_sum_kernel<D, BF16, VAR>), dim3((nseg + 3) / 4, a.H), dim3(256), 0,
                     s, a.K, a.V, a.sizes, a.start, a.perm, a.part, a.psq, a.N, a.C, nseg);
  hipLaunchKernelGGL((cluster_finish_kernel<D, BF16, VAR>), dim3((a.C + 3) / 4, a.H), dim3(256),
                     0, s, a.part, a.psq, a.mu_in, a.mu_out, a.vbar_out, a.kvar, a.sizes, a.start,
                     a.C, nseg);
}

template <int D>
static hipError_t launch_reassign_t(const ReassignArgs& a, bool bf16, hipStream_t s) {
  bool hist_done = false;   // the resident assignment writes the block histograms itself
  if (bf16)
  {
    uint16_t* mup = a.cop;
    uint16_t* aug = a.cop + (size_t)a.H * a.C * D;
    int32_t* fix_count = a.fix;
    int2* fix_list = reinterpret_cast<int2*>(a.fix + fix_list_offset(a.H));
    hipLaunchKernelGGL((centroid_operands_kernel<D>), dim3((a.C + 255) / 256, a.H), dim3(256), 0,
                       s, static_cast<const uint16_t*>(a.mu_in), mup, aug, fix_count, a.C);
    if (a.C <= kAsgResidentRows<D>) {
      if (a.block == 128)
        hipLaunchKernelGGL((assign_resident_bf16_kernel<D, 8, 128>), dim3(a.ncu), dim3(8 * 64), 0,
                           s, static_cast<const uint16_t*>(a.K), mup, aug, a.assign, a.hist,
                           fix_count, fix_list, a.H, a.N, a.C, a.nb);
      else
        hipLaunchKernelGGL((assign_resident_bf16_kernel<D, 8, 64>), dim3(a.ncu), dim3(8 * 64), 0,
                           s, static_cast<const uint16_t*>(a.K), mup, aug, a.assign, a.hist,
                           fix_count, fix_list, a.H, a.N, a.C, a.nb);
      hipLaunchKernelGGL((near_tie_resident_kernel<D, 8>), dim3(a.ncu), dim3(8 * 64), 0, s,
                         static_cast<const uint16_t*>(a.K), mup, aug, fix_count, fix_list,
                         a.assign, a.hist, a.H, a.N, a.C, a.nb, a.block);
      hist_done = true;
    } else {
      constexpr int AW = ASG_WAVES;
      hipLaunchKernelGGL((assign_bf16_kernel<D, AW, ASG_CH>),
                         dim3((a.N + AW * 64 - 1) / (AW * 64), a.H), dim3(AW * 64), 0, s,
                         static_cast<const uint16_t*>(a.K), mup, aug, a.assign, fix_count,
                         fix_list, a.N, a.C);
      hipLaunchKernelGGL((near_tie_kernel<D>), dim3(2 * a.ncu), dim3(256), 0, s,
                         static_cast<const uint16_t*>(a.K), static_cast<const uint16_t*>(a.mu_in),
                         fix_count, fix_list, a.assign, a.H, a.N, a.C);
    }
  }
  else
    hipLaunchKernelGGL((assign_f32_kernel<D>), dim3((a.N + 255) / 256, a.H), dim3(256), 0, s,
                       static_cast<const float*>(a.K), static_cast<const float*>(a.mu_in),
                       a.assign, a.N, a.C);
  if (!hist_done)
    hipLaunchKernelGGL(block_hist_kernel, dim3(a.nb, a.H), dim3(256), a.C * sizeof(int32_t), s,
                       a.assign, a.hist, a.N, a.C, a.nb, a.block);
  hipLaunchKernelGGL(col_scan_kernel, dim3((a.C + 63) / 64, a.H), dim3(1024), 0, s, a.hist,
                     a.off, a.sizes, a.C, a.nb);
  hipLaunchKernelGGL(starts_kernel, dim3(a.H), dim3(1024), 0, s, a.sizes, a.start, a.C);
  hipLaunchKernelGGL(scatter_kernel, dim3(a.nb, a.H), dim3(a.block), 0, s, a.assign, a.off,
                     a.start, a.perm, a.N, a.C, a.nb, a.block);
  {
    const int nseg = (a.N + kSeg - 1) / kSeg;
    if (bf16) {
      if (a.kvar) launch_sums<D, true, true>(a, nseg, s);
      else launch_sums<D, true, false>(a, nseg, s);
    } else {
      if (a.kvar) launch_sums<D, false, true>(a, nseg, s);
      else launch_sums<D, false, false>(a, nseg, s);
    }
  }
  if (a.kblock == a.block && a.C % 8 == 0) {
    const int nslab = (a.C + 511) / 512;
    const int items = a.H * a.npairs * nslab;
    hipLaunchKernelGGL(counts8_kernel, dim3((items + 3) / 4), dim3(256), 0, s, a.hist, a.sizes,
                       a.prowptr, a.pcol, a.counts, a.C, a.nb, a.npairs, a.mask_heads, nslab,
                       items);
  } else if (a.kblock == a.block)
    hipLaunchKernelGGL(counts_kernel, dim3(a.npairs, a.H), dim3(256), 0, s, a.hist, a.sizes,
                       a.prowptr, a.pcol, a.counts, a.C, a.nb, a.npairs, a.mask_heads);
  else
    hipLaunchKernelGGL(counts_keys_kernel, dim3(a.npairs, a.H), dim3(256),
                       2 * a.C * sizeof(int32_t), s, a.assign, a.sizes, a.prowptr, a.pcol,
                       a.counts, a.N, a.C, a.nb, a.npairs, a.mask_heads, a.kblock);
  return hipGetLastError();
}

hipError_t launch_reassign(const ReassignArgs& a, int head_dim, bool bf16, hipStream_t s) {
  if (head_dim == 64) return launch_reassign_t<64>(a, bf16, s);
  if (head_dim == 128) return launch_reassign_t<128>(a, bf16, s);
  return hipErrorInvalidValue;
}

hipError_t prepare_reassign_kernels() {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&block_hist_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(8192 * sizeof(int32_t)));
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&counts_keys_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(2 * 8192 * sizeof(int32_t)));
}

}  // namespace da

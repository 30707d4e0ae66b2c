// Fused decoupled sparse attention forward for gfx950.
//
// One workgroup owns one (head, query block). It walks the query block's exact key blocks
// (the plan's sorted list) and then the cluster-cache tiles (C centroid keys / mean values
// taken BLK at a time), treating both the same way: the tile's keys and values are staged
// in LDS, scores come from MFMA, and a single online softmax (exp2 domain) absorbs every
// tile. Cluster tiles add a per-key logit bias log2(n[b][c]) (-inf where n = 0), which in
// the natural-log domain is the ln-count weight of the DecoupAttn abstract: each cluster
// stands in for the n of its keys left outside the exact blocks.
//
// Work split (bf16): wave w handles 32 query rows. Scores are formed transposed,
// S^T = K * Q^T, so every lane owns one query column and the row max / row sum need only
// one cross-half exchange. O^T = V^T * P^T then leaves each lane with the output of the
// same query, so the online-softmax rescale is a per-lane scalar. V^T operands come
// straight from the row-major V tile through the gfx950 transposed LDS read.
#include "da_device.h"
#include "da_internal.h"

namespace da {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// XCD-aware order: hardware deals workgroup ids round-robin to the 8 XCDs; give each XCD a
// contiguous range of (head, query block) so neighbouring query blocks, which share many
// 3D-local key blocks, hit the same L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  int per = (total + 7) >> 3;
  return (L & 7) * per + (L >> 3);
}

// ----------------------------------------------------------------------------- bf16
// A workgroup owns two adjacent query blocks (2p, 2p+1) of one head: BLK/32 waves per
// block. It walks the ascending union of the two exact lists, so a key block both blocks
// keep exact is fetched once (neighbouring query blocks of a 3D-local mask share most of
// their key blocks), then the cluster tiles, which both blocks use with their own bias
// rows. A wave skips the tiles its block does not keep.
struct TileDesc {
  const char* k;   // tile base (bytes)
  const char* v;
  int valid;       // rows that exist (keys < N, or clusters < C)
  int kind;        // 0 full exact block, 1 ragged exact block, 2 cluster tile
  int c0;          // first cluster of a cluster tile
  int use;         // bit h: query block 2p+h uses this tile
};

// Read-only, wave-uniform loads through the scalar cache.
__device__ __forceinline__ int32_t sload(const int32_t* base, int idx) {
  return ((const __attribute__((address_space(4))) int32_t*)(base))[idx];
}

template <int D, int BLK>
__device__ __forceinline__ TileDesc tile_desc(int t, int n_list, int entry, int N, int C,
                                              const char* Kh, const char* Mh,
                                              const char* VTh) {
  TileDesc d;
  if (t < n_list) {
    const int kb = entry & 0x0fffffff;
    d.k = Kh + (size_t)kb * BLK * D * 2;
    d.v = VTh + (size_t)kb * BLK * D * 2;
    d.valid = min(BLK, N - kb * BLK);
    d.kind = d.valid < BLK ? 1 : 0;
    d.c0 = 0;
    d.use = (entry >> 28) & 3;
  } else {
    const int ct = t - n_list;
    d.c0 = ct * BLK;
    d.k = Mh + (size_t)d.c0 * D * 2;
    d.v = VTh + (size_t)((N + BLK - 1) / BLK + ct) * BLK * D * 2;
    d.valid = min(BLK, C - d.c0);
    d.kind = 2;
    d.use = 3;
  }
  return d;
}

// Value tiles in the layout the PV product reads: tile j of a head (key block j < nb, then
// cluster tile j - nb) is [D rows][BLK columns] with column position p of each 16-column
// group holding key 8*((p>>2)&1) + 4*(p>>3) + (p&3) of that group (zero past N or C). With
// that order the eight k-values a lane feeds to one 32x32x16 MFMA k-step are adjacent, so
// the V^T operand is one 16-byte LDS read, like the K operand.
template <int D, int BLK>
__global__ void __launch_bounds__(256)
vt_pack_kernel(const uint16_t* __restrict__ V, const uint16_t* __restrict__ vbar,
               uint16_t* __restrict__ vt, int N, int C, int nb, int nct) {
  constexpr int PAD = 8;
  __shared__ __attribute__((aligned(16))) uint16_t tile[BLK][D + PAD];
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const uint16_t* src;
  int valid;
  if (j < nb) {
    src = V + ((size_t)h * N + (size_t)j * BLK) * D;
    valid = min(BLK, N - j * BLK);
  } else {
    const int c0 = (j - nb) * BLK;
    src = vbar + ((size_t)h * C + c0) * D;
    valid = min(BLK, C - c0);
  }
  for (int idx = tid; idx < BLK * D / 8; idx += 256) {
    const int row = idx / (D / 8), ch = idx - row * (D / 8);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < valid) v = *reinterpret_cast<const uint4*>(src + (size_t)row * D + ch * 8);
    *reinterpret_cast<uint4*>(&tile[row][ch * 8]) = v;
  }
  __syncthreads();
  uint16_t* dst = vt + ((size_t)h * (nb + nct) + j) * D * BLK;
  for (int idx = tid; idx < D * BLK / 8; idx += 256) {
    const int d = idx / (BLK / 8), c = idx - d * (BLK / 8);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t pair = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pos = c * 8 + e + k;
        const int q = pos & 15;
        const int key = (pos & ~15) + 8 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
        pair |= (uint32_t)tile[key][d] << (16 * k);
      }
      w[e >> 1] = pair;
    }
    *reinterpret_cast<uint4*>(dst + (size_t)d * BLK + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Schedule (8 waves for BLK = 128, one wave of each query block per SIMD): every tile is two
// phases separated by a barrier, and the two query blocks run them in opposite order,
//   phase 1: block 2p   scores + softmax of tile t    | block 2p+1  PV of tile t-1
//   phase 2: block 2p   PV of tile t                  | block 2p+1  scores + softmax of tile t
// so on each SIMD one wave's softmax (VALU, transcendental) and LDS latency overlap the other
// wave's MFMA stream. K(t+1) is prefetched into the free K stage at the start of tile t and
// V(t+1) into the free V stage once block 2p+1 has consumed V(t-1) in phase 1.
template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdArgs p) {
  constexpr int THREADS = BLK * 4;
  constexpr int WPB = BLK / 32;    // waves per query block
  constexpr int KT = BLK / 32;     // 32-key tiles per key block
  constexpr int DT = D / 32;       // 32-dim tiles of the output
  constexpr int DS = D / 16;       // k-steps of the score product
  constexpr int NCH = D / 8;       // 16-byte chunks per K row
  constexpr int TILE = BLK * D * 2;
  constexpr int PER_T = (BLK * NCH) / THREADS;   // 16-byte fetches per thread per tensor
  static_assert(PER_T * THREADS == BLK * NCH, "tile must split evenly");
  constexpr float kRescale = 8.f;  // log2 headroom before the running max is moved
  constexpr int KC = 2;            // 32-key subtiles per softmax chunk

  extern __shared__ __attribute__((aligned(16))) char smem[];
  // K stages at s*TILE, V stages at (2+s)*TILE, then bias rows [stage][half][BLK]
  float* bias_base = reinterpret_cast<float*>(smem + 4 * TILE);

  const int total = p.H * p.npairs;
  const int logical = xcd_remap(blockIdx.x, total);
  if (logical >= total) return;
  const int h = logical / p.npairs;
  const int pr = logical - h * p.npairs;
  const int b0 = 2 * pr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = w / WPB;
  const int wq = w - half * WPB;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int bw = b0 + half;
  const bool block_ok = bw < p.nb;

  const char* Qh = static_cast<const char*>(p.Q) + (size_t)h * p.N * D * 2;
  const char* Kh = static_cast<const char*>(p.K) + (size_t)h * p.N * D * 2;
  const char* Mh = static_cast<const char*>(p.mu) + (size_t)h * p.C * D * 2;
  const char* VTh = static_cast<const char*>(p.vt) + (size_t)h * (p.nb + p.nct) * BLK * D * 2;

  const int mh = p.mask_heads == 1 ? 0 : h;
  const int e0 = sload(p.prowptr, mh * (p.npairs + 1) + pr);
  const int n_list = sload(p.prowptr, mh * (p.npairs + 1) + pr + 1) - e0;
  const int ntiles = n_list + (p.C + BLK - 1) / BLK;

  // Direct-to-LDS fetch of one tile of ROWS x COLS bf16 (K: BLK x D, V^T: D x BLK): the
  // lane filling physical LDS slot (row, pc) reads logical chunk pc ^ swz_key(row); each
  // wave instruction fills 1 KB of consecutive slots. K rows past `valid` re-read the last
  // valid row: their logits are masked to -inf, so their contents only need to be finite.
  auto fetch_k = [&](const char* src, int valid, char* lds_tile) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int slot = i * THREADS + tid;
      const int row = slot / NCH;
      const int pc = slot - row * NCH;
      const int off = min(row, valid - 1) * (D * 2) + ((pc ^ swz_key<D>(row)) << 4);
      __builtin_amdgcn_global_load_lds(
          (const void*)(src + off),
          (__attribute__((address_space(3))) void*)(lds_tile + (i * THREADS + w * 64) * 16),
          16, 0, 0);
    }
  };
  auto fetch_vt = [&](const char* src, char* lds_tile) {
    constexpr int VCH = BLK / 8;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int slot = i * THREADS + tid;
      const int row = slot / VCH;
      const int pc = slot - row * VCH;
      const int off = row * (BLK * 2) + ((pc ^ swz_key<BLK>(row)) << 4);
      __builtin_amdgcn_global_load_lds(
          (const void*)(src + off),
          (__attribute__((address_space(3))) void*)(lds_tile + (i * THREADS + w * 64) * 16),
          16, 0, 0);
    }
  };
  // Bias rows (log2 domain): thread tid < 2*BLK owns [tid / BLK][tid % BLK]: 0 / -inf past
  // N for a ragged exact block, log2 n[b][c] or -inf for a cluster tile.
  const int bq = b0 + tid / BLK;
  const int brow = tid % BLK;
  const int32_t* cnt_row = p.counts + ((size_t)h * p.nb + min(bq, p.nb - 1)) * p.C;
  auto load_count = [&](const TileDesc& d) -> int {
    const int c = d.c0 + brow;
    return (d.kind == 2 && tid < 2 * BLK && c < p.C && bq < p.nb) ? cnt_row[c] : 0;
  };
  auto bias_of = [&](const TileDesc& d, int n) -> float {
    if (d.kind == 1) return brow < d.valid ? 0.f : kNegInf;
    return n > 0 ? fast_log2((float)n) : kNegInf;
  };

  // Q^T operand for this lane's query, all d k-steps.
  const int q = bw * BLK + wq * 32 + l32;
  bf16x8 qreg[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    if (q < p.N)
      qreg[s] = *reinterpret_cast<const bf16x8*>(Qh + ((size_t)q * D + 16 * s + 8 * hl) * 2);
    else
      qreg[s] = bf16x8{};
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -1e30f;   // reference max (log2 domain); finite so exp2(m_run - x) is safe
  float l_run = 0.f;      // this half-wave's share of the row sum
  const float c2 = p.scale_log2e;
  // P of the tile whose PV is pending (bf16, B operand of O^T += V^T P^T): k-step (mk, t2)
  // covers keys 32mk + 16t2 + {0..15}; this lane's eight k-values are keys
  // 32mk + 16t2 + 8i' + 4hl + j (i' = 0,1; j = 0..3) = its score accumulators 8t2 .. 8t2+7.
  bf16x8 pk[KT][2];

  // scores + online softmax of one tile into pk (log2 domain, lazily moved reference max)
  auto scores_softmax = [&](const char* k_lds, const float* bias_lds, int kind) {
#pragma unroll
    for (int ch = 0; ch < KT / KC; ++ch) {
      // two accumulator chains (subtiles 2ch, 2ch+1); K operands are read two k-steps
      // ahead of their MFMA so LDS latency hides behind the MFMA stream
      static_assert(KC == 2, "two score chains per chunk");
      const int r0 = 32 * (ch * KC) + l32, r1 = r0 + 32;
      f32x16 sacc[KC] = {f32x16{}, f32x16{}};
      bf16x8 ra[3], rb[3];
      ra[0] = lds_read_b128(k_lds, swz_byte<D>(r0, hl));
      rb[0] = lds_read_b128(k_lds, swz_byte<D>(r1, hl));
      ra[1] = lds_read_b128(k_lds, swz_byte<D>(r0, 2 + hl));
      rb[1] = lds_read_b128(k_lds, swz_byte<D>(r1, 2 + hl));
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        if (s + 2 < DS) {
          ra[(s + 2) % 3] = lds_read_b128(k_lds, swz_byte<D>(r0, 2 * (s + 2) + hl));
          rb[(s + 2) % 3] = lds_read_b128(k_lds, swz_byte<D>(r1, 2 * (s + 2) + hl));
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        sacc[0] = mfma32x32x16(ra[s % 3], qreg[s], sacc[0]);
        sacc[1] = mfma32x32x16(rb[s % 3], qreg[s], sacc[1]);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      // plain exact tiles keep raw scores and fold the scale into one FMA per element;
      // tiles with a bias row materialise scale*s + bias first
      float mt;
      if (kind == 0) {
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sacc[u][r], sacc[u][r + 1]));
        mt = fmaxf(mx, xor32(mx)) * c2;
      } else {
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 bv =
                *reinterpret_cast<const f32x4*>(bias_lds + 32 * (ch * KC + u) + 8 * i + 4 * hl);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float x = fmaf(sacc[u][4 * i + j], c2, bv[j]);
              sacc[u][4 * i + j] = x;
              mx = fmaxf(mx, x);
            }
          }
        mt = fmaxf(mx, xor32(mx));
      }
      // move the reference max only when some row's max outgrows it by > kRescale; until
      // then probabilities may exceed 1 (at most 2^kRescale), which fp32 and bf16 carry
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescale) != 0) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      float lsum = 0.f;
      const float nm = -m_run;
      const float cs = kind == 0 ? c2 : 1.f;   // biased scores are already scaled
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(sacc[u][r], cs, nm));
          lsum += e;
          pk[ch * KC + u][r >> 3][r & 7] = (__bf16)e;
        }
      l_run += lsum;
    }
  };
  // O^T += V^T P^T for the pending tile; V^T operands are read one k-step group ahead
  auto pv = [&](const char* v_lds) {
    constexpr int NG = KT * 2;   // k-steps of 16 keys
    bf16x8 va[2][DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      va[0][dt] = lds_read_b128(v_lds, swz_byte<BLK>(32 * dt + l32, hl));
    __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (gi + 1 < NG) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          va[(gi + 1) & 1][dt] =
              lds_read_b128(v_lds, swz_byte<BLK>(32 * dt + l32, 2 * (gi + 1) + hl));
        __builtin_amdgcn_sched_group_barrier(0x100, DT, 0);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = mfma32x32x16(va[gi & 1][dt], pk[gi >> 1][gi & 1], oacc[dt]);
      __builtin_amdgcn_sched_group_barrier(0x008, DT, 0);
    }
  };

  // prologue: K(0) and V(0) into stage 0
  TileDesc cur = tile_desc<D, BLK>(0, n_list, n_list > 0 ? sload(p.pcol, e0) : 0, p.N, p.C,
                                   Kh, Mh, VTh);
  fetch_k(cur.k, cur.valid, smem);
  fetch_vt(cur.v, smem + 2 * TILE);
  if (cur.kind != 0 && tid < 2 * BLK) bias_base[tid] = bias_of(cur, load_count(cur));
  int ent_next = n_list > 1 ? sload(p.pcol, e0 + 1) : 0;
  int use_prev = 0;   // use bits of tile t-1 (for block 2p+1's pending PV)
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    const char* k_lds = smem + st * TILE;
    const float* bias_lds = bias_base + (2 * st + half) * BLK;
    const bool mine = block_ok && ((cur.use >> half) & 1);
    const bool mine_prev = block_ok && ((use_prev >> half) & 1);

    // K(t+1) into the K stage last read in tile t-1; the list entry of tile t+2 is read now
    const bool has_next = t + 1 < ntiles;
    const TileDesc nxt = tile_desc<D, BLK>(t + 1, n_list, ent_next, p.N, p.C, Kh, Mh, VTh);
    int cnt_next = 0;
    if (has_next) {
      fetch_k(nxt.k, nxt.valid, smem + (st ^ 1) * TILE);
      cnt_next = load_count(nxt);
    }

    // phase 1
    if (half == 0) {
      if (mine) scores_softmax(k_lds, bias_lds, cur.kind);
    } else {
      if (t > 0 && mine_prev) pv(smem + (2 + (st ^ 1)) * TILE);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
    // V(t+1) into the V stage block 2p+1 just finished reading (V(t-1))
    if (has_next) fetch_vt(nxt.v, smem + (2 + (st ^ 1)) * TILE);
    // phase 2
    if (half == 0) {
      if (mine) pv(smem + (2 + st) * TILE);
    } else {
      if (mine) scores_softmax(k_lds, bias_lds, cur.kind);
    }

    if (has_next && nxt.kind != 0 && tid < 2 * BLK)
      bias_base[2 * (st ^ 1) * BLK + tid] = bias_of(nxt, cnt_next);
    // list entry of tile t+2, read here so no scalar load is in flight during the phases
    // (outstanding scalar loads would force every LDS wait to drain completely)
    ent_next = t + 2 < n_list ? sload(p.pcol, e0 + t + 2) : 0;
    // all waves are done with this tile's stages, and this thread's prefetches have landed
    __syncthreads();
    use_prev = cur.use;
    cur = nxt;
  }
  // block 2p+1 still owes the PV of the last tile (its V stage is intact)
  if (half == 1 && ntiles > 0 && block_ok && ((use_prev >> 1) & 1))
    pv(smem + (2 + ((ntiles - 1) & 1)) * TILE);

  // Epilogue: normalise and store. Lane holds O[q][32dt + 8i + 4hl + j].
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  if (q < p.N) {
    uint16_t* orow = static_cast<uint16_t*>(p.O) + ((size_t)h * p.N + q) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = (uint32_t)f32_to_bf16_rne(oacc[dt][4 * i + 0] * inv) |
                      ((uint32_t)f32_to_bf16_rne(oacc[dt][4 * i + 1] * inv) << 16);
        uint32_t hi = (uint32_t)f32_to_bf16_rne(oacc[dt][4 * i + 2] * inv) |
                      ((uint32_t)f32_to_bf16_rne(oacc[dt][4 * i + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * i + 4 * hl) = make_uint2(lo, hi);
      }
    if (p.lse != nullptr && hl == 0)
      p.lse[(size_t)h * p.N + q] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// ----------------------------------------------------------------------------- fp32
// Same structure with the fp32 32x32x2 MFMA (full fp32 products). K rows are padded by one
// float and V rows by four so the column-wise operand reads do not pile onto one bank.
template <int D, int BLK>
__global__ void __launch_bounds__(BLK * 2)
fwd_f32_kernel(FwdArgs p) {
  constexpr int THREADS = BLK * 2;
  constexpr int KT = BLK / 32;
  constexpr int DT = D / 32;
  constexpr int KS = D / 2;
  constexpr int KST = D + 1;
  constexpr int VST = D + 4;
  constexpr int NC4 = D / 4;
  constexpr int PER_T = (BLK * NC4) / THREADS;

  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* k_lds = reinterpret_cast<float*>(smem);
  float* v_lds = k_lds + BLK * KST;
  float* bias_lds = v_lds + BLK * VST;

  const int total = p.H * p.nb;
  const int logical = xcd_remap(blockIdx.x, total);
  if (logical >= total) return;
  const int h = logical / p.nb;
  const int b = logical - h * p.nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  const float* Qh = static_cast<const float*>(p.Q) + (size_t)h * p.N * D;
  const float* Kh = static_cast<const float*>(p.K) + (size_t)h * p.N * D;
  const float* Vh = static_cast<const float*>(p.V) + (size_t)h * p.N * D;
  const float* Mh = static_cast<const float*>(p.mu) + (size_t)h * p.C * D;
  const float* Bh = static_cast<const float*>(p.vbar) + (size_t)h * p.C * D;
  const int32_t* cnt_row = p.counts + ((size_t)h * p.nb + b) * p.C;
  const int mh = p.mask_heads == 1 ? 0 : h;
  const int e0 = p.rowptr[mh * (p.nb + 1) + b];
  const int n_exact = p.rowptr[mh * (p.nb + 1) + b + 1] - e0;
  const int ntiles = n_exact + (p.C + BLK - 1) / BLK;

  const int q = b * BLK + w * 32 + l32;
  float qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qreg[s] = q < p.N ? Qh[(size_t)q * D + 2 * s + hl] : 0.f;

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const float *ksrc, *vsrc;
    int valid, kind;
    if (t < n_exact) {
      const int kb = p.col[e0 + t];
      ksrc = Kh + (size_t)kb * BLK * D;
      vsrc = Vh + (size_t)kb * BLK * D;
      valid = min(BLK, p.N - kb * BLK);
      kind = valid < BLK ? 1 : 0;
    } else {
      const int c0 = (t - n_exact) * BLK;
      ksrc = Mh + (size_t)c0 * D;
      vsrc = Bh + (size_t)c0 * D;
      valid = min(BLK, p.C - c0);
      kind = 2;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = i * THREADS + tid;
      const int row = idx / NC4;
      const int c4 = idx - row * NC4;
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (row < valid) {
        kv = *reinterpret_cast<const f32x4*>(ksrc + (size_t)row * D + 4 * c4);
        vv = *reinterpret_cast<const f32x4*>(vsrc + (size_t)row * D + 4 * c4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k_lds[row * KST + 4 * c4 + e] = kv[e];
        v_lds[row * VST + 4 * c4 + e] = vv[e];
      }
    }
    if (tid < BLK) {
      float bv = 0.f;
      if (kind == 1) bv = tid < valid ? 0.f : kNegInf;
      if (kind == 2) {
        const int c = (t - n_exact) * BLK + tid;
        const int n = c < p.C ? cnt_row[c] : 0;
        bv = n > 0 ? fast_log2((float)n) : kNegInf;
      }
      bias_lds[tid] = bv;
    }
    __syncthreads();

    f32x16 sacc[KT];
#pragma unroll
    for (int mk = 0; mk < KT; ++mk) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = mfma32x32x2(k_lds[(32 * mk + l32) * KST + 2 * s + hl], qreg[s], acc);
      sacc[mk] = acc;
    }
    float mloc = kNegInf;
#pragma unroll
    for (int mk = 0; mk < KT; ++mk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * mk + 8 * (r >> 2) + 4 * hl + (r & 3);
        const float x = sacc[mk][r] * p.scale_log2e + bias_lds[key];
        sacc[mk][r] = x;
        mloc = fmaxf(mloc, x);
      }
    const float m_new = fmaxf(m_run, fmaxf(mloc, xor32(mloc)));
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int mk = 0; mk < KT; ++mk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(sacc[mk][r] - m_new);
        sacc[mk][r] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    // O^T += V^T P^T: the k-pair (mk, r) is keys 32mk + 8(r/4) + (r%4) (lower half) and
    // +4 (upper half), which are exactly the lane's score accumulator r.
#pragma unroll
    for (int mk = 0; mk < KT; ++mk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * mk + 8 * (r >> 2) + 4 * hl + (r & 3);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          oacc[dt] = mfma32x32x2(v_lds[key * VST + 32 * dt + l32], sacc[mk][r], oacc[dt]);
      }
  }

  const float l_tot = l_run + xor32(l_run);
  if (q < p.N) {
    float* orow = static_cast<float*>(p.O) + ((size_t)h * p.N + q) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = oacc[dt][4 * i + j] / l_tot;
        *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * i + 4 * hl) = o;
      }
    if (p.lse != nullptr && hl == 0)
      p.lse[(size_t)h * p.N + q] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ----------------------------------------------------------------------------- launch
template <int D, int BLK>
static size_t fwd_lds_bytes(bool bf16) {
  return bf16 ? (size_t)4 * BLK * D * 2 + 4 * BLK * 4
              : (size_t)BLK * (D + 1) * 4 + (size_t)BLK * (D + 4) * 4 + BLK * 4;
}

template <int D, int BLK>
static hipError_t launch_fwd_t(const FwdArgs& a, bool bf16, hipStream_t stream) {
  const size_t lds = fwd_lds_bytes<D, BLK>(bf16);
  if (bf16) {
    hipLaunchKernelGGL((vt_pack_kernel<D, BLK>), dim3(a.nb + a.nct, a.H), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.V), static_cast<const uint16_t*>(a.vbar),
                       static_cast<uint16_t*>(a.vt), a.N, a.C, a.nb, a.nct);
    const int total = a.H * a.npairs;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BLK>), dim3(grid), dim3(BLK * 4), lds, stream, a);
  } else {
    const int total = a.H * a.nb;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((fwd_f32_kernel<D, BLK>), dim3(grid), dim3(BLK * 2), lds, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int head_dim, int block, bool bf16,
                          hipStream_t stream) {
  if (head_dim == 64 && block == 64) return launch_fwd_t<64, 64>(a, bf16, stream);
  if (head_dim == 64 && block == 128) return launch_fwd_t<64, 128>(a, bf16, stream);
  if (head_dim == 128 && block == 64) return launch_fwd_t<128, 64>(a, bf16, stream);
  if (head_dim == 128 && block == 128) return launch_fwd_t<128, 128>(a, bf16, stream);
  return hipErrorInvalidValue;
}

template <int D, int BLK>
static hipError_t prep_fwd() {
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fwd_bf16_kernel<D, BLK>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)fwd_lds_bytes<D, BLK>(true));
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_f32_kernel<D, BLK>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)fwd_lds_bytes<D, BLK>(false));
}

hipError_t prepare_forward_kernels() {
  hipError_t e;
  if ((e = prep_fwd<64, 64>()) != hipSuccess) return e;
  if ((e = prep_fwd<64, 128>()) != hipSuccess) return e;
  if ((e = prep_fwd<128, 64>()) != hipSuccess) return e;
  return prep_fwd<128, 128>();
}

}  // namespace da

// Fused decoupled sparse attention forward for gfx950.
//
// A workgroup walks exact tiles (BLK keys: one key block of BLK keys, or BLK/S key blocks
// of S keys gathered from anywhere in K and V) and then the cluster-cache tiles (C centroid
// keys / mean values taken BLK at a time), treating both the same way:
// the tile's keys and values are staged in LDS, scores come from MFMA, and a single online
// softmax (exp2 domain) absorbs every tile. Cluster tiles add a per-key logit bias
// log2(n[b][c]) (-inf where n = 0), which in the natural-log domain is the ln-count weight
// of the DecoupAttn abstract: each cluster stands in for the n of its keys left outside the
// exact blocks. Optionally (the variance-corrected kernels) each cluster logit also gains
// scale^2 kvar_c ||q||^2 / 2, the second-order weight of a cluster whose keys spread with
// variance kvar_c around its centroid. The bf16 kernel gives a workgroup two adjacent query
// blocks (their exact lists merged); the fp32 kernel one query block.
//
// Work split (bf16): wave w handles 32 query rows. Scores are formed transposed,
// S^T = K * Q^T, so every lane owns one query column and the row max / row sum need only
// one cross-half exchange. O^T = V^T * P^T then leaves each lane with the output of the
// same query, so the online-softmax rescale is a per-lane scalar. V^T operands come
// straight from the row-major V tile through the gfx950 transposed LDS read.
#include "da_device.h"
#include "da_internal.h"

namespace da {

// Schedule of the bf16 kernel's pipelined chunk loop (overridable at build time; a sweep on
// the 13B-class layer left these values best): KC 32-key subtiles per softmax chunk; per MFMA
// of a chunk, NV VALU instructions and ND LDS reads beside it; NPRE LDS reads issued ahead of a
// chunk's first MFMA, and Q0PRE ahead of the first chunk of a tile.
#ifndef FWD_KC
#define FWD_KC 2
#endif
#ifndef FWD_NV
#define FWD_NV 5
#endif
#ifndef FWD_ND
#define FWD_ND 2
#endif
#ifndef FWD_NPRE
#define FWD_NPRE 8
#endif
#ifndef FWD_Q0PRE
#define FWD_Q0PRE 12
#endif

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// XCD-aware order (fp32 kernel; the bf16 kernel uses the plan's work-balanced split):
// hardware deals workgroup ids round-robin to the 8 XCDs; give each XCD a contiguous range of
// (head, query block) so neighbouring query blocks, which share many 3D-local key blocks,
// hit the same L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  int per = (total + 7) >> 3;
  return (L & 7) * per + (L >> 3);
}

// ----------------------------------------------------------------------------- bf16
// A workgroup owns two adjacent query blocks (2p, 2p+1) of one head: BLK/32 waves per
// block. It walks the union of the two exact lists, so a key block both blocks keep exact
// is fetched once (neighbouring query blocks of a 3D-local mask share most of their key
// blocks), then the cluster tiles, which both blocks use with their own bias rows. An
// exact tile holds G = BLK/S consecutive list entries; with G > 1 each tile holds key blocks
// of one set of users (both query blocks, or one of them), the tiles ascending by key. A wave
// skips the tiles that hold no key of its block, and the bias row of the tile masks the
// key blocks of a mixed tile that its block does not keep.
struct TileDesc {
  int off;         // cluster tile: byte offset of its first row in the cache arrays
  int valid;       // cluster tile: rows that exist (clusters < C)
  int kind;        // 0 exact tile, 2 cluster tile
  int c0;          // first cluster of a cluster tile
  int use;         // bit h: query block 2p+h uses some key of this tile
  int partial;     // exact tile: one of its key blocks runs past N
};

// A compile-time int passed to a generic lambda.
template <int N>
struct ic {
  static constexpr int value = N;
};

// The list entries of one exact tile (the first G lanes are used). A vector value, not an
// addressable array: an array passed between the helpers below gets placed in LDS by the
// compiler, costing LDS traffic and full waits every tile.
typedef int32_t ents_t __attribute__((ext_vector_type(8)));

// en[first + j] for a per-lane j in [0, R): a chain of selects over scalar registers.
template <int R>
__device__ __forceinline__ int pick(ents_t en, int first, int j) {
  int v = en[first];
#pragma unroll
  for (int i = 1; i < R; ++i) v = j == i ? en[first + i] : v;
  return v;
}

// Tiles t < n_ex are exact, the rest cluster tiles; with PH (the variance-corrected kernels)
// the first nd (0 or 1) tiles after the exact ones are a placeholder every wave skips, which
// evens the exact count.
template <int D, int BLK, int G, bool PH>
__device__ __forceinline__ TileDesc tile_desc(int t, int n_ex, int nd, ents_t en, int C) {
  TileDesc d;
  if (t < n_ex) {
    int u = 0;
#pragma unroll
    for (int j = 0; j < G; ++j) u |= en[j];
    d.off = 0;
    d.valid = BLK;
    d.kind = 0;
    d.c0 = 0;
    d.use = (u >> kEntUse0) & 3;
    d.partial = (u >> kEntPartial) & 1;
  } else {
    const int ct = PH ? max(t - n_ex - nd, 0) : t - n_ex;
    d.c0 = ct * BLK;
    d.off = d.c0 * D * 2;
    d.valid = min(BLK, C - d.c0);
    d.kind = 2;
    d.use = (PH && t < n_ex + nd) ? 0 : 3;
    d.partial = 0;
  }
  return d;
}

// Scheduling groups for one software-pipelined chunk: NPRE LDS reads, then G times {one
// MFMA, ND LDS reads, NV VALU instructions}, so the matrix core and the VALU of one wave
// run side by side and the operand reads run ahead of the MFMAs that consume them.
template <int G, int NV, int ND, int NPRE>
__device__ __forceinline__ void interleave_mfma_valu() {
  if constexpr (NPRE > 0) __builtin_amdgcn_sched_group_barrier(0x100, NPRE, 0);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (ND > 0) __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}

// VARC: variance-corrected cluster logits. Each cluster tile also carries a row
// w_c = scale * kvar_c / 2 (in the score units), and the score accumulator of key row r and
// this lane's query starts from bias_r + w_r * ||q||^2, so the cluster logit gains
// scale^2 kvar_c ||q||^2 / 2 (exact-tile rows have w = 0).
template <int D, int BLK, int S, bool VARC>
__global__ void __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdArgs p) {
  constexpr int G = BLK / S;       // exact key blocks per tile
  static_assert(G * S == BLK && S >= 16 && G <= 8, "key blocks must tile the query block");
  constexpr int THREADS = BLK * 4;
  constexpr int WPB = BLK / 32;    // waves per query block
  constexpr int KT = BLK / 32;     // 32-key subtiles per key block
  constexpr int DT = D / 32;       // 32-dim tiles of the output
  constexpr int DS = D / 16;       // k-steps of the score product
  constexpr int NCH = D / 8;       // 16-byte chunks per row
  constexpr int TILE = BLK * D * 2;
  constexpr int PER_T = (BLK * NCH) / THREADS;   // 16-byte fetches per thread per tensor
  static_assert(PER_T * THREADS == BLK * NCH, "tile must split evenly");
  // Partial row sum (one lane's 32 probabilities of a chunk) that forces a max update. With
  // probabilities kept at most 2^30, a row sum over thousands of chunks stays below 2^43 and O
  // below 2^43 max|v|, far inside fp32; bf16 and fp32 keep their relative precision at any
  // magnitude. (A limit of 2^15 made the cluster tiles, whose log-count biases lift their
  // probabilities, rescale often: 3% of the forward at 5% density, 9% at 1%.)
  constexpr float kSumLimit = 1073741824.f;
  constexpr int KC = FWD_KC;       // 32-key subtiles per softmax chunk

  // Two LDS stages, each stage's K and V tiles a separate object: with the stage chosen
  // statically (the tile loop is unrolled by two) the compiler can tell that the transposed
  // reads of one stage never alias the direct-to-LDS prefetch into the other, and it does
  // not drain the prefetch before them.
  __shared__ __attribute__((aligned(256))) char k_s0[TILE];
  __shared__ __attribute__((aligned(256))) char k_s1[TILE];
  __shared__ __attribute__((aligned(256))) char v_s0[TILE];
  __shared__ __attribute__((aligned(256))) char v_s1[TILE];
  __shared__ __attribute__((aligned(16))) float bias_s0[2 * BLK];   // [half][BLK]
  __shared__ __attribute__((aligned(16))) float bias_s1[2 * BLK];
  __shared__ __attribute__((aligned(16))) float w_s0[VARC ? 2 * BLK : 4];   // VARC rows
  __shared__ __attribute__((aligned(16))) float w_s1[VARC ? 2 * BLK : 4];

  // workgroup id L runs on XCD L % 8 and takes the next item of that XCD's range
  const int xcd = blockIdx.x & 7;
  const int item = p.xstart[xcd] + (int)(blockIdx.x >> 3);
  if (item >= p.xstart[xcd + 1]) return;
  const int h = item / p.npairs;
  const int pr = item - h * p.npairs;
  const int b0 = 2 * pr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept scalar
  const int half = w / WPB;
  const int wq = w - half * WPB;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int g = lane >> 4;
  const int gp = lane & 15;
  const int bw = b0 + half;
  const bool block_ok = bw < p.nb;

  const char* Qh = static_cast<const char*>(p.Q) + (size_t)h * p.N * D * 2;
  const char* Kh = static_cast<const char*>(p.K) + (size_t)h * p.N * D * 2;
  const char* Vh = static_cast<const char*>(p.V) + (size_t)h * p.N * D * 2;
  const char* Mh = static_cast<const char*>(p.mu) + (size_t)h * p.C * D * 2;
  const char* Bh = static_cast<const char*>(p.vbar) + (size_t)h * p.C * D * 2;

  const int mh = p.mask_heads == 1 ? 0 : h;
  const int e0 = sload(p.prowptr, mh * (p.npairs + 1) + pr);
  const int n_ex = (sload(p.prowptr, mh * (p.npairs + 1) + pr + 1) - e0) / G;   // exact tiles
  // VARC: the exact tiles run the plain score initialisation (their correction row is 0) and
  // the cluster tiles the corrected one, as two loops over static stages; a placeholder tile
  // evens an odd exact count so the cluster loop starts on stage 0
  const int nd = VARC ? (n_ex & 1) : 0;
  const int ntiles = n_ex + nd + (p.C + BLK - 1) / BLK;

  // Direct-to-LDS fetch of one K or V tile: the lane filling physical LDS slot (row, pc)
  // reads logical chunk pc ^ swz_key(row); each wave instruction fills 1 KB of consecutive
  // slots. Rows past `valid` re-read the last valid row: their logits are masked to -inf
  // (and their probabilities are 0), so their contents only need to be finite. The loads go
  // through buffer resources (one per head and tensor, bounded by the tensor's size): unlike
  // the global form they are not flat instructions, so while they are in flight the LDS
  // reads of the current tile keep fine-grained waits.
  auto rsrc = [](const char* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufferWord3);
  };
  const __amdgpu_buffer_rsrc_t rK = rsrc(Kh, p.N * D * 2), rV = rsrc(Vh, p.N * D * 2);
  const __amdgpu_buffer_rsrc_t rM = rsrc(Mh, p.C * D * 2), rB = rsrc(Bh, p.C * D * 2);
  // Pass i of a full tile covers rows ROWS_I*i + tid/NCH; ROWS_I is a multiple of 16, so the
  // swizzle key, and with it the whole per-lane offset, is the same in every pass: the lane
  // offset is computed once and each pass only moves the scalar tile offset. Ragged tiles
  // (the last key block, a short last cluster tile) clamp their rows on the slow path.
  constexpr int ROWS_I = THREADS / NCH;
  static_assert(ROWS_I % 16 == 0, "swizzle key must repeat across fetch passes");
  const int f_off0 = (tid / NCH) * (D * 2) + (((tid % NCH) ^ swz_key<D>(tid / NCH)) << 4);
  // Exact tiles: tile row r holds key row (r % S) of the tile's key block r / S. A key
  // block of S >= ROWS_I rows fills whole passes (the block's offset is the pass's scalar
  // offset); smaller ones split a pass, and each lane picks its block's offset (js = the
  // lane's block within the pass). S is a multiple of 16, so the swizzle key of a tile row
  // is that of its key row.
  constexpr int KBB = S * D * 2;   // bytes of one key block
  const int js = (tid / NCH) / S;
  auto fetch_exact = [&](__amdgpu_buffer_rsrc_t r, ents_t en, bool partial, char* lds_tile) {
    if (!partial) {
#pragma unroll
      for (int i = 0; i < PER_T; ++i) {
        auto* dst = (__attribute__((address_space(3))) void*)(lds_tile + (i * THREADS + w * 64) * 16);
        if constexpr (S >= ROWS_I) {
          const int j = (i * ROWS_I) / S;
          const int soff = (en[j] & kEntIndex) * KBB + ((i * ROWS_I) % S) * (D * 2);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, f_off0, soff, 0, 0);
        } else {
          constexpr int R = ROWS_I / S;
          const int kb = pick<R>(en, i * R, js) & kEntIndex;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, f_off0 + (kb - js) * KBB, 0, 0, 0);
        }
      }
    } else {
      // a key block past N: its missing rows re-read the block's last key (masked to -inf)
#pragma unroll
      for (int i = 0; i < PER_T; ++i) {
        const int slot = i * THREADS + tid;
        const int row = slot / NCH;
        const int pc = slot - row * NCH;
        const int kb = pick<G>(en, 0, row / S) & kEntIndex;
        const int valid = min(S, p.N - kb * S);
        const int off = (kb * S + min(row % S, valid - 1)) * (D * 2) + ((pc ^ swz_key<D>(row)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds_tile + (i * THREADS + w * 64) * 16),
            16, off, 0, 0, 0);
      }
    }
  };
  // Cluster tiles: C rows of the cache arrays taken BLK at a time; a short last tile
  // re-reads its last row.
  auto fetch = [&](__amdgpu_buffer_rsrc_t r, int base, int valid, char* lds_tile) {
    if (valid == BLK) {
#pragma unroll
      for (int i = 0; i < PER_T; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds_tile + (i * THREADS + w * 64) * 16),
            16, f_off0, base + i * ROWS_I * D * 2, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < PER_T; ++i) {
        const int slot = i * THREADS + tid;
        const int row = slot / NCH;
        const int pc = slot - row * NCH;
        const int off = base + min(row, valid - 1) * (D * 2) + ((pc ^ swz_key<D>(row)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(lds_tile + (i * THREADS + w * 64) * 16),
            16, off, 0, 0, 0);
      }
    }
  };
  // Bias rows (log2 domain): thread tid < 2*BLK owns [tid / BLK][tid % BLK]: for an exact
  // tile 0 where the row's key block is kept by that query block and the key exists, else
  // -inf; for a cluster tile log2 n[b][c], or -inf where n = 0. The owners are the first
  // 2*BLK/64 waves, so the half is wave-uniform; the row is rebuilt from the lane id where
  // it is used (from an opaque mask, so no register carries it across the tile loop).
  const int bhalf = w / (BLK / 64);
  const int bq = b0 + bhalf;
  const bool bias_owner = w < 2 * BLK / 64;
  auto brow_now = [&]() -> int {
    uint32_t all = ~0u;
    asm volatile("" : "+s"(all));
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(all, __builtin_amdgcn_mbcnt_lo(all, 0u));
    return ((w % (BLK / 64)) << 6) + ln;
  };
  const int32_t* cnt_row = p.counts + ((size_t)h * p.nb + min(bq, p.nb - 1)) * p.C;
  auto load_count = [&](const TileDesc& d) -> int {
    const int c = d.c0 + brow_now();
    return (d.kind == 2 && bias_owner && c < p.C && bq < p.nb) ? cnt_row[c] : 0;
  };
  // Stored divided by the log2-domain scale: the score accumulators start from it, so the
  // softmax of every tile kind is exp2(scale * (b / scale + q.k) - m).
  const float inv_c2 = 1.f / p.scale_log2e;
  auto bias_of = [&](const TileDesc& d, ents_t en, int n) -> float {
    if (d.kind == 0) {
      const int brow = brow_now();
      const int e = pick<G>(en, 0, brow / S);
      const int key = (e & kEntIndex) * S + brow % S;
      return (((e >> (kEntUse0 + bhalf)) & 1) && key < p.N) ? 0.f : kNegInf;
    }
    return n > 0 ? fast_log2((float)n) * inv_c2 : kNegInf;
  };
  // VARC row of a tile (score units): scale * kvar / 2 for a cluster, 0 for an exact key
  const float half_scale = 0.5f * p.scale_log2e * kLn2;
  auto w_of = [&](const TileDesc& d) -> float {
    const int c = d.c0 + brow_now();
    return (d.kind == 2 && c < p.C) ? half_scale * p.kvar[(size_t)h * p.C + c] : 0.f;
  };
  auto fetch_tile = [&](const TileDesc& d, ents_t en, char* kl, char* vl) {
    if (d.kind == 0) {
      fetch_exact(rK, en, d.partial, kl);
      fetch_exact(rV, en, d.partial, vl);
    } else {
      fetch(rM, d.off, d.valid, kl);
      fetch(rB, d.off, d.valid, vl);
    }
  };
  // list entries of exact tile t (wave-uniform). Every pair's list is a whole number of
  // G-entry tiles, so a tile's entries start at a multiple of G: one scalar load of G words.
  auto load_entries = [&](int t) -> ents_t {
    ents_t en = {0, 0, 0, 0, 0, 0, 0, 0};
    if (t < n_ex) {
      const int at = e0 + G * t;
      if constexpr (G == 1) {
        en[0] = sload(p.pcol, at);
      } else {
        typedef int32_t vG __attribute__((ext_vector_type(G)));
        const vG v = *reinterpret_cast<const __attribute__((address_space(4))) vG*>(
            (const __attribute__((address_space(4))) int32_t*)(p.pcol) + at);
#pragma unroll
        for (int j = 0; j < G; ++j) en[j] = v[j];
      }
    }
    return en;
  };

  // prologue: tile 0 into stage 0
  ents_t en = load_entries(0);   // entries of the tile being prefetched
  TileDesc cur = tile_desc<D, BLK, G, VARC>(0, n_ex, nd, en, p.C);
  fetch_tile(cur, en, k_s0, v_s0);
  if (bias_owner) bias_s0[tid] = bias_of(cur, en, load_count(cur));
  if constexpr (VARC) {
    if (bias_owner) w_s0[tid] = w_of(cur);
  }
  en = load_entries(1);

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
  // ||q||^2 of this lane's query (VARC): this lane holds half of its dims, the lane 32 away
  // the other half
  float qn = 0.f;
  if constexpr (VARC) {
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qreg[s][e];
        qn = fmaf(x, x, qn);
      }
    qn += xor32(qn);
  }

  // Lane parts of the swizzled LDS read addresses. The swizzle key of a row depends only on
  // its low four bits, so across the reads of a tile the K address is
  // kx ^ (s << 5) + 32 mk rows and the V address vx ^ (dt << 6) + rows: one base per operand
  // class, the XOR touching bits below 256 and the rest an immediate offset.
  const int kx = l32 * (2 * D) + ((hl ^ swz_key<D>(l32)) << 4);
  const int vr = 4 * (g >> 1) + (gp >> 2);
  const int vc = 2 * (g & 1) + ((gp & 3) >> 1);
  const int vx_lo = vr * (2 * D) + ((vc ^ swz_key<D>(vr)) << 4) + ((gp & 1) << 3);
  const int vx_hi = (vr + 8) * (2 * D) + ((vc ^ swz_key<D>(vr + 8)) << 4) + ((gp & 1) << 3);

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -1e30f;   // reference max (log2 domain); finite so exp2(m_run - x) is safe
  float l_run = 0.f;      // this half-wave's share of the row sum
  const float c2 = p.scale_log2e;
  __syncthreads();

  // one tile: compute on (k_lds, v_lds, bias_cur) while tile t+1 streams into (nk, nv)
  // Score initialisation of this tile: mode 0 from the bias row, 1 from the bias and
  // variance rows (VARC), 2 zero (an exact tile whose bias row is all zero)
  auto tile = [&](auto mode, int t, const char* k_lds, const char* v_lds, const float* bias_cur,
                  const float* w_cur, char* nk, char* nv, float* bias_nxt, float* w_nxt) {
    constexpr bool VN = VARC && decltype(mode)::value == 1;
    constexpr bool ZI = decltype(mode)::value == 2;
    const float* bias_lds = bias_cur + half * BLK;
    const float* w_lds = w_cur + half * BLK;

    // prefetch tile t+1 into the other stage (free since the barrier closing tile t-1)
    const bool has_next = t + 1 < ntiles;
    const TileDesc nxt = tile_desc<D, BLK, G, VARC>(t + 1, n_ex, nd, en, p.C);
    int cnt_next = 0;
    float w_next = 0.f;
    if (has_next) {
      fetch_tile(nxt, en, nk, nv);
      cnt_next = load_count(nxt);
      if constexpr (VARC) w_next = bias_owner ? w_of(nxt) : 0.f;
    }

    if (block_ok && ((cur.use >> half) & 1)) {
      // This stage's read bases as LDS byte addresses, opaque per tile so that the compiler
      // keeps one set live (not both stages' hoisted copies) and folds the row offsets
      // into the reads' immediate field. The tiles are 256-byte aligned, so adding the
      // tile address commutes with the XORs.
      const int ka = lds_addr(k_lds), va = lds_addr(v_lds);
      int kb = kx + ka, vlo = vx_lo + va, vhi = vx_hi + va;
      asm volatile("" : "+v"(kb), "+v"(vlo), "+v"(vhi));
      // The tile is processed in chunks of KC 32-key subtiles, software-pipelined inside
      // each wave: while the VALU computes the softmax of chunk c, the matrix core runs the
      // scores of chunk c+1 and the PV product of chunk c-1 (both independent of it), the
      // two instruction streams interleaved by the scheduling groups below. The lazily
      // moved reference max lets each chunk use it without seeing the rest of the tile.
      constexpr int NCK = KT / KC;
      f32x16 sacc[2][KC];
      // P = exp2(x - m_run) packed to bf16 (the B operand of O^T += V^T P^T: k-step
      // (u, t2) covers keys 32mk + 16t2 + {0..15}; this lane's eight k-values are keys
      // 32mk + 16t2 + 8i' + 4hl + j (i' = 0,1; j = 0..3) = score accumulators 8t2 .. 8t2+7).
      bf16x8 pk[2][KC][2];
      // Scores start from the tile's bias row (0 for a kept key, -inf for a key past N or of
      // a key block the query block does not keep, and log2 of the outside count for a
      // cluster tile, all divided by the scale), or from zero in a tile whose row is known
      // to be all zero.
      auto qk = [&](int ch, f32x16 (&sc)[KC]) {
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (ZI) {
#pragma unroll
              for (int j = 0; j < 4; ++j) sc[u][4 * i + j] = 0.f;
              continue;
            }
            const f32x4 bv = *reinterpret_cast<const f32x4*>(
                bias_lds + 32 * (ch * KC + u) + 8 * i + 4 * hl);
            if constexpr (VN) {
              const f32x4 wv = *reinterpret_cast<const f32x4*>(
                  w_lds + 32 * (ch * KC + u) + 8 * i + 4 * hl);
#pragma unroll
              for (int j = 0; j < 4; ++j) sc[u][4 * i + j] = fmaf(wv[j], qn, bv[j]);
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) sc[u][4 * i + j] = bv[j];
            }
          }
#pragma unroll
        for (int s = 0; s < DS; ++s)
#pragma unroll
          for (int u = 0; u < KC; ++u) {
            const int mk = ch * KC + u;
            const bf16x8 a = lds_read_b128(k_lds, (kb ^ (s << 5)) - ka + mk * 64 * D);
            sc[u] = mfma32x32x16(a, qreg[s], sc[u]);
          }
      };
      // V^T operands straight from the row-major V tile by the transposed LDS read: in
      // each 16-lane group, lane 4s + i/4 addresses keys row (s) and 4 dims, and lane i
      // receives those 4 keys for dim i.
      auto pv = [&](int ch, const bf16x8 (&pc)[KC][2]) {
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const int roff = (32 * (ch * KC + u) + 16 * t2) * (2 * D) - va;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const bf16x4 lo = lds_read_tr16(v_lds, (vlo ^ (dt << 6)) + roff);
              const bf16x4 hi = lds_read_tr16(v_lds, (vhi ^ (dt << 6)) + roff);
              const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              oacc[dt] = mfma32x32x16(a, pc[u][t2], oacc[dt]);
            }
          }
      };
      // The row share is summed in fp32 from the unrounded probabilities (plain adds, which
      // run beside the MFMAs; the packed dot product does not), four partial sums deep.
      auto exp_pack = [&](const f32x16 (&sc)[KC], bf16x8 (&pc)[KC][2]) -> float {
        const float nm = -m_run;
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(sc[u][r], c2, nm));
            pc[u][r >> 3][r & 7] = (__bf16)e;
            ls[r & 3] += e;
          }
        return (ls[0] + ls[1]) + (ls[2] + ls[3]);
      };
      qk(0, sacc[0]);
      // the first chunk's scores have no softmax to hide behind: issue their operand reads
      // well ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, FWD_Q0PRE, 0);
#pragma unroll
      for (int i = 0; i < DS * KC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ch = 0; ch < NCK; ++ch) {
        f32x16 (&sc)[KC] = sacc[ch & 1];
        bf16x8 (&pc)[KC][2] = pk[ch & 1];
        if (ch + 1 < NCK) qk(ch + 1, sacc[(ch + 1) & 1]);
        if (ch > 0) pv(ch - 1, pk[(ch - 1) & 1]);
        float lsum = exp_pack(sc, pc);
        interleave_mfma_valu<16 * KC, FWD_NV, FWD_ND, FWD_NPRE>();
        // The reference max moves only when some row's probabilities outgrow it (a partial
        // row sum above 2^30, or inf on the first tile); then the chunk's true max is taken,
        // O (including the PV of chunk c-1, computed at the old max) and l are rescaled and
        // the chunk is recomputed. Otherwise probabilities may exceed 1 (each at most
        // 2^30), which fp32 and bf16 carry.
        if (__builtin_amdgcn_ballot_w64(!(lsum <= kSumLimit)) != 0) {
          float mx = kNegInf;
#pragma unroll
          for (int u = 0; u < KC; ++u)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sc[u][r], sc[u][r + 1]));
          const float mt = fmaxf(mx, xor32(mx)) * c2;
          const float m_new = fmaxf(m_run, mt);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
          lsum = exp_pack(sc, pc);
        }
        l_run += lsum;
      }
      pv(NCK - 1, pk[(NCK - 1) & 1]);
    }

    if (has_next && bias_owner) bias_nxt[tid] = bias_of(nxt, en, cnt_next);
    if constexpr (VARC) {
      if (has_next && bias_owner) w_nxt[tid] = w_next;
    }
    // list entries of tile t+2, read here so no scalar load is in flight during the compute
    // (an outstanding scalar load forces every LDS wait to drain completely)
    en = load_entries(t + 2);
    // all waves are done with this stage, and this thread's prefetch has landed
    __syncthreads();
    cur = nxt;
  };
  if constexpr (VARC) {
    int t = 0;
    for (; t < n_ex + nd; t += 2) {   // an even count
      tile(ic<0>{}, t, k_s0, v_s0, bias_s0, w_s0, k_s1, v_s1, bias_s1, w_s1);
      tile(ic<0>{}, t + 1, k_s1, v_s1, bias_s1, w_s1, k_s0, v_s0, bias_s0, w_s0);
    }
    for (; t < ntiles; t += 2) {
      tile(ic<1>{}, t, k_s0, v_s0, bias_s0, w_s0, k_s1, v_s1, bias_s1, w_s1);
      if (t + 1 < ntiles)
        tile(ic<1>{}, t + 1, k_s1, v_s1, bias_s1, w_s1, k_s0, v_s0, bias_s0, w_s0);
    }
  } else {
    // With one key block per tile, a used exact tile's bias row is all zero unless its key
    // block runs past N (only the last): an even number of the clean tiles first, scores
    // starting from zero with no bias-row reads, then the rest from their bias rows.
    if constexpr (G == 1) {
      int n_clean = n_ex;
      if (n_ex > 0 && ((sload(p.pcol, e0 + n_ex - 1) >> kEntPartial) & 1)) n_clean -= 1;
      int t = 0;
      for (; t < (n_clean & ~1); t += 2) {
        tile(ic<2>{}, t, k_s0, v_s0, bias_s0, w_s0, k_s1, v_s1, bias_s1, w_s1);
        tile(ic<2>{}, t + 1, k_s1, v_s1, bias_s1, w_s1, k_s0, v_s0, bias_s0, w_s0);
      }
      for (; t < ntiles; t += 2) {
        tile(ic<0>{}, t, k_s0, v_s0, bias_s0, w_s0, k_s1, v_s1, bias_s1, w_s1);
        if (t + 1 < ntiles)
          tile(ic<0>{}, t + 1, k_s1, v_s1, bias_s1, w_s1, k_s0, v_s0, bias_s0, w_s0);
      }
    } else {
      for (int t = 0; t < ntiles; t += 2) {
        tile(ic<0>{}, t, k_s0, v_s0, bias_s0, w_s0, k_s1, v_s1, bias_s1, w_s1);
        if (t + 1 < ntiles)
          tile(ic<0>{}, t + 1, k_s1, v_s1, bias_s1, w_s1, k_s0, v_s0, bias_s0, w_s0);
      }
    }
  }

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
// Same structure with the fp32 32x32x2 MFMA (full fp32 products), one query block per
// workgroup. An exact tile gathers the next BLK/S key blocks of the block's list (S, the key
// block size, is a power of two dividing BLK). K rows are padded by one float and V rows by
// four so the column-wise operand reads do not pile onto one bank.
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
  float* w_lds = bias_lds + BLK;   // variance-correction row (log2 units), when p.kvar is set

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
  const int n_exact = p.rowptr[mh * (p.nb + 1) + b + 1] - e0;   // exact key blocks
  const int S = p.kblock;
  const int sh = __builtin_ctz(S);
  const int G = BLK >> sh;
  const int n_ex = (n_exact + G - 1) / G;                         // exact tiles
  const int ntiles = n_ex + (p.C + BLK - 1) / BLK;

  const int q = b * BLK + w * 32 + l32;
  float qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qreg[s] = q < p.N ? Qh[(size_t)q * D + 2 * s + hl] : 0.f;
  // ||q||^2 (this lane holds the even or odd dims, the lane 32 away the others)
  float qn = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) qn = fmaf(qreg[s], qreg[s], qn);
  qn += xor32(qn);
  // log2 units: scale^2 * kvar / 2 * log2(e)
  const float wscale = 0.5f * p.scale_log2e * p.scale_log2e * kLn2;

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;

  // Source row of tile row `row`: an exact tile's row r is key (r % S) of its (r / S)-th
  // key block, or no key (-1) past the list's end or past N; a cluster tile's row r is
  // cluster c0 + r, or none past C.
  auto src_row = [&](int t, int row) -> int {
    if (t < n_ex) {
      const int e = t * G + (row >> sh);
      const int key = e < n_exact ? (p.col[e0 + e] << sh) + (row & (S - 1)) : p.N;
      return key < p.N ? key : -1;
    }
    const int c = (t - n_ex) * BLK + row;
    return c < p.C ? c : -1;
  };

  for (int t = 0; t < ntiles; ++t) {
    const bool exact = t < n_ex;
    const float* ksrc = exact ? Kh : Mh;
    const float* vsrc = exact ? Vh : Bh;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int idx = i * THREADS + tid;
      const int row = idx / NC4;
      const int c4 = idx - row * NC4;
      const int sr = src_row(t, row);
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (sr >= 0) {
        kv = *reinterpret_cast<const f32x4*>(ksrc + (size_t)sr * D + 4 * c4);
        vv = *reinterpret_cast<const f32x4*>(vsrc + (size_t)sr * D + 4 * c4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k_lds[row * KST + 4 * c4 + e] = kv[e];
        v_lds[row * VST + 4 * c4 + e] = vv[e];
      }
    }
    if (tid < BLK) {
      const int sr = src_row(t, tid);
      float bv = sr >= 0 ? 0.f : kNegInf;
      if (!exact) {
        const int n = sr >= 0 ? cnt_row[sr] : 0;
        bv = n > 0 ? fast_log2((float)n) : kNegInf;
      }
      bias_lds[tid] = bv;
      float wv = 0.f;
      if (!exact && p.kvar != nullptr && sr >= 0) wv = wscale * p.kvar[(size_t)h * p.C + sr];
      w_lds[tid] = wv;
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
        const float x = sacc[mk][r] * p.scale_log2e + fmaf(w_lds[key], qn, bias_lds[key]);
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
              : (size_t)BLK * (D + 1) * 4 + (size_t)BLK * (D + 4) * 4 + 2 * BLK * 4;
}

template <int D, int BLK, int S>
static hipError_t launch_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.kvar != nullptr)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BLK, S, true>), dim3(8 * a.xmax), dim3(BLK * 4), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BLK, S, false>), dim3(8 * a.xmax), dim3(BLK * 4), 0,
                       stream, a);
  return hipGetLastError();
}

template <int D, int BLK>
static hipError_t launch_fwd_t(const FwdArgs& a, int kblock, bool bf16, hipStream_t stream) {
  if (bf16) {
    switch (kblock) {
      case 16: return launch_bf16<D, BLK, 16>(a, stream);
      case 32: return launch_bf16<D, BLK, 32>(a, stream);
      case 64: return launch_bf16<D, BLK, 64>(a, stream);
      case 128:
        if constexpr (BLK >= 128) return launch_bf16<D, BLK, 128>(a, stream);
        break;
      default: break;
    }
    return hipErrorInvalidValue;
  }
  if (kblock < 16 || kblock > BLK || (kblock & (kblock - 1)) != 0) return hipErrorInvalidValue;
  const int total = a.H * a.nb;
  const int grid = ((total + 7) / 8) * 8;
  const size_t lds = fwd_lds_bytes<D, BLK>(false);
  hipLaunchKernelGGL((fwd_f32_kernel<D, BLK>), dim3(grid), dim3(BLK * 2), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int head_dim, int block, int kblock, bool bf16,
                          hipStream_t stream) {
  if (head_dim == 64 && block == 64) return launch_fwd_t<64, 64>(a, kblock, bf16, stream);
  if (head_dim == 64 && block == 128) return launch_fwd_t<64, 128>(a, kblock, bf16, stream);
  if (head_dim == 128 && block == 64) return launch_fwd_t<128, 64>(a, kblock, bf16, stream);
  if (head_dim == 128 && block == 128) return launch_fwd_t<128, 128>(a, kblock, bf16, stream);
  return hipErrorInvalidValue;
}

template <int D, int BLK>
static hipError_t prep_fwd() {
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

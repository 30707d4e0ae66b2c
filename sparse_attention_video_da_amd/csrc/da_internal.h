// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_lists.h"

namespace da {

// Everything the fused forward kernel reads, in device memory.
struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* mu;        // [H][C][d] centroid keys
  const void* vbar;      // [H][C][d] mean values
  const int32_t* counts; // [H][nb][C]
  const int32_t* rowptr; // [mask_heads][nb + 1], absolute offsets into col
  const int32_t* col;    // sorted exact key blocks (of kblock keys)
  const int32_t* prowptr; // [mask_heads][npairs + 1] lists of query-block pairs (2p, 2p+1)
  const int32_t* pcol;    // union of the pair's exact key blocks (entry format: kEnt* above)
  int npairs;
  int xstart[9];         // items (h * npairs + pair) xstart[x] .. xstart[x+1]-1 run on XCD x
  int xmax;              // largest range
  void* O;
  float* lse;            // may be null
  int H, N, C, nb, mask_heads;
  int kblock;            // exact key block size S (divides the query block size)
  float scale_log2e;     // softmax scale * log2(e)
  const float* kvar;     // [H][C] key variance for the variance-corrected cluster logits, or null
};

// Near-tie lists of the bf16 assignment: one counter per head (H ints, padded to 64), then per
// head up to N entries (key, smallest packed distance) as int2, at int offset
// fix_list_offset(H).
inline size_t fix_list_offset(int heads) { return (size_t)(heads + 63) / 64 * 64; }

struct ReassignArgs {
  const void* K;
  const void* V;
  const void* mu_in;
  void* mu_out;
  void* vbar_out;
  int32_t* assign;
  int32_t* sizes;
  int32_t* counts;
  const int32_t* rowptr;
  const int32_t* col;
  const int32_t* prowptr;  // query-block pair lists (as in FwdArgs)
  const int32_t* pcol;
  int npairs;
  uint8_t* hist;   // workspace [H][nb][C] per-block cluster histograms (<= block keys)
  int32_t* off;    // workspace [H][nb][C]
  int32_t* start;  // workspace [H][C]
  int32_t* perm;   // workspace [H][N]
  uint16_t* cop;   // workspace: bf16 distance operands, [H][C][D] (-2 mu) then [H][C][8]
  float* part;     // workspace [H][ceil(N / 256) + C][2][D] partial sums of K and V
  float* psq;      // workspace [H][ceil(N / 256) + C] partial sums of squared key norms
  float* kvar;     // [H][C] key variance output, or null (not computed)
  int32_t* fix;    // workspace: near-tie counters [H], lists [H][N] int2 (fix_list_offset)
  int H, N, C, nb, block, mask_heads;
  int kblock;      // exact key block size S
  int ncu;         // compute units of the device (grid of the persistent assignment)
};

// Return hipSuccess or the first launch error.
hipError_t launch_forward(const FwdArgs& a, int head_dim, int block, int kblock, bool bf16,
                          hipStream_t stream);
hipError_t launch_reassign(const ReassignArgs& a, int head_dim, bool bf16, hipStream_t stream);
// One-time per-process kernel attribute setup (dynamic LDS limits).
hipError_t prepare_kernels();

// Static device scratch of da_reassign_noalloc: kScratchBytes per device, in the library's
// code object. scratch_setup (called once per device, with that device current) records
// its device address; scratch_address returns it (hipErrorNotReady before set-up).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_setup(int device);
hipError_t scratch_address(int device, void** out);

}  // namespace da

// Host-side plan compilation: block mask -> exact lists, query-block-pair tile lists and the
// forward's per-XCD work split. Plain C++ (no HIP), so it also builds for host-only tests.
#pragma once

#include <cstdint>
#include <vector>

namespace da {

// Pair-list entry: key block index | used by query block 2p | used by 2p+1 | the key block
// runs past N. With G = B/S key blocks per tile (S < B) a pair's list is a sequence of
// G-entry tiles, each holding key blocks of one set of users (both, only 2p, only 2p+1),
// ascending by first key block; padding entries repeat a set's last entry with its use
// bits clear.
constexpr int32_t kEntIndex = 0x0fffffff;
constexpr int kEntUse0 = 28, kEntUse1 = 29, kEntPartial = 30;

struct PlanLists {
  std::vector<int32_t> rowptr;   // [mask_heads][nb + 1], absolute offsets into col
  std::vector<int32_t> col;      // ascending exact key blocks of each query block
  std::vector<int32_t> prowptr;  // [mask_heads][npairs + 1], absolute offsets into pcol
  std::vector<int32_t> pcol;     // pair lists (entry format above)
  int32_t npairs = 0;
  // bf16 forward schedule: work items (head, pair) in natural order split into 8 contiguous
  // ranges of about equal work, range x for XCD x
  int32_t xstart[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  int32_t xmax = 0;
};

// mask: [mask_heads][nb][nkb] (nb = ceil(seq_len / block), nkb = ceil(seq_len / key_block)),
// nonzero = exact. Sizes are assumed validated (key_block divides block, int32 ranges).
void build_plan_lists(const uint8_t* mask, int32_t mask_heads, int32_t heads, int32_t seq_len,
                      int32_t block, int32_t key_block, int32_t clusters, PlanLists& out);

}  // namespace da

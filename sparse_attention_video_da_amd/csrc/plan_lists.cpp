// Host-side plan compilation (see plan_lists.h).
#include "plan_lists.h"

#include <algorithm>

namespace da {

void build_plan_lists(const uint8_t* mask, int32_t mask_heads, int32_t heads, int32_t seq_len,
                      int32_t block, int32_t key_block, int32_t clusters, PlanLists& out) {
  const int32_t nb = (seq_len + block - 1) / block;
  const int32_t S = key_block;
  const int32_t nkb = (seq_len + S - 1) / S;
  const int32_t G = block / S;   // exact key blocks per B-row tile
  out = PlanLists{};
  // Exact lists: for each mask head and query block, the ascending key blocks kept exact.
  out.rowptr.resize((size_t)mask_heads * (nb + 1));
  for (int32_t mh = 0; mh < mask_heads; ++mh) {
    const uint8_t* m = mask + (size_t)mh * nb * nkb;
    for (int32_t b = 0; b < nb; ++b) {
      out.rowptr[(size_t)mh * (nb + 1) + b] = (int32_t)out.col.size();
      for (int32_t kb = 0; kb < nkb; ++kb)
        if (m[(size_t)b * nkb + kb]) out.col.push_back(kb);
    }
    out.rowptr[(size_t)mh * (nb + 1) + nb] = (int32_t)out.col.size();
  }
  // Pair lists. With several key blocks per tile, each tile holds key blocks of one set of
  // users (both query blocks, only 2p, or only 2p+1), so a query block's waves skip the
  // tiles that hold none of its keys and never compute a masked key block; each set is cut
  // into tiles in ascending order (its last tile padded with copies of its last entry whose
  // use bits are clear), and the tiles of the three sets are merged by first key block.
  // The walk then stays ascending, as with one key block per tile: workgroups of
  // neighbouring pairs, which run at the same time on one XCD, request the same key blocks
  // close together in time and share them in L2.
  const int32_t npairs = (nb + 1) / 2;
  const bool partial_last = seq_len % S != 0;
  out.npairs = npairs;
  out.prowptr.resize((size_t)mask_heads * (npairs + 1));
  std::vector<int32_t> sets[3];
  for (int32_t mh = 0; mh < mask_heads; ++mh) {
    const uint8_t* m = mask + (size_t)mh * nb * nkb;
    for (int32_t pr = 0; pr < npairs; ++pr) {
      out.prowptr[(size_t)mh * (npairs + 1) + pr] = (int32_t)out.pcol.size();
      const int32_t b0 = 2 * pr, b1 = 2 * pr + 1;
      for (auto& v : sets) v.clear();
      for (int32_t kb = 0; kb < nkb; ++kb) {
        const int32_t f0 = m[(size_t)b0 * nkb + kb] ? 1 : 0;
        const int32_t f1 = (b1 < nb && m[(size_t)b1 * nkb + kb]) ? 1 : 0;
        if (!(f0 | f1)) continue;
        const int32_t ent = kb | (f0 << kEntUse0) | (f1 << kEntUse1) |
                            ((partial_last && kb == nkb - 1) ? 1 << kEntPartial : 0);
        if (G == 1) out.pcol.push_back(ent);
        else sets[(f0 & f1) ? 0 : (f0 ? 1 : 2)].push_back(ent);
      }
      if (G == 1) continue;
      for (auto& v : sets)
        if (v.size() % G != 0) {
          const int32_t pad = v.back() & ~((1 << kEntUse0) | (1 << kEntUse1));
          v.resize((v.size() / G + 1) * G, pad);
        }
      size_t at[3] = {0, 0, 0};
      for (;;) {
        int best = -1;
        for (int i = 0; i < 3; ++i)
          if (at[i] < sets[i].size() &&
              (best < 0 || (sets[i][at[i]] & kEntIndex) < (sets[best][at[best]] & kEntIndex)))
            best = i;
        if (best < 0) break;
        out.pcol.insert(out.pcol.end(), sets[best].begin() + at[best],
                        sets[best].begin() + at[best] + G);
        at[best] += G;
      }
    }
    out.prowptr[(size_t)mh * (npairs + 1) + npairs] = (int32_t)out.pcol.size();
  }
  // Balanced split of the forward's work items over the 8 XCDs (workgroup ids are dealt to
  // XCDs round-robin). An item's work is its tile count: the exact tiles of the pair's
  // union list plus the cluster tiles, plus one tile for its prologue and epilogue. Contiguous
  // ranges keep neighbouring query blocks, which share key blocks, on one L2; equal work
  // per range keeps the XCDs busy equally long when budgets differ across heads or blocks.
  const int64_t items = (int64_t)heads * npairs;
  const int32_t ctiles = (clusters + block - 1) / block;
  std::vector<int64_t> pre((size_t)items + 1, 0);
  for (int64_t i = 0; i < items; ++i) {
    const int32_t h = (int32_t)(i / npairs), pr = (int32_t)(i % npairs);
    const size_t base = (size_t)(mask_heads == 1 ? 0 : h) * (npairs + 1);
    const int64_t len = (out.prowptr[base + pr + 1] - out.prowptr[base + pr]) / G;
    pre[(size_t)i + 1] = pre[(size_t)i] + len + ctiles + 1;
  }
  int64_t at = 0;
  out.xstart[0] = 0;
  for (int x = 1; x < 8; ++x) {
    const int64_t target = (pre[(size_t)items] * x + 4) / 8;
    while (at < items && pre[(size_t)at + 1] <= target) ++at;
    out.xstart[x] = (int32_t)at;
  }
  out.xstart[8] = (int32_t)items;
  for (int x = 0; x < 8; ++x) out.xmax = std::max(out.xmax, out.xstart[x + 1] - out.xstart[x]);
}

}  // namespace da

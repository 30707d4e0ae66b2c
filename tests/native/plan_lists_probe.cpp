// Host-only C entry point over the library's plan compilation, for CPU tests (built with g++
// by the tests; not part of the library).
#include <cstring>

#include "plan_lists.h"

extern "C" int probe_plan_lists(const unsigned char* mask, int mask_heads, int heads,
                                int seq_len, int block, int key_block, int clusters,
                                int* rowptr, int* col, int* prowptr, int* pcol, int* xstart,
                                long long* sizes) {
  da::PlanLists l;
  da::build_plan_lists(mask, mask_heads, heads, seq_len, block, key_block, clusters, l);
  sizes[0] = (long long)l.rowptr.size();
  sizes[1] = (long long)l.col.size();
  sizes[2] = (long long)l.prowptr.size();
  sizes[3] = (long long)l.pcol.size();
  sizes[4] = l.npairs;
  sizes[5] = l.xmax;
  if (rowptr) std::memcpy(rowptr, l.rowptr.data(), l.rowptr.size() * sizeof(int));
  if (col && !l.col.empty()) std::memcpy(col, l.col.data(), l.col.size() * sizeof(int));
  if (prowptr) std::memcpy(prowptr, l.prowptr.data(), l.prowptr.size() * sizeof(int));
  if (pcol && !l.pcol.empty()) std::memcpy(pcol, l.pcol.data(), l.pcol.size() * sizeof(int));
  if (xstart) std::memcpy(xstart, l.xstart, sizeof(l.xstart));
  return 0;
}

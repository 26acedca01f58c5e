// Per-chunk candidate selection: the m best keys of one chunk of positions and
// the best key left out. Used in the epilogue of the score kernel and by the
// stand-alone candidate kernel.
#pragma once

#include "common.h"

namespace dsa {

struct ChunkSmem {
  SelectSmem sel;
  int counts[kWaves];
  int base;
};

// scores: LDS copy of the chunk's scores (entry i is position pos0 + i); count:
// valid entries (<= 0 means none). Writes out[0..m) (best keys in position
// order, 0-padded) and *x_out = the largest key not kept (0 if every valid
// position is kept).
__device__ inline void chunk_candidates(const int32_t* scores, int count, uint32_t pos0, int m,
                                        uint64_t* __restrict__ out, uint64_t* __restrict__ x_out,
                                        ChunkSmem& sm) {
  const int tid = threadIdx.x;
  if (count <= 0) {
    for (int i = tid; i < m; i += kBlock) out[i] = 0;
    if (tid == 0) *x_out = 0;
    return;
  }
  auto key_at = [&](int i) { return make_key(scores[i], pos0 + (uint32_t)i); };
  uint64_t x = 0;
  if (count > m) x = block_kth_largest(count, m + 1, key_at, sm.sel);
  // keys above x (all valid keys when x == 0), in position order
  if (tid == 0) sm.base = 0;
  __syncthreads();
  const int kept = count > m ? m : count;
  for (int r = 0; r < count; r += kBlock) {
    const int i = r + tid;
    uint64_t key = 0;
    bool keep = false;
    if (i < count) {
      key = key_at(i);
      keep = key > x;
    }
    const int slot = block_compact_slot(keep, sm.counts, &sm.base);
    if (keep) out[slot] = key;
  }
  for (int i = kept + tid; i < m; i += kBlock) out[i] = 0;
  if (tid == 0) *x_out = x;
}

}  // namespace dsa

// Per-chunk candidate selection: the m best keys of one chunk of positions and
// the best key left out. Used in the epilogue of the score kernel and by the
// stand-alone candidate kernel.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kChunkPerThread = 16;  // chunk length <= 16 * block size

template <int BLOCK>
struct ChunkSmem {
  RadixSmem radix;  // zero on entry to chunk_candidates (radix_clear once per kernel)
  uint32_t xch[BLOCK / 64][2];
};

// scores: LDS copy of the chunk's scores (entry i is position pos0 + i); count:
// valid entries (<= 0 means none; at most 16 * BLOCK). Writes out[0..m) (the m
// best keys, in position order, 0-padded) and *x_out = the best key not kept
// (0 if every valid position is kept).
//
// The (m+1)-th best score T comes from a radix selection over the scores; the
// kept keys are those scoring above T plus the first (m - #above) positions
// scoring exactly T, which is the key order (score, then lower position).
template <int BLOCK>
__device__ __forceinline__ void chunk_candidates(const int32_t* scores, int count, uint32_t pos0, int m,
                                 uint64_t* __restrict__ out, uint64_t* __restrict__ x_out,
                                 ChunkSmem<BLOCK>& sm) {
  const int tid = threadIdx.x;
  if (count <= m) {
    for (int i = tid; i < m; i += BLOCK)
      out[i] = i < count ? make_key(scores[i], pos0 + (uint32_t)i) : 0ull;
    if (tid == 0) *x_out = 0;
    return;
  }
  const int per = (count + BLOCK - 1) / BLOCK;  // contiguous elements per thread
  const int i0 = tid * per;
  uint32_t u[kChunkPerThread];
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int j = 0; j < kChunkPerThread; ++j) {  // every load issued before any use
    const int i = i0 + j < count ? i0 + j : count - 1;
    u[j] = score_bits(scores[i]);
  }
#pragma unroll
  for (int j = 0; j < kChunkPerThread; ++j) {
    const bool in = j < per && i0 + j < count;
    lo = in && u[j] < lo ? u[j] : lo;
    hi = in && u[j] > hi ? u[j] : hi;
  }
  auto each = [&](auto f) {
#pragma unroll
    for (int j = 0; j < kChunkPerThread; ++j)
      if (j < per && i0 + j < count) f(u[j]);
  };
  DSA_MARK(3, 0);
  {
    const uint32_t mine[2] = {~wave_min_u32(lo), wave_maxr_u32(hi)};
    uint32_t all[BLOCK / 64][2];
    block_exchange<BLOCK, 2>(mine, sm.xch, all);
    uint32_t nlo = 0, mhi = 0;
#pragma unroll
    for (int w = 0; w < BLOCK / 64; ++w) {
      nlo = all[w][0] > nlo ? all[w][0] : nlo;
      mhi = all[w][1] > mhi ? all[w][1] : mhi;
    }
    lo = ~nlo;
    hi = mhi;
  }
  uint32_t above;
  DSA_MARK(3, 1);
  const uint32_t T = block_select_range<BLOCK>(each, lo, hi, m + 1, &above, sm.radix);
  DSA_MARK(3, 8);
  const uint32_t need_eq = (uint32_t)(m + 1) - above;  // >= 1: keys at T up to and including x
  uint32_t gt = 0, eq = 0;
  each([&](uint32_t v) {
    gt += v > T;
    eq += v == T;
  });
  uint32_t total;
  const uint32_t before = block_excl_scan_u32<BLOCK>(gt | (eq << 16), sm.radix.part, &total);
  const uint32_t eq_before = before >> 16;
  uint32_t slot = (before & 0xFFFF) + (eq_before < need_eq - 1 ? eq_before : need_eq - 1);
  uint32_t eqr = eq_before;
  DSA_MARK(3, 9);
#pragma unroll
  for (int j = 0; j < kChunkPerThread; ++j) {
    const int i = i0 + j;
    if (j < per && i < count) {
      const uint64_t key = ((uint64_t)u[j] << 32) | (uint64_t)(0xFFFFFFFFu - (pos0 + (uint32_t)i));
      if (u[j] > T) {
        out[slot++] = key;
      } else if (u[j] == T) {
        if (eqr < need_eq - 1) out[slot++] = key;
        else if (eqr == need_eq - 1) *x_out = key;  // exactly one thread holds it
        ++eqr;
      }
    }
  }
  DSA_MARK(3, 10);
}

}  // namespace dsa

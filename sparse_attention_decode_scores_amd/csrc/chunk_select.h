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

// Histogram of a chunk's scores over monotone log-spaced bins: sign, exponent and
// 4 mantissa bits of the magnitude, so a bin spans at most 1/16 of its values
// (scores of magnitude below 16 get a bin each). 896 of the 1024 bins are used.
constexpr int kHistBins = 1024;
constexpr int kHistGroups = kHistBins / 16;  // one per lane of a wave
static_assert(kHistGroups == 64, "hist_threshold: one group per lane");
__device__ __forceinline__ uint32_t score_bin(int32_t s) {
  // x = |s| for s >= 0, ~s = -s - 1 for s < 0. For x >= 16 with top bit e (4 .. 30)
  // the code is 16(e - 3) + the four bits below it, which is 16·sh + (x >> sh) with
  // sh = e - 4; below 16, sh clamps to 0 and the code is x. Negative scores mirror.
  const uint32_t neg = (uint32_t)(s >> 31);  // all ones for s < 0
  const uint32_t x = (uint32_t)s ^ neg;
  const uint32_t lz = (uint32_t)__builtin_clz(x | 1u);
  const uint32_t sh = lz < 27u ? 27u - lz : 0u;
  const uint32_t code = (sh << 4) + (x >> sh);  // 0 .. 447
  return 448u + (code ^ neg);                   // s < 0: 447 - code
}

// Lowest score that score_bin maps to bin b (b < 896).
__device__ __forceinline__ int32_t bin_floor(uint32_t b) {
  if (b >= 448u) {
    const uint32_t code = b - 448u;
    if (code < 16u) return (int32_t)code;
    const uint32_t e = code / 16u + 3u;
    return (int32_t)((16u + code % 16u) << (e - 4u));
  }
  const uint32_t code = 447u - b;  // magnitudes x of this bin end at xh; the score is ~x
  uint32_t xh = code;
  if (code >= 16u) {
    const uint32_t e = code / 16u + 3u;
    xh = ((16u + code % 16u + 1u) << (e - 4u)) - 1u;
  }
  return (int32_t)~xh;
}

constexpr int kWaveStage = 136;  // staging slots per wave for wave_chunk_candidates (m <= 64, + 8 read slack)

// scores: LDS copy of the chunk's scores, entry i for position
// pos0 + (i / 32)·ustride + i % 32 (ustride = 32: consecutive positions); count:
// valid entries (<= 0 means none; at most 16 * BLOCK). Writes entries 0..m-1 of
// `out` (the m best keys, in position order, 0-padded) and *x_out = the best key not kept
// (0 if every valid position is kept).
//
// The (m+1)-th best score T comes from a radix selection over the scores; the
// kept keys are those scoring above T plus the first (m - #above) positions
// scoring exactly T, which is the key order (score, then lower position).
template <int BLOCK>
__device__ __forceinline__ void chunk_candidates(const int32_t* scores, int count, uint32_t pos0, int m,
                                 CandOut out, uint64_t* __restrict__ x_out,
                                 ChunkSmem<BLOCK>& sm, uint32_t ustride = 32) {
  const int tid = threadIdx.x;
  auto pos = [=](int i) { return pos0 + (uint32_t)(i >> 5) * ustride + (uint32_t)(i & 31); };
  if (count <= m) {
    for (int i = tid; i < m; i += BLOCK)
      out.put(i, i < count ? make_key(scores[i], pos(i)) : 0ull);
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
  const uint32_t T = block_select_range<BLOCK>(each, lo, hi, m + 1, &above, sm.radix);
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
#pragma unroll
  for (int j = 0; j < kChunkPerThread; ++j) {
    const int i = i0 + j;
    if (j < per && i < count) {
      const uint64_t key = ((uint64_t)u[j] << 32) | (uint64_t)(0xFFFFFFFFu - pos(i));
      if (u[j] > T) {
        out.put(slot++, key);
      } else if (u[j] == T) {
        if (eqr < need_eq - 1) out.put(slot++, key);
        else if (eqr == need_eq - 1) *x_out = key;  // exactly one thread holds it
        ++eqr;
      }
    }
  }
}

// Lowest score of the bin that holds the (m+1)-th best of `count` keys (m < count),
// from their histogram over score_bin, computed by one wave: lane l sums bins
// 1008-16l .. 1023-16l (best first) and one wave scan finds the bin. Returns
// false when the histogram does not count `count` keys.
__device__ __forceinline__ bool threshold_floor(const uint32_t* hist, int count, int m, int32_t* tlo) {
  const int l = lane_id();
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int bin0 = kHistBins - 16 - 16 * l;
  uint32_t h[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(hist + bin0 + 4 * q);
    h[4 * q] = v.x;
    h[4 * q + 1] = v.y;
    h[4 * q + 2] = v.z;
    h[4 * q + 3] = v.w;
  }
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) sum += h[j];
  const uint32_t incl = wave_incl_scan_u32(sum);
  if ((uint32_t)__builtin_amdgcn_readlane((int)incl, 63) != (uint32_t)count) return false;
  const uint32_t want = (uint32_t)m + 1;
  // the lane whose 16 bins hold the want-th best key, then within them one row scan:
  // lane j < 16 (and its copies in the other rows) takes bin bin0(L) + 15 - j
  const uint32_t excl = incl - sum;  // keys in better bins than this lane's
  const uint64_t hit = __ballot(excl < want && want <= incl);  // exactly one lane
  const int L = (int)__builtin_ctzll(hit);
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)excl, L);
  const int bj = kHistBins - 1 - 16 * L - (l & 15);
  uint32_t c = hist[bj];
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr1, 0xF, 0xF, false);
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr2, 0xF, 0xF, false);
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr4, 0xF, 0xF, false);
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr8, 0xF, 0xF, false);
  const uint64_t hit2 = __ballot(base + c >= want) & 0xFFFFull;  // first row
  *tlo = bin_floor((uint32_t)(kHistBins - 1 - 16 * L - (int)__builtin_ctzll(hit2)));
  return true;
}

// Lowest score of the bin that holds the want-th best of `count` keys, from their
// histogram over score_bin and its sums over groups of 16 bins (groups[g] = bins
// 16g .. 16g + 15, kept alongside so that this reads one word per lane without bank
// conflicts), by one wave in two levels: lane l takes group 63 - l (best first) and
// a wave scan finds the lane whose group holds it; then 16 lanes read that group's
// bins and a row scan finds the bin. Returns false when the histogram does not
// count `count` keys.
__device__ __forceinline__ bool hist_threshold(const uint32_t* hist, const uint32_t* groups, int count,
                                               uint32_t want, int32_t* tlo) {
  const int l = lane_id();
  const uint32_t sum = groups[kHistGroups - 1 - l];  // bins 1008 - 16l .. 1023 - 16l
  const uint32_t incl = wave_incl_scan_u32(sum);
  if ((uint32_t)__builtin_amdgcn_readlane((int)incl, 63) != (uint32_t)count) return false;
  const uint32_t excl = incl - sum;  // keys in better groups than this lane's
  const uint64_t hit = __ballot(excl < want && want <= incl);  // exactly one lane
  const int L = (int)__builtin_ctzll(hit);
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)excl, L);
  // lane j < 16 (and its copies in the other rows) takes bin 1023 - 16L - j
  const int bj = kHistBins - 1 - 16 * L - (l & 15);
  uint32_t c = hist[bj];
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr1, 0xF, 0xF, false);
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr2, 0xF, 0xF, false);
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr4, 0xF, 0xF, false);
  c += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)c, dpp::kRowShr8, 0xF, 0xF, false);
  const uint64_t hit2 = __ballot(base + c >= want) & 0xFFFFull;  // first row
  const int jstar = (int)__builtin_ctzll(hit2);
  *tlo = bin_floor((uint32_t)(kHistBins - 1 - 16 * L - jstar));
  return true;
}

// The same result as chunk_candidates, computed by one wave without block
// barriers, from a histogram of the chunk's scores over score_bin that the caller
// filled while producing them (hist counts the `count` valid positions):
//  1. threshold_floor finds the bin holding the (m+1)-th best key;
//  2. every key scoring at least that bin's lowest score is staged in LDS in
//     position order (ballot compaction): the keys of higher bins (fewer than m+1)
//     plus that bin's keys;
//  3. each staged key is ranked against the others; the m best go to the output
//     slot of their rank (best first) and the one of rank m is x, the best key
//     left out.
// The chunk's valid scores also go to dst[0, count) as they are read (when the
// threshold step fails they are not read, and the caller stores them).
// Returns false, having written no candidate, when more than m + 64 keys are staged
// (heavy ties) or the histogram does not count `count` keys: the caller then runs
// chunk_candidates. `stage` is this wave's LDS area of kWaveStage keys.
__device__ __forceinline__ bool wave_chunk_candidates(const int32_t* scores, int count, uint32_t pos0,
                                                      int m, const uint32_t* hist,
                                                      CandOut out,
                                                      uint64_t* __restrict__ x_out, uint64_t* stage,
                                                      int32_t* __restrict__ dst) {
  const int l = lane_id();
  if (count <= m) {
    for (int i = l; i < m; i += 64) {
      const int32_t v = scores[i < count ? i : 0];
      if (i < count) dst[i] = v;
      out.put(i, i < count ? make_key(v, pos0 + (uint32_t)i) : 0ull);
    }
    if (l == 0) *x_out = 0;
    return true;
  }
  int32_t tlo;
  if (!threshold_floor(hist, count, m, &tlo)) return false;

  const uint64_t lt = lanemask_lt();
  const uint32_t cap = (uint32_t)m + 64;
  uint32_t ns = 0;
  // rows of 64 positions, eight rows' loads in flight at a time
  for (int r0 = 0; r0 < count; r0 += 8 * 64) {
    int32_t v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = r0 + 64 * t + l;
      v[t] = scores[i < count ? i : count - 1];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = r0 + 64 * t + l;
      if (i < count) dst[i] = v[t];
      const bool in = i < count && v[t] >= tlo;
      const uint64_t b = __ballot(in);
      const uint32_t slot = ns + (uint32_t)__popcll(b & lt);
      if (in && slot < cap) stage[slot] = make_key(v[t], pos0 + (uint32_t)i);
      ns += (uint32_t)__popcll(b);
    }
  }
  if (ns > cap) return false;

  const bool two = ns > 64;
  if (!two) {  // uniform: one key per lane; slots up to a multiple of 8 hold key 0,
    // which is below every staged key (key 0 would be position 2^32 - 1), so no
    // step checks the count
    const uint32_t ns8 = (ns + 7u) & ~7u;
    if ((uint32_t)l >= ns && (uint32_t)l < ns8) stage[l] = 0ull;
  }
  const uint64_t k0 = l < (int)ns ? stage[l] : 0ull;
  const uint64_t k1 = l + 64 < (int)ns ? stage[l + 64] : 0ull;
  uint32_t r0 = 0, r1 = 0;
  // every lane compares its keys with all staged keys: 8 keys per step, read as
  // four 16-byte broadcasts (the staging area has kWaveStage >= cap + 8 slots)
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  if (!two) {  // uniform
    for (int j0 = 0; j0 < (int)ns; j0 += 8) {
      u64x2 e[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) e[t] = *reinterpret_cast<const u64x2*>(stage + j0 + 2 * t);
#pragma unroll
      for (int t = 0; t < 8; ++t) r0 += ((t & 1) ? e[t >> 1].y : e[t >> 1].x) > k0 ? 1u : 0u;
    }
  } else
  for (int j0 = 0; j0 < (int)ns; j0 += 8) {
    u64x2 e[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) e[t] = *reinterpret_cast<const u64x2*>(stage + j0 + 2 * t);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint64_t x = (t & 1) ? e[t >> 1].y : e[t >> 1].x;
      const bool live = j0 + t < (int)ns;
      r0 += (live && x > k0) ? 1u : 0u;
      if (two) r1 += (live && x > k1) ? 1u : 0u;
    }
  }
  // staged keys are distinct, so the ranks are a permutation of 0 .. ns-1
  const bool s0 = l < (int)ns && r0 < (uint32_t)m;
  const bool s1 = l + 64 < (int)ns && r1 < (uint32_t)m;
  if (s0) out.put((int)r0, k0);  // slot = rank: the list is best first
  if (s1) out.put((int)r1, k1);
  const uint64_t xb0 = __ballot(l < (int)ns && r0 == (uint32_t)m);
  const uint64_t xb1 = __ballot(l + 64 < (int)ns && r1 == (uint32_t)m);
  const int xl = xb0 ? __builtin_ctzll(xb0) : __builtin_ctzll(xb1);
  const uint64_t xk = xb0 ? k0 : k1;
  const uint32_t xlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)xk, xl);
  const uint32_t xhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(xk >> 32), xl);
  if (l == 0) *x_out = ((uint64_t)xhi << 32) | xlo;
  return true;
}

// LDS of block_chunk_candidates.
template <int BLOCK>
struct BlockCandSmem {
  uint64_t wstage[BLOCK / 64][kWaveStage];  // each wave's staged keys
  uint64_t all[kWaveStage];                 // all staged keys, position order
  uint32_t rank[kWaveStage];
  uint32_t wcount[BLOCK / 64];
  int32_t tlo;
  uint32_t ok;
};

// The same result as chunk_candidates for one chunk, by the first four waves of
// the block (one per SIMD, so none shares its issue slots); the other waves only
// pass the barriers. Four barriers (the caller's barrier after filling `scores`
// and `hist` comes first): wave 0 finds the threshold bin's lowest score
// (threshold_floor); active wave w stages the keys at or above it from its own
// run of 64-position rows (ballot compaction, position order); the runs are
// concatenated; two or four threads per staged key count the staged keys above
// it, which is its rank; wave 0 writes the m best to the slot of their rank (best
// first) and x = the key of rank m. Returns false (uniformly, nothing written) where
// wave_chunk_candidates does.
template <int BLOCK>
__device__ __forceinline__ bool block_chunk_candidates(const int32_t* scores, int count, uint32_t pos0,
                                                       int m, const uint32_t* hist,
                                                       CandOut out,
                                                       uint64_t* __restrict__ x_out,
                                                       BlockCandSmem<BLOCK>& sm) {
  constexpr int W = 4;            // active waves
  constexpr int AT = 64 * W;      // active threads
  static_assert(BLOCK >= AT, "four waves");
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const bool active = w < W;
  if (count <= m) {
    for (int i = tid; i < m; i += BLOCK) out.put(i, i < count ? make_key(scores[i], pos0 + (uint32_t)i) : 0ull);
    if (tid == 0) *x_out = 0;
    return true;
  }
  // wave 0 finds the threshold; the others wait at the barrier that publishes it
  if (w == 0) {
    int32_t t;
    const bool ok = threshold_floor(hist, count, m, &t);
    if (l == 0) {
      sm.tlo = t;
      sm.ok = ok ? 1u : 0u;
    }
  }
  lds_barrier();
  if (!sm.ok) return false;  // uniform
  const int32_t tlo = sm.tlo;

  const uint64_t lt = lanemask_lt();
  const uint32_t cap = (uint32_t)m + 64;
  uint32_t ns = 0;
  if (active) {
    const int nrows = (count + 63) >> 6;
    const int per = (nrows + W - 1) / W;
    const int rbeg = w * per, rend = rbeg + per < nrows ? rbeg + per : nrows;
    for (int r0 = rbeg; r0 < rend; r0 += 4) {
      int32_t v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = 64 * (r0 + t) + l;
        v[t] = scores[i < count ? i : count - 1];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = 64 * (r0 + t) + l;
        const bool in = r0 + t < rend && i < count && v[t] >= tlo;
        const uint64_t b = __ballot(in);
        const uint32_t slot = ns + (uint32_t)__popcll(b & lt);
        if (in && slot < cap) sm.wstage[w][slot] = make_key(v[t], pos0 + (uint32_t)i);
        ns += (uint32_t)__popcll(b);
      }
    }
    if (l == 0) sm.wcount[w] = ns;
  }
  lds_barrier();
  uint32_t total = 0, off = 0;
#pragma unroll
  for (int q = 0; q < W; ++q) {
    const uint32_t c = sm.wcount[q];
    off += q < w ? c : 0u;
    total += c;
  }
  if (total > cap) return false;  // uniform
  if (active)
    for (int j = l; j < (int)ns; j += 64) sm.all[off + j] = sm.wstage[w][j];
  lds_barrier();

  // rank of staged key i: tpe active threads each compare it with every tpe-th key
  const int tpe = total > (uint32_t)(AT / 4) ? 2 : 4;  // AT / tpe >= cap keys
  const int i = tid / tpe, part = tid % tpe;
  uint32_t r = 0;
  if (active && i < (int)total) {
    const uint64_t me = sm.all[i];
    for (int j = part; j < (int)total; j += tpe) r += sm.all[j] > me ? 1u : 0u;
  }
  r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor1, 0xF, 0xF, false);
  if (tpe == 4) r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor2, 0xF, 0xF, false);
  if (active && part == 0 && i < (int)total) sm.rank[i] = r;
  lds_barrier();

  if (w == 0) {
    for (int q = 0; q < (int)total; q += 64) {
      const int j = q + l;
      const uint32_t rk = j < (int)total ? sm.rank[j] : ~0u;
      if (rk < (uint32_t)m) out.put((int)rk, sm.all[j]);  // slot = rank: best first
      if (rk == (uint32_t)m) *x_out = sm.all[j];
    }
  }
  return true;
}

}  // namespace dsa

// Stage 2 (exact ordered top-k) and stage 3 (sparse attention), plus the
// combine pass of the attention splits.
//
// Selection follows the structure described in the ds4 glm53-m3ultra branch post
// (2026-09-09 "rising" page, long-context paragraph): parallel scans narrow the
// candidates, a small surviving list is ordered, and the original exhaustive
// algorithm handles the ambiguous cases; the same positions come out in the same
// order, and the same outputs, either way.
//  * Candidate path. The score pass left, for every chunk of positions, its m
//    best keys and the best key it dropped (x_c). Every workgroup of this kernel
//    loads that candidate union U (at most 8192 keys, 16 per thread in
//    registers) and narrows it by radix passes over the scores (and, when one
//    score value holds many keys, over the positions of those keys). The top k of
//    U are the top k of the row when every dropped key is below the k-th key of
//    U: then at least k keys of U lie above the best dropped key.
//  * Exhaustive path ("ambiguous" case: some chunk holds more than m keys at or
//    above the k-th key, which happens when many positions tie at the threshold;
//    rows too long for the candidate pass; or the flag forces it): a radix
//    selection over every position of the row gives the same top-k set.
// Two roles share the launch, so no second kernel boundary is spent:
//  * ranking workgroups order the selected keys: each takes a slice and counts,
//    for each of its keys, how many selected keys are larger; that count is the
//    output slot (keys are distinct, so the slots are a permutation);
//  * attention workgroup s takes the selected positions whose output slot lies in
//    [s·per, (s+1)·per) (per = ceil(k / splits)), in output order, and writes one
//    split of the attention. The slots are found by radix narrowing to the two
//    window ends, so this needs no ordering of the whole selection, and the
//    grouping depends on nothing but the output order: both paths, and the
//    stand-alone attention over the ordered indices, sum the same rows in the
//    same groups and order, and their outputs are equal bit for bit.
#include <type_traits>

#include "attn_body.h"
#include "chunk_select.h"
#include "kernels.h"

namespace dsa {

// ------------------------------------------------------------------ candidates over stored scores

constexpr int kSelBlock = kAttnBlock;  // selection, ranking and attention share the launch
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));  // a chunk summary without its padding
constexpr int kSelWaves = kSelBlock / 64;
constexpr int kUPerThread = kCandCap / kSelBlock;  // candidate keys held per thread
constexpr int kSelPerThread = 4096 / kSelBlock;   // selected keys per thread (k <= 4096)
// Ranking workgroups that take part on the exhaustive path (each streams the row).
constexpr int kFallbackRankers = 64;

__global__ __launch_bounds__(kSelBlock) void k_chunk_cand(CandArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  using Smem = ChunkSmem<kSelBlock>;
  Smem& csm = *reinterpret_cast<Smem*>(smem);
  int32_t* sc = reinterpret_cast<int32_t*>(smem + align16(sizeof(Smem)));
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t cbeg = (int64_t)c * a.P;
  const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
  const int count = n64 > a.P ? a.P : (int)(n64 > 0 ? n64 : 0);
  const int32_t* row = a.scores + (int64_t)b * a.N + cbeg;
  radix_clear<kSelBlock>(csm.radix);
  for (int i = threadIdx.x; i < count; i += kSelBlock) sc[i] = row[i];
  lds_barrier();
  chunk_candidates<kSelBlock>(sc, count, (uint32_t)cbeg, a.m, CandOut{a.cand + (int64_t)b * kCandCap, c * a.m},
                              a.xc + (int64_t)b * a.G + c, csm);
}

hipError_t launch_chunk_candidates(const CandArgs& a, int B, hipStream_t s) {
  const size_t lds = align16(sizeof(ChunkSmem<kSelBlock>)) + (size_t)a.P * 4;
  hipError_t e = allow_lds((const void*)k_chunk_cand, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_chunk_cand, dim3(a.G, B), dim3(kSelBlock), lds, s, a);
  return hipGetLastError();
}

int chunk_cand_max_chunk() { return kChunkPerThread * kSelBlock; }

// ------------------------------------------------------------------ selection (+ attention)

// Once the radix bin that holds a sought key has at most this many keys, they are
// ranked among themselves instead of narrowed further.
constexpr uint32_t kMaxBinRank = 256;
constexpr int kBinPad = 16;       // LDS slots before the bin's keys (split_sorted's base may point there)
constexpr int kMaxWindow = kMaxSplitRows;  // selected positions per attention split
// keys gathered around an attention window: the bins of its two ends and the keys between
constexpr int kMaxWindowList = 2 * (int)kMaxBinRank + kMaxWindow;
// Exhaustive path: positions sampled for a threshold, and the keys at or above it that
// the LDS list may hold (kept in the region the attention working set reuses).
constexpr int kSampleMax = 16384;  // 32 per thread
constexpr int kCandList = 8192;
constexpr int kWaveCand = kCandList / kSelWaves;  // one segment per wave
// Keys a segment may take: an append starts at the wave's count capped here, and
// one append adds at most 64, so every store stays inside the segment; a wave that
// keeps more makes the list unusable, which the final count detects.
constexpr int kWaveCap = kWaveCand - 64;

struct SelSmem {
  RadixSmem radix;
  uint32_t xch[kSelWaves][5];
  uint64_t mxw[kSelWaves];          // per wave: the best key a chunk left out; on the exhaustive path,
                                    // [0, 4): chunks whose best dropped key reaches T0
  uint32_t wcnt[kSelWaves][2];      // exhaustive compaction: per-wave counts above / at the threshold
  uint32_t gtw[kSelWaves];          // attention: per-wave counts of keys above the best dropped key
  uint64_t kstar;
  uint32_t tied;
  uint32_t winpos[kMaxWindow];      // attention: the window's positions, in output order
};
static_assert(kUPerThread == 16 && kSelBlock == 512, "cand_slot layout: 512 threads x 16 entries");
static_assert(kBinPad >= kUPerThread, "split_sorted: up <= keys per thread");

// LDS the selection needs in the region that the attention working set reuses
// afterwards: a list of bin or window keys (kBinPad before it) and the sink slots,
// or, on the exhaustive path, first the list of keys at or above the sampled
// threshold (kCandList keys from the region's start).
constexpr size_t kRegionSelect =
    (size_t)(kBinPad + kMaxWindowList + kSelBlock + kUPerThread) * 8 > (size_t)kCandList * 8
        ? (size_t)(kBinPad + kMaxWindowList + kSelBlock + kUPerThread) * 8
        : (size_t)kCandList * 8;

// Exchanges (sum, min, max, max64) over the block in one round.
struct Stats4 {
  uint32_t sum, lo, hi;
  uint64_t mx;
};
__device__ __forceinline__ Stats4 block_stats(uint32_t sum, uint32_t lo, uint32_t hi, uint64_t mx,
                                              SelSmem& sm) {
  const uint64_t wmx = wave_maxr_u64(mx);
  const uint32_t mine[5] = {wave_sum_u32(sum), ~wave_min_u32(lo), wave_maxr_u32(hi),
                            (uint32_t)(wmx >> 32), (uint32_t)wmx};
  uint32_t all[kSelWaves][5];
  block_exchange<kSelBlock, 5>(mine, sm.xch, all);
  Stats4 r{0, 0, 0, 0};
  uint32_t nlo = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    r.sum += all[w][0];
    nlo = all[w][1] > nlo ? all[w][1] : nlo;
    r.hi = all[w][2] > r.hi ? all[w][2] : r.hi;
    const uint64_t m = ((uint64_t)all[w][3] << 32) | all[w][4];
    r.mx = m > r.mx ? m : r.mx;
  }
  r.lo = ~nlo;
  return r;
}

// Calls f(score_bits) for every score of row[0, n), 16 loads per thread in flight
// (coalesced: load j of the block covers 512 consecutive scores).
template <class Row, class F>
__device__ __forceinline__ void for_each_score(Row row, int n, F f) {
  constexpr int U = 16;
  const int64_t tid = threadIdx.x;
  for (int64_t i0 = 0; i0 < n; i0 += (int64_t)kSelBlock * U) {
    int32_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t i = i0 + tid + (int64_t)kSelBlock * j;
      v[j] = row[i < n ? i : n - 1];
    }
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (i0 + tid + (int64_t)kSelBlock * j < n) f(score_bits(v[j]));
  }
}

// The same over positions [p0, p1) for one wave: f(score_bits, position, present)
// is called for every lane of every 64-position row, in position order (one call
// per row per lane, so that callers can use wave-wide ballots).
template <class Row, class F>
__device__ __forceinline__ void wave_rows(Row row, int64_t p0, int64_t p1, F f) {
  constexpr int U = 16;
  const int lane = lane_id();
  for (int64_t q0 = p0; q0 < p1; q0 += 64 * U) {
    int32_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t p = q0 + 64 * j + lane;
      v[j] = row[p < p1 ? p : p1 - 1];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t p = q0 + 64 * j + lane;
      f(score_bits(v[j]), p, p < p1);
    }
  }
}

// Splits the candidates held E per thread around the key range [klo, khi]: keys
// above it go to sel, keys in it to bin, both in union order. Every key is
// written, the others to this thread's slot of sink (one computed address per key
// and no branch: per-key branches cost more than the stores). One barrier.
template <int E>
__device__ __forceinline__ void split_at_bin(const uint64_t (&key)[E], uint32_t vmask, uint64_t klo,
                                             uint64_t khi, uint64_t* sel, uint64_t* bin, uint64_t* sink,
                                             SelSmem& sm) {
  uint32_t up = 0, in = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const bool v = (vmask >> j) & 1u;
    up += v && key[j] > khi ? 1u : 0u;
    in += v && key[j] >= klo && key[j] <= khi ? 1u : 0u;
  }
  uint32_t total;
  // the caller's last barrier separates every earlier reader of the scan slots
  const uint32_t before = block_excl_scan_fresh_u32<kSelBlock>(up | (in << 16), sm.radix.part, &total);
  uint32_t su = before & 0xFFFF, si = before >> 16;
  uint64_t* const mine = sink + threadIdx.x;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const bool v = (vmask >> j) & 1u;
    const bool a = v && key[j] > khi;
    const bool b = v && key[j] >= klo && !a;
    *(a ? sel + su : (b ? bin + si : mine)) = key[j];
    su += a ? 1u : 0u;
    si += b ? 1u : 0u;
  }
}

// split_at_bin for keys that run best first in every thread (absent keys, 0,
// last): the keys above the range are a prefix of each thread's keys and the
// range's keys follow, so key j goes to a base chosen by two counts, plus j (one
// computed address per key, no per-key counters). bin must have kBinPad slots
// before it, and sink kSelBlock + E.
template <int E>
__device__ __forceinline__ void split_sorted(const uint64_t (&key)[E], uint64_t klo, uint64_t khi,
                                             uint64_t* sel, uint64_t* bin, uint64_t* sink, SelSmem& sm) {
  const uint64_t klo1 = klo > 0 ? klo : 1;  // a present key is never 0
  uint32_t up = 0, ge = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    up += key[j] > khi ? 1u : 0u;
    ge += key[j] >= klo1 ? 1u : 0u;
  }
  uint32_t total;
  // the caller's last barrier separates every earlier reader of the scan slots
  const uint32_t before = block_excl_scan_fresh_u32<kSelBlock>(up | ((ge - up) << 16), sm.radix.part, &total);
  const uint32_t su = before & 0xFFFF, si = before >> 16;
  uint64_t* const a = sel + su;              // key j < up goes to a[j]
  uint64_t* const b = bin + si - up;         // key up <= j < ge goes to b[j] (up <= E <= kBinPad)
  uint64_t* const c = sink + threadIdx.x;    // the others to c[j]
#pragma unroll
  for (int j = 0; j < E; ++j) ((uint32_t)j < up ? a : ((uint32_t)j < ge ? b : c))[j] = key[j];
}

// Ranks the n keys of bin among themselves (rank = number of larger keys; keys
// are distinct, so the ranks are a permutation) and writes the need best to
// out[rank], best first; the one of rank need - 1 (the k-th best overall) goes to
// sm.kstar and the number of taken keys with its score to sm.tied. Eight threads
// per key.
__device__ __forceinline__ void rank_bin(const uint64_t* bin, uint32_t n, uint32_t need, uint64_t* out,
                                         SelSmem& sm) {
  const int g = threadIdx.x >> 3, part = threadIdx.x & 7;
  for (uint32_t base = 0; base < n; base += kSelBlock / 8) {
    const uint32_t i = base + (uint32_t)g;
    const uint64_t me = i < n ? bin[i] : ~0ull;
    uint32_t r = 0, te = 0;
    for (uint32_t j = (uint32_t)part; j < n; j += 8) {
      const uint64_t v = bin[j];
      const bool gtr = v > me;
      r += gtr ? 1u : 0u;
      te += gtr && (uint32_t)(v >> 32) == (uint32_t)(me >> 32) ? 1u : 0u;
    }
    // sums over the eight threads of this key
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor1, 0xF, 0xF, false);
    te += (uint32_t)__builtin_amdgcn_mov_dpp((int)te, dpp::kQuadXor1, 0xF, 0xF, false);
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor2, 0xF, 0xF, false);
    te += (uint32_t)__builtin_amdgcn_mov_dpp((int)te, dpp::kQuadXor2, 0xF, 0xF, false);
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kRowHalfMirror, 0xF, 0xF, false);
    te += (uint32_t)__builtin_amdgcn_mov_dpp((int)te, dpp::kRowHalfMirror, 0xF, 0xF, false);
    if (part == 0 && i < n && r < need) {
      out[r] = me;
      if (r == need - 1) {
        sm.kstar = me;
        sm.tied = te + 1;
      }
    }
  }
}

// The union's score range [rng[0], rng[1]] and whether every thread's keys run best
// first, from the chunk summaries (four per lane, all chunks in every wave: no
// exchange between waves).
__device__ __forceinline__ void union_range_from_sums(const u32x3 (&csum)[4], uint32_t* rng, bool* sorted) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0, unordered = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo = csum[i].x < lo ? csum[i].x : lo;
    hi = csum[i].y > hi ? csum[i].y : hi;
    unordered |= csum[i].z == 0u ? 1u : 0u;
  }
  rng[0] = wave_min_u32(lo);
  rng[1] = wave_maxr_u32(hi);
  *sorted = __ballot(unordered != 0u) == 0;
}

// The same from the keys themselves (when no summaries exist), by one block
// exchange, which also publishes the cleared radix histograms and anything the
// caller wrote to LDS before it. A thread's keys run best first when each is at
// least the next (absent keys, 0, come last).
template <int E>
__device__ __forceinline__ void union_range_exchange(const uint64_t (&key)[E], const uint32_t (&sv)[E],
                                                     uint32_t vmask, SelSmem& sm, uint32_t* rng, bool* sorted) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const bool v = (vmask >> j) & 1u;
    lo = v && sv[j] < lo ? sv[j] : lo;
    hi = v && sv[j] > hi ? sv[j] : hi;
  }
  bool desc = true;
#pragma unroll
  for (int j = 0; j + 1 < E; ++j) desc = desc && key[j] >= key[j + 1];
  const uint32_t mine[3] = {~wave_min_u32(lo), wave_maxr_u32(hi), __ballot(!desc) != 0 ? 1u : 0u};
  uint32_t all[kSelWaves][3];
  block_exchange<kSelBlock, 3>(mine, reinterpret_cast<uint32_t(*)[3]>(&sm.xch[0][0]), all);
  uint32_t nlo = 0, mhi = 0, unsorted = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    nlo = all[w][0] > nlo ? all[w][0] : nlo;
    mhi = all[w][1] > mhi ? all[w][1] : mhi;
    unsorted |= all[w][2];
  }
  rng[0] = ~nlo;
  rng[1] = mhi;
  *sorted = unsorted == 0;
}

// A range of 64-bit keys that holds a sought key: `above` keys lie above khi and
// `inbin` keys in [klo, khi].
struct KeyRange {
  uint64_t klo, khi;
  uint32_t above, inbin;
  uint32_t gt;  // keys of a higher score than every key of the range (= above unless tie)
  bool tie;     // the range is a run of positions within one score value
};

// The kk best of the nvalid valid keys held E per thread (score bits sv in [lo, hi];
// `sorted` when every thread's keys run best first): written to sel[0, kk) (the keys
// above the kk-th key's radix range in input order, then the range's best in key
// order); returns the kk-th best key and the number of selected keys with its score.
// With publish_mx, the waves' largest dropped key (mx, one per thread) goes to
// sm.mxw behind the narrowing, published by the last barrier. Every thread gets the
// same results.
struct TopK {
  uint64_t kstar;
  uint32_t tied;
};
template <int E>
__device__ __forceinline__ TopK topk_of_keys(const uint64_t (&key)[E], const uint32_t (&sv)[E], uint32_t vmask,
                                             uint32_t nvalid, uint32_t kk, uint32_t lo, uint32_t hi, bool sorted,
                                             uint64_t* sel, uint64_t* list, uint64_t* sink, SelSmem& sm,
                                             bool publish_mx, uint64_t mx) {
  auto each = [&](auto f) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((vmask >> j) & 1u) f(sv[j]);
  };
  // radix passes until the bin of the kk-th best key is small
  const RadixBin rb = block_narrow<kSelBlock>(each, lo, hi, kk, nvalid, kMaxBinRank, sm.radix);
  const uint64_t wmx = publish_mx ? wave_maxr_u64(mx) : 0ull;
  // the key range that holds the kk-th best key: the keys above it are taken
  uint64_t klo = (uint64_t)rb.binlo << 32, khi = ((uint64_t)rb.binhi << 32) | 0xFFFFFFFFull;
  uint32_t above = rb.above, inbin = rb.inbin, tie_above = 0;
  if (rb.inbin > kMaxBinRank) {  // uniform: one score value T holds that many keys
    // the same narrowing over the low key words of the keys at T (a larger low word
    // is an earlier position)
    const uint32_t T = rb.binlo;
    auto each_tie = [&](auto f) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (((vmask >> j) & 1u) && sv[j] == T) f((uint32_t)key[j]);
    };
    const RadixBin rt = block_narrow<kSelBlock>(each_tie, 0u, 0xFFFFFFFFu, kk - rb.above, rb.inbin, kMaxBinRank,
                                                sm.radix);
    klo = ((uint64_t)T << 32) | rt.binlo;
    khi = ((uint64_t)T << 32) | rt.binhi;
    above += rt.above;
    inbin = rt.inbin;
    tie_above = rt.above;
  }
  // the keys above the range are taken in input order, then the range's best in key
  // order (equal scores: ascending positions)
  if (sorted)  // uniform
    split_sorted<E>(key, klo, khi, sel, list, sink, sm);
  else
    split_at_bin<E>(key, vmask, klo, khi, sel, list, sink, sm);
  if (publish_mx && lane_id() == 0) sm.mxw[wave_id()] = wmx;
  lds_barrier();
  rank_bin(list, inbin, kk - above, sel + above, sm);
  lds_barrier();
  return TopK{sm.kstar, tie_above + sm.tied};
}

// The selection kernel's LDS: SelSmem | selected keys [k] | region, the attention
// working set, which reuses what the selection keeps there (a list of bin or
// window keys, then sink slots; or first the exhaustive path's key list). Taken
// from the dynamic LDS symbol itself, also in the called functions below: pointers
// passed to a called function are generic, and accesses through them take the
// flat path.
struct SelLds {
  SelSmem* sm;
  uint64_t* sel;
  uint8_t* region;
  uint64_t* list;  // bin or window keys
  uint64_t* sink;
};
__device__ __forceinline__ SelLds sel_lds(int k) {
  extern __shared__ __align__(16) uint8_t smem[];
  SelLds l;
  l.sm = reinterpret_cast<SelSmem*>(smem);
  l.sel = reinterpret_cast<uint64_t*>(smem + align16(sizeof(SelSmem)));
  l.region = smem + align16(sizeof(SelSmem)) + align16((size_t)k * 8);
  l.list = reinterpret_cast<uint64_t*>(l.region) + kBinPad;
  l.sink = l.list + kMaxWindowList;
  return l;
}

// The exhaustive path's narrowing (the "scans that narrow before a small sort"):
//  1. a threshold T0 at or below the kk-th best score. With the candidate union at
//     hand (cand_row, entries [0, G m), at least kk valid), a value at or below the
//     union's kk-th best score: the union's keys are row keys, so the row's kk-th
//     best is at least that. Otherwise the rs-th best of up to kSampleMax sampled
//     positions, rs chosen so that about 1.25 kk + 32 of the row's positions are
//     expected at or above it;
//  2. every key of the row scoring at least T0 into an LDS list (the region's first
//     kCandList keys, one segment per wave; no atomics). With the union, a chunk
//     whose best dropped key (xc_row) scores below T0 has no key at or above T0
//     outside the union: the list takes the union's keys at or above T0 from those
//     chunks and rescans only the others, at most kMaxHotChunks of them. Otherwise
//     one streamed pass over the whole row;
//  3. when at least kk keys reached the list and all fitted, the list holds the top
//     kk (the kk-th best scores at least T0). Returns that, with the list's keys in
//     key/sv/vmask (thread (w, lane) holds slots [16 lane, 16 lane + 16) of wave w's
//     segment), their count in *total and their score range in rng. The order of
//     the list depends on the row alone (not on timing): the ranking workgroups each
//     build it and split the selected keys by their place in it.
// Otherwise (a sample far from the row's distribution, more than the list holds at
// or above T0, or one wave's share beyond its segment) the caller falls back to
// select_row_radix.
constexpr int kMaxHotChunks = 32;
// The candidate pass's chunks (row_chunk_units): G chunks of P positions keeping m
// candidates each; ilv: interleaved 32-position units. (The selection kernel gets
// P in SelArgs::have_cand and ilv as the presence of the one-row pass's chunk
// summaries: no argument of their own, which would move or add argument reads
// on the candidate path.)
struct ChunkGeom {
  int G, m, P, ilv;
};

// The selection kernel's arguments as they lie in its argument segment: its
// parameter list in order, each at its natural alignment. The out-of-line
// exhaustive path reads what it needs from there (scalar loads where it starts)
// instead of taking more arguments: values passed to it would stay live through
// the candidate path's code and push its scalar registers into spills.
struct SelectKernArgs {
  const uint64_t* cand;
  const uint64_t* xc;
  const ChunkSum* sums;
  const void* q;
  int G, Hq, Dk, S;
  SelArgs a;
  AttnArgs at;
};
static_assert(offsetof(SelectKernArgs, a) == 48 && offsetof(SelectKernArgs, at) == 48 + sizeof(SelArgs),
              "the selection kernel's argument layout");
typedef const __attribute__((address_space(4))) SelectKernArgs* KernArgPtr;

// One row's inputs to the exhaustive path, from the kernel arguments.
struct ExhRow {
  GlobalI32 row;
  const int32_t* row_in;
  int n, kk, k;
  const uint64_t* cand_row;  // the candidate union, or nullptr when the pass did not run
  const uint64_t* xc_row;    // each chunk's best dropped key
  ChunkGeom cg;
};
__device__ __forceinline__ ExhRow exh_row(const SelectKernArgs* ka_in, int b) {
  const KernArgPtr ka = (KernArgPtr) reinterpret_cast<const SelectKernArgs*>(
      uniform_u64(reinterpret_cast<uint64_t>(ka_in)));
  b = __builtin_amdgcn_readfirstlane(b);
  ExhRow r;
  r.row_in = ka->a.scores + (int64_t)b * ka->a.N;
  r.row = global_view(r.row_in);
  r.n = ka->a.lens.n[b];
  r.k = ka->a.k;
  r.kk = r.k < r.n ? r.k : r.n;
  const int P = ka->a.have_cand;  // the candidate pass's chunk length, or 0
  r.cand_row = P > 0 ? ka->cand + (int64_t)b * kCandCap : nullptr;
  r.xc_row = ka->xc + (int64_t)b * ka->G;
  // the one-row pass (interleaved chunks) is the one that leaves chunk summaries
  r.cg = ChunkGeom{ka->G, ka->a.m, P, ka->sums != nullptr ? 1 : 0};
  return r;
}
__device__ __forceinline__ bool exhaustive_list(GlobalI32 row, const int32_t* row_in, int n, int kk,
                                                const uint64_t* cand_row, const uint64_t* xc_row, int G, int cm,
                                                int P, int ilv, const SelLds& l, uint64_t (&key)[kUPerThread],
                                                uint32_t (&sv)[kUPerThread], uint32_t& vmask, uint32_t* total_out,
                                                uint32_t (&rng)[2]) {
  SelSmem& sm = *l.sm;
  const int tid = threadIdx.x;
  const int w = wave_id(), lane = lane_id();
  const uint64_t lt = lanemask_lt();
  // wave w's list segment; a kept key as stored: make_key without its sign flip
  // (undone when the list is read)
  uint64_t* const wseg = reinterpret_cast<uint64_t*>(l.region) + w * kWaveCand;
  uint32_t* const seg32 = reinterpret_cast<uint32_t*>(wseg);
  uint32_t wn = 0;  // keys this wave kept (uniform)
  // appends the keys of this wave's lanes for which keep holds (score x at
  // position pos): slot = the wave's count so far (capped) + the lane's rank among
  // the kept lanes; the key as two words
  auto append = [&](bool keep, int32_t x, uint32_t pos) {
    const uint64_t bal = __ballot(keep);
    if (keep) {
      const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      uint32_t* const slot = seg32 + 2 * ((wn < (uint32_t)kWaveCap ? wn : (uint32_t)kWaveCap) + r);
      slot[0] = 0xFFFFFFFFu - pos;
      slot[1] = (uint32_t)x;
    }
    wn += (uint32_t)__popcll(bal);
  };

  // 1. the threshold
  uint32_t t0bits = 0;
  bool from_union = false;
  uint64_t u[kUPerThread];  // the union as the selection kernel holds it
  uint32_t uvalid = 0;
  if (cand_row != nullptr) {  // uniform
    // thread t's entries [16t, 16t + 16), eight 16-byte pieces, piece j of all
    // threads contiguous
    typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
    typedef const __attribute__((address_space(1))) u64x2* GlobalU64x2;
    const GlobalU64x2 src = (GlobalU64x2)cand_row + tid;
#pragma unroll
    for (int j = 0; j < kUPerThread / 2; ++j) {
      const u64x2 v = src[(kCandCap / 16) * j];
      u[2 * j] = v.x;
      u[2 * j + 1] = v.y;
    }
    uint32_t cnt = 0, lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int j = 0; j < kUPerThread; ++j) {
      const bool v = kUPerThread * tid + j < G * cm && u[j] != 0ull;  // 0: no position
      uvalid |= v ? 1u << j : 0u;
      cnt += v ? 1u : 0u;
      lo = v && key_ubits(u[j]) < lo ? key_ubits(u[j]) : lo;
      hi = v && key_ubits(u[j]) > hi ? key_ubits(u[j]) : hi;
    }
    const Stats4 st = block_stats(cnt, lo, hi, 0, sm);
    if (st.sum >= (uint32_t)kk) {  // uniform
      auto each_u = [&](auto f) {
#pragma unroll
        for (int j = 0; j < kUPerThread; ++j)
          if ((uvalid >> j) & 1u) f(key_ubits(u[j]));
      };
      // the low end of a radix bin of at most 64 union scores that holds the kk-th
      // (one pass, mostly, instead of narrowing to the value itself)
      t0bits = block_narrow<kSelBlock>(each_u, st.lo, st.hi, (uint32_t)kk, st.sum, 64u, sm.radix).binlo;
      from_union = true;
    }
  }
  if (!from_union) {  // uniform
    // all positions of a short row, else 256 evenly spaced runs of 64 (one coalesced
    // load per wave and run)
    constexpr int SP = kSampleMax / kSelBlock;
    const bool whole = n <= kSampleMax;
    const int ns = whole ? n : kSampleMax;
    const uint64_t want = (uint64_t)kk * 5 / 4 + 32;
    const uint32_t rs0 = (uint32_t)((want * (uint64_t)ns + (uint64_t)n - 1) / (uint64_t)n);
    const uint32_t rs = rs0 < (uint32_t)ns ? (rs0 > 0 ? rs0 : 1u) : (uint32_t)ns;
    int32_t sx[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j) {
      const int i = tid + kSelBlock * j;
      // run w + 8 j starts at its share of the row; runs never overlap (n > 16384)
      const int64_t p = whole ? (i < n ? i : 0) : (int64_t)(w + kSelWaves * j) * n / (kSampleMax / 64) + lane;
      sx[j] = row[p];
    }
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
    for (int j = 0; j < SP; ++j)
      if (!whole || tid + kSelBlock * j < n) {
        const uint32_t v = score_bits(sx[j]);
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
      }
    const Stats4 st = block_stats(0, lo, hi, 0, sm);
    auto each_s = [&](auto f) {
#pragma unroll
      for (int j = 0; j < SP; ++j)
        if (!whole || tid + kSelBlock * j < n) f(score_bits(sx[j]));
    };
    // the low end of a radix bin of at most 16 sampled values that holds the rs-th
    // best (every sampled value of the bin passes, a few more than rs)
    t0bits = block_narrow<kSelBlock>(each_s, st.lo, st.hi, rs, (uint32_t)ns, 16u, sm.radix).binlo;
  }
  const int32_t T0 = (int32_t)(t0bits ^ 0x80000000u);  // as a score

  // 2. the list. With the union: the chunks whose best dropped key reaches T0
  bool listed = false;
  if (from_union) {  // uniform
    typedef const __attribute__((address_space(1))) uint64_t* GlobalU64;
    const bool hot = tid < G && ((GlobalU64)xc_row)[tid] >= ((uint64_t)t0bits << 32);
    const uint64_t hb = __ballot(hot);
    // (in sm.mxw: its last readers, on the ranking side, passed a barrier since)
    static_assert(kMaxChunks / 64 <= kSelWaves, "hot chunk masks");
    if (lane == 0 && w < kMaxChunks / 64) sm.mxw[w] = hb;
    lds_barrier();
    uint64_t hm[kMaxChunks / 64];
    uint32_t nhot = 0;
#pragma unroll
    for (int x = 0; x < kMaxChunks / 64; ++x) {
      hm[x] = sm.mxw[x];
      nhot += (uint32_t)__popcll(hm[x]);
    }
    if (nhot <= (uint32_t)kMaxHotChunks) {  // uniform
      // the union's keys at or above T0 from the other chunks (a thread's 16
      // entries lie in one chunk: cm >= 16)
      const int ct = kUPerThread * tid / cm;
      const bool cold = ct >= kMaxChunks || !((hm[ct >> 6] >> (ct & 63)) & 1ull);
#pragma unroll
      for (int j = 0; j < kUPerThread; ++j)
        append(((uvalid >> j) & 1u) && cold && key_ubits(u[j]) >= t0bits, key_score(u[j]), key_pos(u[j]));
      // every key at or above T0 of the hot chunks: wave w rescans the hot chunks
      // of rank w, w + 8, ... (each a round of up to 16 loads per lane per 1,024
      // positions)
      uint32_t rank = 0;
#pragma unroll
      for (int x = 0; x < kMaxChunks / 64; ++x) {
        uint64_t bits = hm[x];
        while (bits != 0ull) {  // uniform
          const int c = 64 * x + (int)__builtin_ctzll(bits);
          bits &= bits - 1ull;
          if ((int)(rank++ % kSelWaves) != w) continue;
          int cnt;
          const int len = 32 * row_chunk_units(n, c, G, P, ilv, &cnt);  // local positions, last unit cut
          constexpr int R = 16;
          for (int i0 = 0; i0 < len; i0 += 64 * R) {
            int32_t x4[R];
            uint32_t pos[R];
            bool ok[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const int i = i0 + 64 * r + lane;
              pos[r] = (uint32_t)(ilv ? 32 * (c + G * (i >> 5)) + (i & 31) : c * P + i);
              ok[r] = i < len && pos[r] < (uint32_t)n;
              x4[r] = row[ok[r] ? pos[r] : 0u];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) append(ok[r] && x4[r] >= T0, x4[r], pos[r]);
          }
        }
      }
      listed = true;
    }
  }
  if (!listed) {  // uniform
    // one pass over the whole row: the positions before the row's first 16-byte
    // boundary go to wave 0 first; then 16-byte loads, thread t's load j of a pass
    // covering positions h + 4 (q0 + t + 512 j) + [0, 4) (wave w: 64-position
    // slices)
    const int h0 = (int)(((16u - ((uint32_t)reinterpret_cast<uintptr_t>(row_in) & 15u)) & 15u) >> 2);
    const int h = h0 < n ? h0 : n;
    if (w == 0 && h > 0) {  // uniform
      int32_t x = 0;
      if (lane < h) x = row[lane];
      append(lane < h && x >= T0, x, (uint32_t)lane);
    }
    const int64_t m = (int64_t)n - h;  // positions from the boundary on
    const int64_t nq = (m + 3) / 4;    // 16-byte vectors holding them (each holds one)
    const GlobalI32x4 vrow = reinterpret_cast<GlobalI32x4>(row + h);
    constexpr int U = 16;
    constexpr int64_t step = (int64_t)kSelBlock * U;  // vectors per pass
    // keeps the keys of vector v of pass q0 (load j of the pass)
    auto keep_vec = [&](const i32x4& v, int64_t q0, int j, auto full) {
      const int64_t q = q0 + tid + (int64_t)kSelBlock * j;
      const int32_t x4[4] = {v.x, v.y, v.z, v.w};
      // the four compares first and one branch on them all
      bool keep[4];
      uint64_t any = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = x4[e] >= T0 && (decltype(full)::value || 4 * q + e < m);
        any |= __ballot(keep[e]);
      }
      if (any == 0ull) return;  // uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) append(keep[e], x4[e], (uint32_t)(h + 4 * q + e));
    };
    // passes whose vectors all lie inside the row: as soon as load j of a pass is
    // used, the same slot loads its vector of the next pass, so U loads stay in
    // flight (the last pass's follow-up loads repeat that pass rather than branch
    // around the loads)
    const int64_t nfull = (m / 4) / step;
    if (nfull > 0) {  // uniform
      i32x4 v[U];
      // (issued in slot order: the waits below count on it)
#pragma unroll
      for (int j = 0; j < U; ++j) {
        v[j] = vrow[tid + (int64_t)kSelBlock * j];
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int64_t p = 0; p < nfull; ++p) {
        const int64_t q0 = p * step;
        const GlobalI32x4 next = vrow + (p + 1 < nfull ? p + 1 : p) * step + tid;
#pragma unroll
        for (int j = 0; j < U; ++j) {
          keep_vec(v[j], q0, j, std::true_type{});
          v[j] = next[kSelBlock * j];
        }
      }
    }
    if (nfull * step < nq) {  // uniform: the rest, masked at the row's end
      const int64_t q0 = nfull * step;
      i32x4 v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t q = q0 + tid + (int64_t)kSelBlock * j;
        v[j] = vrow[q < nq ? q : nq - 1];  // a vector past the row's end is not read
      }
#pragma unroll
      for (int j = 0; j < U; ++j) keep_vec(v[j], q0, j, std::false_type{});
    }
  }

  // 3. The wave's own keys into registers (only its lanes wrote them, and LDS work
  // of one wave completes in order), and per wave the count and the best kept
  // score: the list's score range is [T0, the best of those] (bounds suffice for
  // the narrowing: no exchange of the keys' own range).
  const uint32_t own = wn < (uint32_t)kWaveCap ? wn : (uint32_t)kWaveCap;
  uint32_t lhi = 0;
  vmask = 0;
#pragma unroll
  for (int j = 0; j < kUPerThread; ++j) {
    const uint32_t i = (uint32_t)(kUPerThread * lane + j);
    key[j] = i < own ? wseg[i] ^ (1ull << 63) : 0ull;  // raw -> make_key
    sv[j] = key_ubits(key[j]);
    vmask |= i < own ? 1u << j : 0u;
    lhi = i < own && sv[j] > lhi ? sv[j] : lhi;
  }
  const uint32_t whi = wave_maxr_u32(lhi);
  if (lane == 0) {
    sm.wcnt[w][0] = wn;
    sm.wcnt[w][1] = whi;
  }
  lds_barrier();
  uint32_t total = 0, fits = 1, hi = 0;
#pragma unroll
  for (int x = 0; x < kSelWaves; ++x) {
    const uint32_t c = sm.wcnt[x][0];
    total += c;
    fits &= c <= (uint32_t)kWaveCap ? 1u : 0u;
    hi = sm.wcnt[x][1] > hi ? sm.wcnt[x][1] : hi;
  }
  if (!fits || total < (uint32_t)kk) return false;  // uniform
  rng[0] = t0bits;
  rng[1] = hi;
  *total_out = total;
  // every thread has read its keys before any writes the region again (the list
  // and sink slots that the narrowing uses lie over the kept keys)
  lds_barrier();
  return true;
}

// The exhaustive path's last resort: a radix selection over every position (a pass
// for the range, one radix pass per 11 bits of it), then a count and a write pass
// of an ordered compaction in which wave w owns one contiguous eighth of the row.
// Writes the kk best keys to sel in position order; returns the kk-th best key and
// sets *tied to the number of selected keys with its score.
__device__ __noinline__ uint64_t select_row_radix(const int32_t* __restrict__ row_in, int n, int kk, int k,
                                                  uint32_t* tied) {
  n = __builtin_amdgcn_readfirstlane(n);
  kk = __builtin_amdgcn_readfirstlane(kk);
  k = __builtin_amdgcn_readfirstlane(k);
  const GlobalI32 row = global_view(
      reinterpret_cast<const int32_t*>(uniform_u64(reinterpret_cast<uint64_t>(row_in))));
  const SelLds l = sel_lds(k);
  SelSmem& sm = *l.sm;
  uint64_t* const sel = l.sel;
  uint32_t lo = 0xFFFFFFFFu, hi = 0;
  for_each_score(row, n, [&](uint32_t u) {
    lo = u < lo ? u : lo;
    hi = u > hi ? u : hi;
  });
  const Stats4 st = block_stats(0, lo, hi, 0, sm);
  auto each = [&](auto f) { for_each_score(row, n, f); };
  uint32_t above;
  const uint32_t T = block_select_range<kSelBlock>(each, st.lo, st.hi, kk, &above, sm.radix);
  const uint32_t need_eq = (uint32_t)kk - above;
  *tied = need_eq;
  const int w = wave_id(), lane = lane_id();
  const int64_t rows = ((int64_t)n + 63) / 64, rpw = (rows + kSelWaves - 1) / kSelWaves;
  const int64_t p0 = (int64_t)w * rpw * 64 < n ? (int64_t)w * rpw * 64 : n;
  const int64_t p1 = p0 + rpw * 64 < n ? p0 + rpw * 64 : n;
  uint32_t gt = 0, eq = 0;
  wave_rows(row, p0, p1, [&](uint32_t u, int64_t, bool in) {
    gt += in && u > T ? 1u : 0u;
    eq += in && u == T ? 1u : 0u;
  });
  gt = wave_sum_u32(gt);
  eq = wave_sum_u32(eq);
  if (lane == 0) {
    sm.wcnt[w][0] = gt;
    sm.wcnt[w][1] = eq;
  }
  lds_barrier();
  uint32_t gb = 0, eb = 0;  // above / at T before this lane's position
  for (int x = 0; x < w; ++x) {
    gb += sm.wcnt[x][0];
    eb += sm.wcnt[x][1];
  }
  const uint64_t lt = lanemask_lt();
  wave_rows(row, p0, p1, [&](uint32_t u, int64_t p, bool in) {
    const bool g = in && u > T, e = in && u == T;
    const uint64_t bg = __ballot(g), be = __ballot(e);
    const uint32_t gbl = gb + (uint32_t)__popcll(bg & lt), ebl = eb + (uint32_t)__popcll(be & lt);
    if (g || (e && ebl < need_eq)) {
      const uint32_t slot = gbl + (ebl < need_eq ? ebl : need_eq);
      const uint64_t key = ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
      sel[slot] = key;
      if (e && ebl == need_eq - 1) sm.kstar = key;  // the last key taken at T is the kk-th best
    }
    gb += (uint32_t)__popcll(bg);
    eb += (uint32_t)__popcll(be);
  });
  lds_barrier();
  return sm.kstar;
}


// Exhaustive selection: the kk best keys of the row's n positions, written to sel
// (in an order that depends on the row alone); returns the kk-th best key and sets
// *tied to the number of selected keys with its score. The narrowed list of
// exhaustive_list, then the same exact top kk as on the candidate path; the radix
// selection when the list does not hold the top kk.
// Called functions get their arguments in vector registers and see generic
// pointers: the uniform arguments are moved back to scalar registers (or the row
// pass does its address and loop arithmetic per lane), the row's address space is
// named, and the LDS comes from its symbol. (Out of line: the exhaustive path is
// rare, and inlined into the selection kernel it made the candidate path's code
// larger and slower.)
__device__ __noinline__ uint64_t select_row_exhaustive(const SelectKernArgs* ka, int b, uint32_t* tied) {
  const ExhRow e = exh_row(ka, b);
  const SelLds l = sel_lds(e.k);
  uint64_t key[kUPerThread];
  uint32_t sv[kUPerThread], vmask = 0, total = 0, rng[2];
  if (e.kk > 0 && exhaustive_list(e.row, e.row_in, e.n, e.kk, e.cand_row, e.xc_row, e.cg.G, e.cg.m, e.cg.P, e.cg.ilv,
                                  l, key, sv, vmask, &total, rng)) {
    const TopK t = topk_of_keys<kUPerThread>(key, sv, vmask, total, (uint32_t)e.kk, rng[0], rng[1], false, l.sel,
                                             l.list, l.sink, *l.sm, false, 0ull);
    *tied = t.tied;
    return t.kstar;
  }
  return select_row_radix(e.row_in, e.n, e.kk, e.k, tied);
}

// Completes the narrowing of one sought key (the need-th largest of the keys held
// E per thread; rb from block_narrow_first) until its range holds at most
// kMaxBinRank keys: further passes over the scores, then, when one score value T
// holds more, over the low key words (positions) of the keys at T. Uniform: every
// thread gets the same range.
template <int E>
__device__ __forceinline__ KeyRange refine_key_range(RadixBin rb, uint32_t need, const uint64_t (&key)[E],
                                                     const uint32_t (&sv)[E], uint32_t vmask, RadixSmem& sm) {
  if (rb.inbin > kMaxBinRank && rb.binlo < rb.binhi) {
    const uint32_t blo = rb.binlo, bhi = rb.binhi;
    auto each_in = [&](auto f) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (((vmask >> j) & 1u) && sv[j] >= blo && sv[j] <= bhi) f(sv[j]);
    };
    const RadixBin r2 = block_narrow<kSelBlock>(each_in, blo, bhi, need - rb.above, rb.inbin, kMaxBinRank, sm);
    rb = RadixBin{r2.binlo, r2.binhi, rb.above + r2.above, r2.inbin};
  }
  if (rb.inbin > kMaxBinRank) {  // one score value T holds that many keys
    const uint32_t T = rb.binlo;
    auto each_tie = [&](auto f) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (((vmask >> j) & 1u) && sv[j] == T) f((uint32_t)key[j]);
    };
    const RadixBin rt = block_narrow<kSelBlock>(each_tie, 0u, 0xFFFFFFFFu, need - rb.above, rb.inbin, kMaxBinRank, sm);
    return KeyRange{((uint64_t)T << 32) | rt.binlo, ((uint64_t)T << 32) | rt.binhi, rb.above + rt.above, rt.inbin,
                    rb.above, true};
  }
  return KeyRange{(uint64_t)rb.binlo << 32, ((uint64_t)rb.binhi << 32) | 0xFFFFFFFFull, rb.above, rb.inbin, rb.above,
                  false};
}

// Attention window: of the n valid keys held E per thread (score bits sv, all in
// [lo, hi]; `sorted` when every thread's keys run best first), the positions of
// those whose rank (0 = best) lies in [r0, r1] go to sm.winpos[rank - r0], that is
// in output order. The two window ends are narrowed together (one shared first
// radix pass), the keys from the lower end's range to the upper end's range are
// collected in wl (at most kMaxWindowList) and ranked among themselves.
// With count_mx, the call also returns the number of valid keys above the best of
// the G dropped keys xc[0, G) (for the candidate path's coverage check). Those are
// requested here and exchanged and counted behind the narrowing, on its barriers:
// a load still in flight where the caller's paths join is waited for there.
// When the window ends at rank kk - 1 (the last selected key), sm.kstar gets that
// key K* and sm.tied the number of selected keys with its score T: K* and the keys
// above it at T, which are collected keys (counted beside the ranks) or, when the
// upper end's range is a run of positions at T, the keys at T above that range.
template <int E>
__device__ __forceinline__ uint32_t window_positions(const uint64_t (&key)[E], const uint32_t (&sv)[E],
                                                     uint32_t vmask, uint32_t n, uint32_t lo, uint32_t hi,
                                                     bool sorted, bool count_mx, const uint64_t* __restrict__ xc,
                                                     int G, uint32_t r0, uint32_t r1, uint32_t kk, uint64_t* wl,
                                                     uint64_t* sink, SelSmem& sm) {
  // one dropped key per thread (clamped address; threads past G count 0)
  const uint64_t mx = count_mx ? xc[threadIdx.x < (unsigned)G ? threadIdx.x : G - 1] : 0ull;
  const uint32_t need[2] = {r0 + 1, r1 + 1};
  auto each = [&](auto f) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((vmask >> j) & 1u) f(sv[j]);
  };
  RadixBin rb[2];
  block_narrow_first<kSelBlock, 2>(each, lo, hi, need, n, sm.radix, rb);
  const KeyRange top = refine_key_range<E>(rb[0], need[0], key, sv, vmask, sm.radix);
  const KeyRange bot = refine_key_range<E>(rb[1], need[1], key, sv, vmask, sm.radix);
  // every key of the window lies in [bot.klo, top.khi]; the keys above top.khi
  // number top.above
  // a present key is never 0, and an absent one is 0: below klo (>= 1) and not
  // above khi, so the comparisons below need no presence test
  const uint64_t klo = bot.klo > 0 ? bot.klo : 1, khi = top.khi;
  uint32_t a = 0, b = 0;  // sorted: the thread's keys in range are its keys [a, b)
#pragma unroll
  for (int j = 0; j < E; ++j) {
    a += key[j] > khi ? 1u : 0u;
    b += key[j] >= klo ? 1u : 0u;
  }
  if (count_mx) {  // uniform
    const uint64_t wmx = wave_maxr_u64(threadIdx.x < (unsigned)G ? mx : 0ull);
    if (lane_id() == 0) sm.mxw[wave_id()] = wmx;
  }
  uint32_t total;
  // the last barrier of the narrowing separates every earlier reader of the scan
  // slots; this scan's barrier publishes the waves' dropped keys
  const uint32_t base = block_excl_scan_fresh_u32<kSelBlock>(b - a, sm.radix.part, &total);
  uint64_t* const mine = sink + threadIdx.x;
  // b - a keys of each thread are in range (keys at or above klo, less those above
  // khi): its keys [a, b) when sorted, otherwise found key by key
  if (sorted) {  // uniform
#pragma unroll
    for (int j = 0; j < E; ++j)
      *(((uint32_t)j >= a && (uint32_t)j < b) ? wl + (base + (uint32_t)j - a) : mine) = key[j];
  } else {
    uint32_t sl = base;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const bool t = key[j] >= klo && key[j] <= khi;
      *(t ? wl + sl : mine) = key[j];
      sl += t ? 1u : 0u;
    }
  }
  if (count_mx) {  // uniform: keys above the largest dropped key, per wave
    uint64_t m = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) m = sm.mxw[w] > m ? sm.mxw[w] : m;
    uint32_t g = 0;  // (an absent key, 0, is above no key)
#pragma unroll
    for (int j = 0; j < E; ++j) g += key[j] > m ? 1u : 0u;
    g = wave_sum_u32(g);
    if (lane_id() == 0) sm.gtw[wave_id()] = g;
  }
  lds_barrier();
  const uint32_t nw = total;
  // rank of a collected key = top.above + number of collected keys above it; eight
  // threads per key, four reads in flight each
  const int grp = threadIdx.x >> 3, part = threadIdx.x & 7;
  const bool last = r1 + 1 == kk;  // uniform
  for (uint32_t b0 = 0; b0 < nw; b0 += kSelBlock / 8) {
    const uint32_t i = b0 + (uint32_t)grp;
    const uint64_t me = i < nw ? wl[i] : ~0ull;
    const uint32_t mes = key_ubits(me);
    uint32_t r = 0, eq = 0;  // collected keys above me; those of them with me's score
    for (uint32_t j0 = (uint32_t)part; j0 < nw; j0 += 32) {
      uint64_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t jj = j0 + 8 * u;
        v[u] = wl[jj < nw ? jj : nw - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool above_me = j0 + 8 * u < nw && v[u] > me;
        r += above_me ? 1u : 0u;
        if (last) eq += above_me && key_ubits(v[u]) == mes ? 1u : 0u;
      }
    }
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor1, 0xF, 0xF, false);
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor2, 0xF, 0xF, false);
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kRowHalfMirror, 0xF, 0xF, false);
    if (last) {
      eq += (uint32_t)__builtin_amdgcn_mov_dpp((int)eq, dpp::kQuadXor1, 0xF, 0xF, false);
      eq += (uint32_t)__builtin_amdgcn_mov_dpp((int)eq, dpp::kQuadXor2, 0xF, 0xF, false);
      eq += (uint32_t)__builtin_amdgcn_mov_dpp((int)eq, dpp::kRowHalfMirror, 0xF, 0xF, false);
    }
    const uint32_t gr = top.above + r;
    if (part == 0 && i < nw && gr >= r0 && gr <= r1) {
      sm.winpos[gr - r0] = key_pos(me);
      if (gr + 1 == kk) {
        // keys at T above the upper end's range: only when that range is a run of
        // positions at T (a range of scores has only higher scores above it)
        const uint32_t at_t_above = top.tie && key_ubits(top.khi) == mes ? top.above - top.gt : 0u;
        sm.kstar = me;
        sm.tied = 1u + eq + at_t_above;
      }
    }
  }
  lds_barrier();
  uint32_t gt = 0;
  if (count_mx)
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) gt += sm.gtw[w];
  return gt;
}

// The attention window on the exhaustive path: the window narrowing over the list
// of exhaustive_list (its ranks are the row's for the top kk), or over the kk keys
// of the radix selection. (Out of line, so that loads in flight on the candidate
// path are not waited for where its code would otherwise join this path's; uniform
// arguments back in scalar registers as in select_row_exhaustive.)
__device__ __noinline__ void exhaustive_window(const SelectKernArgs* ka, int b, uint32_t r0, uint32_t r1) {
  const ExhRow e = exh_row(ka, b);
  const int kk = e.kk;
  r0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)r0);
  r1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)r1);
  const SelLds l = sel_lds(e.k);
  SelSmem& sm = *l.sm;
  uint64_t key[kUPerThread];
  uint32_t sv[kUPerThread], vmask = 0, total = 0, rng[2];
  if (!exhaustive_list(e.row, e.row_in, e.n, kk, e.cand_row, e.xc_row, e.cg.G, e.cg.m, e.cg.P, e.cg.ilv, l, key, sv,
                       vmask, &total, rng)) {
    uint32_t tied;
    select_row_radix(e.row_in, e.n, kk, e.k, &tied);
    vmask = 0;
#pragma unroll
    for (int j = 0; j < kUPerThread; ++j) {
      const int i = kUPerThread * (int)threadIdx.x + j;
      key[j] = i < kk ? l.sel[i] : 0ull;
      sv[j] = key_ubits(key[j]);
      vmask |= i < kk ? 1u << j : 0u;
    }
    total = (uint32_t)kk;
    bool sorted;
    union_range_exchange<kUPerThread>(key, sv, vmask, sm, rng, &sorted);
  }
  window_positions<kUPerThread>(key, sv, vmask, total, rng[0], rng[1], false, false, nullptr, 0, r0, r1,
                                (uint32_t)kk, l.list, l.sink, sm);
}

// The kernel's argument segment, as the exhaustive path reads it.
__device__ __forceinline__ const SelectKernArgs* kernel_args() {
  return (const SelectKernArgs*)(const __attribute__((address_space(4))) SelectKernArgs*)
      __builtin_amdgcn_kernarg_segment_ptr();
}

// LDS as laid out by sel_lds.
// The arguments that the first requests need come first, as separate scalars: the
// leading arguments can be preloaded into scalar registers at wave launch, so the
// candidate, dropped-key, summary and query requests need not wait for a read of the
// argument block (a.cand, a.xc, a.sums, a.G, at.q, at.Hq, at.Dk and at.S, passed
// again).
// PG: the latent cache is a paged pool (at.pages); the window's positions become pool
// rows before the gather.
template <class Attn, bool PG>
__global__ __launch_bounds__(kSelBlock) void k_select(const uint64_t* __restrict__ cand,
                                                      const uint64_t* __restrict__ xc,
                                                      const ChunkSum* __restrict__ sums, const void* __restrict__ q,
                                                      int G, int Hq, int Dk, int S, SelArgs a, AttnArgs at) {
  const SelLds lds = sel_lds(a.k);
  SelSmem& sm = *lds.sm;
  uint64_t* sel = lds.sel;
  uint8_t* region = lds.region;
  uint64_t* list = lds.list;  // bin or window keys
  uint64_t* sink = lds.sink;
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  // With attention (the decode step) every workgroup is an attention split, and the
  // splits' windows are the output; without (the stand-alone selection) every
  // workgroup ranks a slice of the selected keys. One role per instantiation keeps
  // each kernel's registers to its own path.
  constexpr bool kRank = std::is_same<Attn, AttnNone>::value;
  // Requests first, all from preloaded arguments. The candidate union U: thread t
  // holds entries [16t, 16t + 16), eight 16-byte pieces, piece j of all threads
  // contiguous (cand_slot); its workspace region always exists, and the entries are
  // used on the candidate path only.
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  uint64_t key[kUPerThread];
  {
    const u64x2* src = reinterpret_cast<const u64x2*>(cand + (int64_t)b * kCandCap) + tid;
#pragma unroll
    for (int j = 0; j < kUPerThread / 2; ++j) {
      const u64x2 v = src[(kCandCap / 16) * j];
      key[2 * j] = v.x;
      key[2 * j + 1] = v.y;
    }
  }
  // every wave reads all chunk summaries (four per lane; clamped repeats change
  // neither a minimum, a maximum nor an or). The loads are issued in any case (a
  // branch around them leaves their registers possibly in flight where the paths
  // join, and the compiler then waits for every load before reusing one): without
  // summaries they read the candidate region instead, and the values go unused.
  const bool sums_on = sums != nullptr && G > 0;  // uniform
  u32x3 csum[4];  // lo, hi, ordered (the padding word is not read)
  {
    const uint8_t* sp = sums_on ? reinterpret_cast<const uint8_t*>(sums + (int64_t)b * kMaxChunks)
                                : reinterpret_cast<const uint8_t*>(cand + (int64_t)b * kCandCap);
    const int last = G > 0 ? G - 1 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lane_id() + 64 * i;
      csum[i] = *reinterpret_cast<const u32x3*>(sp + sizeof(ChunkSum) * (c < last ? c : last));
    }
  }
  // the requests above go out before anything else (left to itself the scheduler
  // put the attention's address arithmetic first)
  __builtin_amdgcn_sched_barrier(0);
  AttnArgs atq = at;  // the row shape from the preloaded arguments
  atq.q = q;
  atq.Hq = Hq;
  atq.Dk = Dk;
  const typename Attn::QFrag qf = Attn::load_q(atq, b);  // every workgroup: exact wait counts
  // Then fields from every 64-byte line of the argument block, read here and waited
  // for together, so every later argument read hits the scalar cache (read where
  // first used, behind the branches before them, they took several memory round
  // trips in a row).
  // The fields that decide the path pass through the asm as opaque values, and its
  // memory clobber keeps it behind the requests above: left to itself the compiler
  // computed the path, and waited for these reads, ahead of the first request.
  int n = a.lens.n[b], have_cand = a.have_cand, cand_valid = a.cand_valid.n[b], force = a.force, kq = a.k;
  {
    const int32_t* l0 = a.idx;
    asm volatile("" : "+s"(n), "+s"(have_cand), "+s"(cand_valid), "+s"(force), "+s"(kq) : "s"(l0) : "memory");
  }
  // paged: the page table in LDS, past the largest of the selection's and the
  // attention's regions. Its address is formed from kq, which arrives with the reads
  // above: formed from a.k like `region`, it put a wait for the argument block ahead
  // of the union's loads.
  uint32_t* ptab = reinterpret_cast<uint32_t*>(
      reinterpret_cast<uint8_t*>(lds.sm) + align16(sizeof(SelSmem)) + align16((size_t)kq * 8) +
      align16(Attn::lds_bytes(Hq, Dk) > kRegionSelect ? Attn::lds_bytes(Hq, Dk) : kRegionSelect));
  if constexpr (PG) {
    // (these copies end with the staging; the translation below reads the arguments
    // again, from the scalar cache, so nothing stays live through the selection)
    const int32_t* pages = at.pages;
    int pool_pages = at.pool_pages, lds_pages = at.lds_pages;
    asm volatile("" : "+s"(pages), "+s"(pool_pages), "+s"(lds_pages)::"memory");
    // The table into LDS, requested behind the union's loads (the wait for it ends
    // about when those arrive, and the selection needs them first), four entries a
    // thread per round; the window's positions are translated from there.
    constexpr int kPer = 4;
    for (int i0 = 0; i0 < lds_pages; i0 += kPer * kSelBlock) {  // uniform
      int32_t e[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + tid + kSelBlock * u;
        e[u] = i < lds_pages ? pages[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + tid + kSelBlock * u;
        if (i < lds_pages) ptab[i] = (uint32_t)(e[u] < 0 ? 0 : (e[u] >= pool_pages ? pool_pages - 1 : e[u]));
      }
    }
  }
  const int32_t* row = a.scores + (int64_t)b * a.N;

  int reason = force ? 1 : (have_cand ? 0 : 3);
  const int kk = kq < n ? kq : n;  // positions selected on either path
  const uint32_t nvalid = reason == 0 ? (uint32_t)cand_valid : 0u;
  // A union with fewer valid keys than kk dropped some position (it holds every
  // position of a chunk that keeps them all), so it cannot cover the top kk.
  if (reason == 0 && nvalid < (uint32_t)kk) reason = 2;
  if (reason == 0) {
    // entries past the union's end are absent (key 0)
    const int C = G * a.m;
#pragma unroll
    for (int j = 0; j < kUPerThread; ++j) key[j] = kUPerThread * tid + j < C ? key[j] : 0ull;
  }
  radix_clear<kSelBlock>(sm.radix);

  if constexpr (!kRank) {
    // ------------------------------------------------ attention workgroup s
    const int per = (a.k + S - 1) / S;
    const int r0 = (int)blockIdx.x * per;
    const int cnt = kk - r0 < 0 ? 0 : (kk - r0 > per ? per : kk - r0);
    // the window narrowing over the union on the candidate path; when the coverage
    // check fails, or the path is exhaustive, over the exhaustively selected keys
    if (cnt > 0 && reason == 0) {  // uniform
      uint32_t sv[kUPerThread], vmask = 0;
#pragma unroll
      for (int j = 0; j < kUPerThread; ++j) {
        sv[j] = key_ubits(key[j]);
        vmask |= (uint32_t)key[j] != 0u ? 1u << j : 0u;
      }
      uint32_t rng[2];
      bool sorted;
      if (sums_on) {  // uniform
        union_range_from_sums(csum, rng, &sorted);
        lds_barrier();  // publishes the cleared radix histograms
      } else {
        union_range_exchange<kUPerThread>(key, sv, vmask, sm, rng, &sorted);
      }
      const uint32_t above_mx =
          window_positions<kUPerThread>(key, sv, vmask, nvalid, rng[0], rng[1], sorted, true, xc + (int64_t)b * G,
                                        G, (uint32_t)r0, (uint32_t)(r0 + cnt - 1), (uint32_t)kk, list, sink, sm);
      // the union's top kk are the row's when at least kk of its keys lie above every
      // dropped key (nvalid >= kk here, and a union with fewer than k valid keys then
      // holds every position and dropped none)
      if (above_mx < (uint32_t)kk) reason = 2;
    }
    if (cnt > 0 && reason != 0)  // uniform
      exhaustive_window(kernel_args(), b, (uint32_t)r0, (uint32_t)(r0 + cnt - 1));
    // sm.winpos is complete and published (the last barrier of the window
    // narrowing follows its last write), and the LDS region is free again
    {  // the output slots [r0, r0 + per) of the row: the window's positions, then -1 past kk
      int32_t* out = a.idx + (int64_t)b * a.k;
      for (int i = tid; i < per && r0 + i < a.k; i += kSelBlock) out[r0 + i] = i < cnt ? (int32_t)sm.winpos[i] : -1;
      if (cnt > 0 && r0 + cnt == kk && tid == 0) {  // the window of the kk-th best key
        RowStats st;
        st.path = reason == 0 ? 0 : 1;
        st.reason = reason;
        st.selected = kk;
        st.kth_score = key_score(sm.kstar);
        st.candidates = (int32_t)nvalid;
        st.tied_at_kth = (int32_t)sm.tied;
        st.bad_indices = 0;
        st.reserved = 0;
        a.stats[b] = st;
      }
    }
    if constexpr (PG) {
      // a paged latent cache: the window's positions become pool rows before the
      // gather (the table in LDS, or in memory when it did not fit), so the gather is
      // the contiguous one (a translation inside it, per row, put a branch and two
      // dependent reads between its row requests: 0.5 us)
      if (tid < cnt) {
        const uint32_t pos = sm.winpos[tid];
        sm.winpos[tid] = at.lds_pages > 0 ? ptab[pos >> kPageShift] * kPageSize + (pos & (kPageSize - 1))
                                          : page_row(at.pages, at.pool_pages, pos);
      }
      lds_barrier();
    }
    Attn::run(at, b, blockIdx.x, [&](int i) { return (int64_t)sm.winpos[i]; }, cnt, region, qf);
    return;
  }

  // -------------------------------------------------- ranking workgroup r
  uint32_t nsel = 0, tied = 0;
  uint64_t kstar = 0;
  if (reason == 0) {
    uint32_t sv[kUPerThread], vmask = 0;
#pragma unroll
    for (int j = 0; j < kUPerThread; ++j) {
      sv[j] = key_ubits(key[j]);
      vmask |= (uint32_t)key[j] != 0u ? 1u << j : 0u;
    }
    uint32_t rng[2];
    bool sorted;
    if (sums_on) {
      union_range_from_sums(csum, rng, &sorted);
      lds_barrier();  // publishes the cleared radix histograms
    } else {
      union_range_exchange<kUPerThread>(key, sv, vmask, sm, rng, &sorted);
    }
    const uint32_t kku = (uint32_t)kk;  // <= nvalid here
    const uint64_t mx = tid < G ? xc[(int64_t)b * G + tid] : 0ull;  // waited for behind the narrowing
    // the keys above the kk-th key's range in union order, then the range's best in
    // key order
    const TopK t = topk_of_keys<kUPerThread>(key, sv, vmask, nvalid, kku, rng[0], rng[1], sorted, sel, list, sink, sm,
                                             true, mx);
    kstar = t.kstar;
    uint64_t mxall = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) mxall = sm.mxw[w] > mxall ? sm.mxw[w] : mxall;
    // every dropped key is below the k-th candidate: the candidates hold the top k
    const bool ok = mxall < kstar && (nvalid >= (uint32_t)a.k || mxall == 0);
    if (ok) {
      nsel = kku;
      tied = t.tied;
    } else {
      reason = 2;
    }
  }
  // the exhaustive path streams the whole row in every workgroup that takes part,
  // so fewer ranking workgroups take part there, each with a larger slice
  const int R = reason == 0 ? a.R : (a.R < kFallbackRankers ? a.R : kFallbackRankers);
  const int r = (int)blockIdx.x;
  if (r >= R) return;  // uniform
  if (reason != 0) {
    kstar = select_row_exhaustive(kernel_args(), b, &tied);
    nsel = (uint32_t)kk;
  }

  // ranking: the slot of a key is the number of selected keys larger than it
  constexpr int TPE = 32;  // threads per ranked key
  const int per = ((int)nsel + R - 1) / R;
  const int e0 = r * per;
  const int e1 = e0 + per < (int)nsel ? e0 + per : (int)nsel;
  int32_t* out = a.idx + (int64_t)b * a.k;
  for (int base = e0; base < e1; base += kSelBlock / TPE) {
    const int e = base + tid / TPE;
    const int part = tid % TPE;
    const uint64_t me = e < e1 ? sel[e] : ~0ull;
    uint32_t cnt = 0;
    // keys part, part + TPE, ...: eight loads in flight per step, masked past nsel
    for (int x0 = part; x0 < (int)nsel; x0 += 8 * TPE) {
      uint64_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int x = x0 + i * TPE;
        v[i] = sel[x < (int)nsel ? x : (int)nsel - 1];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) cnt += (x0 + i * TPE < (int)nsel) && v[i] > me;
    }
    // sum over the 32 lanes of this key (half a wave)
    cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, dpp::kQuadXor1, 0xF, 0xF, false);
    cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, dpp::kQuadXor2, 0xF, 0xF, false);
    cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, dpp::kRowHalfMirror, 0xF, 0xF, false);
    cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, dpp::kRowMirror, 0xF, 0xF, false);
    cnt += (uint32_t)__shfl_xor((int)cnt, 16);
    if (e < e1 && part == 0) out[cnt] = (int32_t)key_pos(me);
  }
  if (r == 0) {
    for (int j = (int)nsel + tid; j < a.k; j += kSelBlock) out[j] = -1;
    if (tid == 0) {
      RowStats st;
      st.path = reason == 0 ? 0 : 1;
      st.reason = reason;
      st.selected = (int32_t)nsel;
      st.kth_score = key_score(kstar);
      st.candidates = (int32_t)nvalid;
      st.tied_at_kth = (int32_t)tied;
      st.bad_indices = 0;
      st.reserved = 0;
      a.stats[b] = st;
    }
  }
}

// The contiguous selection kernels are instantiated, and so laid out in the code
// object, ahead of the paged ones: where a kernel's code sits measurably changes its
// time (an identical contiguous kernel ran 0.15 us slower, the step 0.4 us, when the
// paged kernels before it changed size), and this keeps paged changes from moving it.
template <class... A>
const void* select_order(int i) {
  const void* const k[] = {(const void*)&k_select<A, false>...};
  return k[i];
}
template const void* select_order<AttnNone, AttnGeneric<float>, AttnGeneric<uint16_t>, AttnMfma<1, 32, 3, true>,
                                  AttnMfma<1, 32, 5, true>, AttnMfma<2, 32, 5, true>, AttnMfma<3, 32, 5, true>,
                                  AttnMfma<4, 32, 5, true>, AttnMfma<1, 32, 5>, AttnMfma<1, 32>, AttnMfma<2, 32>,
                                  AttnMfma<3, 32>, AttnMfma<4, 32>>(int);

template <class Attn>
static size_t select_lds_t(int Hq, int Dk, int k) {
  const size_t ra = Attn::lds_bytes(Hq, Dk);
  return align16(sizeof(SelSmem)) + align16((size_t)k * 8) + (ra > kRegionSelect ? ra : kRegionSelect);
}

template <class Attn>
static hipError_t launch_select_t(const SelArgs& a, const AttnArgs& at, int B, hipStream_t s, KTimer t) {
  size_t lds = select_lds_t<Attn>(at.Hq, at.Dk, a.k);
  auto fn = k_select<Attn, false>;
  if constexpr (!std::is_same<Attn, AttnNone>::value)
    if (at.pages != nullptr) {
      fn = k_select<Attn, true>;
      lds += align16((size_t)at.lds_pages * 4);
    }
  hipError_t e = allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  // attention splits (decode step) or ranking workgroups (stand-alone selection)
  const int grid = std::is_same<Attn, AttnNone>::value ? a.R : at.S;
  return launch_timed(fn, dim3(grid, B), dim3(kSelBlock), lds, s, t, a.cand, a.xc, a.sums, at.q, a.G, at.Hq,
                      at.Dk, at.S, a, at);
}

// ------------------------------------------------------------------ attention over given indices

template <class Attn>
__global__ __launch_bounds__(kSelBlock) void k_attend_idx(const int32_t* __restrict__ idx, int k,
                                                          int32_t* __restrict__ part_bad, AttnArgs at) {
  extern __shared__ __align__(16) uint8_t smem[];
  SelSmem& sm = *reinterpret_cast<SelSmem*>(smem);
  const int per = (k + at.S - 1) / at.S;
  int32_t* posl = reinterpret_cast<int32_t*>(smem + align16(sizeof(SelSmem)));
  uint8_t* region = smem + align16(sizeof(SelSmem)) + align16((size_t)per * 4);
  const int tid = threadIdx.x;
  const int b = blockIdx.y, j = blockIdx.x;
  const int e0 = j * per;
  const int e1 = e0 + per < k ? e0 + per : k;
  const int32_t* row = idx + (int64_t)b * k;
  const typename Attn::QFrag qf = Attn::load_q(at, b);
  uint32_t bad = 0, run = 0;
  for (int r0 = e0; r0 < e1; r0 += kSelBlock) {
    const int i = r0 + tid;
    const int32_t v = i < e1 ? row[i] : -1;
    const bool keep = v >= 0 && (int64_t)v < at.N;
    bad += (v != -1 && !keep);
    // a paged latent cache: the listed positions become pool rows
    const int32_t row_at = keep && at.pages != nullptr ? (int32_t)page_row(at.pages, at.pool_pages, v) : v;
    uint32_t total;
    const uint32_t slot = run + block_excl_scan_u32<kSelBlock>(keep ? 1u : 0u, sm.radix.part, &total);
    if (keep) posl[slot] = row_at;
    run += total;
  }
  bad = block_stats(bad, 0, 0, 0, sm).sum;
  if (tid == 0) part_bad[(int64_t)b * at.S + j] = (int32_t)bad;
  Attn::run(at, b, j, [&](int i) { return (int64_t)posl[i]; }, (int)run, region, qf);
}

template <class Attn>
static hipError_t launch_attend_t(const int32_t* idx, int k, int32_t* part_bad, const AttnArgs& at,
                                  int B, hipStream_t s) {
  const int per = (k + at.S - 1) / at.S;
  const size_t lds = align16(sizeof(SelSmem)) + align16((size_t)per * 4) + Attn::lds_bytes(at.Hq, at.Dk);
  auto fn = k_attend_idx<Attn>;
  hipError_t e = allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(at.S, B), dim3(kSelBlock), lds, s, idx, k, part_bad, at);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch

AttnChoice choose_attn(int dt, int Hq, int Dk, int Dv) {
  AttnChoice c{ATTN_NONE, 0, 0, 0, 0};
  if (dt != DT_F32 && Hq >= 1 && Hq <= 64 && Dk % 32 == 0 && Dk <= 1024 && Dv % 16 == 0 && Dv <= 512 &&
      Dv <= Dk) {
    c.kind = ATTN_MFMA_BF16;
    c.hqt = (Hq + 15) / 16;
    c.sb = 32;  // a split's 32 rows form one sub-block
    if (dt == DT_BF16_Q_E4M3_KV) {
      // one gather pass of 16-byte loads over Dk-byte rows: three per thread cover
      // Dk <= 768 (the 576-value latent row), five Dk <= 1024
      c.kv8 = 1;
      c.nl = c.hqt == 1 && (Dk / 16) * c.sb <= AttnMfma<1, 32, 3, true>::kMaxLoads * kAttnBlock ? 3 : 5;
      return c;
    }
    // one gather pass; five loads per thread cover Dk <= 640 (the 576-value latent row)
    c.nl = c.hqt == 1 && (Dk / 8) * c.sb <= AttnMfma<1, 32, 5>::kMaxLoads * kAttnBlock ? 5 : 9;
    if ((Dk / 8) * c.sb <= AttnMfma<1, 32>::kMaxLoads * kAttnBlock) return c;
    c = AttnChoice{ATTN_NONE, 0, 0, 0, 0};
  }
  if (dt != DT_BF16_Q_E4M3_KV && Hq >= 1 && Hq * Dv <= 4096 && Dk <= 512 && Dv <= Dk) {
    c.kind = dt == DT_BF16 ? ATTN_GENERIC_BF16 : ATTN_GENERIC_F32;
    c.sb = AttnGeneric<float>::SB;
  }
  return c;
}

#define DSA_ATTN_DISPATCH(FN, ...)                                                     \
  switch (ch.kind) {                                                                   \
    case ATTN_NONE: return FN<AttnNone>(__VA_ARGS__);                                  \
    case ATTN_GENERIC_F32: return FN<AttnGeneric<float>>(__VA_ARGS__);                 \
    case ATTN_GENERIC_BF16: return FN<AttnGeneric<uint16_t>>(__VA_ARGS__);             \
    case ATTN_MFMA_BF16:                                                               \
      if (ch.kv8) {                                                                    \
        switch (ch.hqt) {                                                              \
          case 1:                                                                      \
            if (ch.nl == 3) return FN<AttnMfma<1, 32, 3, true>>(__VA_ARGS__);          \
            return FN<AttnMfma<1, 32, 5, true>>(__VA_ARGS__);                          \
          case 2: return FN<AttnMfma<2, 32, 5, true>>(__VA_ARGS__);                    \
          case 3: return FN<AttnMfma<3, 32, 5, true>>(__VA_ARGS__);                    \
          case 4: return FN<AttnMfma<4, 32, 5, true>>(__VA_ARGS__);                    \
        }                                                                              \
        break;                                                                         \
      }                                                                                \
      switch (ch.hqt) {                                                                \
        case 1:                                                                        \
          if (ch.nl == 5) return FN<AttnMfma<1, 32, 5>>(__VA_ARGS__);                  \
          return FN<AttnMfma<1, 32>>(__VA_ARGS__);                                     \
        case 2: return FN<AttnMfma<2, 32>>(__VA_ARGS__);                               \
        case 3: return FN<AttnMfma<3, 32>>(__VA_ARGS__);                               \
        case 4: return FN<AttnMfma<4, 32>>(__VA_ARGS__);                               \
      }                                                                                \
      break;                                                                           \
    default: break;                                                                    \
  }                                                                                    \
  return hipErrorInvalidValue;

using AttnM1x32 = AttnMfma<1, 32>;
using AttnM2x32 = AttnMfma<2, 32>;
using AttnM3x32 = AttnMfma<3, 32>;
using AttnM4x32 = AttnMfma<4, 32>;

static size_t select_lds_dispatch(AttnChoice ch, int Hq, int Dk, int k) {
  switch (ch.kind) {
    case ATTN_NONE: return select_lds_t<AttnNone>(Hq, Dk, k);
    case ATTN_GENERIC_F32: return select_lds_t<AttnGeneric<float>>(Hq, Dk, k);
    case ATTN_GENERIC_BF16: return select_lds_t<AttnGeneric<uint16_t>>(Hq, Dk, k);
    case ATTN_MFMA_BF16:
      switch (ch.hqt) {
        case 1: return select_lds_t<AttnM1x32>(Hq, Dk, k);
        case 2: return select_lds_t<AttnM2x32>(Hq, Dk, k);
        case 3: return select_lds_t<AttnM3x32>(Hq, Dk, k);
        default: return select_lds_t<AttnM4x32>(Hq, Dk, k);
      }
  }
  return ~(size_t)0;
}

size_t select_lds_bytes(AttnChoice ch, int Hq, int Dk, int k) {
  return select_lds_dispatch(ch, Hq, Dk, k);
}

hipError_t launch_select(const SelArgs& a, const AttnArgs& at, AttnChoice ch, int B, hipStream_t s,
                         KTimer t) {
  DSA_ATTN_DISPATCH(launch_select_t, a, at, B, s, t)
}

hipError_t launch_attend_idx(const int32_t* idx, int k, int32_t* part_bad, const AttnArgs& at,
                             AttnChoice ch, int B, hipStream_t s) {
  if (ch.kind == ATTN_NONE) return hipErrorInvalidValue;
  DSA_ATTN_DISPATCH(launch_attend_t, idx, k, part_bad, at, B, s)
}

// ------------------------------------------------------------------ combine

constexpr int kCombWideBlock = 256;

// The combine for many splits (up to kMaxWideSplits; partials in accumulator
// order): one workgroup per 16 output elements of that order (4 heads x 16
// values). It forms the split weights of its 4 heads (64 thread groups,
// fixed-order reductions), then 16 thread groups each sum every 16th split and the
// groups are added in order, so the result does not depend on timing.
// (the partials' addresses and shape come first, preloaded at wave launch: at.part_ml,
// at.part_o, at.S, at.Hq and at.Dv, passed again)
__global__ __launch_bounds__(kCombWideBlock) void k_combine_wide(const float2* __restrict__ part_ml,
                                                                 const float* __restrict__ part_o, int S, int Hq,
                                                                 int Dv, const int32_t* __restrict__ part_bad,
                                                                 RowStats* __restrict__ stats, float* __restrict__ out) {
  __shared__ float wt[4][kMaxWideSplits];
  __shared__ float red[4][65];
  __shared__ v4f part[16][16];
  const int b = blockIdx.y, t = threadIdx.x;
  const int HP = (Hq + 15) / 16 * 16, tiles = Dv / 16;
  const int quad = blockIdx.x, tile = quad >> 2, l0 = 16 * (quad & 3);
  const int h0 = 16 * (tile / tiles) + 4 * (quad & 3);  // heads h0 .. h0 + 3
  // every load first: this thread's (max, sum) pairs, then its partial outputs
  const int h = t & 3, g = t >> 2;
  const int hh = h0 + h < Hq ? h0 + h : Hq - 1;
  float2 ml[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sp = g + 64 * i;
    ml[i] = part_ml[((int64_t)b * S + (sp < S ? sp : S - 1)) * Hq + hh];
  }
  const int e = t & 15, q = t >> 4;
  const float* po = part_o + (int64_t)b * S * HP * Dv;
  const int64_t el = (int64_t)tile * 64 + l0 + e;  // 16-byte element
  constexpr int kPer = kMaxWideSplits / 16;
  v4f v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int sp = q + 16 * i;
    v[i] = *(const v4f*)(po + (int64_t)(sp < S ? sp : S - 1) * HP * Dv + el * 4);
  }
  // split weights e^(m_s - M) / L of the four heads
  red[h][g] = fmaxf(g < S ? ml[0].x : -INFINITY, g + 64 < S ? ml[1].x : -INFINITY);
  lds_barrier();
  if (t < 4) {
    float M = -INFINITY;
    for (int j = 0; j < 64; ++j) M = fmaxf(M, red[t][j]);
    red[t][64] = M;
  }
  lds_barrier();
  const float M = red[h][64];
  float ew[2], sum = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sp = g + 64 * i;
    ew[i] = (sp < S && ml[i].x != -INFINITY) ? __expf(ml[i].x - M) : 0.f;
    sum = fmaf(ew[i], ml[i].y, sum);
  }
  red[h][g] = sum;
  lds_barrier();
  if (t < 4) {
    float L = 0.f;
    for (int j = 0; j < 64; ++j) L += red[t][j];
    red[t][64] = (h0 + t < Hq && L > 0.f) ? 1.f / L : 0.f;
  }
  lds_barrier();
  const float inv = red[h][64];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sp = g + 64 * i;
    if (sp < S) wt[h][sp] = ew[i] * inv;
  }
  lds_barrier();
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int sp = q + 16 * i;
    if (sp < S)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fmaf(wt[r][sp], v[i][r], acc[r]);
  }
  part[q][e] = acc;
  lds_barrier();
  if (t < 16) {
    v4f tot = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) tot += part[j][t];
    const int vcol = 16 * (tile % tiles) + t;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (h0 + r < Hq) out[((int64_t)b * Hq + h0 + r) * Dv + vcol] = tot[r];
  }
  // the count of invalid indices (stand-alone attention), read last
  if (part_bad != nullptr && quad == 0 && t < 64) {
    uint32_t nb = 0;
    for (int sp = t; sp < S; sp += 64) nb += (uint32_t)part_bad[(int64_t)b * S + sp];
    nb = wave_sum_u32(nb);
    if (t == 0) stats[b].bad_indices = (int32_t)nb;
  }
}

hipError_t launch_combine_wide(const AttnArgs& at, const int32_t* part_bad, RowStats* stats, float* out,
                               int B, hipStream_t s, KTimer t) {
  if (!at.frag || at.S > kMaxWideSplits) return hipErrorInvalidValue;
  const int quads = (at.Hq + 15) / 16 * (at.Dv / 16) * 4;
  return launch_timed(k_combine_wide, dim3(quads, B), dim3(kCombWideBlock), 0, s, t, at.part_ml, at.part_o, at.S,
                      at.Hq, at.Dv, part_bad, stats, out);
}

constexpr int kCombBlock = 64;

// out[b][h][v] = sum_s w_s o_s[h][v] with w_s = e^(m_s - M) / sum_s e^(m_s - M) l_s,
// M = max_s m_s, splits summed in index order. FRAG: partials in the matrix-core
// accumulator order (4 heads per 16-byte element, see AttnMfma); otherwise
// row-major [head][value]. Each workgroup (one wave) first forms the split
// weights of every head, then combines 64 elements.
template <bool FRAG>
__global__ __launch_bounds__(kCombBlock) void k_combine(AttnArgs at, const int32_t* __restrict__ part_bad,
                                                       RowStats* __restrict__ stats, float* __restrict__ out) {
  __shared__ __align__(16) float wsh[64][kMaxSplits];  // split weights per head (0 past S)
  const int b = blockIdx.y, lane = threadIdx.x;
  const int S = at.S, Hq = at.Hq, Dv = at.Dv;
  const int HP = FRAG ? (Hq + 15) / 16 * 16 : Hq;
  // Every load is issued before any arithmetic: first the (max, sum) pairs this lane
  // turns into weights, then the partial outputs this lane combines (they do not
  // depend on the weights), so the whole pass waits for one memory round trip.
  const int64_t split_stride = (int64_t)HP * Dv;
  const float* po = at.part_o + (int64_t)b * S * split_stride;
  const int h = lane < Hq ? lane : Hq - 1;
  float2 ml[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int sc = s < S ? s : S - 1;
    ml[s] = at.part_ml[((int64_t)b * S + sc) * Hq + h];
  }
  const int nel = FRAG ? HP * Dv / 4 : Hq * Dv;           // 16-byte (FRAG) or 4-byte elements
  const int el = blockIdx.x * kCombBlock + lane;
  const int elc = el < nel ? el : nel - 1;
  v4f part[FRAG ? kMaxSplits : 1];
  float partf[FRAG ? 1 : kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int sc = s < S ? s : S - 1;  // weight 0 past S
    if (FRAG) part[FRAG ? s : 0] = *(const v4f*)(po + sc * split_stride + (int64_t)elc * 4);
    else partf[FRAG ? 0 : s] = po[sc * split_stride + elc];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic below
  {
    // lane h forms the weights of head h over the splits (no cross-lane work)
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) M = fmaxf(M, s < S ? ml[s].x : -INFINITY);
    float e[kMaxSplits], den = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      e[s] = (s < S && ml[s].x != -INFINITY) ? __expf(ml[s].x - M) : 0.f;
      den = fmaf(e[s], ml[s].y, den);
    }
    const float inv = (lane < Hq && den > 0.f) ? 1.f / den : 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; s += 4)
      *(v4f*)&wsh[lane][s] = v4f{e[s] * inv, e[s + 1] * inv, e[s + 2] * inv, e[s + 3] * inv};
  }
  lds_barrier();
  // the count of invalid indices (stand-alone attention) is read last, so its wait
  // does not hold up the combine
  const bool count_bad = part_bad != nullptr && blockIdx.x == 0;
  if (el < nel && FRAG) {
    const int tiles = Dv / 16;
    const int tile = el >> 6, l = el & 63;
    const int h0 = 16 * (tile / tiles) + 4 * (l >> 4), v = 16 * (tile % tiles) + (l & 15);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v4f* wrow = reinterpret_cast<const v4f*>(wsh[h0 + r]);
#pragma unroll
      for (int s4 = 0; s4 < kMaxSplits / 4; ++s4) {
        const v4f w = wrow[s4];
        acc[r] = fmaf(w[0], part[FRAG ? 4 * s4 : 0][r], acc[r]);
        acc[r] = fmaf(w[1], part[FRAG ? 4 * s4 + 1 : 0][r], acc[r]);
        acc[r] = fmaf(w[2], part[FRAG ? 4 * s4 + 2 : 0][r], acc[r]);
        acc[r] = fmaf(w[3], part[FRAG ? 4 * s4 + 3 : 0][r], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (h0 + r < Hq) out[((int64_t)b * Hq + h0 + r) * Dv + v] = acc[r];
  } else if (el < nel) {
    const int hh = el / Dv;
    const v4f* wrow = reinterpret_cast<const v4f*>(wsh[hh]);
    float acc = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < kMaxSplits / 4; ++s4) {
      const v4f w = wrow[s4];
      acc = fmaf(w[0], partf[FRAG ? 0 : 4 * s4], acc);
      acc = fmaf(w[1], partf[FRAG ? 0 : 4 * s4 + 1], acc);
      acc = fmaf(w[2], partf[FRAG ? 0 : 4 * s4 + 2], acc);
      acc = fmaf(w[3], partf[FRAG ? 0 : 4 * s4 + 3], acc);
    }
    out[(int64_t)b * Hq * Dv + el] = acc;
  }
  if (count_bad) {
    const uint32_t nb = wave_sum_u32(lane < S ? (uint32_t)part_bad[(int64_t)b * S + lane] : 0u);
    if (lane == 0) stats[b].bad_indices = (int32_t)nb;
  }
}

hipError_t launch_combine(const AttnArgs& at, const int32_t* part_bad, RowStats* stats, float* out,
                          int B, hipStream_t s, KTimer t) {
  if (at.frag) {
    const int hp = (at.Hq + 15) / 16 * 16;
    const int grid = (hp * at.Dv / 4 + kCombBlock - 1) / kCombBlock;
    return launch_timed(k_combine<true>, dim3(grid, B), dim3(kCombBlock), 0, s, t, at, part_bad, stats, out);
  }
  const int grid = (at.Hq * at.Dv + kCombBlock - 1) / kCombBlock;
  return launch_timed(k_combine<false>, dim3(grid, B), dim3(kCombBlock), 0, s, t, at, part_bad, stats, out);
}

}  // namespace dsa

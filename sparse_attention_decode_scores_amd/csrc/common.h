// Device-side building blocks shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kMaxBatch = 16;
constexpr int kCandCap = 8192;         // candidate keys per row kept by the chunk pass
constexpr int kMaxChunks = 256;
constexpr int kMaxSplits = 32;         // attention splits per row (vector-ALU attention)
constexpr int kMaxWideSplits = 128;    // attention splits per row (matrix-core attention)
constexpr int kMaxRankBlocks = 128;
constexpr int kMaxSplitRows = 128;     // selected rows one attention split may take
// Rows of a batch share one launch: their splits together aim at one workgroup per
// compute unit of the chip (256 on gfx950). A constant, not the device's count, so
// that the split of the sum, and with it every rounding, is the same on any device.
constexpr int kSplitGrid = 256;
// Paged caches: a pool of pages of kPageSize positions each (a 1,048,576-token pool
// held in 4,096 pages), and a sequence's page table mapping its logical page j
// (positions 256j .. 256j + 255) to a pool page.
constexpr int kPageSize = 256;
constexpr int kPageShift = 8;

// Pool row of logical position pos through the page table; entries outside
// [0, pool_pages) are clamped into the pool, so a bad table never reads past it.
__device__ __forceinline__ uint32_t page_row(const int32_t* __restrict__ pages, int pool_pages, int64_t pos) {
  int32_t e = pages[pos >> kPageShift];
  e = e < 0 ? 0 : (e >= pool_pages ? pool_pages - 1 : e);
  return (uint32_t)e * (uint32_t)kPageSize + (uint32_t)(pos & (kPageSize - 1));
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Storage slot of entry u of a row's candidate union (kCandCap entries per row).
// The selection kernel's thread t (of 512) holds entries 16t .. 16t + 15 and reads
// them as eight 16-byte pieces; piece j of every thread lies in one contiguous run,
// so each of those loads is fully coalesced: entry 16t + 2j + e sits at slot
// 1024j + 2t + e.
__host__ __device__ __forceinline__ int cand_slot(int u) {
  return ((u >> 1) & 7) * 1024 + (u >> 4) * 2 + (u & 1);
}

// One chunk's candidate list: entries u0 .. u0 + m - 1 of its row's union.
struct CandOut {
  uint64_t* row;  // the row's kCandCap slots
  int u0;
  __device__ __forceinline__ void put(int i, uint64_t key) const { row[cand_slot(u0 + i)] = key; }
};

// Per-row lengths passed by value (kernel arguments are captured by HIP graphs).
struct RowLens {
  int32_t n[kMaxBatch];
};

// Per-row record written by the selection kernels (same layout as dsa_row_stats).
struct RowStats {
  int32_t path, reason, selected, kth_score, candidates, tied_at_kth, bad_indices, reserved;
};

// Order-preserving map of an int32 score onto uint32.
__device__ __forceinline__ uint32_t score_bits(int32_t s) { return (uint32_t)s ^ 0x80000000u; }

// A position's ordering key: score first, then the complement of the position so
// that, for equal scores, the lower position has the larger key. Larger key =
// earlier in the output. Keys of distinct positions are distinct, and every real
// key is >= 2^31, so 0 stands for "no position".
__device__ __forceinline__ uint64_t make_key(int32_t score, uint32_t pos) {
  return ((uint64_t)score_bits(score) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}
__device__ __forceinline__ uint32_t key_pos(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }
__device__ __forceinline__ uint32_t key_ubits(uint64_t key) { return (uint32_t)(key >> 32); }
__device__ __forceinline__ int32_t key_score(uint64_t key) {
  return (int32_t)(key_ubits(key) ^ 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Global-memory views for code in a called (not inlined) function, which sees
// generic pointers: accesses through them take the flat path, which is slower and
// also counts against the LDS wait counter.
typedef const __attribute__((address_space(1))) int32_t* GlobalI32;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) i32x4* GlobalI32x4;
__device__ __forceinline__ GlobalI32 global_view(const int32_t* p) { return (GlobalI32)p; }
// A 64-bit value known to be the same in every lane, in scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Workgroup barrier for LDS communication only: waits for this wave's LDS
// operations, not for its outstanding global loads and stores (a full
// __syncthreads() also drains those, a memory round trip when stores are in
// flight). Use __syncthreads() where waves exchange data through global memory.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// The wave's index in the workgroup, as a scalar (uniform) value, so loops and
// branches on it stay uniform control flow.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// ---- wave primitives on the DPP datapath (VALU-speed lane exchange; the ds_
// shuffle path costs an LDS round trip per step).
namespace dpp {
constexpr int kQuadXor1 = 0xB1;      // quad_perm 1,0,3,2
constexpr int kQuadXor2 = 0x4E;      // quad_perm 2,3,0,1
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowMirror = 0x140, kRowHalfMirror = 0x141;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
}  // namespace dpp

// Reduction of a 32-bit value over the wave; every lane gets the result.
// Within each 16-lane row by DPP, then across the four rows through readlane.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kQuadXor1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kQuadXor2, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kRowHalfMirror, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kRowMirror, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}
// The same over each 32-lane half of the wave: lanes 0..31 get the reduction of
// lanes 0..31, lanes 32..63 that of lanes 32..63.
template <class Op>
__device__ __forceinline__ uint32_t half_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kQuadXor1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kQuadXor2, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kRowHalfMirror, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, dpp::kRowMirror, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
  return lane_id() < 32 ? op(r0, r1) : op(r2, r3);
}
__device__ __forceinline__ float half_reduce_max_f(float v) {
  return __uint_as_float(half_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float half_reduce_sum_f(float v) {
  return __uint_as_float(half_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_maxr_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint64_t wave_maxr_u64(uint64_t v) {
  // the high word decides; the low word only among lanes holding the top high word
  const uint32_t hi = wave_maxr_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_maxr_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float wave_reduce_max_f(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_reduce_sum_f(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// a * b + c on the low 24 bits of a and b (signed), one v_mad_i32_i24.
__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowShr1, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowShr2, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowShr4, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowShr8, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowBcast15, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, dpp::kRowBcast31, 0xC, 0xF, false);
  return v;
}

// Exclusive prefix sum over the block (thread order); *total gets the block sum.
// `part` is LDS scratch of BLOCK/64 words. Two barriers.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* part, uint32_t* total) {
  const uint32_t incl = wave_incl_scan_u32(v);
  const uint32_t wtot = __builtin_amdgcn_readlane((int)incl, 63);
  lds_barrier();  // previous users of `part` are done
  if (lane_id() == 0) part[wave_id()] = wtot;
  lds_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w) {
    const uint32_t s = part[w];
    before += w < wave_id() ? s : 0u;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// LDS state of the radix selection below.
constexpr int kRadixBits = 11;
constexpr int kRadixBins = 1 << kRadixBits;
struct RadixSmem {
  uint32_t hist[2][kRadixBins];  // alternate passes; each pass leaves its buffer zeroed
  uint32_t part[16];
  uint32_t digit, above, inbin;
  uint32_t tdigit[2], tabove[2], tinbin[2];  // block_narrow_first: one record per target
};

// Zeroes both histogram buffers; call once before the first block_select_range
// (early, so it overlaps other work), followed by any barrier.
template <int BLOCK>
__device__ __forceinline__ void radix_clear(RadixSmem& sm) {
  for (int i = threadIdx.x; i < 2 * kRadixBins; i += BLOCK) (&sm.hist[0][0])[i] = 0;
}

// block_excl_scan_u32 without its first barrier: for callers whose last
// barrier already separates every earlier use of `part`. One barrier.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_excl_scan_fresh_u32(uint32_t v, uint32_t* part, uint32_t* total) {
  const uint32_t incl = wave_incl_scan_u32(v);
  const uint32_t wtot = __builtin_amdgcn_readlane((int)incl, 63);
  if (lane_id() == 0) part[wave_id()] = wtot;
  lds_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w) {
    const uint32_t s = part[w];
    before += w < wave_id() ? s : 0u;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// Result of block_narrow: the rank-th largest value lies in [binlo, binhi], which
// holds `inbin` values; `above` values are larger than binhi.
struct RadixBin {
  uint32_t binlo, binhi, above, inbin;
};

// Score-level radix narrowing. `each(f)` calls f(v) for every value this thread
// contributes; lo and hi are the smallest and largest of all n contributed values.
// The digits are 11-bit slices of v - lo, most significant first, over the bit
// length of hi - lo: each pass spreads the values over up to 2048 bins (values
// crowding a narrow band still spread out; LDS atomics on one bin serialise) and
// keeps the bin that holds the rank-th largest value (1 <= rank <= n). Passes stop
// once that bin holds at most `cap` values, or is a single value (a range of 2^21
// takes two passes). Three barriers per pass. Every thread of the block calls it
// and gets the same result; each pass leaves its histogram buffer zeroed.
template <int BLOCK, class Each>
__device__ __forceinline__ RadixBin block_narrow(Each each, uint32_t lo, uint32_t hi, uint32_t rank, uint32_t n,
                                                 uint32_t cap, RadixSmem& sm) {
  static_assert(kRadixBins % BLOCK == 0, "bins per thread");
  constexpr int BPT = kRadixBins / BLOCK;
  const int tid = threadIdx.x;
  const uint32_t range = hi - lo;
  if (range == 0) return RadixBin{hi, hi, 0u, n};  // every value is equal
  if (n <= cap) return RadixBin{lo, hi, 0u, n};    // the whole range is one bin
  int shift = 32 - __clz(range);  // low bits of v - lo still undecided
  uint32_t prefix = 0;            // decided high bits of v - lo
  uint32_t above = 0, inbin = n;
  uint32_t need = rank;
  int buf = 0;
  bool first = true;
  while (shift > 0 && inbin > cap) {
    const int nshift = shift > kRadixBits ? shift - kRadixBits : 0;
    uint32_t* hist = sm.hist[buf];
    if (first) {  // every value is in range: no prefix to match (and shift may be 32)
      each([&](uint32_t v) { atomicAdd(&hist[((v - lo) >> nshift) & (kRadixBins - 1)], 1u); });
    } else {  // shift < 32 from the second pass on
      each([&](uint32_t v) {
        const uint32_t off = v - lo;
        if ((off >> shift) == prefix) atomicAdd(&hist[(off >> nshift) & (kRadixBins - 1)], 1u);
      });
    }
    first = false;
    lds_barrier();
    uint32_t h[BPT], own = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      h[j] = hist[tid * BPT + j];
      hist[tid * BPT + j] = 0;  // only this thread reads these bins
      own += h[j];
    }
    uint32_t total;
    // the histogram barrier above separates every earlier reader of sm.part
    const uint32_t before = block_excl_scan_fresh_u32<BLOCK>(own, sm.part, &total);
    uint32_t ab = total - before - own;  // values in bins above this thread's bins
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (ab < need && need <= ab + h[j]) {
        sm.digit = tid * BPT + j;
        sm.above = ab;
        sm.inbin = h[j];
      }
      ab += h[j];
    }
    lds_barrier();
    const uint32_t d = sm.digit, ab2 = sm.above;
    inbin = sm.inbin;
    need -= ab2;
    above += ab2;
    prefix = (prefix << (shift - nshift)) | d;
    shift = nshift;
    buf ^= 1;
  }
  const uint32_t binlo = lo + (prefix << shift);  // shift <= 21 after a pass
  const uint32_t top = binlo + ((1u << shift) - 1u);  // values above hi do not occur
  return RadixBin{binlo, (top < binlo || top > hi) ? hi : top, above, inbin};
}

// The first radix pass of block_narrow for NT <= 2 ranks at once (one histogram
// serves every rank): out[t] is the bin that holds the need[t]-th largest value
// (1 <= need[t] <= n). Every thread gets the same results; the pass leaves its
// histogram buffer zeroed. Three barriers (none when every value is equal).
template <int BLOCK, int NT, class Each>
__device__ __forceinline__ void block_narrow_first(Each each, uint32_t lo, uint32_t hi, const uint32_t (&need)[NT],
                                                   uint32_t n, RadixSmem& sm, RadixBin (&out)[NT]) {
  static_assert(kRadixBins % BLOCK == 0 && NT >= 1 && NT <= 2, "bins per thread, targets");
  constexpr int BPT = kRadixBins / BLOCK;
  const int tid = threadIdx.x;
  const uint32_t range = hi - lo;
  if (range == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) out[t] = RadixBin{hi, hi, 0u, n};
    return;
  }
  const int shift = 32 - __clz(range);
  const int nshift = shift > kRadixBits ? shift - kRadixBits : 0;
  uint32_t* hist = sm.hist[0];
  each([&](uint32_t v) { atomicAdd(&hist[((v - lo) >> nshift) & (kRadixBins - 1)], 1u); });
  lds_barrier();
  uint32_t h[BPT], own = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    h[j] = hist[tid * BPT + j];
    hist[tid * BPT + j] = 0;
    own += h[j];
  }
  uint32_t total;
  const uint32_t before = block_excl_scan_fresh_u32<BLOCK>(own, sm.part, &total);
  uint32_t ab = total - before - own;
#pragma unroll
  for (int j = BPT - 1; j >= 0; --j) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (ab < need[t] && need[t] <= ab + h[j]) {
        sm.tdigit[t] = tid * BPT + j;
        sm.tabove[t] = ab;
        sm.tinbin[t] = h[j];
      }
    ab += h[j];
  }
  lds_barrier();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t binlo = lo + (sm.tdigit[t] << nshift);
    const uint32_t top = binlo + ((1u << nshift) - 1u);
    out[t] = RadixBin{binlo, (top < binlo || top > hi) ? hi : top, sm.tabove[t], sm.tinbin[t]};
  }
}

// Score-level radix selection: T, the rank-th largest value, and the number of
// values above T (block_narrow down to a single value).
template <int BLOCK, class Each>
__device__ __forceinline__ uint32_t block_select_range(Each each, uint32_t lo, uint32_t hi, int rank,
                                                       uint32_t* above_out, RadixSmem& sm) {
  const RadixBin r = block_narrow<BLOCK>(each, lo, hi, (uint32_t)rank, 0xFFFFFFFFu, 0u, sm);
  *above_out = r.above;
  return r.binlo;
}

// Block exchange of per-wave partial results: lane 0 of each wave stores its
// wave's values, then every thread reads all of them. Two barriers.
template <int BLOCK, int NV>
__device__ __forceinline__ void block_exchange(const uint32_t (&mine)[NV], uint32_t (*slots)[NV],
                                               uint32_t (&all)[BLOCK / 64][NV]) {
  lds_barrier();
  if (lane_id() == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) slots[wave_id()][i] = mine[i];
  lds_barrier();
#pragma unroll
  for (int w = 0; w < BLOCK / 64; ++w)
#pragma unroll
    for (int i = 0; i < NV; ++i) all[w][i] = slots[w][i];
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace dsa

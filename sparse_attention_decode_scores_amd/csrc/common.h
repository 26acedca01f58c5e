// Device-side building blocks shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kMaxBatch = 16;
constexpr int kBlock = 256;            // threads per workgroup for every kernel
constexpr int kWaves = kBlock / 64;
constexpr int kCandCap = 8192;         // candidate keys per row kept by the chunk pass
constexpr int kMaxChunks = 256;
constexpr int kMaxSplits = 32;         // attention splits per row
constexpr int kMaxRankBlocks = 128;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Per-row lengths passed by value (kernel arguments are captured by HIP graphs).
struct RowLens {
  int32_t n[kMaxBatch];
};

// Per-row record written by the selection kernels (same layout as dsa_row_stats).
struct RowStats {
  int32_t path, reason, selected, kth_score, candidates, tied_at_kth, bad_indices, reserved;
};

// A position's ordering key: score first (order-preserving map of int32 onto
// uint32), then the complement of the position so that, for equal scores, the
// lower position has the larger key. Larger key = earlier in the output. Keys of
// distinct positions are distinct, and every real key is >= 2^31, so 0 can stand
// for "no position".
__device__ __forceinline__ uint64_t make_key(int32_t score, uint32_t pos) {
  return ((uint64_t)((uint32_t)score ^ 0x80000000u) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}
__device__ __forceinline__ uint32_t key_pos(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }
__device__ __forceinline__ int32_t key_score(uint64_t key) {
  return (int32_t)((uint32_t)(key >> 32) ^ 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Block-wide reductions through a small LDS scratch (>= kWaves slots).
__device__ __forceinline__ int block_sum(int v, int* scratch) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += scratch[w];
  return t;
}
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* scratch) {
  v = wave_max_u64(v);
  __syncthreads();
  if (lane_id() == 0) scratch[wave_id()] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t = scratch[w] > t ? scratch[w] : t;
  return t;
}

// LDS state used by block_kth_largest.
struct SelectSmem {
  uint32_t hist[256];
  uint64_t red[kWaves];
  uint32_t digit, above, found;
  uint64_t result;
};

// Exact value of the rank-th largest of `count` distinct keys produced by
// key_at(i) (rank is 1-based, 1 <= rank <= count), by most-significant-digit
// radix selection: each pass histograms one byte of the keys that match the
// bytes fixed so far and fixes the byte holding the rank-th key. Leading bytes
// shared by the smallest and largest key are fixed without a pass; a pass
// that leaves a single matching key ends the search. Every thread of the
// block must call it; every thread gets the result.
template <typename KeyAt>
__device__ uint64_t block_kth_largest(int count, int rank, KeyAt key_at, SelectSmem& sm) {
  const int tid = threadIdx.x;
  // min and max key decide which leading bytes need no pass
  uint64_t lo = ~0ull, hi = 0;
  for (int i = tid; i < count; i += kBlock) {
    uint64_t k = key_at(i);
    lo = k < lo ? k : lo;
    hi = k > hi ? k : hi;
  }
  hi = block_max_u64(hi, sm.red);
  lo = ~block_max_u64(~lo, sm.red);
  if (rank == 1) return hi;
  if (rank == count) return lo;
  uint64_t diff = lo ^ hi;
  int byte = 7;
  while (byte > 0 && ((diff >> (8 * byte)) & 0xFF) == 0) --byte;
  uint64_t prefix = hi & (byte == 7 ? 0ull : (~0ull << (8 * (byte + 1))));
  int need = rank;
  for (;; --byte) {
    const uint64_t hmask = byte == 7 ? 0ull : (~0ull << (8 * (byte + 1)));
    for (int i = tid; i < 256; i += kBlock) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < count; i += kBlock) {
      uint64_t k = key_at(i);
      if (((k ^ prefix) & hmask) == 0) atomicAdd(&sm.hist[(k >> (8 * byte)) & 0xFF], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L owns digits 4L..4L+3; find d with above(d) < need <= above(d) + hist[d]
      const int L = tid;
      uint32_t h0 = sm.hist[4 * L], h1 = sm.hist[4 * L + 1], h2 = sm.hist[4 * L + 2],
               h3 = sm.hist[4 * L + 3];
      uint32_t own = h0 + h1 + h2 + h3;
      // inclusive scan from the top lane down: s = sum over lanes >= L
      uint32_t s = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_down(s, o);
        if (L + o < 64) s += t;
      }
      uint32_t above = s - own;  // keys in digits above 4L+3
      uint32_t hs[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < (uint32_t)need && (uint32_t)need <= above + hs[j]) {
          sm.digit = 4 * L + j;
          sm.above = above;
          sm.found = hs[j];
        }
        above += hs[j];
      }
    }
    __syncthreads();
    const uint32_t d = sm.digit, ab = sm.above, cnt = sm.found;
    __syncthreads();
    need -= (int)ab;
    prefix |= (uint64_t)d << (8 * byte);
    if (byte == 0) return prefix;
    if (cnt == 1) {
      // the only key that matches the fixed bytes is the answer
      const uint64_t m2 = ~0ull << (8 * byte);
      for (int i = tid; i < count; i += kBlock) {
        uint64_t k = key_at(i);
        if (((k ^ prefix) & m2) == 0) sm.result = k;
      }
      __syncthreads();
      uint64_t r = sm.result;
      __syncthreads();
      return r;
    }
  }
}

// Ordered stream compaction of a block: call with the same `round` sequence
// on every thread; returns the output slot of this thread's element when
// `keep` is true. `base` (LDS) carries the running count across rounds and must
// start at 0; counts[kWaves] is LDS scratch.
__device__ __forceinline__ int block_compact_slot(bool keep, int* counts, int* base) {
  const uint64_t bal = __ballot(keep);
  const int in_wave = __popcll(bal & lanemask_lt());
  __syncthreads();
  if (lane_id() == 0) counts[wave_id()] = __popcll(bal);
  __syncthreads();
  int before = *base;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave_id()) before += counts[w];
    total += counts[w];
  }
  __syncthreads();
  if (threadIdx.x == 0) *base += total;
  return before + in_wave;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace dsa

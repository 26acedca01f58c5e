// Internal launch interface between the C API (api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace dsa {

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Optional timing of one launch: the runtime stamps `start` with the dispatch's
// begin time and `stop` with its end time (the timestamps a kernel trace shows).
struct KTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};

// A kernel's dynamic-LDS limit (hipFuncSetAttribute), raised only when a launch needs
// more than was already allowed for that kernel on the current device, so a launch
// of a known size makes no attribute call (thread-safe).
hipError_t allow_lds(const void* fn, size_t lds);

template <class F, class... A>
inline hipError_t launch_timed(F fn, dim3 grid, dim3 block, size_t lds, hipStream_t s, KTimer t,
                               A... args) {
  if (t.start != nullptr || t.stop != nullptr)
    hipExtLaunchKernelGGL(fn, grid, block, (uint32_t)lds, s, t.start, t.stop, 0u, args...);
  else
    hipLaunchKernelGGL(fn, grid, block, lds, s, args...);
  return hipGetLastError();
}

// Per chunk of the one-row score pass: the lowest and highest score bits of its
// kept candidates (an empty chunk has lo > hi) and whether its list runs best
// first. The selection takes the union's range and order from these instead of
// reducing them over its keys.
struct ChunkSum {
  uint32_t lo, hi, ordered, pad;
};

struct ScoreArgs {
  // paged key cache: ik is the pool ([pool_pages * kPageSize][Di]) and pages[j] the
  // pool page of logical page j (kernels instantiated for paging only; first, so that
  // the one-row kernel's early argument reads share one line)
  const int32_t* pages;
  int pool_pages;
  const int8_t* iq;
  const int8_t* iw;
  const int8_t* ik;
  int32_t* scores;
  uint64_t* cand;  // [B][kCandCap] candidate union per row (entry c*m + i at cand_slot)
  uint64_t* xc;    // [B][G] best key left out of each chunk
  ChunkSum* sums;  // one-row kernel: [B][kMaxChunks] chunk summaries, or nullptr
  RowLens lens;
  int64_t N;       // row stride of scores
  int nmax;        // largest ctx_len: positions at or past it are never scored
  int b0, Bg;      // this launch scores rows b0 .. b0+Bg-1
  int Hi, Di;
  int P;           // positions per chunk (multiple of 64; of 32 for the one-row kernel)
  int G;           // chunks per row
  int m;           // candidates kept per chunk
};

// Geometry of chunk c of a row of n positions in units of 32 positions: with ilv,
// the chunk holds the row's units c, c + G, c + 2G, ...; otherwise the P / 32
// consecutive units from c·P / 32 (P a multiple of 32). Returns the chunk's unit
// count and sets *count to its valid positions (only its last unit can be cut
// short by the row's end).
__host__ __device__ inline int row_chunk_units(int n, int c, int G, int P, int ilv, int* count) {
  const int U = (n + 31) / 32;
  const int us = ilv ? 1 : P / 32, js = ilv ? G : 1;
  int units;
  if (ilv) units = c < U ? (U - c + G - 1) / G : 0;
  else units = U - c * us < us ? (U - c * us > 0 ? U - c * us : 0) : us;
  if (units == 0) {
    *count = 0;
    return 0;
  }
  const int64_t last = 32 * ((int64_t)c * us + (int64_t)(units - 1) * js);  // its last unit's first position
  *count = 32 * (units - 1) + (n - last < 32 ? (int)(n - last) : 32);
  return units;
}

// Query bytes (rows x padded heads x dims) one score launch stages; the launch
// planner keeps Bg * HP * DI at or below it, and Bg * HP at or below the block size.
constexpr int kScoreQBytes = 65536;

hipError_t launch_score(const ScoreArgs& a, int MT, int KT, bool cand, int grid, hipStream_t s,
                        KTimer t = {});
// One query row with candidates (the decode hot path): chunks of P = 32u positions,
// kScoreRowDepth units of 32 keys in flight per wave (2 or 3; two measured faster:
// three keep more requests queued without raising the key stream's rate).
hipError_t launch_score_row(const ScoreArgs& a, int MT, int KT, int grid, hipStream_t s, KTimer t = {});
constexpr int kScoreRowDepth = 2;
size_t score_row_lds_bytes(int P, bool paged);
int score_row_max_chunk();
int score_max_chunk();        // longest chunk the score kernel's candidate pass takes
int chunk_cand_max_chunk();   // the same for the stand-alone candidate kernel
size_t score_lds_bytes(int MT, int KT, int Bg, int P, bool cand, bool paged);

// Stand-alone candidate pass over scores already in memory.
struct CandArgs {
  const int32_t* scores;
  uint64_t* cand;
  uint64_t* xc;
  RowLens lens;
  int64_t N;
  int P, G, m;
};
hipError_t launch_chunk_candidates(const CandArgs& a, int B, hipStream_t s);

// Attention operands.
struct AttnArgs {
  const void* q;   // [B][Hq][Dk]
  const void* kv;  // [N][Dk]
  int64_t N;
  int Hq, Dk, Dv;
  float scale;
  float2* part_ml;  // [B][S][Hq] running max and sum of each split
  float* part_o;    // [B][S][Hp*Dv] unnormalised output of each split (layout per `frag`)
  int S;            // splits per row
  int frag;         // 1: part_o in matrix-core accumulator order with Hp = Hq rounded to 16
  // paged latent cache, or nullptr: kv is the pool ([pool_pages * kPageSize][Dk]) and
  // pages[j] the pool page of logical page j
  const int32_t* pages;
  int pool_pages;
  int lds_pages;  // selection kernel: table entries it stages in LDS (0: it reads the table in memory)
};

enum AttnKind { ATTN_NONE = 0, ATTN_MFMA_BF16 = 1, ATTN_GENERIC_F32 = 2, ATTN_GENERIC_BF16 = 3 };

// Selection stage (+ attention when kind != ATTN_NONE), one launch.
struct SelArgs {
  const int32_t* scores;
  const uint64_t* cand;
  const uint64_t* xc;
  const ChunkSum* sums;  // [B][kMaxChunks] from the one-row score pass (interleaved chunks), or nullptr
  int32_t* idx;        // [B][k]
  RowStats* stats;     // [B]
  RowLens lens;
  int64_t N;
  int k;
  int G, m;            // candidate layout
  int have_cand;       // the candidate pass's chunk length P, or 0 when it did not run (chunks too long)
  RowLens cand_valid;  // per row: union entries that hold a candidate (the rest are 0)
  int force;           // DSA_FLAG_FORCE_FALLBACK
  int R;               // ranking workgroups per row
};

struct AttnChoice {
  AttnKind kind;
  int hqt;   // 16-head tiles (MFMA path)
  int sb;    // rows staged per sub-block
  int nl;    // MFMA path: 16-byte row loads per thread per sub-block (bf16: 5 or 9; fp8: 3 or 5)
  int kv8;   // MFMA path: the latent cache holds FP8 E4M3 values (queries bf16)
};

// Attention input formats (the values of dsa_dtype).
enum AttnDtype { DT_F32 = 0, DT_BF16 = 1, DT_BF16_Q_E4M3_KV = 2 };

AttnChoice choose_attn(int dt, int Hq, int Dk, int Dv);
// LDS bytes of one workgroup of the selection kernel (largest of the two roles).
size_t select_lds_bytes(AttnChoice ch, int Hq, int Dk, int k);
hipError_t launch_select(const SelArgs& a, const AttnArgs& at, AttnChoice ch, int B, hipStream_t s,
                         KTimer t = {});
hipError_t launch_attend_idx(const int32_t* idx, int k, int32_t* part_bad, const AttnArgs& at,
                             AttnChoice ch, int B, hipStream_t s);
hipError_t launch_combine(const AttnArgs& at, const int32_t* part_bad, RowStats* stats, float* out,
                          int B, hipStream_t s, KTimer t = {});
// The combine for more than kMaxSplits splits (matrix-core partial layout).
hipError_t launch_combine_wide(const AttnArgs& at, const int32_t* part_bad, RowStats* stats, float* out,
                               int B, hipStream_t s, KTimer t = {});

}  // namespace dsa

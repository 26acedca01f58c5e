// Stage 1: the indexer score pass.
//
// score[b][s] = sum_h w[b][h] * max(0, sum_d q[b][h][d] * k[s][d])   (int8 in, int32 out)
//
// This is a dense contraction of the indexer heads against every cached key
// (heads x dim times dim x positions), so it runs on the int8 matrix cores:
// v_mfma_i32_32x32x32_i8 with the query heads as the A operand (32 heads per
// tile, held in registers or LDS) and 32 keys per tile streamed from HBM as the B
// operand with 16-byte loads, three tiles per wave in flight. The ReLU, the per-head weight and the sum over heads
// are applied to the accumulators in registers; one cross-lane add finishes the
// head sum. The key cache is read exactly once per launch.
//
// With candidates enabled, each workgroup owns one contiguous chunk of positions
// and, after scoring it, keeps the chunk's m best keys (and the best key it
// drops) for the selection stage: the "scans that narrow the candidates" of the
// ds4 glm53-m3ultra branch post (2026-09-09 "rising" page, long-context paragraph).
#include "chunk_select.h"
#include "kernels.h"

namespace dsa {

constexpr int kScoreBlock = 512;
constexpr int kScoreWaves = kScoreBlock / 64;
static_assert(kScoreQBytes % (16 * kScoreBlock) == 0, "query staging slots");

namespace {

// Key fragment of the B operand: lane l holds 16 consecutive dims of key
// (64*tile + 32*t + (l & 31)) of the chunk, starting at dim 32*kt + 16*(l >> 5).
// Raw buffer loads against a resource that covers exactly the chunk's valid keys:
// always issued (so the compiler's wait counts stay exact), zero past the end
// without touching memory.
template <int KT>
__device__ __forceinline__ void load_keys(v4i (&kf)[2][KT], __amdgpu_buffer_rsrc_t rs, int tile) {
  const int lane = lane_id();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int off = (64 * tile + 32 * t + (lane & 31)) * (32 * KT) + 16 * (lane >> 5);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      kf[t][kt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * kt, 0, 0));
  }
}

}  // namespace

template <int MT, int KT, bool CAND, bool ONE>
__global__ __launch_bounds__(kScoreBlock) void k_score(ScoreArgs a) {
  constexpr int HP = 32 * MT;  // heads padded to whole tiles (padding has q = 0, w = 0)
  constexpr int DI = 32 * KT;
  extern __shared__ __align__(16) uint8_t smem[];
  using Smem = ChunkSmem<kScoreBlock>;
  Smem& csm = *reinterpret_cast<Smem*>(smem);
  int8_t* qs = reinterpret_cast<int8_t*>(smem + align16(sizeof(Smem)));       // [Bg][HP][DI]
  int8_t* wsm = qs + a.Bg * HP * DI;                                           // [Bg][HP]
  int32_t* sc = reinterpret_cast<int32_t*>(wsm + a.Bg * HP);                   // [Bg][P]
  uint32_t* hist = reinterpret_cast<uint32_t*>(sc + a.Bg * a.P);              // [Bg][kHistBins]
  using CandSmem = BlockCandSmem<kScoreBlock>;
  CandSmem& bsm = *reinterpret_cast<CandSmem*>(hist + a.Bg * kHistBins);
  int* fallback = reinterpret_cast<int*>(&bsm + 1);                             // [Bg]

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int c = blockIdx.x;
  DSA_TRACE_BEGIN();
  DSA_MARK(0, 0);
  const int64_t cbeg = (int64_t)c * a.P;
  const int64_t clen64 = (int64_t)a.nmax - cbeg;
  const int clen = clen64 > a.P ? a.P : (int)(clen64 > 0 ? clen64 : 0);
  const int npairs = (clen + 63) >> 6;

  // Requests go out in this order: this launch's query heads and weights (into
  // registers), then the first three key tiles of every wave (a whole chunk of up
  // to 1,536 positions), whose latency then overlaps the query staging; each tile
  // buffer is refilled as soon as it is consumed. Every load is unconditional
  // (clamped addresses; padding is zeroed when stored), so no register copy has
  // to wait for a load that is still in flight.
  constexpr int kQPer = ONE ? (MT * KT + 7) / 8 : kScoreQBytes / 16 / kScoreBlock;
  const int nq = a.Bg * HP * (DI / 16);
  v4i qv[kQPer];
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    int i = tid + kScoreBlock * j;
    i = i < nq ? i : nq - 1;
    const int bb = i / (HP * (DI / 16));
    const int rem = i - bb * (HP * (DI / 16));
    int h = rem / (DI / 16);
    const int part = rem - h * (DI / 16);
    h = h < a.Hi ? h : a.Hi - 1;
    qv[j] = *(const v4i*)(a.iq + ((int64_t)(a.b0 + bb) * a.Hi + h) * DI + 16 * part);
  }
  const int wi = tid < a.Bg * HP ? tid : a.Bg * HP - 1;
  const int wh = wi % HP < a.Hi ? wi % HP : a.Hi - 1;
  const int8_t wv = a.iw[(int64_t)(a.b0 + wi / HP) * a.Hi + wh];

  // buffer resource word 3 for gfx9 raw buffers: 32-bit data format, no swizzle
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(a.ik + cbeg * DI), (short)0, clen * DI, 0x00020000);
  v4i kb0[2][KT], kb1[2][KT], kb2[2][KT];
  load_keys<KT>(kb0, rs, wave);
  load_keys<KT>(kb1, rs, wave + kScoreWaves);
  load_keys<KT>(kb2, rs, wave + 2 * kScoreWaves);

  if (CAND) {
    radix_clear<kScoreBlock>(csm.radix);
    for (int i = tid; i < a.Bg * kHistBins; i += kScoreBlock) hist[i] = 0;
  }
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int i = tid + kScoreBlock * j;
    const int h = (i % (HP * (DI / 16))) / (DI / 16);
    if (i < nq) *(v4i*)(qs + 16 * i) = h < a.Hi ? qv[j] : v4i{0, 0, 0, 0};
  }
  if (tid < a.Bg * HP) wsm[tid] = tid % HP < a.Hi ? wv : (int8_t)0;
  lds_barrier();

  // A fragments and weights of a single row stay in registers for the whole chunk.
  v4i qreg[ONE ? MT : 1][ONE ? KT : 1];
  int wreg[ONE ? MT : 1][ONE ? 16 : 1];
  if (ONE) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        qreg[ONE ? mt : 0][ONE ? kt : 0] =
            *(const v4i*)(qs + (32 * mt + (lane & 31)) * DI + 32 * kt + 16 * (lane >> 5));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int wd = *(const int*)(wsm + 32 * mt + 8 * g + 4 * (lane >> 5));
#pragma unroll
        for (int j = 0; j < 4; ++j) wreg[ONE ? mt : 0][ONE ? 4 * g + j : 0] = (int)(int8_t)(wd >> (8 * j));
      }
    }
  }

  // Scores of 64 positions (tile tp) from the key fragments `cur`, which are then
  // refilled with tile tp + 24. With candidates, scores stay in LDS until the chunk
  // is done (no global store in the loop: its completion would be waited for later).
  auto tile = [&](v4i(&cur)[2][KT], int tp) {
    const int64_t p0 = cbeg + 64 * tp;
    const int nb = ONE ? 1 : a.Bg;  // a compile-time trip count keeps the wait counts exact
    for (int bb = 0; bb < nb; ++bb) {
      const int8_t* qb = qs + bb * HP * DI;
      int half[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        v16i acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = v16i{};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const v4i qf = ONE ? qreg[ONE ? mt : 0][ONE ? kt : 0]
                               : *(const v4i*)(qb + (32 * mt + (lane & 31)) * DI + 32 * kt +
                                               16 * (lane >> 5));
            acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qf, cur[t][kt], acc[mt], 0, 0, 0);
          }
        }
        // accumulator r of lane l holds head 32*mt + 8*(r/4) + 4*(l/32) + r%4 of key l%32
        int part = 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            int wd = 0;
            if (!ONE) wd = *(const int*)(wsm + bb * HP + 32 * mt + 8 * g + 4 * (lane >> 5));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int w = ONE ? wreg[ONE ? mt : 0][ONE ? 4 * g + j : 0] : (int)(int8_t)(wd >> (8 * j));
              const int v = acc[mt][4 * g + j];
              part += __mul24(w, v > 0 ? v : 0);
            }
          }
        }
        part += __shfl_xor(part, 32);
        half[t] = part;
      }
      const int val = lane < 32 ? half[0] : half[1];
      const int64_t pos = p0 + lane;
      if (CAND) {
        sc[bb * a.P + (int)(pos - cbeg)] = val;
        if (pos < a.lens.n[a.b0 + bb]) atomicAdd(&hist[bb * kHistBins + score_bin(val)], 1u);
      } else if (pos < a.lens.n[a.b0 + bb]) {
        a.scores[(int64_t)(a.b0 + bb) * a.N + pos] = val;
      }
    }
    load_keys<KT>(cur, rs, tp + 3 * kScoreWaves);
  };

  DSA_MARK(0, 1);
  // three key buffers rotate by name (a register copy would wait for its load)
  for (int tp = wave; tp < npairs; tp += 3 * kScoreWaves) {
    tile(kb0, tp);
    if (tp + kScoreWaves >= npairs) break;
    tile(kb1, tp + kScoreWaves);
    if (tp + 2 * kScoreWaves >= npairs) break;
    tile(kb2, tp + 2 * kScoreWaves);
  }

  DSA_MARK(0, 2);
  if (CAND) {
    lds_barrier();
    DSA_MARK(0, 3);
    // the scores leave LDS first: the selection below waits for no memory
    // operation, so these stores complete underneath it. The key requests past
    // the chunk's end (buffer reads that return zeros) are drained before them,
    // so no later wait for those registers covers the stores.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt(0), expcnt and lgkmcnt untouched
    for (int bb = 0; bb < a.Bg; ++bb) {
      const int b = a.b0 + bb;
      const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      int32_t* dst = a.scores + (int64_t)b * a.N + cbeg;
      for (int i = tid; i < count; i += kScoreBlock) dst[i] = sc[bb * a.P + i];
    }
    if (ONE) {
      // one row: the whole block selects the chunk's candidates
      const int b = a.b0;
      const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      const bool ok = block_chunk_candidates<kScoreBlock>(sc, count, (uint32_t)cbeg, a.m, hist,
                                                          a.cand + ((int64_t)b * a.G + c) * a.m,
                                                          a.xc + (int64_t)b * a.G + c, bsm);
      if (tid == 0) fallback[0] = ok ? 0 : 1;
    } else {
      // several rows: wave w selects the candidates of rows w, w + 8, ...
      for (int bb = wave; bb < a.Bg; bb += kScoreWaves) {
        const int b = a.b0 + bb;
        const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
        const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
        const bool ok = wave_chunk_candidates(sc + bb * a.P, count, (uint32_t)cbeg, a.m, hist + bb * kHistBins,
                                              a.cand + ((int64_t)b * a.G + c) * a.m,
                                              a.xc + (int64_t)b * a.G + c, bsm.wstage[wave]);
        if (lane == 0) fallback[bb] = ok ? 0 : 1;
      }
    }
    DSA_MARK(0, 5);
    lds_barrier();
    for (int bb = 0; bb < a.Bg; ++bb) {  // rows whose threshold bin held too many keys
      if (!fallback[bb]) continue;
      const int b = a.b0 + bb;
      const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      chunk_candidates<kScoreBlock>(sc + bb * a.P, count, (uint32_t)cbeg, a.m,
                                    a.cand + ((int64_t)b * a.G + c) * a.m, a.xc + (int64_t)b * a.G + c,
                                    csm);
      lds_barrier();
    }
    DSA_MARK(0, 4);
  }
  DSA_TRACE_FLUSH();
}

int score_max_chunk() { return kChunkPerThread * kScoreBlock; }

size_t score_lds_bytes(int MT, int KT, int Bg, int P, bool cand) {
  return align16(sizeof(ChunkSmem<kScoreBlock>)) + (size_t)Bg * 32 * MT * 32 * KT + (size_t)Bg * 32 * MT +
         (cand ? (size_t)Bg * P * 4 + (size_t)Bg * kHistBins * 4 + sizeof(BlockCandSmem<kScoreBlock>) +
                     (size_t)Bg * 4
               : 0) +
         16;
}

template <int MT, int KT, bool CAND, bool ONE>
static hipError_t launch_score_t(const ScoreArgs& a, int grid, size_t lds, hipStream_t s, KTimer t) {
  auto fn = k_score<MT, KT, CAND, ONE>;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  return launch_timed(fn, dim3(grid), dim3(kScoreBlock), lds, s, t, a);
}

template <int MT, int KT>
static hipError_t launch_score_mk(const ScoreArgs& a, bool cand, int grid, size_t lds, hipStream_t s,
                                  KTimer t) {
  const bool one = a.Bg == 1;
  if (cand) return one ? launch_score_t<MT, KT, true, true>(a, grid, lds, s, t)
                       : launch_score_t<MT, KT, true, false>(a, grid, lds, s, t);
  return one ? launch_score_t<MT, KT, false, true>(a, grid, lds, s, t)
             : launch_score_t<MT, KT, false, false>(a, grid, lds, s, t);
}

hipError_t launch_score(const ScoreArgs& a, int MT, int KT, bool cand, int grid, hipStream_t s, KTimer t) {
  const size_t lds = score_lds_bytes(MT, KT, a.Bg, a.P, cand);
#define DSA_SCORE_CASE(M, K) \
  if (MT == M && KT == K) return launch_score_mk<M, K>(a, cand, grid, lds, s, t);
  DSA_SCORE_CASE(1, 1) DSA_SCORE_CASE(1, 2) DSA_SCORE_CASE(1, 3) DSA_SCORE_CASE(1, 4)
  DSA_SCORE_CASE(1, 5) DSA_SCORE_CASE(1, 6) DSA_SCORE_CASE(1, 7) DSA_SCORE_CASE(1, 8)
  DSA_SCORE_CASE(2, 1) DSA_SCORE_CASE(2, 2) DSA_SCORE_CASE(2, 3) DSA_SCORE_CASE(2, 4)
  DSA_SCORE_CASE(2, 5) DSA_SCORE_CASE(2, 6) DSA_SCORE_CASE(2, 7) DSA_SCORE_CASE(2, 8)
#undef DSA_SCORE_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa

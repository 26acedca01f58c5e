// Stage 1: the indexer score pass.
//
// score[b][s] = sum_h w[b][h] * max(0, sum_d q[b][h][d] * k[s][d])   (int8 in, int32 out)
//
// This is a dense contraction of the indexer heads against every cached key
// (heads x dim times dim x positions), so it runs on the int8 matrix cores:
// v_mfma_i32_32x32x32_i8 with the query heads as the A operand (32 heads per
// tile, held in registers or LDS) and 32 keys per tile streamed from HBM as the B
// operand with 16-byte loads. The ReLU, the per-head weight and the sum over heads
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

namespace {

// Key fragment of the B operand: lane l holds 16 consecutive dims of key
// (p0 + (l & 31)), starting at dim 32*kt + 16*(l >> 5).
template <int KT>
__device__ __forceinline__ void load_keys(v4i (&kf)[2][KT], const int8_t* __restrict__ ik,
                                          int64_t p0, int64_t last) {
  const int lane = lane_id();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int64_t pos = p0 + 32 * t + (lane & 31);
    pos = pos > last ? last : pos;
    const int8_t* row = ik + pos * (32 * KT) + 16 * (lane >> 5);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) kf[t][kt] = *(const v4i*)(row + 32 * kt);
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

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int c = blockIdx.x;
  DSA_MARK(0, 0);
  if (CAND) radix_clear<kScoreBlock>(csm.radix);

  for (int i = tid; i < a.Bg * HP * (DI / 16); i += kScoreBlock) {
    const int bb = i / (HP * (DI / 16));
    const int rem = i - bb * (HP * (DI / 16));
    const int h = rem / (DI / 16), part = rem - h * (DI / 16);
    v4i v = {0, 0, 0, 0};
    if (h < a.Hi) v = *(const v4i*)(a.iq + ((int64_t)(a.b0 + bb) * a.Hi + h) * DI + 16 * part);
    *(v4i*)(qs + (bb * HP + h) * DI + 16 * part) = v;
  }
  for (int i = tid; i < a.Bg * HP; i += kScoreBlock) {
    const int bb = i / HP, h = i - bb * HP;
    wsm[i] = h < a.Hi ? a.iw[(int64_t)(a.b0 + bb) * a.Hi + h] : (int8_t)0;
  }
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

  DSA_MARK(0, 1);
  const int64_t cbeg = (int64_t)c * a.P;
  const int64_t last = (int64_t)a.nmax - 1;
  const int64_t clen64 = (int64_t)a.nmax - cbeg;
  const int clen = clen64 > a.P ? a.P : (int)(clen64 > 0 ? clen64 : 0);
  const int npairs = (clen + 63) >> 6;

  v4i kcur[2][KT], knext[2][KT];
  if (wave < npairs) load_keys<KT>(kcur, a.ik, cbeg + 64 * wave, last);
  for (int tp = wave; tp < npairs; tp += kScoreWaves) {
    const int64_t p0 = cbeg + 64 * tp;
    if (tp + kScoreWaves < npairs) load_keys<KT>(knext, a.ik, p0 + 64 * kScoreWaves, last);
    for (int bb = 0; bb < a.Bg; ++bb) {
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
            acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qf, kcur[t][kt], acc[mt], 0, 0, 0);
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
      if (pos < a.lens.n[a.b0 + bb]) a.scores[(int64_t)(a.b0 + bb) * a.N + pos] = val;
      if (CAND) sc[bb * a.P + (int)(pos - cbeg)] = val;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) kcur[t][kt] = knext[t][kt];
  }

  DSA_MARK(0, 2);
  if (CAND) {
    lds_barrier();
    DSA_MARK(0, 3);
    for (int bb = 0; bb < a.Bg; ++bb) {
      const int b = a.b0 + bb;
      const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      chunk_candidates<kScoreBlock>(sc + bb * a.P, count, (uint32_t)cbeg, a.m,
                                    a.cand + ((int64_t)b * a.G + c) * a.m,
                                    a.xc + (int64_t)b * a.G + c, csm);
      lds_barrier();
    }
    DSA_MARK(0, 4);
  }
}

int score_max_chunk() { return kChunkPerThread * kScoreBlock; }

size_t score_lds_bytes(int MT, int KT, int Bg, int P, bool cand) {
  return align16(sizeof(ChunkSmem<kScoreBlock>)) + (size_t)Bg * 32 * MT * 32 * KT + (size_t)Bg * 32 * MT +
         (cand ? (size_t)Bg * P * 4 : 0) + 16;
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

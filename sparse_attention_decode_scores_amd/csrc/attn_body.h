// Attention over a list of selected positions, as one split of a split-K
// (flash-decoding style) reduction: the workgroup gathers its rows of the latent
// cache, computes the logits of every query head, keeps a running maximum and sum
// per head (online softmax) and an unnormalised output, and writes them as the
// split's partial result. A separate pass combines the splits in a fixed order.
//
// One shared latent row per position serves every head: the key is the whole row
// (latent + rope values), the value its first Dv values (MQA fold, Speed section of
// the GLM-5.3-Flash-Alis-MLX-4bit model card; latent KV cache of the
// glm53-tensorfold-spark README).
#pragma once

#include <math.h>

#include "kernels.h"

namespace dsa {

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Online-softmax bookkeeping of one sub-block: wave w updates heads w, w+4, ...;
// lane r is row r of the sub-block (sb <= 64). lg[h][r] holds scaled logits
// (-inf for absent rows) and is overwritten with exp(logit - new max).
__device__ __forceinline__ void softmax_update(float* lg, int sb, int nheads, float* mrun,
                                               float* lrun, float* alpha) {
  const int lane = lane_id();
  for (int h = wave_id(); h < nheads; h += kWaves) {
    const float v = lane < sb ? lg[h * sb + lane] : -INFINITY;
    const float mo = mrun[h];
    const float mn = fmaxf(mo, wave_max_f(v));
    const float p = v == -INFINITY ? 0.f : __expf(v - mn);
    if (lane < sb) lg[h * sb + lane] = p;
    const float sum = wave_sum_f(p);
    if (lane == 0) {
      const float a = mo == -INFINITY ? 0.f : __expf(mo - mn);
      lrun[h] = lrun[h] * a + sum;
      mrun[h] = mn;
      alpha[h] = a;
    }
  }
}

// bf16 inputs on the matrix cores (v_mfma_f32_16x16x32_bf16): logits = Q K^T with
// 16 heads per tile as the A operand and 16 staged rows per tile as the B
// operand; output = P V with P split into two bf16 terms (high part exact,
// remainder rounded) so the probabilities keep ~16 bits. Needs Dk % 32 == 0,
// Dv % 64 == 0, Dv <= 512, Hq <= 16 * HQT.
template <int HQT, int SB>
struct AttnMfma {
  static constexpr int HP = 16 * HQT;
  static constexpr int kMaxTilesPerWave = 8;  // Dv <= 512
  __host__ __device__ static int row_bytes(int Dk) { return Dk * 2 + 16; }
  __host__ __device__ static size_t lds_bytes(int Hq, int Dk) {
    (void)Hq;
    return align16((size_t)SB * row_bytes(Dk)) + (size_t)HP * SB * 4 + 3 * HP * 4;
  }

  template <typename PosAt>
  __device__ static void run(const AttnArgs& p, int b, int split, PosAt pos_at, int cnt,
                             uint8_t* work) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int Dk = p.Dk, Dv = p.Dv, KS = Dk >> 5, rb = row_bytes(Dk);
    const int ntw = Dv >> 6;  // 16-wide output tiles per wave
    uint8_t* rows = work;
    float* lg = reinterpret_cast<float*>(work + align16((size_t)SB * rb));
    float* mrun = lg + HP * SB;
    float* lrun = mrun + HP;
    float* alpha = lrun + HP;
    const __bf16* q = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.Hq * Dk;
    const uint8_t* kv = reinterpret_cast<const uint8_t*>(p.kv);

    v4f o[HQT][kMaxTilesPerWave];
#pragma unroll
    for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
      for (int j = 0; j < kMaxTilesPerWave; ++j) o[mt][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int h = tid; h < HP; h += kBlock) {
      mrun[h] = -INFINITY;
      lrun[h] = 0.f;
    }

    for (int s0 = 0; s0 < cnt; s0 += SB) {
      const int nr = cnt - s0 < SB ? cnt - s0 : SB;
      // gather the sub-block's rows with 16-byte loads
      const int cpr = Dk >> 3;
      for (int i = tid; i < SB * cpr; i += kBlock) {
        const int r = i / cpr, c = i - r * cpr;
        v4i v = {0, 0, 0, 0};
        if (r < nr) {
          const int64_t pos = pos_at(s0 + r);
          v = *(const v4i*)(kv + (pos * Dk + 8 * c) * 2);
        }
        *(v4i*)(rows + r * rb + 16 * c) = v;
      }
      __syncthreads();
      // logits: D[head][row], head = 16*mt + 4*(l/16) + r, row = 16*nt + l%16
      for (int nt = wave; nt < SB / 16; nt += kWaves) {
        v4f acc[HQT];
#pragma unroll
        for (int mt = 0; mt < HQT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
        const uint8_t* rrow = rows + (16 * nt + (lane & 15)) * rb + 16 * (lane >> 4);
        for (int kk = 0; kk < KS; ++kk) {
          const v8bf bfr = *(const v8bf*)(rrow + 64 * kk);
#pragma unroll
          for (int mt = 0; mt < HQT; ++mt) {
            const int h = 16 * mt + (lane & 15);
            v8bf afr = {};
            if (h < p.Hq) afr = *(const v8bf*)(q + (int64_t)h * Dk + 32 * kk + 8 * (lane >> 4));
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr, acc[mt], 0, 0, 0);
          }
        }
        const int row = 16 * nt + (lane & 15);
#pragma unroll
        for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            lg[(16 * mt + 4 * (lane >> 4) + r) * SB + row] =
                row < nr ? acc[mt][r] * p.scale : -INFINITY;
      }
      __syncthreads();
      softmax_update(lg, SB, HP, mrun, lrun, alpha);
      __syncthreads();
      // output: D[head][dv] += P[head][row] V[row][dv]
#pragma unroll
      for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = alpha[16 * mt + 4 * (lane >> 4) + r];
#pragma unroll
          for (int j = 0; j < kMaxTilesPerWave; ++j)
            if (j < ntw) o[mt][j][r] *= a;
        }
      for (int kk = 0; kk < SB / 32; ++kk) {
        v8bf ahi[HQT], alo[HQT];
#pragma unroll
        for (int mt = 0; mt < HQT; ++mt) {
          const float* pp = lg + (16 * mt + (lane & 15)) * SB + 32 * kk + 8 * (lane >> 4);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float pv = pp[t];
            const float hi = __uint_as_float(__float_as_uint(pv) & 0xFFFF0000u);
            ahi[mt][t] = (__bf16)hi;
            alo[mt][t] = (__bf16)(pv - hi);
          }
        }
#pragma unroll
        for (int j = 0; j < kMaxTilesPerWave; ++j) {
          if (j >= ntw) break;
          const int nt = wave + kWaves * j;
          const uint8_t* vb = rows + (32 * kk + 8 * (lane >> 4)) * rb + (16 * nt + (lane & 15)) * 2;
          v8bf bfr;
#pragma unroll
          for (int t = 0; t < 8; ++t) bfr[t] = *(const __bf16*)(vb + t * rb);
#pragma unroll
          for (int mt = 0; mt < HQT; ++mt) {
            o[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[mt], bfr, o[mt][j], 0, 0, 0);
            o[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[mt], bfr, o[mt][j], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }

    const int64_t pb = (int64_t)b * p.S + split;
    for (int h = tid; h < p.Hq; h += kBlock) p.part_ml[pb * p.Hq + h] = make_float2(mrun[h], lrun[h]);
#pragma unroll
    for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
      for (int j = 0; j < kMaxTilesPerWave; ++j) {
        if (j >= ntw) break;
        const int dv = 16 * (wave + kWaves * j) + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 16 * mt + 4 * (lane >> 4) + r;
          if (h < p.Hq) p.part_o[(pb * p.Hq + h) * Dv + dv] = o[mt][j][r];
        }
      }
  }
};

// Plain vector-ALU path for any small shape, fp32 or bf16 inputs widened to fp32
// in LDS. Needs Hq * Dv <= 4096 and Dk <= 512.
template <typename T>
struct AttnGeneric {
  static constexpr int SB = 32;
  static constexpr int kMaxPerThread = 16;
  __host__ __device__ static size_t lds_bytes(int Hq, int Dk) {
    return (size_t)SB * Dk * 4 + (size_t)Hq * Dk * 4 + (size_t)Hq * SB * 4 + 3 * (size_t)Hq * 4;
  }
  __device__ static float ld(const void* base, int64_t i) {
    if constexpr (sizeof(T) == 4) return reinterpret_cast<const float*>(base)[i];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  }

  template <typename PosAt>
  __device__ static void run(const AttnArgs& p, int b, int split, PosAt pos_at, int cnt,
                             uint8_t* work) {
    const int tid = threadIdx.x;
    const int Hq = p.Hq, Dk = p.Dk, Dv = p.Dv;
    float* rows = reinterpret_cast<float*>(work);
    float* qs = rows + SB * Dk;
    float* lg = qs + Hq * Dk;
    float* mrun = lg + Hq * SB;
    float* lrun = mrun + Hq;
    float* alpha = lrun + Hq;
    for (int i = tid; i < Hq * Dk; i += kBlock) qs[i] = ld(p.q, (int64_t)b * Hq * Dk + i);
    for (int h = tid; h < Hq; h += kBlock) {
      mrun[h] = -INFINITY;
      lrun[h] = 0.f;
    }
    float o[kMaxPerThread];
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) o[j] = 0.f;

    for (int s0 = 0; s0 < cnt; s0 += SB) {
      const int nr = cnt - s0 < SB ? cnt - s0 : SB;
      for (int i = tid; i < SB * Dk; i += kBlock) {
        const int r = i / Dk, d = i - r * Dk;
        rows[i] = r < nr ? ld(p.kv, pos_at(s0 + r) * Dk + d) : 0.f;
      }
      __syncthreads();
      for (int pr = tid; pr < Hq * SB; pr += kBlock) {
        const int h = pr / SB, r = pr - h * SB;
        float dot = 0.f;
        if (r < nr)
          for (int d = 0; d < Dk; ++d) dot = fmaf(qs[h * Dk + d], rows[r * Dk + d], dot);
        lg[pr] = r < nr ? dot * p.scale : -INFINITY;
      }
      __syncthreads();
      softmax_update(lg, SB, Hq, mrun, lrun, alpha);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kMaxPerThread; ++j) {
        const int pr = tid + kBlock * j;
        if (pr < Hq * Dv) {
          const int h = pr / Dv, dv = pr - h * Dv;
          float acc = o[j] * alpha[h];
          for (int r = 0; r < nr; ++r) acc = fmaf(lg[h * SB + r], rows[r * Dk + dv], acc);
          o[j] = acc;
        }
      }
      __syncthreads();
    }
    const int64_t pb = (int64_t)b * p.S + split;
    for (int h = tid; h < Hq; h += kBlock) p.part_ml[pb * Hq + h] = make_float2(mrun[h], lrun[h]);
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
      const int pr = tid + kBlock * j;
      if (pr < Hq * Dv) p.part_o[pb * Hq * Dv + pr] = o[j];
    }
  }
};

// Selection only (no attention role).
struct AttnNone {
  __host__ __device__ static size_t lds_bytes(int, int) { return 0; }
  template <typename PosAt>
  __device__ static void run(const AttnArgs&, int, int, PosAt, int, uint8_t*) {}
};

}  // namespace dsa

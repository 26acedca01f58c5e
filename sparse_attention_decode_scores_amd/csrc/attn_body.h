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

constexpr int kAttnBlock = 512;
constexpr int kAttnWaves = kAttnBlock / 64;

// Online-softmax bookkeeping of one sub-block: wave w updates heads w, w+8, ...;
// lane r is row r of the sub-block (sb <= 64). lg[h][r] holds scaled logits
// (-inf for absent rows) and is overwritten with exp(logit - new max).
__device__ __forceinline__ void softmax_update(float* lg, int sb, int nheads, float* mrun,
                                               float* lrun, float* alpha) {
  const int lane = lane_id();
  for (int h = wave_id(); h < nheads; h += kAttnWaves) {
    const float v = lane < sb ? lg[h * sb + lane] : -INFINITY;
    const float mo = mrun[h];
    const float mn = fmaxf(mo, wave_reduce_max_f(v));
    const float p = v == -INFINITY ? 0.f : __expf(v - mn);
    if (lane < sb) lg[h * sb + lane] = p;
    const float sum = wave_reduce_sum_f(p);
    if (lane == 0) {
      const float a = mo == -INFINITY ? 0.f : __expf(mo - mn);
      lrun[h] = lrun[h] * a + sum;
      mrun[h] = mn;
      alpha[h] = a;
    }
  }
}

// The same update for 32-row sub-blocks from partial logits: the logit of head
// h, row r is scale * sum over q < parts of lgp[(q * hp + h) * 32 + r] (summed in
// that order), -inf for rows whose bit in `live` is clear; lg receives the
// probabilities. Each wave takes two heads at once, one per 32-lane half.
__device__ __forceinline__ void softmax_update_parts32(const float* lgp, int parts, int hp, uint64_t live,
                                                       float scale, float* lg, int nheads, float* mrun,
                                                       float* lrun, float* alpha) {
  const int lane = lane_id(), r = lane & 31;
  const bool in = (live >> r) & 1ull;
  for (int h0 = wave_id(); h0 < nheads; h0 += 2 * kAttnWaves) {
    const int h = h0 + kAttnWaves * (lane >> 5);
    const bool hv = h < nheads;
    const int hc = hv ? h : h0;  // a present head (its result is discarded)
    const float mo = mrun[hc];
    float t = 0.f;
    for (int q = 0; q < parts; ++q) t += lgp[(q * hp + hc) * 32 + r];
    const float v = in && hv ? t * scale : -INFINITY;
    const float mn = fmaxf(mo, half_reduce_max_f(v));
    const float p = v == -INFINITY ? 0.f : __expf(v - mn);
    if (hv) lg[h * 32 + r] = p;
    const float sum = half_reduce_sum_f(p);
    if (r == 0 && hv) {
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
// Dv % 16 == 0, Dv <= 512, Hq <= 16 * HQT, (Dk / 8) * SB <= NL * block size. NL, the
// 16-byte row loads per thread per sub-block, is fitted to Dk by the caller: slots
// past the sub-block re-read a present row, so spare slots are spare address work
// on the latency-critical gather.
// KV8: the latent cache holds FP8 E4M3 (e4m3fn) values, one byte each, widened to
// bf16 as the gathered rows are staged (exact: every e4m3 value is a bf16 value), so
// the gather reads half the bytes and everything after the staging is unchanged.
// (FP8 KV storage: glm53-tensorfold-spark README, introduction, patch list.)
template <int HQT, int SB, int NL = 9, bool KV8 = false>
struct AttnMfma {
  static constexpr int HP = 16 * HQT;
  static constexpr int kKvBytes = KV8 ? 1 : 2;  // bytes per cached value in memory
  static constexpr int kLdsPerChunk = 16 / kKvBytes * 2;  // LDS bytes one 16-byte load stages
  static constexpr int kMaxTilesPerWave = 32 / kAttnWaves;  // Dv <= 512
  static constexpr int kMaxLoads = NL;                      // 16-byte loads per thread per sub-block
  static constexpr int kLogitBatch = HQT == 1 ? 6 : (HQT == 2 ? 4 : 2);  // k-steps loaded together
  static constexpr bool kQInLds = HQT == 1;                 // query heads staged in LDS
  static constexpr int kTiles = SB / 16;                    // 16-row tiles of a sub-block
  static constexpr int kParts = kAttnWaves / kTiles;        // waves per tile, each a share of the k-steps
  static_assert(SB == 32 && kAttnWaves % kTiles == 0, "32-row sub-blocks (the softmax takes one row per lane of a half-wave)");
  __host__ __device__ static int row_bytes(int Dk) { return Dk * 2 + 16; }
  __host__ __device__ static size_t q_bytes(int Dk) {
    return kQInLds ? align16((size_t)HP * row_bytes(Dk)) : 0;
  }
  __host__ __device__ static size_t lds_bytes(int Hq, int Dk) {
    (void)Hq;
    return q_bytes(Dk) + align16((size_t)SB * row_bytes(Dk)) + (size_t)HP * SB * 4 + 3 * HP * 4 +
           (size_t)kParts * HP * SB * 4;
  }

  // The row's query heads travel in two steps: load_q requests them into registers
  // (call it first, so the loads overlap other work) and store_q writes them to
  // LDS (zero rows for padded heads) before run; run's first barrier publishes them.
  static constexpr int kQPer = 4;  // 16 heads x at most 1,024 values, 16 bytes per slot
  struct QFrag {
    v4i v[kQInLds ? kQPer : 1];
    int rr[kMaxLoads], cc[kMaxLoads];  // gather slot j of this thread: row, 16-byte column
    int lo[kMaxLoads];                 // its LDS byte offset among the staged rows
  };
  __device__ __forceinline__ static QFrag load_q(const AttnArgs& p, int b) {
    QFrag f;
    {
      // gather slot j of this thread is chunk i = tid + 512 j of a sub-block: row
      // i / cpr, 16-byte column i % cpr of the cached row, stepped without dividing
      // (a divide by a runtime value costs dozens of instructions); worked out
      // here, before the positions are known
      const int cpr = p.Dk * kKvBytes / 16;
      const int step_r = kAttnBlock / cpr, step_c = kAttnBlock - step_r * cpr;
      int r = (int)threadIdx.x / cpr, c = (int)threadIdx.x - r * cpr;
#pragma unroll
      for (int j = 0; j < kMaxLoads; ++j) {
        f.rr[j] = r;
        f.cc[j] = c;
        f.lo[j] = r * row_bytes(p.Dk) + kLdsPerChunk * c;
        c += step_c;
        r += step_r;
        if (c >= cpr) {
          c -= cpr;
          ++r;
        }
      }
      // computed here, while the kernel waits for its first loads: the empty asm
      // keeps the compiler from recomputing them where they are used
#pragma unroll
      for (int j = 0; j < kMaxLoads; ++j) asm volatile("" : "+v"(f.rr[j]), "+v"(f.cc[j]), "+v"(f.lo[j]));
    }
    if (!kQInLds) return f;
    const int Dk = p.Dk, cpr = Dk >> 3;
    const uint8_t* q = reinterpret_cast<const uint8_t*>(p.q) + (int64_t)b * p.Hq * Dk * 2;
    const int step_h = kAttnBlock / cpr, step_c = kAttnBlock - step_h * cpr;
    int h = (int)threadIdx.x / cpr, c = (int)threadIdx.x - h * cpr;  // one divide, then steps
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {  // every slot loads a present value (clamped head)
      const int hc = h < p.Hq ? h : p.Hq - 1;
      f.v[kQInLds ? j : 0] = *(const v4i*)(q + ((int64_t)hc * Dk + 8 * c) * 2);
      c += step_c;
      h += step_h;
      if (c >= cpr) {
        c -= cpr;
        ++h;
      }
    }
    return f;
  }
  __device__ __forceinline__ static void store_q(const QFrag& f, const AttnArgs& p, uint8_t* work) {
    if (!kQInLds) return;
    const int Dk = p.Dk, rb = row_bytes(Dk), cpr = Dk >> 3;
    const int step_h = kAttnBlock / cpr, step_c = kAttnBlock - step_h * cpr;
    int h = (int)threadIdx.x / cpr, c = (int)threadIdx.x - h * cpr;  // one divide, then steps
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      if ((int)threadIdx.x + kAttnBlock * j < HP * cpr)
        *(v4i*)(work + h * rb + 16 * c) = h < p.Hq ? f.v[kQInLds ? j : 0] : v4i{0, 0, 0, 0};
      c += step_c;
      h += step_h;
      if (c >= cpr) {
        c -= cpr;
        ++h;
      }
    }
  }

  // LDS working set: [query heads (kQInLds)] [SB staged rows] [probabilities HP x SB]
  // [running max, sum, rescale per head] [partial logits kParts x HP x SB].
  struct Work {
    const uint8_t* qs;
    uint8_t* rows;
    float *lg, *mrun, *lrun, *alpha, *lgp;
  };
  __device__ __forceinline__ static Work work_of(const AttnArgs& p, uint8_t* work) {
    Work w;
    w.qs = work;
    w.rows = work + q_bytes(p.Dk);
    w.lg = reinterpret_cast<float*>(w.rows + align16((size_t)SB * row_bytes(p.Dk)));
    w.mrun = w.lg + HP * SB;
    w.lrun = w.mrun + HP;
    w.alpha = w.lrun + HP;
    w.lgp = w.alpha + HP;
    return w;
  }
  typedef v4f Acc[HQT][kMaxTilesPerWave];

  // The rows of one sub-block in flight: gather slot j of this thread holds the
  // 16-byte column qf.cc[j] of sub-block row qf.rr[j] (rows at or past nr re-read row
  // nr - 1: every load is issued, so the compiler's wait counts stay exact).
  struct Rows {
    v4i v[kMaxLoads];
  };
  template <typename PosAt>
  __device__ __forceinline__ static Rows gather(const AttnArgs& p, const QFrag& qf, PosAt pos_at, int nr) {
    const uint8_t* kv = reinterpret_cast<const uint8_t*>(p.kv);
    int32_t rp[kMaxLoads];
#pragma unroll
    for (int j = 0; j < kMaxLoads; ++j) rp[j] = (int32_t)pos_at(qf.rr[j] < nr ? qf.rr[j] : nr - 1);
    Rows r;
#pragma unroll
    for (int j = 0; j < kMaxLoads; ++j)
      r.v[j] = *(const v4i*)(kv + (int64_t)rp[j] * p.Dk * kKvBytes + 16 * qf.cc[j]);
    return r;
  }
  // Stores gathered rows (absent rows as zeros) and, with `with_q`, the query heads;
  // the next barrier publishes them.
  __device__ __forceinline__ static void put(const Rows& r, const QFrag& qf, const AttnArgs& p, int nr, bool with_q,
                             uint8_t* work) {
    const Work w = work_of(p, work);
    const int nch = SB * (p.Dk * kKvBytes / 16);  // nch <= kMaxLoads * block size
    if (with_q) store_q(qf, p, work);
#pragma unroll
    for (int j = 0; j < kMaxLoads; ++j)
      if ((int)threadIdx.x + kAttnBlock * j < nch) {
        const v4i v = qf.rr[j] < nr ? r.v[j] : v4i{0, 0, 0, 0};
        if constexpr (KV8) {
          // 16 e4m3 values -> 16 bf16 values (the hardware's conversion with scale 1:
          // exact, NaN codes to NaN), in order
          v4i lo, hi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[d], 1.0f, false);
            const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[d], 1.0f, true);
            const int ia = __builtin_bit_cast(int, a), ib = __builtin_bit_cast(int, b);
            if (d < 2) {
              lo[2 * d] = ia;
              lo[2 * d + 1] = ib;
            } else {
              hi[2 * d - 4] = ia;
              hi[2 * d - 3] = ib;
            }
          }
          *(v4i*)(w.rows + qf.lo[j]) = lo;
          *(v4i*)(w.rows + qf.lo[j] + 16) = hi;
        } else {
          *(v4i*)(w.rows + qf.lo[j]) = v;
        }
      }
  }
  __device__ __forceinline__ static void begin(const AttnArgs& p, uint8_t* work, Acc& o) {
    const Work w = work_of(p, work);
#pragma unroll
    for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
      for (int j = 0; j < kMaxTilesPerWave; ++j) o[mt][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int h = threadIdx.x; h < HP; h += kAttnBlock) {
      w.mrun[h] = -INFINITY;
      w.lrun[h] = 0.f;
    }
  }

  // One staged sub-block: row r takes part iff bit r of `live` is set. Logits on
  // the matrix cores, online-softmax update, then P V accumulated into o. With
  // `last`, no barrier follows (nothing overwrites the staged rows afterwards, and
  // finish reads only what the softmax barrier published).
  __device__ __forceinline__ static void sub_block(const AttnArgs& p, int b, uint64_t live, uint8_t* work, Acc& o,
                                   bool last) {
    const int lane = lane_id(), wave = wave_id();
    const int Dk = p.Dk, KS = Dk >> 5, rb = row_bytes(Dk), nt_all = p.Dv >> 4;
    const Work w = work_of(p, work);
    const __bf16* q = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.Hq * Dk;
    lds_barrier();
    // logits: D[head][row], head = 16*mt + 4*(l/16) + r, row = 16*nt + l%16. Wave w
    // takes row tile w % kTiles and the w / kTiles-th share of the k-steps (every
    // wave works; one wave per tile would chain all k-steps), and writes its
    // partial sums; the softmax adds the shares in a fixed order.
    {
      const int nt = wave % kTiles, kq = wave / kTiles;
      const int ks0 = KS * kq / kParts, ks1 = KS * (kq + 1) / kParts;
      v4f acc[HQT];
#pragma unroll
      for (int mt = 0; mt < HQT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
      const uint8_t* rrow = w.rows + (16 * nt + (lane & 15)) * rb + 16 * (lane >> 4);
      const int h_a = lane & 15;
      auto afrag = [&](int mt, int kk) {
        if (kQInLds) return *(const v8bf*)(w.qs + (16 * mt + h_a) * rb + 64 * kk + 16 * (lane >> 4));
        // heads past Hq read a present head (always issued) and are zeroed at use
        const int h = 16 * mt + h_a < p.Hq ? 16 * mt + h_a : p.Hq - 1;
        return *(const v8bf*)(q + (int64_t)h * Dk + 32 * kk + 8 * (lane >> 4));
      };
      // fragments of kLogitBatch k-steps are loaded before their matrix-core steps
      for (int k0 = ks0; k0 < ks1; k0 += kLogitBatch) {
        v8bf bfrag[kLogitBatch];
        v8bf afr[HQT][kLogitBatch];
#pragma unroll
        for (int t = 0; t < kLogitBatch; ++t) {
          if (k0 + t < ks1) {
            bfrag[t] = *(const v8bf*)(rrow + 64 * (k0 + t));
#pragma unroll
            for (int mt = 0; mt < HQT; ++mt) afr[mt][t] = afrag(mt, k0 + t);
          }
        }
#pragma unroll
        for (int t = 0; t < kLogitBatch; ++t) {
          if (k0 + t < ks1) {
#pragma unroll
            for (int mt = 0; mt < HQT; ++mt) {
              v8bf a = afr[mt][t];
              if (!kQInLds && 16 * mt + h_a >= p.Hq) a = v8bf{};
              acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfrag[t], acc[mt], 0, 0, 0);
            }
          }
        }
      }
      const int row = 16 * nt + (lane & 15);
#pragma unroll
      for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) w.lgp[(kq * HP + 16 * mt + 4 * (lane >> 4) + r) * SB + row] = acc[mt][r];
    }
    lds_barrier();
    softmax_update_parts32(w.lgp, kParts, HP, live, p.scale, w.lg, HP, w.mrun, w.lrun, w.alpha);
    lds_barrier();
    // output: D[head][dv] += P[head][row] V[row][dv]
#pragma unroll
    for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = w.alpha[16 * mt + 4 * (lane >> 4) + r];
#pragma unroll
        for (int j = 0; j < kMaxTilesPerWave; ++j)
          if (wave + kAttnWaves * j < nt_all) o[mt][j][r] *= a;
      }
    for (int kk = 0; kk < SB / 32; ++kk) {
      v8bf ahi[HQT], alo[HQT];
#pragma unroll
      for (int mt = 0; mt < HQT; ++mt) {
        const float* pp = w.lg + (16 * mt + (lane & 15)) * SB + 32 * kk + 8 * (lane >> 4);
        const v4f p0 = *(const v4f*)pp, p1 = *(const v4f*)(pp + 4);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float pv = t < 4 ? p0[t] : p1[t - 4];
          const float hi = __uint_as_float(__float_as_uint(pv) & 0xFFFF0000u);
          ahi[mt][t] = (__bf16)hi;
          alo[mt][t] = (__bf16)(pv - hi);
        }
      }
      // B fragment: V[rows 32*kk + 8*(l/16) + t][dv 16*nt + l%16], t < 8, read with two
      // transposing LDS loads: lane j of each 16-lane group names the 4-value chunk
      // (row base + j/4, columns 4*(j%4)..+3) and receives column j of the 4 rows.
      // Every tile's fragment is read before the first matrix-core step.
      const int tr_row = 32 * kk + 8 * (lane >> 4) + ((lane & 15) >> 2);
      const int tr_col = 4 * (lane & 3);
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s lds_v4s;
      typedef short v8s __attribute__((ext_vector_type(8)));
      v4s vr[kMaxTilesPerWave][2];
#pragma unroll
      for (int j = 0; j < kMaxTilesPerWave; ++j) {
        const int nt = wave + kAttnWaves * j;
        if (nt < nt_all) {
          const uint8_t* va = w.rows + tr_row * rb + (16 * nt + tr_col) * 2;
          vr[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(va));
          vr[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(va + 4 * rb));
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxTilesPerWave; ++j) {
        const int nt = wave + kAttnWaves * j;
        if (nt < nt_all) {
          const v8s both = __builtin_shufflevector(vr[j][0], vr[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
          const v8bf bfr = __builtin_bit_cast(v8bf, both);
#pragma unroll
          for (int mt = 0; mt < HQT; ++mt) {
            o[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[mt], bfr, o[mt][j], 0, 0, 0);
            o[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[mt], bfr, o[mt][j], 0, 0, 0);
          }
        }
      }
    }
    if (!last) lds_barrier();  // uniform
  }

  // The split's partial result: (max, sum) per head and the unnormalised output in
  // accumulator order: element ((mt * tiles + nt) * 64 + lane) * 4 + r is head
  // 16*mt + 4*(lane/16) + r, value 16*nt + lane%16 (one 16-byte store per tile).
  __device__ __forceinline__ static void finish(const AttnArgs& p, int b, int split, uint8_t* work, const Acc& o) {
    const int lane = lane_id(), wave = wave_id(), nt_all = p.Dv >> 4;
    const Work w = work_of(p, work);
    const int64_t pb = (int64_t)b * p.S + split;
    for (int h = threadIdx.x; h < p.Hq; h += kAttnBlock) p.part_ml[pb * p.Hq + h] = make_float2(w.mrun[h], w.lrun[h]);
    float* po = p.part_o + pb * HP * p.Dv;
#pragma unroll
    for (int mt = 0; mt < HQT; ++mt)
#pragma unroll
      for (int j = 0; j < kMaxTilesPerWave; ++j) {
        const int nt = wave + kAttnWaves * j;
        if (nt >= nt_all) break;
        *(v4f*)(po + ((int64_t)(mt * nt_all + nt) * 64 + lane) * 4) = o[mt][j];
      }
  }

  // Attention over cnt listed positions (pos_at(i), i < cnt) as split `split`: the
  // positions are staged SB at a time; the query fragments (load_q) are written to
  // LDS once the first sub-block's row loads are in flight. When a split has more
  // than one sub-block, the next one's rows are requested before this one's
  // products, so their latency hides behind them.
  template <typename PosAt>
  __device__ __forceinline__ static void run(const AttnArgs& p, int b, int split, PosAt pos_at, int cnt,
                             uint8_t* work, const QFrag& qf) {
    Acc o;
    begin(p, work, o);
    Rows r;
    if (cnt > 0) r = gather(p, qf, pos_at, cnt < SB ? cnt : SB);  // uniform
    for (int s0 = 0; s0 < cnt; s0 += SB) {
      const int nr = cnt - s0 < SB ? cnt - s0 : SB;
      put(r, qf, p, nr, s0 == 0, work);
      const int s1 = s0 + SB;
      if (s1 < cnt)  // uniform
        r = gather(p, qf, [&](int i) { return pos_at(s1 + i); }, cnt - s1 < SB ? cnt - s1 : SB);
      sub_block(p, b, nr >= 64 ? ~0ull : (1ull << nr) - 1ull, work, o, s1 >= cnt);
    }
    finish(p, b, split, work, o);
  }
};

// Plain vector-ALU path for any small shape, fp32 or bf16 inputs widened to fp32
// in LDS. Needs Hq * Dv <= 4096 and Dk <= 512.
template <typename T>
struct AttnGeneric {
  static constexpr int SB = 32;
  static constexpr int kMaxPerThread = 4096 / kAttnBlock;
  __host__ __device__ static size_t lds_bytes(int Hq, int Dk) {
    return (size_t)SB * Dk * 4 + (size_t)Hq * Dk * 4 + (size_t)Hq * SB * 4 + 3 * (size_t)Hq * 4;
  }
  __device__ __forceinline__ static float ld(const void* base, int64_t i) {
    if constexpr (sizeof(T) == 4) return reinterpret_cast<const float*>(base)[i];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
  }

  struct QFrag {};
  __device__ __forceinline__ static QFrag load_q(const AttnArgs&, int) { return QFrag{}; }
  __device__ __forceinline__ static void store_q(const QFrag&, const AttnArgs&, uint8_t*) {}

  template <typename PosAt>
  __device__ __forceinline__ static void run(const AttnArgs& p, int b, int split, PosAt pos_at, int cnt,
                             uint8_t* work, const QFrag&) {
    const int tid = threadIdx.x;
    const int Hq = p.Hq, Dk = p.Dk, Dv = p.Dv;
    float* rows = reinterpret_cast<float*>(work);
    float* qs = rows + SB * Dk;
    float* lg = qs + Hq * Dk;
    float* mrun = lg + Hq * SB;
    float* lrun = mrun + Hq;
    float* alpha = lrun + Hq;
    for (int i = tid; i < Hq * Dk; i += kAttnBlock) qs[i] = ld(p.q, (int64_t)b * Hq * Dk + i);
    for (int h = tid; h < Hq; h += kAttnBlock) {
      mrun[h] = -INFINITY;
      lrun[h] = 0.f;
    }
    float o[kMaxPerThread];
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) o[j] = 0.f;

    for (int s0 = 0; s0 < cnt; s0 += SB) {
      const int nr = cnt - s0 < SB ? cnt - s0 : SB;
      for (int i = tid; i < SB * Dk; i += kAttnBlock) {
        const int r = i / Dk, d = i - r * Dk;
        rows[i] = r < nr ? ld(p.kv, pos_at(s0 + r) * Dk + d) : 0.f;
      }
      lds_barrier();
      for (int pr = tid; pr < Hq * SB; pr += kAttnBlock) {
        const int h = pr / SB, r = pr - h * SB;
        float dot = 0.f;
        if (r < nr)
          for (int d = 0; d < Dk; ++d) dot = fmaf(qs[h * Dk + d], rows[r * Dk + d], dot);
        lg[pr] = r < nr ? dot * p.scale : -INFINITY;
      }
      lds_barrier();
      softmax_update(lg, SB, Hq, mrun, lrun, alpha);
      lds_barrier();
#pragma unroll
      for (int j = 0; j < kMaxPerThread; ++j) {
        const int pr = tid + kAttnBlock * j;
        if (pr < Hq * Dv) {
          const int h = pr / Dv, dv = pr - h * Dv;
          float acc = o[j] * alpha[h];
          for (int r = 0; r < nr; ++r) acc = fmaf(lg[h * SB + r], rows[r * Dk + dv], acc);
          o[j] = acc;
        }
      }
      lds_barrier();
    }
    const int64_t pb = (int64_t)b * p.S + split;
    for (int h = tid; h < Hq; h += kAttnBlock) p.part_ml[pb * Hq + h] = make_float2(mrun[h], lrun[h]);
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
      const int pr = tid + kAttnBlock * j;
      if (pr < Hq * Dv) p.part_o[pb * Hq * Dv + pr] = o[j];
    }
  }
};

// Selection only (no attention role).
struct AttnNone {
  __host__ __device__ static size_t lds_bytes(int, int) { return 0; }
  struct QFrag {};
  __device__ __forceinline__ static QFrag load_q(const AttnArgs&, int) { return QFrag{}; }
  __device__ __forceinline__ static void store_q(const QFrag&, const AttnArgs&, uint8_t*) {}
  template <typename PosAt>
  __device__ __forceinline__ static void run(const AttnArgs&, int, int, PosAt, int, uint8_t*, const QFrag&) {}
};

}  // namespace dsa

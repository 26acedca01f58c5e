// Stage 2 (exact ordered top-k) and stage 3 (sparse attention), plus the
// combine pass of the attention splits.
//
// Selection follows the structure described in the ds4 glm53-m3ultra branch post
// (2026-09-09 "rising" page, long-context paragraph): parallel scans narrow the
// candidates, a small surviving list is ordered, and the original exhaustive
// algorithm handles the ambiguous cases; the same positions come out in the same
// order either way.
//  * Candidate path. The score pass left, for every chunk of positions, its m
//    best keys and the best key it dropped (x_c). Every workgroup of this kernel
//    loads that candidate union U (at most 8192 keys, LDS resident), finds the
//    k-th largest key K* of U by radix selection, and checks that no chunk
//    dropped a key >= K*. When that holds, the top k of the row are exactly the
//    keys of U that are >= K*; they are compacted in position order.
//  * Exhaustive path ("ambiguous" case: a chunk holds more than m keys at or
//    above K*, which happens when many positions tie at the threshold; or the
//    flag forces it): the top-k set comes from a radix selection over every
//    position of the row, and the ordered output from a full stable sort of the
//    row by score (least-significant-digit radix sort, which keeps the position
//    order of equal scores).
// Two roles share the launch, so no second kernel boundary is spent:
//  * ranking workgroups order the selected keys: each takes a slice and counts,
//    for each of its keys, how many selected keys are larger; that count is the
//    output slot (keys are distinct, so the slots are a permutation);
//  * attention workgroups each take a slice of the selected positions (in position
//    order, identical on both paths) and write one split of the attention.
#include "attn_body.h"
#include "chunk_select.h"
#include "kernels.h"

namespace dsa {

// ------------------------------------------------------------------ candidates over stored scores

__global__ __launch_bounds__(kBlock) void k_chunk_cand(CandArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  ChunkSmem& csm = *reinterpret_cast<ChunkSmem*>(smem);
  int32_t* sc = reinterpret_cast<int32_t*>(smem + align16(sizeof(ChunkSmem)));
  const int c = blockIdx.x, b = blockIdx.y;
  const int64_t cbeg = (int64_t)c * a.P;
  const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
  const int count = n64 > a.P ? a.P : (int)(n64 > 0 ? n64 : 0);
  const int32_t* row = a.scores + (int64_t)b * a.N + cbeg;
  for (int i = threadIdx.x; i < count; i += kBlock) sc[i] = row[i];
  __syncthreads();
  chunk_candidates(sc, count, (uint32_t)cbeg, a.m, a.cand + ((int64_t)b * a.G + c) * a.m,
                   a.xc + (int64_t)b * a.G + c, csm);
}

hipError_t launch_chunk_candidates(const CandArgs& a, int B, hipStream_t s) {
  const size_t lds = align16(sizeof(ChunkSmem)) + (size_t)a.P * 4;
  hipError_t e = hipFuncSetAttribute((const void*)k_chunk_cand,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_chunk_cand, dim3(a.G, B), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ exhaustive ordered sort

struct SortSmem {
  uint32_t hist[256];
  uint32_t base[256];
  uint32_t wc[kWaves][256];
  int skip;
};

// Stable sort of the row's (score, position) pairs by score descending, four
// byte-wide counting passes from the least significant byte. The input is built
// in position order, so equal scores keep ascending positions. Returns the
// buffer that holds the result (bufA or bufB). One workgroup.
__device__ const uint64_t* block_sort_row(const int32_t* __restrict__ scores, int n,
                                          uint64_t* bufA, uint64_t* bufB, SortSmem& ss) {
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  for (int i = tid; i < n; i += kBlock)
    bufA[i] = ((uint64_t)((uint32_t)scores[i] ^ 0x80000000u) << 32) | (uint32_t)i;
  for (int i = tid; i < kWaves * 256; i += kBlock) (&ss.wc[0][0])[i] = 0;
  __threadfence_block();
  __syncthreads();
  uint64_t* src = bufA;
  uint64_t* dst = bufB;
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 32 + 8 * pass;
    auto digit = [sh](uint64_t e) { return 255u - (uint32_t)((e >> sh) & 0xFF); };
    ss.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kBlock) atomicAdd(&ss.hist[digit(src[i])], 1u);
    __syncthreads();
    if (tid < 64) {
      const uint32_t h0 = ss.hist[4 * tid], h1 = ss.hist[4 * tid + 1], h2 = ss.hist[4 * tid + 2],
                     h3 = ss.hist[4 * tid + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t s = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(s, o);
        if (tid >= o) s += t;
      }
      uint32_t ex = s - own;
      ss.base[4 * tid] = ex;
      ss.base[4 * tid + 1] = ex + h0;
      ss.base[4 * tid + 2] = ex + h0 + h1;
      ss.base[4 * tid + 3] = ex + h0 + h1 + h2;
      const bool one = h0 == (uint32_t)n || h1 == (uint32_t)n || h2 == (uint32_t)n || h3 == (uint32_t)n;
      const uint64_t any = __ballot(one);
      if (tid == 0) ss.skip = any != 0;
    }
    __syncthreads();
    if (ss.skip) {
      __syncthreads();
      continue;  // every element has the same digit: the order is unchanged
    }
    for (int t0 = 0; t0 < n; t0 += kBlock) {
      const int i = t0 + tid;
      const bool valid = i < n;
      const uint64_t e = valid ? src[i] : 0;
      const uint32_t d = valid ? digit(e) : 0;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool set = (d >> bit) & 1;
        const uint64_t bb = __ballot(valid && set);
        peers &= set ? bb : ~bb;
      }
      if (!valid) peers = 0;
      const int rank = __popcll(peers & lanemask_lt());
      const bool last = valid && (peers & ~((2ull << lane) - 1ull)) == 0;
      if (last) ss.wc[wave][d] = rank + 1;
      __syncthreads();
      if (valid) {
        uint32_t off = ss.base[d] + rank;
        for (int w = 0; w < wave; ++w) off += ss.wc[w][d];
        dst[off] = e;
      }
      __syncthreads();
      {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          t += ss.wc[w][tid];
          ss.wc[w][tid] = 0;
        }
        ss.base[tid] += t;
      }
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
    uint64_t* tmp = src;
    src = dst;
    dst = tmp;
  }
  return src;
}

// ------------------------------------------------------------------ selection (+ attention)

struct SelSmem {
  SelectSmem sel;
  SortSmem sort;
  int counts[kWaves];
  int base;
  int ired[kWaves];
  uint64_t ured[kWaves];
};

// LDS: SelSmem | selected keys [k] | region shared by the candidate union and
// the attention working set.
template <class Attn>
__global__ __launch_bounds__(kBlock) void k_select(SelArgs a, AttnArgs at) {
  extern __shared__ __align__(16) uint8_t smem[];
  SelSmem& sm = *reinterpret_cast<SelSmem*>(smem);
  uint64_t* sel = reinterpret_cast<uint64_t*>(smem + align16(sizeof(SelSmem)));
  uint8_t* region = smem + align16(sizeof(SelSmem)) + align16((size_t)a.k * 8);
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int S = at.S;
  const bool attn_role = (int)blockIdx.x < S;
  const int n = a.lens.n[b];
  const int32_t* row = a.scores + (int64_t)b * a.N;

  int reason = a.force ? 1 : (a.have_cand ? 0 : 3);
  int nvalid = 0, nsel = 0;
  uint64_t kstar = 0;
  if (reason == 0) {
    const int C = a.G * a.m;
    uint64_t* U = reinterpret_cast<uint64_t*>(region);
    const uint64_t* cu = a.cand + (int64_t)b * C;
    int nz = 0;
    for (int i = tid; i < C; i += kBlock) {
      const uint64_t v = cu[i];
      U[i] = v;
      nz += v != 0;
    }
    uint64_t mx = 0;
    for (int i = tid; i < a.G; i += kBlock) {
      const uint64_t v = a.xc[(int64_t)b * a.G + i];
      mx = v > mx ? v : mx;
    }
    nvalid = block_sum(nz, sm.ired);
    mx = block_max_u64(mx, sm.ured);
    const int kk = a.k < nvalid ? a.k : nvalid;
    kstar = block_kth_largest(C, kk, [&](int i) { return U[i]; }, sm.sel);
    const bool ok = mx < kstar && (nvalid >= a.k || mx == 0);
    if (ok) {
      if (tid == 0) sm.base = 0;
      __syncthreads();
      for (int r0 = 0; r0 < C; r0 += kBlock) {
        const int i = r0 + tid;
        const uint64_t v = i < C ? U[i] : 0;
        const bool keep = i < C && v >= kstar;
        const int slot = block_compact_slot(keep, sm.counts, &sm.base);
        if (keep) sel[slot] = v;
      }
      nsel = kk;
    } else {
      reason = 2;
    }
    __syncthreads();
  }

  if (reason != 0) {
    if (!attn_role) {
      if ((int)blockIdx.x != S) return;  // one ranking workgroup sorts the whole row
      uint64_t* ba = a.sortbuf + (int64_t)b * 2 * a.N;
      const uint64_t* sorted = block_sort_row(row, n, ba, ba + a.N, sm.sort);
      const int kk = a.k < n ? a.k : n;
      int32_t* out = a.idx + (int64_t)b * a.k;
      const uint32_t ulast = (uint32_t)(sorted[kk - 1] >> 32);
      int tied = 0;
      for (int j = tid; j < a.k; j += kBlock) {
        if (j < kk) {
          const uint64_t e = sorted[j];
          out[j] = (int32_t)(uint32_t)e;
          tied += (uint32_t)(e >> 32) == ulast;
        } else {
          out[j] = -1;
        }
      }
      tied = block_sum(tied, sm.ired);
      if (tid == 0) {
        RowStats st;
        st.path = 1;
        st.reason = reason;
        st.selected = kk;
        st.kth_score = (int32_t)(ulast ^ 0x80000000u);
        st.candidates = nvalid;
        st.tied_at_kth = tied;
        st.bad_indices = 0;
        st.reserved = 0;
        a.stats[b] = st;
      }
      return;
    }
    // attention workgroups select the same set over every position
    const int kk = a.k < n ? a.k : n;
    auto key_at = [&](int i) { return make_key(row[i], (uint32_t)i); };
    kstar = block_kth_largest(n, kk, key_at, sm.sel);
    if (tid == 0) sm.base = 0;
    __syncthreads();
    for (int r0 = 0; r0 < n; r0 += kBlock) {
      const int i = r0 + tid;
      uint64_t v = 0;
      bool keep = false;
      if (i < n) {
        v = key_at(i);
        keep = v >= kstar;
      }
      const int slot = block_compact_slot(keep, sm.counts, &sm.base);
      if (keep) sel[slot] = v;
    }
    nsel = kk;
  }
  __syncthreads();

  if (attn_role) {
    const int per = (nsel + S - 1) / S;
    const int e0 = (int)blockIdx.x * per;
    int cnt = nsel - e0;
    cnt = cnt < 0 ? 0 : (cnt > per ? per : cnt);
    Attn::run(at, b, blockIdx.x, [&](int i) { return (int64_t)key_pos(sel[e0 + i]); }, cnt,
              region);
    return;
  }

  // ranking: slot of a key = number of selected keys larger than it
  const int r = (int)blockIdx.x - S;
  const int per = (nsel + a.R - 1) / a.R;
  const int e0 = r * per;
  const int e1 = e0 + per < nsel ? e0 + per : nsel;
  int32_t* out = a.idx + (int64_t)b * a.k;
  for (int base = e0; base < e1; base += kBlock / 16) {
    const int e = base + (tid >> 4);
    const int part = tid & 15;
    const uint64_t me = e < e1 ? sel[e] : ~0ull;
    int cnt = 0;
    if (e < e1)
      for (int x = part; x < nsel; x += 16) cnt += sel[x] > me;
    cnt += __shfl_xor(cnt, 8);
    cnt += __shfl_xor(cnt, 4);
    cnt += __shfl_xor(cnt, 2);
    cnt += __shfl_xor(cnt, 1);
    if (e < e1 && part == 0) out[cnt] = (int32_t)key_pos(me);
  }
  if (r == 0) {
    for (int j = nsel + tid; j < a.k; j += kBlock) out[j] = -1;
    const uint32_t ulast = (uint32_t)(kstar >> 32);
    int tied = 0;
    for (int i = tid; i < nsel; i += kBlock) tied += (uint32_t)(sel[i] >> 32) == ulast;
    tied = block_sum(tied, sm.ired);
    if (tid == 0) {
      RowStats st;
      st.path = 0;
      st.reason = 0;
      st.selected = nsel;
      st.kth_score = key_score(kstar);
      st.candidates = nvalid;
      st.tied_at_kth = tied;
      st.bad_indices = 0;
      st.reserved = 0;
      a.stats[b] = st;
    }
  }
}

template <class Attn>
static size_t select_lds_t(int Hq, int Dk, int k) {
  const size_t region_c = (size_t)kCandCap * 8;
  const size_t region_a = Attn::lds_bytes(Hq, Dk);
  return align16(sizeof(SelSmem)) + align16((size_t)k * 8) +
         (region_c > region_a ? region_c : region_a);
}

template <class Attn>
static hipError_t launch_select_t(const SelArgs& a, const AttnArgs& at, int B, hipStream_t s) {
  const size_t lds = select_lds_t<Attn>(at.Hq, at.Dk, a.k);
  auto fn = k_select<Attn>;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(at.S + a.R, B), dim3(kBlock), lds, s, a, at);
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention over given indices

template <class Attn>
__global__ __launch_bounds__(kBlock) void k_attend_idx(const int32_t* __restrict__ idx, int k,
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
  if (tid == 0) sm.base = 0;
  __syncthreads();
  int bad = 0;
  for (int r0 = e0; r0 < e1; r0 += kBlock) {
    const int i = r0 + tid;
    const int32_t v = i < e1 ? row[i] : -1;
    const bool keep = v >= 0 && (int64_t)v < at.N;
    bad += (v != -1 && !keep);
    const int slot = block_compact_slot(keep, sm.counts, &sm.base);
    if (keep) posl[slot] = v;
  }
  bad = block_sum(bad, sm.ired);
  const int cnt = sm.base;
  __syncthreads();
  if (tid == 0) part_bad[(int64_t)b * at.S + j] = bad;
  Attn::run(at, b, j, [&](int i) { return (int64_t)posl[i]; }, cnt, region);
}

template <class Attn>
static hipError_t launch_attend_t(const int32_t* idx, int k, int32_t* part_bad, const AttnArgs& at,
                                  int B, hipStream_t s) {
  const int per = (k + at.S - 1) / at.S;
  const size_t lds = align16(sizeof(SelSmem)) + align16((size_t)per * 4) + Attn::lds_bytes(at.Hq, at.Dk);
  auto fn = k_attend_idx<Attn>;
  hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(at.S, B), dim3(kBlock), lds, s, idx, k, part_bad, at);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch

AttnChoice choose_attn(int dt_bf16, int Hq, int Dk, int Dv) {
  AttnChoice c{ATTN_NONE, 0, 0};
  if (dt_bf16 && Hq >= 1 && Hq <= 64 && Dk % 32 == 0 && Dk <= 1024 && Dv % 64 == 0 && Dv <= 512 &&
      Dv <= Dk) {
    c.kind = ATTN_MFMA_BF16;
    c.hqt = (Hq + 15) / 16;
    c.sb = Dk <= 576 ? 64 : 32;
    return c;
  }
  if (Hq >= 1 && Hq * Dv <= 4096 && Dk <= 512 && Dv <= Dk) {
    c.kind = dt_bf16 ? ATTN_GENERIC_BF16 : ATTN_GENERIC_F32;
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
      if (ch.sb == 64) {                                                               \
        switch (ch.hqt) {                                                              \
          case 1: return FN<AttnMfma<1, 64>>(__VA_ARGS__);                             \
          case 2: return FN<AttnMfma<2, 64>>(__VA_ARGS__);                             \
          case 3: return FN<AttnMfma<3, 64>>(__VA_ARGS__);                             \
          case 4: return FN<AttnMfma<4, 64>>(__VA_ARGS__);                             \
        }                                                                              \
      } else {                                                                         \
        switch (ch.hqt) {                                                              \
          case 1: return FN<AttnMfma<1, 32>>(__VA_ARGS__);                             \
          case 2: return FN<AttnMfma<2, 32>>(__VA_ARGS__);                             \
          case 3: return FN<AttnMfma<3, 32>>(__VA_ARGS__);                             \
          case 4: return FN<AttnMfma<4, 32>>(__VA_ARGS__);                             \
        }                                                                              \
      }                                                                                \
  }                                                                                    \
  return hipErrorInvalidValue;

using AttnM1x64 = AttnMfma<1, 64>;
using AttnM2x64 = AttnMfma<2, 64>;
using AttnM3x64 = AttnMfma<3, 64>;
using AttnM4x64 = AttnMfma<4, 64>;
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
      if (ch.sb == 64) {
        switch (ch.hqt) {
          case 1: return select_lds_t<AttnM1x64>(Hq, Dk, k);
          case 2: return select_lds_t<AttnM2x64>(Hq, Dk, k);
          case 3: return select_lds_t<AttnM3x64>(Hq, Dk, k);
          default: return select_lds_t<AttnM4x64>(Hq, Dk, k);
        }
      }
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

hipError_t launch_select(const SelArgs& a, const AttnArgs& at, AttnChoice ch, int B, hipStream_t s) {
  DSA_ATTN_DISPATCH(launch_select_t, a, at, B, s)
}

hipError_t launch_attend_idx(const int32_t* idx, int k, int32_t* part_bad, const AttnArgs& at,
                             AttnChoice ch, int B, hipStream_t s) {
  if (ch.kind == ATTN_NONE) return hipErrorInvalidValue;
  DSA_ATTN_DISPATCH(launch_attend_t, idx, k, part_bad, at, B, s)
}

// ------------------------------------------------------------------ combine

// out[b][h][v] = sum_s e^(m_s - M) o_s[h][v] / sum_s e^(m_s - M) l_s, splits in order.
__global__ __launch_bounds__(kBlock) void k_combine(AttnArgs at, const int32_t* __restrict__ part_bad,
                                                    RowStats* __restrict__ stats, float* __restrict__ out) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (part_bad != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    int t = 0;
    for (int s = 0; s < at.S; ++s) t += part_bad[(int64_t)b * at.S + s];
    stats[b].bad_indices = t;
  }
  if (i >= at.Hq * at.Dv) return;
  const int h = i / at.Dv;
  const float2* ml = at.part_ml + (int64_t)b * at.S * at.Hq + h;
  float M = -INFINITY;
  for (int s = 0; s < at.S; ++s) M = fmaxf(M, ml[(int64_t)s * at.Hq].x);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    const float* po = at.part_o + (int64_t)b * at.S * at.Hq * at.Dv + i;
    for (int s = 0; s < at.S; ++s) {
      const float2 v = ml[(int64_t)s * at.Hq];
      if (v.x == -INFINITY) continue;
      const float w = __expf(v.x - M);
      num = fmaf(w, po[(int64_t)s * at.Hq * at.Dv], num);
      den = fmaf(w, v.y, den);
    }
  }
  out[(int64_t)b * at.Hq * at.Dv + i] = den > 0.f ? num / den : 0.f;
}

hipError_t launch_combine(const AttnArgs& at, const int32_t* part_bad, RowStats* stats, float* out,
                          int B, hipStream_t s) {
  const int grid = (at.Hq * at.Dv + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_combine, dim3(grid, B), dim3(kBlock), 0, s, at, part_bad, stats, out);
  return hipGetLastError();
}

}  // namespace dsa

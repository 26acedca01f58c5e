// Stage 1: the indexer score pass.
//
// score[b][s] = sum_h w[b][h] * max(0, sum_d q[b][h][d] * k[s][d])   (int8 in, int32 out)
//
// This is a dense contraction of the indexer heads against every cached key
// (heads x dim times dim x positions), so it runs on the int8 matrix cores:
// v_mfma_i32_32x32x32_i8 with the query heads as the A operand (32 heads per
// tile, held in registers or LDS) and 32 keys per tile streamed from HBM as the B
// operand with 16-byte loads (k_score_row, one query row: two 32-key units per
// wave in flight; k_score, several rows: three 64-key tiles). The ReLU, the
// per-head weight and the sum over heads are applied to the accumulators in
// registers; one cross-lane add finishes the head sum. The key cache is read
// exactly once per launch.
//
// With candidates enabled, each workgroup owns one chunk of positions (for one
// row: every G-th 32-key unit of the row; for several rows: a contiguous stretch)
// and, after scoring it, keeps the chunk's m best keys (and the best key it
// drops) for the selection stage: the "scans that narrow the candidates" of the
// ds4 glm53-m3ultra branch post (2026-09-09 "rising" page, long-context paragraph).
#include "chunk_select.h"
#include "kernels.h"

namespace dsa {

constexpr int kScoreBlock = 512;
constexpr int kScoreWaves = kScoreBlock / 64;
constexpr int kMaxTiles = kChunkPerThread * kScoreBlock / 64;  // 64-key tiles of the longest chunk
static_assert(kScoreQBytes % (16 * kScoreBlock) == 0, "query staging slots");

namespace {

// Key fragment of the B operand: lane l holds 16 consecutive dims of key
// (64*tile + 32*t + (l & 31)) of the chunk, starting at dim 32*kt + 16*(l >> 5);
// keys are Di bytes apart. Raw buffer loads against a resource that covers exactly
// the chunk's valid keys: always issued (so the compiler's wait counts stay exact),
// zero past the end without touching memory. (When Di = 32·KT - 16, the last
// fragment's upper half reads the next key's first dims or zeros; the query's
// matching half is zero, so those products vanish.)
template <int KT>
__device__ __forceinline__ void load_keys(v4i (&kf)[2][KT], __amdgpu_buffer_rsrc_t rs, int tile, int Di) {
  const int lane = lane_id();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int off = (64 * tile + 32 * t + (lane & 31)) * Di + 16 * (lane >> 5);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      kf[t][kt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * kt, 0, 0));
  }
}

// The same for a paged pool: the tile's 64 keys are consecutive pool rows starting
// `base` bytes into the pool (a 64-aligned tile lies inside one page); a base past
// the pool gives zeros.
template <int KT>
__device__ __forceinline__ void load_keys_at(v4i (&kf)[2][KT], __amdgpu_buffer_rsrc_t rs, uint32_t base, int Di) {
  const int lane = lane_id();
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t off = base + (uint32_t)((32 * t + (lane & 31)) * Di + 16 * (lane >> 5));
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      kf[t][kt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * kt, 0, 0));
  }
}

}  // namespace

// NB: key tile buffers per wave (3, rotating, refilled as each is consumed; or 1
// when a chunk has at most one 64-key tile per wave, so no request is issued for
// tiles past the chunk: those requests returned zeros but took the address units'
// time ahead of the query requests of the waves behind). PG: the keys live in a
// paged pool (a.ik) behind the page table a.pages.
template <int MT, int KT, bool CAND, bool ONE, int NB, bool PG>
__global__ __launch_bounds__(kScoreBlock) void k_score(ScoreArgs a) {
  constexpr int HP = 32 * MT;  // heads padded to whole tiles (padding has q = 0, w = 0)
  constexpr int DI = 32 * KT;
  // LDS row stride of a staged query head: 16 bytes past its DI, so that the A
  // fragment reads (32 heads a wave, DI bytes apart) spread over the banks
  constexpr int DIP = DI + 16;
  extern __shared__ __align__(16) uint8_t smem[];
  using Smem = ChunkSmem<kScoreBlock>;
  Smem& csm = *reinterpret_cast<Smem*>(smem);
  int8_t* qs = reinterpret_cast<int8_t*>(smem + align16(sizeof(Smem)));       // [Bg][HP][DIP]
  int32_t* wsm = reinterpret_cast<int32_t*>(qs + a.Bg * HP * DIP);             // [Bg][HP] head weights
  // paged: pool byte offset of each 64-key tile of the chunk
  uint32_t* toff = reinterpret_cast<uint32_t*>(wsm + a.Bg * HP);              // [kMaxTiles] (PG)
  int32_t* sc = wsm + a.Bg * HP + (PG ? kMaxTiles : 0);                       // [Bg][P]
  uint32_t* hist = reinterpret_cast<uint32_t*>(sc + a.Bg * a.P);              // [Bg][kHistBins]
  using CandSmem = BlockCandSmem<kScoreBlock>;
  CandSmem& bsm = *reinterpret_cast<CandSmem*>(hist + a.Bg * kHistBins);
  int* fallback = reinterpret_cast<int*>(&bsm + 1);                             // [Bg]

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int c = blockIdx.x;
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
    // 16-byte parts past Di (Di = 32·KT - 16) read a present part and are zeroed below
    qv[j] = *(const v4i*)(a.iq + ((int64_t)(a.b0 + bb) * a.Hi + h) * a.Di + (16 * part < a.Di ? 16 * part : 0));
  }
  const int wi = tid < a.Bg * HP ? tid : a.Bg * HP - 1;
  const int wh = wi % HP < a.Hi ? wi % HP : a.Hi - 1;
  const int8_t wv = a.iw[(int64_t)(a.b0 + wi / HP) * a.Hi + wh];

  // buffer resource word 3 for gfx9 raw buffers: 32-bit data format, no swizzle.
  // Contiguous keys: the resource covers the chunk's valid keys. Paged: it covers
  // the pool, tile tp starts at pool byte tile_at(tp, e) with e its table entry, and
  // a tile past the chunk gets an offset past the pool (zeros). The first tiles'
  // entries are read per wave; thread t reads tile t's for the LDS list (toff) the
  // refills use. All of them are read unconditionally (entry 0 standing in for a
  // tile past the chunk), so their requests go out together.
  const uint32_t pool_bytes = PG ? (uint32_t)a.pool_pages * (uint32_t)kPageSize * (uint32_t)a.Di : 0u;
  const __amdgpu_buffer_rsrc_t rs =
      PG ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.ik), (short)0, (int)pool_bytes, 0x00020000)
         : __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.ik + cbeg * a.Di), (short)0, clen * a.Di,
                                             0x00020000);
  auto entry_of = [&](int tp) -> int64_t { return tp < npairs ? (cbeg + 64 * tp) >> kPageShift : 0; };
  auto tile_at = [&](int tp, int32_t e) -> uint32_t {
    e = e < 0 ? 0 : (e >= a.pool_pages ? a.pool_pages - 1 : e);
    return tp < npairs ? ((uint32_t)e * kPageSize + (uint32_t)((cbeg + 64 * tp) & (kPageSize - 1))) * (uint32_t)a.Di
                       : pool_bytes;
  };
  v4i kb0[2][KT], kb1[2][KT], kb2[2][KT];
  int32_t te = 0;  // paged: thread t's tile entry, stored to LDS (as an offset) below
  if constexpr (PG) {
    int32_t e0 = a.pages[entry_of(wave)], e1 = 0, e2 = 0;
    if constexpr (NB > 1) {
      e1 = a.pages[entry_of(wave + kScoreWaves)];
      e2 = a.pages[entry_of(wave + 2 * kScoreWaves)];
    }
    te = a.pages[entry_of(tid)];
    asm volatile("" : "+s"(e0), "+s"(e1), "+s"(e2));  // (read here, not behind a branch each)
    load_keys_at<KT>(kb0, rs, tile_at(wave, e0), a.Di);
    if constexpr (NB > 1) {
      load_keys_at<KT>(kb1, rs, tile_at(wave + kScoreWaves, e1), a.Di);
      load_keys_at<KT>(kb2, rs, tile_at(wave + 2 * kScoreWaves, e2), a.Di);
    }
  } else {
    load_keys<KT>(kb0, rs, wave, a.Di);
    if constexpr (NB > 1) {
      load_keys<KT>(kb1, rs, wave + kScoreWaves, a.Di);
      load_keys<KT>(kb2, rs, wave + 2 * kScoreWaves, a.Di);
    }
  }

  if (CAND) {
    radix_clear<kScoreBlock>(csm.radix);
    for (int i = tid; i < a.Bg * kHistBins; i += kScoreBlock) hist[i] = 0;
  }
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int i = tid + kScoreBlock * j;
    const int hrow = i / (DI / 16);  // bb * HP + h
    const int h = hrow % HP;
    const int part = i % (DI / 16);
    if (i < nq) *(v4i*)(qs + hrow * DIP + 16 * part) = h < a.Hi && 16 * part < a.Di ? qv[j] : v4i{0, 0, 0, 0};
  }
  if (tid < a.Bg * HP) wsm[tid] = tid % HP < a.Hi ? (int32_t)wv : 0;
  if constexpr (PG)
    if (tid < npairs) toff[tid] = tile_at(tid, te);
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
            *(const v4i*)(qs + (32 * mt + (lane & 31)) * DIP + 32 * kt + 16 * (lane >> 5));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4i wd = *(const v4i*)(wsm + 32 * mt + 8 * g + 4 * (lane >> 5));
#pragma unroll
        for (int j = 0; j < 4; ++j) wreg[ONE ? mt : 0][ONE ? 4 * g + j : 0] = wd[j];
      }
    }
  }

  // Scores of 64 positions (tile tp) from the key fragments `cur`, which are then
  // refilled with tile tp + 24. With candidates, scores stay in LDS until the chunk
  // is done (no global store in the loop: its completion would be waited for later).
  // Per row the tile is two 32-key halves, and the rows form a pipeline over them:
  // the matrix cores take a row's second half, then the next row's first half,
  // while the vector ALU weighs the half before (otherwise the two waves of a SIMD
  // run their products and their weighing in step, and each unit idles half the time).
  auto load_a = [&](int bb, v4i(&qa)[MT][KT]) {  // A fragments of row bb
    const int8_t* qb = qs + bb * HP * DIP;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        qa[mt][kt] = ONE ? qreg[ONE ? mt : 0][ONE ? kt : 0]
                         : *(const v4i*)(qb + (32 * mt + (lane & 31)) * DIP + 32 * kt + 16 * (lane >> 5));
  };
  auto load_w = [&](int bb, int(&w)[MT][16]) {  // weights of the lane's accumulator heads
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (ONE) {
#pragma unroll
          for (int j = 0; j < 4; ++j) w[mt][4 * g + j] = wreg[ONE ? mt : 0][ONE ? 4 * g + j : 0];
        } else {
          const v4i wd = *(const v4i*)(wsm + bb * HP + 32 * mt + 8 * g + 4 * (lane >> 5));
#pragma unroll
          for (int j = 0; j < 4; ++j) w[mt][4 * g + j] = wd[j];
        }
      }
  };
  auto mm = [&](v16i(&acc)[MT], const v4i(&qa)[MT][KT], const v4i(&kf)[KT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v16i{};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[mt][kt], kf[kt], acc[mt], 0, 0, 0);
  };
  // accumulator r of lane l holds head 32*mt + 8*(r/4) + 4*(l/32) + r%4 of key l%32;
  // two independent multiply-add chains
  auto weigh = [&](const v16i(&acc)[MT], const int(&w)[MT][16]) {
    int c0 = 0, c1 = 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int v0 = acc[mt][r], v1 = acc[mt][r + 1];
        c0 = mad_i24(w[mt][r], v0 > 0 ? v0 : 0, c0);
        c1 = mad_i24(w[mt][r + 1], v1 > 0 ? v1 : 0, c1);
      }
    return c0 + c1;
  };
  auto tile = [&](v4i(&cur)[2][KT], int tp) {
    const int64_t p0 = cbeg + 64 * tp;
    const int nb = ONE ? 1 : a.Bg;  // a compile-time trip count keeps the wait counts exact
    v4i qa[MT][KT];
    int w[MT][16];
    v16i a0[MT], a1[MT];
    load_a(0, qa);
    mm(a0, qa, cur[0]);
    for (int bb = 0; bb < nb; ++bb) {
      mm(a1, qa, cur[1]);
      load_w(bb, w);
      const int h0 = weigh(a0, w);
      if (bb + 1 < nb) {  // uniform
        load_a(bb + 1, qa);
        mm(a0, qa, cur[0]);
      }
      const int h1 = weigh(a1, w);
      // lanes l and l ^ 32 hold the same key's other heads: one lane-half swap gives
      // lane l < 32 key l of the first 32 (half 0), lane l >= 32 key l of the tile
      const auto sw = __builtin_amdgcn_permlane32_swap(h0, h1, false, false);
      const int val = sw[0] + sw[1];
      const int64_t pos = p0 + lane;
      if (CAND) {
        sc[bb * a.P + (int)(pos - cbeg)] = val;
        if (pos < a.lens.n[a.b0 + bb]) atomicAdd(&hist[bb * kHistBins + score_bin(val)], 1u);
      } else if (pos < a.lens.n[a.b0 + bb]) {
        a.scores[(int64_t)(a.b0 + bb) * a.N + pos] = val;
      }
    }
    if constexpr (NB > 1) {
      if constexpr (PG) {
        const int tn = tp + 3 * kScoreWaves;
        load_keys_at<KT>(cur, rs, tn < npairs ? toff[tn] : pool_bytes, a.Di);
      } else {
        load_keys<KT>(cur, rs, tp + 3 * kScoreWaves, a.Di);
      }
    }
  };

  if constexpr (NB == 1) {
    if (wave < npairs) tile(kb0, wave);
  } else {
    // three key buffers rotate by name (a register copy would wait for its load)
    for (int tp = wave; tp < npairs; tp += 3 * kScoreWaves) {
      tile(kb0, tp);
      if (tp + kScoreWaves >= npairs) break;
      tile(kb1, tp + kScoreWaves);
      if (tp + 2 * kScoreWaves >= npairs) break;
      tile(kb2, tp + 2 * kScoreWaves);
    }
  }

  if (CAND) {
    lds_barrier();
    // the scores leave LDS first (one row: here; several: in each row's epilogue, as
    // it reads them): the selection waits for no memory operation, so these stores
    // complete underneath it. The key requests past the chunk's end (buffer reads
    // that return zeros) are drained before them, so no later wait for those
    // registers covers the stores.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // gfx9 encoding: vmcnt(0), expcnt and lgkmcnt untouched
    if (ONE) {
      const int64_t n64 = (int64_t)a.lens.n[a.b0] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      int32_t* dst = a.scores + (int64_t)a.b0 * a.N + cbeg;
      for (int i = tid; i < count; i += kScoreBlock) dst[i] = sc[i];
    }
    if (ONE) {
      // one row: the whole block selects the chunk's candidates
      const int b = a.b0;
      const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      const bool ok = block_chunk_candidates<kScoreBlock>(sc, count, (uint32_t)cbeg, a.m, hist,
                                                          CandOut{a.cand + (int64_t)b * kCandCap, c * a.m},
                                                          a.xc + (int64_t)b * a.G + c, bsm);
      if (tid == 0) fallback[0] = ok ? 0 : 1;
    } else {
      // several rows: wave w selects the candidates of rows w, w + 8, ...
      for (int bb = wave; bb < a.Bg; bb += kScoreWaves) {
        const int b = a.b0 + bb;
        const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
        const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
        const bool ok = wave_chunk_candidates(sc + bb * a.P, count, (uint32_t)cbeg, a.m, hist + bb * kHistBins,
                                              CandOut{a.cand + (int64_t)b * kCandCap, c * a.m},
                                              a.xc + (int64_t)b * a.G + c, bsm.wstage[wave],
                                              a.scores + (int64_t)b * a.N + cbeg);
        if (lane == 0) fallback[bb] = ok ? 0 : 1;
      }
    }
    lds_barrier();
    for (int bb = 0; bb < a.Bg; ++bb) {  // rows whose threshold bin held too many keys
      if (!fallback[bb]) continue;
      const int b = a.b0 + bb;
      const int64_t n64 = (int64_t)a.lens.n[b] - cbeg;
      const int count = n64 > clen ? clen : (int)(n64 > 0 ? n64 : 0);
      if (!ONE) {  // the epilogue may not have stored them
        int32_t* dst = a.scores + (int64_t)b * a.N + cbeg;
        for (int i = tid; i < count; i += kScoreBlock) dst[i] = sc[bb * a.P + i];
      }
      chunk_candidates<kScoreBlock>(sc + bb * a.P, count, (uint32_t)cbeg, a.m,
                                    CandOut{a.cand + (int64_t)b * kCandCap, c * a.m}, a.xc + (int64_t)b * a.G + c,
                                    csm);
      lds_barrier();
    }
  }
}

// ------------------------------------------------------------------ one query row
//
// The decode hot path (one query row per launch, candidates on). Every wave is
// independent until the chunk's scores are complete: it loads its own query
// fragments straight into registers and keeps D units of 32 keys in flight, so
// no wave waits on another while the key cache streams in (a block barrier after
// the loads are issued would hold every wave until the slowest one has had its
// whole share of the chunk accepted by the memory pipeline).

constexpr int kUnit = 32;                                    // keys per matrix-core tile
constexpr int kMaxUnits = kChunkPerThread * kScoreBlock / kUnit;
constexpr int kRowStage = 144;  // >= cap (m + 64 <= 128) + 16 read slack

struct RowCandSmem {
  uint64_t all[kRowStage];  // staged keys, in order of arrival
  uint32_t nstaged;
  uint32_t next;            // the chunk's next unclaimed unit
};

namespace {

// B fragments of the chunk's unit j (keys 32j·js .. 32j·js + 31 from the chunk's
// first key, Di bytes apart): lane l holds dims 32kt + 16(l >> 5) .. +15 of the
// unit's key l & 31. Raw buffer loads against a resource that ends with the chunk's
// last valid key (zeros past it); dims past Di meet a zero query half (load_keys).
template <int KT>
__device__ __forceinline__ void load_unit(v4i (&kf)[KT], __amdgpu_buffer_rsrc_t rs, int j, int js, int Di) {
  const int lane = lane_id();
  const int off = (kUnit * j * js + (lane & 31)) * Di + 16 * (lane >> 5);
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
    kf[kt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * kt, 0, 0));
}

// The same for a paged pool: the unit's 32 keys are consecutive pool rows starting
// `base` bytes into the pool (a 32-aligned unit lies inside one page); a base past
// the pool gives zeros.
template <int KT>
__device__ __forceinline__ void load_unit_at(v4i (&kf)[KT], __amdgpu_buffer_rsrc_t rs, uint32_t base, int Di) {
  const int lane = lane_id();
  const uint32_t off = base + (uint32_t)((lane & 31) * Di + 16 * (lane >> 5));
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
    kf[kt] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * kt, 0, 0));
}

}  // namespace

// The arguments that the first requests need come first, as separate scalars: the
// leading arguments can be preloaded into scalar registers at wave launch, so the
// query and key requests need not wait for a read of the argument block (a.iq,
// a.iw, a.ik, a.pages, a.lens.n[0], a.G, a.P, and a.Hi | a.Di << 16, passed again).
template <int MT, int KT, int D, bool PG>
__global__ __launch_bounds__(kScoreBlock) void k_score_row(const int8_t* __restrict__ iq,
                                                           const int8_t* __restrict__ iw,
                                                           const int8_t* __restrict__ ik,
                                                           const int32_t* __restrict__ pages, int n, int G, int P,
                                                           int hidi, ScoreArgs a) {
  static_assert(D == 2 || D == 3, "units in flight per wave");
  const int Hi = hidi & 0xFFFF, Di = hidi >> 16;
  extern __shared__ __align__(16) uint8_t smem[];
  using Smem = ChunkSmem<kScoreBlock>;
  Smem& csm = *reinterpret_cast<Smem*>(smem);
  int32_t* sc = reinterpret_cast<int32_t*>(smem + align16(sizeof(Smem)));                     // [P]
  uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(sc) + align16((size_t)P * 4));
  uint32_t* hgroup = hist + kHistBins;  // [kHistGroups]: sums of 16 bins
  RowCandSmem& rsm = *reinterpret_cast<RowCandSmem*>(hgroup + kHistGroups);
  // the query heads, rows DI + 16 bytes apart (the A-fragment reads of 32 heads then
  // spread over the banks)
  constexpr int DI = 32 * KT, DIP = DI + 16;
  int8_t* qs = reinterpret_cast<int8_t*>(&rsm) + align16(sizeof(RowCandSmem));  // [32 MT][DIP]
  int32_t* wsm = reinterpret_cast<int32_t*>(qs + 64 * (256 + 16));               // [64] head weights
  uint32_t* uoff = reinterpret_cast<uint32_t*>(wsm + 64);                        // [kMaxUnits] (PG)

  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  // a batch of one: the row is row 0, a constant, so that every argument address is
  // known at entry and their reads go out together (an index read from the argument
  // block would put a second round trip before the first key request)
  const int c = blockIdx.x, b = 0;
  // Chunk c is the row's 32-key units c, c + G, c + 2G, ... (interleaved, so that at
  // any moment the launch streams one contiguous stretch of keys): local unit j is
  // row unit c + j·G.
  const int js = G;
  int count;  // valid positions of the chunk
  const int units = row_chunk_units(n, c, G, P, 1, &count);
  const int64_t cbeg = (int64_t)kUnit * c;          // the chunk's first position
  const uint32_t ustride = (uint32_t)(kUnit * js);  // positions from one local unit to the next
  // local entry i is position cbeg + (i / 32)·ustride + i % 32; span: row positions
  // from the chunk's first to its last valid one
  const int span = units > 0 ? (int)((int64_t)(units - 1) * ustride) + (count - kUnit * (units - 1)) : 0;

  // Paged keys (PG): the resource covers the pool, the chunk's unit j starts at pool
  // byte base_of(j, e) with e its table entry (the row's unit c + jG is slot
  // (c + jG) % 8 of logical page (c + jG) / 8), and a unit past the chunk gets an
  // offset past the pool (zeros). Each wave requests its first units' entries before
  // anything else (they gate its first key requests); thread t reads unit t's entry
  // for the LDS list the refills use. Entries are read unconditionally, entry 0
  // standing in for a unit past the chunk (read behind a branch each, the first
  // units' entries were three round trips in a row).
  const uint32_t pool_bytes = PG ? (uint32_t)a.pool_pages * (uint32_t)kPageSize * (uint32_t)Di : 0u;
  auto entry_of = [&](int j) -> int { return j < units ? (c + j * G) >> 3 : 0; };
  auto base_of = [&](int j, int32_t e) -> uint32_t {
    e = e < 0 ? 0 : (e >= a.pool_pages ? a.pool_pages - 1 : e);
    return j < units ? ((uint32_t)e * kPageSize + (uint32_t)(kUnit * ((c + j * G) & 7))) * (uint32_t)Di : pool_bytes;
  };
  int32_t e0 = 0, e1 = 0, e2 = 0;
  if constexpr (PG) {
    e0 = pages[entry_of(wave)];
    e1 = pages[entry_of(wave + kScoreWaves)];
    if constexpr (D == 3) e2 = pages[entry_of(wave + 2 * kScoreWaves)];
  }

  // The query: the block requests it once, one 16-byte piece per thread (two when
  // Hi·Di > 8 KB), before any key, and stages it in LDS, from where every wave takes
  // its A operand (lane l: head 32mt + (l & 31), dims 32kt + 16(l >> 5) .. +15). Each
  // wave requesting the whole query itself cost eight requests per wave, and the
  // waves' first units started up to 2 µs apart. The head weights go the same way
  // (the first wave requests them; 0 for padding heads).
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(iq + (int64_t)b * Hi * Di), (short)0, Hi * Di, 0x00020000);
  const int npc = Hi * Di / 16;  // 16-byte pieces of the query (Di % 16 == 0)
  v4i qp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pc = tid + kScoreBlock * u;
    qp[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * (pc < npc ? pc : 0), 0, 0));
  }
  int wl = 0;
  if (wave == 0) wl = (int)iw[(int64_t)b * Hi + (lane < Hi ? lane : Hi - 1)];
  // (thread t's entry: requested here, unconditionally, and turned into an offset only
  // where it is stored, behind the key requests, so no wait for it comes first)
  int32_t ue = 0;
  if constexpr (PG) ue = pages[entry_of(tid)];

  // the histogram is shared by the waves: cleared before any of them adds to it
  for (int i = tid; i < kHistBins + kHistGroups; i += kScoreBlock) hist[i] = 0;  // and hgroup
  if (tid == 0) {
    rsm.nstaged = 0;
    rsm.next = kScoreWaves * D;  // units 0 .. 8D - 1 are requested below, D per wave
  }
  uint32_t fb[3] = {0u, 0u, 0u};
  if constexpr (PG) {
    // the entries as opaque values here, where the barrier below waits anyway: left
    // to itself the compiler moved each read behind its unit's branch
    asm volatile("" : "+s"(e0), "+s"(e1), "+s"(e2));
    fb[0] = base_of(wave, e0);
    fb[1] = base_of(wave + kScoreWaves, e1);
    if constexpr (D == 3) fb[2] = base_of(wave + 2 * kScoreWaves, e2);
  }
  lds_barrier();

  const __amdgpu_buffer_rsrc_t rs =
      PG ? __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(ik), (short)0, (int)pool_bytes, 0x00020000)
         : __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(ik + cbeg * Di), (short)0, span * Di, 0x00020000);
  v4i kb0[KT], kb1[KT], kb2[KT];
  if constexpr (PG) {
    load_unit_at<KT>(kb0, rs, fb[0], Di);
    load_unit_at<KT>(kb1, rs, fb[1], Di);
    if constexpr (D == 3) load_unit_at<KT>(kb2, rs, fb[2], Di);
  } else {
    load_unit<KT>(kb0, rs, wave, js, Di);
    load_unit<KT>(kb1, rs, wave + kScoreWaves, js, Di);
    if constexpr (D == 3) load_unit<KT>(kb2, rs, wave + 2 * kScoreWaves, js, Di);
  }

  // the query into LDS: head h's dims [0, Di), then zeros for dims [Di, DI) (the
  // last key fragment's upper half there reads the next key's dims or zeros)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pc = tid + kScoreBlock * u;
    if (pc < npc) {
      const int h = (16 * pc) / Di, d = 16 * pc - h * Di;
      *reinterpret_cast<v4i*>(qs + h * DIP + d) = qp[u];
    }
  }
  if (Di < DI && tid < Hi) *reinterpret_cast<v4i*>(qs + tid * DIP + Di) = v4i{0, 0, 0, 0};
  if (wave == 0) wsm[lane] = lane < Hi ? wl : 0;
  if constexpr (PG)
    if (tid < units) uoff[tid] = base_of(tid, ue);
  lds_barrier();
  v4i qreg[MT][KT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      qreg[mt][kt] = *reinterpret_cast<const v4i*>(qs + (32 * mt + (lane & 31)) * DIP + 32 * kt + 16 * (lane >> 5));

  // weights in accumulator order: value r of tile mt at lane l is head
  // 32mt + 8(r / 4) + 4(l >> 5) + r % 4 (four consecutive heads a read); padding
  // heads (q = 0) have weight 0
  int wreg[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const v4i wd = *reinterpret_cast<const v4i*>(wsm + 32 * mt + 8 * g + 4 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; ++j) wreg[mt][4 * g + j] = wd[j];
    }
    if (32 * mt + (lane & 31) >= Hi)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) qreg[mt][kt] = v4i{0, 0, 0, 0};
  }

  // Unit j of the chunk in buffer kf: scores into LDS and the histogram. The
  // buffer is refilled with the next unclaimed unit (an LDS counter, so the waves
  // whose keys come back first take more of the chunk; the requests of the later
  // waves otherwise queue behind theirs every round) and j becomes that unit, which
  // is past the chunk's end once every unit is taken (its loads then return zeros).
  // A buffer whose unit is past the end is only refilled; the refill is issued
  // on both paths between the products and the rest (an if/else around it would
  // let the compiler hoist it into fresh registers and copy them back every
  // iteration, which waits for every load).
  auto unit = [&](v4i(&kf)[KT], int& j) {
    uint32_t nxt = 0;
    if (lane == 0) nxt = atomicAdd(&rsm.next, 1u);  // back during the matrix products
    const bool live = j < units;                    // uniform over the wave
    v16i acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v16i{};
    if (live) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qreg[mt][kt], kf[kt], acc[mt], 0, 0, 0);
    }
    const int jn = __builtin_amdgcn_readfirstlane((int)nxt);
    if constexpr (PG)
      load_unit_at<KT>(kf, rs, jn < units ? uoff[jn] : pool_bytes, Di);
    else
      load_unit<KT>(kf, rs, jn, js, Di);
    if (live) {
      // two independent multiply-add chains (left to itself the compiler pairs the
      // products with three-input adds, 2.5 instructions per head instead of 2)
      int p0 = 0, p1 = 0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int v0 = acc[mt][r], v1 = acc[mt][r + 1];
          p0 = mad_i24(wreg[mt][r], v0 > 0 ? v0 : 0, p0);
          p1 = mad_i24(wreg[mt][r + 1], v1 > 0 ? v1 : 0, p1);
        }
      // lanes l and l ^ 32 hold the same key's other heads: one lane-half swap
      const int ph = p0 + p1;
      const auto sw = __builtin_amdgcn_permlane32_swap(ph, ph, false, false);
      const int part = sw[0] + sw[1];
      const int p = kUnit * j + (lane & 31);
      if (lane < 32) {
        sc[p] = part;
        if (p < count) {
          const uint32_t bn = score_bin(part);
          atomicAdd(&hist[bn], 1u);
          atomicAdd(&hgroup[bn >> 4], 1u);
        }
      }
    }
    j = jn;
  };

  // The buffers rotate by name (a register copy would wait for its load) and are
  // taken in the order their loads were issued, every iteration the same, and the
  // loop only exits at its head. Claimed units increase, so j0 < j1 (< j2)
  // throughout: once j0 is past the end, so are the others.
  int j0 = wave, j1 = wave + kScoreWaves, j2 = wave + 2 * kScoreWaves;
  while (j0 < units) {
    unit(kb0, j0);
    unit(kb1, j1);
    if constexpr (D == 3) unit(kb2, j2);
  }
  lds_barrier();  // every score and histogram count of the chunk is in LDS

  const int m = a.m;
  const CandOut out{a.cand + (int64_t)b * kCandCap, c * m};
  uint64_t* xout = a.xc + (int64_t)b * G + c;
  // the scores leave for HBM as they are read below (raw buffer stores against a
  // resource that covers exactly the chunk's valid positions: the padding is
  // dropped without a branch); nothing waits for these stores
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + (int64_t)b * a.N + cbeg, (short)0, span * 4, 0x00020000);
  // row position of local entry i, and its offset from the chunk's first position
  auto rel = [&](int i) { return (uint32_t)(i >> 5) * ustride + (uint32_t)(i & 31); };
  const uint64_t lt = lanemask_lt();
  if (count <= m) {  // every valid position is a candidate
    for (int i = tid; i < m; i += kScoreBlock) {
      const int32_t v = sc[i < units * kUnit ? i : 0];
      if (i < units * kUnit) __builtin_amdgcn_raw_buffer_store_b32(v, rsc, 4 * rel(i), 0, 0);
      out.put(i, i < count ? make_key(v, (uint32_t)cbeg + rel(i)) : 0ull);
    }
    if (tid == 0) *xout = 0;
    if (a.sums != nullptr && wave == 0) {  // m <= 64: the first wave covers the list
      const bool v = lane < count;
      const uint32_t u = v ? score_bits(sc[lane]) : 0u;
      const uint32_t lo = wave_min_u32(v ? u : 0xFFFFFFFFu), hi = wave_maxr_u32(u);
      // position order: best first only when at most one key is present
      if (lane == 0) a.sums[(int64_t)b * kMaxChunks + c] = ChunkSum{lo, hi, count <= 1 ? 1u : 0u, 0u};
    }
    return;
  }

  // 1. every wave finds the bin that holds the (m+1)-th best key (same result in each)
  int32_t tlo = 0;
  const bool hok = hist_threshold(hist, hgroup, count, (uint32_t)m + 1, &tlo);
  // 2. every key scoring at least that bin's floor is staged, in order of arrival
  //    (the ranks below fix the output order): four positions per thread per pass
  for (int i0 = 0; i0 < units * kUnit; i0 += 4 * kScoreBlock) {
    int32_t v[4];
    uint64_t bal[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // every read before any use
      const int i = i0 + tid + kScoreBlock * q;
      v[q] = sc[i < units * kUnit ? i : 0];
    }
    uint32_t nb = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + tid + kScoreBlock * q;
      __builtin_amdgcn_raw_buffer_store_b32(v[q], rsc, 4 * rel(i), 0, 0);
      bal[q] = __ballot(i < count && v[q] >= tlo);
      nb += (uint32_t)__popcll(bal[q]);
    }
    if (nb == 0) continue;
    uint32_t slot = 0;
    if (lane == 0) slot = atomicAdd(&rsm.nstaged, nb);
    slot = (uint32_t)__builtin_amdgcn_readfirstlane((int)slot);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + tid + kScoreBlock * q;
      const uint32_t at = slot + (uint32_t)__popcll(bal[q] & lt);
      if (((bal[q] >> lane) & 1ull) && at < (uint32_t)kRowStage) rsm.all[at] = make_key(v[q], (uint32_t)cbeg + rel(i));
      slot += (uint32_t)__popcll(bal[q]);
    }
  }
  lds_barrier();
  const uint32_t total = rsm.nstaged;
  const bool fast = hok && total <= (uint32_t)m + 64;  // uniform over the block
  if (fast) {
    // 3. rank of staged key t = number of staged keys above it (eight threads per
    //    key when at most 64 keys are staged, the usual case, else four). Staged
    //    keys are distinct and include the m + 1 best, so ranks 0 .. m are the
    //    chunk's m + 1 best keys in order: rank r < m goes to slot r of the output
    //    (best first; keys of equal score stay in position order), and rank m is
    //    x, the best key left out.
    const bool wide = total <= 64u;  // uniform
    const int tpk = wide ? 8 : 4, t = tid / tpk, part = tid % tpk;
    uint32_t r = 0;
    uint64_t me = 0;
    if (t < (int)total) {
      me = rsm.all[t];
      for (int s0 = 0; s0 < (int)total; s0 += 4 * tpk) {
        uint64_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = rsm.all[s0 + part + tpk * u];  // < kRowStage
#pragma unroll
        for (int u = 0; u < 4; ++u) r += (s0 + part + tpk * u < (int)total && v[u] > me) ? 1u : 0u;
      }
    }
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor1, 0xF, 0xF, false);
    r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kQuadXor2, 0xF, 0xF, false);
    if (wide) r += (uint32_t)__builtin_amdgcn_mov_dpp((int)r, dpp::kRowHalfMirror, 0xF, 0xF, false);
    if (part == 0 && t < (int)total) {
      if (r < (uint32_t)m) out.put((int)r, me);
      else if (r == (uint32_t)m) *xout = me;
      if (a.sums != nullptr) {  // the list runs best first: its ends give the range
        ChunkSum* cs = a.sums + (int64_t)b * kMaxChunks + c;
        if (r == 0) {
          cs->hi = key_ubits(me);
          cs->ordered = 1u;
        }
        if (r == (uint32_t)m - 1) cs->lo = key_ubits(me);
      }
    }
  } else {
    // heavy ties at the threshold: exact radix selection over the chunk's scores
    radix_clear<kScoreBlock>(csm.radix);
    lds_barrier();
    chunk_candidates<kScoreBlock>(sc, count, (uint32_t)cbeg, m, out, xout, csm, ustride);
    // a list in position order; the whole score range bounds it
    if (a.sums != nullptr && tid == 0)
      a.sums[(int64_t)b * kMaxChunks + c] = ChunkSum{0u, 0xFFFFFFFFu, 0u, 0u};
  }
}

// The contiguous score kernels are instantiated, and so laid out in the code object,
// ahead of the paged ones (as in select.hip: a kernel's place in the code object
// changes its time, and this keeps changes to the paged kernels from moving these).
#define DSA_ROW(M, K) (const void*)&k_score_row<M, K, kScoreRowDepth, false>,
#define DSA_MK(M, K)                                                                                      \
  (const void*)&k_score<M, K, true, false, 1, false>, (const void*)&k_score<M, K, true, true, 3, false>,   \
      (const void*)&k_score<M, K, true, false, 3, false>, (const void*)&k_score<M, K, false, true, 3, false>, \
      (const void*)&k_score<M, K, false, false, 3, false>,
#define DSA_ALL(X) X(1, 1) X(1, 2) X(1, 3) X(1, 4) X(1, 5) X(1, 6) X(1, 7) X(1, 8) \
  X(2, 1) X(2, 2) X(2, 3) X(2, 4) X(2, 5) X(2, 6) X(2, 7) X(2, 8)
const void* score_order(int i) {
  static const void* const k[] = {DSA_ALL(DSA_ROW) DSA_ALL(DSA_MK)};
  return k[i];
}
#undef DSA_ROW
#undef DSA_MK
#undef DSA_ALL

size_t score_row_lds_bytes(int P, bool paged) {
  // ... + the staged query at its largest (64 heads, rows of 256 + 16 bytes), the
  // weights and, paged, the units' pool offsets
  return align16(sizeof(ChunkSmem<kScoreBlock>)) + align16((size_t)P * 4) + (size_t)(kHistBins + kHistGroups) * 4 +
         align16(sizeof(RowCandSmem)) + (size_t)64 * (256 + 16) + 64 * 4 + (paged ? (size_t)kMaxUnits * 4 : 0) + 16;
}

int score_row_max_chunk() { return kMaxUnits * kUnit; }

template <int MT, int KT>
static hipError_t launch_score_row_t(const ScoreArgs& a, int grid, hipStream_t s, KTimer t) {
  const bool paged = a.pages != nullptr;
  auto fn = paged ? k_score_row<MT, KT, kScoreRowDepth, true> : k_score_row<MT, KT, kScoreRowDepth, false>;
  const size_t lds = score_row_lds_bytes(a.P, paged);
  hipError_t e = allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  return launch_timed(fn, dim3(grid), dim3(kScoreBlock), lds, s, t, a.iq, a.iw, a.ik, a.pages, a.lens.n[0], a.G, a.P,
                      a.Hi | a.Di << 16, a);
}

hipError_t launch_score_row(const ScoreArgs& a, int MT, int KT, int grid, hipStream_t s, KTimer t) {
#define DSA_SCORE_ROW_CASE(M, K) \
  if (MT == M && KT == K) return launch_score_row_t<M, K>(a, grid, s, t);
  DSA_SCORE_ROW_CASE(1, 1) DSA_SCORE_ROW_CASE(1, 2) DSA_SCORE_ROW_CASE(1, 3) DSA_SCORE_ROW_CASE(1, 4)
  DSA_SCORE_ROW_CASE(1, 5) DSA_SCORE_ROW_CASE(1, 6) DSA_SCORE_ROW_CASE(1, 7) DSA_SCORE_ROW_CASE(1, 8)
  DSA_SCORE_ROW_CASE(2, 1) DSA_SCORE_ROW_CASE(2, 2) DSA_SCORE_ROW_CASE(2, 3) DSA_SCORE_ROW_CASE(2, 4)
  DSA_SCORE_ROW_CASE(2, 5) DSA_SCORE_ROW_CASE(2, 6) DSA_SCORE_ROW_CASE(2, 7) DSA_SCORE_ROW_CASE(2, 8)
#undef DSA_SCORE_ROW_CASE
  return hipErrorInvalidValue;
}

int score_max_chunk() { return kChunkPerThread * kScoreBlock; }

size_t score_lds_bytes(int MT, int KT, int Bg, int P, bool cand, bool paged) {
  return align16(sizeof(ChunkSmem<kScoreBlock>)) + (size_t)Bg * 32 * MT * (32 * KT + 16) + (size_t)Bg * 32 * MT * 4 +
         (paged ? (size_t)kMaxTiles * 4 : 0) +
         (cand ? (size_t)Bg * P * 4 + (size_t)Bg * kHistBins * 4 + sizeof(BlockCandSmem<kScoreBlock>) +
                     (size_t)Bg * 4
               : 0) +
         16;
}

template <int MT, int KT, bool CAND, bool ONE, int NB = 3>
static hipError_t launch_score_t(const ScoreArgs& a, int grid, size_t lds, hipStream_t s, KTimer t) {
  auto fn = a.pages != nullptr ? k_score<MT, KT, CAND, ONE, NB, true> : k_score<MT, KT, CAND, ONE, NB, false>;
  hipError_t e = allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  return launch_timed(fn, dim3(grid), dim3(kScoreBlock), lds, s, t, a);
}

template <int MT, int KT>
static hipError_t launch_score_mk(const ScoreArgs& a, bool cand, int grid, size_t lds, hipStream_t s,
                                  KTimer t) {
  const bool one = a.Bg == 1;
  // several rows with candidates: one key tile per wave when the chunk has at most
  // kScoreWaves tiles of 64 keys
  if (cand && !one && (a.P + 63) / 64 <= kScoreWaves) return launch_score_t<MT, KT, true, false, 1>(a, grid, lds, s, t);
  if (cand) return one ? launch_score_t<MT, KT, true, true>(a, grid, lds, s, t)
                       : launch_score_t<MT, KT, true, false>(a, grid, lds, s, t);
  return one ? launch_score_t<MT, KT, false, true>(a, grid, lds, s, t)
             : launch_score_t<MT, KT, false, false>(a, grid, lds, s, t);
}

hipError_t launch_score(const ScoreArgs& a, int MT, int KT, bool cand, int grid, hipStream_t s, KTimer t) {
  // paged: a chunk's tiles must fit the kernel's list of tile offsets
  if (a.pages != nullptr && (a.P + 63) / 64 > kMaxTiles) return hipErrorInvalidValue;
  const size_t lds = score_lds_bytes(MT, KT, a.Bg, a.P, cand, a.pages != nullptr);
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

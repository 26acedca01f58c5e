// C entry points of libdsa: host-side validation, workspace layout and launch
// planning. Every check runs before anything is enqueued; nothing here allocates
// device memory or synchronises (except dsa_read_stats, documented as such).
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/dsa.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Attention splits per row: 64 selected rows per split on the vector-ALU paths;
// 32 on the matrix-core path (more workgroups, each with half the serial work).
// With B rows, the count is halved (each split taking twice the rows, at most
// kMaxSplitRows) while the B rows' splits would exceed kSplitGrid workgroups: a
// split's rows are a serial loop, and a second round of workgroups costs more
// than a longer loop (one workgroup per compute unit fits the selection's LDS).
int splits_for(int k, bool mfma = false, int B = 1) {
  int s = mfma ? (k + 31) / 32 : (k + 63) / 64;
  const int cap = mfma ? kMaxWideSplits : kMaxSplits;
  s = s < 1 ? 1 : (s > cap ? cap : s);
  while (s > 1 && s * B > kSplitGrid) {
    const int h = (s + 1) / 2;
    if ((k + h - 1) / h > kMaxSplitRows) break;
    s = h;
  }
  return s;
}
int rankers_for(int k) {
  int r = (k + 15) / 16;
  return r < 1 ? 1 : (r > kMaxRankBlocks ? kMaxRankBlocks : r);
}

// Byte offsets of the workspace regions.
struct Layout {
  size_t stats, cand, xc, sums, ml, o, bad, total;
};
Layout layout(int B, int64_t N, int k, int Hq, int Dv) {
  const int S = splits_for(k, true);  // the larger of the two split counts
  Layout L;
  L.stats = 0;
  L.cand = up(sizeof(RowStats) * kMaxBatch);
  L.xc = L.cand + up((size_t)B * kCandCap * 8);
  L.sums = L.xc + up((size_t)B * kMaxChunks * 8);
  L.ml = L.sums + up((size_t)B * kMaxChunks * sizeof(ChunkSum));
  L.o = L.ml + up((size_t)B * S * Hq * 8);
  L.bad = L.o + up((size_t)B * S * ((Hq + 15) / 16 * 16) * Dv * 4);
  L.total = L.bad + up((size_t)B * S * 4);
  return L;
}

// LDS bytes a workgroup may use on the current device (gfx950: 160 KiB; that value
// is also assumed when no device can be queried, so host-only validation behaves
// as on the GPU).
int lds_limit() {
  constexpr int kGfx950Lds = 160 * 1024;
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kGfx950Lds;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0)
      v = kGfx950Lds;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct LdsAllowed {
  const void* fn;
  int dev;
  size_t lds;
};
std::mutex g_lds_mu;
std::vector<LdsAllowed> g_lds_allowed;  // one entry per kernel and device launched

}  // namespace

hipError_t allow_lds(const void* fn, size_t lds) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  {
    std::lock_guard<std::mutex> g(g_lds_mu);
    for (const LdsAllowed& e : g_lds_allowed)
      if (e.fn == fn && e.dev == dev && e.lds >= lds) return hipSuccess;
  }
  const hipError_t r = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (r != hipSuccess) return r;
  std::lock_guard<std::mutex> g(g_lds_mu);
  for (LdsAllowed& e : g_lds_allowed)
    if (e.fn == fn && e.dev == dev) {
      e.lds = e.lds > lds ? e.lds : lds;
      return hipSuccess;
    }
  g_lds_allowed.push_back(LdsAllowed{fn, dev, lds});
  return hipSuccess;
}

namespace {

dsa_status check_rows(const int32_t* ctx_len, int B, int64_t N, RowLens* lens, int* nmax) {
  if (ctx_len == nullptr || B < 1 || B > DSA_MAX_BATCH || N < 1 || N > INT32_MAX)
    return DSA_ERR_INVALID_ARG;
  memset(lens, 0, sizeof(*lens));
  int mx = 0;
  for (int b = 0; b < B; ++b) {
    if (ctx_len[b] < 1 || (int64_t)ctx_len[b] > N) return DSA_ERR_INVALID_ARG;
    lens->n[b] = ctx_len[b];
    mx = ctx_len[b] > mx ? ctx_len[b] : mx;
  }
  *nmax = mx;
  return DSA_OK;
}

// Indexer shapes: Hi >= 1 and Di a positive multiple of 16 are valid; the kernels
// are built for Hi <= 64 and Di <= 256 (DSA_ERR_UNSUPPORTED beyond).
dsa_status check_index(const int8_t* iq, const int8_t* iw, const int8_t* ik, int Hi, int Di) {
  if (!iq || !iw || !ik) return DSA_ERR_INVALID_ARG;
  if (Hi < 1 || Di < 16 || Di % 16 != 0) return DSA_ERR_INVALID_ARG;
  if (!aligned(iq, 16) || !aligned(ik, 16)) return DSA_ERR_INVALID_ARG;
  if (Hi > DSA_MAX_INDEX_HEADS || Di > DSA_MAX_INDEX_DIM) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status check_attn(const void* q, const void* kv, int Hq, int Dk, int Dv, float scale,
                      dsa_dtype dt, AttnChoice* ch) {
  // valid: Hq >= 1, Dk a positive multiple of 8, 1 <= Dv <= Dk; built: Hq <= 64, Dk <= 1024
  if (!q || !kv) return DSA_ERR_INVALID_ARG;
  if (Hq < 1 || Dk < 8 || Dk % 8 != 0 || Dv < 1 || Dv > Dk) return DSA_ERR_INVALID_ARG;
  if (dt != DSA_F32 && dt != DSA_BF16 && dt != DSA_FP8_E4M3) return DSA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16)) return DSA_ERR_INVALID_ARG;
  if (Hq > DSA_MAX_ATTN_HEADS || Dk > DSA_MAX_ATTN_DIM) return DSA_ERR_UNSUPPORTED;
  static_assert((int)DSA_F32 == DT_F32 && (int)DSA_BF16 == DT_BF16 && (int)DSA_FP8_E4M3 == DT_BF16_Q_E4M3_KV,
                "dtype codes");
  *ch = choose_attn((int)dt, Hq, Dk, Dv);
  if (ch->kind == ATTN_NONE) return DSA_ERR_UNSUPPORTED;
  if (select_lds_bytes(*ch, Hq, Dk, DSA_MAX_K) > (size_t)lds_limit()) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status check_ws(void* ws, size_t ws_bytes, const Layout& L) {
  if (ws == nullptr || !aligned(ws, 256)) return DSA_ERR_WORKSPACE;
  if (ws_bytes < L.total) return DSA_ERR_WORKSPACE;
  return DSA_OK;
}

// A sequence's page table into a paged pool (pages == nullptr: contiguous caches).
struct Paging {
  const int32_t* pages = nullptr;
  int pool_pages = 0;
  int npages = 0;  // table entries: ceil(N / kPageSize)
};

// Paged calls: a table of ceil(N / DSA_PAGE_SIZE) entries (N <= DSA_MAX_PAGES pages'
// worth), a pool of at least one page whose rows an int32 counts, and (row_bytes > 0,
// the indexer key pool) a pool the score kernels address with 32-bit offsets.
dsa_status check_paging(const int32_t* pages, int64_t pool_pages, int64_t N, int64_t row_bytes, Paging* pg) {
  if (pages == nullptr || !aligned(pages, 4) || pool_pages < 1) return DSA_ERR_INVALID_ARG;
  if (pool_pages > INT32_MAX / kPageSize) return DSA_ERR_UNSUPPORTED;
  if (N > (int64_t)DSA_MAX_PAGES * kPageSize) return DSA_ERR_UNSUPPORTED;
  if (row_bytes > 0 && pool_pages * kPageSize * row_bytes >= ((int64_t)1 << 31)) return DSA_ERR_UNSUPPORTED;
  pg->pages = pages;
  pg->pool_pages = (int)pool_pages;
  pg->npages = (int)((N + kPageSize - 1) / kPageSize);
  return DSA_OK;
}

// Chunking of the candidate pass for rows of at most nmax positions.
struct ChunkPlan {
  int P, G, m;
  int ilv;  // 1: chunk c holds the row's 32-key units c, c + G, ... (one-row plan; row_chunk_units)
};
// One-row plan (score kernel k_score_row): chunks of whole 32-key units,
// interleaved over the row, as many chunks as candidate slots allow (at most one
// per compute unit; the chunk's waves claim its units as they go, so any count of
// units balances). (cand_fits takes the plan only when a chunk fits the kernel,
// which bounds a row to 2^21 positions, so every key offset fits a buffer offset.)
ChunkPlan chunk_plan_row(int nmax, int k, int Di) {
  ChunkPlan c;
  c.m = k <= 2048 ? 32 : 64;
  c.ilv = 1;
  const int gmax = kCandCap / c.m < kMaxChunks ? kCandCap / c.m : kMaxChunks;
  const int64_t units = ((int64_t)nmax + 31) / 32;
  const int64_t per = (units + gmax - 1) / gmax;
  c.P = (int)(per * 32);
  c.G = (int)(((int64_t)nmax + c.P - 1) / c.P);
  return c;
}

ChunkPlan chunk_plan(int nmax, int k, bool row, int Di) {
  if (row) return chunk_plan_row(nmax, k, Di);
  ChunkPlan c;
  c.ilv = 0;
  if (nmax <= kCandCap) {  // short rows: every position is a candidate
    c.P = 64;
    c.m = 64;
    c.G = (nmax + 63) / 64;
    return c;
  }
  c.m = k <= 2048 ? 32 : 64;
  const int gmax = kCandCap / c.m;
  const int64_t per = ((int64_t)nmax + gmax - 1) / gmax;
  c.P = (int)((per + 63) / 64 * 64);
  c.G = (int)(((int64_t)nmax + c.P - 1) / c.P);
  return c;
}

int rows_per_score_launch(int Hi, int Di, int B) {
  const int hp = (Hi + 31) / 32 * 32;  // Hi <= 64 and Di <= 256 give at least 4 rows
  const int dp = (Di + 31) / 32 * 32;  // staged with whole 32-dim steps
  int bg = kScoreQBytes / (hp * dp);
  bg = bg < 1 ? 1 : bg;
  bg = bg * hp > 512 ? 512 / hp : bg;  // one head weight per thread of the block
  return bg < B ? bg : B;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Scratch of dsa_decode_step_noalloc: one array per device, held for the life of the
// process. Host code uses only the device address returned by hipGetSymbolAddress
// (the array's name is a host-side stand-in there), looked up once per device with
// that device current.
constexpr size_t kScratchBytes = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_lock;

// The current device's scratch address, or nullptr if it cannot be resolved.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> hold(g_scratch_lock);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}


dsa_status run_scores(const int8_t* iq, const int8_t* iw, const int8_t* ik, const RowLens& lens,
                      int B, int Hi, int Di, int64_t N, int nmax, int32_t* scores, bool cand,
                      const ChunkPlan& cp, uint64_t* cbuf, uint64_t* xbuf, hipStream_t s,
                      KTimer t = {}, ChunkSum* sums = nullptr, Paging pg = {}) {
  ScoreArgs a;
  a.pages = pg.pages;
  a.pool_pages = pg.pool_pages;
  a.iq = iq;
  a.iw = iw;
  a.ik = ik;
  a.scores = scores;
  a.cand = cbuf;
  a.xc = xbuf;
  a.sums = nullptr;
  a.lens = lens;
  a.N = N;
  a.nmax = nmax;
  a.Hi = Hi;
  a.Di = Di;
  a.m = cp.m;
  if (cand) {
    a.P = cp.P;
    a.G = cp.G;
  } else {
    a.P = (int)((((int64_t)nmax + 64 * 2048 - 1) / (64 * 2048)) * 64);
    a.G = (int)(((int64_t)nmax + a.P - 1) / a.P);
  }
  const int MT = (Hi + 31) / 32, KT = (Di + 31) / 32;
  if (cand && B == 1) {  // the decode hot path: one row, candidates on
    a.b0 = 0;
    a.Bg = 1;
    a.sums = sums;
    return hip_status(launch_score_row(a, MT, KT, a.G, s, t));
  }
  const int bg = rows_per_score_launch(Hi, Di, B);
  for (int b0 = 0; b0 < B; b0 += bg) {
    a.b0 = b0;
    a.Bg = B - b0 < bg ? B - b0 : bg;
    KTimer tl;  // the first launch starts the stage's time, the last one ends it
    if (b0 == 0) tl.start = t.start;
    if (b0 + bg >= B) tl.stop = t.stop;
    hipError_t e = launch_score(a, MT, KT, cand, a.G, s, tl);
    if (e != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

bool cand_fits(int Hi, int Di, int B, const ChunkPlan& cp, bool fused, bool paged = false) {
  size_t need;
  if (fused && B == 1) {
    if (cp.P > score_row_max_chunk()) return false;
    // the kernel addresses a chunk's keys, interleaved over the row, by 32-bit offsets
    // (a paged pool's size is checked against the same bound by check_paging)
    if (!paged && (int64_t)cp.G * cp.P * Di >= ((int64_t)1 << 31)) return false;
    need = score_row_lds_bytes(cp.P, paged);
  } else if (fused) {
    if (cp.P > score_max_chunk()) return false;
    const int bg = rows_per_score_launch(Hi, Di, B);
    need = score_lds_bytes((Hi + 31) / 32, (Di + 31) / 32, bg, cp.P, true, paged);
  } else {
    if (cp.P > chunk_cand_max_chunk()) return false;
    need = 8192 + (size_t)cp.P * 4;
  }
  return need <= (size_t)lds_limit();
}

AttnArgs attn_args(const void* q, const void* kv, int64_t N, int Hq, int Dk, int Dv, float scale,
                   int k, uint8_t* w, const Layout& L, Paging pg = {}) {
  AttnArgs at;
  at.pages = pg.pages;
  at.pool_pages = pg.pool_pages;
  at.lds_pages = 0;
  at.q = q;
  at.kv = kv;
  at.N = N;
  at.Hq = Hq;
  at.Dk = Dk;
  at.Dv = Dv;
  at.scale = scale;
  at.part_ml = reinterpret_cast<float2*>(w + L.ml);
  at.part_o = reinterpret_cast<float*>(w + L.o);
  at.S = splits_for(k);
  at.frag = 0;
  return at;
}

// Split count and partial layout for the chosen attention path.
void set_attn_path(AttnArgs* at, const AttnChoice& ch, int k, int B) {
  at->frag = ch.kind == ATTN_MFMA_BF16;
  at->S = splits_for(k, at->frag != 0, B);
}

hipError_t combine(const AttnArgs& at, const int32_t* part_bad, RowStats* stats, float* out, int B,
                   hipStream_t s, KTimer t = {}) {
  if (at.S > kMaxSplits) return launch_combine_wide(at, part_bad, stats, out, B, s, t);
  return launch_combine(at, part_bad, stats, out, B, s, t);
}

SelArgs sel_args(const int32_t* scores, const RowLens& lens, int64_t N, int k, int32_t* idx,
                 uint8_t* w, const Layout& L, const ChunkPlan& cp, bool have_cand, unsigned flags,
                 bool sums = false) {
  SelArgs a;
  a.scores = scores;
  a.cand = reinterpret_cast<const uint64_t*>(w + L.cand);
  a.xc = reinterpret_cast<const uint64_t*>(w + L.xc);
  a.sums = sums && have_cand ? reinterpret_cast<const ChunkSum*>(w + L.sums) : nullptr;
  a.idx = idx;
  a.stats = reinterpret_cast<RowStats*>(w + L.stats);
  a.lens = lens;
  a.N = N;
  a.k = k;
  a.G = cp.G;
  a.m = cp.m;
  a.have_cand = have_cand ? cp.P : 0;
  memset(&a.cand_valid, 0, sizeof(a.cand_valid));
  for (int b = 0; b < kMaxBatch; ++b) {  // each chunk keeps min(m, its valid positions)
    int64_t v = 0;
    for (int c = 0; c < cp.G && have_cand && lens.n[b] > 0; ++c) {
      int cnt;
      row_chunk_units(lens.n[b], c, cp.G, cp.P, cp.ilv, &cnt);
      v += cnt < cp.m ? cnt : cp.m;
    }
    a.cand_valid.n[b] = (int32_t)v;
  }
  a.force = (flags & DSA_FLAG_FORCE_FALLBACK) ? 1 : 0;
  a.R = rankers_for(k);
  return a;
}

// The three calls on contiguous caches (pages == nullptr) or, through a page table,
// on paged pools (ik and kv are then the pools).
dsa_status index_scores_impl(const int8_t* iq, const int8_t* iw, const int8_t* ik, const int32_t* ctx_len, int B,
                             int Hi, int Di, int64_t N, int32_t* scores, hipStream_t stream,
                             const int32_t* pages, int64_t pool_pages) {
  RowLens lens;
  int nmax = 0;
  dsa_status st = check_rows(ctx_len, B, N, &lens, &nmax);
  if (st != DSA_OK) return st;
  if ((st = check_index(iq, iw, ik, Hi, Di)) != DSA_OK) return st;
  if (!scores || !aligned(scores, 4)) return DSA_ERR_INVALID_ARG;
  Paging pg;
  if (pages != nullptr && (st = check_paging(pages, pool_pages, N, Di, &pg)) != DSA_OK) return st;
  ChunkPlan cp{64, 1, 32, 0};
  return run_scores(iq, iw, ik, lens, B, Hi, Di, N, nmax, scores, false, cp, nullptr, nullptr,
                    stream, {}, nullptr, pg);
}

dsa_status sparse_attn_impl(const void* q, const void* kv, const int32_t* idx, int B, int Hq, int Dk, int Dv,
                            int64_t N, int k, float scale, dsa_dtype dt, float* out, void* ws, size_t ws_bytes,
                            hipStream_t stream, const int32_t* pages, int64_t pool_pages) {
  if (B < 1 || B > DSA_MAX_BATCH || N < 1 || N > INT32_MAX || k < 1 || k > DSA_MAX_K || !idx || !out)
    return DSA_ERR_INVALID_ARG;
  AttnChoice ch;
  dsa_status st = check_attn(q, kv, Hq, Dk, Dv, scale, dt, &ch);
  if (st != DSA_OK) return st;
  Paging pg;
  if (pages != nullptr && (st = check_paging(pages, pool_pages, N, 0, &pg)) != DSA_OK) return st;
  const Layout L = layout(B, N, k, Hq, Dv);
  if ((st = check_ws(ws, ws_bytes, L)) != DSA_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(ws);
  AttnArgs at = attn_args(q, kv, N, Hq, Dk, Dv, scale, k, w, L, pg);
  set_attn_path(&at, ch, k, B);
  int32_t* bad = reinterpret_cast<int32_t*>(w + L.bad);
  if (launch_attend_idx(idx, k, bad, at, ch, B, stream) != hipSuccess) return DSA_ERR_HIP;
  return hip_status(combine(at, bad, reinterpret_cast<RowStats*>(w + L.stats), out, B, stream));
}

dsa_status decode_step_impl(const int8_t* iq, const int8_t* iw, const int8_t* ik, const void* q, const void* kv,
                            const int32_t* ctx_len, int B, int Hi, int Di, int Hq, int Dk, int Dv, int64_t N,
                            int k, float scale, dsa_dtype dt, int32_t* scores, int32_t* idx, float* out, void* ws,
                            size_t ws_bytes, unsigned flags, hipStream_t stream, hipEvent_t* kernel_events,
                            const int32_t* pages, int64_t pool_pages) {
  RowLens lens;
  int nmax = 0;
  dsa_status st = check_rows(ctx_len, B, N, &lens, &nmax);
  if (st != DSA_OK) return st;
  if ((st = check_index(iq, iw, ik, Hi, Di)) != DSA_OK) return st;
  const unsigned known = DSA_FLAG_FORCE_FALLBACK | (pages != nullptr ? DSA_FLAG_TABLE_IN_MEMORY : 0u);
  if (!scores || !idx || !out || k < 1 || k > DSA_MAX_K || (flags & ~known)) return DSA_ERR_INVALID_ARG;
  AttnChoice ch;
  if ((st = check_attn(q, kv, Hq, Dk, Dv, scale, dt, &ch)) != DSA_OK) return st;
  Paging pg;
  if (pages != nullptr && (st = check_paging(pages, pool_pages, N, Di, &pg)) != DSA_OK) return st;
  const Layout L = layout(B, N, k, Hq, Dv);
  if ((st = check_ws(ws, ws_bytes, L)) != DSA_OK) return st;
  KTimer tm[3];
  if (kernel_events != nullptr) {
    for (int i = 0; i < 6; ++i)
      if (kernel_events[i] == nullptr) return DSA_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i) tm[i] = KTimer{kernel_events[2 * i], kernel_events[2 * i + 1]};
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  const ChunkPlan cp = chunk_plan(nmax, k, B == 1, Di);
  // (the forced exhaustive path still gets the candidate score pass: it changes the
  // selection only, and its narrowing takes a threshold from the union)
  const bool have = cand_fits(Hi, Di, B, cp, true, pg.pages != nullptr);
  // the one-row score pass also leaves per-chunk summaries for the selection
  const bool sums = have && B == 1;
  st = run_scores(iq, iw, ik, lens, B, Hi, Di, N, nmax, scores, have, cp,
                  reinterpret_cast<uint64_t*>(w + L.cand), reinterpret_cast<uint64_t*>(w + L.xc),
                  stream, tm[0], sums ? reinterpret_cast<ChunkSum*>(w + L.sums) : nullptr, pg);
  if (st != DSA_OK) return st;
  SelArgs sa = sel_args(scores, lens, N, k, idx, w, L, cp, have, flags, sums);
  // no ranking workgroups: the attention splits' windows are the output slots, so
  // they write the indices and the row's record themselves
  sa.R = 0;
  AttnArgs at = attn_args(q, kv, N, Hq, Dk, Dv, scale, k, w, L, pg);
  set_attn_path(&at, ch, k, B);
  // a paged latent cache: the selection kernel stages the table in LDS when it fits
  if (pg.pages != nullptr && !(flags & DSA_FLAG_TABLE_IN_MEMORY) &&
      select_lds_bytes(ch, Hq, Dk, k) + align16((size_t)pg.npages * 4) <= (size_t)lds_limit())
    at.lds_pages = pg.npages;
  if (launch_select(sa, at, ch, B, stream, tm[1]) != hipSuccess) return DSA_ERR_HIP;
  return hip_status(combine(at, nullptr, nullptr, out, B, stream, tm[2]));
}

}  // namespace
}  // namespace dsa

using namespace dsa;

extern "C" {

const char* dsa_status_string(dsa_status status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: an argument is out of range";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape outside the built kernels";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: the HIP runtime refused a launch";
  }
  return "unknown dsa_status";
}

size_t dsa_workspace_size(int B, int64_t N, int k, int Hq, int Dv) {
  if (B < 1 || B > DSA_MAX_BATCH || N < 1 || N > INT32_MAX || k < 1 || k > DSA_MAX_K || Hq < 1 ||
      Hq > DSA_MAX_ATTN_HEADS || Dv < 1 || Dv > DSA_MAX_ATTN_DIM)
    return 0;
  return layout(B, N, k, Hq, Dv).total;
}

dsa_status dsa_index_scores(const int8_t* iq, const int8_t* iw, const int8_t* ik,
                            const int32_t* ctx_len, int B, int Hi, int Di, int64_t N,
                            int32_t* scores, hipStream_t stream) {
  return index_scores_impl(iq, iw, ik, ctx_len, B, Hi, Di, N, scores, stream, nullptr, 0);
}

dsa_status dsa_index_scores_paged(const int8_t* iq, const int8_t* iw, const int8_t* ik_pool,
                                  const int32_t* page_table, int64_t pool_pages, const int32_t* ctx_len,
                                  int B, int Hi, int Di, int64_t N, int32_t* scores, hipStream_t stream) {
  if (page_table == nullptr) return DSA_ERR_INVALID_ARG;
  return index_scores_impl(iq, iw, ik_pool, ctx_len, B, Hi, Di, N, scores, stream, page_table, pool_pages);
}

dsa_status dsa_topk_select(const int32_t* scores, const int32_t* ctx_len, int B, int64_t N, int k,
                           int32_t* idx, void* ws, size_t ws_bytes, unsigned flags,
                           hipStream_t stream) {
  RowLens lens;
  int nmax = 0;
  dsa_status st = check_rows(ctx_len, B, N, &lens, &nmax);
  if (st != DSA_OK) return st;
  if (!scores || !idx || k < 1 || k > DSA_MAX_K || (flags & ~DSA_FLAG_FORCE_FALLBACK))
    return DSA_ERR_INVALID_ARG;
  const Layout L = layout(B, N, k, 1, 1);
  if ((st = check_ws(ws, ws_bytes, L)) != DSA_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const ChunkPlan cp = chunk_plan(nmax, k, false, 0);
  const bool have = cand_fits(0, 32, B, cp, false) && !(flags & DSA_FLAG_FORCE_FALLBACK);
  if (have) {
    CandArgs ca;
    ca.scores = scores;
    ca.cand = reinterpret_cast<uint64_t*>(w + L.cand);
    ca.xc = reinterpret_cast<uint64_t*>(w + L.xc);
    ca.lens = lens;
    ca.N = N;
    ca.P = cp.P;
    ca.G = cp.G;
    ca.m = cp.m;
    if (launch_chunk_candidates(ca, B, stream) != hipSuccess) return DSA_ERR_HIP;
  }
  const SelArgs sa = sel_args(scores, lens, N, k, idx, w, L, cp, have, flags);
  AttnArgs at{};
  at.S = 0;
  return hip_status(launch_select(sa, at, AttnChoice{ATTN_NONE, 0, 0, 0, 0}, B, stream));
}

dsa_status dsa_sparse_attn(const void* q, const void* kv, const int32_t* idx, int B, int Hq, int Dk,
                           int Dv, int64_t N, int k, float scale, dsa_dtype dt, float* out,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return sparse_attn_impl(q, kv, idx, B, Hq, Dk, Dv, N, k, scale, dt, out, ws, ws_bytes, stream, nullptr, 0);
}

dsa_status dsa_sparse_attn_paged(const void* q, const void* kv_pool, const int32_t* page_table,
                                 int64_t pool_pages, const int32_t* idx, int B, int Hq, int Dk, int Dv,
                                 int64_t N, int k, float scale, dsa_dtype dt, float* out, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (page_table == nullptr) return DSA_ERR_INVALID_ARG;
  return sparse_attn_impl(q, kv_pool, idx, B, Hq, Dk, Dv, N, k, scale, dt, out, ws, ws_bytes, stream, page_table,
                          pool_pages);
}

dsa_status dsa_decode_step_timed(const int8_t* iq, const int8_t* iw, const int8_t* ik,
                                 const void* q, const void* kv, const int32_t* ctx_len, int B,
                                 int Hi, int Di, int Hq, int Dk, int Dv, int64_t N, int k,
                                 float scale, dsa_dtype dt, int32_t* scores, int32_t* idx,
                                 float* out, void* ws, size_t ws_bytes, unsigned flags,
                                 hipStream_t stream, hipEvent_t* kernel_events) {
  return decode_step_impl(iq, iw, ik, q, kv, ctx_len, B, Hi, Di, Hq, Dk, Dv, N, k, scale, dt, scores, idx, out, ws,
                          ws_bytes, flags, stream, kernel_events, nullptr, 0);
}

dsa_status dsa_decode_step_paged(const int8_t* iq, const int8_t* iw, const int8_t* ik_pool, const void* q,
                                 const void* kv_pool, const int32_t* page_table, int64_t pool_pages,
                                 const int32_t* ctx_len, int B, int Hi, int Di, int Hq, int Dk, int Dv,
                                 int64_t N, int k, float scale, dsa_dtype dt, int32_t* scores, int32_t* idx,
                                 float* out, void* ws, size_t ws_bytes, unsigned flags, hipStream_t stream,
                                 hipEvent_t* kernel_events) {
  if (page_table == nullptr) return DSA_ERR_INVALID_ARG;
  return decode_step_impl(iq, iw, ik_pool, q, kv_pool, ctx_len, B, Hi, Di, Hq, Dk, Dv, N, k, scale, dt, scores, idx,
                          out, ws, ws_bytes, flags, stream, kernel_events, page_table, pool_pages);
}

dsa_status dsa_decode_step(const int8_t* iq, const int8_t* iw, const int8_t* ik, const void* q,
                           const void* kv, const int32_t* ctx_len, int B, int Hi, int Di, int Hq,
                           int Dk, int Dv, int64_t N, int k, float scale, dsa_dtype dt,
                           int32_t* scores, int32_t* idx, float* out, void* ws, size_t ws_bytes,
                           unsigned flags, hipStream_t stream) {
  return dsa_decode_step_timed(iq, iw, ik, q, kv, ctx_len, B, Hi, Di, Hq, Dk, Dv, N, k, scale, dt,
                               scores, idx, out, ws, ws_bytes, flags, stream, nullptr);
}

dsa_status dsa_decode_step_noalloc(const int8_t* iq, const int8_t* iw, const int8_t* ik, const void* q,
                                   const void* kv, const int32_t* ctx_len, int B, int Hi, int Di, int Hq,
                                   int Dk, int Dv, int64_t N, int k, float scale, dsa_dtype dt,
                                   int32_t* scores, int32_t* idx, float* out, unsigned flags,
                                   hipStream_t stream) {
  const size_t need = dsa_workspace_size(B, N, k, Hq, Dv);
  if (need == 0) return DSA_ERR_INVALID_ARG;
  if (need > kScratchBytes) return DSA_ERR_WORKSPACE;  // beyond the static scratch
  void* ws = device_scratch();
  if (ws == nullptr) return DSA_ERR_HIP;
  return dsa_decode_step(iq, iw, ik, q, kv, ctx_len, B, Hi, Di, Hq, Dk, Dv, N, k, scale, dt, scores, idx, out,
                         ws, kScratchBytes, flags, stream);
}

dsa_status dsa_read_stats(const void* ws, size_t ws_bytes, int B, dsa_row_stats* stats,
                          hipStream_t stream) {
  if (!ws || !stats || B < 1 || B > DSA_MAX_BATCH) return DSA_ERR_INVALID_ARG;
  if (ws_bytes < sizeof(RowStats) * (size_t)B) return DSA_ERR_WORKSPACE;
  static_assert(sizeof(RowStats) == sizeof(dsa_row_stats), "stats layout");
  if (hipMemcpyAsync(stats, ws, sizeof(RowStats) * B, hipMemcpyDeviceToHost, stream) != hipSuccess)
    return DSA_ERR_HIP;
  return hip_status(hipStreamSynchronize(stream));
}

}  // extern "C"

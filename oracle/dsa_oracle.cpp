// Plain CPU oracle for the DSA decode step: indexer scores, exact top-k,
// softmax attention over the selected positions.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
// this file: only the test-suite, the smoke check and the CPU-baseline leg of the
// benchmark use it. It shares no code, header or constant with the HIP library.
//
// What it follows (the pages describe the behaviour, not the arithmetic):
//  * ds4 glm53-m3ultra branch post (2026-09-09 "rising" page), paragraph on very
//    long context: a lightweight indexer scores every cached position, about 2,048
//    positions are selected, attention runs over only those, and the faster
//    selector picks the same positions in the same order with the same outputs.
//  * GLM-5.3-Flash-Alis-MLX-4bit model card, "What changed" list (the FIXED item
//    on left-padded batches): a row's validity comes from that row's own length,
//    so positions past it are never candidates.
//  * Same model card, Speed section (MQA fold): at decode one shared latent row
//    per position serves every head, as key (latent + rope) and as value (latent).
//  * glm53-tensorfold-spark README, introduction and "What's new (2026-09-30)": the
//    KV cache is one pool of fixed-size pages (1,048,576 tokens in 4,096 pages, so
//    256 positions a page) shared by the sequences. A paged step reads a sequence's
//    positions through its page table; it computes what the contiguous step
//    computes on the cache the table describes, so the oracle gathers that cache
//    and runs the contiguous step.
//  * The pages leave the indexer arithmetic, the tie rule and the softmax precision
//    open. This file takes the plainest reading: int8 query heads against one shared
//    int8 key, ReLU, int8 per-head weight, sum over heads, an int32 result; order by
//    score descending with ties to the lower position; softmax in fp64.
//
// Everything here is written for obviousness, not speed: int64 accumulation,
// std::stable_sort over all valid positions, fp64 softmax with std::exp. Built with
// -fopenmp (the all-core CPU baseline), the loops over positions (scores) and over
// heads (attention) are split over threads; each iteration is independent and writes
// only its own outputs, so the results are the same. The sort stays sequential.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

// Threads the loops above use (1 without OpenMP).
int dsa_ref_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// Return codes of the oracle (its own, unrelated to the library's).
enum { REF_OK = 0, REF_BAD_ARG = 1, REF_OVERFLOW = 2 };

// scores[b*N + s] for s < ctx_len[b]; entries at or past ctx_len[b] are not written.
//   acc_h  = sum_d iq[b,h,d] * ik[s,d]          (exact, int64)
//   score  = sum_h iw[b,h] * max(0, acc_h)       (exact, int64, must fit int32)
int dsa_ref_index_scores(const int8_t* iq, const int8_t* iw, const int8_t* ik,
                         const int32_t* ctx_len, int B, int Hi, int Di, int64_t N,
                         int32_t* scores) {
  if (B < 1 || Hi < 1 || Di < 1 || N < 1) return REF_BAD_ARG;
  for (int b = 0; b < B; ++b) {
    if (ctx_len[b] < 0 || ctx_len[b] > N) return REF_BAD_ARG;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t s = 0; s < ctx_len[b]; ++s) {
      int64_t score = 0;
      for (int h = 0; h < Hi; ++h) {
        int64_t acc = 0;
        for (int d = 0; d < Di; ++d)
          acc += (int64_t)iq[((int64_t)b * Hi + h) * Di + d] * (int64_t)ik[s * Di + d];
        int64_t relu = acc > 0 ? acc : 0;
        score += (int64_t)iw[(int64_t)b * Hi + h] * relu;
      }
      if (score > INT32_MAX || score < INT32_MIN)
        overflow = 1;
      else
        scores[(int64_t)b * N + s] = (int32_t)score;
    }
    if (overflow) return REF_OVERFLOW;
  }
  return REF_OK;
}

// idx[b*k + j]: the first min(k, ctx_len[b]) positions of [0, ctx_len[b]) in
// (score descending, position ascending) order, then -1.
int dsa_ref_topk_select(const int32_t* scores, const int32_t* ctx_len, int B, int64_t N,
                        int k, int32_t* idx) {
  if (B < 1 || N < 1 || k < 1) return REF_BAD_ARG;
  for (int b = 0; b < B; ++b) {
    int64_t n = ctx_len[b];
    if (n < 0 || n > N) return REF_BAD_ARG;
    const int32_t* row = scores + (int64_t)b * N;
    std::vector<int64_t> order(n);
    for (int64_t s = 0; s < n; ++s) order[s] = s;  // ascending positions
    // A stable sort on "higher score first" keeps equal scores in ascending position.
    std::stable_sort(order.begin(), order.end(),
                     [row](int64_t x, int64_t y) { return row[x] > row[y]; });
    int64_t m = std::min<int64_t>(k, n);
    for (int64_t j = 0; j < k; ++j)
      idx[(int64_t)b * k + j] = j < m ? (int32_t)order[j] : -1;
  }
  return REF_OK;
}

// One FP8 E4M3 value (the OCP 8-bit "e4m3fn" format: 1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits; no infinities; exponent and mantissa all ones is NaN),
// decoded from its definition:
//   exponent 0:   (-1)^s * m * 2^-9              (subnormal: m/8 * 2^(1-7))
//   otherwise:    (-1)^s * (1 + m/8) * 2^(e-7)
// Every such value is a double exactly. The pages name FP8 KV storage
// (glm53-tensorfold-spark README, introduction: patch list) without fixing the
// format; e4m3fn is the plainest reading for stored activations.
static inline double e4m3_to_double(uint8_t v) {
  const int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? std::ldexp((double)m, -9) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

// The decode of n codes, for the checks that pin it.
void dsa_ref_e4m3_to_f64(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_double(codes[i]);
}

static inline double bf16_to_double(uint16_t b) {
  // bf16: the 16 stored bits are the high half of an fp32.
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Element i of a query (kv = 0) or latent-cache (kv = 1) array of the given dtype:
// 0 = fp32 both, 1 = bf16 both, 2 = bf16 queries with an FP8 E4M3 latent cache.
static inline double load_elem(const void* p, int dtype, int kv, int64_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  if (dtype == 2 && kv) return e4m3_to_double(((const uint8_t*)p)[i]);
  return bf16_to_double(((const uint16_t*)p)[i]);
}

// out[(b*Hq + h)*Dv + v] (fp64) = sum_i p_i * kv[idx_i, v] / sum_i p_i with
//   l_i = scale * sum_{d<Dk} q[b,h,d] * kv[idx_i, d],  p_i = exp(l_i - max_j l_j),
// over the entries of idx[b, 0:k] that are not -1. K is the whole row (Dk values),
// V is its first Dv values. dtype 0 = fp32 inputs, 1 = bf16 inputs, 2 = bf16
// queries with an FP8 E4M3 latent cache (decoded exactly).
// A row with no valid entry gets zeros.
int dsa_ref_sparse_attn(const void* q, const void* kv, const int32_t* idx, int B, int Hq,
                        int Dk, int Dv, int64_t N, int k, double scale, int dtype,
                        double* out) {
  if (B < 1 || Hq < 1 || Dk < 1 || Dv < 1 || Dv > Dk || N < 1 || k < 1) return REF_BAD_ARG;
  if (dtype < 0 || dtype > 2) return REF_BAD_ARG;
  for (int b = 0; b < B; ++b) {
    std::vector<int64_t> rows;
    for (int j = 0; j < k; ++j) {
      int32_t r = idx[(int64_t)b * k + j];
      if (r == -1) continue;
      if (r < 0 || r >= N) return REF_BAD_ARG;
      rows.push_back(r);
    }
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hq; ++h) {
      double* o = out + ((int64_t)b * Hq + h) * Dv;
      for (int v = 0; v < Dv; ++v) o[v] = 0.0;
      if (rows.empty()) continue;
      const int64_t qoff = ((int64_t)b * Hq + h) * Dk;
      std::vector<double> logit(rows.size());
      double mx = -INFINITY;
      for (size_t i = 0; i < rows.size(); ++i) {
        double dot = 0.0;
        for (int d = 0; d < Dk; ++d)
          dot += load_elem(q, dtype, 0, qoff + d) * load_elem(kv, dtype, 1, rows[i] * Dk + d);
        logit[i] = scale * dot;
        mx = std::max(mx, logit[i]);
      }
      double denom = 0.0;
      for (size_t i = 0; i < rows.size(); ++i) {
        double p = std::exp(logit[i] - mx);
        denom += p;
        for (int v = 0; v < Dv; ++v) o[v] += p * load_elem(kv, dtype, 1, rows[i] * Dk + v);
      }
      for (int v = 0; v < Dv; ++v) o[v] /= denom;
    }
  }
  return REF_OK;
}

// The three stages in sequence, as one decode step through one DSA layer.
int dsa_ref_decode_step(const int8_t* iq, const int8_t* iw, const int8_t* ik, const void* q,
                        const void* kv, const int32_t* ctx_len, int B, int Hi, int Di, int Hq,
                        int Dk, int Dv, int64_t N, int k, double scale, int dtype,
                        int32_t* scores, int32_t* idx, double* out) {
  int rc = dsa_ref_index_scores(iq, iw, ik, ctx_len, B, Hi, Di, N, scores);
  if (rc != REF_OK) return rc;
  rc = dsa_ref_topk_select(scores, ctx_len, B, N, k, idx);
  if (rc != REF_OK) return rc;
  return dsa_ref_sparse_attn(q, kv, idx, B, Hq, Dk, Dv, N, k, scale, dtype, out);
}

// The contiguous cache a page table describes: row s of `out` (s < N) is pool row
// page_table[s / page] * page + s % page, row_bytes bytes each. A table entry
// outside [0, pool_pages) is an error.
int dsa_ref_gather_pages(const uint8_t* pool, int64_t row_bytes, const int32_t* page_table,
                         int64_t pool_pages, int page, int64_t N, uint8_t* out) {
  if (row_bytes < 1 || pool_pages < 1 || page < 1 || N < 1) return REF_BAD_ARG;
  for (int64_t s = 0; s < N; ++s) {
    const int64_t p = page_table[s / page];
    if (p < 0 || p >= pool_pages) return REF_BAD_ARG;
    std::memcpy(out + s * row_bytes, pool + (p * page + s % page) * row_bytes, (size_t)row_bytes);
  }
  return REF_OK;
}

}  // extern "C"

// TEST INFRASTRUCTURE ONLY - the CPU oracle for tile-group precision-routed attention.
//
// Only the test suite, the package smoke check and the CPU-baseline leg of the benchmark may
// load this library. The product (the HIP library and its Python binding) never calls it and
// shares no code, header or table with it.
//
// What it computes follows "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
// Acceleration" (arXiv 2608.17336):
//   * attention S = Q K^T / sqrt(d), P = softmax(S), O = P V             (Section 3.1)
//   * quantization (A_hat, delta_A) = psi(A), C ~= delta_A delta_B (A_hat B_hat)   (Section 3.2)
//   * routing map R[h_k, m, g_j]: 1 -> INT8 score path, 0 -> FP16 score path   (Section 4.2)
//   * grouping: one bit covers g adjacent key tiles, g_j = floor(n / g)      (Section 4.2, grouping eq.)
//   * packed word b = sum_j R_j 2^j, lookup R = (b >> g_j) & 1               (Section 4.2, pack/decode eqs.)
//   * routed score: INT8 tiles use Rescale(Q8 K8^T)/sqrt(d) with integer accumulation,
//     FP16 tiles use Q K^T / sqrt(d)                                         (Section 4.3, routed-score eq.)
//   * GQA map h_k = floor(h_q / (H_q / H_k)); cu_seqlens varlen              (Section 4.1)
//
// The softmax is evaluated in plain two-pass form (row max, then exponentials and their sum),
// which is the definition the online recurrence of Section 3.1 reproduces exactly in exact
// arithmetic. All arithmetic after the integer dot products is fp64; outputs are written as fp32.
//
// Readings where the pages are silent (each listed with its reason in the design notes):
//   * quantization is symmetric, per token and per head (one scale per row of head_dim):
//     a = max|x|, inv = 127/a and delta = a/127 (both correctly rounded fp32 divisions),
//     q = clamp(rint(x * inv), -127, 127) with an fp32 product and round-half-to-even;
//     a == 0 gives delta = 0 and q = 0. This integer decision is made in fp32, the kernel's
//     precision, on both sides.
//   * causal alignment is bottom-right: key j is legal for query i iff j <= i + (L_k - L_q).
//     A query with no legal key gets O = 0 and LSE = -inf.
//   * route tiles never straddle sequences: route row r = cu_mtiles[b] + floor(i / BM_r).
//   * a route map with more than 64 groups per row is spread over ceil(T_mask/64) words;
//     group g_j lives in word g_j >> 6 at bit g_j & 63 (the single-word case is the pages').
//   * INT8 K/V cache: the cache stands for K = delta_k * k8 and V = delta_v * v8 exactly; the
//     FP16 path uses that dequantized K, P.V uses that dequantized V.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

namespace {

// IEEE 754 binary16 -> double, by the bit-level definition of the format.
double decode_binary16(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 10) & 0x1f;
  const int mant = h & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = std::ldexp(static_cast<double>(mant), -24);  // subnormal: mant * 2^-14 * 2^-10
  } else if (expo == 31) {
    mag = mant ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
  } else {
    mag = std::ldexp(static_cast<double>(1024 + mant), expo - 25);  // (1 + mant/1024) * 2^(expo-15)
  }
  return sign ? -mag : mag;
}

const double* binary16_table() {
  static const std::vector<double> table = [] {
    std::vector<double> t(65536);
    for (int i = 0; i < 65536; ++i) t[i] = decode_binary16(static_cast<uint16_t>(i));
    return t;
  }();
  return table.data();
}

}  // namespace

extern "C" {

int oracle_version(void) { return 1; }

int oracle_max_threads(void) { return omp_get_max_threads(); }

double oracle_decode_fp16(uint16_t h) { return decode_binary16(h); }

// Symmetric INT8 quantization of `rows` rows of `d` fp16 values (row r starts at x + r*row_stride),
// one scale per row. q is [rows, d] contiguous, scale is [rows].
int oracle_quantize_rows(const uint16_t* x, int64_t rows, int32_t d, int64_t row_stride,
                         int8_t* q, float* scale) {
  if (!x || !q || !scale || rows < 0 || d <= 0 || row_stride < d) return -1;
  const double* f16 = binary16_table();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* row = x + r * row_stride;
    float a = 0.0f;
    for (int c = 0; c < d; ++c) {
      const float v = static_cast<float>(std::fabs(f16[row[c]]));  // fp16 -> fp32 is exact
      if (v > a) a = v;
    }
    int8_t* qr = q + r * static_cast<int64_t>(d);
    if (a == 0.0f) {
      scale[r] = 0.0f;
      for (int c = 0; c < d; ++c) qr[c] = 0;
      continue;
    }
    const float inv = 127.0f / a;
    scale[r] = a / 127.0f;
    for (int c = 0; c < d; ++c) {
      const float prod = static_cast<float>(f16[row[c]]) * inv;
      float k = std::rint(prod);  // round half to even (default rounding mode)
      if (k > 127.0f) k = 127.0f;
      if (k < -127.0f) k = -127.0f;
      qr[c] = static_cast<int8_t>(k);
    }
  }
  return 0;
}

// Block-wise symmetric INT8 quantization: the TileMix paper quantizes Q and K "blockwise" with one
// scale per block (Section 4.3, INT8 path; quantizer psi of Section 3.2). A block is `block_rows`
// consecutive tokens of one sequence (the last block of a sequence may be shorter; blocks never
// straddle sequences) and one head: a = max|x| over its rows and all d channels, then the same
// fp32 steps as the per-row quantizer with that a. x is fp16 bits [T, heads, d] contiguous, q is
// [T, heads, d], scale is [T, heads] and every row holds its block's scale.
int oracle_quantize_blocks(const uint16_t* x, int64_t T, int32_t heads, int32_t d,
                           const int32_t* cu, int32_t batch, int32_t block_rows, int8_t* q,
                           float* scale) {
  if (!x || !q || !scale || !cu || T < 0 || heads < 1 || d < 1 || batch < 1 || block_rows < 1) return -1;
  if (cu[0] != 0 || cu[batch] != T) return -1;
  for (int b = 0; b < batch; ++b)
    if (cu[b + 1] < cu[b]) return -1;
  const double* f16 = binary16_table();
  for (int b = 0; b < batch; ++b) {
    for (int64_t t0 = cu[b]; t0 < cu[b + 1]; t0 += block_rows) {
      const int64_t t1 = std::min<int64_t>(cu[b + 1], t0 + block_rows);
      for (int h = 0; h < heads; ++h) {
        float a = 0.0f;
        for (int64_t t = t0; t < t1; ++t)
          for (int c = 0; c < d; ++c) {
            const float v = static_cast<float>(std::fabs(f16[x[(t * heads + h) * d + c]]));
            if (v > a) a = v;
          }
        const float inv = a > 0.0f ? 127.0f / a : 0.0f;
        const float delta = a > 0.0f ? a / 127.0f : 0.0f;
        for (int64_t t = t0; t < t1; ++t) {
          scale[t * heads + h] = delta;
          for (int c = 0; c < d; ++c) {
            const int64_t i = (t * heads + h) * d + c;
            float k = std::rint(static_cast<float>(f16[x[i]]) * inv);
            if (k > 127.0f) k = 127.0f;
            if (k < -127.0f) k = -127.0f;
            q[i] = static_cast<int8_t>(k);
          }
        }
      }
    }
  }
  return 0;
}

// Packs R [rows, t_mask] of 0/1 bytes into words [rows, wpr]: bit g_j of a row is word g_j>>6,
// bit g_j&63. Unused high bits are zero. Returns -1 on a value other than 0/1 or a short row.
int oracle_pack_route(const uint8_t* R, int64_t rows, int32_t t_mask, uint64_t* words,
                      int32_t wpr) {
  if (!R || !words || rows < 0 || t_mask < 0 || wpr < 1 || t_mask > 64 * wpr) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int w = 0; w < wpr; ++w) words[r * wpr + w] = 0;
    for (int g = 0; g < t_mask; ++g) {
      const uint8_t bit = R[r * t_mask + g];
      if (bit > 1) return -1;
      if (bit) words[r * wpr + (g >> 6)] |= (uint64_t{1} << (g & 63));
    }
  }
  return 0;
}

}  // extern "C"

typedef struct {
  int32_t batch, hq, hk, d;
  int64_t total_q, total_k;
  const int32_t* cu_q;       // [batch+1] token prefix sums of queries
  const int32_t* cu_k;       // [batch+1] token prefix sums of keys
  const int32_t* cu_mtiles;  // [batch+1] prefix sums of ceil(L_q,b / BM_r)
  int32_t total_mtiles;
  const uint16_t* q;         // fp16 bits [total_q, hq, d]
  const uint16_t* k;         // fp16 bits [total_k, hk, d]; unused when kv_int8
  const uint16_t* v;         // fp16 bits [total_k, hk, d]; unused when kv_int8
  const int8_t* q8;          // [total_q, hq, d]
  const float* q_scale;      // [total_q, hq]
  const int8_t* k8;          // [total_k, hk, d]
  const float* k_scale;      // [total_k, hk]
  const int8_t* v8;          // [total_k, hk, d], kv_int8 only
  const float* v_scale;      // [total_k, hk],    kv_int8 only
  int32_t kv_int8;
  const uint64_t* words;     // [hk, total_mtiles, wpr]
  int32_t wpr, bm_r, bn_r, group;
  int32_t causal;
  double softmax_scale;      // <= 0 means 1/sqrt(d)
} oracle_problem;

namespace {

struct RowPlace {
  int b;
  int64_t i;  // local query index within sequence b
};

bool locate(const oracle_problem& p, int64_t t, RowPlace* out) {
  for (int b = 0; b < p.batch; ++b) {
    if (t >= p.cu_q[b] && t < p.cu_q[b + 1]) {
      out->b = b;
      out->i = t - p.cu_q[b];
      return true;
    }
  }
  return false;
}

// R_{h_k, m, g_j} = (b_{h_k, m} >> g_j) & 1, with the row's words stored consecutively.
int route_bit(const oracle_problem& p, int hk, int64_t route_row, int64_t gj) {
  const uint64_t* row = p.words + (static_cast<int64_t>(hk) * p.total_mtiles + route_row) * p.wpr;
  return static_cast<int>((row[gj >> 6] >> (gj & 63)) & 1u);
}

bool key_legal(const oracle_problem& p, int64_t i, int64_t j, int64_t Lq, int64_t Lk) {
  if (j < 0 || j >= Lk) return false;
  if (p.causal && j > i + (Lk - Lq)) return false;
  return true;
}

int check_problem(const oracle_problem& p) {
  if (p.batch < 1 || p.hq < 1 || p.hk < 1 || p.d < 1 || p.hq % p.hk) return -1;
  if (!p.cu_q || !p.cu_k || !p.cu_mtiles || !p.words || !p.q8 || !p.q_scale || !p.k8 || !p.k_scale)
    return -1;
  if (p.kv_int8) {
    if (!p.v8 || !p.v_scale) return -1;
  } else {
    if (!p.q || !p.k || !p.v) return -1;
  }
  if (p.bm_r < 1 || p.bn_r < 1 || p.group < 1 || p.wpr < 1) return -1;
  for (int b = 0; b < p.batch; ++b) {
    const int64_t Lq = p.cu_q[b + 1] - p.cu_q[b];
    const int64_t Lk = p.cu_k[b + 1] - p.cu_k[b];
    if (Lq < 0 || Lk < 0) return -1;
    if (p.cu_mtiles[b + 1] - p.cu_mtiles[b] != (Lq + p.bm_r - 1) / p.bm_r) return -1;
    const int64_t ngroups = (Lk + static_cast<int64_t>(p.bn_r) * p.group - 1) /
                            (static_cast<int64_t>(p.bn_r) * p.group);
    if (ngroups > 64LL * p.wpr) return -1;
  }
  if (p.cu_q[p.batch] != p.total_q || p.cu_k[p.batch] != p.total_k) return -1;
  if (p.cu_mtiles[p.batch] != p.total_mtiles) return -1;
  return 0;
}

}  // namespace

extern "C" {

// Routed attention for the selected query tokens (all heads).
//   rows: global query token indices, or NULL for all total_q tokens in order.
//   out:  fp32 [n_rows, hq, d];  lse: fp32 [hq, n_rows] (natural log), may be NULL.
//   int8_pairs / legal_pairs (optional): count of legal (query, key, head) pairs routed to INT8
//   and in total, over the selected rows.
int oracle_prefill(const oracle_problem* prob, const int64_t* rows, int64_t n_rows, float* out,
                   float* lse, int64_t* int8_pairs, int64_t* legal_pairs) {
  if (!prob || !out) return -1;
  const oracle_problem& p = *prob;
  if (check_problem(p)) return -1;
  const int64_t n = rows ? n_rows : p.total_q;
  const double scale = p.softmax_scale > 0 ? p.softmax_scale : 1.0 / std::sqrt(static_cast<double>(p.d));
  const double* f16 = binary16_table();
  const int group_q = p.hq / p.hk;
  const int d = p.d;
  int64_t max_lk = 0;
  for (int b = 0; b < p.batch; ++b) max_lk = std::max<int64_t>(max_lk, p.cu_k[b + 1] - p.cu_k[b]);
  for (int64_t s = 0; s < n; ++s) {
    RowPlace rp;
    if (!locate(p, rows ? rows[s] : s, &rp)) return -1;
  }
  int64_t n8 = 0, nall = 0;

#pragma omp parallel reduction(+ : n8, nall)
  {
    std::vector<double> sc(static_cast<size_t>(max_lk) + 1);
    std::vector<double> acc(d);
#pragma omp for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < n; ++s) {
      for (int h = 0; h < p.hq; ++h) {
        const int64_t t = rows ? rows[s] : s;
        RowPlace rp{0, 0};
        locate(p, t, &rp);  // every selected row was located above
        const int b = rp.b;
        const int64_t i = rp.i;
        const int64_t Lq = p.cu_q[b + 1] - p.cu_q[b];
        const int64_t Lk = p.cu_k[b + 1] - p.cu_k[b];
        const int hk = h / group_q;
        const int64_t route_row = p.cu_mtiles[b] + i / p.bm_r;
        float* o = out + (s * p.hq + h) * d;

        // Pass 1: every legal score, routed per key-tile group, and the row maximum.
        double row_max = -std::numeric_limits<double>::infinity();
        int64_t n_legal = 0;
        for (int64_t j = 0; j < Lk; ++j) {
          if (!key_legal(p, i, j, Lq, Lk)) continue;
          const int64_t tk = p.cu_k[b] + j;
          const int64_t tile_n = j / p.bn_r;
          const int64_t gj = tile_n / p.group;
          double sij;
          if (route_bit(p, hk, route_row, gj)) {
            const int8_t* qa = p.q8 + (t * p.hq + h) * d;
            const int8_t* ka = p.k8 + (tk * p.hk + hk) * d;
            int64_t dot = 0;
            for (int c = 0; c < d; ++c) dot += static_cast<int64_t>(qa[c]) * ka[c];
            sij = static_cast<double>(dot) * static_cast<double>(p.q_scale[t * p.hq + h]) *
                  static_cast<double>(p.k_scale[tk * p.hk + hk]) * scale;
            ++n8;
          } else {
            const uint16_t* qa = p.q + (t * p.hq + h) * d;
            double dot = 0.0;
            if (p.kv_int8) {
              const int8_t* ka = p.k8 + (tk * p.hk + hk) * d;
              const double ks = p.k_scale[tk * p.hk + hk];
              for (int c = 0; c < d; ++c) dot += f16[qa[c]] * (static_cast<double>(ka[c]) * ks);
            } else {
              const uint16_t* ka = p.k + (tk * p.hk + hk) * d;
              for (int c = 0; c < d; ++c) dot += f16[qa[c]] * f16[ka[c]];
            }
            sij = dot * scale;
          }
          sc[j] = sij;
          if (sij > row_max) row_max = sij;
          ++n_legal;
        }
        nall += n_legal;
        if (n_legal == 0) {
          for (int c = 0; c < d; ++c) o[c] = 0.0f;
          if (lse) lse[h * n + s] = -std::numeric_limits<float>::infinity();
          continue;
        }

        // Pass 2: exponentials, their sum and the weighted sum of values.
        double l = 0.0;
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t j = 0; j < Lk; ++j) {
          if (!key_legal(p, i, j, Lq, Lk)) continue;
          const int64_t tk = p.cu_k[b] + j;
          const double pij = std::exp(sc[j] - row_max);
          l += pij;
          if (p.kv_int8) {
            const int8_t* va = p.v8 + (tk * p.hk + hk) * d;
            const double vs = p.v_scale[tk * p.hk + hk];
            for (int c = 0; c < d; ++c) acc[c] += pij * (static_cast<double>(va[c]) * vs);
          } else {
            const uint16_t* va = p.v + (tk * p.hk + hk) * d;
            for (int c = 0; c < d; ++c) acc[c] += pij * f16[va[c]];
          }
        }
        for (int c = 0; c < d; ++c) o[c] = static_cast<float>(acc[c] / l);
        if (lse) lse[h * n + s] = static_cast<float>(row_max + std::log(l));
      }
    }
  }
  if (int8_pairs) *int8_pairs = n8;
  if (legal_pairs) *legal_pairs = nall;
  return 0;
}

// Integer accumulators Q8 K8^T of the INT8-routed route tiles, for one query head and the route
// rows [m0, m0 + m_count). Layout: dump[(r - m0), n, ii, jj] with shape
// [m_count, ntiles_max, bm_r, bn_r]; every in-sequence element of each INT8-routed route tile
// that holds at least one legal pair is written (masked positions included, the product is
// defined there); everything else is left untouched.
int oracle_int32_tiles(const oracle_problem* prob, int32_t head, int32_t m0, int32_t m_count,
                       int32_t ntiles_max, int32_t* dump) {
  if (!prob || !dump) return -1;
  const oracle_problem& p = *prob;
  if (check_problem(p) || head < 0 || head >= p.hq || m0 < 0 || m_count < 0 ||
      m0 + m_count > p.total_mtiles || ntiles_max < 1)
    return -1;
  const int hk = head / (p.hq / p.hk);
  const int d = p.d;
  for (int r = m0; r < m0 + m_count; ++r) {
    int b = 0;
    while (b < p.batch && !(r >= p.cu_mtiles[b] && r < p.cu_mtiles[b + 1])) ++b;
    if (b == p.batch) return -1;
    const int64_t Lq = p.cu_q[b + 1] - p.cu_q[b];
    const int64_t Lk = p.cu_k[b + 1] - p.cu_k[b];
    const int64_t m = r - p.cu_mtiles[b];
    const int64_t i_lo = m * p.bm_r, i_hi = std::min<int64_t>(i_lo + p.bm_r, Lq);
    const int64_t ntiles = (Lk + p.bn_r - 1) / p.bn_r;
    if (ntiles > ntiles_max) return -1;
    for (int64_t tn = 0; tn < ntiles; ++tn) {
      const int64_t j_lo = tn * p.bn_r, j_hi = std::min<int64_t>(j_lo + p.bn_r, Lk);
      if (!route_bit(p, hk, r, tn / p.group)) continue;
      bool any_legal = false;
      for (int64_t i = i_lo; i < i_hi && !any_legal; ++i)
        for (int64_t j = j_lo; j < j_hi && !any_legal; ++j) any_legal = key_legal(p, i, j, Lq, Lk);
      if (!any_legal) continue;
#pragma omp parallel for schedule(static)
      for (int64_t i = i_lo; i < i_hi; ++i) {
        const int64_t t = p.cu_q[b] + i;
        for (int64_t j = j_lo; j < j_hi; ++j) {
          const int64_t tk = p.cu_k[b] + j;
          const int8_t* qa = p.q8 + (t * p.hq + head) * d;
          const int8_t* ka = p.k8 + (tk * p.hk + hk) * d;
          int64_t dot = 0;
          for (int c = 0; c < d; ++c) dot += static_cast<int64_t>(qa[c]) * ka[c];
          const int64_t idx =
              ((static_cast<int64_t>(r - m0) * ntiles_max + tn) * p.bm_r + (i - i_lo)) * p.bn_r +
              (j - j_lo);
          dump[idx] = static_cast<int32_t>(dot);
        }
      }
    }
  }
  return 0;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Routing policies: the step that produces R before packing. The pages let any static or adaptive
// policy supply R (TileMix paper, Section 4.2 "Policy definition", and the Limitations section);
// their own templates are defined in an appendix the pages do not hold. These are the two policies
// the library computes on the device (readings listed with the others in the design notes):
//   * top-k by max|K|: per sequence and KV head, the ceil(T * per_mille / 1000) key-tile groups
//     with the largest max|K| over their keys and channels take the FP16 path (R = 0) in every
//     query-tile row of the sequence; ties go to the lower group index; the other groups below the
//     sequence's T = ceil(L_k / (BN_r * g)) are INT8 (R = 1). With an INT8 cache, |K| of a key is
//     the fp32 product k_scale * |k8|.
//   * coverage-budget Bernoulli: every (KV head, route row, group) below T is FP16 iff the first
//     output word of Philox4x32-10 at counter (g_j, route row, h_k, 0) and key (seed low 32 bits,
//     seed high 32 bits) is below thr = floor(per_mille * 2^32 / 1000).
// R is [hk, total_mtiles, t_mask]; groups at or past a sequence's own T are 0.

namespace {

// One Philox4x32 round and the Weyl key schedule, from the generator's definition in Salmon,
// Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011).
void philox_round(uint32_t x[4], const uint32_t k[2]) {
  const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x[0];
  const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * x[2];
  const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
  const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
  const uint32_t y0 = hi1 ^ x[1] ^ k[0];
  const uint32_t y2 = hi0 ^ x[3] ^ k[1];
  x[0] = y0;
  x[1] = lo1;
  x[2] = y2;
  x[3] = lo0;
}

void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(x, k);
  }
  for (int i = 0; i < 4; ++i) out[i] = x[i];
}

// Shared argument checks of the two policies; on success *span is BN_r * g.
int check_route_args(const int32_t* cu_k, const int32_t* cu_mtiles, int32_t batch, int32_t hk,
                     int32_t bn_r, int32_t group, int32_t per_mille, int32_t t_mask, uint8_t* R,
                     int64_t* span) {
  if (!cu_k || !cu_mtiles || !R || batch < 1 || hk < 1 || bn_r < 1 || group < 1 || t_mask < 0 ||
      per_mille < 0 || per_mille > 1000)
    return -1;
  *span = static_cast<int64_t>(bn_r) * group;
  for (int b = 0; b < batch; ++b) {
    const int64_t Lk = cu_k[b + 1] - cu_k[b];
    if (Lk < 0 || cu_mtiles[b + 1] < cu_mtiles[b]) return -1;
    if ((Lk + *span - 1) / *span > t_mask) return -1;
  }
  return 0;
}

}  // namespace

extern "C" {

void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
  philox4x32_10(ctr, key, out);
}

// k: fp16 bits [total_k, hk, d] contiguous, or NULL to read the INT8 cache k8 [total_k, hk, d]
// with k_scale [total_k, hk].
int oracle_route_topk_maxabs(const int32_t* cu_k, const int32_t* cu_mtiles, int32_t batch,
                             int32_t hk, int32_t d, const uint16_t* k, const int8_t* k8,
                             const float* k_scale, int32_t bn_r, int32_t group, int32_t per_mille,
                             int32_t t_mask, uint8_t* R) {
  int64_t span = 0;
  if (check_route_args(cu_k, cu_mtiles, batch, hk, bn_r, group, per_mille, t_mask, R, &span)) return -1;
  if (d < 1 || (!k && (!k8 || !k_scale))) return -1;
  const double* f16 = binary16_table();
  const int64_t total_mtiles = cu_mtiles[batch];
  std::memset(R, 0, static_cast<size_t>(hk) * total_mtiles * t_mask);
  for (int b = 0; b < batch; ++b) {
    const int64_t k0 = cu_k[b], Lk = cu_k[b + 1] - cu_k[b];
    const int64_t T = (Lk + span - 1) / span;
    const int64_t nsel = (T * per_mille + 999) / 1000;
    for (int h = 0; h < hk; ++h) {
      std::vector<double> score(T, 0.0);
      for (int64_t g = 0; g < T; ++g) {
        for (int64_t j = g * span; j < std::min(Lk, (g + 1) * span); ++j) {
          const int64_t row = ((k0 + j) * hk + h) * static_cast<int64_t>(d);
          for (int c = 0; c < d; ++c) {
            double a;
            if (k) {
              a = std::fabs(f16[k[row + c]]);
            } else {
              const float prod = k_scale[(k0 + j) * hk + h] * static_cast<float>(std::abs(static_cast<int>(k8[row + c])));
              a = static_cast<double>(prod);
            }
            score[g] = std::max(score[g], a);
          }
        }
      }
      // descending max|K|; the stable sort keeps equal maxima in ascending group order
      std::vector<int64_t> order(T);
      for (int64_t g = 0; g < T; ++g) order[g] = g;
      std::stable_sort(order.begin(), order.end(),
                       [&](int64_t x, int64_t y) { return score[x] > score[y]; });
      std::vector<uint8_t> bit(T, 1);
      for (int64_t i = 0; i < nsel; ++i) bit[order[i]] = 0;
      for (int64_t r = cu_mtiles[b]; r < cu_mtiles[b + 1]; ++r)
        for (int64_t g = 0; g < T; ++g) R[(h * total_mtiles + r) * t_mask + g] = bit[g];
    }
  }
  return 0;
}

int oracle_route_bernoulli(const int32_t* cu_k, const int32_t* cu_mtiles, int32_t batch,
                           int32_t hk, int32_t bn_r, int32_t group, int32_t per_mille,
                           uint64_t seed, int32_t t_mask, uint8_t* R) {
  int64_t span = 0;
  if (check_route_args(cu_k, cu_mtiles, batch, hk, bn_r, group, per_mille, t_mask, R, &span)) return -1;
  const int64_t total_mtiles = cu_mtiles[batch];
  const uint64_t thr = (static_cast<uint64_t>(per_mille) << 32) / 1000;
  const uint32_t key[2] = {static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32)};
  std::memset(R, 0, static_cast<size_t>(hk) * total_mtiles * t_mask);
  for (int b = 0; b < batch; ++b) {
    const int64_t T = (cu_k[b + 1] - cu_k[b] + span - 1) / span;
    for (int h = 0; h < hk; ++h)
      for (int64_t r = cu_mtiles[b]; r < cu_mtiles[b + 1]; ++r)
        for (int64_t g = 0; g < T; ++g) {
          const uint32_t ctr[4] = {static_cast<uint32_t>(g), static_cast<uint32_t>(r),
                                   static_cast<uint32_t>(h), 0u};
          uint32_t x[4];
          philox4x32_10(ctr, key, x);
          R[(h * total_mtiles + r) * t_mask + g] = x[0] < thr ? 0 : 1;
        }
  }
  return 0;
}

}  // extern "C"

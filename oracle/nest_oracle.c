/*
 * nest_oracle.c -- plain CPU oracle of the nested-weight speculative round.
 *
 * TEST INFRASTRUCTURE ONLY. This code is the checker, not the product.
 * Only the tests, the package's smoke check and the CPU-baseline leg of the
 * benchmark may load or call it. It shares no code, header or table with
 * the HIP library, and it includes nothing from it.
 *
 * It is written to be read against the pages, not to be fast. It uses
 * loops in the order the definitions give. Integer sums are exact in
 * int64. The quantizer's fp32 decisions are taken in fp32, because the
 * format fixes fp32 weights and scales. Attention is computed in fp64.
 * OpenMP pragmas only spread independent output rows over threads and
 * never change an operation's order.
 *
 * Citations name the page and its figure, table, section or equation:
 *   [BitNest]  "BitNest: Bit-Nested Speculative Decoding for Memory-
 *              Efficient LLM Inference Acceleration" (figure captions and
 *              tables; the method text is not on the page).
 *   [Blog]     "How Speculative Decoding Speeds Up Inference".
 *   [SpecKV]   "SpecKV: Adaptive Speculative Decoding with Compression-
 *              Aware Gamma Selection", section "The Core Idea".
 *
 * Readings of points the pages leave open (each listed in the design
 * notes):
 *   group = 128 consecutive reduction-dimension weights of one output row;
 *   base scale s = max|w|/7 with codes in [-7, 7]; refinement scale s/16
 *   with codes in [-8, 7] (a residual of +8 clamps to 7); rint ties to
 *   even; the residual takes one fma rounding; even element in the low
 *   nibble; activations per row at max|x|/127 in [-127, 127]; the fp32 fold
 *   runs over groups in ascending order; the argmax takes the lowest index
 *   of the maxima; the V cache is stored dim-major inside each block.
 *
 * KV append (the write path after verification) is a reading of its own:
 * new tokens' fp32 values are kept, and each block they touch is quantized
 * again over its valid tokens with the rest taken as 0.
 *
 * Speculative sampling is read as the published method the [Blog] page
 * names: keep d with probability min(1, p(d)/q(d)), else draw from
 * max(0, p - q) normalized; the bonus from the last position; scores are
 * softmax(logits / T); draws by inverse CDF with uniforms passed in.
 *
 * Parity status: every exported function is pinned by the CPU tests
 * against page values, closed forms, library routines or brute force.
 * The worked round of [Blog] Table 1 and Eq. (1) pin the accept rule.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* threads                                                            */
/* ------------------------------------------------------------------ */

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* nested quantization of one group  [BitNest Fig. 2]                  */
/* ------------------------------------------------------------------ */

static int clamp_int(int v, int lo, int hi) {
  if (v < lo) return lo;
  if (v > hi) return hi;
  return v;
}

/* [BitNest Fig. 2]: first a b-bit base code for each weight, then an
 * r-bit code for the error the base leaves. Here b = r = 4. The base scale
 * is s = max|w|/7 (symmetric, codes -7..7). The refinement step is s/16,
 * so 16*q_b + q_r is an 8-bit code at scale s/16, which is the "full 8-bit
 * representation" of [BitNest Fig. 3]. */
void oracle_quantize_group(const float* w, int64_t n, int8_t* qb, int8_t* qr,
                           float* s_out) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; i++) {
    float a = fabsf(w[i]);
    if (a > m) m = a;
  }
  float s = m / 7.0f;
  *s_out = s;
  if (s == 0.0f) {
    for (int64_t i = 0; i < n; i++) {
      qb[i] = 0;
      qr[i] = 0;
    }
    return;
  }
  float s16 = s * 0.0625f;
  for (int64_t i = 0; i < n; i++) {
    float qbase = rintf(w[i] / s);
    int b = clamp_int((int)qbase, -7, 7);
    float err = fmaf(-s, (float)b, w[i]);
    int r = 0;
    if (s16 != 0.0f) {
      float qref = rintf(err / s16);
      /* clamp in float first so a huge quotient cannot overflow the int */
      if (qref < -8.0f) qref = -8.0f;
      if (qref > 7.0f) qref = 7.0f;
      r = (int)qref;
    }
    qb[i] = (int8_t)b;
    qr[i] = (int8_t)r;
  }
}

/* ------------------------------------------------------------------ */
/* planes  [BitNest Fig. 3]: two independent 4-bit streams, N/2 bytes  */
/* ------------------------------------------------------------------ */

/* Element 2j goes to the low nibble of byte j, element 2j+1 to the high
 * nibble, as 4-bit two's complement. */
void oracle_pack_nibbles(const int8_t* codes, int64_t n, uint8_t* plane) {
  for (int64_t j = 0; j < n / 2; j++) {
    uint8_t lo = (uint8_t)(codes[2 * j] & 0x0F);
    uint8_t hi = (uint8_t)(codes[2 * j + 1] & 0x0F);
    plane[j] = (uint8_t)(lo | (hi << 4));
  }
}

static int nibble_at(const uint8_t* plane, int64_t e) {
  int v = (plane[e / 2] >> (4 * (e % 2))) & 0x0F;
  return v >= 8 ? v - 16 : v;
}

void oracle_unpack_nibbles(const uint8_t* plane, int64_t n, int8_t* codes) {
  for (int64_t e = 0; e < n; e++) codes[e] = (int8_t)nibble_at(plane, e);
}

/* nest_pack: every group of every row through oracle_quantize_group, then
 * both code streams into their own plane. Returns 0, or -1 on bad sizes. */
int oracle_nest_pack(const float* w, int64_t rows, int64_t cols, int64_t group,
                     uint8_t* base, uint8_t* refine, float* scales) {
  if (rows < 1 || cols < 2 || group < 2 || group % 2 || cols % group) return -1;
  int64_t G = cols / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    int8_t* qb = (int8_t*)malloc((size_t)group);
    int8_t* qr = (int8_t*)malloc((size_t)group);
    for (int64_t g = 0; g < G; g++) {
      const float* wg = w + r * cols + g * group;
      oracle_quantize_group(wg, group, qb, qr, &scales[r * G + g]);
      oracle_pack_nibbles(qb, group, base + (r * cols + g * group) / 2);
      oracle_pack_nibbles(qr, group, refine + (r * cols + g * group) / 2);
    }
    free(qb);
    free(qr);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* activations: the "A8" of W4A8 / W8A8  [BitNest Table 1]             */
/* ------------------------------------------------------------------ */

void oracle_act_quant(const float* x, int64_t M, int64_t K, int8_t* qa,
                      float* sa) {
  for (int64_t m = 0; m < M; m++) {
    float mx = 0.0f;
    for (int64_t k = 0; k < K; k++) {
      float a = fabsf(x[m * K + k]);
      if (a > mx) mx = a;
    }
    float s = mx / 127.0f;
    sa[m] = s;
    for (int64_t k = 0; k < K; k++) {
      if (s == 0.0f) {
        qa[m * K + k] = 0;
        continue;
      }
      float q = rintf(x[m * K + k] / s);
      if (q < -127.0f) q = -127.0f;
      if (q > 127.0f) q = 127.0f;
      qa[m * K + k] = (int8_t)q;
    }
  }
}

/* ------------------------------------------------------------------ */
/* draft and verify products  [BitNest Fig. 3, Table 1]                */
/* ------------------------------------------------------------------ */

/* Draft: W4A8 over the base plane only. Per group an exact integer sum of
 * qa * q_b, folded in ascending group order with one fma per group at
 * scale s, then scaled by the activation scale. acc (nullable) receives
 * the exact group sums [M][N][G]. */
void oracle_draft_gemv(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                       const uint8_t* base, const float* scales, int64_t N,
                       int64_t group, float* y, int32_t* acc) {
  int64_t G = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    const uint8_t* brow = base + n * (K / 2);
    for (int64_t m = 0; m < M; m++) {
      float run = 0.0f;
      for (int64_t g = 0; g < G; g++) {
        int64_t sum = 0;
        for (int64_t k = g * group; k < (g + 1) * group; k++)
          sum += (int64_t)qa[m * K + k] * (int64_t)nibble_at(brow, k);
        if (acc) acc[(m * N + n) * G + g] = (int32_t)sum;
        run = fmaf(scales[n * G + g], (float)sum, run);
      }
      y[m * N + n] = run * sa[m];
    }
  }
}

/* Verify: W8A8 over both planes. The 8-bit code is 16*q_b + q_r at scale
 * s/16 ([BitNest Fig. 3], "both planes ... the full 8-bit
 * representation"). The fold is the same, with step s*2^-4. */
void oracle_verify_gemm(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                        const uint8_t* base, const uint8_t* refine,
                        const float* scales, int64_t N, int64_t group, float* y,
                        int32_t* acc) {
  int64_t G = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++) {
    const uint8_t* brow = base + n * (K / 2);
    const uint8_t* rrow = refine + n * (K / 2);
    for (int64_t m = 0; m < M; m++) {
      float run = 0.0f;
      for (int64_t g = 0; g < G; g++) {
        int64_t sum = 0;
        for (int64_t k = g * group; k < (g + 1) * group; k++) {
          int64_t code = 16 * (int64_t)nibble_at(brow, k) + nibble_at(rrow, k);
          sum += (int64_t)qa[m * K + k] * code;
        }
        if (acc) acc[(m * N + n) * G + g] = (int32_t)sum;
        run = fmaf(scales[n * G + g] * 0.0625f, (float)sum, run);
      }
      y[m * N + n] = run * sa[m];
    }
  }
}

/* ------------------------------------------------------------------ */
/* greedy choice and the accept rule  [Blog, round steps and Table 1]  */
/* ------------------------------------------------------------------ */

/* Greedy choice: the largest value, and the lowest index among equals.
 * (-0 and +0 compare equal.) */
int64_t oracle_argmax(const float* y, int64_t n) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; i++)
    if (y[i] > y[best]) best = i;
  return best;
}

/* One round [Blog, "Drafting and checking tokens"]. The drafts are walked
 * in order while each equals the target's choice for its slot; the first
 * one that differs gives way to the target's choice, and nothing after it
 * survives. When none differs, one more token, the target's choice after
 * the last draft, follows, so a round emits 1 to k+1 tokens ([Blog]
 * ibid.; [SpecKV] tokens = k+1).
 * draft[i-1] is d_i and target[i] is t_i, the target's choice after slot
 * i. d_i is checked against t_{i-1}. Writes t_0..t_a to emitted, -1
 * after them, and returns a+1. */
int oracle_accept(const int32_t* draft, const int32_t* target, int64_t k,
                  int32_t* emitted) {
  int64_t a = 0;
  while (a < k && draft[a] == target[a]) a++;
  for (int64_t j = 0; j <= k; j++) emitted[j] = (j <= a) ? target[j] : -1;
  return (int)(a + 1);
}

/* Verify pass through the nested LM head and the accept rule, for B
 * sequences of k+1 rows each. y (nullable) receives the logits. */
void oracle_verify_accept(const int8_t* qa, const float* sa, int64_t B, int64_t k,
                          int64_t K, const uint8_t* base, const uint8_t* refine,
                          const float* scales, int64_t V, int64_t group,
                          const int32_t* draft, int32_t* target,
                          int32_t* n_emitted, int32_t* emitted, float* y) {
  int64_t M = B * (k + 1);
  float* logits = y ? y : (float*)malloc((size_t)(M * V) * sizeof(float));
  oracle_verify_gemm(qa, sa, M, K, base, refine, scales, V, group, logits, NULL);
  for (int64_t b = 0; b < B; b++) {
    for (int64_t i = 0; i <= k; i++)
      target[b * (k + 1) + i] =
          (int32_t)oracle_argmax(logits + (b * (k + 1) + i) * V, V);
    n_emitted[b] = oracle_accept(draft + b * k, target + b * (k + 1), k,
                                 emitted + b * (k + 1));
  }
  if (!y) free(logits);
}

/* ------------------------------------------------------------------ */
/* nested KV cache  [BitNest Fig. 4]                                   */
/* ------------------------------------------------------------------ */

/* Element index of (head h, token t, dim j) in each plane's layout.
 * K is token-major. V is stored dim-major inside each block of `block`
 * tokens. */
static int64_t k_index(int64_t h, int64_t t, int64_t j, int64_t cap, int64_t d) {
  return (h * cap + t) * d + j;
}
static int64_t v_index(int64_t h, int64_t t, int64_t j, int64_t cap, int64_t d,
                       int64_t block) {
  int64_t b = t / block;
  return h * cap * d + (b * d + j) * block + (t % block);
}

/* Quantize block b of head h, for K and for V, with tokens at or past
 * `valid` (counted from the block start) taken as 0. The values are
 * gathered in the plane's element order, quantized by the same rule as the
 * weights, and packed. With valid == block this is the plain block group of
 * kv_nest_pack. A zero never raises max|v|, so the scale of a partial block
 * covers exactly its valid tokens. */
static void kv_pack_block(const float* kf, const float* vf, int64_t h, int64_t b,
                          int64_t valid, int64_t cap, int64_t d, int64_t block,
                          uint8_t* kb, uint8_t* kr, float* ks, uint8_t* vb,
                          uint8_t* vr, float* vs) {
  int64_t nb = cap / block, n = block * d, hb = h * nb + b;
  float* gk = (float*)malloc((size_t)n * sizeof(float));
  float* gv = (float*)malloc((size_t)n * sizeof(float));
  int8_t* q1 = (int8_t*)malloc((size_t)n);
  int8_t* q2 = (int8_t*)malloc((size_t)n);
  for (int64_t t = b * block; t < (b + 1) * block; t++)
    for (int64_t j = 0; j < d; j++) {
      int live = t - b * block < valid;
      gk[k_index(h, t, j, cap, d) - h * cap * d - b * n] = live ? kf[(h * cap + t) * d + j] : 0.0f;
      gv[v_index(h, t, j, cap, d, block) - h * cap * d - b * n] = live ? vf[(h * cap + t) * d + j] : 0.0f;
    }
  int64_t off = (h * cap * d + b * n) / 2;
  oracle_quantize_group(gk, n, q1, q2, &ks[hb]);
  oracle_pack_nibbles(q1, n, kb + off);
  oracle_pack_nibbles(q2, n, kr + off);
  oracle_quantize_group(gv, n, q1, q2, &vs[hb]);
  oracle_pack_nibbles(q1, n, vb + off);
  oracle_pack_nibbles(q2, n, vr + off);
  free(gk);
  free(gv);
  free(q1);
  free(q2);
}

/* One group per (head, block), for K and for V [BitNest Fig. 4]. */
int oracle_kv_nest_pack(const float* kf, const float* vf, int64_t Hkv,
                        int64_t cap, int64_t d, int64_t block, uint8_t* kb,
                        uint8_t* kr, float* ks, uint8_t* vb, uint8_t* vr,
                        float* vs) {
  if (Hkv < 1 || cap < 1 || block < 2 || block % 2 || d < 2 || d % 2 ||
      cap % block)
    return -1;
  int64_t nb = cap / block;
#pragma omp parallel for schedule(static)
  for (int64_t hb = 0; hb < Hkv * nb; hb++)
    kv_pack_block(kf, vf, hb / nb, hb % nb, block, cap, d, block, kb, kr, ks, vb, vr, vs);
  return 0;
}

/* Append n tokens at positions pos .. pos+n-1 [BitNest Fig. 4: kept
 * entries stay; a rejected suffix is dropped by the caller's length
 * update and later overwritten by the next append]. kf and vf hold
 * every token's fp32 value [Hkv][cap][d]; the new values are written there,
 * then every block the new tokens touch is quantized again over its valid
 * tokens (those before pos + n), the rest taken as 0. A block that fills
 * thereby equals the kv_nest_pack block of its values. */
int oracle_kv_append(float* kf, float* vf, const float* k_new, const float* v_new,
                     int64_t Hkv, int64_t cap, int64_t d, int64_t block, int64_t pos,
                     int64_t n, uint8_t* kb, uint8_t* kr, float* ks, uint8_t* vb,
                     uint8_t* vr, float* vs) {
  if (Hkv < 1 || block < 2 || block % 2 || d < 2 || d % 2 || cap % block || pos < 0 ||
      n < 1 || pos + n > cap)
    return -1;
  for (int64_t h = 0; h < Hkv; h++)
    for (int64_t t = pos; t < pos + n; t++)
      for (int64_t j = 0; j < d; j++) {
        kf[(h * cap + t) * d + j] = k_new[(h * n + t - pos) * d + j];
        vf[(h * cap + t) * d + j] = v_new[(h * n + t - pos) * d + j];
      }
  int64_t end = pos + n;
  for (int64_t h = 0; h < Hkv; h++)
    for (int64_t b = pos / block; b <= (end - 1) / block; b++) {
      int64_t valid = end - b * block < block ? end - b * block : block;
      kv_pack_block(kf, vf, h, b, valid, cap, d, block, kb, kr, ks, vb, vr, vs);
    }
  return 0;
}

/* Value of one cache element in a view: base view s*q_b (draft), full view
 * (s/16)*(16*q_b + q_r) (verify) [BitNest Fig. 4]. */
static double kv_value(const uint8_t* pb, const uint8_t* pr, const float* sc,
                       int64_t idx, int64_t scale_idx, int view) {
  double s = (double)sc[scale_idx];
  if (view == 0) return s * (double)nibble_at(pb, idx);
  return (s / 16.0) * (double)(16 * nibble_at(pb, idx) + nibble_at(pr, idx));
}

static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Decode attention over the nested cache, in fp64. Query i sits at position
 * ctx - nq + i and sees tokens 0..that position. Query head hq reads kv
 * head hq/(Hq/Hkv). The score is q.k/sqrt(d). The softmax subtracts the
 * maximum score, and out is the weighted sum of v in the same view. */
void oracle_kv_attend(const uint16_t* q, int64_t nq, int64_t Hq, int64_t Hkv,
                      int64_t d, int64_t cap, int64_t block, const uint8_t* kb,
                      const uint8_t* kr, const float* ks, const uint8_t* vb,
                      const uint8_t* vr, const float* vs, int64_t ctx, int view,
                      double* out) {
  int64_t group = Hq / Hkv, nb = cap / block;
#pragma omp parallel for schedule(dynamic)
  for (int64_t iq = 0; iq < nq * Hq; iq++) {
    int64_t i = iq / Hq, hq = iq % Hq, h = hq / group;
    int64_t pos = ctx - nq + i;
    double* score = (double*)malloc((size_t)(pos + 1) * sizeof(double));
    double mx = -INFINITY;
    for (int64_t t = 0; t <= pos; t++) {
      double dot = 0.0;
      for (int64_t j = 0; j < d; j++)
        dot += bf16_to_double(q[(i * Hq + hq) * d + j]) *
               kv_value(kb, kr, ks, k_index(h, t, j, cap, d), h * nb + t / block, view);
      score[t] = dot / sqrt((double)d);
      if (score[t] > mx) mx = score[t];
    }
    double denom = 0.0;
    for (int64_t t = 0; t <= pos; t++) {
      score[t] = exp(score[t] - mx);
      denom += score[t];
    }
    for (int64_t j = 0; j < d; j++) {
      double acc = 0.0;
      for (int64_t t = 0; t <= pos; t++)
        acc += score[t] * kv_value(vb, vr, vs, v_index(h, t, j, cap, d, block),
                                   h * nb + t / block, view);
      out[(i * Hq + hq) * d + j] = acc / denom;
    }
    free(score);
  }
}

/* ------------------------------------------------------------------ */
/* choosing k: Eq. (1) and Eq. (2) of [Blog], section "Tokens per pass  */
/* and time per token"                                                  */
/* ------------------------------------------------------------------ */

/* Eq. (1): E = (1 - a^(k+1)) / (1 - a), with its limit k + 1 at a = 1. */
double oracle_expected_tokens(double alpha, int64_t k) {
  if (alpha == 1.0) return (double)(k + 1);
  return (1.0 - pow(alpha, (double)(k + 1))) / (1.0 - alpha);
}

/* Eq. (2): t_token = (t_pass + k t_draft) / E. */
double oracle_token_time(double alpha, int64_t k, double t_draft, double t_pass) {
  return (t_pass + (double)k * t_draft) / oracle_expected_tokens(alpha, k);
}

/* The k in [0, kmax] with the least time per token, t_pass[k] being the
 * pass time with k draft tokens; the smallest k among equal times. */
int64_t oracle_choose_k(double alpha, double t_draft, const double* t_pass, int64_t kmax) {
  int64_t best = 0;
  double tb = oracle_token_time(alpha, 0, t_draft, t_pass[0]);
  for (int64_t k = 1; k <= kmax; k++) {
    double t = oracle_token_time(alpha, k, t_draft, t_pass[k]);
    if (t < tb) {
      tb = t;
      best = k;
    }
  }
  return best;
}

/* Running acceptance rate from rounds: round r kept a_r of k_r drafts.
 * Under the independence of Eq. (1), a_r counts accepted slots and a round
 * with a_r < k_r ends in one rejected slot, so the estimate is accepted
 * slots over judged slots. Older rounds weigh decay^(age); the prior counts
 * weigh as a round before the first. */
double oracle_alpha_estimate(const int64_t* accepted, const int64_t* k, int64_t rounds, double decay,
                             double prior_accepted, double prior_rejected) {
  double acc = prior_accepted, rej = prior_rejected;
  for (int64_t r = 0; r < rounds; r++) {
    acc = decay * acc + (double)accepted[r];
    rej = decay * rej + (accepted[r] < k[r] ? 1.0 : 0.0);
  }
  return acc + rej > 0.0 ? acc / (acc + rej) : 0.0;
}

/* ------------------------------------------------------------------ */
/* speculative sampling ([Blog], section "The same output as the large  */
/* model alone": each draft token is kept with a probability set by the */
/* scores of both models, and after a rejection a replacement is drawn  */
/* from a corrected distribution; the method of Leviathan et al. and    */
/* Chen et al. that the page names, whose result follows the target's   */
/* distribution exactly). Readings: the scores are softmax(logits / T); */
/* a slot keeps d when u * q(d) < p(d) (probability min(1, p/q)); the   */
/* corrected distribution is max(0, p - q) normalized; a token is drawn */
/* by inverse CDF: the smallest t whose running weight exceeds u times  */
/* the total. Computed in fp64.                                         */
/* ------------------------------------------------------------------ */

/* softmax(y / T) in fp64. */
static void softmax_row(const float* y, int64_t V, double T, double* p) {
  double m = -INFINITY, s = 0.0;
  for (int64_t t = 0; t < V; t++)
    if ((double)y[t] > m) m = (double)y[t];
  for (int64_t t = 0; t < V; t++) {
    p[t] = exp(((double)y[t] - m) / T);
    s += p[t];
  }
  for (int64_t t = 0; t < V; t++) p[t] /= s;
}

/* Inverse CDF over the weights w: the smallest t whose running sum exceeds
 * u * sum(w); if rounding leaves none, the last t of positive weight.
 * Reports t's interval [lo, hi) of the running sum and the target u*sum. */
static int64_t inverse_cdf(const double* w, int64_t V, double u, double* lo, double* hi,
                           double* target) {
  double total = 0.0;
  for (int64_t t = 0; t < V; t++) total += w[t];
  const double tg = u * total;
  double run = 0.0;
  int64_t pick = -1;
  double at = 0.0;
  for (int64_t t = 0; t < V; t++) {
    if (run + w[t] > tg) {
      pick = t;
      at = run;
      break;
    }
    run += w[t];
  }
  if (pick < 0) {
    double r2 = 0.0;
    for (int64_t t = 0; t < V; t++) {
      if (w[t] > 0.0) {
        pick = t;
        at = r2;
      }
      r2 += w[t];
    }
  }
  *lo = at;
  *hi = at + w[pick];
  *target = tg;
  return pick;
}

/* Distance of the target from the nearer edge of [lo, hi). */
static double edge_margin(double lo, double hi, double tg) { return fmin(tg - lo, hi - tg); }

/* One token from softmax(y / T) with the uniform u; *margin (if non-NULL)
 * is the target's distance, in probability, from the drawn token's
 * interval edges. */
int64_t oracle_sample(const float* y, int64_t V, float T, float u, double* margin) {
  double* p = (double*)malloc((size_t)V * sizeof(double));
  softmax_row(y, V, (double)T, p);
  double lo, hi, tg;
  int64_t t = inverse_cdf(p, V, (double)u, &lo, &hi, &tg);
  if (margin) *margin = edge_margin(lo, hi, tg);
  free(p);
  return t;
}

/* The interval [lo, hi) of token t in the running sum of softmax(y / T),
 * and the target u * 1: lets a caller check a token drawn elsewhere. */
void oracle_sample_interval(const float* y, int64_t V, float T, float u, int64_t t, double* lo,
                            double* hi, double* target) {
  double* p = (double*)malloc((size_t)V * sizeof(double));
  softmax_row(y, V, (double)T, p);
  double run = 0.0, tot = 0.0;
  for (int64_t j = 0; j < V; j++) tot += p[j];
  for (int64_t j = 0; j < t; j++) run += p[j];
  *lo = run;
  *hi = run + p[t];
  *target = (double)u * tot;
  free(p);
}

/* The distribution a round draws its last token from, after a kept
 * drafts: max(0, p_{a+1} - q_{a+1}) when slot a+1 was rejected (a < k),
 * else p_{k+1} (the bonus). w gets V weights in probability units. */
static void final_weights(const float* yt, const float* yd, int64_t k, int64_t V, double T, int64_t a,
                          double* w, double* q) {
  softmax_row(yt + a * V, V, T, w);
  if (a < k) {
    softmax_row(yd + a * V, V, T, q);
    double tot = 0.0;
    for (int64_t t = 0; t < V; t++) tot += fmax(0.0, w[t] - q[t]);
    /* a rejection leaves mass in max(0, p - q) (p(d) < q(d)); only if
     * rounding took all of it is the draw made from p itself */
    if (tot > 0.0)
      for (int64_t t = 0; t < V; t++) w[t] = fmax(0.0, w[t] - q[t]);
  }
}

/* One speculative-sampling round of one sequence. yt [k+1][V]: the
 * target's logits at the k+1 positions (row i-1 scores draft slot i, row k
 * the bonus); yd [k][V]: the draft's logits draft token i was drawn from
 * (row i-1). Slot i keeps d_i when u_acc[i-1] * q_i(d_i) < p_i(d_i). At
 * the first slot that fails, the last token is drawn with u_fin from
 * max(0, p_i - q_i); when every slot is kept, from p_{k+1}. emitted gets
 * the kept drafts and the drawn token (-1 after); returns their number
 * a + 1. ratio (k values, if non-NULL) gets p_i(d_i) / q_i(d_i) of every
 * slot; *margin the drawn token's edge margin in probability units. */
int64_t oracle_verify_sample(const float* yt, const float* yd, int64_t k, int64_t V, float T,
                             const int32_t* draft, const float* u_acc, float u_fin,
                             int32_t* emitted, double* ratio, double* margin) {
  double* p = (double*)malloc((size_t)V * sizeof(double));
  double* q = (double*)malloc((size_t)V * sizeof(double));
  int64_t a = 0;
  int rejected = 0;
  for (int64_t i = 1; i <= k; i++) {
    softmax_row(yt + (i - 1) * V, V, (double)T, p);
    softmax_row(yd + (i - 1) * V, V, (double)T, q);
    const int32_t d = draft[i - 1];
    /* an id outside the vocabulary has no probability under either model
     * and is never kept */
    const double r = (d >= 0 && d < V) ? p[d] / q[d] : 0.0;
    if (ratio) ratio[i - 1] = r;
    if (!rejected) {
      if (d >= 0 && d < V && (double)u_acc[i - 1] * q[d] < p[d])
        emitted[a++] = d;
      else
        rejected = 1;
    }
  }
  final_weights(yt, yd, k, V, (double)T, a, p, q);
  double lo, hi, tg;
  emitted[a] = (int32_t)inverse_cdf(p, V, (double)u_fin, &lo, &hi, &tg);
  if (margin) *margin = edge_margin(lo, hi, tg);
  for (int64_t j = a + 1; j <= k; j++) emitted[j] = -1;
  free(p);
  free(q);
  return a + 1;
}

/* The interval [lo, hi) of token t in the running sum of the last token's
 * distribution after a kept drafts, and the target u_fin * total. */
void oracle_final_interval(const float* yt, const float* yd, int64_t k, int64_t V, float T, int64_t a,
                           float u_fin, int64_t t, double* lo, double* hi, double* target) {
  double* w = (double*)malloc((size_t)V * sizeof(double));
  double* q = (double*)malloc((size_t)V * sizeof(double));
  final_weights(yt, yd, k, V, (double)T, a, w, q);
  double run = 0.0, tot = 0.0;
  for (int64_t j = 0; j < V; j++) tot += w[j];
  for (int64_t j = 0; j < t; j++) run += w[j];
  *lo = run;
  *hi = run + w[t];
  *target = (double)u_fin * tot;
  free(w);
  free(q);
}

/*
 * eta_oracle.c -- plain fp64 CPU reference of ETA block-sparse decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * library under long_context_decode_eta_amd/) never links, loads or calls it,
 * and this file shares no code, header, table or constant with that path.
 *
 * Source of every formula: the paper "Elastic Threshold Attention: Learned
 * Contextual Sparsity for Long-Context Decoding" as summarised on the
 * picx.dev page "Summary (Overview)":
 *   - Theoretical Foundation: dense attention A_ts = softmax_s(<q_t,k_s>/sqrt(d_h)),
 *     o_t = sum_s A_ts v_s, and sparse attention over an active index set.
 *   - Methodology 1, Eq. 1: tau_t = qbar_t W_tau + b_tau, qbar_t = concatenation
 *     of the H per-head query vectors.
 *   - Methodology 2, Eqs. 2-3: gate m_ts = sigmoid(beta (S_ts - tau)), gated
 *     logits S_ts * M_ts with M_tt = 1 (the query's own key is never gated).
 *   - Methodology 4, Eq. 5: per-block centroid mu_B, per-coordinate variance
 *     sigma2_B, max key norm M_B; Score = (1/sqrt(d_h)) min(<q,mu_B> +
 *     z sigma_S, ||q||_2 M_B), sigma_S = sqrt(sum_i q_i^2 sigma2_B,i); a block
 *     whose score is below the threshold is skipped.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes):
 *   - the variance is the population variance (divide by b), two-pass;
 *   - M_B is the largest Euclidean key norm in the block;
 *   - a block is pruned iff Score < threshold, so a tie is kept;
 *   - the block holding the newest key (position T-1) is always admitted: it
 *     holds the ungated diagonal key of Eq. 3 and, when partial, has no
 *     statistics; a partial block is never scored;
 *   - attention over the admitted keys is normalised over those keys only
 *     (what an online softmax over the loaded blocks computes);
 *   - z = +infinity means the geometric term alone (no inf*0);
 *   - the screening threshold is tau - a ("threshold adjustment" a), while
 *     the gate of Eq. 2 uses tau itself.
 *
 * Numbers: every quantity is double.  Inputs are the same bits the GPU reads:
 * q, W, b_tau are float; K and V are float or bfloat16 (raw 16-bit patterns,
 * widened exactly).
 *
 * Layouts (row-major):
 *   q      [B][H][d]          (qbar of Eq. 1 is q[b] read as [H*d])
 *   K, V   [B][H][cap][d]     (one stream of cap key slots per sequence/head)
 *   W      [H*d][H]
 *   mu,var [B][H][nbcap][d], M [B][H][nbcap]   (nbcap = ceil(cap/b))
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_GATED 0
#define ORC_RAW 1

/* One key/value element widened to double.  A bfloat16 is the upper half of
 * an IEEE binary32, so the widening is exact. */
static double elem(const void* base, int dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ---------------------------------------------------------------------- */
/* Block statistics (Methodology 4): for every complete block j of b keys,
 * mu_j = mean of the keys, var_j = population variance per coordinate
 * (two passes), M_j = max Euclidean key norm.  Only floor(T/b) blocks are
 * complete; the partial tail block gets no statistics. */
int eta_oracle_block_meta(const void* K, int dtype, int T, int d, int b,
                          double* mu, double* var, double* maxnorm) {
  int nbc = T / b;
  for (int j = 0; j < nbc; ++j) {
    for (int i = 0; i < d; ++i) {
      double s = 0.0;
      for (int r = 0; r < b; ++r) s += elem(K, dtype, (size_t)(j * b + r) * d + i);
      mu[(size_t)j * d + i] = s / b;
    }
    for (int i = 0; i < d; ++i) {
      double m = mu[(size_t)j * d + i], s = 0.0;
      for (int r = 0; r < b; ++r) {
        double x = elem(K, dtype, (size_t)(j * b + r) * d + i) - m;
        s += x * x;
      }
      var[(size_t)j * d + i] = s / b;
    }
    double best = 0.0;
    for (int r = 0; r < b; ++r) {
      double n2 = 0.0;
      for (int i = 0; i < d; ++i) {
        double x = elem(K, dtype, (size_t)(j * b + r) * d + i);
        n2 += x * x;
      }
      double n = sqrt(n2);
      if (n > best) best = n;
    }
    maxnorm[j] = best;
  }
  return nbc;
}

/* ---------------------------------------------------------------------- */
/* Stored form of the block index.  The pages fix no storage precision; this
 * implementation stores mu and var as bfloat16, each rounded to nearest (ties
 * to even) from its exact value: 8 significant bits.  x = m 2^e with
 * 0.5 <= |m| < 1, so m 2^8 lies in [128, 256) and rounding it to an integer
 * (nearbyint: the default round-to-nearest-even mode) keeps 8 bits.  Zero,
 * infinities and NaN pass unchanged; values below the bfloat16 normal range
 * do not occur in block statistics of finite keys of moderate size. */
double eta_oracle_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  double m = frexp(x, &e);
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

void eta_oracle_round_bf16_array(double* x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = eta_oracle_round_bf16(x[i]);
}

/* ---------------------------------------------------------------------- */
/* Threshold (Methodology 1, Eq. 1).  Dynamic: tau[b][h] = sum_j qbar[b][j]
 * W[j][h] + bias[h].  Frozen (W == NULL): tau[b][h] = c[h], the per-head
 * constants of offline calibration.  The screen uses tau - a. */
void eta_oracle_predict_tau(int B, int H, int d, const float* q, const float* W,
                            const float* bias_or_c, double a, double* tau,
                            double* tau_screen) {
  for (int bb = 0; bb < B; ++bb)
    for (int h = 0; h < H; ++h) {
      double t = (double)bias_or_c[h];
      if (W) {
        double s = 0.0;
        for (int j = 0; j < H * d; ++j)
          s += (double)q[(size_t)bb * H * d + j] * (double)W[(size_t)j * H + h];
        t += s;
      }
      tau[bb * H + h] = t;
      tau_screen[bb * H + h] = t - a;
    }
}

/* ---------------------------------------------------------------------- */
/* Dual screening score of one block (Methodology 4, Eq. 5). */
double eta_oracle_block_score(const float* q, const double* mu, const double* var,
                              double maxnorm, int d, double z, double scale) {
  double dot = 0.0, mom = 0.0, qq = 0.0;
  for (int i = 0; i < d; ++i) {
    double qi = (double)q[i];
    dot += qi * mu[i];
    mom += qi * qi * var[i];
    qq += qi * qi;
  }
  double geometric = sqrt(qq) * maxnorm;
  if (isinf(z)) return scale * geometric;
  double probabilistic = dot + z * sqrt(mom);
  return scale * (probabilistic < geometric ? probabilistic : geometric);
}

/* Admission of every block of one stream of T keys.  nb = ceil(T/b) blocks;
 * complete block j is admitted iff score[j] >= tau_screen; the block holding
 * key T-1 is always admitted.  Returns the number of admitted blocks. */
int eta_oracle_admit(int T, int b, const double* score, double tau_screen,
                     uint8_t* active) {
  int nb = (T + b - 1) / b, nbc = T / b, cnt = 0;
  for (int j = 0; j < nb; ++j) {
    int on = (j == nb - 1) || (j < nbc && score[j] >= tau_screen);
    active[j] = (uint8_t)on;
    cnt += on;
  }
  return cnt;
}

/* ---------------------------------------------------------------------- */
/* Attention of one query over the admitted keys of one stream (Theoretical
 * Foundation, sparse form; logits per Methodology 2, Eq. 3 in GATED mode).
 * S_s = scale <q, k_s>.  GATED: l_s = S_s * sigmoid(beta (S_s - tau)) for
 * s != T-1, l_{T-1} = S_{T-1}.  RAW: l_s = S_s.  Softmax over admitted s.
 * With no admitted key (T == 0) the output is zero. */
void eta_oracle_attend(const float* q, const void* K, const void* V, int dtype,
                       int T, int d, int b, const uint8_t* active, int mode,
                       double beta, double tau, double scale, double* out) {
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  if (T <= 0) return;
  double* logit = (double*)malloc(sizeof(double) * (size_t)T);
  double top = -INFINITY;
  for (int s = 0; s < T; ++s) {
    if (!active[s / b]) continue;
    double S = 0.0;
    for (int i = 0; i < d; ++i) S += (double)q[i] * elem(K, dtype, (size_t)s * d + i);
    S *= scale;
    double l = S;
    if (mode == ORC_GATED && s != T - 1) l = S * (1.0 / (1.0 + exp(-beta * (S - tau))));
    logit[s] = l;
    if (l > top) top = l;
  }
  double den = 0.0;
  for (int s = 0; s < T; ++s) {
    if (!active[s / b]) continue;
    double w = exp(logit[s] - top);
    den += w;
    for (int i = 0; i < d; ++i) out[i] += w * elem(V, dtype, (size_t)s * d + i);
  }
  for (int i = 0; i < d; ++i) out[i] /= den;
  free(logit);
}

/* Dense decode attention (Theoretical Foundation, dense form). */
void eta_oracle_dense(const float* q, const void* K, const void* V, int dtype, int T,
                      int d, double scale, double* out) {
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  if (T <= 0) return;
  double* S = (double*)malloc(sizeof(double) * (size_t)T);
  double top = -INFINITY;
  for (int s = 0; s < T; ++s) {
    double x = 0.0;
    for (int i = 0; i < d; ++i) x += (double)q[i] * elem(K, dtype, (size_t)s * d + i);
    S[s] = scale * x;
    if (S[s] > top) top = S[s];
  }
  double den = 0.0;
  for (int s = 0; s < T; ++s) {
    double w = exp(S[s] - top);
    den += w;
    for (int i = 0; i < d; ++i) out[i] += w * elem(V, dtype, (size_t)s * d + i);
  }
  for (int i = 0; i < d; ++i) out[i] /= den;
  free(S);
}

/* Threads an OpenMP region of the batch drivers uses. */
int eta_oracle_threads(void) { return omp_get_max_threads(); }
void eta_oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ---------------------------------------------------------------------- */
/* Batch drivers: the same steps for every (sequence, head) stream, one
 * OpenMP iteration per stream.  elt_bytes of K/V follows dtype. */
static size_t elt_bytes(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

void eta_oracle_meta_batch(int B, int H, int d, int b, int cap, int dtype,
                           const int32_t* seq_len, const void* K, double* mu,
                           double* var, double* maxnorm) {
  int nbcap = (cap + b - 1) / b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < B * H; ++u) {
    const char* k = (const char*)K + (size_t)u * cap * d * elt_bytes(dtype);
    eta_oracle_block_meta(k, dtype, seq_len[u / H], d, b, mu + (size_t)u * nbcap * d,
                          var + (size_t)u * nbcap * d, maxnorm + (size_t)u * nbcap);
  }
}

/* Screen and attention for a batch, given the thresholds (fp64):
 * score [B][H][nbcap] (complete blocks only, NaN elsewhere), active
 * [B][H][nbcap], cnt [B][H] admitted blocks, tokens [B][H] admitted keys,
 * out [B][H][d]. */
void eta_oracle_screen_attend_batch(int B, int H, int d, int b, int cap, int dtype,
                                    const int32_t* seq_len, const float* q, const void* K,
                                    const void* V, const double* mu, const double* var,
                                    const double* maxnorm, const double* tau,
                                    const double* tau_screen, double z, double scale, int mode,
                                    double beta, double* score, uint8_t* active, int32_t* cnt,
                                    int64_t* tokens, double* out) {
  int nbcap = (cap + b - 1) / b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < B * H; ++u) {
    int T = seq_len[u / H];
    const float* qu = q + (size_t)u * d;
    size_t kv_off = (size_t)u * cap * d * elt_bytes(dtype);
    double* sc = score + (size_t)u * nbcap;
    uint8_t* act = active + (size_t)u * nbcap;
    for (int j = 0; j < nbcap; ++j) sc[j] = NAN;
    for (int j = 0; j < T / b; ++j)
      sc[j] = eta_oracle_block_score(qu, mu + ((size_t)u * nbcap + j) * d,
                                     var + ((size_t)u * nbcap + j) * d,
                                     maxnorm[(size_t)u * nbcap + j], d, z, scale);
    memset(act, 0, (size_t)nbcap);
    cnt[u] = eta_oracle_admit(T, b, sc, tau_screen[u], act);
    int64_t tk = 0;
    for (int s = 0; s < T; ++s) tk += act[s / b];
    tokens[u] = tk;
    eta_oracle_attend(qu, (const char*)K + kv_off, (const char*)V + kv_off, dtype, T, d, b,
                      act, mode, beta, tau[u], scale, out + (size_t)u * d);
  }
}

/* One decode step for a batch: threshold (Eq. 1), then screen and attention. */
void eta_oracle_step_batch(int B, int H, int d, int b, int cap, int dtype,
                           const int32_t* seq_len, const float* q, const void* K,
                           const void* V, const double* mu, const double* var,
                           const double* maxnorm, const float* W, const float* bias_or_c,
                           double a, double z, double scale, int mode, double beta,
                           double* tau, double* tau_screen, double* score,
                           uint8_t* active, int32_t* cnt, int64_t* tokens, double* out) {
  eta_oracle_predict_tau(B, H, d, q, W, bias_or_c, a, tau, tau_screen);
  eta_oracle_screen_attend_batch(B, H, d, b, cap, dtype, seq_len, q, K, V, mu, var, maxnorm,
                                 tau, tau_screen, z, scale, mode, beta, score, active, cnt,
                                 tokens, out);
}

/* Attention of every stream over a given admission mask (used to re-evaluate
 * the output on a mask that differs from the oracle's own only at near-ties). */
void eta_oracle_attend_batch(int B, int H, int d, int b, int cap, int dtype,
                             const int32_t* seq_len, const float* q, const void* K,
                             const void* V, const uint8_t* active, int mode, double beta,
                             const double* tau, double scale, double* out) {
  int nbcap = (cap + b - 1) / b;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < B * H; ++u) {
    size_t kv_off = (size_t)u * cap * d * elt_bytes(dtype);
    eta_oracle_attend(q + (size_t)u * d, (const char*)K + kv_off, (const char*)V + kv_off,
                      dtype, seq_len[u / H], d, b, active + (size_t)u * nbcap, mode, beta,
                      tau[u], scale, out + (size_t)u * d);
  }
}

void eta_oracle_dense_batch(int B, int H, int d, int cap, int dtype, const int32_t* seq_len,
                            const float* q, const void* K, const void* V, double scale,
                            double* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < B * H; ++u) {
    size_t kv_off = (size_t)u * cap * d * elt_bytes(dtype);
    eta_oracle_dense(q + (size_t)u * d, (const char*)K + kv_off, (const char*)V + kv_off,
                     dtype, seq_len[u / H], d, scale, out + (size_t)u * d);
  }
}

/* ---------------------------------------------------------------------- */
/* Grouped-query decode (the pages' benchmark shape: several query heads
 * share one KV head; v2 page, Table 5; summary, Theoretical and Practical
 * Implications on the GQA-union bandwidth).  Query head h = kv * G + g reads
 * KV head kv.  Each query head is screened with its own query and threshold
 * against the KV head's block statistics (Eq. 5), attends only over the
 * blocks it admits itself (D_head), and a KV block is loaded when any head of
 * the group admits it (the union, D_union).
 *   q [B][Hkv*G][d], tau/tau_screen [B][Hkv*G]; K, V, statistics per KV head.
 * Outputs: score/active [B][Hkv*G][nbcap], cnt/tokens [B][Hkv*G],
 * union_active [B][Hkv][nbcap], union_cnt/union_tokens [B][Hkv], out
 * [B][Hkv*G][d]. */
void eta_oracle_gqa_screen_attend_batch(int B, int Hkv, int G, int d, int b, int cap, int dtype,
                                        const int32_t* seq_len, const float* q, const void* K,
                                        const void* V, const double* mu, const double* var,
                                        const double* maxnorm, const double* tau,
                                        const double* tau_screen, double z, double scale,
                                        int mode, double beta, double* score, uint8_t* active,
                                        int32_t* cnt, int64_t* tokens, uint8_t* union_active,
                                        int32_t* union_cnt, int64_t* union_tokens, double* out) {
  int nbcap = (cap + b - 1) / b;
  int Hq = Hkv * G;
#pragma omp parallel for schedule(dynamic, 1)
  for (int uq = 0; uq < B * Hq; ++uq) {
    int bb = uq / Hq, kv = (uq % Hq) / G;
    size_t ukv = (size_t)bb * Hkv + kv;
    int T = seq_len[bb];
    const float* qu = q + (size_t)uq * d;
    size_t kv_off = ukv * cap * d * elt_bytes(dtype);
    double* sc = score + (size_t)uq * nbcap;
    uint8_t* act = active + (size_t)uq * nbcap;
    for (int j = 0; j < nbcap; ++j) sc[j] = NAN;
    for (int j = 0; j < T / b; ++j)
      sc[j] = eta_oracle_block_score(qu, mu + (ukv * nbcap + j) * d, var + (ukv * nbcap + j) * d,
                                     maxnorm[ukv * nbcap + j], d, z, scale);
    memset(act, 0, (size_t)nbcap);
    cnt[uq] = eta_oracle_admit(T, b, sc, tau_screen[uq], act);
    int64_t tk = 0;
    for (int s = 0; s < T; ++s) tk += act[s / b];
    tokens[uq] = tk;
    eta_oracle_attend(qu, (const char*)K + kv_off, (const char*)V + kv_off, dtype, T, d, b, act,
                      mode, beta, tau[uq], scale, out + (size_t)uq * d);
  }
  for (int u = 0; u < B * Hkv; ++u) {
    int T = seq_len[u / Hkv];
    uint8_t* un = union_active + (size_t)u * nbcap;
    int c = 0;
    int64_t tk = 0;
    for (int j = 0; j < nbcap; ++j) {
      uint8_t on = 0;
      for (int g = 0; g < G; ++g) on |= active[((size_t)u * G + g) * nbcap + j];
      un[j] = on;
      c += on;
    }
    for (int s = 0; s < T; ++s) tk += un[s / b];
    union_cnt[u] = c;
    union_tokens[u] = tk;
  }
}

/* Dense grouped-query decode: every query head over every key of its KV head. */
void eta_oracle_gqa_dense_batch(int B, int Hkv, int G, int d, int cap, int dtype,
                                const int32_t* seq_len, const float* q, const void* K,
                                const void* V, double scale, double* out) {
  int Hq = Hkv * G;
#pragma omp parallel for schedule(dynamic, 1)
  for (int uq = 0; uq < B * Hq; ++uq) {
    int bb = uq / Hq, kv = (uq % Hq) / G;
    size_t kv_off = ((size_t)bb * Hkv + kv) * cap * d * elt_bytes(dtype);
    eta_oracle_dense(q + (size_t)uq * d, (const char*)K + kv_off, (const char*)V + kv_off, dtype,
                     seq_len[bb], d, scale, out + (size_t)uq * d);
  }
}

/* ---------------------------------------------------------------------- */
/* Gated causal attention over a whole sequence: the forward pass of the
 * model's own attention in prefill or training (summary, Methodology 2,
 * Eqs. 2-3), and the per-row density term of the sparsity loss (Methodology
 * 3, Eq. 4).  Query head h of sequence b reads KV head h / G.  For query
 * position t (0-based) and keys s = 0..t:
 *   S_ts   = scale <q_t, k_s>
 *   m_ts   = sigmoid(beta (S_ts - tau_t))                      (Eq. 2)
 *   l_ts   = S_ts for s = t, S_ts m_ts otherwise; causal softmax (Eq. 3)
 *   out_t  = sum_s softmax(l_t.)_s v_s
 *   dens_t = (1 / (t + 1)) sum_{s <= t} m_ts   (the inner average of Eq. 4)
 * The layer's sparsity term is lambda / (H T) sum_h sum_t dens_t.  q, K and
 * V share one element type; tau is [B][H_q][T]. */
void eta_oracle_prefill(int B, int Hkv, int G, int T, int d, int dtype, const void* q,
                        const void* K, const void* V, const double* tau, double beta,
                        double scale, double* out, double* dens) {
  int Hq = Hkv * G;
  size_t eb = elt_bytes(dtype);
#pragma omp parallel for schedule(dynamic, 1)
  for (long long row = 0; row < (long long)B * Hq * T; ++row) {
    int t = (int)(row % T);
    long long uq = row / T;
    int bb = (int)(uq / Hq), kv = (int)((uq % Hq) / G);
    const char* qt = (const char*)q + (size_t)row * d * eb;
    const char* Ku = (const char*)K + ((size_t)bb * Hkv + kv) * (size_t)T * d * eb;
    const char* Vu = (const char*)V + ((size_t)bb * Hkv + kv) * (size_t)T * d * eb;
    double tt = tau[row];
    double* logit = (double*)malloc(sizeof(double) * (size_t)(t + 1));
    double top = -INFINITY, msum = 0.0;
    for (int s = 0; s <= t; ++s) {
      double S = 0.0;
      for (int i = 0; i < d; ++i) S += elem(qt, dtype, (size_t)i) * elem(Ku, dtype, (size_t)s * d + i);
      S *= scale;
      double m = 1.0 / (1.0 + exp(-beta * (S - tt)));
      msum += m;
      double l = (s == t) ? S : S * m;
      logit[s] = l;
      if (l > top) top = l;
    }
    double* o = out + (size_t)row * d;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    double den = 0.0;
    for (int s = 0; s <= t; ++s) {
      double w = exp(logit[s] - top);
      den += w;
      for (int i = 0; i < d; ++i) o[i] += w * elem(Vu, dtype, (size_t)s * d + i);
    }
    for (int i = 0; i < d; ++i) o[i] /= den;
    if (dens) dens[row] = msum / (double)(t + 1);
    free(logit);
  }
}

/* ---------------------------------------------------------------------- */
/* Offline calibration of frozen per-head constants (the pages describe an
 * offline algorithm that freezes per-(layer, head) thresholds but give no
 * steps; this is the plain quantile reading).  For head h, pool over the
 * calibration query sets n and sequences b the values
 *     x = Score(q_{n,b,h}, block j) - tau0_{n,b,h}
 * of every complete block j that is not the always-admitted last block
 * (tau0 = the query-dependent part of the threshold, 0 for frozen use).
 * The last block of every stream is admitted regardless and contributes its
 * tokens F.  With all blocks holding b tokens, admitting k pooled blocks
 * gives density (F + k b) / sum T; k = round((rho sum T - F) / b), clamped to
 * [0, N].  c_h is the midpoint of the k-th and (k+1)-th largest pooled
 * values (-inf when k = N, +inf when k = 0), so exactly the top k pass
 * x >= c_h when those two values differ. */
static int cmp_desc(const void* pa, const void* pb) {
  double a = *(const double*)pa, b = *(const double*)pb;
  return (a < b) - (a > b);
}

void eta_oracle_calibrate(int n_sets, int B, int H, int d, int b, int cap,
                          const int32_t* seq_len, const float* q_sets, const double* mu,
                          const double* var, const double* maxnorm, const double* tau0,
                          double z, double scale, double rho, double* c_out,
                          int64_t* k_out) {
  int nbcap = (cap + b - 1) / b;
  for (int h = 0; h < H; ++h) {
    size_t n = 0;
    double total = 0.0, forced = 0.0;
    for (int bb = 0; bb < B; ++bb) {
      int T = seq_len[bb];
      if (T <= 0) continue;
      int nb = (T + b - 1) / b;
      n += (size_t)n_sets * (nb - 1);
      total += (double)n_sets * T;
      forced += (double)n_sets * (T - (nb - 1) * b);
    }
    double* x = (double*)malloc(sizeof(double) * (n ? n : 1));
    size_t p = 0;
    for (int s = 0; s < n_sets; ++s)
      for (int bb = 0; bb < B; ++bb) {
        int T = seq_len[bb];
        if (T <= 0) continue;
        int cand = (T + b - 1) / b - 1; /* every block but the last is complete */
        size_t u = (size_t)bb * H + h;
        const float* qv = q_sets + (((size_t)s * B + bb) * H + h) * d;
        double t0 = tau0 ? tau0[((size_t)s * B + bb) * H + h] : 0.0;
        for (int j = 0; j < cand; ++j)
          x[p++] = eta_oracle_block_score(qv, mu + (u * nbcap + j) * d,
                                          var + (u * nbcap + j) * d, maxnorm[u * nbcap + j],
                                          d, z, scale) - t0;
      }
    qsort(x, n, sizeof(double), cmp_desc);
    double want = (rho * total - forced) / b;
    long long k = (long long)floor(want + 0.5);
    if (k < 0) k = 0;
    if (k > (long long)n) k = (long long)n;
    double c;
    if (k == (long long)n) c = -INFINITY;
    else if (k == 0) c = INFINITY;
    else c = 0.5 * (x[k - 1] + x[k]);
    c_out[h] = c;
    if (k_out) k_out[h] = k;
    free(x);
  }
}

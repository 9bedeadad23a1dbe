/*
 * dust_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU oracle for Dust's per-token zeroth-order weight
 * gradient estimator of one linear layer y_t = W x_t.  Only tests/, the
 * package's smoke() entry and bench.py's cpu_baseline leg may load this
 * library.  It shares no code, header, table or constant generator with the
 * HIP path under token_activation_perturbation_amd/csrc, and it includes
 * nothing from there.
 *
 * What it computes, step by step, in the order the method is written:
 *   1. y_t = W x_t, delta_t = y_t - target_t and the clean per-token loss
 *      L_t = 1/2 ||delta_t||^2  (layer-local squared error stands in for the
 *      network; "Dust: every token is a member of the population", section
 *      "Perturb the activations, not the weights": dL/dW = sum_t delta_t x_t^T).
 *   2. For every draw i and token t the literal perturbed loss
 *      L_t^(i) = 1/2 ||y_t + s_i sigma a_t^(n(i)) - target_t||^2 and the loss
 *      reduction rho_t^(i) = L_t - L_t^(i)  (same page, section "What the
 *      released code actually does", step 2: reward = clean minus perturbed).
 *   3. Centring across the K draws of one call, which share one forward:
 *      c_t^(i) = rho_t^(i) - (1/K) sum_j rho_t^(j)  (same section, step 2,
 *      and the definition of c_s under the estimator equations).
 *   4. Discounted credit, reset at every sequence end:
 *      r_t^(i) = sum_{s >= t, s in seq(t)} gamma^(s-t) c_s^(i), computed as
 *      the reverse recursion r_t = c_t + gamma r_{t+1}  (estimator equation
 *      for r_t, section "Perturb the activations, not the weights").
 *   5. g_t = -1/(K sigma) sum_i r_t^(i) s_i a_t^(n(i))  (estimator equation
 *      for g_t, same section; the antithetic sign s_i is part of the jitter
 *      of draw i, section "What a zeroth-order gradient is").
 *   6. G_W = sum_t g_t x_t^T  (estimator equation for G_W, same section;
 *      the einsum 'btd,bti->di' of "What the released code actually does",
 *      step 7).  Not divided by the token count.
 *
 * A second scoring rule replaces the loss of steps 1-2 with a linear score
 * against a supplied error estimate e_t of the layer's output ("What the
 * released code actually does", step 4: a perturbation of an attention
 * internal earns the score c_s = -<g_s, Delta o_s>, the inner product of
 * the output's change with an error estimate of that output; keys and
 * values decay later tokens' scores by gamma = 0.98, queries keep their own).
 * Reading used: the jittered output is the layer's own, Delta o_t^(i) =
 * s_i sigma a_t^(n(i)), so the score of draw i at token t is
 * rho_t^(i) = -<e_t, Delta o_t^(i)>, evaluated literally; steps 3-6 then
 * run unchanged (dust_oracle_estimate_local).
 *
 * In the page's own form of that step the perturbed internal is a query,
 * key or value of an attention block, the block's attention is evaluated
 * again from the activations kept from the clean forward, and the score
 * uses the change of the attention output.  Reading used: one block's
 * causal softmax attention with H heads of width d_head inside each
 * sequence, o_s = sum_{t <= s} softmax_t(<q_s, k_t> / sqrt(d_head)) v_t per
 * head; the site (queries, keys or values, a [T][H d_head] array whose head
 * h holds channels h d_head .. h d_head + d_head - 1) takes draw i's jitter
 * s_i sigma a_t^(n(i)) over its channels; every output of the sequence is
 * recomputed literally with the jittered site, and the score of token s is
 * rho_s^(i) = -sum_h <e_s,h, o'_s,h - o_s,h>, e the supplied error estimate
 * of the attention output [T][H d_head]; steps 3-6 then run unchanged, the
 * site's weight gradient being sum_t g_t x_t^T with x the block's input
 * (dust_oracle_estimate_attention).
 *
 * A third scoring rule is the model's head: cross-entropy of the logits
 * z_t = W x_t against a label y_t, its logits perturbed in 256-column
 * slabs of the vocabulary ("What the released code actually does", step 5).
 * Reading used: every slab j is its own site with K draws; draw i of slab j
 * adds s_i sigma a_t^(n(i))[c] to the logits of the slab's columns c only
 * (the same noise values as the full-width jitter, restricted to the slab),
 * rho = CE(z_t) - CE(z_t + jitter), evaluated literally with a full
 * log-sum-exp over all columns; the centring is over the K draws of the same
 * slab and token; gamma = 0 (the loss is per token); g_t's columns of slab j
 * come from slab j's draws (dust_oracle_estimate_head).
 *
 * A fourth site is a token embedding o_t = E[id_t] ("What the released code
 * actually does", step 7: an embedding's error becomes its weight gradient
 * by a scatter-add, and every estimate is divided by the token count before
 * it is written to .grad).  Reading used: the layer-local loss of step 1
 * with y_t = E[id_t] (a gather in place of W x_t), steps 2-5 unchanged, and
 * step 6 replaced by G_E[v] = scale sum_{t: id_t = v} g_t, summed in token
 * order, rows of ids that do not occur being zero; scale = 1/T writes what
 * the page writes to .grad, scale = 1 the plain sum
 * (dust_oracle_estimate_embedding, dust_oracle_reassemble_embedding).
 *
 * Noise (the pages fix no generator; they name Philox as a counter-based
 * generator whose n-th output is a pure function of (seed, n): "Scaling To
 * Unfathomable Depth", section "MeZO", last paragraphs).  Reading used here:
 *   draw i uses noise index n(i) = i, or floor(i/2) with antithetic pairs,
 *   and sign s_i = +1, or (-1)^i with antithetic pairs;
 *   channel quad q = floor(c/4) of token t under noise index n takes the four
 *   words of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with counter
 *   (q, t, n, 0) and key (seed mod 2^32, floor(seed / 2^32));
 *   words (w0,w1) give channels 4q, 4q+1 and (w2,w3) channels 4q+2, 4q+3 by
 *   Box-Muller on 23-bit uniforms (the top 23 bits of each word):
 *   u = 1 - (w_even >> 9) 2^-23 in (0,1], v = (w_odd >> 9) 2^-23 in [0,1),
 *   R = sqrt(-2 ln u), a_even = R cos(2 pi v), a_odd = R sin(2 pi v).
 *
 * Parity is pinned (see tests/): Philox words against an independent library
 * implementation, the Gaussians by distribution tests, each estimator step
 * by closed forms, brute-force sums and statistical laws.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_TWO_PI 6.283185307179586476925286766559

/* Philox4x32 round constants (Salmon et al., SC'11, section on Philox). */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* Philox4x32-10: ten rounds of two 32x32->64 multiplies and xors, the key
 * bumped by the Weyl constants between rounds. */
void dust_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                               uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;
    uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)x2;
    uint32_t y0 = (uint32_t)(prod1 >> 32) ^ x1 ^ k0;
    uint32_t y1 = (uint32_t)prod1;
    uint32_t y2 = (uint32_t)(prod0 >> 32) ^ x3 ^ k1;
    uint32_t y3 = (uint32_t)prod0;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* The four words of quad q of token t under noise index n. */
static void quad_words(uint64_t seed, uint32_t n, uint32_t t, uint32_t q,
                       uint32_t w[4]) {
  uint32_t ctr[4] = {q, t, n, 0u};
  uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  dust_oracle_philox4x32_10(ctr, key, w);
}

/* Box-Muller on one pair of words, in fp64. */
static void box_muller(uint32_t w_even, uint32_t w_odd, double *a_even,
                       double *a_odd) {
  double u = 1.0 - (double)(w_even >> 9) * (1.0 / 8388608.0);
  double v = (double)(w_odd >> 9) * (1.0 / 8388608.0);
  double radius = sqrt(-2.0 * log(u));
  *a_even = radius * cos(ORACLE_TWO_PI * v);
  *a_odd = radius * sin(ORACLE_TWO_PI * v);
}

/* The noise vector a_t^(n) over all d_out channels, in fp64. */
static void noise_vector(uint64_t seed, uint32_t n, uint32_t t, int64_t d_out,
                         double *a) {
  int64_t n_quads = (d_out + 3) / 4;
  for (int64_t q = 0; q < n_quads; ++q) {
    uint32_t w[4];
    double g[4];
    quad_words(seed, n, t, (uint32_t)q, w);
    box_muller(w[0], w[1], &g[0], &g[1]);
    box_muller(w[2], w[3], &g[2], &g[3]);
    for (int j = 0; j < 4; ++j) {
      int64_t c = 4 * q + j;
      if (c < d_out) a[c] = g[j];
    }
  }
}

/* Test hook: words[n][t][4*ceil(d_out/4)] and gauss[n][t][d_out] for the
 * noise indices n0..n0+n_cnt-1 and tokens t0..t0+t_cnt-1.  Either output may
 * be NULL. */
void dust_oracle_noise_fill(uint64_t seed, int64_t n0, int64_t n_cnt,
                            int64_t t0, int64_t t_cnt, int64_t d_out,
                            uint32_t *words, double *gauss) {
  int64_t n_quads = (d_out + 3) / 4;
  for (int64_t ni = 0; ni < n_cnt; ++ni) {
    for (int64_t ti = 0; ti < t_cnt; ++ti) {
      uint32_t n = (uint32_t)(n0 + ni), t = (uint32_t)(t0 + ti);
      if (words) {
        uint32_t *dst = words + (ni * t_cnt + ti) * 4 * n_quads;
        for (int64_t q = 0; q < n_quads; ++q)
          quad_words(seed, n, t, (uint32_t)q, dst + 4 * q);
      }
      if (gauss) noise_vector(seed, n, t, d_out, gauss + (ni * t_cnt + ti) * d_out);
    }
  }
}

/* ------------------------------------------------------------------------ */

typedef struct {
  const float *X, *W, *target;
  const float *E;         /* error estimate [T][d_out] (local scoring only) */
  const int32_t *ids;     /* token ids [T] (embedding only; W is the table) */
  const float *Qa, *Ka, *Va; /* cached attention activations [T][H d_head] */
  int64_t heads, d_head;  /* attention site: heads and head width */
  int32_t site;           /* 0 queries, 1 keys, 2 values */
  int64_t T, d_in, d_out, seq_len;
  int32_t K;
  double sigma, gamma;
  uint64_t seed;
  int32_t antithetic;
  int64_t t_begin, t_end; /* token range handled by this call */
  double *delta;          /* [t_end - t_begin][d_out]  (scratch) */
  double *loss;           /* [t range] */
  double *rho;            /* [t range][K] */
  double *reward;         /* [t range][K] */
  double *g;              /* [t range][d_out] */
  double *G;              /* [d_out][d_in] */
  int n_threads;
} oracle_job;

typedef struct {
  oracle_job *job;
  int tid;
} worker_arg;

static int32_t noise_index(const oracle_job *j, int32_t i) {
  return j->antithetic ? i / 2 : i;
}
static double draw_sign(const oracle_job *j, int32_t i) {
  return (j->antithetic && (i % 2 == 1)) ? -1.0 : 1.0;
}

/* Step 1: y_t = W x_t, delta_t, L_t.  Tokens split across threads. */
static void *phase_forward(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t n_tok = j->t_end - j->t_begin;
  for (int64_t lt = wa->tid; lt < n_tok; lt += j->n_threads) {
    int64_t t = j->t_begin + lt;
    double loss = 0.0;
    for (int64_t c = 0; c < j->d_out; ++c) {
      double y = 0.0;
      for (int64_t k = 0; k < j->d_in; ++k)
        y += (double)j->W[c * j->d_in + k] * (double)j->X[t * j->d_in + k];
      double d = y - (double)j->target[t * j->d_out + c];
      j->delta[lt * j->d_out + c] = d;
      loss += 0.5 * d * d;
    }
    j->loss[lt] = loss;
  }
  return NULL;
}

/* Step 1 for an embedding: y_t = E[id_t] (row id_t of the table, held in
 * W as [V][d_out]), delta_t and L_t. */
static void *phase_gather(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t n_tok = j->t_end - j->t_begin;
  for (int64_t lt = wa->tid; lt < n_tok; lt += j->n_threads) {
    int64_t t = j->t_begin + lt;
    const float *row = j->W + (int64_t)j->ids[t] * j->d_out;
    double loss = 0.0;
    for (int64_t c = 0; c < j->d_out; ++c) {
      double d = (double)row[c] - (double)j->target[t * j->d_out + c];
      j->delta[lt * j->d_out + c] = d;
      loss += 0.5 * d * d;
    }
    j->loss[lt] = loss;
  }
  return NULL;
}

/* Step 2: literal perturbed losses and rho.  Each distinct noise vector is
 * generated once per token and used by every draw that shares it. */
static void *phase_rho(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t n_tok = j->t_end - j->t_begin;
  double *a = (double *)malloc(sizeof(double) * (size_t)j->d_out);
  for (int64_t lt = wa->tid; lt < n_tok; lt += j->n_threads) {
    int64_t t = j->t_begin + lt;
    const double *delta = j->delta + lt * j->d_out;
    int32_t last_n = -1;
    for (int32_t i = 0; i < j->K; ++i) {
      int32_t n = noise_index(j, i);
      if (n != last_n) {
        noise_vector(j->seed, (uint32_t)n, (uint32_t)t, j->d_out, a);
        last_n = n;
      }
      double s = draw_sign(j, i);
      double perturbed = 0.0;
      for (int64_t c = 0; c < j->d_out; ++c) {
        /* y + s sigma a - target = delta + s sigma a */
        double e = delta[c] + s * j->sigma * a[c];
        perturbed += 0.5 * e * e;
      }
      j->rho[lt * j->K + i] = j->loss[lt] - perturbed;
    }
  }
  free(a);
  return NULL;
}

/* Local scoring in place of steps 1-2: the jitter of draw i is the layer's
 * own output change Delta o = s_i sigma a, scored against the error
 * estimate e_t: rho_t^(i) = -<e_t, Delta o>. */
static void *phase_score(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t n_tok = j->t_end - j->t_begin;
  double *a = (double *)malloc(sizeof(double) * (size_t)j->d_out);
  for (int64_t lt = wa->tid; lt < n_tok; lt += j->n_threads) {
    int64_t t = j->t_begin + lt;
    const float *e = j->E + t * j->d_out;
    int32_t last_n = -1;
    for (int32_t i = 0; i < j->K; ++i) {
      int32_t n = noise_index(j, i);
      if (n != last_n) {
        noise_vector(j->seed, (uint32_t)n, (uint32_t)t, j->d_out, a);
        last_n = n;
      }
      double s = draw_sign(j, i);
      double score = 0.0;
      for (int64_t c = 0; c < j->d_out; ++c) {
        double delta_o = s * j->sigma * a[c];
        score -= (double)e[c] * delta_o;
      }
      j->rho[lt * j->K + i] = score;
    }
  }
  free(a);
  return NULL;
}

/* Steps 3 and 4: centring over draws, then the reverse discounted scan that
 * restarts at every sequence end.  Sequences split across threads. */
static void *phase_credit(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t seq0 = j->t_begin / j->seq_len, seq1 = j->t_end / j->seq_len;
  double *centred = (double *)malloc(sizeof(double) * (size_t)j->K);
  for (int64_t sq = seq0 + wa->tid; sq < seq1; sq += j->n_threads) {
    int64_t first = sq * j->seq_len, last = first + j->seq_len - 1;
    for (int64_t t = last; t >= first; --t) {
      int64_t lt = t - j->t_begin;
      double mean = 0.0;
      for (int32_t i = 0; i < j->K; ++i) mean += j->rho[lt * j->K + i];
      mean /= (double)j->K;
      for (int32_t i = 0; i < j->K; ++i)
        centred[i] = j->rho[lt * j->K + i] - mean;
      for (int32_t i = 0; i < j->K; ++i) {
        double later = (t == last) ? 0.0 : j->reward[(lt + 1) * j->K + i];
        j->reward[lt * j->K + i] = centred[i] + j->gamma * later;
      }
    }
  }
  free(centred);
  return NULL;
}

/* Step 5: g_t = -1/(K sigma) sum_i r_t^(i) s_i a_t^(n(i)). */
static void *phase_error(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t n_tok = j->t_end - j->t_begin;
  double *a = (double *)malloc(sizeof(double) * (size_t)j->d_out);
  double scale = -1.0 / ((double)j->K * j->sigma);
  for (int64_t lt = wa->tid; lt < n_tok; lt += j->n_threads) {
    int64_t t = j->t_begin + lt;
    double *g = j->g + lt * j->d_out;
    for (int64_t c = 0; c < j->d_out; ++c) g[c] = 0.0;
    int32_t last_n = -1;
    for (int32_t i = 0; i < j->K; ++i) {
      int32_t n = noise_index(j, i);
      if (n != last_n) {
        noise_vector(j->seed, (uint32_t)n, (uint32_t)t, j->d_out, a);
        last_n = n;
      }
      double coef = j->reward[lt * j->K + i] * draw_sign(j, i);
      for (int64_t c = 0; c < j->d_out; ++c) g[c] += coef * a[c];
    }
    for (int64_t c = 0; c < j->d_out; ++c) g[c] *= scale;
  }
  free(a);
  return NULL;
}

/* Step 6: G_W[c][k] = sum_t g_t[c] x_t[k], tokens summed in order.  Rows of
 * G split across threads. */
static void *phase_outer(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  int64_t n_tok = j->t_end - j->t_begin;
  for (int64_t c = wa->tid; c < j->d_out; c += j->n_threads) {
    double *row = j->G + c * j->d_in;
    for (int64_t k = 0; k < j->d_in; ++k) row[k] = 0.0;
    for (int64_t lt = 0; lt < n_tok; ++lt) {
      double gc = j->g[lt * j->d_out + c];
      const float *x = j->X + (j->t_begin + lt) * j->d_in;
      for (int64_t k = 0; k < j->d_in; ++k) row[k] += gc * (double)x[k];
    }
  }
  return NULL;
}

static void run_phase(oracle_job *j, void *(*fn)(void *)) {
  int nt = j->n_threads;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
  worker_arg *args = (worker_arg *)malloc(sizeof(worker_arg) * (size_t)nt);
  for (int i = 0; i < nt; ++i) {
    args[i].job = j;
    args[i].tid = i;
    pthread_create(&th[i], NULL, fn, &args[i]);
  }
  for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
  free(th);
  free(args);
}

/*
 * The whole estimator over the sequences seq_begin..seq_end-1 (all of them
 * when seq_end <= seq_begin is passed as 0,0 -> use every sequence).
 * Inputs are fp32 host arrays holding the exact values the GPU receives
 * (bf16 inputs are widened exactly); sigma and gamma are the fp32 values the
 * GPU receives, widened.  Outputs are fp64 host arrays sized for the token
 * range handled: loss[n_tok], rho[n_tok][K], reward[n_tok][K],
 * g[n_tok][d_out], G[d_out][d_in] (the contribution of that token range).
 * Returns 0, or -1 on an argument error.
 */
int dust_oracle_estimate(const float *X, const float *W, const float *target,
                         int64_t T, int64_t d_in, int64_t d_out,
                         int64_t seq_len, int32_t K, float sigma, float gamma,
                         uint64_t seed, int32_t antithetic, int64_t seq_begin,
                         int64_t seq_end, int32_t n_threads, double *G,
                         double *loss, double *rho, double *reward, double *g) {
  if (!X || !W || !target || !G || !loss || !rho || !reward || !g) return -1;
  if (T <= 0 || d_in <= 0 || d_out <= 0 || seq_len <= 0 || T % seq_len != 0)
    return -1;
  if (K < 2 || (antithetic && K % 2 != 0)) return -1;
  int64_t n_seq = T / seq_len;
  if (seq_end <= seq_begin) {
    seq_begin = 0;
    seq_end = n_seq;
  }
  if (seq_begin < 0 || seq_end > n_seq) return -1;
  if (n_threads < 1) n_threads = 1;

  oracle_job j;
  memset(&j, 0, sizeof(j));
  j.X = X;
  j.W = W;
  j.target = target;
  j.T = T;
  j.d_in = d_in;
  j.d_out = d_out;
  j.seq_len = seq_len;
  j.K = K;
  j.sigma = (double)sigma;
  j.gamma = (double)gamma;
  j.seed = seed;
  j.antithetic = antithetic;
  j.t_begin = seq_begin * seq_len;
  j.t_end = seq_end * seq_len;
  j.n_threads = n_threads;
  int64_t n_tok = j.t_end - j.t_begin;
  j.delta = (double *)malloc(sizeof(double) * (size_t)(n_tok * d_out));
  if (!j.delta) return -1;
  j.loss = loss;
  j.rho = rho;
  j.reward = reward;
  j.g = g;
  j.G = G;

  run_phase(&j, phase_forward);
  run_phase(&j, phase_rho);
  run_phase(&j, phase_credit);
  run_phase(&j, phase_error);
  run_phase(&j, phase_outer);
  free(j.delta);
  return 0;
}

/* The backprop gradient of the layer-local loss, sum_t delta_t x_t^T, and
 * delta itself ("Perturb the activations, not the weights": the weight
 * gradient of a linear layer is the outer product of output error and
 * input).  Used by the statistical pins (expectation and cosine laws). */
void dust_oracle_true_gradient(const float *X, const float *W,
                               const float *target, int64_t T, int64_t d_in,
                               int64_t d_out, double *delta, double *G_true) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < d_out; ++c) {
      double y = 0.0;
      for (int64_t k = 0; k < d_in; ++k)
        y += (double)W[c * d_in + k] * (double)X[t * d_in + k];
      delta[t * d_out + c] = y - (double)target[t * d_out + c];
    }
  for (int64_t c = 0; c < d_out; ++c)
    for (int64_t k = 0; k < d_in; ++k) {
      double s = 0.0;
      for (int64_t t = 0; t < T; ++t)
        s += delta[t * d_out + c] * (double)X[t * d_in + k];
      G_true[c * d_in + k] = s;
    }
}

/*
 * The estimator with local scoring over the sequences seq_begin..seq_end-1
 * (0, 0 for all): E [T][d_out] is the supplied error estimate of the layer's
 * output (fp32, as the GPU receives it); no forward and no loss.  Outputs as
 * for dust_oracle_estimate, with rho[n_tok][K] holding the scores.  Returns
 * 0, or -1 on an argument error.
 */
int dust_oracle_estimate_local(const float *X, const float *E, int64_t T,
                               int64_t d_in, int64_t d_out, int64_t seq_len,
                               int32_t K, float sigma, float gamma,
                               uint64_t seed, int32_t antithetic,
                               int64_t seq_begin, int64_t seq_end,
                               int32_t n_threads, double *G, double *rho,
                               double *reward, double *g) {
  if (!X || !E || !G || !rho || !reward || !g) return -1;
  if (T <= 0 || d_in <= 0 || d_out <= 0 || seq_len <= 0 || T % seq_len != 0)
    return -1;
  if (K < 2 || (antithetic && K % 2 != 0)) return -1;
  int64_t n_seq = T / seq_len;
  if (seq_end <= seq_begin) {
    seq_begin = 0;
    seq_end = n_seq;
  }
  if (seq_begin < 0 || seq_end > n_seq) return -1;
  if (n_threads < 1) n_threads = 1;

  oracle_job j;
  memset(&j, 0, sizeof(j));
  j.X = X;
  j.E = E;
  j.T = T;
  j.d_in = d_in;
  j.d_out = d_out;
  j.seq_len = seq_len;
  j.K = K;
  j.sigma = (double)sigma;
  j.gamma = (double)gamma;
  j.seed = seed;
  j.antithetic = antithetic;
  j.t_begin = seq_begin * seq_len;
  j.t_end = seq_end * seq_len;
  j.n_threads = n_threads;
  j.rho = rho;
  j.reward = reward;
  j.g = g;
  j.G = G;

  run_phase(&j, phase_score);
  run_phase(&j, phase_credit);
  run_phase(&j, phase_error);
  run_phase(&j, phase_outer);
  return 0;
}

/* Causal softmax attention of one head over one sequence of L tokens:
 * out_s = sum_{t <= s} w_st v_t, w_st = exp(l_st - max) / sum, l_st =
 * <q_s, k_t> / sqrt(dh).  q, k, v, out are [L][dh]; w is scratch [L]. */
static void attend(const double *q, const double *k, const double *v, int64_t L,
                   int64_t dh, double *w, double *out) {
  const double scale = 1.0 / sqrt((double)dh);
  for (int64_t s = 0; s < L; ++s) {
    double m = -INFINITY;
    for (int64_t t = 0; t <= s; ++t) {
      double l = 0.0;
      for (int64_t c = 0; c < dh; ++c) l += q[s * dh + c] * k[t * dh + c];
      w[t] = l * scale;
      if (w[t] > m) m = w[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t <= s; ++t) {
      w[t] = exp(w[t] - m);
      z += w[t];
    }
    for (int64_t c = 0; c < dh; ++c) out[s * dh + c] = 0.0;
    for (int64_t t = 0; t <= s; ++t)
      for (int64_t c = 0; c < dh; ++c) out[s * dh + c] += (w[t] / z) * v[t * dh + c];
  }
}

/* Scores through a recomputed attention, in place of steps 1-2: for every
 * sequence, head and draw, the jittered site's attention is recomputed and
 * its output change scored against the error estimate.  Sequences split
 * across threads. */
static void *phase_attn_score(void *p) {
  worker_arg *wa = (worker_arg *)p;
  oracle_job *j = wa->job;
  const int64_t L = j->seq_len, H = j->heads, dh = j->d_head, D = H * dh;
  const int64_t seq0 = j->t_begin / L, seq1 = j->t_end / L;
  double *A = (double *)malloc(sizeof(double) * (size_t)(L * D));
  double *act[3], *jit[3];
  for (int u = 0; u < 3; ++u) {
    act[u] = (double *)malloc(sizeof(double) * (size_t)(H * L * dh));
    jit[u] = (double *)malloc(sizeof(double) * (size_t)(L * dh));
  }
  double *clean = (double *)malloc(sizeof(double) * (size_t)(H * L * dh));
  double *o2 = (double *)malloc(sizeof(double) * (size_t)(L * dh));
  double *w = (double *)malloc(sizeof(double) * (size_t)L);
  const float *src[3] = {j->Qa, j->Ka, j->Va};
  for (int64_t sq = seq0 + wa->tid; sq < seq1; sq += j->n_threads) {
    const int64_t first = sq * L;
    /* the cached activations of this sequence, per head, and the clean
       outputs */
    for (int u = 0; u < 3; ++u)
      for (int64_t h = 0; h < H; ++h)
        for (int64_t t = 0; t < L; ++t)
          for (int64_t c = 0; c < dh; ++c)
            act[u][(h * L + t) * dh + c] = (double)src[u][(first + t) * D + h * dh + c];
    for (int64_t h = 0; h < H; ++h)
      attend(act[0] + h * L * dh, act[1] + h * L * dh, act[2] + h * L * dh, L, dh, w,
             clean + h * L * dh);
    for (int64_t t = 0; t < L; ++t)
      for (int32_t i = 0; i < j->K; ++i) j->rho[(first + t - j->t_begin) * j->K + i] = 0.0;
    int32_t last_n = -1;
    for (int32_t i = 0; i < j->K; ++i) {
      const int32_t n = noise_index(j, i);
      if (n != last_n) {
        for (int64_t t = 0; t < L; ++t)
          noise_vector(j->seed, (uint32_t)n, (uint32_t)(first + t), D, A + t * D);
        last_n = n;
      }
      const double amp = draw_sign(j, i) * j->sigma;
      for (int64_t h = 0; h < H; ++h) {
        const double *in[3];
        for (int u = 0; u < 3; ++u) in[u] = act[u] + h * L * dh;
        /* the jittered site of this head */
        double *site = jit[j->site];
        for (int64_t t = 0; t < L; ++t)
          for (int64_t c = 0; c < dh; ++c)
            site[t * dh + c] = in[j->site][t * dh + c] + amp * A[t * D + h * dh + c];
        in[j->site] = site;
        attend(in[0], in[1], in[2], L, dh, w, o2);
        const double *oc = clean + h * L * dh;
        for (int64_t s = 0; s < L; ++s) {
          double score = 0.0;
          for (int64_t c = 0; c < dh; ++c)
            score -= (double)j->E[(first + s) * D + h * dh + c] *
                     (o2[s * dh + c] - oc[s * dh + c]);
          j->rho[(first + s - j->t_begin) * j->K + i] += score;
        }
      }
    }
  }
  free(A);
  for (int u = 0; u < 3; ++u) {
    free(act[u]);
    free(jit[u]);
  }
  free(clean);
  free(o2);
  free(w);
  return NULL;
}

/*
 * The estimator with scores through a recomputed attention over the
 * sequences seq_begin..seq_end-1 (0, 0 for all).  Qa, Ka, Va [T][heads
 * d_head] are the cached queries, keys and values of one block (fp32, as the
 * GPU receives them); site 0, 1 or 2 jitters the queries, keys or values;
 * E [T][heads d_head] is the supplied error estimate of the attention
 * output.  X [T][d_in] (the block's input) gives the site's weight gradient
 * G [heads d_head][d_in]; with X NULL, G is left untouched.  Outputs as for
 * dust_oracle_estimate_local.  Returns 0, or -1 on an argument error.
 */
int dust_oracle_estimate_attention(const float *X, const float *Qa, const float *Ka,
                                   const float *Va, const float *E, int64_t T,
                                   int64_t d_in, int64_t heads, int64_t d_head,
                                   int64_t seq_len, int32_t site, int32_t K,
                                   float sigma, float gamma, uint64_t seed,
                                   int32_t antithetic, int64_t seq_begin,
                                   int64_t seq_end, int32_t n_threads, double *G,
                                   double *rho, double *reward, double *g) {
  if (!Qa || !Ka || !Va || !E || !rho || !reward || !g || (X && !G)) return -1;
  if (T <= 0 || heads <= 0 || d_head <= 0 || seq_len <= 0 || T % seq_len != 0)
    return -1;
  if (X && d_in <= 0) return -1;
  if (site < 0 || site > 2) return -1;
  if (K < 2 || (antithetic && K % 2 != 0)) return -1;
  int64_t n_seq = T / seq_len;
  if (seq_end <= seq_begin) {
    seq_begin = 0;
    seq_end = n_seq;
  }
  if (seq_begin < 0 || seq_end > n_seq) return -1;
  if (n_threads < 1) n_threads = 1;

  oracle_job j;
  memset(&j, 0, sizeof(j));
  j.X = X;
  j.Qa = Qa;
  j.Ka = Ka;
  j.Va = Va;
  j.E = E;
  j.T = T;
  j.d_in = d_in;
  j.d_out = heads * d_head;
  j.heads = heads;
  j.d_head = d_head;
  j.site = site;
  j.seq_len = seq_len;
  j.K = K;
  j.sigma = (double)sigma;
  j.gamma = (double)gamma;
  j.seed = seed;
  j.antithetic = antithetic;
  j.t_begin = seq_begin * seq_len;
  j.t_end = seq_end * seq_len;
  j.n_threads = n_threads;
  j.rho = rho;
  j.reward = reward;
  j.g = g;
  j.G = G;

  run_phase(&j, phase_attn_score);
  run_phase(&j, phase_credit);
  run_phase(&j, phase_error);
  if (X) run_phase(&j, phase_outer);
  return 0;
}

/*
 * The embedding's weight gradient from per-token errors: G_E[v][c] =
 * scale sum_{t: ids[t] = v} g[t][c], the tokens added in order, every row
 * written (zero for ids that do not occur).  g [T][d] fp64, G_E [V][d] fp64.
 * Returns 0, or -1 on an argument error (an id outside [0, V) included).
 */
int dust_oracle_reassemble_embedding(const int32_t *ids, const double *g, int64_t T,
                                     int64_t V, int64_t d, double scale, double *G_E) {
  if (!ids || !g || !G_E || T < 0 || V <= 0 || d <= 0) return -1;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return -1;
  for (int64_t i = 0; i < V * d; ++i) G_E[i] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    double *row = G_E + (int64_t)ids[t] * d;
    for (int64_t c = 0; c < d; ++c) row[c] += g[t * d + c];
  }
  for (int64_t i = 0; i < V * d; ++i) G_E[i] *= scale;
  return 0;
}

/*
 * The estimator for a token embedding over the sequences
 * seq_begin..seq_end-1 (0, 0 for all): table [V][d] and target [T][d] (fp32
 * holding the exact input values), ids [T] in [0, V).  Outputs for the
 * handled tokens as for dust_oracle_estimate (loss, rho, reward, g with
 * d_out = d), and G_E [V][d] = scale x (their scatter-added g).  Returns 0,
 * or -1 on an argument error.
 */
int dust_oracle_estimate_embedding(const float *table, const int32_t *ids,
                                   const float *target, int64_t T, int64_t V, int64_t d,
                                   int64_t seq_len, int32_t K, float sigma, float gamma,
                                   uint64_t seed, int32_t antithetic, double scale,
                                   int64_t seq_begin, int64_t seq_end, int32_t n_threads,
                                   double *G_E, double *loss, double *rho, double *reward,
                                   double *g) {
  if (!table || !ids || !target || !G_E || !loss || !rho || !reward || !g) return -1;
  if (T <= 0 || V <= 0 || d <= 0 || seq_len <= 0 || T % seq_len != 0) return -1;
  if (K < 2 || (antithetic && K % 2 != 0)) return -1;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return -1;
  int64_t n_seq = T / seq_len;
  if (seq_end <= seq_begin) {
    seq_begin = 0;
    seq_end = n_seq;
  }
  if (seq_begin < 0 || seq_end > n_seq) return -1;
  if (n_threads < 1) n_threads = 1;

  oracle_job j;
  memset(&j, 0, sizeof(j));
  j.W = table;
  j.ids = ids;
  j.target = target;
  j.T = T;
  j.d_out = d;
  j.seq_len = seq_len;
  j.K = K;
  j.sigma = (double)sigma;
  j.gamma = (double)gamma;
  j.seed = seed;
  j.antithetic = antithetic;
  j.t_begin = seq_begin * seq_len;
  j.t_end = seq_end * seq_len;
  j.n_threads = n_threads;
  int64_t n_tok = j.t_end - j.t_begin;
  j.delta = (double *)malloc(sizeof(double) * (size_t)(n_tok * d));
  if (!j.delta) return -1;
  j.loss = loss;
  j.rho = rho;
  j.reward = reward;
  j.g = g;

  run_phase(&j, phase_gather);
  run_phase(&j, phase_rho);
  run_phase(&j, phase_credit);
  run_phase(&j, phase_error);
  free(j.delta);
  return dust_oracle_reassemble_embedding(ids + j.t_begin, g, n_tok, V, d, scale, G_E);
}

/* ------------------------------------------------------------------------ */
/* Cross-entropy head. */

typedef struct {
  const float *X, *W;
  const int32_t *labels;
  int64_t T, d_in, V, slab;
  int32_t K;
  double sigma;
  uint64_t seed;
  int32_t antithetic;
  int64_t t_begin, t_end;
  double *loss, *rho, *g; /* [n_tok], [n_tok][n_slab][K], [n_tok][V] */
  double *G;              /* [V][d_in] */
  int n_threads;
} head_job;

typedef struct {
  head_job *job;
  int tid;
} head_arg;

/* log sum_c exp(z_c), with the maximum taken out first. */
static double log_sum_exp(const double *z, int64_t n) {
  double m = z[0];
  for (int64_t c = 1; c < n; ++c)
    if (z[c] > m) m = z[c];
  double s = 0.0;
  for (int64_t c = 0; c < n; ++c) s += exp(z[c] - m);
  return m + log(s);
}

/* Per token: logits, the clean cross-entropy, then for every slab and draw
 * the literal perturbed cross-entropy, the centring over the slab's draws
 * and the slab's columns of g. */
static void *head_token(void *p) {
  head_arg *ha = (head_arg *)p;
  head_job *j = ha->job;
  int64_t n_tok = j->t_end - j->t_begin, n_slab = j->V / j->slab;
  double *z = (double *)malloc(sizeof(double) * (size_t)j->V);
  double *zp = (double *)malloc(sizeof(double) * (size_t)j->V);
  double *a = (double *)malloc(sizeof(double) * (size_t)j->V);
  double *rho = (double *)malloc(sizeof(double) * (size_t)j->K);
  double scale = -1.0 / ((double)j->K * j->sigma);
  for (int64_t lt = ha->tid; lt < n_tok; lt += j->n_threads) {
    int64_t t = j->t_begin + lt;
    for (int64_t c = 0; c < j->V; ++c) {
      double y = 0.0;
      for (int64_t k = 0; k < j->d_in; ++k)
        y += (double)j->W[c * j->d_in + k] * (double)j->X[t * j->d_in + k];
      z[c] = y;
    }
    int32_t label = j->labels[t];
    double ce = log_sum_exp(z, j->V) - z[label];
    j->loss[lt] = ce;
    double *g = j->g + lt * j->V;
    for (int64_t c = 0; c < j->V; ++c) g[c] = 0.0;
    for (int64_t sl = 0; sl < n_slab; ++sl) {
      int64_t c0 = sl * j->slab, c1 = c0 + j->slab;
      double mean = 0.0;
      int32_t last_n = -1;
      for (int32_t i = 0; i < j->K; ++i) {
        int32_t n = j->antithetic ? i / 2 : i;
        double s = (j->antithetic && (i % 2 == 1)) ? -1.0 : 1.0;
        if (n != last_n) {
          noise_vector(j->seed, (uint32_t)n, (uint32_t)t, j->V, a);
          last_n = n;
        }
        memcpy(zp, z, sizeof(double) * (size_t)j->V);
        for (int64_t c = c0; c < c1; ++c) zp[c] += s * j->sigma * a[c];
        double ce_p = log_sum_exp(zp, j->V) - zp[label];
        rho[i] = ce - ce_p;
        mean += rho[i];
      }
      mean /= (double)j->K;
      double *rho_out = j->rho + (lt * n_slab + sl) * j->K;
      last_n = -1;
      for (int32_t i = 0; i < j->K; ++i) {
        int32_t n = j->antithetic ? i / 2 : i;
        double s = (j->antithetic && (i % 2 == 1)) ? -1.0 : 1.0;
        if (n != last_n) {
          noise_vector(j->seed, (uint32_t)n, (uint32_t)t, j->V, a);
          last_n = n;
        }
        rho_out[i] = rho[i];
        double coef = (rho[i] - mean) * s;
        for (int64_t c = c0; c < c1; ++c) g[c] += coef * a[c];
      }
      for (int64_t c = c0; c < c1; ++c) g[c] *= scale;
    }
  }
  free(z);
  free(zp);
  free(a);
  free(rho);
  return NULL;
}

/* G_W[c][k] = sum_t g_t[c] x_t[k] over the handled tokens, in token order. */
static void *head_outer(void *p) {
  head_arg *ha = (head_arg *)p;
  head_job *j = ha->job;
  int64_t n_tok = j->t_end - j->t_begin;
  for (int64_t c = ha->tid; c < j->V; c += j->n_threads) {
    double *row = j->G + c * j->d_in;
    for (int64_t k = 0; k < j->d_in; ++k) row[k] = 0.0;
    for (int64_t lt = 0; lt < n_tok; ++lt) {
      double gc = j->g[lt * j->V + c];
      const float *x = j->X + (j->t_begin + lt) * j->d_in;
      for (int64_t k = 0; k < j->d_in; ++k) row[k] += gc * (double)x[k];
    }
  }
  return NULL;
}

static void run_head_phase(head_job *j, void *(*fn)(void *)) {
  int nt = j->n_threads;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
  head_arg *args = (head_arg *)malloc(sizeof(head_arg) * (size_t)nt);
  for (int i = 0; i < nt; ++i) {
    args[i].job = j;
    args[i].tid = i;
    pthread_create(&th[i], NULL, fn, &args[i]);
  }
  for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
  free(th);
  free(args);
}

/*
 * The cross-entropy head estimator over tokens t_begin..t_end-1 (0, 0 for
 * all): X [T][d_in], W [V][d_in] (fp32 holding the exact input values),
 * labels [T] in [0, V); V a multiple of slab.  Outputs for the handled
 * tokens: loss[n] (clean cross-entropy), rho[n][V/slab][K] (loss reductions
 * per slab and draw), g[n][V], and G[V][d_in] (their contribution).
 * Returns 0, or -1 on an argument error.
 */
int dust_oracle_estimate_head(const float *X, const float *W, const int32_t *labels,
                              int64_t T, int64_t d_in, int64_t V, int64_t slab,
                              int32_t K, float sigma, uint64_t seed, int32_t antithetic,
                              int64_t t_begin, int64_t t_end, int32_t n_threads,
                              double *G, double *loss, double *rho, double *g) {
  if (!X || !W || !labels || !G || !loss || !rho || !g) return -1;
  if (T <= 0 || d_in <= 0 || V <= 0 || slab <= 0 || V % slab != 0) return -1;
  if (K < 2 || (antithetic && K % 2 != 0)) return -1;
  if (t_end <= t_begin) {
    t_begin = 0;
    t_end = T;
  }
  if (t_begin < 0 || t_end > T) return -1;
  for (int64_t t = t_begin; t < t_end; ++t)
    if (labels[t] < 0 || labels[t] >= V) return -1;
  if (n_threads < 1) n_threads = 1;
  head_job j;
  memset(&j, 0, sizeof(j));
  j.X = X;
  j.W = W;
  j.labels = labels;
  j.T = T;
  j.d_in = d_in;
  j.V = V;
  j.slab = slab;
  j.K = K;
  j.sigma = (double)sigma;
  j.seed = seed;
  j.antithetic = antithetic;
  j.t_begin = t_begin;
  j.t_end = t_end;
  j.loss = loss;
  j.rho = rho;
  j.g = g;
  j.G = G;
  j.n_threads = n_threads;
  run_head_phase(&j, head_token);
  run_head_phase(&j, head_outer);
  return 0;
}

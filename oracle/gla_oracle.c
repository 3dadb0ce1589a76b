/*
 * gla_oracle.c -- fp64 CPU oracle for the gated linear attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never links, loads or calls it, and it shares no source with that path.
 *
 * Sources (web pages; cited by title and section):
 *   [LCT] "Engineering Long-Context Training for Trillion-Parameter MoE Models:
 *          Three Key Breakthroughs"
 *   [STM] "Scaling Trillion-Parameter MoE and Long-Context LLMs: Architecture
 *          and Engineering in Practice"
 *   [ESU] "Engineering Stability in Ultra-Long Context and Trillion-Parameter
 *          Sparse Models"
 *
 * What it computes.  [LCT §3.1] and [ESU §2.1] describe linear attention whose
 * state is carried from token to token and multiplied by a per-position decay;
 * the cumulative product of those decays is the factor Gamma.  The pages never
 * write the recurrence out; the plainest reading, which this file implements
 * literally, one token at a time, is
 *
 *     S_{-1} = S0                       (dk x dv; zero when S0 is absent)
 *     S_t    = a_t * S_{t-1} + k_t v_t^T
 *     o_t    = S_t^T q_t                (token t sees its own key/value)
 *     S_T    = S_{T-1}
 *
 * with a_t = exp(g_t) and the log-decay g_t taken from the gate of [LCT §3.2]:
 *     bounded gate:        g = -5 * sigmoid(x)        range (-5, 0)
 *     negative softplus:   g = -softplus(-x) = log(sigmoid(x))  range (-inf, 0)
 * (the second is the unbounded conventional form kept for the ablation; its
 * sign follows the strong-decay reading, so that x ~ N(-4,1) decays strongly).
 *
 * There is no chunking, blocking, tiling or reordering here: the chunked
 * method of [LCT §3.1] reaches the same result up to rounding order.
 *
 * Inputs are read after their storage rounding: q, k, v are bf16 bit patterns
 * (qkv_is_bf16 = 1) or fp32 values; x is fp32; S0 is given in double (an fp32
 * initial state widens exactly; a double one lets states be chained without
 * rounding).  Every value is widened to double before any arithmetic, and all
 * arithmetic is double.
 *
 * The backward pass (gla_oracle_backward) is the reverse-mode chain rule of the
 * same recurrence, also one token at a time; see its comment.
 *
 * Layouts (row-major, contiguous; BH = batch * heads, heads independent):
 *   q, k [BH][T][dk]   v [BH][T][dv]   x [BH][T]   S0 [BH][dk][dv] or NULL
 *   o    [BH][T][dv]   S_T [BH][dk][dv]             (outputs, double)
 * Work is split over (head, block of `col_block` value columns) with OpenMP:
 * the columns of S evolve independently, so the split does not change any
 * arithmetic, only which thread performs it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Planted-mistake builds: the test suite compiles this file with
 * -DGLA_ORACLE_MUTANT=n to check that its pins catch each mistake.  The normal
 * build defines nothing and takes none of these branches. */
#ifndef GLA_ORACLE_MUTANT
#define GLA_ORACLE_MUTANT 0
#endif

enum { ORACLE_GATE_BOUNDED_SIGMOID = 0, ORACLE_GATE_NEG_SOFTPLUS = 1 };

static double widen(const void* p, int is_bf16, size_t idx) {
  if (is_bf16) {
    /* a bf16 value is the upper half of the fp32 with the same bits */
    uint32_t u = (uint32_t)((const uint16_t*)p)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)p)[idx];
}

/* sigmoid(x) = 1 / (1 + e^-x), evaluated so that no intermediate overflows */
static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/* softplus(z) = log(1 + e^z) = max(z, 0) + log1p(e^-|z|) */
static double softplus(double z) {
  return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
}

/* log-decay g(x) [LCT §3.2]: bounded g = g_min * sigmoid(x) with g_min = -5,
 * or the conventional unbounded negative softplus. */
double gla_oracle_gate(double x, int gate) {
#if GLA_ORACLE_MUTANT == 4
  x = -x; /* planted: gate argument sign flipped */
#endif
  if (gate == ORACLE_GATE_NEG_SOFTPLUS) return -softplus(-x);
  return -5.0 * sigmoid(x);
}

/* Returns 0 on success, 1 on a bad argument. */
int gla_oracle_forward(const void* q, const void* k, const void* v, int qkv_is_bf16,
                       const float* x, const double* S0, double* o, double* S_T,
                       long long BH, long long T, int dk, int dv, int gate,
                       int col_block, int nthreads) {
  if (!q || !k || !v || !x || !o || !S_T) return 1;
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
  if (gate != ORACLE_GATE_BOUNDED_SIGMOID && gate != ORACLE_GATE_NEG_SOFTPLUS) return 1;
  if (col_block <= 0 || col_block > dv) col_block = dv;
  const long long ncb = (dv + col_block - 1) / col_block;
  const long long tasks = BH * ncb;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (long long task = 0; task < tasks; ++task) {
    const long long bh = task / ncb;
    const int n0 = (int)(task % ncb) * col_block;
    const int nc = (n0 + col_block <= dv) ? col_block : dv - n0;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)nc);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* vt = (double*)malloc(sizeof(double) * (size_t)nc);

    for (int d = 0; d < dk; ++d)
      for (int n = 0; n < nc; ++n)
        S[(size_t)d * nc + n] = S0 ? S0[((size_t)bh * dk + d) * dv + n0 + n] : 0.0;

    for (long long t = 0; t < T; ++t) {
      const size_t row = (size_t)bh * (size_t)T + (size_t)t;
#if GLA_ORACLE_MUTANT == 5
      /* planted: decay index shifted by one token (a_0 = 1, a_t from x[t-1]) */
      const double a = t == 0 ? 1.0 : exp(gla_oracle_gate((double)x[row - 1], gate));
#elif GLA_ORACLE_MUTANT == 6
      /* planted: the initial state is not decayed at the first token */
      const double a = t == 0 ? 1.0 : exp(gla_oracle_gate((double)x[row], gate));
#else
      const double a = exp(gla_oracle_gate((double)x[row], gate));
#endif
      for (int d = 0; d < dk; ++d) {
#if GLA_ORACLE_MUTANT == 3
        /* planted: query and key roles swapped */
        qt[d] = widen(k, qkv_is_bf16, row * (size_t)dk + d);
        kt[d] = widen(q, qkv_is_bf16, row * (size_t)dk + d);
#else
        kt[d] = widen(k, qkv_is_bf16, row * (size_t)dk + d);
        qt[d] = widen(q, qkv_is_bf16, row * (size_t)dk + d);
#endif
      }
      for (int n = 0; n < nc; ++n) vt[n] = widen(v, qkv_is_bf16, row * (size_t)dv + n0 + n);

#if GLA_ORACLE_MUTANT == 1
      /* planted: output read before this token's update (drops token t) */
      for (int n = 0; n < nc; ++n) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += S[(size_t)d * nc + n] * qt[d];
        o[row * (size_t)dv + n0 + n] = acc;
      }
#endif
      /* S_t = a_t S_{t-1} + k_t v_t^T */
      for (int d = 0; d < dk; ++d)
        for (int n = 0; n < nc; ++n) {
#if GLA_ORACLE_MUTANT == 2
          /* planted: decay also applied to the new outer product */
          S[(size_t)d * nc + n] = a * (S[(size_t)d * nc + n] + kt[d] * vt[n]);
#else
          S[(size_t)d * nc + n] = a * S[(size_t)d * nc + n] + kt[d] * vt[n];
#endif
        }
#if GLA_ORACLE_MUTANT != 1
      /* o_t = S_t^T q_t */
      for (int n = 0; n < nc; ++n) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += S[(size_t)d * nc + n] * qt[d];
        o[row * (size_t)dv + n0 + n] = acc;
      }
#endif
    }
    for (int d = 0; d < dk; ++d)
      for (int n = 0; n < nc; ++n)
        S_T[((size_t)bh * dk + d) * dv + n0 + n] = S[(size_t)d * nc + n];
    free(S);
    free(kt);
    free(qt);
    free(vt);
  }
  return 0;
}

/* Per-channel decay.  [LCT §3.1] speaks of a per-position cumulative decay
 * without saying whether it is one scalar per position or one value per key
 * channel; the second reading, in which each row d of the state has its own
 * decay, is the gated-linear-attention form the scalar one specialises:
 *
 *     S_t[d][n] = a_t[d] * S_{t-1}[d][n] + k_t[d] v_t[n],   a_t[d] = exp(g(x_t[d]))
 *     o_t       = S_t^T q_t
 *
 * with x of layout [BH][T][dk] and the same gates.  When every channel has the
 * same x it is exactly the scalar recurrence above.  One token at a time, same
 * threading as gla_oracle_forward. */
int gla_oracle_forward_pc(const void* q, const void* k, const void* v, int qkv_is_bf16,
                          const float* x, const double* S0, double* o, double* S_T,
                          long long BH, long long T, int dk, int dv, int gate,
                          int col_block, int nthreads) {
  if (!q || !k || !v || !x || !o || !S_T) return 1;
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
  if (gate != ORACLE_GATE_BOUNDED_SIGMOID && gate != ORACLE_GATE_NEG_SOFTPLUS) return 1;
  if (col_block <= 0 || col_block > dv) col_block = dv;
  const long long ncb = (dv + col_block - 1) / col_block;
  const long long tasks = BH * ncb;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (long long task = 0; task < tasks; ++task) {
    const long long bh = task / ncb;
    const int n0 = (int)(task % ncb) * col_block;
    const int nc = (n0 + col_block <= dv) ? col_block : dv - n0;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)nc);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* at = (double*)malloc(sizeof(double) * (size_t)dk);
    double* vt = (double*)malloc(sizeof(double) * (size_t)nc);

    for (int d = 0; d < dk; ++d)
      for (int n = 0; n < nc; ++n)
        S[(size_t)d * nc + n] = S0 ? S0[((size_t)bh * dk + d) * dv + n0 + n] : 0.0;

    for (long long t = 0; t < T; ++t) {
      const size_t row = (size_t)bh * (size_t)T + (size_t)t;
      for (int d = 0; d < dk; ++d) {
        kt[d] = widen(k, qkv_is_bf16, row * (size_t)dk + d);
        qt[d] = widen(q, qkv_is_bf16, row * (size_t)dk + d);
#if GLA_ORACLE_MUTANT == 12
        /* planted: every channel takes channel 0's decay */
        at[d] = exp(gla_oracle_gate((double)x[row * (size_t)dk], gate));
#elif GLA_ORACLE_MUTANT == 13
        /* planted: decay index shifted by one token */
        at[d] = t == 0 ? 1.0 : exp(gla_oracle_gate((double)x[(row - 1) * (size_t)dk + d], gate));
#else
        at[d] = exp(gla_oracle_gate((double)x[row * (size_t)dk + d], gate));
#endif
      }
      for (int n = 0; n < nc; ++n) vt[n] = widen(v, qkv_is_bf16, row * (size_t)dv + n0 + n);

      /* S_t = diag(a_t) S_{t-1} + k_t v_t^T */
      for (int d = 0; d < dk; ++d)
        for (int n = 0; n < nc; ++n) {
#if GLA_ORACLE_MUTANT == 11
          /* planted: decay taken by value column instead of key row */
          const double a = at[(n0 + n) % dk];
#else
          const double a = at[d];
#endif
          S[(size_t)d * nc + n] = a * S[(size_t)d * nc + n] + kt[d] * vt[n];
        }
      /* o_t = S_t^T q_t */
      for (int n = 0; n < nc; ++n) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += S[(size_t)d * nc + n] * qt[d];
        o[row * (size_t)dv + n0 + n] = acc;
      }
    }
    for (int d = 0; d < dk; ++d)
      for (int n = 0; n < nc; ++n)
        S_T[((size_t)bh * dk + d) * dv + n0 + n] = S[(size_t)d * nc + n];
    free(S);
    free(kt);
    free(qt);
    free(at);
    free(vt);
  }
  return 0;
}

/* Gated delta rule.  [LCT §3.1] and [§3.3] name Delta-Net-style structures as the
 * other family whose chunked form has the same diagonal-tile problem; the pages do
 * not write their recurrence.  The plainest reading, the gated delta rule with the
 * same decay gate, is
 *
 *     S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t
 *
 * with a_t = exp(g(x_t)) one scalar per token and beta_t in [0, 1] a given per-token
 * write strength (fp32 [BH][T]).  One token at a time, in the order written: the
 * projection k_t^T S_{t-1}, the decayed erase-and-write, then the read-out. */
int gla_oracle_forward_delta(const void* q, const void* k, const void* v, int qkv_is_bf16,
                             const float* x, const float* beta, const double* S0, double* o, double* S_T,
                             long long BH, long long T, int dk, int dv, int gate, int col_block,
                             int nthreads) {
  if (!q || !k || !v || !x || !beta || !o || !S_T) return 1;
  if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
  if (gate != ORACLE_GATE_BOUNDED_SIGMOID && gate != ORACLE_GATE_NEG_SOFTPLUS) return 1;
  if (col_block <= 0 || col_block > dv) col_block = dv;
  const long long ncb = (dv + col_block - 1) / col_block;
  const long long tasks = BH * ncb;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (long long task = 0; task < tasks; ++task) {
    const long long bh = task / ncb;
    const int n0 = (int)(task % ncb) * col_block;
    const int nc = (n0 + col_block <= dv) ? col_block : dv - n0;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)nc);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* vt = (double*)malloc(sizeof(double) * (size_t)nc);
    double* proj = (double*)malloc(sizeof(double) * (size_t)nc);

    for (int d = 0; d < dk; ++d)
      for (int n = 0; n < nc; ++n)
        S[(size_t)d * nc + n] = S0 ? S0[((size_t)bh * dk + d) * dv + n0 + n] : 0.0;

    for (long long t = 0; t < T; ++t) {
      const size_t row = (size_t)bh * (size_t)T + (size_t)t;
      const double a = exp(gla_oracle_gate((double)x[row], gate));
      const double bt = (double)beta[row];
      for (int d = 0; d < dk; ++d) {
        kt[d] = widen(k, qkv_is_bf16, row * (size_t)dk + d);
        qt[d] = widen(q, qkv_is_bf16, row * (size_t)dk + d);
      }
      for (int n = 0; n < nc; ++n) vt[n] = widen(v, qkv_is_bf16, row * (size_t)dv + n0 + n);
      /* proj = S_{t-1}^T k_t  (what the state currently returns for key k_t) */
      for (int n = 0; n < nc; ++n) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += S[(size_t)d * nc + n] * kt[d];
        proj[n] = acc;
      }
      /* S_t = a (S - beta k proj^T) + beta k v^T */
      for (int d = 0; d < dk; ++d)
        for (int n = 0; n < nc; ++n) {
#if GLA_ORACLE_MUTANT == 14
          /* planted: the erase term is not decayed */
          S[(size_t)d * nc + n] = a * S[(size_t)d * nc + n] - bt * kt[d] * proj[n] + bt * kt[d] * vt[n];
#elif GLA_ORACLE_MUTANT == 15
          /* planted: the write is not scaled by beta */
          S[(size_t)d * nc + n] = a * (S[(size_t)d * nc + n] - bt * kt[d] * proj[n]) + kt[d] * vt[n];
#else
          S[(size_t)d * nc + n] = a * (S[(size_t)d * nc + n] - bt * kt[d] * proj[n]) + bt * kt[d] * vt[n];
#endif
        }
      for (int n = 0; n < nc; ++n) {
        double acc = 0.0;
        for (int d = 0; d < dk; ++d) acc += S[(size_t)d * nc + n] * qt[d];
        o[row * (size_t)dv + n0 + n] = acc;
      }
    }
    for (int d = 0; d < dk; ++d)
      for (int n = 0; n < nc; ++n)
        S_T[((size_t)bh * dk + d) * dv + n0 + n] = S[(size_t)d * nc + n];
    free(S);
    free(kt);
    free(qt);
    free(vt);
    free(proj);
  }
  return 0;
}

/* d g / d x of the gate: bounded -5 sigmoid(x) (1 - sigmoid(x)); negative
 * softplus -softplus(-x) has derivative sigmoid(-x). */
static double gate_slope(double x, int gate) {
  if (gate == ORACLE_GATE_NEG_SOFTPLUS) return sigmoid(-x);
  const double s = sigmoid(x);
  return -5.0 * s * (1.0 - s);
}

/* Backward pass of the recurrence, by the reverse-mode chain rule one token at a
 * time.  Given dO = dL/do [BH][T][dv] and dS_T = dL/dS_T [BH][dk][dv] (NULL: zero),
 * with D_t = dL/dS_t through o_t and every later state,
 *
 *     D_{T-1} = q_{T-1} dO_{T-1}^T + dS_T
 *     D_t     = q_t dO_t^T + a_{t+1} D_{t+1}
 *     dq_t = S_t dO_t        dk_t = D_t v_t        dv_t = D_t^T k_t
 *     dL/da_t = <D_t, S_{t-1}>  (Frobenius),  dx_t = dL/da_t * a_t * g'(x_t)
 *     dS0 = a_0 D_0
 *
 * S_t is needed in reverse order; it is recomputed forward inside blocks of 64
 * tokens from checkpoints of S taken on a first forward sweep (the recurrence is
 * never run backwards).  Outputs are double: dq, dk [BH][T][dk], dv [BH][T][dv],
 * dx [BH][T], dS0 [BH][dk][dv].  Heads run in parallel (OpenMP).
 * Returns 0 on success, 1 on a bad argument, 2 when memory runs out. */
int gla_oracle_backward(const void* q, const void* k, const void* v, int qkv_is_bf16,
                        const float* x, const double* S0, const double* dO, const double* dST,
                        double* dq, double* dk, double* dv, double* dx, double* dS0,
                        long long BH, long long T, int dkd, int dvd, int gate, int nthreads) {
  if (!q || !k || !v || !x || !dO || !dq || !dk || !dv || !dx || !dS0) return 1;
  if (BH < 0 || T < 0 || dkd <= 0 || dvd <= 0) return 1;
  if (gate != ORACLE_GATE_BOUNDED_SIGMOID && gate != ORACLE_GATE_NEG_SOFTPLUS) return 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const long long B = 64;  /* tokens per recompute block */
  const long long nblk = (T + B - 1) / B;
  const size_t SZ = (size_t)dkd * (size_t)dvd;
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (long long bh = 0; bh < BH; ++bh) {
    double* ck = (double*)malloc(sizeof(double) * SZ * (size_t)(nblk > 0 ? nblk : 1)); /* S before each block */
    double* Sb = (double*)malloc(sizeof(double) * SZ * (size_t)B);                    /* S_t inside a block */
    double* S = (double*)malloc(sizeof(double) * SZ);
    double* D = (double*)malloc(sizeof(double) * SZ);
    double* a = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    if (!ck || !Sb || !S || !D || !a) {
#pragma omp atomic write
      failed = 1;
      free(ck); free(Sb); free(S); free(D); free(a);
      continue;
    }
    const size_t r0 = (size_t)bh * (size_t)T;
    for (long long t = 0; t < T; ++t) a[t] = exp(gla_oracle_gate((double)x[r0 + t], gate));
#define KQ(arr, t, d) widen(arr, qkv_is_bf16, (r0 + (size_t)(t)) * (size_t)dkd + (size_t)(d))
#define VV(t, n) widen(v, qkv_is_bf16, (r0 + (size_t)(t)) * (size_t)dvd + (size_t)(n))
    /* forward sweep: checkpoints of S_{64c-1} */
    for (size_t i = 0; i < SZ; ++i) S[i] = S0 ? S0[(size_t)bh * SZ + i] : 0.0;
    for (long long t = 0; t < T; ++t) {
      if (t % B == 0) memcpy(ck + (size_t)(t / B) * SZ, S, sizeof(double) * SZ);
      for (int d = 0; d < dkd; ++d) {
        const double kd = KQ(k, t, d);
        for (int n = 0; n < dvd; ++n) S[(size_t)d * dvd + n] = a[t] * S[(size_t)d * dvd + n] + kd * VV(t, n);
      }
    }
    /* backward sweep */
    for (size_t i = 0; i < SZ; ++i) D[i] = dST ? dST[(size_t)bh * SZ + i] : 0.0;
    for (long long c = nblk - 1; c >= 0; --c) {
      const long long t0 = c * B, t1 = (t0 + B < T) ? t0 + B : T;
      /* S_t for t in [t0, t1) */
      memcpy(S, ck + (size_t)c * SZ, sizeof(double) * SZ);
      for (long long t = t0; t < t1; ++t) {
        double* St = Sb + (size_t)(t - t0) * SZ;
        for (int d = 0; d < dkd; ++d) {
          const double kd = KQ(k, t, d);
          for (int n = 0; n < dvd; ++n) {
            S[(size_t)d * dvd + n] = a[t] * S[(size_t)d * dvd + n] + kd * VV(t, n);
            St[(size_t)d * dvd + n] = S[(size_t)d * dvd + n];
          }
        }
      }
      for (long long t = t1 - 1; t >= t0; --t) {
        const double* St = Sb + (size_t)(t - t0) * SZ;
        const double* Sp = (t > t0) ? Sb + (size_t)(t - t0 - 1) * SZ : ck + (size_t)c * SZ;
        const double* g = dO + (r0 + (size_t)t) * (size_t)dvd;
        /* D_t = q_t dO_t^T + (carried a_{t+1} D_{t+1}) */
        for (int d = 0; d < dkd; ++d) {
          const double qd = KQ(q, t, d);
          for (int n = 0; n < dvd; ++n) D[(size_t)d * dvd + n] += qd * g[n];
        }
        for (int d = 0; d < dkd; ++d) {
          double accq = 0.0, acck = 0.0;
          for (int n = 0; n < dvd; ++n) {
#if GLA_ORACLE_MUTANT == 9
            accq += Sp[(size_t)d * dvd + n] * g[n];  /* planted: dq from S_{t-1} */
#else
            accq += St[(size_t)d * dvd + n] * g[n];
#endif
            acck += D[(size_t)d * dvd + n] * VV(t, n);
          }
          dq[(r0 + (size_t)t) * (size_t)dkd + d] = accq;
          dk[(r0 + (size_t)t) * (size_t)dkd + d] = acck;
        }
        for (int n = 0; n < dvd; ++n) {
          double acc = 0.0;
          for (int d = 0; d < dkd; ++d)
#if GLA_ORACLE_MUTANT == 10
            acc += D[(size_t)d * dvd + n] * KQ(q, t, d);  /* planted: dv from q instead of k */
#else
            acc += D[(size_t)d * dvd + n] * KQ(k, t, d);
#endif
          dv[(r0 + (size_t)t) * (size_t)dvd + n] = acc;
        }
        double da = 0.0;
        for (size_t i = 0; i < SZ; ++i) da += D[i] * Sp[i];
#if GLA_ORACLE_MUTANT == 8
        dx[r0 + (size_t)t] = da * gate_slope((double)x[r0 + t], gate);  /* planted: a_t factor dropped */
#else
        dx[r0 + (size_t)t] = da * a[t] * gate_slope((double)x[r0 + t], gate);
#endif
#if GLA_ORACLE_MUTANT != 7
        for (size_t i = 0; i < SZ; ++i) D[i] *= a[t];  /* carry a_t D_t to t-1 */
#endif
      }
    }
#undef KQ
#undef VV
    memcpy(dS0 + (size_t)bh * SZ, D, sizeof(double) * SZ);  /* a_0 D_0 (dS_T when T = 0) */
    free(ck); free(Sb); free(S); free(D); free(a);
  }
  return failed ? 2 : 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int gla_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * oracle.c -- plain fp64 CPU oracle for the GPT-2 / nanoGPT causal
 * self-attention layer (forward and exact backward).
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load this code.
 * It shares no source, header or build step with the HIP library.
 *
 * What it computes, and where each step comes from:
 *   page "nanoGPT global flow" (devpress.csdn.net), section 2.5 (B)
 *   CausalSelfAttention, and page "nanoGPT architecture explained step by
 *   step" (lzwjava.github.io), section 3 (causal self-attention) with its
 *   closing formula Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V.
 *
 *   1. qkv = x . W_attn + b_attn               (c_attn, one fused linear)
 *   2. q, k, v = column blocks [0,C), [C,2C), [2C,3C) of qkv; head h owns
 *      columns [h*hs, (h+1)*hs) of each block  (split, view, transpose)
 *   3. s_ij = (q_i . k_j) * (1/sqrt(hs))       (scores, scale)
 *   4. s_ij = -inf for j > i, diagonal kept    (tril mask, masked_fill)
 *   5. p_ij = softmax over j of s_ij           (row softmax)
 *   6. o_i  = sum_j p_ij v_j                   (att @ v)
 *   7. y_m[b,i,h*hs+d] = o[b,h,i,d]            (transpose back, merge heads)
 *   8. y = y_m . W_proj + b_proj               (c_proj)
 *   Dropout is the identity (dropout 0.0 in GPTConfig, page "nanoGPT global
 *   flow", section 2.1).
 *
 * Around the layer (the "next" pieces of a Block):
 *   LayerNorm: (x - mean) / sqrt(var + 1e-5) * w + b over the embedding, with
 *     the biased variance of F.layer_norm (page "nanoGPT global flow",
 *     section 2.5 (A));
 *   attention half of a Pre-LN block: out = x + attn(ln_1(x)) (same page,
 *     section 2.5, Block.forward; page "nanoGPT architecture explained step
 *     by step", section 2);
 *   MLP sublayer: c_proj(gelu(c_fc(x))) with gelu(u) = u * Phi(u), Phi the
 *     standard normal CDF written with erf (page "nanoGPT architecture
 *     explained step by step", section 4; page "nanoGPT global flow",
 *     section 2.5 (C)).
 *
 * Weights are taken as [in, out] row-major, i.e. the transpose of the
 * nn.Linear storage: y = x . W + b.
 *
 * The softmax is the two-pass textbook form over the whole visible row
 * (max, then exponentials, then the sum, then division); future positions
 * get probability exactly 0, which is what masked_fill(-inf) followed by
 * softmax produces.
 *
 * The backward is the exact gradient of steps 1-8 by the chain rule (the
 * pages only say that autograd applies the chain rule; page "nanoGPT global
 * flow", section 3 training loop).  The softmax gradient uses the Jacobian
 * form dS_ij = p_ij (dP_ij - sum_j' p_ij' dP_ij').
 *
 * Dropout (training; nn.Dropout on the attention weights after the softmax
 * and on the c_proj output, page "nanoGPT architecture explained step by
 * step", section 3, attn_dropout / resid_dropout; rate config.dropout) is
 * available as a separate entry point.  Each element keeps or drops on bits
 * of the Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011): an attention
 * weight on a 16-bit half of a word (dropped iff below floor(p * 2^16)), a
 * c_proj output element on a 32-bit word (dropped iff below
 * floor(p * 2^32)); kept values are scaled by 1/(1-p).
 *
 * Everything is double precision; callers pass the exact values the GPU
 * receives (bf16 and fp32 upcast exactly).  Work is split over threads by
 * output rows or by (batch, head) pairs only; no sum is reordered.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Round to the nearest bfloat16 value (8 significant bits), ties to even.
 * Only used to mimic a path that STORES an intermediate in bfloat16 (the
 * bf16 path keeps q, k, v and the merged heads in bf16); all arithmetic stays
 * double.  Normal range only (the layer's values are far from bf16's
 * limits). */
static double round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  const double f = frexp(v, &e); /* v = f * 2^e, 0.5 <= |f| < 1 */
  return ldexp(nearbyint(ldexp(f, 8)), e - 8);
}

static void round_all(double *a, size_t n) {
  for (size_t i = 0; i < n; ++i) a[i] = round_bf16(a[i]);
}

/* ------------------------------------------------------------------ */
/* A minimal parallel-for: items [0, n) handed out one by one.        */
/* ------------------------------------------------------------------ */
typedef void (*item_fn)(void *ctx, long item, double *scratch);

typedef struct {
  item_fn fn;
  void *ctx;
  long n;
  long next; /* shared counter */
  size_t scratch_doubles;
  int failed;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  double *scratch = NULL;
  if (p->scratch_doubles) {
    scratch = (double *)malloc(p->scratch_doubles * sizeof(double));
    if (!scratch) {
      __atomic_store_n(&p->failed, 1, __ATOMIC_SEQ_CST);
      return NULL;
    }
  }
  for (;;) {
    long i = __atomic_fetch_add(&p->next, 1, __ATOMIC_SEQ_CST);
    if (i >= p->n) break;
    p->fn(p->ctx, i, scratch);
  }
  free(scratch);
  return NULL;
}

static int parallel_for(long n, int nthreads, item_fn fn, void *ctx,
                        size_t scratch_doubles) {
  pool_t p = {fn, ctx, n, 0, scratch_doubles, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t tid[256];
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&tid[started], NULL, pool_worker, &p) != 0) break;
    ++started;
  }
  pool_worker(&p);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  return p.failed ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Dense linear layer: out[m][n] = bias[n] + sum_k in[m][k] * W[k][n]  */
/* (nn.Linear with the weight given as [in, out]).  One item = one row. */
/* ------------------------------------------------------------------ */
typedef struct {
  int K, N;
  const double *in, *W, *bias;
  double *out;
} linear_ctx;

static void linear_row(void *vctx, long m, double *scratch) {
  (void)scratch;
  const linear_ctx *c = (const linear_ctx *)vctx;
  double *row = c->out + (size_t)m * c->N;
  for (int n = 0; n < c->N; ++n) row[n] = 0.0;
  for (int k = 0; k < c->K; ++k) {
    const double a = c->in[(size_t)m * c->K + k];
    const double *w = c->W + (size_t)k * c->N;
    for (int n = 0; n < c->N; ++n) row[n] += a * w[n];
  }
  if (c->bias)
    for (int n = 0; n < c->N; ++n) row[n] += c->bias[n];
}

static int linear(int M, int K, int N, const double *in, const double *W,
                  const double *bias, double *out, int nthreads) {
  linear_ctx c = {K, N, in, W, bias, out};
  return parallel_for(M, nthreads, linear_row, &c, 0);
}

/* ------------------------------------------------------------------ */
/* Causal attention for one (b, h) pair.                               */
/* ------------------------------------------------------------------ */
typedef struct {
  int B, T, C, H;
  const double *qkv; /* [B*T][3C] */
  double *ym;        /* [B*T][C] merged heads */
  double *P;         /* optional [B][H][T][T] */
  double *lse;       /* optional [B][H][T] */
  int round_p;       /* weights of o = sum_j p_j v_j as the bf16 path rounds them */
} attn_ctx;

/* Scores of query row i of head (b, h): s[j] = (q_i . k_j) / sqrt(hs) for
 * j <= i.  Returns their maximum. */
static double score_row(const double *qkv, int T, int C, int H, int b, int h,
                        int i, double *s) {
  const int hs = C / H;
  const size_t ld = (size_t)3 * C;
  const double scale = 1.0 / sqrt((double)hs);
  const double *q = qkv + ((size_t)b * T + i) * ld + (size_t)h * hs;
  double m = -INFINITY;
  for (int j = 0; j <= i; ++j) {
    const double *k = qkv + ((size_t)b * T + j) * ld + C + (size_t)h * hs;
    double dot = 0.0;
    for (int d = 0; d < hs; ++d) dot += q[d] * k[d];
    s[j] = dot * scale;
    if (s[j] > m) m = s[j];
  }
  return m;
}

/* Probabilities of query row i of head (b, h): p[j] for j <= i.
 * s_j = (q_i . k_j) / sqrt(hs); two-pass softmax.  Returns the row's
 * log-sum-exp log(sum_j exp(s_j)). */
static double prob_row(const double *qkv, int T, int C, int H, int b, int h,
                       int i, double *p) {
  const double m = score_row(qkv, T, C, H, b, h, i, p);
  double Z = 0.0;
  for (int j = 0; j <= i; ++j) {
    p[j] = exp(p[j] - m);
    Z += p[j];
  }
  for (int j = 0; j <= i; ++j) p[j] /= Z;
  return m + log(Z);
}

/* The weights with which a bf16 path forms o_i = sum_j p_ij v_j when it
 * feeds each weight to its bf16 matrix product as a bf16 value and
 * normalises by the sum of the unrounded weights.  The unnormalised weight
 * is taken relative to a whole power of two, u_j = 2^(t_j - M) with
 * t_j = s_j log2(e) and M = ceil(max_j t_j), so that its rounding does not
 * depend on which reference the path used: rounding to 8 significant bits
 * commutes with scaling by any power of two.  w[j] = bf16(u_j) / sum_j' u_j'.
 * s: the row's scaled scores (j < n); w may alias s. */
static void pv_weights_bf16(const double *s, int n, double *w) {
  const double log2e = 1.0 / log(2.0);
  double tmax = -INFINITY;
  for (int j = 0; j < n; ++j)
    if (s[j] * log2e > tmax) tmax = s[j] * log2e;
  const double M = ceil(tmax);
  double U = 0.0;
  for (int j = 0; j < n; ++j) {
    w[j] = exp2(s[j] * log2e - M);
    U += w[j];
  }
  for (int j = 0; j < n; ++j) w[j] = round_bf16(w[j]) / U;
}

static void attn_head(void *vctx, long item, double *p) {
  const attn_ctx *c = (const attn_ctx *)vctx;
  const int b = (int)(item / c->H), h = (int)(item % c->H);
  const int T = c->T, C = c->C, H = c->H, hs = C / H;
  const size_t ld = (size_t)3 * C;
  double *wp = c->round_p ? p + T : p; /* weights of the value rows */
  for (int i = 0; i < T; ++i) {
    const double l = prob_row(c->qkv, T, C, H, b, h, i, p);
    if (c->round_p) {
      score_row(c->qkv, T, C, H, b, h, i, wp);
      pv_weights_bf16(wp, i + 1, wp);
    }
    double *o = c->ym + ((size_t)b * T + i) * C + (size_t)h * hs;
    for (int d = 0; d < hs; ++d) o[d] = 0.0;
    for (int j = 0; j <= i; ++j) {
      const double *v =
          c->qkv + ((size_t)b * T + j) * ld + 2 * (size_t)C + (size_t)h * hs;
      for (int d = 0; d < hs; ++d) o[d] += wp[j] * v[d];
    }
    if (c->P) {
      double *row = c->P + (((size_t)b * H + h) * T + i) * T;
      for (int j = 0; j < T; ++j) row[j] = (j <= i) ? p[j] : 0.0;
    }
    if (c->lse) c->lse[((size_t)b * H + h) * T + i] = l;
  }
}

/* ------------------------------------------------------------------ */
/* Forward.                                                            */
/* ------------------------------------------------------------------ */
/* x [B][T][C], W_attn [C][3C], b_attn [3C] or NULL, W_proj [C][C],
 * b_proj [C] or NULL.  Outputs: y [B][T][C] (required); qkv [B][T][3C],
 * ym [B][T][C], P [B][H][T][T], lse [B][H][T] (each optional, NULL = not
 * wanted).  store_bf16: bit 0 rounds qkv to bfloat16 after step 1, bit 1
 * rounds the merged heads after step 7, bit 5 (value 32) forms step 6 with
 * the weights a bf16 path feeds its P.V product (pv_weights_bf16); P and
 * lse stay the exact softmax (0 = exact fp64 throughout).
 * Returns 0, or -1 on bad arguments / allocation failure. */
int oracle_forward(int B, int T, int C, int H, const double *x,
                   const double *W_attn, const double *b_attn,
                   const double *W_proj, const double *b_proj, double *y,
                   double *qkv_out, double *ym_out, double *P_out,
                   double *lse_out, int store_bf16, int nthreads) {
  if (B < 0 || T < 0 || C <= 0 || H <= 0 || C % H != 0) return -1;
  if (!x || !W_attn || !W_proj || !y) return -1;
  const long M = (long)B * T;
  if (M == 0) return 0;
  double *qkv = qkv_out ? qkv_out : (double *)malloc((size_t)M * 3 * C * sizeof(double));
  double *ym = ym_out ? ym_out : (double *)malloc((size_t)M * C * sizeof(double));
  int rc = -1;
  if (!qkv || !ym) goto done;
  if (linear((int)M, C, 3 * C, x, W_attn, b_attn, qkv, nthreads)) goto done;
  if (store_bf16 & 1) round_all(qkv, (size_t)M * 3 * C);
  {
    attn_ctx a = {B, T, C, H, qkv, ym, P_out, lse_out, (store_bf16 & 32) != 0};
    if (parallel_for((long)B * H, nthreads, attn_head, &a, (size_t)2 * T)) goto done;
  }
  if (store_bf16 & 2) round_all(ym, (size_t)M * C);
  if (linear((int)M, C, C, ym, W_proj, b_proj, y, nthreads)) goto done;
  rc = 0;
done:
  if (!qkv_out) free(qkv);
  if (!ym_out) free(ym);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Backward pieces.                                                    */
/* ------------------------------------------------------------------ */
/* dW[k][n] = sum_m in[m][k] * dout[m][n]; one item = one row k. */
typedef struct {
  int M, K, N;
  const double *in, *dout;
  double *dW;
} wgrad_ctx;

static void wgrad_row(void *vctx, long k, double *scratch) {
  (void)scratch;
  const wgrad_ctx *c = (const wgrad_ctx *)vctx;
  double *row = c->dW + (size_t)k * c->N;
  for (int n = 0; n < c->N; ++n) row[n] = 0.0;
  for (int m = 0; m < c->M; ++m) {
    const double a = c->in[(size_t)m * c->K + k];
    const double *g = c->dout + (size_t)m * c->N;
    for (int n = 0; n < c->N; ++n) row[n] += a * g[n];
  }
}

/* db[n] = sum_m dout[m][n] (single thread; cheap). */
static void bias_grad(int M, int N, const double *dout, double *db) {
  for (int n = 0; n < N; ++n) db[n] = 0.0;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n) db[n] += dout[(size_t)m * N + n];
}

/* din[m][k] = sum_n dout[m][n] * W[k][n]; one item = one row m. */
typedef struct {
  int K, N;
  const double *dout, *W;
  double *din;
} dgrad_ctx;

static void dgrad_row(void *vctx, long m, double *scratch) {
  (void)scratch;
  const dgrad_ctx *c = (const dgrad_ctx *)vctx;
  const double *g = c->dout + (size_t)m * c->N;
  for (int k = 0; k < c->K; ++k) {
    const double *w = c->W + (size_t)k * c->N;
    double s = 0.0;
    for (int n = 0; n < c->N; ++n) s += g[n] * w[n];
    c->din[(size_t)m * c->K + k] = s;
  }
}

/* Factor of a kept element under dropout rate p, 1 / (1 - p); with
 * scale32 the float nearest to it, the factor a path that computes in single
 * precision multiplies by. */
static double keep_scale_of(double p, int scale32) {
  const double s = 1.0 / (1.0 - p);
  return scale32 ? (double)(float)s : s;
}

/* Attention backward for one (b, h): from dym (gradient of the merged
 * heads) to the q, k, v column blocks of dqkv. */
typedef struct {
  int B, T, C, H;
  const double *qkv, *dym;
  const double *ym; /* merged heads as stored by the forward */
  double *dqkv;
  double p;      /* dropout rate of the attention weights (0: none) */
  uint64_t seed;
  int round_pb;  /* dv_j sums bf16(p_ij z_ij) dO_i, as a bf16 path's product */
  int row_from_o; /* row term as dO_i . o_i over the stored merged heads */
  int round_ds;   /* dq, dk sum bf16(ds_ij), as a bf16 path's products */
  int scale32;    /* keep factor held in single precision */
} attn_bwd_ctx;

int oracle_dropout_keep_attn(int b, int h, int H, int i, int j, uint64_t seed, uint32_t thresh16);
uint32_t oracle_dropout_threshold(double p);
uint32_t oracle_dropout_threshold16(double p);

static void attn_bwd_head(void *vctx, long item, double *scratch) {
  const attn_bwd_ctx *c = (const attn_bwd_ctx *)vctx;
  const int b = (int)(item / c->H), h = (int)(item % c->H);
  const int T = c->T, C = c->C, H = c->H, hs = C / H;
  const size_t ld = (size_t)3 * C;
  const double scale = 1.0 / sqrt((double)hs);
  double *p = scratch;       /* [T] probabilities of row i */
  double *dp = scratch + T;  /* [T] dL/dp_ij               */
  /* dropout: weight p_ij enters o_i as p_ij z_ij with z_ij = 1/(1-p) if
   * kept, 0 if dropped (z = 1 without dropout) */
  const double keep_scale = c->p > 0.0 ? keep_scale_of(c->p, c->scale32) : 1.0;
  const uint32_t thresh = c->p > 0.0 ? oracle_dropout_threshold16(c->p) : 0u;
  /* zero this head's dq, dk, dv columns */
  for (int t = 0; t < T; ++t) {
    double *r = c->dqkv + ((size_t)b * T + t) * ld + (size_t)h * hs;
    for (int d = 0; d < hs; ++d) r[d] = r[C + d] = r[2 * C + d] = 0.0;
  }
  for (int i = 0; i < T; ++i) {
    prob_row(c->qkv, T, C, H, b, h, i, p);
    const double *dO = c->dym + ((size_t)b * T + i) * C + (size_t)h * hs;
    const double *qi = c->qkv + ((size_t)b * T + i) * ld + (size_t)h * hs;
    /* dp_ij = dO_i . v_j ;  dv_j += p_ij dO_i */
    double rowdot = 0.0;
    for (int j = 0; j <= i; ++j) {
      const double *vj = c->qkv + ((size_t)b * T + j) * ld + 2 * (size_t)C + (size_t)h * hs;
      double *dvj = c->dqkv + ((size_t)b * T + j) * ld + 2 * (size_t)C + (size_t)h * hs;
      const double z =
          (c->p > 0.0 && !oracle_dropout_keep_attn(b, h, H, i, j, c->seed, thresh)) ? 0.0
                                                                                    : keep_scale;
      double pv = p[j] * z;
      if (c->round_pb) pv = round_bf16(pv);
      double s = 0.0;
      for (int d = 0; d < hs; ++d) {
        s += dO[d] * vj[d];
        dvj[d] += pv * dO[d];
      }
      dp[j] = s * z;
      rowdot += p[j] * dp[j];
    }
    /* softmax Jacobian: ds_ij = p_ij (dp_ij - sum_j' p_ij' dp_ij');
     * scores s_ij = scale q_i . k_j  =>  dq_i += scale ds_ij k_j,
     * dk_j += scale ds_ij q_i.  The row term equals dO_i . o_i (o_i is
     * sum_j p_ij z_ij v_j); row_from_o forms it that way from the stored
     * merged heads, as a path that keeps only those does. */
    if (c->row_from_o) {
      const double *oi = c->ym + ((size_t)b * T + i) * C + (size_t)h * hs;
      rowdot = 0.0;
      for (int d = 0; d < hs; ++d) rowdot += dO[d] * oi[d];
    }
    double *dqi = c->dqkv + ((size_t)b * T + i) * ld + (size_t)h * hs;
    for (int j = 0; j <= i; ++j) {
      double ds = p[j] * (dp[j] - rowdot);
      if (c->round_ds) ds = round_bf16(ds);
      const double *kj = c->qkv + ((size_t)b * T + j) * ld + C + (size_t)h * hs;
      double *dkj = c->dqkv + ((size_t)b * T + j) * ld + C + (size_t)h * hs;
      for (int d = 0; d < hs; ++d) {
        dqi[d] += scale * ds * kj[d];
        dkj[d] += scale * ds * qi[d];
      }
    }
  }
}

/* Exact gradient of the layer for upstream gradient dY [B][T][C].
 * Outputs (each required, fully overwritten): dx [B][T][C],
 * dW_attn [C][3C], dW_proj [C][C]; db_attn [3C] and db_proj [C] are
 * written when non-NULL (NULL = the layer has no bias).  Optional:
 * dqkv [B][T][3C] and dym [B][T][C] intermediates.
 * store_bf16 rounds stored tensors to bfloat16 where a bf16 path stores
 * them: bit 0 qkv and bit 1 the merged heads (as in oracle_forward), bit 2
 * the gradient of the merged heads, bit 3 the gradient of qkv; every
 * gradient is then the exact chain rule through those stored values.  Bit 5
 * (32) forms the forward's merged heads with the bf16 path's P.V weights
 * (as in oracle_forward); bit 6 (64) sums dv_j over bf16(p_ij z_ij), the
 * value-gradient operand a bf16 path feeds its matrix product (the softmax
 * gradient keeps the exact p); bit 7 (128) forms the softmax gradient's row
 * term as dO_i . o_i from the merged heads the forward stored (rounded when
 * bit 1 is set); bit 8 (256) rounds each ds_ij to bfloat16 before the query
 * and key gradients, as a bf16 path's operands; bit 9 (512) holds the
 * dropout keep factor 1/(1-p) in single precision. */
static int forward_dropout_impl(int B, int T, int C, int H, const double *x,
                                const double *W_attn, const double *b_attn,
                                const double *W_proj, const double *b_proj, double p,
                                uint64_t seed, double *y, double *qkv, double *ym,
                                int store_bf16, int nthreads);
int oracle_dropout_keep_resid(long m, int n, uint64_t seed, uint32_t thresh);

static int backward_impl(int B, int T, int C, int H, const double *x, const double *W_attn,
                         const double *b_attn, const double *W_proj, const double *b_proj,
                         const double *dY, double p_drop, uint64_t seed, double *dx,
                         double *dW_attn, double *db_attn, double *dW_proj, double *db_proj,
                         double *dqkv_out, double *dym_out, int store_bf16, int nthreads) {
  if (B < 0 || T < 0 || C <= 0 || H <= 0 || C % H != 0) return -1;
  if (!x || !W_attn || !W_proj || !dY || !dx || !dW_attn || !dW_proj) return -1;
  if (!(p_drop >= 0.0 && p_drop < 1.0)) return -1;
  const long M = (long)B * T;
  int rc = -1;
  double *qkv = (double *)malloc(((size_t)M * 3 * C + 1) * sizeof(double));
  double *ym = (double *)malloc(((size_t)M * C + 1) * sizeof(double));
  double *y = (double *)malloc(((size_t)M * C + 1) * sizeof(double));
  double *dyd = (double *)malloc(((size_t)M * C + 1) * sizeof(double));
  double *dym = dym_out ? dym_out : (double *)malloc(((size_t)M * C + 1) * sizeof(double));
  double *dqkv = dqkv_out ? dqkv_out : (double *)malloc(((size_t)M * 3 * C + 1) * sizeof(double));
  if (!qkv || !ym || !y || !dyd || !dym || !dqkv) goto done;
  if (p_drop > 0.0) {
    if (M > 0 && forward_dropout_impl(B, T, C, H, x, W_attn, b_attn, W_proj, b_proj, p_drop,
                                      seed, y, qkv, ym, store_bf16 & 547, nthreads))
      goto done;
    /* resid_dropout: y = drop(ym . W_proj + b_proj)  =>  the c_proj
     * gradients see dY z with z = 1/(1-p) (kept) or 0 (dropped) */
    const uint32_t thresh = oracle_dropout_threshold(p_drop);
    const double ks = keep_scale_of(p_drop, (store_bf16 & 512) != 0);
    for (long m = 0; m < M; ++m)
      for (int n = 0; n < C; ++n)
        dyd[(size_t)m * C + n] = oracle_dropout_keep_resid(m, n, seed, thresh)
                                     ? dY[(size_t)m * C + n] * ks
                                     : 0.0;
    if (store_bf16 & 16) round_all(dyd, (size_t)M * C);
  } else {
    if (oracle_forward(B, T, C, H, x, W_attn, b_attn, W_proj, b_proj, y, qkv, ym,
                       NULL, NULL, store_bf16 & 35, nthreads))
      goto done;
    memcpy(dyd, dY, (size_t)M * C * sizeof(double));
  }
  /* c_proj: y = ym . W_proj + b_proj */
  if (db_proj) bias_grad((int)M, C, dyd, db_proj);
  {
    wgrad_ctx w = {(int)M, C, C, ym, dyd, dW_proj};
    if (parallel_for(C, nthreads, wgrad_row, &w, 0)) goto done;
    dgrad_ctx g = {C, C, dyd, W_proj, dym};
    if (parallel_for(M, nthreads, dgrad_row, &g, 0)) goto done;
  }
  if (store_bf16 & 4) round_all(dym, (size_t)M * C);
  /* attention core */
  {
    attn_bwd_ctx a = {B,     T,     C,          H,
                      qkv,   dym,   ym,         dqkv,
                      p_drop, seed, (store_bf16 & 64) != 0, (store_bf16 & 128) != 0,
                      (store_bf16 & 256) != 0, (store_bf16 & 512) != 0};
    if (parallel_for((long)B * H, nthreads, attn_bwd_head, &a, (size_t)2 * T + 2))
      goto done;
  }
  if (store_bf16 & 8) round_all(dqkv, (size_t)M * 3 * C);
  /* c_attn: qkv = x . W_attn + b_attn */
  if (db_attn) bias_grad((int)M, 3 * C, dqkv, db_attn);
  {
    wgrad_ctx w = {(int)M, C, 3 * C, x, dqkv, dW_attn};
    if (parallel_for(C, nthreads, wgrad_row, &w, 0)) goto done;
    dgrad_ctx g = {C, 3 * C, dqkv, W_attn, dx};
    if (parallel_for(M, nthreads, dgrad_row, &g, 0)) goto done;
  }
  (void)b_attn;
  rc = 0;
done:
  free(qkv);
  free(ym);
  free(y);
  free(dyd);
  if (!dym_out) free(dym);
  if (!dqkv_out) free(dqkv);
  return rc;
}

int oracle_backward(int B, int T, int C, int H, const double *x,
                    const double *W_attn, const double *b_attn,
                    const double *W_proj, const double *b_proj,
                    const double *dY, double *dx, double *dW_attn,
                    double *db_attn, double *dW_proj, double *db_proj,
                    double *dqkv_out, double *dym_out, int store_bf16,
                    int nthreads) {
  return backward_impl(B, T, C, H, x, W_attn, b_attn, W_proj, b_proj, dY, 0.0, 0, dx, dW_attn,
                       db_attn, dW_proj, db_proj, dqkv_out, dym_out, store_bf16, nthreads);
}

/* Exact gradient of the forward with dropout rate p and generator seed
 * (oracle_forward_dropout): the same masks scale the gradients that flow
 * through the dropped weights and outputs.  store_bf16 bit 4 (value 16)
 * additionally rounds the masked, rescaled upstream gradient of the c_proj
 * output, which a bf16 path stores. */
int oracle_backward_dropout(int B, int T, int C, int H, const double *x, const double *W_attn,
                            const double *b_attn, const double *W_proj, const double *b_proj,
                            const double *dY, double p, uint64_t seed, double *dx,
                            double *dW_attn, double *db_attn, double *dW_proj,
                            double *db_proj, double *dqkv_out, double *dym_out, int store_bf16,
                            int nthreads) {
  return backward_impl(B, T, C, H, x, W_attn, b_attn, W_proj, b_proj, dY, p, seed, dx, dW_attn,
                       db_attn, dW_proj, db_proj, dqkv_out, dym_out, store_bf16, nthreads);
}

/* ------------------------------------------------------------------ */
/* LayerNorm, attention half of a Pre-LN block, MLP sublayer.          */
/* ------------------------------------------------------------------ */
typedef struct {
  int C;
  const double *x, *w, *b;
  double *out;
} ln_ctx;

static void ln_row(void *vctx, long m, double *scratch) {
  (void)scratch;
  const ln_ctx *c = (const ln_ctx *)vctx;
  const double *row = c->x + (size_t)m * c->C;
  double mean = 0.0;
  for (int i = 0; i < c->C; ++i) mean += row[i];
  mean /= c->C;
  double var = 0.0;
  for (int i = 0; i < c->C; ++i) var += (row[i] - mean) * (row[i] - mean);
  var /= c->C; /* biased, as F.layer_norm */
  const double inv = 1.0 / sqrt(var + 1e-5);
  double *o = c->out + (size_t)m * c->C;
  for (int i = 0; i < c->C; ++i)
    o[i] = (row[i] - mean) * inv * c->w[i] + (c->b ? c->b[i] : 0.0);
}

/* out = LayerNorm(x) row by row; x, out [M][C]; b may be NULL. */
int oracle_layernorm(int M, int C, const double *x, const double *w, const double *b,
                     double *out, int nthreads) {
  if (M < 0 || C <= 0 || !x || !w || !out) return -1;
  ln_ctx c = {C, x, w, b, out};
  return parallel_for(M, nthreads, ln_row, &c, 0);
}

/* Attention half of a Pre-LN block: out = x + layer(ln_1(x)).
 * store_bf16 bits 0/1/5 as in oracle_forward; bit 4 rounds the LayerNorm
 * output (the layer's input) to bfloat16.  ln_out [B][T][C] optional. */
int oracle_block_attn_forward(int B, int T, int C, int H, const double *x,
                              const double *ln_w, const double *ln_b,
                              const double *W_attn, const double *b_attn,
                              const double *W_proj, const double *b_proj,
                              double *out, double *ln_out, int store_bf16,
                              int nthreads) {
  if (B < 0 || T < 0 || C <= 0 || H <= 0 || C % H != 0 || !x || !ln_w || !out) return -1;
  const long M = (long)B * T;
  int rc = -1;
  double *ln = ln_out ? ln_out : (double *)malloc(((size_t)M * C + 1) * sizeof(double));
  double *y = (double *)malloc(((size_t)M * C + 1) * sizeof(double));
  if (!ln || !y) goto done;
  if (oracle_layernorm((int)M, C, x, ln_w, ln_b, ln, nthreads)) goto done;
  if (store_bf16 & 16) round_all(ln, (size_t)M * C);
  if (oracle_forward(B, T, C, H, ln, W_attn, b_attn, W_proj, b_proj, y, NULL, NULL,
                     NULL, NULL, store_bf16 & 35, nthreads))
    goto done;
  for (size_t i = 0; i < (size_t)M * C; ++i) out[i] = x[i] + y[i];
  rc = 0;
done:
  if (!ln_out) free(ln);
  free(y);
  return rc;
}

/* gelu(u) = u * Phi(u) = u * (1 + erf(u / sqrt(2))) / 2 */
static double gelu(double u) { return u * 0.5 * (1.0 + erf(u / sqrt(2.0))); }

/* MLP sublayer: y = gelu(x . W_fc + b_fc) . W_proj + b_proj.
 * x [M][C], W_fc [C][F], b_fc [F] or NULL, W_proj [F][C], b_proj [C] or NULL,
 * y [M][C]; h_out [M][F] (optional) receives gelu's output.  store_bf16 bit
 * 0 rounds that hidden activation to bfloat16. */
int oracle_mlp_forward(int M, int C, int F, const double *x, const double *W_fc,
                       const double *b_fc, const double *W_proj, const double *b_proj,
                       double *y, double *h_out, int store_bf16, int nthreads) {
  if (M < 0 || C <= 0 || F <= 0 || !x || !W_fc || !W_proj || !y) return -1;
  double *h = h_out ? h_out : (double *)malloc(((size_t)M * F + 1) * sizeof(double));
  if (!h) return -1;
  int rc = -1;
  if (linear(M, C, F, x, W_fc, b_fc, h, nthreads)) goto done;
  for (size_t i = 0; i < (size_t)M * F; ++i) h[i] = gelu(h[i]);
  if (store_bf16 & 1) round_all(h, (size_t)M * F);
  if (linear(M, F, C, h, W_proj, b_proj, y, nthreads)) goto done;
  rc = 0;
done:
  if (!h_out) free(h);
  return rc;
}


/* ------------------------------------------------------------------ */
/* Philox4x32-10 and dropout.                                          */
/* ------------------------------------------------------------------ */
/* One Philox4x32 round: two 32x32->64 products of counter words 0 and 2 by
 * the round multipliers; the high halves are mixed with words 1 and 3 and
 * the round key, the low halves move to words 1 and 3.  Between rounds the
 * key advances by the Weyl constants.  Ten rounds (Salmon et al., SC 2011,
 * section 4, Philox-4x32 with R = 10). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* Drop threshold of rate p: a 32-bit word w drops its element iff w < t,
 * t = floor(p * 2^32) (capped at 2^32 - 1), so P(drop) = t / 2^32. */
uint32_t oracle_dropout_threshold(double p) {
  const double t = floor(p * 4294967296.0);
  return t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
}

/* The same for a 16-bit value u: dropped iff u < t16, t16 = floor(p * 2^16)
 * (capped at 2^16 - 1), so P(drop) = t16 / 2^16, within 2^-16 of p. */
uint32_t oracle_dropout_threshold16(double p) {
  const double t = floor(p * 65536.0);
  return t >= 65535.0 ? 0xFFFFu : (uint32_t)t;
}

/* Keep decision of one element: the word (c0 & 3) of Philox(ctr = {c0 >> 2,
 * c1, c2, stream}, key = seed split into low / high 32 bits). */
static int keep_elem(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t stream, uint64_t seed,
                     uint32_t thresh) {
  const uint32_t ctr[4] = {c0 >> 2, c1, c2, stream};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  oracle_philox4x32_10(ctr, key, w);
  return w[c0 & 3] >= thresh;
}

/* Keep mask of the attention weights of head (b, h), query i, key j
 * (stream 1): one Philox call covers the eight keys of the aligned group
 * j / 8, counter {j / 8, i, b*H + h, 1}; key j takes the low (j even) or high
 * (j odd) 16-bit half of word (j % 8) / 2 and is dropped iff that value is
 * below thresh16.  Of the c_proj output element (row m = b*T + t, column n):
 * stream 2, keep_elem over counter words (n, m, 0). */
int oracle_dropout_keep_attn(int b, int h, int H, int i, int j, uint64_t seed, uint32_t thresh16) {
  const uint32_t ctr[4] = {(uint32_t)j >> 3, (uint32_t)i, (uint32_t)(b * H + h), 1u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  oracle_philox4x32_10(ctr, key, w);
  const uint32_t u = (w[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFFu;
  return u >= thresh16;
}
int oracle_dropout_keep_resid(long m, int n, uint64_t seed, uint32_t thresh) {
  return keep_elem((uint32_t)n, (uint32_t)m, 0u, 2u, seed, thresh);
}

typedef struct {
  int B, T, C, H;
  const double *qkv;
  double *ym;
  double p;
  uint64_t seed;
  uint32_t thresh16; /* attention-weight drop threshold (16-bit values) */
  int round_p; /* as attn_ctx.round_p */
  int scale32; /* keep factor held in single precision */
} drop_attn_ctx;

/* Head (b, h) with dropout on the softmax weights: the row is normalised
 * over all visible keys first, then each weight is dropped or scaled by
 * 1/(1-p) before it weights its value row. */
static void drop_attn_head(void *vctx, long item, double *p) {
  const drop_attn_ctx *c = (const drop_attn_ctx *)vctx;
  const int b = (int)(item / c->H), h = (int)(item % c->H);
  const int T = c->T, C = c->C, H = c->H, hs = C / H;
  const size_t ld = (size_t)3 * C;
  const double keep_scale = keep_scale_of(c->p, c->scale32);
  double *wp = c->round_p ? p + T : p; /* weights of the value rows */
  for (int i = 0; i < T; ++i) {
    prob_row(c->qkv, T, C, H, b, h, i, p);
    if (c->round_p) {
      score_row(c->qkv, T, C, H, b, h, i, wp);
      pv_weights_bf16(wp, i + 1, wp);
    }
    double *o = c->ym + ((size_t)b * T + i) * C + (size_t)h * hs;
    for (int d = 0; d < hs; ++d) o[d] = 0.0;
    for (int j = 0; j <= i; ++j) {
      if (!oracle_dropout_keep_attn(b, h, H, i, j, c->seed, c->thresh16)) continue;
      const double w = wp[j] * keep_scale;
      const double *v = c->qkv + ((size_t)b * T + j) * ld + 2 * (size_t)C + (size_t)h * hs;
      for (int d = 0; d < hs; ++d) o[d] += w * v[d];
    }
  }
}

/* Forward with dropout rate p (0 <= p < 1) on the attention weights and on
 * the c_proj output, masks from Philox keyed by `seed` as above.  Arguments
 * otherwise as oracle_forward (ym_out optional; store_bf16 bits 0 / 1 round
 * qkv / merged heads, bit 5 takes the bf16 path's P.V weights, bit 9 (512)
 * holds the keep factor 1/(1-p) in single precision).  p = 0 keeps everything (same result as
 * oracle_forward). */
static int forward_dropout_impl(int B, int T, int C, int H, const double *x,
                                const double *W_attn, const double *b_attn,
                                const double *W_proj, const double *b_proj, double p,
                                uint64_t seed, double *y, double *qkv, double *ym,
                                int store_bf16, int nthreads) {
  const long M = (long)B * T;
  const uint32_t thresh = oracle_dropout_threshold(p);
  if (linear((int)M, C, 3 * C, x, W_attn, b_attn, qkv, nthreads)) return -1;
  if (store_bf16 & 1) round_all(qkv, (size_t)M * 3 * C);
  {
    drop_attn_ctx a = {B,   T,  C, H, qkv, ym, p, seed, oracle_dropout_threshold16(p),
                       (store_bf16 & 32) != 0, (store_bf16 & 512) != 0};
    if (parallel_for((long)B * H, nthreads, drop_attn_head, &a, (size_t)2 * T)) return -1;
  }
  if (store_bf16 & 2) round_all(ym, (size_t)M * C);
  if (linear((int)M, C, C, ym, W_proj, b_proj, y, nthreads)) return -1;
  const double keep_scale = keep_scale_of(p, (store_bf16 & 512) != 0);
  for (long m = 0; m < M; ++m)
    for (int n = 0; n < C; ++n)
      y[(size_t)m * C + n] = oracle_dropout_keep_resid(m, n, seed, thresh)
                                 ? y[(size_t)m * C + n] * keep_scale
                                 : 0.0;
  return 0;
}

int oracle_forward_dropout(int B, int T, int C, int H, const double *x, const double *W_attn,
                           const double *b_attn, const double *W_proj, const double *b_proj,
                           double p, uint64_t seed, double *y, double *ym_out, int store_bf16,
                           int nthreads) {
  if (B < 0 || T < 0 || C <= 0 || H <= 0 || C % H != 0) return -1;
  if (!x || !W_attn || !W_proj || !y || !(p >= 0.0 && p < 1.0)) return -1;
  const long M = (long)B * T;
  if (M == 0) return 0;
  double *qkv = (double *)malloc((size_t)M * 3 * C * sizeof(double));
  double *ym = ym_out ? ym_out : (double *)malloc((size_t)M * C * sizeof(double));
  int rc = -1;
  if (qkv && ym)
    rc = forward_dropout_impl(B, T, C, H, x, W_attn, b_attn, W_proj, b_proj, p, seed, y, qkv,
                              ym, store_bf16, nthreads);
  free(qkv);
  if (!ym_out) free(ym);
  return rc;
}

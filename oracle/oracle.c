/*
 * oracle.c -- plain fp64 CPU oracle for one GPU's share of head/sequence
 * parallel attention.  TEST INFRASTRUCTURE ONLY: it is called by the tests,
 * by __graft_entry__.smoke() and by bench.py's CPU-baseline leg, never by the
 * product path.  It shares no code, header or table with the HIP library.
 *
 * Every routine computes the plain definition of its result, written out as
 * loops in double precision.  No tiling, no online rescaling, no fusion.
 *
 * Sources (pages, by title and section):
 *  - "Megatron-LM - Training Multi-Billion Parameter Language Models Using
 *    Model Parallelism" (blog notes), section on the linear algebra of
 *    attention: scores are Q K^T scaled by 1/sqrt(d_k), normalised by softmax,
 *    then used to weight V.
 *  - "adv07: Sequence Parallel", question Q4: out[i] = softmax(q[i] K^T /
 *    sqrt(d)) V, and the causal mask hides only future keys (j > i); every
 *    key j <= i takes part.  Section 4 (implementation details): row i depends
 *    on q[i] only.  Question Q5: a Q chunk placed at a later position attends
 *    to the prefix before it (global positions).
 *  - "parallel multi-head attention" (mlwithme), section 3.2 (forward pass):
 *    layout [batch, seq, heads, head_dim], an additive mask on the scores,
 *    softmax over the key axis, then the product with V; heads independent.
 *  - "Support deepspeed sequence parallel" (transformers PR 31525), data
 *    collator: rank r holds tokens [r*S/P, (r+1)*S/P), position ids are global,
 *    and the key mask is "token is not padding".
 *
 * Readings where the pages are silent (each documented in the design notes):
 *  - masked score = -infinity (weight exactly 0); a row with no visible key
 *    gives out = 0 and lse = -infinity;
 *  - causal visibility uses global positions: key j visible to query i iff
 *    k_pos0 + j <= q_pos0 + i (diagonal included);
 *  - key padding: key j visible iff j < kv_len[b] (kv_len clamped to [0, Sk]);
 *  - lse = natural log of the softmax denominator including the max shift;
 *  - the merge of partial results is the log-sum-exp combination
 *    (not on the pages; pinned by "chunked + merged == unchunked").
 *
 * Inputs: element type 0 = float32, 1 = bfloat16 (raw 16-bit patterns).
 * bfloat16 -> double is exact (bit shift into a float, then widen).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ---- element access -------------------------------------------------- */

static double elem_to_double(const void* base, int dtype, size_t idx) {
  if (dtype == ORACLE_BF16) {
    uint16_t h = ((const uint16_t*)base)[idx];
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

/* Offset of element [b, s, h, d] in a contiguous [B, S, H, D] tensor. */
static size_t bshd(int64_t b, int64_t s, int64_t h, int64_t d, int64_t S, int64_t H, int64_t D) {
  return (size_t)(((b * S + s) * H + h) * D + d);
}

/* Visibility of key j to query i (readings above). */
static int visible(int causal, int64_t q_pos0, int64_t k_pos0, int64_t i, int64_t j,
                   int64_t len_b) {
  if (len_b >= 0 && j >= len_b) return 0;
  if (causal && k_pos0 + j > q_pos0 + i) return 0;
  return 1;
}

static int64_t clamp_len(const int32_t* kv_len, int64_t b, int64_t Sk) {
  if (!kv_len) return -1; /* no key padding */
  int64_t L = kv_len[b];
  if (L < 0) L = 0;
  if (L > Sk) L = Sk;
  return L;
}

/* ---- attention, two-pass per row ------------------------------------- */

typedef struct {
  const void *q, *k, *v;
  int dtype;
  int64_t B, Sq, Sk, H, D;
  int causal;
  int64_t q_pos0, k_pos0;
  const int32_t* kv_len;
  double scale;
  int64_t n_rows;
  const int64_t* rows; /* flat b*Sq + i, or NULL for all rows in order */
  double* out;         /* [n_rows, H, D] */
  double* lse;         /* [n_rows, H] */
  int64_t next;        /* work counter (row index), guarded by mu */
  pthread_mutex_t mu;
} attn_job;

/* One (row, head): out_i = sum_j softmax_j(s) v_j, s_j = scale * q_i . k_j. */
static void attn_row(attn_job* J, int64_t r, int64_t h, double* s, double* qd, double* acc) {
  const int64_t flat = J->rows ? J->rows[r] : r;
  const int64_t b = flat / J->Sq, i = flat % J->Sq;
  const int64_t D = J->D;
  const int64_t len_b = clamp_len(J->kv_len, b, J->Sk);
  double* o = J->out + ((size_t)r * J->H + h) * D;
  for (int64_t d = 0; d < D; ++d) qd[d] = elem_to_double(J->q, J->dtype, bshd(b, i, h, d, J->Sq, J->H, D));

  /* pass 1: scores of visible keys and their maximum */
  double m = -INFINITY;
  int64_t n = 0;
  for (int64_t j = 0; j < J->Sk; ++j) {
    if (!visible(J->causal, J->q_pos0, J->k_pos0, i, j, len_b)) {
      s[j] = -INFINITY;
      continue;
    }
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qd[d] * elem_to_double(J->k, J->dtype, bshd(b, j, h, d, J->Sk, J->H, D));
    s[j] = dot * J->scale;
    if (s[j] > m) m = s[j];
    ++n;
  }
  if (n == 0) {
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    J->lse[(size_t)r * J->H + h] = -INFINITY;
    return;
  }
  /* pass 2: exponentials, their sum, and the weighted sum of values */
  double l = 0.0;
  for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
  for (int64_t j = 0; j < J->Sk; ++j) {
    if (s[j] == -INFINITY) continue;
    double e = exp(s[j] - m);
    l += e;
    for (int64_t d = 0; d < D; ++d) acc[d] += e * elem_to_double(J->v, J->dtype, bshd(b, j, h, d, J->Sk, J->H, D));
  }
  for (int64_t d = 0; d < D; ++d) o[d] = acc[d] / l;
  J->lse[(size_t)r * J->H + h] = m + log(l);
}

static void* attn_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  double* s = (double*)malloc(sizeof(double) * (size_t)(J->Sk > 0 ? J->Sk : 1));
  double* qd = (double*)malloc(sizeof(double) * (size_t)J->D);
  double* acc = (double*)malloc(sizeof(double) * (size_t)J->D);
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t r = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (r >= J->n_rows) break;
    for (int64_t h = 0; h < J->H; ++h) attn_row(J, r, h, s, qd, acc);
  }
  free(s);
  free(qd);
  free(acc);
  return NULL;
}

static int pick_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/*
 * oracle_attention: for the listed query rows (flat index b*Sq + i; rows ==
 * NULL means every row in order) and every head h, writes
 *   out[r, h, :] = softmax over visible keys of (scale * q . k) applied to V
 *   lse[r, h]    = log of the softmax denominator (natural log)
 * Q is [B, Sq, H, D]; K and V are [B, Sk, H, D]; kv_len is [B] or NULL.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t Sq,
                     int64_t Sk, int64_t H, int64_t D, int causal, int64_t q_pos0, int64_t k_pos0,
                     const int32_t* kv_len, double scale, int64_t n_rows, const int64_t* rows,
                     double* out, double* lse, int nthreads) {
  if (!q || !k || !v || !out || !lse || B <= 0 || Sq <= 0 || Sk <= 0 || H <= 0 || D <= 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  if (!rows) n_rows = B * Sq;
  for (int64_t r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= B * Sq) return -1;
  attn_job J;
  memset(&J, 0, sizeof J);
  J.q = q, J.k = k, J.v = v, J.dtype = dtype;
  J.B = B, J.Sq = Sq, J.Sk = Sk, J.H = H, J.D = D;
  J.causal = causal, J.q_pos0 = q_pos0, J.k_pos0 = k_pos0, J.kv_len = kv_len, J.scale = scale;
  J.n_rows = n_rows, J.rows = rows, J.out = out, J.lse = lse, J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  int nt = pick_threads(nthreads);
  if (nt > n_rows) nt = (int)n_rows;
  if (nt < 1) nt = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int t = 1; t < nt; ++t) pthread_create(&th[t], NULL, attn_worker, &J);
  attn_worker(&J);
  for (int t = 1; t < nt; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/*
 * oracle_attention_bruteforce: a second, independent route to the same
 * result for tiny shapes.  Per (b, h) it materialises the whole score matrix,
 * sets hidden entries to -inf, exponentiates WITHOUT a max shift, normalises
 * each row by its sum to get the probability matrix P, then forms P V as a
 * dense matrix product.  P is written out ([B, H, Sq, Sk]) so row sums can
 * be checked.  Only safe where exp(score) does not overflow (tiny inputs).
 * out is [B, Sq, H, D]; lse is [B, H, Sq].
 */
int oracle_attention_bruteforce(const void* q, const void* k, const void* v, int dtype, int64_t B,
                                int64_t Sq, int64_t Sk, int64_t H, int64_t D, int causal,
                                int64_t q_pos0, int64_t k_pos0, const int32_t* kv_len, double scale,
                                double* out, double* lse, double* P) {
  if (!q || !k || !v || !out || !lse || !P || B <= 0 || Sq <= 0 || Sk <= 0 || H <= 0 || D <= 0) return -1;
  double* Sm = (double*)malloc(sizeof(double) * (size_t)(Sq * Sk));
  for (int64_t b = 0; b < B; ++b) {
    const int64_t len_b = clamp_len(kv_len, b, Sk);
    for (int64_t h = 0; h < H; ++h) {
      double* Pbh = P + (size_t)((b * H + h) * Sq * Sk);
      /* score matrix S = scale * Q K^T */
      for (int64_t i = 0; i < Sq; ++i)
        for (int64_t j = 0; j < Sk; ++j) {
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d)
            dot += elem_to_double(q, dtype, bshd(b, i, h, d, Sq, H, D)) *
                   elem_to_double(k, dtype, bshd(b, j, h, d, Sk, H, D));
          Sm[i * Sk + j] = visible(causal, q_pos0, k_pos0, i, j, len_b) ? dot * scale : -INFINITY;
        }
      /* P = exp(S) / rowsum(exp(S)); exp(-inf) = 0 */
      for (int64_t i = 0; i < Sq; ++i) {
        double z = 0.0;
        for (int64_t j = 0; j < Sk; ++j) z += exp(Sm[i * Sk + j]);
        for (int64_t j = 0; j < Sk; ++j) Pbh[i * Sk + j] = z > 0.0 ? exp(Sm[i * Sk + j]) / z : 0.0;
        lse[(size_t)((b * H + h) * Sq + i)] = log(z); /* log(0) = -inf */
      }
      /* out = P V */
      for (int64_t i = 0; i < Sq; ++i)
        for (int64_t d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int64_t j = 0; j < Sk; ++j)
            acc += Pbh[i * Sk + j] * elem_to_double(v, dtype, bshd(b, j, h, d, Sk, H, D));
          out[bshd(b, i, h, d, Sq, H, D)] = acc;
        }
    }
  }
  free(Sm);
  return 0;
}

/*
 * oracle_merge_lse: combines n partial attention results over disjoint key
 * sets into the result over their union (reading: log-sum-exp combination).
 * For each row (b, s, h):  M = max_k lse_k;  if M = -inf the row saw no key:
 * out = 0, lse = -inf.  Otherwise w_k = exp(lse_k - M), W = sum_k w_k,
 * out = sum_k (w_k / W) o_k, lse = M + log W.
 * o_parts[k] is [B, S, H, D]; lse_parts[k] is [B, H, S]; all double.
 */
int oracle_merge_lse(int n, const double* const* o_parts, const double* const* lse_parts, int64_t B,
                     int64_t S, int64_t H, int64_t D, double* out, double* lse_out) {
  if (n < 1 || !o_parts || !lse_parts || !out || !lse_out) return -1;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t s = 0; s < S; ++s)
      for (int64_t h = 0; h < H; ++h) {
        const size_t li = (size_t)((b * H + h) * S + s);
        double M = -INFINITY;
        for (int k = 0; k < n; ++k)
          if (lse_parts[k][li] > M) M = lse_parts[k][li];
        double* o = out + bshd(b, s, h, 0, S, H, D);
        if (M == -INFINITY) {
          for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
          lse_out[li] = -INFINITY;
          continue;
        }
        double W = 0.0;
        for (int k = 0; k < n; ++k) W += exp(lse_parts[k][li] - M);
        for (int64_t d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int k = 0; k < n; ++k)
            acc += exp(lse_parts[k][li] - M) / W * o_parts[k][bshd(b, s, h, d, S, H, D)];
          o[d] = acc;
        }
        lse_out[li] = M + log(W);
      }
  return 0;
}

/*
 * oracle_shard_permute: the local layout effect of the sequence-gather /
 * head-scatter all-to-all.  Shard i holds tokens [i*S/P, (i+1)*S/P) of the
 * sequence with all H heads ([B, S/P, H, D]); head group g is heads
 * [g*H/P, (g+1)*H/P).  out is [B, S, H/P, D]:
 *   out[b, i*S/P + t, hh, d] = shard_i[b, t, g*H/P + hh, d].
 * Element bytes are copied verbatim.
 */
int oracle_shard_permute(const void* const* shards, int P, int group, int64_t B, int64_t S, int64_t H,
                         int64_t D, int elem_bytes, void* out) {
  if (!shards || !out || P < 1 || group < 0 || group >= P || B <= 0 || S <= 0 || H <= 0 || D <= 0 ||
      elem_bytes <= 0 || S % P != 0 || H % P != 0)
    return -1;
  const int64_t Sl = S / P, Hl = H / P;
  for (int i = 0; i < P; ++i)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < Sl; ++t)
        for (int64_t hh = 0; hh < Hl; ++hh)
          for (int64_t d = 0; d < D; ++d) {
            size_t src = bshd(b, t, (int64_t)group * Hl + hh, d, Sl, H, D);
            size_t dst = bshd(b, (int64_t)i * Sl + t, hh, d, S, Hl, D);
            memcpy((char*)out + dst * (size_t)elem_bytes, (const char*)shards[i] + src * (size_t)elem_bytes,
                   (size_t)elem_bytes);
          }
  return 0;
}

/*
 * oracle_shard_unpermute: the inverse layout, the local effect of the
 * all-to-all that returns head-sharded output to sequence shards.  Given the
 * head-group outputs og[g] = [B, S, H/P, D] for all g, writes shard i as
 *   shard_i[b, t, g*H/P + hh, d] = og[g][b, i*S/P + t, hh, d].
 */
int oracle_shard_unpermute(const void* const* groups, int P, int64_t B, int64_t S, int64_t H, int64_t D,
                           int elem_bytes, void* const* shards) {
  if (!groups || !shards || P < 1 || B <= 0 || S <= 0 || H <= 0 || D <= 0 || elem_bytes <= 0 ||
      S % P != 0 || H % P != 0)
    return -1;
  const int64_t Sl = S / P, Hl = H / P;
  for (int g = 0; g < P; ++g)
    for (int i = 0; i < P; ++i)
      for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < Sl; ++t)
          for (int64_t hh = 0; hh < Hl; ++hh)
            for (int64_t d = 0; d < D; ++d) {
              size_t src = bshd(b, (int64_t)i * Sl + t, hh, d, S, Hl, D);
              size_t dst = bshd(b, t, (int64_t)g * Hl + hh, d, Sl, H, D);
              memcpy((char*)shards[i] + dst * (size_t)elem_bytes, (const char*)groups[g] + src * (size_t)elem_bytes,
                     (size_t)elem_bytes);
            }
  return 0;
}

/*
 * oracle_all_to_all: the local effect of an all-to-all with a scatter dim and a
 * gather dim ("Support deepspeed sequence parallel", PR body: the sequence
 * all-to-all is parameterised by a scatter index and a gather index, and
 * all_to_all_single replaces all_to_all).  Each of the P ranks holds a tensor of
 * shape `shape` (ndim dims, row-major); rank i splits its tensor into P equal
 * chunks along scatter_dim and sends chunk r to rank r; rank r concatenates what
 * it receives, in rank order, along gather_dim.  So rank r's result has
 * shape[scatter_dim] / P at scatter_dim and shape[gather_dim] * P at gather_dim,
 * and its element at index o (a multi-index) is input i's element at index o
 * with  o[gather_dim] replaced by o[gather_dim] - i * shape[gather_dim]  (i =
 * o[gather_dim] / shape[gather_dim])  and  o[scatter_dim] replaced by
 * r * shape[scatter_dim] / P + o[scatter_dim].  Written out per element with
 * multi-indices.  Returns 0, or -1 on a bad argument.
 */
int oracle_all_to_all(const void* const* inputs, int P, int rank, int ndim, const int64_t* shape, int scatter_dim,
                      int gather_dim, int elem_bytes, void* out) {
  if (!inputs || !out || !shape || P < 1 || rank < 0 || rank >= P || ndim < 1 || ndim > 8 || elem_bytes <= 0)
    return -1;
  if (scatter_dim < 0 || scatter_dim >= ndim || gather_dim < 0 || gather_dim >= ndim || scatter_dim == gather_dim)
    return -1;
  int64_t in_shape[8], out_shape[8], total = 1;
  for (int d = 0; d < ndim; ++d) {
    if (shape[d] <= 0) return -1;
    in_shape[d] = out_shape[d] = shape[d];
    total *= shape[d];
  }
  if (in_shape[scatter_dim] % P != 0) return -1;
  out_shape[scatter_dim] = in_shape[scatter_dim] / P;
  out_shape[gather_dim] = in_shape[gather_dim] * P;
  int64_t o[8], src[8];
  for (int64_t e = 0; e < total; ++e) { /* output elements in row-major order (P * total/P of them) */
    int64_t rem = e;
    for (int d = ndim - 1; d >= 0; --d) {
      o[d] = rem % out_shape[d];
      rem /= out_shape[d];
    }
    const int64_t i = o[gather_dim] / in_shape[gather_dim];
    for (int d = 0; d < ndim; ++d) src[d] = o[d];
    src[gather_dim] = o[gather_dim] - i * in_shape[gather_dim];
    src[scatter_dim] = (int64_t)rank * out_shape[scatter_dim] + o[scatter_dim];
    int64_t flat = 0;
    for (int d = 0; d < ndim; ++d) flat = flat * in_shape[d] + src[d];
    memcpy((char*)out + (size_t)e * (size_t)elem_bytes, (const char*)inputs[i] + (size_t)flat * (size_t)elem_bytes,
           (size_t)elem_bytes);
  }
  return 0;
}

/* ---- attention backward (the vector-Jacobian product of attention) ------ */

/*
 * The gradients of a scalar loss L through attention, given dout = dL/dout.
 * Nothing on the pages writes these out; they are the derivative of the forward
 * definition above (reading: the chain rule through softmax), which is what the
 * pages' training workloads ("Support deepspeed sequence parallel", a training
 * script; "关于数据分割和合并", the gradient of the attention output) need.
 * Per (b, h), over visible pairs (i, j) only:
 *   P_ij  = softmax_j(s_i),  s_ij = scale * q_i . k_j
 *   dV_j  = sum_i P_ij dout_i
 *   dP_ij = dout_i . v_j
 *   dS_ij = P_ij * (dP_ij - sum_l P_il dP_il)       (Jacobian of softmax)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * A query row with no visible key contributes nothing (its output is the
 * constant 0).
 */
typedef struct {
  const void *q, *k, *v, *dout;
  int dtype;
  int64_t B, Sq, Sk, H, D;
  int causal;
  int64_t q_pos0, k_pos0;
  const int32_t* kv_len;
  double scale;
  double *dq, *dk, *dv; /* [B,Sq,H,D], [B,Sk,H,D], [B,Sk,H,D] */
  int64_t next;         /* work counter over (b, h), guarded by mu */
  pthread_mutex_t mu;
} bwd_job;

static double qkv(const bwd_job* J, const void* t, int64_t b, int64_t s, int64_t S, int64_t h, int64_t d) {
  return elem_to_double(t, J->dtype, bshd(b, s, h, d, S, J->H, J->D));
}

/* All query rows of one (b, h); dk / dv of this (b, h) are owned by the caller's thread. */
static void bwd_head(bwd_job* J, int64_t b, int64_t h, double* P, double* dP) {
  const int64_t Sq = J->Sq, Sk = J->Sk, D = J->D;
  const int64_t len_b = clamp_len(J->kv_len, b, Sk);
  for (int64_t i = 0; i < Sq; ++i) {
    /* the softmax row P_i (two passes: max, then normalised exponentials) */
    double m = -INFINITY;
    for (int64_t j = 0; j < Sk; ++j) {
      if (!visible(J->causal, J->q_pos0, J->k_pos0, i, j, len_b)) {
        P[j] = -INFINITY;
        continue;
      }
      double dot = 0.0;
      for (int64_t d = 0; d < D; ++d) dot += qkv(J, J->q, b, i, Sq, h, d) * qkv(J, J->k, b, j, Sk, h, d);
      P[j] = dot * J->scale;
      if (P[j] > m) m = P[j];
    }
    for (int64_t d = 0; d < D; ++d) J->dq[bshd(b, i, h, d, Sq, J->H, D)] = 0.0;
    if (m == -INFINITY) continue; /* no visible key */
    double z = 0.0;
    for (int64_t j = 0; j < Sk; ++j) z += P[j] == -INFINITY ? 0.0 : exp(P[j] - m);
    for (int64_t j = 0; j < Sk; ++j) P[j] = P[j] == -INFINITY ? 0.0 : exp(P[j] - m) / z;
    /* dP_ij = dout_i . v_j and the row's sum_l P_il dP_il */
    double delta = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
      if (P[j] == 0.0) {
        dP[j] = 0.0;
        continue;
      }
      double dot = 0.0;
      for (int64_t d = 0; d < D; ++d) dot += qkv(J, J->dout, b, i, Sq, h, d) * qkv(J, J->v, b, j, Sk, h, d);
      dP[j] = dot;
      delta += P[j] * dot;
    }
    for (int64_t j = 0; j < Sk; ++j) {
      if (P[j] == 0.0) continue;
      const double ds = P[j] * (dP[j] - delta);
      for (int64_t d = 0; d < D; ++d) {
        J->dq[bshd(b, i, h, d, Sq, J->H, D)] += J->scale * ds * qkv(J, J->k, b, j, Sk, h, d);
        J->dk[bshd(b, j, h, d, Sk, J->H, D)] += J->scale * ds * qkv(J, J->q, b, i, Sq, h, d);
        J->dv[bshd(b, j, h, d, Sk, J->H, D)] += P[j] * qkv(J, J->dout, b, i, Sq, h, d);
      }
    }
  }
}

static void* bwd_worker(void* arg) {
  bwd_job* J = (bwd_job*)arg;
  double* P = (double*)malloc(sizeof(double) * (size_t)J->Sk);
  double* dP = (double*)malloc(sizeof(double) * (size_t)J->Sk);
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= J->B * J->H) break;
    bwd_head(J, w / J->H, w % J->H, P, dP);
  }
  free(P);
  free(dP);
  return NULL;
}

/*
 * oracle_attention_backward: dq [B,Sq,H,D], dk and dv [B,Sk,H,D] (double, overwritten) for
 * inputs q [B,Sq,H,D], k, v [B,Sk,H,D] and dout [B,Sq,H,D] of element type dtype, with the
 * same masks, positions and scale as oracle_attention.  Returns 0, or -1 on a bad argument.
 */
int oracle_attention_backward(const void* q, const void* k, const void* v, const void* dout, int dtype,
                              int64_t B, int64_t Sq, int64_t Sk, int64_t H, int64_t D, int causal,
                              int64_t q_pos0, int64_t k_pos0, const int32_t* kv_len, double scale,
                              double* dq, double* dk, double* dv, int nthreads) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv || B <= 0 || Sq <= 0 || Sk <= 0 || H <= 0 || D <= 0)
    return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  for (size_t i = 0; i < (size_t)(B * Sk * H * D); ++i) dk[i] = dv[i] = 0.0;
  bwd_job J;
  memset(&J, 0, sizeof J);
  J.q = q, J.k = k, J.v = v, J.dout = dout, J.dtype = dtype;
  J.B = B, J.Sq = Sq, J.Sk = Sk, J.H = H, J.D = D;
  J.causal = causal, J.q_pos0 = q_pos0, J.k_pos0 = k_pos0, J.kv_len = kv_len, J.scale = scale;
  J.dq = dq, J.dk = dk, J.dv = dv, J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  int nt = pick_threads(nthreads);
  if (nt > B * H) nt = (int)(B * H);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int t = 1; t < nt; ++t) pthread_create(&th[t], NULL, bwd_worker, &J);
  bwd_worker(&J);
  for (int t = 1; t < nt; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

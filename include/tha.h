/*
 * tha.h -- C ABI of libtha.so: one MI355X's share of multi-head scaled
 * dot-product attention under sequence and head parallelism.
 *
 * What the calls compute (pages, by title and section):
 *  - attention per head: out = softmax(Q K^T * scale + mask) V, with
 *    scale = 1/sqrt(head_dim) by default ("Megatron-LM - Training
 *    Multi-Billion Parameter Language Models Using Model Parallelism", the
 *    linear-algebra-of-attention section; "adv07: Sequence Parallel", Q4;
 *    "parallel multi-head attention", section 3.2);
 *  - the Ulysses local layout: sequence shards -> one head group over the
 *    whole sequence ("adv07: Sequence Parallel", section 5, DeepSpeed Ulysses;
 *    the all-to-all described as a transpose in the issue thread
 *    "关于数据分割和合并" of long-context-attention);
 *  - the Ring local step: attention of one Q chunk against one KV chunk at
 *    global positions, blocks accumulated into the full result ("adv07:
 *    Sequence Parallel", Q5 and section 5, Ring Attention).
 *
 * Conventions shared by every call:
 *  - Tensors are contiguous, row-major [batch, seq, heads, head_dim]
 *    ("parallel multi-head attention" section 3.2; the [b, s/p, n, h] input
 *    of "Support deepspeed sequence parallel"), head_dim fastest.
 *    Per-row log-sum-exp tensors are [batch, heads, seq] float32.
 *  - Every tensor pointer is a DEVICE pointer on the current HIP device.
 *    Arrays of pointers (o_parts, lse_parts, shards) are HOST arrays holding
 *    device pointers; the library copies them into kernel arguments, so the
 *    host arrays may be freed as soon as the call returns.
 *  - The caller allocates and owns every buffer.  The library allocates no
 *    memory and keeps no state between calls; calls are safe from several
 *    host threads.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream).  Outputs are valid once the stream has reached the call.
 *  - Return value: THA_OK, or a negative tha_status.  Argument errors are
 *    detected on the host before anything is enqueued (no HIP call is made).
 *    THA_ERR_HIP means a launch failed; faults inside a kernel surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 *  - Outputs must not overlap inputs unless a call says otherwise.
 */
#ifndef THA_H
#define THA_H

#ifdef __cplusplus
extern "C" {
#endif

#define THA_API __attribute__((visibility("default")))

typedef enum {
  THA_OK = 0,
  THA_ERR_INVALID = -1,     /* null pointer, non-positive size, inconsistent sizes */
  THA_ERR_UNSUPPORTED = -2, /* a valid request this build does not implement */
  THA_ERR_HIP = -3,         /* a HIP launch failed */
  THA_ERR_TOO_LARGE = -4    /* exceeds the fixed scratch capacity of a no-allocation entry point */
} tha_status;

/* Element types. */
enum { THA_F32 = 0, THA_BF16 = 1 };

/* attn_fwd mask flags (combinable). */
enum {
  THA_MASK_NONE = 0,
  THA_MASK_CAUSAL = 1,     /* key visible iff k_pos0 + j <= q_pos0 + i ("adv07: Sequence Parallel", Q4) */
  THA_MASK_KEY_PADDING = 2, /* key j of sequence b visible iff j < kv_len[b] ("Support deepspeed
                               sequence parallel": the mask is 'token is not padding') */
  THA_ACCUMULATE = 4,        /* attn_fwd_ex only: merge into the running (o, lse), see there */
  /* attn_fwd_ex only: force the kernel of the bf16, head-size-128 path (see attn_fwd); a 3-bit
     field, 0 = automatic choice.  Ignored for other dtypes and head sizes. */
  THA_KERNEL_AUTO = 0,
  THA_KERNEL_NARROW = 1 << 3,
  THA_KERNEL_WIDE = 2 << 3,
  THA_KERNEL_SPLIT = 3 << 3,
  THA_KERNEL_SPLIT64 = 4 << 3,
  THA_KERNEL_MASK = 7 << 3
};

/* Largest pointer arrays accepted by attn_merge_lse and the permutes. */
#define THA_MAX_PARTS 64
#define THA_MAX_SHARDS 64
/* Most tensors one shard_permute_n / shard_unpermute_n call moves. */
#define THA_MAX_PERMUTE_TENSORS 4
/* Largest B*H*Sq that attn_bwd_noalloc takes (its fixed Delta scratch, 16 MiB per device). */
#define THA_NOALLOC_MAX_DELTA (4 * 1024 * 1024)

/*
 * attn_fwd -- attention of every query row against the visible keys, per head.
 *
 *   q      [B, Sq, H, D] of in_dt         k, v   [B, Sk, H, D] of in_dt
 *   o      [B, Sq, H, D] of out_dt        lse    [B, H, Sq] float32, or NULL
 *
 * For batch b, head h and query row i, with s_j = scale * (q_i . k_j) over the
 * visible keys j:  o_i = sum_j softmax(s)_j v_j,  lse_i = log(sum_j exp(s_j))
 * (natural log).  Masked keys get weight exactly 0.  A row with no visible key
 * gets o_i = 0 and lse_i = -inf, so that partial results over disjoint key
 * blocks can be combined with attn_merge_lse.
 *
 * mask_flags: THA_MASK_CAUSAL and/or THA_MASK_KEY_PADDING.  q_pos0 / k_pos0 are
 * the global sequence positions of query row 0 and key 0 (global position ids,
 * as in the data collator of "Support deepspeed sequence parallel"); they only
 * matter with THA_MASK_CAUSAL, and only through q_pos0 - k_pos0 (any values
 * with |q_pos0|, |k_pos0| < 2^62 are exact).  kv_len: device int32 [B], required iff
 * THA_MASK_KEY_PADDING (values are clamped to [0, Sk] on the device).
 * scale: multiplies q.k, finite and > 0; pass 1/sqrt(D) for standard attention.
 *
 * Supported: in_dt = THA_BF16 with D = 64 or 128 (matrix-core path: bf16
 * products, fp32 accumulation and softmax, probabilities rounded to bf16 before
 * the product with V, as the forward pass of "parallel multi-head attention"
 * section 3.2 casts the fp32 softmax back to the input type);
 * in_dt = THA_F32 with 1 <= D <= 256 (fp32 throughout).  out_dt may be THA_BF16
 * or THA_F32 in both cases (fp32 output keeps ring partials unrounded).
 * Kernel choice for bf16, D = 128, by grid size: a wide kernel (256 query rows per
 * workgroup) when its grid holds at least two workgroups per compute unit, else a
 * narrow one (128 rows) when its grid does, else the narrow kernel in a split form
 * (two wavefront groups per workgroup on the two halves of the key range, merged by
 * log-sum-exp before the output is written): on 64-row query tiles (THA_KERNEL_SPLIT64)
 * when 128-row tiles would leave half the compute units idle, or when the mask is
 * causal, the 128-row tiles are no more than the compute units and the last of them
 * needs at least twice the keys of the first (the 64-row tiles, launched heaviest
 * first, even out the units' loads); else on 128-row tiles (THA_KERNEL_SPLIT).
 * All four compute the same function; the wide and narrow kernels give identical
 * bits, the split forms differ from them and from each other only by where the key
 * range is halved (within the stated tolerances).
 * The automatic choice depends on B*H, Sq, the causal extent (mask, Sq, Sk and
 * q_pos0 - k_pos0) and the device's compute-unit count, so the
 * same rows computed by calls of different sizes (a query split, a Ring chunk against
 * the whole call) may differ in the last bits when the calls take different forms;
 * calls that take the same form give the same bits for the same rows.  attn_fwd_ex's
 * THA_KERNEL_* flags force one form for every size.
 * Errors: THA_ERR_INVALID for null q/k/v/o, non-positive sizes, unknown mask
 * bits, KEY_PADDING without kv_len, scale not finite and positive, |q_pos0| or |k_pos0| >=
 * 2^62; THA_ERR_UNSUPPORTED for other dtypes / head dims.
 */
THA_API int attn_fwd(const void* q, const void* k, const void* v, void* o, int out_dt, float* lse, int B, int Sq,
             int Sk, int H, int D, int in_dt, unsigned mask_flags, long long q_pos0, long long k_pos0,
             const int* kv_len, float scale, void* stream);

/*
 * attn_fwd_ex -- attn_fwd with explicit tensor strides and an optional fused Ring step.
 *
 * strides: NULL (contiguous [B,S,H,D] tensors, as attn_fwd) or 8 element strides
 *   { q_batch, q_token, k_batch, k_token, v_batch, v_token, o_batch, o_token }:
 *   element (b, s, h, d) of q lives at q[b*q_batch + s*q_token + h*D + d], and likewise for k,
 *   v and o (heads contiguous at stride D inside a token, dims contiguous).  This takes the
 *   packed-QKV layout [B,S,3,H,D] ("Megatron-LM ..." notes and "关于数据分割和合并": separate or
 *   packed Q/K/V inputs) as three views (token stride 3*H*D) and head-subset views of a wider
 *   tensor (token stride H_total*D) without copies.  Requirements: every token stride >= H*D and
 *   <= 2^24; with B > 1 every batch stride >= (tokens of that tensor) * token stride (no
 *   overlap); k_token == v_token (THA_ERR_UNSUPPORTED otherwise); on the bf16 path q, k, v
 *   16-byte aligned with strides multiples of 8 elements, o 8-byte (bf16) or 16-byte (fp32)
 *   aligned with strides multiples of 4 elements (THA_ERR_UNSUPPORTED otherwise).
 *
 * flags: the mask flags of attn_fwd, plus THA_ACCUMULATE and a THA_KERNEL_* value (bf16, D = 128
 *   only: THA_KERNEL_NARROW, _WIDE or _SPLIT forces that form of the kernel instead of the
 *   automatic choice described at attn_fwd, e.g. to get bit-identical rows from calls of different
 *   sizes).  With THA_ACCUMULATE, o (out_dt must
 *   be THA_F32) and lse (required) hold a running result over other keys, and this call merges
 *   its own result into them in place by the log-sum-exp rule of attn_merge_lse (the Ring step
 *   that accumulates block results into the full attention, "adv07: Sequence Parallel" Q5),
 *   with no separate partial buffers or merge pass.  A row whose running lse is -inf counts as
 *   having no keys yet: its o is not read (so a Ring pass may start from lse = -inf and any o).
 *   Calls that overlap on the same rows of o / lse race.
 * Other arguments, results and errors as attn_fwd; THA_ERR_INVALID also for THA_ACCUMULATE
 * with a bf16 o or a null lse.
 */
THA_API int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, int out_dt, float* lse, int B, int Sq,
                int Sk, int H, int D, int in_dt, unsigned flags, long long q_pos0, long long k_pos0,
                const int* kv_len, float scale, const long long* strides, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd with respect to q, k and v for the cotangent
 * dout = dL/do.  The pages' workloads are training ("Support deepspeed sequence
 * parallel", a training script; "关于数据分割和合并", the gradient of the attention
 * output); the formulas are the chain rule through attn_fwd's softmax (a reading:
 * the pages do not write them out).  With P the softmax of attn_fwd (same masks,
 * positions and scale), dP_ij = dout_i . v_j and Delta_i = dout_i . o_i:
 *   dv_j += sum_i P_ij dout_i
 *   dq_i += scale * sum_j P_ij (dP_ij - Delta_i) k_j
 *   dk_j += scale * sum_i P_ij (dP_ij - Delta_i) q_i
 * o and lse must be attn_fwd's output and lse of the same query rows over their
 * FULL key set (for a Ring share: the merged o and lse), so that P is recovered
 * exactly as exp(scale q.k - lse) and Delta_i equals sum_j P_ij dP_ij.
 *
 * q, o, dout: [B,Sq,H,D]; k, v: [B,Sk,H,D], all of element type in_dt; lse
 * [B,H,Sq] fp32.  dq [B,Sq,H,D], dk and dv [B,Sk,H,D] are fp32 and ACCUMULATED
 * into: zero them for a plain backward; the steps of a Ring share add their
 * partial gradients into the same buffers.  workspace: device fp32 array of at
 * least B*H*Sq elements owned by the caller, overwritten (it holds Delta).
 * Masks, positions, kv_len and scale as in attn_fwd.
 * Supported: in_dt = THA_BF16 with D = 64 or 128 (matrix-core path: bf16
 * products with fp32 accumulation, P and dS rounded to bf16 as operands of the
 * products that consume them); in_dt = THA_F32 with 1 <= D <= 256 (fp32
 * throughout).
 * Errors: as attn_fwd, plus THA_ERR_INVALID for a null o, dout, lse, dq, dk, dv
 * or workspace; on the bf16 path THA_ERR_UNSUPPORTED when q, k, v, dout, dq, dk or dv
 * is not 16-byte aligned (the kernels move 16-byte vectors).
 */
THA_API int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             float* dq, float* dk, float* dv, float* workspace, int B, int Sq, int Sk, int H, int D, int in_dt,
             unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len, float scale, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and errors as attn_bwd without the workspace: Delta lives in a scratch array the library keeps
 * in device memory, THA_NOALLOC_MAX_DELTA floats (16 MiB) per device for the life of the process.
 * The call allocates nothing (no hipMalloc / hipFree and no allocating library routine).
 * B*H*Sq above THA_NOALLOC_MAX_DELTA returns THA_ERR_TOO_LARGE (checked on the host before any HIP
 * call).  Every call on a device shares that device's scratch array (it is fully rewritten by each
 * call before it is read), so calls that overlap on one device -- on different streams or from
 * different host threads without ordering -- race; calls on different devices do not.
 */
THA_API int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, float* dq, float* dk, float* dv, int B, int Sq, int Sk, int H, int D,
                             int in_dt, unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len,
                             float scale, void* stream);

/*
 * attn_merge_lse -- combine n partial attention results over disjoint key
 * sets into the result over their union (the Ring step "accumulate block
 * results into the full attention", "adv07: Sequence Parallel" Q5; the
 * combination rule itself is the standard log-sum-exp one, a reading):
 *   M = max_k lse_k;  w_k = exp(lse_k - M);  o = sum_k w_k o_k / sum_k w_k;
 *   lse = M + log(sum_k w_k);  rows where every lse_k = -inf give o = 0,
 *   lse = -inf.
 *
 *   o_parts   host array of n_parts device pointers, each [B, S, H, D] of part_dt
 *   lse_parts host array of n_parts device pointers, each [B, H, S] float32
 *   o_out     [B, S, H, D] of out_dt; may be any o_parts[k] when part_dt == out_dt
 *             (in place: each element is written by the thread that read it
 *             from every part)
 *   lse_out   [B, H, S] float32 or NULL; may be any lse_parts[k] (a row's lse
 *             values are all read before its one lse store)
 * Partial overlaps between o_out and a part are not allowed.
 * 1 <= n_parts <= THA_MAX_PARTS; part_dt, out_dt in {THA_F32, THA_BF16}.
 * Errors: THA_ERR_INVALID for null pointers, n_parts out of range,
 * non-positive sizes, or o_out equal to an o_parts[k] with differing dtypes;
 * THA_ERR_UNSUPPORTED for other dtypes.
 */
THA_API int attn_merge_lse(int n_parts, const void* const* o_parts, const float* const* lse_parts, int part_dt,
                   void* o_out, int out_dt, float* lse_out, int B, int S, int H, int D, void* stream);

/*
 * shard_permute -- the local layout effect of the Ulysses all-to-all that
 * gathers the sequence and scatters heads ("adv07: Sequence Parallel" section
 * 5, DeepSpeed Ulysses: each device computes its heads over all positions;
 * the issue thread "关于数据分割和合并" calls it a transpose).  Shard i holds
 * tokens [i*S/P, (i+1)*S/P) with all H heads (the per-rank slices of the data
 * collator in "Support deepspeed sequence parallel"); head group g is heads
 * [g*H/P, (g+1)*H/P) (whole heads per device, "parallel multi-head attention"
 * sections 2.2 and 3.1).
 *
 *   shards  host array of P device pointers, each [B, S/P, H, D]
 *   out     [B, S, H/P, D]:  out[b, i*S/P + t, hh, d] = shard_i[b, t, g*H/P + hh, d]
 * elem_bytes in {1, 2, 4, 8}; bytes are copied verbatim (bit-exact).
 * Errors: THA_ERR_INVALID for null pointers, P outside [1, THA_MAX_SHARDS],
 * group outside [0, P), S or H not divisible by P, non-positive sizes;
 * THA_ERR_UNSUPPORTED for other elem_bytes.
 */
THA_API int shard_permute(const void* const* shards, int P, int group, void* out, int B, int S, int H, int D,
                  int elem_bytes, void* stream);

/*
 * shard_unpermute -- the inverse layout (the all-to-all that returns each
 * device's heads to sequence shards after attention, issue thread
 * "关于数据分割和合并": outputs stay sequence-sharded, (bs, seqlen/N, hidden)).
 *
 *   in      [B, S, H/P, D], head group `group` over the whole sequence
 *   shards  host array of P device pointers, each [B, S/P, H, D]; only the
 *           heads of `group` are written:
 *           shard_i[b, t, g*H/P + hh, d] = in[b, i*S/P + t, hh, d]
 * Same argument rules and errors as shard_permute.
 */
THA_API int shard_unpermute(const void* in, int P, int group, void* const* shards, int B, int S, int H, int D,
                    int elem_bytes, void* stream);

/*
 * shard_permute_n / shard_unpermute_n -- shard_permute / shard_unpermute of n tensors of the same
 * shape and element size in one launch (Q, K and V of a Ulysses step: "adv07: Sequence Parallel"
 * section 5, one all-to-all per tensor), with the tensors' address streams interleaved.  Results
 * are those of n separate calls, bit for bit.
 *
 *   shards  host array of n*P device pointers, tensor-major: shards[t*P + i] is shard i of tensor t
 *   outs / ins  host array of n device pointers, the grouped tensors [B, S, H/P, D]
 * 1 <= n <= THA_MAX_PERMUTE_TENSORS; otherwise the arguments, rules and errors of shard_permute
 * (THA_ERR_INVALID also for n out of range or a null entry in either array).
 */
THA_API int shard_permute_n(int n, const void* const* shards, int P, int group, void* const* outs, int B, int S,
                            int H, int D, int elem_bytes, void* stream);
THA_API int shard_unpermute_n(int n, const void* const* ins, int P, int group, void* const* shards, int B, int S,
                              int H, int D, int elem_bytes, void* stream);

/*
 * shard_all_to_all -- the local layout of an all-to-all with a general scatter dim and gather
 * dim ("Support deepspeed sequence parallel", PR body: the sequence all-to-all takes a scatter
 * index and a gather index, and uses all_to_all_single into one contiguous output).  Each of P
 * ranks holds a tensor of shape `shape`; rank i splits it into P equal chunks along scatter_dim
 * and sends chunk r to rank r; rank r concatenates the chunks it receives, in rank order, along
 * gather_dim.  This call computes what rank `rank` holds afterwards, from all P tensors:
 *
 *   inputs  host array of P device pointers, each a contiguous row-major tensor of `shape`
 *   shape   host array of ndim sizes (1 <= ndim <= 8), every size >= 1
 *   out     contiguous, of `shape` with shape[scatter_dim] / P at scatter_dim and
 *           shape[gather_dim] * P at gather_dim:
 *           out[.., i*shape[gather_dim] + t (gather_dim), .., hh (scatter_dim), ..]
 *             = inputs[i][.., t, .., rank*shape[scatter_dim]/P + hh, ..]
 *
 * The Ulysses cases on [B, S, H, D]: scatter_dim 2, gather_dim 1 is shard_permute (the inputs
 * are the sequence shards); scatter_dim 1, gather_dim 2 is the return all-to-all (the inputs are
 * the P ranks' [B, S, H/P, D] head-group tensors, the result rank r's sequence shard).  A
 * sequence-first layout [S, B, H, D] is scatter_dim 2, gather_dim 0; packed QKV [B, S, 3, H, D]
 * is scatter_dim 3, gather_dim 1.  Bytes are copied verbatim (bit-exact); elem_bytes in
 * {1, 2, 4, 8}.  out must not overlap any input.
 * Errors: THA_ERR_INVALID for null pointers, P outside [1, THA_MAX_SHARDS], rank outside
 * [0, P), ndim outside [1, 8], a size < 1, scatter_dim or gather_dim outside [0, ndim) or equal,
 * shape[scatter_dim] not divisible by P, or more than 2^48 elements per tensor;
 * THA_ERR_UNSUPPORTED for other elem_bytes.
 */
THA_API int shard_all_to_all(const void* const* inputs, int P, int rank, void* out, int ndim, const long long* shape,
                             int scatter_dim, int gather_dim, int elem_bytes, void* stream);

/* Static description of a status code (never NULL). */
THA_API const char* tha_status_string(int status);

/* Library ABI version (major * 100 + minor): 101 adds shard_permute_n, shard_unpermute_n,
   shard_all_to_all, attn_bwd_noalloc, THA_ERR_TOO_LARGE and the THA_KERNEL_* flags of attn_fwd_ex. */
THA_API int tha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* THA_H */

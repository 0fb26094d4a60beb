// api.hip -- the C ABI of libtha.so (declared in include/tha.h): argument
// validation on the host, then dispatch to the kernel launchers.  Validation
// runs before any HIP call, so every argument error is reported without
// touching a device.
#include <math.h>
#include <stdint.h>

#include "tha.h"
#include "tha_kernels.h"

namespace {

constexpr long long kMaxPos = 1LL << 62;
constexpr int64_t kMaxRowElems = 1LL << 24;  // H*D per token: tile offsets stay 32-bit

int hip_status(hipError_t e) { return e == hipSuccess ? THA_OK : THA_ERR_HIP; }

// Causal visibility depends on the positions only through their difference: key j is visible to
// query row i iff j - i <= q_pos0 - k_pos0.  The kernels receive that difference as q_pos0 (with
// k_pos0 = 0), clamped to +-2^40, far beyond any row or key index (< 2^31), so the visible sets
// are unchanged and the kernels' 64-bit index sums (position + index) cannot overflow.
constexpr long long kPosDiffClamp = 1LL << 40;
long long pos_diff(long long q_pos0, long long k_pos0) {  // |q_pos0|, |k_pos0| < 2^62: no overflow
  const long long d = q_pos0 - k_pos0;
  return d > kPosDiffClamp ? kPosDiffClamp : (d < -kPosDiffClamp ? -kPosDiffClamp : d);
}

bool dtype_ok(int dt) { return dt == THA_F32 || dt == THA_BF16; }

// Elements per token of a contiguous [B, S, H, D] tensor, for the default strides; sizes that the
// checks reject get 1, so forming the strides cannot overflow before they are rejected.
long long contiguous_row(int H, int D) {
  const long long hd = (long long)H * D;  // both int: no overflow in 64 bits
  return (H > 0 && D > 0 && hd <= kMaxRowElems) ? hd : 1;
}

// Checks of the permute calls (n tensors), filling the kernel's pointer block.
int check_permute_n(int n, const void* const* shards, int P, int group, const void* const* grouped, int B, int S,
                    int H, int D, int elem_bytes, tha::MultiShardPtrs& mp) {
  if (!grouped || !shards) return THA_ERR_INVALID;
  if (n < 1 || n > THA_MAX_PERMUTE_TENSORS) return THA_ERR_INVALID;
  if (P < 1 || P > THA_MAX_SHARDS) return THA_ERR_INVALID;
  if (group < 0 || group >= P) return THA_ERR_INVALID;
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return THA_ERR_INVALID;
  if (S % P != 0 || H % P != 0) return THA_ERR_INVALID;
  mp = tha::MultiShardPtrs{};
  for (int t = 0; t < n; ++t) {
    if (!grouped[t]) return THA_ERR_INVALID;
    mp.grouped[t] = const_cast<void*>(grouped[t]);
    for (int i = 0; i < P; ++i) {
      if (!shards[t * P + i]) return THA_ERR_INVALID;
      mp.shard[t][i] = const_cast<void*>(shards[t * P + i]);
    }
  }
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return THA_ERR_UNSUPPORTED;
  if ((int64_t)H * D > kMaxRowElems) return THA_ERR_UNSUPPORTED;
  return THA_OK;
}

}  // namespace

namespace tha {

int attn_bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   const float* dq, const float* dk, const float* dv, int B, int Sq, int Sk, int H, int D, int in_dt,
                   unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len, float scale) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return THA_ERR_INVALID;
  if (B <= 0 || Sq <= 0 || Sk <= 0 || H <= 0 || D <= 0) return THA_ERR_INVALID;
  if (mask_flags & ~(unsigned)(THA_MASK_CAUSAL | THA_MASK_KEY_PADDING)) return THA_ERR_INVALID;
  if ((mask_flags & THA_MASK_KEY_PADDING) && !kv_len) return THA_ERR_INVALID;
  if (!isfinite(scale) || !(scale > 0.f)) return THA_ERR_INVALID;
  if (q_pos0 >= kMaxPos || q_pos0 <= -kMaxPos || k_pos0 >= kMaxPos || k_pos0 <= -kMaxPos) return THA_ERR_INVALID;
  if (!dtype_ok(in_dt)) return THA_ERR_UNSUPPORTED;
  if ((int64_t)H * D > kMaxRowElems) return THA_ERR_UNSUPPORTED;
  if (in_dt == THA_BF16 && D != 128 && D != 64) return THA_ERR_UNSUPPORTED;
  if (in_dt == THA_F32 && D > 256) return THA_ERR_UNSUPPORTED;
  if (in_dt == THA_BF16) {  // 16-byte loads of q, k, v, dout and 16-byte read-modify-writes of dq, dk, dv
    const void* p16[7] = {q, k, v, dout, dq, dk, dv};
    for (const void* p : p16)
      if ((uintptr_t)p % 16) return THA_ERR_UNSUPPORTED;
  }
  return THA_OK;
}

int attn_bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    float* dq, float* dk, float* dv, float* delta, int B, int Sq, int Sk, int H, int D, int in_dt,
                    unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len, float scale,
                    void* stream) {
  AttnBwdArgs a;
  a.q = q, a.k = k, a.v = v, a.o = o, a.dout = dout, a.lse = lse;
  a.dq = dq, a.dk = dk, a.dv = dv, a.delta = delta;
  a.kv_len = (mask_flags & THA_MASK_KEY_PADDING) ? kv_len : nullptr;
  a.B = B, a.Sq = Sq, a.Sk = Sk, a.H = H, a.D = D;
  a.causal = (mask_flags & THA_MASK_CAUSAL) != 0;
  a.q_pos0 = pos_diff(q_pos0, k_pos0), a.k_pos0 = 0;
  a.scale = scale;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_attn_bwd_delta(a, in_dt, st);
  if (e != hipSuccess) return THA_ERR_HIP;
  return hip_status(in_dt == THA_BF16 ? launch_attn_bwd_bf16(a, st) : launch_attn_bwd_f32(a, st));
}

}  // namespace tha

extern "C" {

int tha_version(void) { return 101; }

const char* tha_status_string(int status) {
  switch (status) {
    case THA_OK: return "ok";
    case THA_ERR_INVALID: return "invalid argument";
    case THA_ERR_UNSUPPORTED: return "unsupported dtype, head dim or size";
    case THA_ERR_HIP: return "HIP launch failed";
    case THA_ERR_TOO_LARGE: return "request exceeds the fixed scratch capacity of a no-allocation entry point";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Shared body of attn_fwd and attn_fwd_ex; st8: {q_bs, q_rs, k_bs, k_rs, v_bs, v_rs, o_bs, o_rs}.
int fwd_common(const void* q, const void* k, const void* v, void* o, int out_dt, float* lse, int B, int Sq, int Sk,
               int H, int D, int in_dt, unsigned flags, long long q_pos0, long long k_pos0, const int* kv_len,
               float scale, const long long* st8, void* stream) {
  if (!q || !k || !v || !o) return THA_ERR_INVALID;
  if (B <= 0 || Sq <= 0 || Sk <= 0 || H <= 0 || D <= 0) return THA_ERR_INVALID;
  if (flags & ~(unsigned)(THA_MASK_CAUSAL | THA_MASK_KEY_PADDING | THA_ACCUMULATE | THA_KERNEL_MASK))
    return THA_ERR_INVALID;
  const unsigned kernel = flags & THA_KERNEL_MASK;
  if (kernel > THA_KERNEL_SPLIT64) return THA_ERR_INVALID;
  if ((flags & THA_MASK_KEY_PADDING) && !kv_len) return THA_ERR_INVALID;
  if (!isfinite(scale) || !(scale > 0.f)) return THA_ERR_INVALID;
  if (q_pos0 >= kMaxPos || q_pos0 <= -kMaxPos || k_pos0 >= kMaxPos || k_pos0 <= -kMaxPos) return THA_ERR_INVALID;
  const bool accumulate = (flags & THA_ACCUMULATE) != 0;
  if (accumulate && (out_dt != THA_F32 || !lse)) return THA_ERR_INVALID;
  if (!dtype_ok(in_dt) || !dtype_ok(out_dt)) return THA_ERR_UNSUPPORTED;
  if ((int64_t)H * D > kMaxRowElems) return THA_ERR_UNSUPPORTED;
  if (in_dt == THA_BF16 && D != 128 && D != 64) return THA_ERR_UNSUPPORTED;
  if (in_dt == THA_F32 && D > 256) return THA_ERR_UNSUPPORTED;
  const int64_t hd = (int64_t)H * D;
  const int64_t rows[4] = {Sq, Sk, Sk, Sq};
  for (int t = 0; t < 4; ++t) {
    const int64_t bs = st8[2 * t], rs = st8[2 * t + 1];
    if (rs < hd || rs > kMaxRowElems || bs < 0) return THA_ERR_INVALID;
    if (B > 1 && bs < rows[t] * rs) return THA_ERR_INVALID;  // batches must not overlap
  }
  if (st8[3] != st8[5]) return THA_ERR_UNSUPPORTED;  // k and v share one token stride
  if (in_dt == THA_BF16) {  // 16-byte vector accesses of q, k, v; 4-element vectors of o
    for (int t = 0; t < 3; ++t)
      if (st8[2 * t] % 8 || st8[2 * t + 1] % 8) return THA_ERR_UNSUPPORTED;
    if ((uintptr_t)q % 16 || (uintptr_t)k % 16 || (uintptr_t)v % 16) return THA_ERR_UNSUPPORTED;
    if (st8[6] % 4 || st8[7] % 4 || (uintptr_t)o % (out_dt == THA_BF16 ? 8 : 16)) return THA_ERR_UNSUPPORTED;
  }
  tha::AttnArgs a;
  a.q = q, a.k = k, a.v = v, a.o = o, a.lse = lse;
  a.kv_len = (flags & THA_MASK_KEY_PADDING) ? kv_len : nullptr;
  a.B = B, a.Sq = Sq, a.Sk = Sk, a.H = H, a.D = D;
  a.out_dt = out_dt;
  a.causal = (flags & THA_MASK_CAUSAL) != 0;
  a.q_pos0 = pos_diff(q_pos0, k_pos0), a.k_pos0 = 0;
  a.scale = scale;
  a.q_bs = st8[0], a.q_rs = st8[1], a.k_bs = st8[2], a.k_rs = st8[3];
  a.v_bs = st8[4], a.v_rs = st8[5], a.o_bs = st8[6], a.o_rs = st8[7];
  a.accumulate = accumulate;
  a.kernel = kernel == THA_KERNEL_NARROW ? tha::AttnArgs::kNarrow
           : kernel == THA_KERNEL_WIDE   ? tha::AttnArgs::kWide
           : kernel == THA_KERNEL_SPLIT  ? tha::AttnArgs::kSplit
           : kernel == THA_KERNEL_SPLIT64 ? tha::AttnArgs::kSplit64
                                         : tha::AttnArgs::kAuto;
  hipStream_t s = (hipStream_t)stream;
  return hip_status(in_dt == THA_BF16 ? tha::launch_attn_bf16(a, s) : tha::launch_attn_f32(a, s));
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, int out_dt, float* lse, int B, int Sq, int Sk,
             int H, int D, int in_dt, unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len,
             float scale, void* stream) {
  if (mask_flags & (THA_ACCUMULATE | THA_KERNEL_MASK)) return THA_ERR_INVALID;  // attn_fwd_ex only
  const long long hd = contiguous_row(H, D);
  const long long st8[8] = {Sq * hd, hd, Sk * hd, hd, Sk * hd, hd, Sq * hd, hd};
  return fwd_common(q, k, v, o, out_dt, lse, B, Sq, Sk, H, D, in_dt, mask_flags, q_pos0, k_pos0, kv_len, scale, st8,
                    stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, int out_dt, float* lse, int B, int Sq, int Sk,
                int H, int D, int in_dt, unsigned flags, long long q_pos0, long long k_pos0, const int* kv_len,
                float scale, const long long* strides, void* stream) {
  const long long hd = contiguous_row(H, D);
  const long long dflt[8] = {Sq * hd, hd, Sk * hd, hd, Sk * hd, hd, Sq * hd, hd};
  return fwd_common(q, k, v, o, out_dt, lse, B, Sq, Sk, H, D, in_dt, flags, q_pos0, k_pos0, kv_len, scale,
                    strides ? strides : dflt, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, float* dq,
             float* dk, float* dv, float* workspace, int B, int Sq, int Sk, int H, int D, int in_dt,
             unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len, float scale, void* stream) {
  if (!workspace) return THA_ERR_INVALID;
  const int rc = tha::attn_bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, Sq, Sk, H, D, in_dt, mask_flags, q_pos0,
                                     k_pos0, kv_len, scale);
  if (rc != THA_OK) return rc;
  return tha::attn_bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, Sq, Sk, H, D, in_dt, mask_flags,
                              q_pos0, k_pos0, kv_len, scale, stream);
}

int attn_merge_lse(int n_parts, const void* const* o_parts, const float* const* lse_parts, int part_dt, void* o_out,
                   int out_dt, float* lse_out, int B, int S, int H, int D, void* stream) {
  if (n_parts < 1 || n_parts > THA_MAX_PARTS) return THA_ERR_INVALID;
  if (!o_parts || !lse_parts || !o_out) return THA_ERR_INVALID;
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return THA_ERR_INVALID;
  tha::PartPtrs pp = {};
  for (int i = 0; i < n_parts; ++i) {
    if (!o_parts[i] || !lse_parts[i]) return THA_ERR_INVALID;
    pp.o[i] = o_parts[i];
    pp.lse[i] = lse_parts[i];
  }
  if (!dtype_ok(part_dt) || !dtype_ok(out_dt)) return THA_ERR_UNSUPPORTED;
  for (int i = 0; i < n_parts && part_dt != out_dt; ++i)  // in place needs equal element sizes
    if (o_out == o_parts[i]) return THA_ERR_INVALID;
  return hip_status(
      tha::launch_merge_lse(n_parts, pp, part_dt, o_out, out_dt, lse_out, B, S, H, D, (hipStream_t)stream));
}

int shard_permute(const void* const* shards, int P, int group, void* out, int B, int S, int H, int D, int elem_bytes,
                  void* stream) {
  return shard_permute_n(1, shards, P, group, &out, B, S, H, D, elem_bytes, stream);
}

int shard_unpermute(const void* in, int P, int group, void* const* shards, int B, int S, int H, int D, int elem_bytes,
                    void* stream) {
  return shard_unpermute_n(1, &in, P, group, shards, B, S, H, D, elem_bytes, stream);
}

int shard_permute_n(int n, const void* const* shards, int P, int group, void* const* outs, int B, int S, int H, int D,
                    int elem_bytes, void* stream) {
  tha::MultiShardPtrs mp;
  const int rc = check_permute_n(n, shards, P, group, (const void* const*)outs, B, S, H, D, elem_bytes, mp);
  if (rc != THA_OK) return rc;
  return hip_status(tha::launch_shard_permute(mp, n, P, group, B, S, H, D, elem_bytes, (hipStream_t)stream));
}

int shard_unpermute_n(int n, const void* const* ins, int P, int group, void* const* shards, int B, int S, int H, int D,
                      int elem_bytes, void* stream) {
  tha::MultiShardPtrs mp;
  const int rc = check_permute_n(n, (const void* const*)shards, P, group, ins, B, S, H, D, elem_bytes, mp);
  if (rc != THA_OK) return rc;
  return hip_status(tha::launch_shard_unpermute(mp, n, P, group, B, S, H, D, elem_bytes, (hipStream_t)stream));
}

int shard_all_to_all(const void* const* inputs, int P, int rank, void* out, int ndim, const long long* shape,
                     int scatter_dim, int gather_dim, int elem_bytes, void* stream) {
  if (!inputs || !out || !shape) return THA_ERR_INVALID;
  if (P < 1 || P > THA_MAX_SHARDS || rank < 0 || rank >= P) return THA_ERR_INVALID;
  if (ndim < 1 || ndim > 8) return THA_ERR_INVALID;
  if (scatter_dim < 0 || scatter_dim >= ndim || gather_dim < 0 || gather_dim >= ndim || scatter_dim == gather_dim)
    return THA_ERR_INVALID;
  constexpr int64_t kMaxElems = 1LL << 48;
  int64_t sh[8], total = 1;
  for (int d = 0; d < ndim; ++d) {
    if (shape[d] < 1 || shape[d] > kMaxElems / total) return THA_ERR_INVALID;  // total * shape[d] <= 2^48
    sh[d] = shape[d];
    total *= sh[d];
  }
  if (sh[scatter_dim] % P != 0) return THA_ERR_INVALID;
  tha::ShardPtrs sp = {};
  for (int i = 0; i < P; ++i) {
    if (!inputs[i]) return THA_ERR_INVALID;
    sp.p[i] = const_cast<void*>(inputs[i]);
  }
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return THA_ERR_UNSUPPORTED;
  return hip_status(
      tha::launch_all_to_all(sp, P, rank, out, ndim, sh, scatter_dim, gather_dim, elem_bytes, (hipStream_t)stream));
}

}  // extern "C"

// tha_kernels.h -- internal launcher interface between the C ABI (api.hip) and the
// kernel translation units.  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tha.h"

namespace tha {

// Device pointers passed by value in the kernel argument block.
struct ShardPtrs {
  void* p[THA_MAX_SHARDS];
};
// n tensors (at most THA_MAX_PERMUTE_TENSORS) of P shards each, and their grouped tensors.
struct MultiShardPtrs {
  void* shard[THA_MAX_PERMUTE_TENSORS][THA_MAX_SHARDS];
  void* grouped[THA_MAX_PERMUTE_TENSORS];
};
struct PartPtrs {
  const void* o[THA_MAX_PARTS];
  const float* lse[THA_MAX_PARTS];
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* kv_len;  // nullptr unless key padding
  int B, Sq, Sk, H, D;
  int out_dt;
  bool causal;
  long long q_pos0, k_pos0;
  float scale;
  // element strides between batches (bs) and between tokens (rs); heads at stride D, dims at 1.
  // k and v share one token stride (k_rs == v_rs).
  int64_t q_bs, q_rs, k_bs, k_rs, v_bs, v_rs, o_bs, o_rs;
  bool accumulate;  // o (fp32) and lse hold a running result: merge this call's result into them
  // bf16, head size 128: which form of the kernel runs (kAuto = chosen by grid size)
  enum Kernel { kAuto, kNarrow, kWide, kSplit, kSplit64 } kernel = kAuto;
};

struct AttnBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // [B,H,Sq] workspace
  const int* kv_len;
  int B, Sq, Sk, H, D;
  bool causal;
  long long q_pos0, k_pos0;
  float scale;
};

// attn_bwd's argument checks (all but the workspace) and its launch with a given Delta buffer
// ([B,H,Sq] floats); shared by attn_bwd and attn_bwd_noalloc.
int attn_bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   const float* dq, const float* dk, const float* dv, int B, int Sq, int Sk, int H, int D, int in_dt,
                   unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len, float scale);
int attn_bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    float* dq, float* dk, float* dv, float* delta, int B, int Sq, int Sk, int H, int D, int in_dt,
                    unsigned mask_flags, long long q_pos0, long long k_pos0, const int* kv_len, float scale,
                    void* stream);

hipError_t launch_shard_permute(const MultiShardPtrs& ptrs, int n, int P, int group, int B, int S, int H, int D,
                                int elem_bytes, hipStream_t stream);
hipError_t launch_shard_unpermute(const MultiShardPtrs& ptrs, int n, int P, int group, int B, int S, int H, int D,
                                  int elem_bytes, hipStream_t stream);
hipError_t launch_all_to_all(const ShardPtrs& in, int P, int rank, void* out, int ndim, const int64_t* shape,
                             int scatter_dim, int gather_dim, int elem_bytes, hipStream_t stream);
hipError_t launch_merge_lse(int n_parts, const PartPtrs& parts, int part_dt, void* o_out, int out_dt, float* lse_out,
                            int B, int S, int H, int D, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);
// Forms of the 128-row / 64-row pipelined kernel (attn_bf16_d128.hip).
enum class D128Form { kNarrow, kSplit, kSplit64 };
hipError_t launch_attn_bf16_d128(const AttnArgs& a, hipStream_t stream, D128Form form);
int64_t attn_bf16_d128_blocks(const AttnArgs& a);
hipError_t launch_attn_bf16_d128_wide(const AttnArgs& a, hipStream_t stream);
int64_t attn_bf16_d128_wide_blocks(const AttnArgs& a);
hipError_t launch_attn_bwd_delta(const AttnBwdArgs& a, int in_dt, hipStream_t stream);
hipError_t launch_attn_bwd_f32(const AttnBwdArgs& a, hipStream_t stream);
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream);

}  // namespace tha

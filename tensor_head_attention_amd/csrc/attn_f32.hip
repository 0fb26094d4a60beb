// attn_f32.hip -- exact-fp32 attention for small head dims (1 <= D <= 256).
//
// out_i = sum_j softmax(scale * q_i . k_j) v_j over the visible keys j, per
// head ("Megatron-LM - Training Multi-Billion Parameter Language Models Using
// Model Parallelism", linear algebra of attention; "adv07: Sequence Parallel"
// Q4), with the causal / key-padding visibility of tha.h.  Everything stays in
// fp32 (no matrix-core shortcut), so results match fp64 to ~1e-6.
//
// One wavefront per (b, h, query row).  Keys are taken 64 at a time: lane j
// scores key j0 + j against the row's query (held in LDS), the chunk's maximum
// and sum come from wavefront reductions, and each lane accumulates the
// dimensions d = lane, lane + 64, ... of the output (online softmax across
// chunks).  This path serves the fp32 workloads only and is not tuned.
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

struct F32Strides {
  int64_t q_bs, q_rs, k_bs, k_rs, v_bs, o_bs, o_rs;  // elements (batch, token); v_rs == k_rs
};

template <typename OutT>
__global__ void __launch_bounds__(kWaves * 64) attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                               const float* __restrict__ v, OutT* __restrict__ o,
                                                               float* __restrict__ lse, const int* __restrict__ kv_len,
                                                               int B, int Sq, int Sk, int H, int D, int causal,
                                                               long long q_pos0, long long k_pos0, float scale,
                                                               F32Strides st, int accumulate) {
  __shared__ float qs[kWaves][kMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row_id = (int64_t)blockIdx.x * kWaves + wave;
  if (row_id >= (int64_t)B * H * Sq) return;  // whole wavefronts leave together; no block barrier below
  const int i = (int)(row_id % Sq);
  const int64_t bh = row_id / Sq;
  const int h = (int)(bh % H);
  const int b = (int)(bh / H);
  const int64_t rs = st.k_rs;  // K/V elements between consecutive tokens
  const float* qrow = q + (int64_t)b * st.q_bs + (int64_t)i * st.q_rs + (int64_t)h * D;
  const float* kb = k + (int64_t)b * st.k_bs + (int64_t)h * D;
  const float* vb = v + (int64_t)b * st.v_bs + (int64_t)h * D;
  for (int d = lane; d < D; d += 64) qs[wave][d] = qrow[d];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // Visible keys are exactly j < j_end (causal prefix and/or padding length).
  long long j_end = Sk;
  if (kv_len) {
    long long L = kv_len[b];
    j_end = L < 0 ? 0 : (L > Sk ? Sk : L);
  }
  if (causal) {
    const long long last = q_pos0 + i - k_pos0;  // largest visible key index
    if (last + 1 < j_end) j_end = last + 1 < 0 ? 0 : last + 1;
  }

  float m = -INFINITY, l = 0.f;
  float acc[kMaxD / 64];
#pragma unroll
  for (int r = 0; r < kMaxD / 64; ++r) acc[r] = 0.f;

  for (long long j0 = 0; j0 < j_end; j0 += 64) {
    const long long j = j0 + lane;
    float s = -INFINITY;
    if (j < j_end) {
      const float* kr = kb + j * rs;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[wave][d], kr[d], dot);
      s = dot * scale;
    }
    const float m_new = fmaxf(m, wave_max(s));  // finite: key j0 is visible
    const float alpha = expf(m - m_new);         // 0 on the first chunk (m = -inf)
    const float p = (j < j_end) ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int r = 0; r < kMaxD / 64; ++r) acc[r] *= alpha;
    const int cnt = (int)((j_end - j0) < 64 ? (j_end - j0) : 64);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj, 64);
      const float* vr = vb + (j0 + jj) * rs;
#pragma unroll
      for (int r = 0; r < kMaxD / 64; ++r) {
        const int d = lane + 64 * r;
        if (d < D) acc[r] = fmaf(pj, vr[d], acc[r]);
      }
    }
    m = m_new;
  }
  OutT* orow = o + (int64_t)b * st.o_bs + (int64_t)i * st.o_rs + (int64_t)h * D;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const float lse_c = l > 0.f ? m + logf(l) : -INFINITY;
  float* lse_p = lse ? lse + ((int64_t)b * H + h) * Sq + i : nullptr;
  if constexpr (sizeof(OutT) == 4) {
    if (accumulate) {  // merge into the running result (every lane reads lse before lane 0 writes it)
      const MergeW w = merge_weights(*lse_p, lse_c);
#pragma unroll
      for (int r = 0; r < kMaxD / 64; ++r) {
        const int d = lane + 64 * r;
        if (d < D) orow[d] = (w.a != 0.f ? w.a * (float)orow[d] : 0.f) + w.c * (acc[r] * inv);
      }
      if (lane == 0) *lse_p = w.lse;
      return;
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxD / 64; ++r) {
    const int d = lane + 64 * r;
    if (d < D) orow[d] = (OutT)(acc[r] * inv);
  }
  if (lse_p && lane == 0) *lse_p = lse_c;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.H * a.Sq;
  const int64_t blocks = (rows + kWaves - 1) / kWaves;
  if (blocks > 0x7fffffff || a.D > kMaxD) return hipErrorInvalidValue;
  const F32Strides ss = {a.q_bs, a.q_rs, a.k_bs, a.k_rs, a.v_bs, a.o_bs, a.o_rs};
  if (a.out_dt == THA_F32)
    hipLaunchKernelGGL(attn_f32_kernel<float>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, st, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.kv_len, a.B, a.Sq, a.Sk, a.H, a.D,
                       (int)a.causal, a.q_pos0, a.k_pos0, a.scale, ss, a.accumulate ? 1 : 0);
  else
    hipLaunchKernelGGL(attn_f32_kernel<__bf16>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, st, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (__bf16*)a.o, a.lse, a.kv_len, a.B, a.Sq, a.Sk, a.H, a.D,
                       (int)a.causal, a.q_pos0, a.k_pos0, a.scale, ss, 0);
  return hipGetLastError();
}

}  // namespace tha

// attn_bwd_f32.hip -- attention backward: the Delta pre-pass (both dtypes) and the exact-fp32
// path for small head dims (1 <= D <= 256).
//
// Gradients of out_i = sum_j softmax_j(scale q_i . k_j) v_j for the cotangent dout (the chain
// rule through the softmax; the pages' training workloads need them, "Support deepspeed sequence
// parallel" and "关于数据分割和合并", the formulas themselves are a reading):
//   P_ij = exp(scale q_i . k_j - lse_i)   (lse from the forward pass over the full key set)
//   dP_ij = dout_i . v_j,   Delta_i = dout_i . o_i,   dS_ij = P_ij (dP_ij - Delta_i)
//   dv_j += sum_i P_ij dout_i,  dq_i += scale sum_j dS_ij k_j,  dk_j += scale sum_i dS_ij q_i
// Visibility (causal with global positions, key padding) as in the forward kernels.
//
// The fp32 path keeps everything in fp32 (results match fp64 to ~1e-6): one wavefront per query
// row for dq (lanes over keys for the scores, over dims for the accumulation), one wavefront per
// key row for dk and dv (lanes over queries, then over dims).  It serves the fp32 workloads and
// is not tuned.
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return (float)p[i];
}

// Delta_i = dout_i . o_i for every (b, h, i), into delta [B, H, Sq]; vector form.  A row of D
// elements is `lanes` = D / (16-byte vector) consecutive threads, rows taken in memory order
// ([B, Sq, H] rows of o and dout are contiguous), so both inputs stream as whole lines; blocks are
// spread so that each XCD takes a contiguous share of the tokens, and the 4-byte delta writes of
// neighbouring tokens (adjacent in [B, H, Sq]) stay in one XCD's L2.  HBM-bound: 2 * D * elem
// bytes read and 4 written per row.
template <typename T>
__global__ void __launch_bounds__(256) bwd_delta_vec_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                           float* __restrict__ delta, int64_t rows, int Sq, int H,
                                                           int D, int lanes_log2) {
  constexpr int kE = 16 / (int)sizeof(T);
  const int lanes = 1 << lanes_log2;
  const int lir = threadIdx.x & (lanes - 1);
  const int64_t r = (int64_t)xcd_contiguous_block(blockIdx.x, gridDim.x) * (256 >> lanes_log2) +
                    (threadIdx.x >> lanes_log2);  // (b*Sq + i)*H + h
  float acc = 0.f;
  if (r < rows) {
    const int64_t off = r * D + (int64_t)lir * kE;
    const i32x4 x = __builtin_nontemporal_load((const i32x4*)(o + off));
    const i32x4 y = __builtin_nontemporal_load((const i32x4*)(dout + off));
    const T* xv = (const T*)&x;
    const T* yv = (const T*)&y;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc = fmaf((float)xv[e], (float)yv[e], acc);
  }
  for (int m = lanes >> 1; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);  // within the row's lanes
  if (r < rows && lir == 0) {
    const int64_t bi = r / H;
    const int h = (int)(r - bi * H);
    const int64_t b = bi / Sq;
    const int i = (int)(bi - b * Sq);
    delta[(b * H + h) * Sq + i] = acc;
  }
}

// Delta for any D and alignment: one wavefront per row.
template <typename T>
__global__ void __launch_bounds__(kWaves * 64) bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                                float* __restrict__ delta, int B, int Sq, int H, int D) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row_id = (int64_t)blockIdx.x * kWaves + wave;  // (b*H + h)*Sq + i
  if (row_id >= (int64_t)B * H * Sq) return;
  const int i = (int)(row_id % Sq);
  const int64_t bh = row_id / Sq;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int64_t base = (((int64_t)b * Sq + i) * H + h) * D;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) acc = fmaf(ld(o, base + d), ld(dout, base + d), acc);
  acc = wave_sum(acc);
  if (lane == 0) delta[row_id] = acc;
}

// Keys visible to query row i are exactly j < key_end(i); queries that see key j are exactly
// i >= query_begin(j) (and i < Sq), with the key itself visible iff j < kv_lim.
__device__ __forceinline__ long long key_end(int causal, long long q_pos0, long long k_pos0, int i, int kv_lim) {
  long long e = kv_lim;
  if (causal) {
    const long long last = q_pos0 + i - k_pos0;
    if (last + 1 < e) e = last + 1 < 0 ? 0 : last + 1;
  }
  return e;
}

__global__ void __launch_bounds__(kWaves * 64) bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dq, const int* __restrict__ kv_len, int B, int Sq, int Sk, int H, int D, int causal,
    long long q_pos0, long long k_pos0, float scale) {
  __shared__ float qs[kWaves][kMaxD], ds_[kWaves][kMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row_id = (int64_t)blockIdx.x * kWaves + wave;  // (b*H + h)*Sq + i
  if (row_id >= (int64_t)B * H * Sq) return;  // whole wavefronts leave together; no block barrier below
  const int i = (int)(row_id % Sq);
  const int64_t bh = row_id / Sq;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int64_t rs = (int64_t)H * D;
  const int64_t qoff = ((int64_t)b * Sq + i) * rs + (int64_t)h * D;
  for (int d = lane; d < D; d += 64) {
    qs[wave][d] = q[qoff + d];
    ds_[wave][d] = dout[qoff + d];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int kv_lim = Sk;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > Sk ? Sk : L);
  }
  const long long j_end = key_end(causal, q_pos0, k_pos0, i, kv_lim);
  const float L = lse[row_id], Dl = delta[row_id];
  const float* kb = k + (int64_t)b * Sk * rs + (int64_t)h * D;
  const float* vb = v + (int64_t)b * Sk * rs + (int64_t)h * D;
  float acc[kMaxD / 64];
#pragma unroll
  for (int r = 0; r < kMaxD / 64; ++r) acc[r] = 0.f;
  for (long long j0 = 0; j0 < j_end; j0 += 64) {
    const long long j = j0 + lane;
    float dsv = 0.f;
    if (j < j_end) {
      const float* kr = kb + j * rs;
      const float* vr = vb + j * rs;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(qs[wave][d], kr[d], s);
        dp = fmaf(ds_[wave][d], vr[d], dp);
      }
      const float p = expf(s * scale - L);
      dsv = p * (dp - Dl);
    }
    const int cnt = (int)((j_end - j0) < 64 ? (j_end - j0) : 64);
    for (int jj = 0; jj < cnt; ++jj) {
      const float dsj = __shfl(dsv, jj, 64);
      const float* kr = kb + (j0 + jj) * rs;
#pragma unroll
      for (int r = 0; r < kMaxD / 64; ++r) {
        const int d = lane + 64 * r;
        if (d < D) acc[r] = fmaf(dsj, kr[d], acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxD / 64; ++r) {
    const int d = lane + 64 * r;
    if (d < D) dq[qoff + d] += scale * acc[r];
  }
}

__global__ void __launch_bounds__(kWaves * 64) bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    float* __restrict__ dk, float* __restrict__ dv, const int* __restrict__ kv_len, int B, int Sq, int Sk, int H,
    int D, int causal, long long q_pos0, long long k_pos0, float scale) {
  __shared__ float ks[kWaves][kMaxD], vs[kWaves][kMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t key_id = (int64_t)blockIdx.x * kWaves + wave;  // (b*H + h)*Sk + j
  if (key_id >= (int64_t)B * H * Sk) return;
  const int j = (int)(key_id % Sk);
  const int64_t bh = key_id / Sk;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int64_t rs = (int64_t)H * D;
  int kv_lim = Sk;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > Sk ? Sk : L);
  }
  if (j >= kv_lim) return;  // a padding key is seen by no query: nothing to add
  const int64_t koff = ((int64_t)b * Sk + j) * rs + (int64_t)h * D;
  for (int d = lane; d < D; d += 64) {
    ks[wave][d] = k[koff + d];
    vs[wave][d] = v[koff + d];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  long long i_begin = 0;  // causal: query i sees key j iff q_pos0 + i >= k_pos0 + j
  if (causal) {
    const long long first = k_pos0 + j - q_pos0;
    i_begin = first < 0 ? 0 : first;
  }
  const float* qb = q + (int64_t)b * Sq * rs + (int64_t)h * D;
  const float* db = dout + (int64_t)b * Sq * rs + (int64_t)h * D;
  const float* lb = lse + bh * Sq;
  const float* deb = delta + bh * Sq;
  float acck[kMaxD / 64], accv[kMaxD / 64];
#pragma unroll
  for (int r = 0; r < kMaxD / 64; ++r) acck[r] = accv[r] = 0.f;
  for (long long i0 = i_begin; i0 < Sq; i0 += 64) {
    const long long i = i0 + lane;
    float p = 0.f, dsv = 0.f;
    if (i < Sq) {
      const float L = lb[i];
      if (L != -INFINITY) {
        const float* qr = qb + i * rs;
        const float* dr = db + i * rs;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(qr[d], ks[wave][d], s);
          dp = fmaf(dr[d], vs[wave][d], dp);
        }
        p = expf(s * scale - L);
        dsv = p * (dp - deb[i]);
      }
    }
    const int cnt = (int)((Sq - i0) < 64 ? (Sq - i0) : 64);
    for (int ii = 0; ii < cnt; ++ii) {
      const float pi = __shfl(p, ii, 64), dsi = __shfl(dsv, ii, 64);
      const float* qr = qb + (i0 + ii) * rs;
      const float* dr = db + (i0 + ii) * rs;
#pragma unroll
      for (int r = 0; r < kMaxD / 64; ++r) {
        const int d = lane + 64 * r;
        if (d < D) {
          acck[r] = fmaf(dsi, qr[d], acck[r]);
          accv[r] = fmaf(pi, dr[d], accv[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxD / 64; ++r) {
    const int d = lane + 64 * r;
    if (d < D) {
      dk[koff + d] += scale * acck[r];
      dv[koff + d] += accv[r];
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd_delta(const AttnBwdArgs& a, int in_dt, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.H * a.Sq;
  {
    const int ke = in_dt == THA_F32 ? 4 : 8;  // elements per 16-byte vector
    const int lanes = a.D / ke;
    const bool vec = a.D % ke == 0 && lanes >= 1 && lanes <= 64 && (lanes & (lanes - 1)) == 0 &&
                     (uintptr_t)a.o % 16 == 0 && (uintptr_t)a.dout % 16 == 0;
    if (vec) {
      int ll = 0;
      while ((1 << ll) < lanes) ++ll;
      const int64_t rpb = 256 >> ll;
      const int64_t vblocks = (rows + rpb - 1) / rpb;
      if (vblocks > 0x7fffffff) return hipErrorInvalidValue;
      if (in_dt == THA_F32)
        hipLaunchKernelGGL(bwd_delta_vec_kernel<float>, dim3((unsigned)vblocks), dim3(256), 0, st, (const float*)a.o,
                           (const float*)a.dout, a.delta, rows, a.Sq, a.H, a.D, ll);
      else
        hipLaunchKernelGGL(bwd_delta_vec_kernel<__bf16>, dim3((unsigned)vblocks), dim3(256), 0, st,
                           (const __bf16*)a.o, (const __bf16*)a.dout, a.delta, rows, a.Sq, a.H, a.D, ll);
      return hipGetLastError();
    }
  }
  const int64_t blocks = (rows + kWaves - 1) / kWaves;
  if (blocks > 0x7fffffff || a.D > 1024) return hipErrorInvalidValue;
  if (in_dt == THA_F32)
    hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, st, (const float*)a.o,
                       (const float*)a.dout, a.delta, a.B, a.Sq, a.H, a.D);
  else
    hipLaunchKernelGGL(bwd_delta_kernel<__bf16>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, st,
                       (const __bf16*)a.o, (const __bf16*)a.dout, a.delta, a.B, a.Sq, a.H, a.D);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_f32(const AttnBwdArgs& a, hipStream_t st) {
  if (a.D > kMaxD) return hipErrorInvalidValue;
  const int64_t qblocks = ((int64_t)a.B * a.H * a.Sq + kWaves - 1) / kWaves;
  const int64_t kblocks = ((int64_t)a.B * a.H * a.Sk + kWaves - 1) / kWaves;
  if (qblocks > 0x7fffffff || kblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)qblocks), dim3(kWaves * 64), 0, st, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse, a.delta, a.dq, a.kv_len, a.B,
                     a.Sq, a.Sk, a.H, a.D, (int)a.causal, a.q_pos0, a.k_pos0, a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_f32_kernel, dim3((unsigned)kblocks), dim3(kWaves * 64), 0, st, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse, a.delta, a.dk, a.dv,
                     a.kv_len, a.B, a.Sq, a.Sk, a.H, a.D, (int)a.causal, a.q_pos0, a.k_pos0, a.scale);
  return hipGetLastError();
}

}  // namespace tha

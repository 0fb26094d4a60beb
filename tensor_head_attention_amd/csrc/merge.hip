// merge.hip -- log-sum-exp combination of partial attention results over
// disjoint key blocks (the Ring step that accumulates block results into the
// full attention, "adv07: Sequence Parallel" Q5 and section 5, Ring Attention;
// the combination rule is the standard log-sum-exp one, a reading):
//   M = max_k lse_k; w_k = exp(lse_k - M); o = sum_k w_k o_k / sum_k w_k;
//   lse = M + log(sum_k w_k); all parts empty (-inf) -> o = 0, lse = -inf.
//
// HBM-bound streaming kernel.  A row (b, s, h) of D elements is handled by
// `lanes` lanes of one wavefront (a power of two dividing 64), each owning
// chunks of kVec consecutive elements.  Keeping a row inside one wavefront
// makes in-place use safe: every lane reads the row's lse values before the
// row's single lse store, and each output element is written by the lane
// that read it.
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  __device__ static f32x4 load(const void* p, int64_t i) { return *(const f32x4*)((const float*)p + i); }
  __device__ static void store(void* p, int64_t i, f32x4 v) { *(f32x4*)((float*)p + i) = v; }
};
template <>
struct Vec4<__bf16> {
  __device__ static f32x4 load(const void* p, int64_t i) {
    bf16x4 v = *(const bf16x4*)((const __bf16*)p + i);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
  __device__ static void store(void* p, int64_t i, f32x4 v) {
    bf16x4 r = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(bf16x4*)((__bf16*)p + i) = r;
  }
};

template <typename T>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  return (float)((const T*)p)[i];
}
template <typename T>
__device__ __forceinline__ void store1(void* p, int64_t i, float v) {
  ((T*)p)[i] = (T)v;
}

// kVec = 4: D % 4 == 0 and 8/16-byte aligned rows; kVec = 1: any D.
template <typename PartT, typename OutT, int kVec>
__global__ void __launch_bounds__(kThreads) merge_kernel(PartPtrs parts, int n, void* o_out, float* lse_out,
                                                        int64_t rows, int S, int H, int D, int lanes_log2) {
  const int lanes = 1 << lanes_log2;
  const int rows_per_block = kThreads >> lanes_log2;
  const int lane_in_row = threadIdx.x & (lanes - 1);
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + (threadIdx.x >> lanes_log2);
  if (row >= rows) return;  // whole rows leave together
  // row = (b*S + s)*H + h  ->  lse index (b*H + h)*S + s
  const int64_t bs = row / H;
  const int h = (int)(row - bs * H);
  const int64_t b = bs / S;
  const int s = (int)(bs - b * S);
  const int64_t li = (b * H + h) * S + s;

  float M = -INFINITY;
  for (int k = 0; k < n; ++k) M = fmaxf(M, parts.lse[k][li]);
  const int64_t obase = row * D;
  if (M == -INFINITY) {
    for (int c = lane_in_row * kVec; c < D; c += lanes * kVec) {
      if constexpr (kVec == 4)
        Vec4<OutT>::store(o_out, obase + c, f32x4{0.f, 0.f, 0.f, 0.f});
      else
        store1<OutT>(o_out, obase + c, 0.f);
    }
    if (lse_out && lane_in_row == 0) lse_out[li] = -INFINITY;
    return;
  }
  float W = 0.f;
  for (int k = 0; k < n; ++k) W += expf(parts.lse[k][li] - M);
  const float inv_w = 1.0f / W;
  for (int c = lane_in_row * kVec; c < D; c += lanes * kVec) {
    if constexpr (kVec == 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int k = 0;
      for (; k + 4 <= n; k += 4) {  // four independent loads in flight
        f32x4 x0 = Vec4<PartT>::load(parts.o[k], obase + c);
        f32x4 x1 = Vec4<PartT>::load(parts.o[k + 1], obase + c);
        f32x4 x2 = Vec4<PartT>::load(parts.o[k + 2], obase + c);
        f32x4 x3 = Vec4<PartT>::load(parts.o[k + 3], obase + c);
        const float w0 = expf(parts.lse[k][li] - M) * inv_w, w1 = expf(parts.lse[k + 1][li] - M) * inv_w;
        const float w2 = expf(parts.lse[k + 2][li] - M) * inv_w, w3 = expf(parts.lse[k + 3][li] - M) * inv_w;
        acc += x0 * w0;
        acc += x1 * w1;
        acc += x2 * w2;
        acc += x3 * w3;
      }
      for (; k < n; ++k) acc += Vec4<PartT>::load(parts.o[k], obase + c) * (expf(parts.lse[k][li] - M) * inv_w);
      Vec4<OutT>::store(o_out, obase + c, acc);
    } else {
      float acc = 0.f;
      for (int k = 0; k < n; ++k) acc += load1<PartT>(parts.o[k], obase + c) * (expf(parts.lse[k][li] - M) * inv_w);
      store1<OutT>(o_out, obase + c, acc);
    }
  }
  if (lse_out && lane_in_row == 0) lse_out[li] = M + logf(W);
}

template <typename PartT, typename OutT>
hipError_t launch_typed(int n, const PartPtrs& parts, void* o_out, float* lse_out, int B, int S, int H, int D,
                        bool vec, hipStream_t st) {
  const int chunks = vec ? D / 4 : D;
  int lanes_log2 = 0;
  while ((1 << lanes_log2) < chunks && lanes_log2 < 6) ++lanes_log2;
  const int64_t rows = (int64_t)B * S * H;
  const int rows_per_block = kThreads >> lanes_log2;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((merge_kernel<PartT, OutT, 4>), dim3((unsigned)blocks), dim3(kThreads), 0, st, parts, n, o_out,
                       lse_out, rows, S, H, D, lanes_log2);
  else
    hipLaunchKernelGGL((merge_kernel<PartT, OutT, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, st, parts, n, o_out,
                       lse_out, rows, S, H, D, lanes_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_lse(int n, const PartPtrs& parts, int part_dt, void* o_out, int out_dt, float* lse_out, int B,
                            int S, int H, int D, hipStream_t st) {
  const int pb = part_dt == THA_F32 ? 4 : 2, ob = out_dt == THA_F32 ? 4 : 2;
  bool vec = (D % 4 == 0) && ((uintptr_t)o_out % (4 * ob) == 0);
  for (int k = 0; k < n && vec; ++k) vec = ((uintptr_t)parts.o[k] % (4 * pb) == 0);
  if (part_dt == THA_F32 && out_dt == THA_F32)
    return launch_typed<float, float>(n, parts, o_out, lse_out, B, S, H, D, vec, st);
  if (part_dt == THA_F32 && out_dt == THA_BF16)
    return launch_typed<float, __bf16>(n, parts, o_out, lse_out, B, S, H, D, vec, st);
  if (part_dt == THA_BF16 && out_dt == THA_F32)
    return launch_typed<__bf16, float>(n, parts, o_out, lse_out, B, S, H, D, vec, st);
  return launch_typed<__bf16, __bf16>(n, parts, o_out, lse_out, B, S, H, D, vec, st);
}

}  // namespace tha

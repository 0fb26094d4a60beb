// merge.hip -- log-sum-exp combination of partial attention results over
// disjoint key blocks (the Ring step that accumulates block results into the
// full attention, "adv07: Sequence Parallel" Q5 and section 5, Ring Attention;
// the combination rule is the standard log-sum-exp one, a reading):
//   M = max_k lse_k; w_k = exp(lse_k - M); o = sum_k w_k o_k / sum_k w_k;
//   lse = M + log(sum_k w_k); all parts empty (-inf) -> o = 0, lse = -inf.
//
// HBM-bound streaming kernel: every partial is read once (non-temporal) and
// the result written once.  Blocks are spread so that each XCD takes a
// contiguous eighth of the rows (xcd_contiguous_block): the lse vectors, read
// and written 4 bytes per row, then have no cache line shared between XCDs,
// which measured 29.4 -> 23.2 us for 8 fp32 partials [4096, 8, 128].  See the
// two kernels below for how in-place use stays race-free.
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
  __device__ static f32x4 load_nt(const void* p, int64_t i) {
    return __builtin_nontemporal_load((const f32x4*)((const float*)p + i));
  }
  __device__ static void store(void* p, int64_t i, f32x4 v) { *(f32x4*)((float*)p + i) = v; }
};
template <>
struct Vec4<__bf16> {
  __device__ static f32x4 load(const void* p, int64_t i) {
    bf16x4 v = *(const bf16x4*)((const __bf16*)p + i);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
  __device__ static f32x4 load_nt(const void* p, int64_t i) {
    const uint64_t u = __builtin_nontemporal_load((const uint64_t*)((const __bf16*)p + i));
    bf16x4 v = __builtin_bit_cast(bf16x4, u);
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

// Vector path (D % 4 == 0, D <= 1024, 8/16-byte aligned rows): each thread owns one chunk of 4
// consecutive elements of one row; a row is `lanes` consecutive threads of the block (lanes a power
// of two, <= 256).  The data loads of the first 8 parts are issued before the lse reads, so a
// workgroup waits for memory once rather than twice (lse, then data).  In-place use: each output
// element is written by the thread that read it from every part, so o_out may be any o_parts[k] of
// the same element type; the row's single lse store comes after a block barrier that follows every
// read of the row's lse values (the first 8 parts and the max before the first barrier; the later
// parts, read while weighting, before a second barrier that only rows spanning several wavefronts
// need), so lse_out may be any lse_parts[k].  No thread leaves before a barrier.
template <typename PartT, typename OutT>
__global__ void __launch_bounds__(kThreads) merge_vec_kernel(PartPtrs parts, int n, void* o_out, float* lse_out,
                                                            int64_t rows, int S, int H, int D, int lanes_log2) {
  constexpr int kChunk = 8;  // parts whose loads are in flight together
  const int lanes = 1 << lanes_log2;
  const int lane_in_row = threadIdx.x & (lanes - 1);
  const int64_t row = (int64_t)xcd_contiguous_block(blockIdx.x, gridDim.x) * (kThreads >> lanes_log2) +
                      (threadIdx.x >> lanes_log2);
  const bool live = row < rows;
  const int c = lane_in_row * 4;
  const int64_t off = row * D + c;
  const bool act = live && c < D;
  const int n0 = min(kChunk, n);
  f32x4 x[kChunk];
#pragma unroll
  for (int u = 0; u < kChunk; ++u)
    if (u < n0 && act) x[u] = Vec4<PartT>::load_nt(parts.o[u], off);
  int64_t li = 0;
  float M = -INFINITY, l0[kChunk];
  if (live) {
    // row = (b*S + s)*H + h  ->  lse index (b*H + h)*S + s
    const int64_t bs = row / H;
    const int h = (int)(row - bs * H);
    const int64_t b = bs / S;
    const int s = (int)(bs - b * S);
    li = (b * H + h) * S + s;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      l0[u] = u < n0 ? parts.lse[u][li] : -INFINITY;
      M = fmaxf(M, l0[u]);
    }
    for (int k = kChunk; k < n; ++k) M = fmaxf(M, parts.lse[k][li]);
  }
  __syncthreads();  // the lse reads above precede every lse write of the block
  const bool work = live && M != -INFINITY;  // M = -inf: every part empty -> o = 0, lse = -inf
  float W = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (work) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (u < n0) {
        const float w = expf(l0[u] - M);
        W += w;
        if (c < D) acc += x[u] * w;
      }
    // further parts in chunks of 8: all loads of a chunk in flight before its weights are applied
    for (int k0 = kChunk; k0 < n; k0 += kChunk) {
      const int kn = min(kChunk, n - k0);
      float w[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        w[u] = 0.f;
        if (u < kn) {
          if (c < D) x[u] = Vec4<PartT>::load_nt(parts.o[k0 + u], off);
          w[u] = expf(parts.lse[k0 + u][li] - M);
        }
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (u < kn) {
          W += w[u];
          if (c < D) acc += x[u] * w[u];
        }
    }
    acc = acc * (1.0f / W);
  }
  if (act) Vec4<OutT>::store(o_out, off, acc);
  // A row of more than 64 lanes spans several wavefronts: the reads of parts 8.. above, in every
  // one of them, must precede the row's lse store (n and lanes are uniform over the grid).
  if (n > kChunk && lanes_log2 > 6) __syncthreads();
  if (live && lse_out && lane_in_row == 0) lse_out[li] = work ? M + logf(W) : -INFINITY;
}

// Scalar path (any D): a row is handled by `lanes` lanes of one wavefront (a power of two
// dividing 64), each owning elements lane_in_row, lane_in_row + lanes, ...; a row stays inside one
// wavefront, so every lane reads the row's lse values before the row's single lse store.
template <typename PartT, typename OutT>
__global__ void __launch_bounds__(kThreads) merge_scalar_kernel(PartPtrs parts, int n, void* o_out, float* lse_out,
                                                               int64_t rows, int S, int H, int D, int lanes_log2) {
  const int lanes = 1 << lanes_log2;
  const int lane_in_row = threadIdx.x & (lanes - 1);
  const int64_t row = (int64_t)xcd_contiguous_block(blockIdx.x, gridDim.x) * (kThreads >> lanes_log2) +
                      (threadIdx.x >> lanes_log2);
  if (row >= rows) return;  // whole rows leave together
  const int64_t bs = row / H;
  const int h = (int)(row - bs * H);
  const int64_t b = bs / S;
  const int s = (int)(bs - b * S);
  const int64_t li = (b * H + h) * S + s;
  float M = -INFINITY;
  for (int k = 0; k < n; ++k) M = fmaxf(M, parts.lse[k][li]);
  const int64_t obase = row * D;
  if (M == -INFINITY) {
    for (int c = lane_in_row; c < D; c += lanes) store1<OutT>(o_out, obase + c, 0.f);
    if (lse_out && lane_in_row == 0) lse_out[li] = -INFINITY;
    return;
  }
  float W = 0.f;
  for (int k = 0; k < n; ++k) W += expf(parts.lse[k][li] - M);
  const float inv_w = 1.0f / W;
  for (int c = lane_in_row; c < D; c += lanes) {
    float acc = 0.f;
    for (int k = 0; k < n; ++k) acc += load1<PartT>(parts.o[k], obase + c) * (expf(parts.lse[k][li] - M) * inv_w);
    store1<OutT>(o_out, obase + c, acc);
  }
  if (lse_out && lane_in_row == 0) lse_out[li] = M + logf(W);
}

template <typename PartT, typename OutT>
hipError_t launch_typed(int n, const PartPtrs& parts, void* o_out, float* lse_out, int B, int S, int H, int D,
                        bool vec, hipStream_t st) {
  const int chunks = vec ? D / 4 : D;
  const int max_lanes_log2 = vec ? 8 : 6;
  int lanes_log2 = 0;
  while ((1 << lanes_log2) < chunks && lanes_log2 < max_lanes_log2) ++lanes_log2;
  const int64_t rows = (int64_t)B * S * H;
  const int rows_per_block = kThreads >> lanes_log2;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL((merge_vec_kernel<PartT, OutT>), dim3((unsigned)blocks), dim3(kThreads), 0, st, parts, n, o_out,
                       lse_out, rows, S, H, D, lanes_log2);
  else
    hipLaunchKernelGGL((merge_scalar_kernel<PartT, OutT>), dim3((unsigned)blocks), dim3(kThreads), 0, st, parts, n,
                       o_out, lse_out, rows, S, H, D, lanes_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_lse(int n, const PartPtrs& parts, int part_dt, void* o_out, int out_dt, float* lse_out, int B,
                            int S, int H, int D, hipStream_t st) {
  const int pb = part_dt == THA_F32 ? 4 : 2, ob = out_dt == THA_F32 ? 4 : 2;
  bool vec = (D % 4 == 0) && D <= 1024 && ((uintptr_t)o_out % (4 * ob) == 0);
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

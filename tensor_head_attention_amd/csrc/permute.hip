// permute.hip -- Ulysses local layout kernels: sequence shards <-> one head group
// over the whole sequence (the local effect of the all-to-all that "adv07:
// Sequence Parallel", section 5 (DeepSpeed Ulysses) describes, a transpose of
// the sequence and head axes in the issue thread "关于数据分割和合并").
//
// Both directions are a gather/scatter of contiguous runs: for every (b, s)
// token the head group's heads are R = (H/P)*D*elem_bytes contiguous bytes in
// the shard (inside a row of H*D elements) and R contiguous bytes in the
// grouped tensor.  The grouped side is walked linearly so that one side of
// every copy is a fully contiguous stream; the other side is R-byte runs.
//
// HBM-bound: each byte is read once and written once.  16-byte vector path when
// R and every pointer are 16-byte aligned; element-wise fallback otherwise.
//
// One launch moves n tensors of the same shape (Q, K and V of a Ulysses step):
// workgroup w works on tensor w mod n, so the tensors' address streams are in
// flight together.  On MI355X the runs of one head group at the plain row pitch
// (2 KiB at 16 KiB for 8 of 64 heads of 128 dims) read slowly as one stream;
// three interleaved streams in one launch measured 6.2-6.3 TB/s against
// 5.3-5.5 TB/s for the same three tensors in three launches.
//
// Visiting order (vector path): the tokens of each shard are taken even ones
// first, then odd ones, so the workgroups in flight touch a shard's runs at
// twice its row pitch.  The set of bytes is the same; only their order changes
// (measured 25.5 -> 24.3 us per 128 MiB permute).
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kThreads = 256;

// Vector path: one 16-byte vector per thread (the most loads in flight across the chip, which
// measured fastest for this strided-read / contiguous-write mix), non-temporal both ways since
// every byte is touched once.  Workgroup w handles tensor w mod n and, within it, thread item idx
// (of 16 B) of block w / n: vector v = idx % run_vecs of the idx / run_vecs-th token in visiting
// order: token (b, s) with s = i*Sl + t for shard i, where the j-th visited token of a shard is
// t = 2j (j < Sl/2), else 2(j - Sl/2) + 1 when Sl is even, and t = j when Sl is odd.  A bijection
// on the tokens of every tensor.
template <bool kToGroup>
__global__ void __launch_bounds__(kThreads) permute_vec_kernel(MultiShardPtrs ptrs, int n, int64_t total_vecs,
                                                              uint32_t run_vecs, uint32_t run_shift, int S, int Sl,
                                                              int64_t shard_row_bytes, int64_t group_off_bytes) {
  const int tensor = (int)(blockIdx.x % (unsigned)n);
  const int64_t idx = (int64_t)(blockIdx.x / (unsigned)n) * kThreads + threadIdx.x;
  if (idx >= total_vecs) return;
  int64_t lt;
  uint32_t v;
  if (run_shift != 0xffffffffu) {  // power-of-two run length
    lt = idx >> run_shift;
    v = (uint32_t)(idx & (run_vecs - 1));
  } else {
    lt = idx / run_vecs;
    v = (uint32_t)(idx - lt * run_vecs);
  }
  const int64_t b = lt / S;
  const int s_vis = (int)(lt - b * S);
  const int i = s_vis / Sl;
  const int j = s_vis - i * Sl;
  const int half = Sl >> 1;
  const int t = (Sl & 1) ? j : (j < half ? 2 * j : 2 * (j - half) + 1);
  char* shard_p = (char*)ptrs.shard[tensor][i] + (b * Sl + t) * shard_row_bytes + group_off_bytes + (int64_t)v * 16;
  char* group_p = (char*)ptrs.grouped[tensor] + (((b * S + (int64_t)i * Sl + t) * run_vecs) + v) * 16;
  const i32x4 x = __builtin_nontemporal_load((const i32x4*)(kToGroup ? shard_p : group_p));
  __builtin_nontemporal_store(x, (i32x4*)(kToGroup ? group_p : shard_p));
}

// Element-wise fallback for unaligned or odd-sized runs: grid-stride over the n tensors' elements.
template <typename T, bool kToGroup>
__global__ void __launch_bounds__(kThreads) permute_elem_kernel(MultiShardPtrs ptrs, int n, int64_t total,
                                                               int64_t run_elems, int S, int Sl,
                                                               int64_t shard_row_elems, int64_t group_off_elems) {
  for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < total * n; k += (int64_t)gridDim.x * kThreads) {
    const int tensor = (int)(k / total);
    const int64_t idx = k - tensor * total;
    const int64_t tok = idx / run_elems;
    const int64_t e = idx - tok * run_elems;
    const int64_t b = tok / S;
    const int s = (int)(tok - b * S);
    const int i = s / Sl;
    const int t = s - i * Sl;
    T* shard_p = (T*)ptrs.shard[tensor][i] + (b * Sl + t) * shard_row_elems + group_off_elems + e;
    T* grouped = (T*)ptrs.grouped[tensor];
    if (kToGroup)
      grouped[idx] = *shard_p;
    else
      *shard_p = grouped[idx];
  }
}

template <typename T, bool kToGroup>
hipError_t launch_elem(const MultiShardPtrs& sp, int n, int64_t total, int64_t run_elems, int S, int Sl,
                       int64_t row_elems, int64_t off_elems, hipStream_t st) {
  int64_t blocks = (total * n + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((permute_elem_kernel<T, kToGroup>), dim3((unsigned)blocks), dim3(kThreads), 0, st, sp, n, total,
                     run_elems, S, Sl, row_elems, off_elems);
  return hipGetLastError();
}

template <bool kToGroup>
hipError_t launch_permute(const MultiShardPtrs& sp, int n, int P, int group, int B, int S, int H, int D, int eb,
                          hipStream_t st) {
  const int Sl = S / P, Hl = H / P;
  const int64_t run_bytes = (int64_t)Hl * D * eb;
  const int64_t row_bytes = (int64_t)H * D * eb;
  const int64_t off_bytes = (int64_t)group * Hl * D * eb;
  bool aligned = (run_bytes % 16 == 0) && (row_bytes % 16 == 0) && (off_bytes % 16 == 0);
  for (int t = 0; t < n && aligned; ++t) {
    aligned = (uintptr_t)sp.grouped[t] % 16 == 0;
    for (int i = 0; i < P && aligned; ++i) aligned = ((uintptr_t)sp.shard[t][i] % 16 == 0);
  }
  const int64_t tokens = (int64_t)B * S;
  if (aligned && run_bytes / 16 <= 0x7fffffff) {
    const uint32_t run_vecs = (uint32_t)(run_bytes / 16);
    uint32_t shift = 0xffffffffu;
    if ((run_vecs & (run_vecs - 1)) == 0) {
      shift = 0;
      while ((1u << shift) < run_vecs) ++shift;
    }
    const int64_t total = tokens * run_vecs;
    const int64_t blocks = (total + kThreads - 1) / kThreads * n;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((permute_vec_kernel<kToGroup>), dim3((unsigned)blocks), dim3(kThreads), 0, st, sp, n, total,
                       run_vecs, shift, S, Sl, row_bytes, off_bytes);
    return hipGetLastError();
  }
  const int64_t run_elems = (int64_t)Hl * D;
  const int64_t total = tokens * run_elems;
  const int64_t row_elems = (int64_t)H * D, off_elems = (int64_t)group * Hl * D;
  switch (eb) {
    case 1: return launch_elem<uint8_t, kToGroup>(sp, n, total, run_elems, S, Sl, row_elems, off_elems, st);
    case 2: return launch_elem<uint16_t, kToGroup>(sp, n, total, run_elems, S, Sl, row_elems, off_elems, st);
    case 4: return launch_elem<uint32_t, kToGroup>(sp, n, total, run_elems, S, Sl, row_elems, off_elems, st);
    case 8: return launch_elem<uint64_t, kToGroup>(sp, n, total, run_elems, S, Sl, row_elems, off_elems, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_shard_permute(const MultiShardPtrs& ptrs, int n, int P, int group, int B, int S, int H, int D,
                                int elem_bytes, hipStream_t stream) {
  return launch_permute<true>(ptrs, n, P, group, B, S, H, D, elem_bytes, stream);
}

hipError_t launch_shard_unpermute(const MultiShardPtrs& ptrs, int n, int P, int group, int B, int S, int H, int D,
                                  int elem_bytes, hipStream_t stream) {
  return launch_permute<false>(ptrs, n, P, group, B, S, H, D, elem_bytes, stream);
}

}  // namespace tha

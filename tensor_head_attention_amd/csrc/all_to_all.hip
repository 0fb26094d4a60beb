// all_to_all.hip -- the local layout of an all-to-all with a general scatter dim and gather dim
// ("Support deepspeed sequence parallel", PR body: the sequence all-to-all takes a scatter index
// and a gather index; all_to_all_single with a contiguous output).  Rank r's result is the
// concatenation along the gather dim, in rank order, of chunk r of every rank's tensor split into
// P equal chunks along the scatter dim.  shard_permute / shard_unpermute are the two Ulysses cases
// on [B, S, H, D] with their own tuned visiting order; this kernel takes any row-major shape.
//
// Host side: the shape collapses to five dims [A, X, M, Y, C] around the two special dims (X the
// earlier of them, Y the later; A, M, C the products of the dims before, between and after).  Every
// output element then belongs to a contiguous run of R elements that is also contiguous in one
// input:
//  - gather dim first (X gathered, Y scattered): R = (Y/P)*C; out = [A, P, X, M, Y/P*C], run
//    (a, i, t, m) reads input i at run ((a*X + t)*M + m)*P + rank (runs of R elements).
//  - scatter dim first (X scattered, Y gathered): R = Y*C; out = [A, X/P, M, P, Y*C], run
//    (a, hh, m, i) reads input i at run (a*X + rank*X/P + hh)*M + m.
// HBM-bound: each byte read once (non-temporal) and written once.  16-byte vectors when R and
// every pointer allow, else one element per thread.
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kThreads = 256;

// Unsigned 32-bit division by an invariant divisor as a multiply and shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994, section 4):
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l for every
// 32-bit n (the sum taken in 64 bits).
struct FastDiv {
  uint32_t d, m, l;
};

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.l = 0;
  while ((1ull << f.l) < d) ++f.l;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << f.l) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.l);
}

// Source run (in runs of R elements) and input index of output run `run`.
template <bool kGatherFirst>
__device__ __forceinline__ int64_t source_run(uint32_t run, const FastDiv& r0, const FastDiv& r1, const FastDiv& r2,
                                              uint32_t X, uint32_t M, uint32_t P, uint32_t rank, uint32_t Xl,
                                              uint32_t& input) {
  const uint32_t q1 = fdiv(run, r0), d0 = run - q1 * r0.d;
  const uint32_t q2 = fdiv(q1, r1), d1 = q1 - q2 * r1.d;
  const uint32_t d3 = fdiv(q2, r2), d2 = q2 - d3 * r2.d;
  if (kGatherFirst) {  // digits (m, t, i, a), radices (M, X, P)
    input = d2;
    return (((int64_t)d3 * X + d1) * M + d0) * P + rank;
  }
  // digits (i, m, hh, a), radices (P, M, X/P)
  input = d0;
  return ((int64_t)d3 * X + (int64_t)rank * Xl + d2) * M + d1;
}

template <bool kGatherFirst>
__global__ void __launch_bounds__(kThreads) a2a_vec_kernel(ShardPtrs in, char* out, uint32_t total_vecs,
                                                          FastDiv run_vecs, FastDiv r0, FastDiv r1, FastDiv r2,
                                                          uint32_t X, uint32_t M, uint32_t P, uint32_t rank,
                                                          uint32_t Xl) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total_vecs) return;
  const uint32_t run = fdiv(idx, run_vecs);
  const uint32_t v = idx - run * run_vecs.d;
  uint32_t input;
  const int64_t src = source_run<kGatherFirst>(run, r0, r1, r2, X, M, P, rank, Xl, input);
  const char* sp = (const char*)in.p[input] + (src * run_vecs.d + v) * 16;
  const i32x4 x = __builtin_nontemporal_load((const i32x4*)sp);
  __builtin_nontemporal_store(x, (i32x4*)(out + (int64_t)idx * 16));
}

// Element path (any run length or alignment), 64-bit indices, grid-stride.
template <typename T, bool kGatherFirst>
__global__ void __launch_bounds__(kThreads) a2a_elem_kernel(ShardPtrs in, T* out, int64_t total, int64_t R,
                                                           int64_t X, int64_t M, int64_t P, int64_t rank) {
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += (int64_t)gridDim.x * kThreads) {
    int64_t run = e / R;
    const int64_t off = e - run * R;
    int64_t input, src;
    if (kGatherFirst) {
      const int64_t m = run % M;
      run /= M;
      const int64_t t = run % X;
      run /= X;
      input = run % P;
      const int64_t a = run / P;
      src = ((a * X + t) * M + m) * P + rank;
    } else {
      input = run % P;
      run /= P;
      const int64_t m = run % M;
      run /= M;
      const int64_t Xl = X / P;
      const int64_t hh = run % Xl;
      const int64_t a = run / Xl;
      src = (a * X + rank * Xl + hh) * M + m;
    }
    out[e] = ((const T*)in.p[input])[src * R + off];
  }
}

template <typename T, bool kG>
hipError_t launch_elem(const ShardPtrs& in, void* out, int64_t total, int64_t R, int64_t X, int64_t M, int P, int rank,
                       hipStream_t st) {
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((a2a_elem_kernel<T, kG>), dim3((unsigned)blocks), dim3(kThreads), 0, st, in, (T*)out, total, R,
                     X, M, (int64_t)P, (int64_t)rank);
  return hipGetLastError();
}

template <bool kG>
hipError_t launch_dir(const ShardPtrs& in, int P, int rank, void* out, int64_t A, int64_t X, int64_t M, int64_t Y,
                      int64_t C, int eb, hipStream_t st) {
  const int64_t R = kG ? (Y / P) * C : Y * C;  // run length in elements
  const int64_t total = A * X * M * Y * C;     // elements of one input = elements of the output
  const int64_t run_bytes = R * eb;
  bool aligned = run_bytes % 16 == 0 && (uintptr_t)out % 16 == 0;
  for (int i = 0; i < P && aligned; ++i) aligned = (uintptr_t)in.p[i] % 16 == 0;
  const int64_t total_vecs = total * eb / 16;
  // the vector path's indices are 32-bit: vectors (hence runs and digits) and every radix below 2^32
  if (aligned && total_vecs < (1LL << 32) && X < (1LL << 32) && M < (1LL << 32)) {
    const FastDiv rv = make_fastdiv((uint32_t)(run_bytes / 16));
    const FastDiv r0 = make_fastdiv((uint32_t)(kG ? M : P));
    const FastDiv r1 = make_fastdiv((uint32_t)(kG ? X : M));
    const FastDiv r2 = make_fastdiv((uint32_t)(kG ? P : X / P));
    const int64_t blocks = (total_vecs + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((a2a_vec_kernel<kG>), dim3((unsigned)blocks), dim3(kThreads), 0, st, in, (char*)out,
                       (uint32_t)total_vecs, rv, r0, r1, r2, (uint32_t)X, (uint32_t)M, (uint32_t)P, (uint32_t)rank,
                       (uint32_t)(X / P));
    return hipGetLastError();
  }
  switch (eb) {
    case 1: return launch_elem<uint8_t, kG>(in, out, total, R, X, M, P, rank, st);
    case 2: return launch_elem<uint16_t, kG>(in, out, total, R, X, M, P, rank, st);
    case 4: return launch_elem<uint32_t, kG>(in, out, total, R, X, M, P, rank, st);
    case 8: return launch_elem<uint64_t, kG>(in, out, total, R, X, M, P, rank, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_all_to_all(const ShardPtrs& in, int P, int rank, void* out, int ndim, const int64_t* shape,
                             int scatter_dim, int gather_dim, int eb, hipStream_t st) {
  const int lo = scatter_dim < gather_dim ? scatter_dim : gather_dim;
  const int hi = scatter_dim < gather_dim ? gather_dim : scatter_dim;
  int64_t A = 1, M = 1, C = 1;
  for (int d = 0; d < lo; ++d) A *= shape[d];
  for (int d = lo + 1; d < hi; ++d) M *= shape[d];
  for (int d = hi + 1; d < ndim; ++d) C *= shape[d];
  const int64_t X = shape[lo], Y = shape[hi];
  if (gather_dim < scatter_dim) return launch_dir<true>(in, P, rank, out, A, X, M, Y, C, eb, st);
  return launch_dir<false>(in, P, rank, out, A, X, M, Y, C, eb, st);
}

}  // namespace tha

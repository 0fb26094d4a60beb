// attn_bf16.hip -- bf16 matrix-core attention forward for CDNA4 (gfx950).
//
// Computes, per head, out = softmax(scale * Q K^T + mask) V and the per-row
// log-sum-exp ("Megatron-LM - Training Multi-Billion Parameter Language Models
// Using Model Parallelism", linear algebra of attention; "adv07: Sequence
// Parallel" Q4 for the row definition and the causal rule; "parallel
// multi-head attention" section 3.2 for the [b, s, h, d] layout, fp32 softmax
// and the cast of the probabilities back to the input type before the product
// with V).
//
// Design (MI355X-first):
//  * A workgroup of 4 wavefronts owns 128 query rows of one (batch, head);
//    each wavefront owns 32 rows.  Keys stream through LDS in tiles of 64,
//    double buffered, shared by the 4 wavefronts.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    A = 32 keys x 16 dims of K (one 16-byte LDS read per lane), B = Q^T held
//    in registers for the whole kernel.  In the accumulator layout a lane holds
//    one query (its column) and 16 of the 32 keys, so the softmax row max and
//    row sum are in-lane reductions plus one v_permlane32_swap.
//  * The probabilities P^T (converted to bf16 in registers) are directly the
//    B operand of O^T += V^T P^T: the accumulator's key order (4-key groups
//    interleaved between the two half-waves) is matched by reading V^T with
//    ds_read_b64_tr_b16, which transposes 16-bit elements out of the row-major
//    V tile, so V never needs a transposed copy.
//  * Online softmax in the exp2 domain with scale*log2(e) folded into one FMA;
//    O^T is rescaled per lane (a lane's column is one query).
//  * Masking (causal with global positions, key padding, sequence tails) is
//    applied only on tiles that need it; tiles wholly in a wavefront's future
//    are skipped.  Tail loads use buffer loads, which return zero out of range.
//  * Heaviest causal query tiles are launched first; consecutive workgroups
//    take different heads of one query tile, so each head's workgroups land on
//    one XCD (dispatch is round-robin over the 8 XCDs) and share its L2.
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBlockM = kWaves * kRowsPerWave;  // 128 query rows per workgroup
constexpr int kBlockN = 64;                     // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

// Swizzles of the 16-byte chunk index inside a tile row (row = key):
//  K tile: read as 32 keys x one chunk per instruction -> spread keys over chunks.
//  V tile: read with ds_read_b64_tr_b16 as 4 keys x 4 chunks per half-wave.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return row & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  const int r = row & 3;
  if constexpr (D == 128)
    return ((r & 1) * 6) ^ ((r >> 1) * 12);  // 0, 6, 12, 10
  else
    return 2 * r;  // 0, 2, 4, 6
}

template <int D>
struct Smem {
  static constexpr int kTileBytes = kBlockN * D * 2;
  char k[2][kTileBytes];
  char v[2][kTileBytes];
};

struct KernelArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  void* o;
  float* lse;
  const int* kv_len;
  int B, Sq, Sk, H;
  int causal;
  long long q_pos0, k_pos0;
  float scale;       // natural-log scale (for lse)
  float scale_log2;  // scale * log2(e)
};

template <int D, typename OutT>
__global__ void __launch_bounds__(kThreads, 2) attn_bf16_kernel(KernelArgs a) {
  constexpr int kChunks = D / 8;           // 16-byte chunks per row
  constexpr int kDSteps = D / 16;          // k-steps of the score product
  constexpr int kDBlocks = D / 32;         // 32-row blocks of O^T
  constexpr int kLoadIters = kBlockN * kChunks / kThreads;  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(16))) Smem<D> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31;   // this lane's query column within the wavefront
  const int hi = lane >> 5;   // half-wave
  const int BH = a.B * a.H;
  const int n_qt = (a.Sq + kBlockM - 1) / kBlockM;
  const int qt = n_qt - 1 - (int)(blockIdx.x / BH);  // heaviest causal tiles first
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / a.H, h = bh % a.H;
  const int64_t row_stride = (int64_t)a.H * D;     // elements between consecutive tokens
  const uint32_t row_bytes = (uint32_t)(row_stride * 2);

  // Visible key range of the workgroup.
  int kv_lim = a.Sk;
  if (a.kv_len) {
    const int L = a.kv_len[b];
    kv_lim = L < 0 ? 0 : (L > a.Sk ? a.Sk : L);
  }
  long long kv_end = kv_lim;
  const int q_first = qt * kBlockM;
  if (a.causal) {
    const int q_last = min(a.Sq, q_first + kBlockM) - 1;
    const long long last_vis = a.q_pos0 + q_last - a.k_pos0;  // largest key index visible to the last row
    if (last_vis + 1 < kv_end) kv_end = last_vis + 1 < 0 ? 0 : last_vis + 1;
  }
  const int n_kt = (int)((kv_end + kBlockN - 1) / kBlockN);

  // Q^T fragments: lane holds query q0 + lq, dims [16t + 8hi, +8) for each k-step t.
  const int q0 = q_first + wave * kRowsPerWave;
  bf16x8 qf[kDSteps];
  {
    const int rows_valid = max(0, min(kRowsPerWave, a.Sq - q0));
    const __bf16* qbase = a.q + (((int64_t)b * a.Sq + min(q0, a.Sq - 1)) * a.H + h) * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, (uint32_t)rows_valid * row_bytes);
#pragma unroll
    for (int t = 0; t < kDSteps; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, buffer_load_16(rq, (uint32_t)lq * row_bytes + (uint32_t)(16 * t + 8 * hi) * 2));
  }

  const __bf16* kbase = a.k + ((int64_t)b * a.Sk * a.H + h) * D;
  const __bf16* vbase = a.v + ((int64_t)b * a.Sk * a.H + h) * D;

  // Global -> register staging of one K/V tile: thread loads chunks id = tid + 256u.
  i32x4 kst[kLoadIters], vst[kLoadIters];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBlockN;
    const int rows_valid = min(kBlockN, kv_lim - key0);
    const uint32_t nbytes = (uint32_t)max(rows_valid, 0) * row_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)key0 * row_stride, nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (int64_t)key0 * row_stride, nbytes);
#pragma unroll
    for (int u = 0; u < kLoadIters; ++u) {
      const int id = tid + kThreads * u;
      const int row = id / kChunks, c = id % kChunks;
      const uint32_t off = (uint32_t)row * row_bytes + (uint32_t)c * 16;
      kst[u] = buffer_load_16(rk, off);
      vst[u] = buffer_load_16(rv, off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kLoadIters; ++u) {
      const int id = tid + kThreads * u;
      const int row = id / kChunks, c = id % kChunks;
      *(i32x4*)(sm.k[buf] + row * (D * 2) + ((c ^ k_swz<D>(row)) * 16)) = kst[u];
      *(i32x4*)(sm.v[buf] + row * (D * 2) + ((c ^ v_swz<D>(row)) * 16)) = vst[u];
    }
  };

  f32x16 o_acc[kDBlocks];
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) o_acc[i][j] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores q.k (this lane's query)
  float l_run = 0.f;        // running sum over this half-wave's keys (exp2 domain)

  const long long q_pos = a.q_pos0 + q0 + lq;
  const bool wave_live = q0 < a.Sq;

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);

    const int key0 = kt * kBlockN;
    // Wave-uniform tile classification.
    bool skip = !wave_live;
    bool need_mask = key0 + kBlockN > kv_lim;
    if (a.causal) {
      const long long first_kpos = a.k_pos0 + key0;
      if (first_kpos > a.q_pos0 + q0 + kRowsPerWave - 1) skip = true;
      if (first_kpos + kBlockN - 1 > a.q_pos0 + q0) need_mask = true;
    }
    if (!skip) {
      // ---- S^T = K Q^T for two 32-key blocks -------------------------------
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
        const int row = kb * 32 + lq;
        const char* krow = sm.k[buf] + row * (D * 2);
        const int sw = k_swz<D>(row);
#pragma unroll
        for (int t = 0; t < kDSteps; ++t) {
          const bf16x8 kf = *(const bf16x8*)(krow + (((2 * t + hi) ^ sw) * 16));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kb], 0, 0, 0);
        }
      }
      // ---- mask -----------------------------------------------------------
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = key0 + kb * 32 + (j >> 2) * 8 + hi * 4 + (j & 3);
            bool hide = key >= kv_lim;
            if (a.causal) hide = hide || (a.k_pos0 + key > q_pos);
            if (hide) s[kb][j] = -INFINITY;
          }
      }
      // ---- online softmax (exp2 domain) -------------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb][j]);
      mx = max_across_halves(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float neg_mc = -m_use * a.scale_log2;
      const float alpha = __builtin_amdgcn_exp2f(fmaf(m_run, a.scale_log2, neg_mc));
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][j], a.scale_log2, neg_mc));
          s[kb][j] = p;
          rs += p;
        }
      l_run = fmaf(l_run, alpha, rs);
#pragma unroll
      for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) o_acc[i][j] *= alpha;
      // ---- P^T to bf16: B operands of the four 16-key steps -----------------
      bf16x8 pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, base = (ks & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ks][e] = (__bf16)s[kb][base + e];
      }
      // ---- O^T += V^T P^T ------------------------------------------------------
      // Lane (group G = lane/16, s = lane%16) addresses row 16ks + 4hi + s/4 (+8 for the
      // second read) and dims 32db + 16(G&1) + 4(s&3); the transpose read hands each
      // lane 4 consecutive keys of one dim.
      const int g = lane >> 4, sl = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int r0 = 16 * ks + 4 * hi + (sl >> 2);
        const int r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          const int c = 4 * db + 2 * (g & 1) + ((sl & 3) >> 1);
          const int byte_in = (sl & 1) * 8;
          const lds_char* vb = (const lds_char*)sm.v[buf];
          const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vb + r0 * (D * 2) + ((c ^ v_swz<D>(r0)) * 16) + byte_in));
          const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vb + r1 * (D * 2) + ((c ^ v_swz<D>(r1)) * 16) + byte_in));
          const s16x8 t = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
          o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), pb[ks], o_acc[db], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------
  if (!wave_live) return;
  const float l_tot = sum_across_halves(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const int qrow = q0 + lq;
  if (qrow < a.Sq) {
    OutT* orow = (OutT*)a.o + (((int64_t)b * a.Sq + qrow) * a.H + h) * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hi;
        if constexpr (sizeof(OutT) == 2) {
          bf16x4 r = {(__bf16)(o_acc[db][4 * jg] * inv), (__bf16)(o_acc[db][4 * jg + 1] * inv),
                      (__bf16)(o_acc[db][4 * jg + 2] * inv), (__bf16)(o_acc[db][4 * jg + 3] * inv)};
          *(bf16x4*)(orow + d0) = r;
        } else {
          f32x4 r = {o_acc[db][4 * jg] * inv, o_acc[db][4 * jg + 1] * inv, o_acc[db][4 * jg + 2] * inv,
                     o_acc[db][4 * jg + 3] * inv};
          *(f32x4*)(orow + d0) = r;
        }
      }
    if (a.lse && hi == 0)
      a.lse[((int64_t)b * a.H + h) * a.Sq + qrow] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& x, hipStream_t st) {
  KernelArgs a;
  a.q = (const __bf16*)x.q;
  a.k = (const __bf16*)x.k;
  a.v = (const __bf16*)x.v;
  a.o = x.o;
  a.lse = x.lse;
  a.kv_len = x.kv_len;
  a.B = x.B, a.Sq = x.Sq, a.Sk = x.Sk, a.H = x.H;
  a.causal = x.causal ? 1 : 0;
  a.q_pos0 = x.q_pos0, a.k_pos0 = x.k_pos0;
  a.scale = x.scale;
  a.scale_log2 = x.scale * kLog2e;
  const int64_t n_qt = (x.Sq + kBlockM - 1) / kBlockM;
  const int64_t blocks = n_qt * x.B * x.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (x.out_dt == THA_F32)
    hipLaunchKernelGGL((attn_bf16_kernel<D, float>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, __bf16>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  if (a.D == 128) return launch_d<128>(a, st);
  if (a.D == 64) return launch_d<64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tha

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
// This file's kernel serves head size 64; head size 128 goes to the software-pipelined
// kernel of attn_bf16_d128.hip, which keeps the same layout and work split.
//
// Design (MI355X-first):
//  * A workgroup of 4 wavefronts owns 128 query rows of one (batch, head);
//    each wavefront owns 32 rows.  Keys stream through LDS in tiles of 64,
//    double buffered and shared by the 4 wavefronts.  Tiles are copied
//    global -> LDS by buffer_load ... lds (no register staging); the copy of
//    tile t+1 runs while tile t is computed.
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
//  * Online softmax in the exp2 domain with scale*log2(e) folded into one FMA.
//    The running max is raised only when a row's new maximum exceeds it by
//    more than 2^8 in probability terms (then the row's O and sum are rescaled);
//    otherwise probabilities up to 256 are accumulated as they are.  The final
//    normalisation divides by the matching sum, so the result is the same up to
//    rounding and most tiles skip the rescale.
//  * Masking (causal with global positions, key padding, sequence tails) is
//    applied only on tiles that need it; tiles wholly in a wavefront's future
//    are skipped.  Out-of-range loads return zero (buffer range checking).
//  * Heaviest causal query tiles are launched first, and the workgroups that
//    one XCD receives (dispatch is round-robin over the 8 XCDs) walk one
//    (batch, head) at a time, so they share that head's K/V in the XCD's L2
//    (work_item in device_common.h).
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "attn_epilogue.h"
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
constexpr float kRescaleLog2 = 8.0f;  // raise the running max only past a 2^8 growth

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
  float rescale_raw; // kRescaleLog2 / scale_log2: raw-score growth that triggers a rescale
  int64_t q_bs, q_rs, k_bs, k_rs, v_bs, o_bs, o_rs;  // element strides (batch, token); v_rs == k_rs
  int accumulate;
};

template <int D, typename OutT>
__global__ void __launch_bounds__(kThreads, 2) attn_bf16_kernel(KernelArgs a) {
  constexpr int kChunks = D / 8;                     // 16-byte chunks per row
  constexpr int kDSteps = D / 16;                    // k-steps of the score product
  constexpr int kDBlocks = D / 32;                   // 32-row blocks of O^T
  constexpr int kTileBytes = kBlockN * D * 2;
  constexpr int kRowsPerLoad = 1024 / (D * 2);       // tile rows written by one wave-wide 16 B load
  constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * kTileBytes];  // [buf][K|V][tile]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;   // this lane's query column within the wavefront
  const int hi = lane >> 5;   // half-wave
  const int BH = a.B * a.H;
  const int n_qt = (a.Sq + kBlockM - 1) / kBlockM;
  const WorkItem wi = work_item((int)blockIdx.x, n_qt, BH, true);  // heaviest causal tiles first
  const int qt = wi.tile, bh = wi.bh;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t row_stride = a.k_rs;                // K/V elements between consecutive tokens
  const uint32_t row_bytes = (uint32_t)(row_stride * 2);
  const uint32_t q_row_bytes = (uint32_t)(a.q_rs * 2);

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
  const bool wave_live = q0 < a.Sq;
  bf16x8 qf[kDSteps];
  {
    const int rows_valid = max(0, min(kRowsPerWave, a.Sq - q0));
    const __bf16* qbase = a.q + (int64_t)b * a.q_bs + (int64_t)min(q0, a.Sq - 1) * a.q_rs + (int64_t)h * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, (uint32_t)rows_valid * q_row_bytes);
#pragma unroll
    for (int t = 0; t < kDSteps; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, buffer_load_16(rq, (uint32_t)lq * q_row_bytes + (uint32_t)(16 * t + 8 * hi) * 2));
  }

  const __bf16* kbase = a.k + (int64_t)b * a.k_bs + (int64_t)h * D;
  const __bf16* vbase = a.v + (int64_t)b * a.v_bs + (int64_t)h * D;

  // Per-lane global offsets of this wave's share of a tile copy: wave-wide load u fills
  // LDS bytes [(wave*kLoadsPerWave + u) * 1024, +1024), lane i its 16 bytes at i*16, i.e.
  // tile row r = (wave*kLoadsPerWave + u)*kRowsPerLoad + i/kChunks, stored chunk i%kChunks,
  // which holds logical chunk (i%kChunks) ^ swizzle(r).
  uint32_t koff[kLoadsPerWave], voff[kLoadsPerWave];
#pragma unroll
  for (int u = 0; u < kLoadsPerWave; ++u) {
    const int r = (wave * kLoadsPerWave + u) * kRowsPerLoad + lane / kChunks;
    const int p = lane % kChunks;
    koff[u] = (uint32_t)r * row_bytes + (uint32_t)((p ^ k_swz<D>(r)) * 16);
    voff[u] = (uint32_t)r * row_bytes + (uint32_t)((p ^ v_swz<D>(r)) * 16);
  }
  auto issue_tile = [&](int kt, int buf) {
    const int key0 = kt * kBlockN;
    const int rows_valid = min(kBlockN, kv_lim - key0);
    const uint32_t nbytes = (uint32_t)max(rows_valid, 0) * row_bytes;
    const i32x4 rk = make_rsrc_words(kbase + (int64_t)key0 * row_stride, nbytes);
    const i32x4 rv = make_rsrc_words(vbase + (int64_t)key0 * row_stride, nbytes);
    const uint32_t kl = lds_addr(smem + (buf * 2 + 0) * kTileBytes + wave * kLoadsPerWave * 1024);
    const uint32_t vl = lds_addr(smem + (buf * 2 + 1) * kTileBytes + wave * kLoadsPerWave * 1024);
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) {
      buffer_load_lds_16(rk, kl + u * 1024, koff[u]);
      buffer_load_lds_16(rv, vl + u * 1024, voff[u]);
    }
  };

  f32x16 o_acc[kDBlocks];
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) o_acc[i][j] = 0.f;
  float m_run = -INFINITY;  // reference max of raw scores q.k (this lane's query)
  float l_run = 0.f;        // running sum over this half-wave's keys (exp2 domain)

  const long long q_pos = a.q_pos0 + q0 + lq;

  // Per-lane LDS read offsets inside a tile.
  // K (A operand of S^T): key row kb*32 + lq, logical chunk 2t + hi.
  // V (transpose reads): lane (group g = lane/16, sl = lane%16) addresses row
  // 16ks + 4hi + sl/4 (+8 for the second read) and dims 32db + 16(g&1) + 4(sl&3).
  const int g = lane >> 4, sl = lane & 15;
  const int vrow0 = 4 * hi + (sl >> 2);
  const int vbyte_in = (sl & 1) * 8;
  const int vchunk_base = 2 * (g & 1) + ((sl & 3) >> 1);

  if (n_kt > 0) issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) issue_tile(kt + 1, buf ^ 1);

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
      const char* ks = smem + (buf * 2 + 0) * kTileBytes;
      const lds_char* vs = (const lds_char*)(smem + (buf * 2 + 1) * kTileBytes);
      // ---- S^T = K Q^T for two 32-key blocks -------------------------------
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
        const int row = kb * 32 + lq;
        const char* krow = ks + row * (D * 2);
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
      // ---- online softmax (exp2 domain, lazy rescale) -------------------------
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int j = 2; j < 16; ++j) mx = fmaxf(mx, s[0][j]);
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[1][j]);
      mx = max_across_halves(mx);
      // Raise the reference max only when it grows past the threshold (or is still -inf).
      const bool grow = mx > m_run + a.rescale_raw;
      if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2) : 1.0f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
          for (int j = 0; j < 16; ++j) o_acc[i][j] *= alpha;
      }
      const float neg_mc = m_run == -INFINITY ? 0.f : -m_run * a.scale_log2;
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[0][j], a.scale_log2, neg_mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[1][j], a.scale_log2, neg_mc));
        s[0][j] = p0;
        s[1][j] = p1;
        rs0 += p0;
        rs1 += p1;
      }
      l_run += rs0 + rs1;
      // ---- P^T to bf16: B operands of the four 16-key steps -----------------
      bf16x8 pb[4];
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const int kb = ks4 >> 1, base = (ks4 & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[ks4][e] = (__bf16)s[kb][base + e];
      }
      // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const int r0 = 16 * ks4 + vrow0;
        const int r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          const int c = 4 * db + vchunk_base;
          const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vs + r0 * (D * 2) + ((c ^ v_swz<D>(r0)) * 16) + vbyte_in));
          const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vs + r1 * (D * 2) + ((c ^ v_swz<D>(r1)) * 16) + vbyte_in));
          const s16x8 t = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
          o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, t), pb[ks4], o_acc[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of tile kt+1 has landed in LDS
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------
  if (!wave_live) return;
  const float l_tot = sum_across_halves(l_run);
  const int qrow = q0 + lq;
  if (qrow < a.Sq) {
    OutT* orow = (OutT*)a.o + (int64_t)b * a.o_bs + (int64_t)qrow * a.o_rs + (int64_t)h * D;
    float* lse_p = a.lse ? a.lse + ((int64_t)b * a.H + h) * a.Sq + qrow : nullptr;
    store_row<kDBlocks>(o_acc, orow, lse_p, hi, l_tot, m_run, a.scale, a.accumulate != 0);
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
  a.rescale_raw = kRescaleLog2 / a.scale_log2;
  a.q_bs = x.q_bs, a.q_rs = x.q_rs, a.k_bs = x.k_bs, a.k_rs = x.k_rs, a.v_bs = x.v_bs;
  a.o_bs = x.o_bs, a.o_rs = x.o_rs, a.accumulate = x.accumulate ? 1 : 0;
  const int64_t n_qt = (x.Sq + kBlockM - 1) / kBlockM;
  const int64_t blocks = n_qt * x.B * x.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (x.out_dt == THA_F32)
    hipLaunchKernelGGL((attn_bf16_kernel<D, float>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, __bf16>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// Head size 128, by grid size (CU count read once per device): the wide kernel (256 rows per
// workgroup, one workgroup per CU) when its grid fills every CU at least twice; else the narrow
// one (128 rows, two workgroups per CU) when its grid does; else a split form (two wavefront
// groups per workgroup share the key range), so small grids still keep every SIMD busy: the
// 64-row split form when the 128-row one would leave half the CUs idle, or when the call is
// causal, its 128-row tiles are no more than the CUs (each CU would hold one, and the heaviest
// sets the time) and its last query tile needs at least twice the keys of its first (then the
// 64-row tiles, launched heaviest first, even out the CUs' loads); else the 128-row split form
// (two wavefronts per SIMD; with more tiles than CUs the light ones already fill in behind the
// heavy ones).  A caller's forced choice (AttnArgs::kernel) overrides this.
enum class D128 { kNarrow, kWide, kSplit, kSplit64 };

// Keys the causal rows up to row `rows` - 1 see (key padding ignored), clamped to [0, Sk].
int64_t causal_keys(const AttnArgs& a, int64_t rows) {
  int64_t d = a.q_pos0 - a.k_pos0;  // |q_pos0|, |k_pos0| < 2^62: no overflow
  d = d < -(1LL << 40) ? -(1LL << 40) : (d > (1LL << 40) ? (1LL << 40) : d);
  const int64_t e = d + rows;
  return e < 0 ? 0 : (e > a.Sk ? a.Sk : e);
}

D128 choose_d128(const AttnArgs& a) {
  if (a.kernel == AttnArgs::kWide) return D128::kWide;
  if (a.kernel == AttnArgs::kNarrow) return D128::kNarrow;
  if (a.kernel == AttnArgs::kSplit) return D128::kSplit;
  if (a.kernel == AttnArgs::kSplit64) return D128::kSplit64;
  static std::atomic<int> cu_count[64];  // per device, filled on first use (any thread may fill it)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return D128::kNarrow;
  int cus = cu_count[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return D128::kNarrow;
    cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  if (attn_bf16_d128_wide_blocks(a) >= 2 * (int64_t)cus) return D128::kWide;
  const int64_t blocks = attn_bf16_d128_blocks(a);
  if (blocks >= 2 * (int64_t)cus) return D128::kNarrow;
  if (2 * blocks <= (int64_t)cus) return D128::kSplit64;
  if (a.causal && blocks <= (int64_t)cus && 2 * causal_keys(a, a.Sq < 128 ? a.Sq : 128) <= causal_keys(a, a.Sq))
    return D128::kSplit64;
  return D128::kSplit;
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  if (a.D == 128) {
    const D128 k = choose_d128(a);
    if (k == D128::kWide) return launch_attn_bf16_d128_wide(a, st);
    return launch_attn_bf16_d128(a, st, k == D128::kSplit    ? D128Form::kSplit
                                        : k == D128::kSplit64 ? D128Form::kSplit64
                                                              : D128Form::kNarrow);
  }
  if (a.D == 64) return launch_d<64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tha

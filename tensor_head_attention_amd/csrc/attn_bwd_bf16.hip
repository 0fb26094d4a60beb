// attn_bwd_bf16.hip -- attention backward on bf16 matrix cores (gfx950), head size 64 or 128.
//
// Gradients of the attention of attn_bf16*.hip for the cotangent dout (the chain rule through
// the softmax; the pages' training workloads need them, "Support deepspeed sequence parallel" and
// "关于数据分割和合并"; the formulas are a reading):
//   P_ij = exp(scale q_i . k_j - lse_i),  dP_ij = dout_i . v_j,  dS_ij = P_ij (dP_ij - Delta_i)
//   dv_j += sum_i P_ij dout_i,  dq_i += scale sum_j dS_ij k_j,  dk_j += scale sum_i dS_ij q_i
// with lse from the forward pass and Delta_i = dout_i . o_i from the pre-pass (attn_bwd_f32.hip).
// Products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are rounded to bf16
// as operands of the products that consume them (as the forward rounds P before P V).
//
// Two kernels, neither needs atomics, so results are deterministic:
//  * dq: a workgroup owns 128 query rows (4 wavefronts x 32) of one (b, h) and streams 64-key
//    tiles of K and V through LDS, as the forward kernels do.  Per tile a wavefront computes
//    S^T = K Q^T and dP^T = V dO^T (Q^T and dO^T are register-resident B operands), P^T and dS^T
//    in the accumulator layout (one query per lane, so lse and Delta are per-lane scalars), and
//    dQ^T += K^T dS^T with K^T read from the row-major K tile by ds_read_b64_tr_b16.
//  * dk/dv: a workgroup owns 128 keys (4 wavefronts x 32) and streams 64-query tiles of Q and
//    dO.  Per tile: S = Q K^T and dP = dO V^T (K^T and V^T register-resident), P and dS in the
//    accumulator layout (one key per lane; the 16 queries a lane holds read their lse and Delta
//    from LDS as four 4-wide vectors), dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//    by ds_read_b64_tr_b16.
// The accumulator layout puts the 16 rows of a 16-step in the order {0-3, 8-11} / {4-7, 12-15}
// between the half-waves; the transposing reads address the matching rows, so packed P / dS
// feed the next product directly (as in the forward kernels).
// Tiles read both row-wise (ds_read_b128 of 32 rows x one 16-byte chunk) and transposed (4 rows
// x 4 chunks per half-wave) use one XOR swizzle of the chunk index that is a bijection for both
// patterns: D = 128: chunk ^ ((row & 3) << 2 | (row >> 2) & 3); D = 64 (two rows per bank line):
// chunk ^ (((row >> 1) & 1) << 2 | (row >> 2) & 3).  Tiles are copied by buffer_load ... lds,
// double buffered.  Both kernels launch heaviest causal blocks first, in the XCD-aware order of
// work_item (device_common.h).
#include "device_common.h"
#include "tha_kernels.h"

namespace tha {

namespace {

constexpr int kWaves = 4, kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // owned rows per workgroup
constexpr int kTile = 64;                          // streamed rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128)
    return ((row & 3) << 2) | ((row >> 2) & 3);
  else
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

struct KArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  const int* kv_len;
  int B, Sq, Sk, H;
  int causal;
  long long q_pos0, k_pos0;
  float scale, scale_log2;
};

__device__ __forceinline__ int clamp_kv(const int* kv_len, int b, int Sk) {
  if (!kv_len) return Sk;
  const int L = kv_len[b];
  return L < 0 ? 0 : (L > Sk ? Sk : L);
}

// Per-lane offsets for copying a tile of R rows (rows of row_bytes, D bf16) into LDS, swizzled on
// the global side so the LDS side is written linearly: wave w issues R*D/2048 copies of 512/D rows
// (each copy is 64 lanes x 16 bytes = 1 KiB).
template <int D, int R = 64>
struct TileCopy {
  static constexpr int kLoads = R * D / 2048;  // per wave per tile
  static constexpr int kRowsPerLoad = 512 / D;
  static constexpr int kChunks = D / 8;
  uint32_t off[kLoads];
  __device__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int r = (wave * kLoads + u) * kRowsPerLoad + lane / kChunks;
      const int p = lane % kChunks;
      off[u] = (uint32_t)r * row_bytes + (uint32_t)((p ^ swz<D>(r)) * 16);
    }
  }
  // rows [row0, row0 + R) of a tensor whose row 0 is at base; rows >= valid_end read 0
  __device__ void copy(const __bf16* base, int64_t row_stride, int row0, int valid_end, char* dst, int wave) const {
    const int rows_valid = min(R, valid_end - row0);
    const i32x4 rs = make_rsrc_words(base + (int64_t)row0 * row_stride,
                                     (uint32_t)max(rows_valid, 0) * (uint32_t)(row_stride * 2));
    const uint32_t l = lds_addr(dst + wave * kLoads * 1024);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) buffer_load_lds_16(rs, l + u * 1024, off[u]);
  }
};

// Row-fragment read (A operand from rows): row rb*32 + lq, logical chunk 2t + hi.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int lq, int hi, int rb, int t) {
  const int row = rb * 32 + lq;
  return *(const bf16x8*)(tile + row * (D * 2) + (((2 * t + hi) ^ swz<D>(row)) * 16));
}

// Transposed fragment (A operand [dim][row]): 16-row step ks, 32-dim block db.  Lane (g, sl)
// reads rows 16ks + 4hi + sl/4 and +8, dims 32db + 16(g&1) + 4(sl&3) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int lane, int ks, int db) {
  const int g = lane >> 4, sl = lane & 15, hi = lane >> 5;
  const int c = 4 * db + 2 * (g & 1) + ((sl & 3) >> 1);
  const int r0 = 16 * ks + 4 * hi + (sl >> 2), r1 = r0 + 8;
  const int byte_in = (sl & 1) * 8;
  const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + r0 * (D * 2) + ((c ^ swz<D>(r0)) * 16) + byte_in));
  const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + r1 * (D * 2) + ((c ^ swz<D>(r1)) * 16) + byte_in));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B-operand fragments of 32 register-resident rows (row r0 + lq): dims 16t + 8hi .. +7.
template <int D>
__device__ __forceinline__ void load_rows(bf16x8 (&f)[D / 16], const __bf16* base, int64_t row_stride, int r0,
                                          int valid_end, int lq, int hi) {
  const int rows_valid = max(0, min(kRowsPerWave, valid_end - r0));
  const uint32_t row_bytes = (uint32_t)(row_stride * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)min(r0, max(valid_end - 1, 0)) * row_stride,
                                              (uint32_t)rows_valid * row_bytes);
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    f[t] = __builtin_bit_cast(bf16x8, buffer_load_16(rs, (uint32_t)lq * row_bytes + (uint32_t)(16 * t + 8 * hi) * 2));
}

// ---------------------------------------------------------------------------------------------
// dq: 128 query rows per workgroup, 64-key tiles.
template <int D>
__global__ void __launch_bounds__(kThreads, 1) bwd_dq_kernel(KArgs a) {
  constexpr int kDSteps = D / 16, kDBlocks = D / 32, kTileBytes = kTile * D * 2;
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes];  // K[0], K[1], V[0], V[1]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const int n_qt = (a.Sq + kBlockRows - 1) / kBlockRows;
  const WorkItem wi = work_item((int)blockIdx.x, n_qt, BH, true);
  const int qt = wi.tile, bh = wi.bh;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t rs = (int64_t)a.H * D;
  const int kv_lim = clamp_kv(a.kv_len, b, a.Sk);
  long long kv_end = kv_lim;
  const int q_first = qt * kBlockRows;
  if (a.causal) {
    const int q_last = min(a.Sq, q_first + kBlockRows) - 1;
    const long long last_vis = a.q_pos0 + q_last - a.k_pos0;
    if (last_vis + 1 < kv_end) kv_end = last_vis + 1 < 0 ? 0 : last_vis + 1;
  }
  const int n_kt = (int)((kv_end + kTile - 1) / kTile);

  const int q0 = q_first + wave * kRowsPerWave;
  const __bf16* qbase = a.q + (int64_t)b * a.Sq * rs + (int64_t)h * D;
  const __bf16* dbase = a.dout + (int64_t)b * a.Sq * rs + (int64_t)h * D;
  bf16x8 qf[kDSteps], df[kDSteps];
  load_rows<D>(qf, qbase, rs, q0, a.Sq, lq, hi);
  load_rows<D>(df, dbase, rs, q0, a.Sq, lq, hi);
  const int qrow = q0 + lq;
  float Lc = INFINITY, Dl = 0.f;  // P = exp2(s*c - Lc); +inf gives 0 (no key, or a row past Sq)
  if (qrow < a.Sq) {
    const float L = a.lse[(int64_t)bh * a.Sq + qrow];
    Lc = L == -INFINITY ? INFINITY : L * kLog2e;
    Dl = a.delta[(int64_t)bh * a.Sq + qrow];
  }
  long long lim_abs = kv_lim;  // key index visible to this lane's query iff key < lim_abs
  if (a.causal) {
    const long long c = a.q_pos0 + qrow - a.k_pos0 + 1;
    lim_abs = c < lim_abs ? c : lim_abs;
  }

  TileCopy<D> cp;
  cp.init(wave, lane, (uint32_t)(rs * 2));
  const __bf16* kbase = a.k + (int64_t)b * a.Sk * rs + (int64_t)h * D;
  const __bf16* vbase = a.v + (int64_t)b * a.Sk * rs + (int64_t)h * D;
  char* const kbuf = smem;
  char* const vbuf = smem + 2 * kTileBytes;

  f32x16 acc[kDBlocks];
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;

  if (n_kt > 0) {
    cp.copy(kbase, rs, 0, kv_lim, kbuf, wave);
    cp.copy(vbase, rs, 0, kv_lim, vbuf, wave);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) {
      cp.copy(kbase, rs, (kt + 1) * kTile, kv_lim, kbuf + (buf ^ 1) * kTileBytes, wave);
      cp.copy(vbase, rs, (kt + 1) * kTile, kv_lim, vbuf + (buf ^ 1) * kTileBytes, wave);
    }
    const int key0 = kt * kTile;
    bool skip = q0 >= a.Sq;
    bool need_mask = key0 + kTile > kv_lim;
    if (a.causal) {
      const long long first_kpos = a.k_pos0 + key0;
      if (first_kpos > a.q_pos0 + q0 + kRowsPerWave - 1) skip = true;
      if (first_kpos + kTile - 1 > a.q_pos0 + q0) need_mask = true;
    }
    if (!skip) {
      const char* kt_ = kbuf + buf * kTileBytes;
      const char* vt_ = vbuf + buf * kTileBytes;
      // fenced phases, as in the dk/dv kernel
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = dp[kb][j] = 0.f;
#pragma unroll
        for (int t = 0; t < kDSteps; ++t) {
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(kt_, lq, hi, kb, t), qf[t], s[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(vt_, lq, hi, kb, t), df[t], dp[kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // element j of block kb is key key0 + 32kb + 8(j/4) + 4hi + j%4 of this lane's query; it is
      // hidden iff 32kb + 8(j/4) + j%4 >= bnd (one 32-bit compare and select per element)
      long long bound = lim_abs - key0;
      bound = bound < 0 ? 0 : (bound > kTile ? kTile : bound);
      const int bnd = need_mask ? (int)bound - 4 * hi : kTile;
      bf16x8 dsb[4];  // B operands of the 16-key steps ks = 2kb + j/8
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float e = __builtin_amdgcn_exp2f(s[kb][j] * a.scale_log2 - Lc);
          const float p = kb * 32 + (j >> 2) * 8 + (j & 3) >= bnd ? 0.f : e;
          dsb[2 * kb + (j >> 3)][j & 7] = (__bf16)(p * (dp[kb][j] - Dl));  // dS^T
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(kt_, lane, ks, db), dsb[ks], acc[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of tile kt+1 has landed in LDS
    __syncthreads();
  }
  if (qrow < a.Sq) {
    float* dqrow = a.dq + ((int64_t)b * a.Sq + qrow) * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        f32x4* p = (f32x4*)(dqrow + 32 * db + 8 * jg + 4 * hi);
        f32x4 x = *p;
        x += f32x4{acc[db][4 * jg], acc[db][4 * jg + 1], acc[db][4 * jg + 2], acc[db][4 * jg + 3]} * a.scale;
        *p = x;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dk, dv: 128 keys per workgroup, 32-query tiles.  K^T is register-resident (B operand of S);
// the workgroup's 128 V rows sit in LDS for the whole kernel (B operand of dP, read as row
// fragments), so a wavefront needs ~250 registers and two workgroups (2 x 64.5 KiB of LDS for
// D = 128) share a CU: two wavefronts per SIMD.
constexpr int kTq = 32;  // query rows per streamed tile of the dk/dv kernel

template <int D>
__global__ void __launch_bounds__(kThreads, 2) bwd_dkdv_kernel(KArgs a) {
  constexpr int kDSteps = D / 16, kDBlocks = D / 32, kTileBytes = kTq * D * 2;
  // V rows of this workgroup, then Q[0], Q[1], dO[0], dO[1]
  __shared__ __attribute__((aligned(1024))) char smem[kBlockRows * D * 2 + 4 * kTileBytes];
  __shared__ __attribute__((aligned(16))) float lt[2][kTq], dt[2][kTq];  // lse*log2(e) (+inf: P = 0), Delta
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  // ascending: the earliest keys are seen by the most queries
  const WorkItem wi = work_item((int)blockIdx.x, (a.Sk + kBlockRows - 1) / kBlockRows, BH, false);
  const int kblk = wi.tile, bh = wi.bh;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t rs = (int64_t)a.H * D;
  const int kv_lim = clamp_kv(a.kv_len, b, a.Sk);
  const int key_first = kblk * kBlockRows;
  if (key_first >= kv_lim) return;  // only padding keys: seen by no query (uniform per workgroup)
  long long q_begin = 0;           // first query that sees any key of this workgroup
  if (a.causal) {
    const long long f = a.k_pos0 + key_first - a.q_pos0;
    q_begin = f < 0 ? 0 : f;
  }
  const int qt0 = (int)(q_begin / kTq);
  const int n_qt = (a.Sq + kTq - 1) / kTq;

  const int k0 = key_first + wave * kRowsPerWave;
  const __bf16* kbase = a.k + (int64_t)b * a.Sk * rs + (int64_t)h * D;
  const __bf16* vbase = a.v + (int64_t)b * a.Sk * rs + (int64_t)h * D;
  bf16x8 kf[kDSteps];
  load_rows<D>(kf, kbase, rs, k0, kv_lim, lq, hi);
  const int key = k0 + lq;
  const bool key_live = key < kv_lim;
  // causal: query index i sees this lane's key iff i >= qmin
  long long qmin = 0;
  if (a.causal) qmin = a.k_pos0 + key - a.q_pos0;

  char* const vrows = smem;
  char* const qbuf = smem + kBlockRows * D * 2;
  char* const dbuf = qbuf + 2 * kTileBytes;
  {
    TileCopy<D, 64> vc;  // the 128 V rows as two 64-row halves (the swizzle depends on row % 16 only)
    vc.init(wave, lane, (uint32_t)(rs * 2));
    vc.copy(vbase, rs, key_first, kv_lim, vrows, wave);
    vc.copy(vbase, rs, key_first + 64, kv_lim, vrows + 64 * D * 2, wave);
  }
  TileCopy<D, kTq> cp;
  cp.init(wave, lane, (uint32_t)(rs * 2));
  const __bf16* qbase = a.q + (int64_t)b * a.Sq * rs + (int64_t)h * D;
  const __bf16* dbase = a.dout + (int64_t)b * a.Sq * rs + (int64_t)h * D;
  // lse and Delta of the 32 rows of query tile t: loaded by the first 32 lanes (load_stats) and
  // stored to LDS after the tile's products (store_stats), so the loads' latency is hidden
  float st_l = -INFINITY, st_d = 0.f;
  auto load_stats = [&](int t) {
    if (tid < kTq) {
      const int r = t * kTq + tid;
      st_l = -INFINITY;
      st_d = 0.f;
      if (r < a.Sq) {
        st_l = a.lse[(int64_t)bh * a.Sq + r];
        st_d = a.delta[(int64_t)bh * a.Sq + r];
      }
    }
  };
  auto store_stats = [&](int slot) {
    if (tid < kTq) {
      lt[slot][tid] = st_l == -INFINITY ? INFINITY : st_l * kLog2e;
      dt[slot][tid] = st_d;
    }
  };

  f32x16 acck[kDBlocks], accv[kDBlocks];
#pragma unroll
  for (int i = 0; i < kDBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acck[i][j] = accv[i][j] = 0.f;

  if (qt0 < n_qt) {
    cp.copy(qbase, rs, qt0 * kTq, a.Sq, qbuf, wave);
    cp.copy(dbase, rs, qt0 * kTq, a.Sq, dbuf, wave);
    load_stats(qt0);
    store_stats(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = qt0; t < n_qt; ++t) {
    const int buf = (t - qt0) & 1;
    if (t + 1 < n_qt) {
      cp.copy(qbase, rs, (t + 1) * kTq, a.Sq, qbuf + (buf ^ 1) * kTileBytes, wave);
      cp.copy(dbase, rs, (t + 1) * kTq, a.Sq, dbuf + (buf ^ 1) * kTileBytes, wave);
      load_stats(t + 1);
    }
    const int qt0_row = t * kTq;
    bool skip = k0 >= kv_lim;
    bool need_mask = false;
    if (a.causal) {
      // wave keys k0 .. k0+31 are seen by queries >= k_pos0 + key - q_pos0
      if ((long long)qt0_row + kTq - 1 < a.k_pos0 + k0 - a.q_pos0) skip = true;
      if ((long long)qt0_row < a.k_pos0 + k0 + kRowsPerWave - 1 - a.q_pos0) need_mask = true;
    }
    if (!skip) {
      const char* qt_ = qbuf + buf * kTileBytes;
      const char* dt_ = dbuf + buf * kTileBytes;
      // The tile body runs in fenced phases (sched_barrier) so the scheduler does not hoist every
      // LDS fragment of the tile at once, which would exceed the register budget.
      f32x16 s, dp;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = dp[j] = 0.f;
#pragma unroll
      for (int d = 0; d < kDSteps; ++d) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(qt_, lq, hi, 0, d), kf[d], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(dt_, lq, hi, 0, d), row_frag<D>(vrows, lq, hi, wave, d),
                                                     dp, 0, 0, 0);
        if (d % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
      // element j is query qt0_row + 8(j/4) + 4hi + j%4 against this lane's key; it is hidden iff
      // 8(j/4) + j%4 < ithr (one 32-bit compare and select per element; a padding key hides all,
      // a tile without causal overlap none)
      long long thr = qmin - qt0_row - 4 * hi;
      thr = thr < -1 ? -1 : (thr > 2 * kTq ? 2 * kTq : thr);
      const int ithr = !key_live ? 2 * kTq : (need_mask ? (int)thr : -1);
      bf16x8 pb[2], dsb[2];  // B operands of the 16-query steps ks = j/8
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 L4 = *(const f32x4*)&lt[buf][8 * g + 4 * hi];
        const f32x4 D4 = *(const f32x4*)&dt[buf][8 * g + 4 * hi];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * g + jj;
          const float e = __builtin_amdgcn_exp2f(s[j] * a.scale_log2 - L4[jj]);
          const float pv = 8 * g + jj < ithr ? 0.f : e;
          pb[j >> 3][j & 7] = (__bf16)pv;
          dsb[j >> 3][j & 7] = (__bf16)(pv * (dp[j] - D4[jj]));  // dS
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          accv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(dt_, lane, ks, db), pb[ks], accv[db], 0, 0, 0);
          acck[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qt_, lane, ks, db), dsb[ks], acck[db], 0, 0, 0);
          if (db % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (t + 1 < n_qt) store_stats(buf ^ 1);  // the other slot: read by no wave in this tile
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (key < a.Sk) {
    float* dkrow = a.dk + ((int64_t)b * a.Sk + key) * rs + (int64_t)h * D;
    float* dvrow = a.dv + ((int64_t)b * a.Sk + key) * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hi;
        f32x4 x = *(f32x4*)(dkrow + d0);
        x += f32x4{acck[db][4 * jg], acck[db][4 * jg + 1], acck[db][4 * jg + 2], acck[db][4 * jg + 3]} * a.scale;
        *(f32x4*)(dkrow + d0) = x;
        f32x4 y = *(f32x4*)(dvrow + d0);
        y += f32x4{accv[db][4 * jg], accv[db][4 * jg + 1], accv[db][4 * jg + 2], accv[db][4 * jg + 3]};
        *(f32x4*)(dvrow + d0) = y;
      }
  }
}

template <int D>
hipError_t launch_d(const AttnBwdArgs& x, hipStream_t st) {
  KArgs a;
  a.q = (const __bf16*)x.q, a.k = (const __bf16*)x.k, a.v = (const __bf16*)x.v, a.dout = (const __bf16*)x.dout;
  a.lse = x.lse, a.delta = x.delta, a.dq = x.dq, a.dk = x.dk, a.dv = x.dv, a.kv_len = x.kv_len;
  a.B = x.B, a.Sq = x.Sq, a.Sk = x.Sk, a.H = x.H;
  a.causal = x.causal ? 1 : 0;
  a.q_pos0 = x.q_pos0, a.k_pos0 = x.k_pos0;
  a.scale = x.scale, a.scale_log2 = x.scale * kLog2e;
  const int64_t BH = (int64_t)x.B * x.H;
  const int64_t qblocks = (int64_t)((x.Sq + kBlockRows - 1) / kBlockRows) * BH;
  const int64_t kblocks = (int64_t)((x.Sk + kBlockRows - 1) / kBlockRows) * BH;
  if (qblocks > 0x7fffffff || kblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)qblocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)kblocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t st) {
  if (a.D == 128) return launch_d<128>(a, st);
  if (a.D == 64) return launch_d<64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tha

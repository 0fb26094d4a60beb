// attn_epilogue.h -- the output step shared by the bf16 attention kernels (attn_bf16.hip,
// attn_bf16_d128.hip, attn_bf16_d128_wide.hip): O = O^T / l and lse = m * scale + ln(l) for one
// lane's query row, or, in accumulate mode, the log-sum-exp merge of that result into a running
// fp32 result over other keys ("adv07: Sequence Parallel" Q5: the Ring step that accumulates
// block results into the full attention; the merge rule is attn_merge_lse's).
#pragma once
#include "device_common.h"

namespace tha {

// acc[db] holds, for this lane's query row, the 16 accumulator elements of 32-dim block db at
// dims 32db + 8(j/4) + 4hi + j%4 (the v_mfma_f32_32x32x16_bf16 accumulator layout of O^T).
// l_tot: the row's softmax sum (both half-waves hold it); m_run: its reference max (raw score).
// orow: the row's D outputs; lse_p: the row's lse (may be null when not accumulating).
// Accumulate mode (OutT = float only): every lane of the row reads the running lse before the
// half-wave-0 lane writes the merged one (one instruction stream, data dependent); a running lse
// of -inf marks a row with no keys yet, whose o is not read.
template <int NB, typename OutT>
__device__ __forceinline__ void store_row(const f32x16 (&acc)[NB], OutT* orow, float* lse_p, int hi, float l_tot,
                                          float m_run, float scale, bool accumulate) {
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse_c = l_tot > 0.f ? m_run * scale + logf(l_tot) : -INFINITY;
  if constexpr (sizeof(OutT) == 4) {
    if (accumulate) {
      const MergeW w = merge_weights(*lse_p, lse_c);
      const float cw = w.c * inv;
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          f32x4* p = (f32x4*)(orow + 32 * db + 8 * jg + 4 * hi);
          f32x4 x = f32x4{acc[db][4 * jg], acc[db][4 * jg + 1], acc[db][4 * jg + 2], acc[db][4 * jg + 3]} * cw;
          if (w.a != 0.f) x += *p * w.a;
          *p = x;
        }
      if (hi == 0) *lse_p = w.lse;
      return;
    }
  }
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = 32 * db + 8 * jg + 4 * hi;
      if constexpr (sizeof(OutT) == 2) {
        bf16x4 r = {(__bf16)(acc[db][4 * jg] * inv), (__bf16)(acc[db][4 * jg + 1] * inv),
                    (__bf16)(acc[db][4 * jg + 2] * inv), (__bf16)(acc[db][4 * jg + 3] * inv)};
        *(bf16x4*)(orow + d0) = r;
      } else {
        f32x4 r = {acc[db][4 * jg] * inv, acc[db][4 * jg + 1] * inv, acc[db][4 * jg + 2] * inv,
                   acc[db][4 * jg + 3] * inv};
        *(f32x4*)(orow + d0) = r;
      }
    }
  if (lse_p && hi == 0) *lse_p = lse_c;
}

}  // namespace tha

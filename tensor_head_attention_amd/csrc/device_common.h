// device_common.h -- small CDNA4 (gfx950) helpers shared by the library's kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;

// Buffer resource word 3 for raw (untyped, unswizzled) buffer access on gfx9-class parts:
// 32-bit data format, no index stride.  Loads at offsets >= num_records return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// The base and size must be wave-uniform; readfirstlane states that to the compiler so the
// descriptor lives in SGPRs (a descriptor it believes divergent costs a loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* up = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, (short)0, (int)__builtin_amdgcn_readfirstlane(num_bytes),
                                           kBufferRsrcWord3);
}

// The same descriptor as four raw dwords (for the inline-asm copy below).
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t num_bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = (int)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);  // stride 0
  r[2] = (int)__builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = kBufferRsrcWord3;
  return r;
}

// Direct global -> LDS copy (buffer_load_dwordx4 ... lds): lane i's 16 bytes, read at byte
// offset voff of the buffer (zero when out of range), land at LDS byte lds_base + 16*i.
// lds_base must be wave-uniform.  Written as inline asm so the compiler does not order later
// LDS reads behind it; the caller waits (vmcnt) before a barrier that publishes the data.
// The kernels that use it issue no other M0-based instruction.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set inside the statement on purpose
__device__ __forceinline__ void buffer_load_lds_16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_char*)p);
}

__device__ __forceinline__ i32x4 buffer_load_16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// Exchange a value with the lane 32 positions away; returns (own, partner) combined by the caller.
// v_permlane32_swap swaps the upper half of the first operand with the lower half of the second;
// calling it with (x, x) leaves {x_low, x_high} in the two results on every lane.
__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Weights that fold a chunk's attention result (o_c, lse_c) into a running one (o_r, lse_r) over
// a disjoint key set, by the log-sum-exp rule of attn_merge_lse: o = a*o_r + c*o_c, lse = lse.
// Neither side saw a key: a = c = 0, lse = -inf.  A chunk that saw no key gives a = 1, c = 0 and
// lse = lse_r exactly.
struct MergeW {
  float a, c, lse;
};
__device__ __forceinline__ MergeW merge_weights(float lse_r, float lse_c) {
  const float M = fmaxf(lse_r, lse_c);
  if (M == -INFINITY) return {0.f, 0.f, -INFINITY};
  const float wr = expf(lse_r - M), wc = expf(lse_c - M);
  const float W = wr + wc;
  return {wr / W, wc / W, M + logf(W)};
}

// Work order of the attention kernels: workgroup `blk` of a grid of n_tiles x BH (tile index,
// (batch, head)) items.  Workgroups reach the 8 XCDs round-robin (blk % 8), each XCD with its own
// L2.  When BH is a multiple of 8, the workgroups one XCD receives walk one (batch, head) at a time,
// so the K/V (or Q/dO) rows they stream are shared in that XCD's L2; otherwise consecutive
// workgroups take consecutive (batch, head)s.  Within a (batch, head) the tiles come in the order
// `first`, first +- 1, ... (`descending` = last tile first).  Any order is correct: it is a bijection
// of [0, n_tiles * BH).
constexpr int kXcds = 8;
struct WorkItem {
  int tile, bh;
};
__device__ __forceinline__ WorkItem work_item(int blk, int n_tiles, int BH, bool descending) {
  int t, bh;
  if (BH % kXcds == 0) {
    const int x = blk % kXcds, slot = blk / kXcds;
    const int bl = slot / n_tiles;
    t = slot - bl * n_tiles;
    bh = bl * kXcds + x;
  } else {
    t = blk / BH;
    bh = blk - t * BH;
  }
  return {descending ? n_tiles - 1 - t : t, bh};
}

// Block order of the streaming kernels: workgroups reach the XCDs round-robin (blk % 8), and this
// maps them so that XCD x takes the contiguous block range [x*q + min(x, r), ...) of a grid of
// nb = 8q + r blocks.  Each XCD then streams its own contiguous share of the rows, and no cache line
// of a row-indexed array (an lse vector read or written 4 bytes per row, the output) is shared by
// the L2s of several XCDs.  A bijection on [0, nb); any order is correct.
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t blk, uint32_t nb) {
  const uint32_t q = nb / kXcds, r = nb % kXcds, x = blk % kXcds, slot = blk / kXcds;
  return x * q + (x < r ? x : r) + slot;
}

// Round-to-nearest-even fp32 -> bf16 pair (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace tha

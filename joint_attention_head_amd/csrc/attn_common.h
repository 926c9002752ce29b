// Device helpers shared by the two attention kernels (bf16 MFMA and fp8
// MFMA): vector types, buffer descriptors, conversions, the ping-pong wave
// grouping and the XCD-aware block order.
#pragma once

#include "fluxattn_internal.h"

namespace fluxattn {
namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr uint32_t kRsrcWord3 = 0x00020000u;      // raw buffer, 32-bit data format

template <int R>
struct Slot {
  static constexpr int value = R;
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Four fp32 -> four E4M3 codes (round to nearest even), byte i = value i.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// The same into a register whose old contents are dead: the first convert
// writes only the low half, so passing the old word (instead of 0) spares
// the v_mov that would clear the high half; the second convert overwrites it.
__device__ __forceinline__ uint32_t f32x4_to_e4m3_over(float a, float b, float c, float d, int old) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Raw buffer descriptor words (base, no stride, `bytes` records, 32-bit
// data format); out-of-range offsets read as zero.
__device__ __forceinline__ i32x4_t rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = (int)(uint32_t)p;
  r[1] = (int)((uint32_t)(p >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = (int)kRsrcWord3;
  return r;
}

// Position of this wave in the ping-pong order of an 8-wave workgroup:
// waves sorted by (SIMD, wave id), so consecutive positions share a SIMD
// and alternate between the two groups.  `simd_of_wave` is an 8-entry LDS
// array; the call contains a workgroup barrier.
__device__ __forceinline__ int pingpong_order(int *simd_of_wave, int wave, int lane) {
  if (lane == 0) simd_of_wave[wave] = (int)__builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));
  __syncthreads();
  int order = 0;
  const int mine = simd_of_wave[wave] * 8 + wave;
#pragma unroll
  for (int w = 0; w < 8; ++w) order += (simd_of_wave[w] * 8 + w) < mine;
  // the sort key is the same in every lane of a wave: keep it scalar
  return __builtin_amdgcn_readfirstlane(order);
}

// Logical block of a dispatched block id: the dispatcher deals blocks to
// the 8 XCDs round-robin (XCD = id % 8), and each XCD gets a contiguous
// range of logical blocks, so consecutive query tiles of one (b,h) share
// that XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int total) {
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  return xcd * q8 + min(xcd, r8) + (bid >> 3);
}

// One (b,h) head of a [B,H,N,D] view: base pointer, bytes per token row,
// and the buffer extent (ends with row N-1, so rows past N read as zero
// and stores there are dropped).
struct HeadView {
  const char *base;
  uint32_t row;
  uint32_t bytes;
};

template <bool STRIDED>
__device__ __forceinline__ HeadView head_view(const void *p, const Strides &st, int esize, int bh, int H, int N) {
  HeadView v;
  if constexpr (STRIDED) {
    const int64_t b = bh / H, h = bh - b * H;
    v.base = static_cast<const char *>(p) + (b * st.b + h * st.h) * esize;
    v.row = (uint32_t)st.n * (uint32_t)esize;
    v.bytes = (uint32_t)(N - 1) * v.row + (uint32_t)(kHeadDim * esize);
  } else {
    v.base = static_cast<const char *>(p) + (size_t)bh * N * kHeadDim * esize;
    v.row = (uint32_t)(kHeadDim * esize);
    v.bytes = (uint32_t)N * v.row;
  }
  return v;
}

// Buffer descriptor words of key tile t (tile_keys rows) of a head, for the
// direct global -> LDS copies: base moved to the tile, records cut to what
// is left of the head, so lane offsets stay tile-independent.  Scalar
// arithmetic only.
__device__ __forceinline__ i32x4_t tile_words(const HeadView &v, int t, int tile_keys) {
  const uint32_t skip = (uint32_t)t * (uint32_t)tile_keys * v.row;
  return rsrc_words(v.base + skip, v.bytes - skip);
}

// Norm weights of a token's stream.
__device__ __forceinline__ const float *stream_weights(const ForwardArgs &a, int tok) {
  const int sid = (tok >= a.streams.start[1]) + (tok >= a.streams.start[2]) + (tok >= a.streams.start[3]);
  return a.w_q + sid * kHeadDim;
}

// Rotation angle of head-dim pair `pr` of a token at positions pos[3], as
// (sin, cos): the frequency is 2^(j * rope_log2_step[axis]) for the pair's
// index j inside its axis block; the angle is reduced to [0, 1) revolutions
// and fed to the hardware sin / cos (absolute error about 1e-6 + 4e-8 |angle|
// rad, the size of the fp32 rounding of the angle itself at FLUX's positions).
__device__ __forceinline__ void pair_rotation(const ForwardArgs &a, const int32_t (&pos)[3], int pr, float &sn,
                                              float &cs) {
  const int ax = pr < a.rope_first[1] ? 0 : (pr < a.rope_first[2] ? 1 : 2);
  const int jj = pr - (ax == 0 ? 0 : (ax == 1 ? a.rope_first[1] : a.rope_first[2]));
  const float step = ax == 0 ? a.rope_log2_step[0] : (ax == 1 ? a.rope_log2_step[1] : a.rope_log2_step[2]);
  const int32_t p = ax == 0 ? pos[0] : (ax == 1 ? pos[1] : pos[2]);
  const float rev = __builtin_amdgcn_fractf((float)p * exp2f((float)jj * step) * 0.15915494309189535f);
  sn = __builtin_amdgcn_sinf(rev);
  cs = __builtin_amdgcn_cosf(rev);
}

}  // namespace attn
}  // namespace fluxattn

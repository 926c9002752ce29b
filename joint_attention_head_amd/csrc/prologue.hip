// Fused per-head RMSNorm + 3-axis RoPE on queries and keys (gfx950).
//
// The QKV projection of a FLUX-style MM-DiT block is followed by query/key
// normalisation and a rotary position embedding (NVIDIA blog post "Speed up
// image generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
// "GEMM kernel optimization").  This kernel is the standalone form of that
// step; it is bound by HBM bandwidth (about 1.5 flop per byte).
//
// Work decomposition: a 256-thread block owns 16 consecutive tokens.  Lane
// group g (16 lanes) holds token g, and lane c of the group owns head dims
// [8c, 8c+8) = rotation pairs 4c..4c+3.  The four rotation angles of a lane
// depend only on its token, so their sin/cos are evaluated once (the angle
// in revolutions, reduced to one turn, through the hardware sine and
// cosine: absolute error about 1e-6 rad plus the fp32 rounding of the
// product, 6e-8 of the angle) and reused
// for the (b,h) rows of Q and of K that the block walks: all of them, or a
// chunk of them per grid.y index where the token blocks alone would leave
// the chip short of work (bf16: fewer than about 1024 blocks).  For a fixed
// (b,h) the block reads and writes one contiguous 4 KiB (bf16) or 2 KiB
// (fp8) span.
#include "fluxattn_internal.h"

#include <algorithm>

namespace fluxattn {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = kThreads / 16;
constexpr int kUnroll = 4;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;  // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// DPP moves inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row: xor 1, xor 2 (quad permutes), then the
// half-row mirror (lane i <-> 7-i) and the row mirror (lane i <-> 15-i).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Normalise and rotate the 8 values of one lane: f holds x (dequantised),
// w the lane's 8 weights, cs/sn the 4 pair angles.  rstd comes from the sum
// of squares over the whole 128-dim row.
__device__ __forceinline__ void norm_rope8(float (&f)[8], const float (&w)[8],
                                           const float (&cs)[4], const float (&sn)[4],
                                           float eps) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
  ss = row16_sum(ss);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = f[2 * i] * w[2 * i] * rstd;
    const float v = f[2 * i + 1] * w[2 * i + 1] * rstd;
    f[2 * i] = u * cs[i] - v * sn[i];
    f[2 * i + 1] = u * sn[i] + v * cs[i];
  }
}

// Walks the heads bh = 0, 1, 2, ... (b = bh / H, h = bh % H) of an input
// and an output view, keeping each head's element offset b*st.b + h*st.h
// without a division.  Every value is uniform over the workgroup.
struct HeadWalk {
  int64_t in, out;   // offsets of the current head in the two views
  int32_t h;
  __device__ __forceinline__ void next(const Strides &si, const Strides &so, int32_t H) {
    if (++h == H) {
      h = 0;
      in += si.b - (int64_t)(H - 1) * si.h;
      out += so.b - (int64_t)(H - 1) * so.h;
    } else {
      in += si.h;
      out += so.h;
    }
  }
};

// Stream (norm-weight set) of a token.
__device__ __forceinline__ int stream_of(const Streams &ss, int tok) {
  return (tok >= ss.start[1]) + (tok >= ss.start[2]) + (tok >= ss.start[3]);
}

__device__ __forceinline__ void lane_angles(const PrologueArgs &a, const RopeTable &t,
                                            int tok, int c, float (&cs)[4], float (&sn)[4]) {
  const int32_t p0 = a.pos[3 * (int64_t)tok + 0];
  const int32_t p1 = a.pos[3 * (int64_t)tok + 1];
  const int32_t p2 = a.pos[3 * (int64_t)tok + 2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pr = 4 * c + i;
    const int ax = t.axis[pr];
    const int32_t p = ax == 0 ? p0 : (ax == 1 ? p1 : p2);
    const float rev = __builtin_amdgcn_fractf((float)p * t.freq[pr]);
    sn[i] = __builtin_amdgcn_sinf(rev);
    cs[i] = __builtin_amdgcn_cosf(rev);
  }
}

__global__ __launch_bounds__(kThreads) void prologue_bf16_kernel(PrologueArgs a, RopeTable t) {
  const int c = threadIdx.x & 15;
  const int tok = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 4);
  if (tok >= a.N) return;  // the 16 lanes of a token leave together

  float cs[4], sn[4];
  lane_angles(a, t, tok, c, cs, sn);

  const int64_t bh_begin = (int64_t)blockIdx.y * a.bh_chunk;
  const int64_t bh_end = min((int64_t)a.BH, bh_begin + a.bh_chunk);
  const int sid = stream_of(a.streams, tok);
  for (int which = a.q ? 0 : 1; which < 2; ++which) {   // no q: keys only
    const uint16_t *src = static_cast<const uint16_t *>(which ? a.k : a.q);
    uint16_t *dst = static_cast<uint16_t *>(which ? a.k_out : a.q_out);
    const Strides &si = which ? a.sk : a.sq;
    const Strides &so = which ? a.sko : a.sqo;
    const float *wp = (which ? a.w_k : a.w_q) + sid * kHeadDim;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = wp[8 * c + i];

    const int64_t tin = (int64_t)tok * si.n + 8 * c, tout = (int64_t)tok * so.n + 8 * c;
    HeadWalk walk;
    {
      const int64_t b = bh_begin / a.H, h = bh_begin - b * a.H;
      walk.in = b * si.b + h * si.h;
      walk.out = b * so.b + h * so.h;
      walk.h = (int32_t)h;
    }
    for (int64_t bh0 = bh_begin; bh0 < bh_end; bh0 += kUnroll) {
      int64_t oin[kUnroll], oout[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        oin[u] = walk.in + tin;
        oout[u] = walk.out + tout;
        walk.next(si, so, a.H);
      }
      uint4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (bh0 + u < bh_end) x[u] = *reinterpret_cast<const uint4 *>(src + oin[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (bh0 + u >= bh_end) break;
        float f[8] = {bf16_lo(x[u].x), bf16_hi(x[u].x), bf16_lo(x[u].y), bf16_hi(x[u].y),
                      bf16_lo(x[u].z), bf16_hi(x[u].z), bf16_lo(x[u].w), bf16_hi(x[u].w)};
        norm_rope8(f, w, cs, sn, a.eps);
        uint4 y;
        y.x = pack_bf16(f[0], f[1]);
        y.y = pack_bf16(f[2], f[3]);
        y.z = pack_bf16(f[4], f[5]);
        y.w = pack_bf16(f[6], f[7]);
        *reinterpret_cast<uint4 *>(dst + oout[u]) = y;
      }
    }
  }
}

// OCP E4M3 pair decode / encode with the gfx950 conversion instructions.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *f) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

__device__ __forceinline__ uint32_t f32x4_to_e4m3(const float *f) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w, true);
  return (uint32_t)w;
}

// fp8 rows are 128 B: 8 lanes per token, 16 codes (8 rotation pairs) per
// lane, so every lane moves 16 bytes per load and store; 32 tokens per block.
// The (b,h) rows are split over grid.y in chunks of a.bh_chunk (sized on
// the host for about twelve blocks per compute unit), which gives the
// half-size fp8 stream enough blocks in flight.
constexpr int kLanes8 = 8;
constexpr int kTokensPerBlock8 = kThreads / kLanes8;
constexpr int64_t kMaxGridY = 65535;

__device__ __forceinline__ float row8_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
  return x;
}

__global__ __launch_bounds__(kThreads) void prologue_fp8_kernel(PrologueArgs a, RopeTable t) {
  const int lane = threadIdx.x & 63;
  // Output scale sqrt(D) * max|w| / 448: every output lies within +-448 of it.
  float sq, sk;
  {
    float mq = 0.f, mk = 0.f;
    for (int st = 0; st < a.num_streams; ++st) {
      if (a.w_q) mq = fmaxf(mq, fmaxf(fabsf(a.w_q[st * kHeadDim + lane]), fabsf(a.w_q[st * kHeadDim + lane + 64])));
      mk = fmaxf(mk, fmaxf(fabsf(a.w_k[st * kHeadDim + lane]), fabsf(a.w_k[st * kHeadDim + lane + 64])));
    }
    mq = wave_max(mq);
    mk = wave_max(mk);
    const float root_d = 11.313708498984760f;  // sqrt(128)
    sq = mq > 0.f ? root_d * mq / 448.f : 1.f;
    sk = mk > 0.f ? root_d * mk / 448.f : 1.f;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int64_t i = threadIdx.x; i < a.BH; i += kThreads) {
      if (a.q_scale_out) a.q_scale_out[i] = sq;
      a.k_scale_out[i] = sk;
    }
  }
  const int c = threadIdx.x & 7;
  const int tok = blockIdx.x * kTokensPerBlock8 + (threadIdx.x >> 3);
  if (tok >= a.N) return;  // the 8 lanes of a token leave together

  // the lane's 8 pairs 8c .. 8c+7: angles once per token
  float cs[8], sn[8];
  {
    const int32_t p0 = a.pos[3 * (int64_t)tok + 0];
    const int32_t p1 = a.pos[3 * (int64_t)tok + 1];
    const int32_t p2 = a.pos[3 * (int64_t)tok + 2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pr = 8 * c + i;
      const int ax = t.axis[pr];
      const int32_t p = ax == 0 ? p0 : (ax == 1 ? p1 : p2);
      const float rev = __builtin_amdgcn_fractf((float)p * t.freq[pr]);
      sn[i] = __builtin_amdgcn_sinf(rev);
      cs[i] = __builtin_amdgcn_cosf(rev);
    }
  }

  const int64_t bh_begin = (int64_t)blockIdx.y * a.bh_chunk;
  const int64_t bh_end = min((int64_t)a.BH, bh_begin + a.bh_chunk);
  const int sid = stream_of(a.streams, tok);
  for (int which = a.q ? 0 : 1; which < 2; ++which) {   // no q: keys only
    const uint8_t *src = static_cast<const uint8_t *>(which ? a.k : a.q);
    uint8_t *dst = static_cast<uint8_t *>(which ? a.k_out : a.q_out);
    const Strides &si = which ? a.sk : a.sq;
    const Strides &so = which ? a.sko : a.sqo;
    const float *wp = (which ? a.w_k : a.w_q) + sid * kHeadDim;
    const float *s_in = which ? a.k_scale : a.q_scale;
    const float inv_out = 1.0f / (which ? sk : sq);
    // weights times the rotation of each of the lane's pairs (even dim e,
    // odd dim o): out_e = u w_e cos - v w_o sin, out_o = u w_e sin + v w_o cos
    float ra[8], rb[8], rc[8], rd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float we = wp[16 * c + 2 * i], wo = wp[16 * c + 2 * i + 1];
      ra[i] = we * cs[i];
      rb[i] = wo * sn[i];
      rc[i] = we * sn[i];
      rd[i] = wo * cs[i];
    }

    const int64_t tin = (int64_t)tok * si.n + 16 * c, tout = (int64_t)tok * so.n + 16 * c;
    HeadWalk walk;
    {
      const int64_t b = bh_begin / a.H, h = bh_begin - b * a.H;
      walk.in = b * si.b + h * si.h;
      walk.out = b * so.b + h * so.h;
      walk.h = (int32_t)h;
    }
    for (int64_t bh0 = bh_begin; bh0 < bh_end; bh0 += kUnroll) {
      int64_t oin[kUnroll], oout[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        oin[u] = walk.in + tin;
        oout[u] = walk.out + tout;
        walk.next(si, so, a.H);
      }
      uint4 x[kUnroll];
      float s[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (bh0 + u < bh_end) {
          x[u] = *reinterpret_cast<const uint4 *>(src + oin[u]);
          s[u] = s_in[bh0 + u];
        }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (bh0 + u >= bh_end) break;
        float f[16];
        e4m3x4_to_f32(x[u].x, f);
        e4m3x4_to_f32(x[u].y, f + 4);
        e4m3x4_to_f32(x[u].z, f + 8);
        e4m3x4_to_f32(x[u].w, f + 12);
        // The row is s * codes: its sum of squares is s^2 times that of the
        // codes, and x w rstd = codes w (s rstd), so the dequantisation
        // scale and the output scale meet in one factor g per row.
        float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ss0 = fmaf(f[2 * i], f[2 * i], ss0);
          ss1 = fmaf(f[2 * i + 1], f[2 * i + 1], ss1);
        }
        const float ss = row8_sum(ss0 + ss1);
        const float su = s[u];
        const float g = su * __builtin_amdgcn_rsqf((su * su) * ss * (1.0f / kHeadDim) + a.eps) * inv_out;
        // |out| <= sqrt(D) max|w| / s_out = 448 up to fp32 rounding, and the
        // conversion rounds everything below 464 to 448: no clamp.  (eps = 0
        // with an all-zero row gives 0/0 = NaN, as in the bf16 path.)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float uu = f[2 * i] * g, vv = f[2 * i + 1] * g;
          f[2 * i] = fmaf(uu, ra[i], -vv * rb[i]);
          f[2 * i + 1] = fmaf(uu, rc[i], vv * rd[i]);
        }
        uint4 y;
        y.x = f32x4_to_e4m3(f);
        y.y = f32x4_to_e4m3(f + 4);
        y.z = f32x4_to_e4m3(f + 8);
        y.w = f32x4_to_e4m3(f + 12);
        *reinterpret_cast<uint4 *>(dst + oout[u]) = y;
      }
    }
  }
}

}  // namespace

// (b,h) rows per block along grid.y for bx token blocks: the fewest chunks
// that give about `blocks` blocks in all, each a multiple of the 4-row
// unroll, and grid.y within its limit
int32_t bh_chunk_for(int64_t BH, int64_t bx, int64_t blocks) {
  const int64_t want = std::max<int64_t>(1, (blocks + bx - 1) / bx);
  int64_t chunk = (BH + want - 1) / want;
  chunk = (chunk + kUnroll - 1) / kUnroll * kUnroll;
  return (int32_t)std::max<int64_t>(chunk, (BH + kMaxGridY - 1) / kMaxGridY);
}

hipError_t launch_prologue_bf16(const PrologueArgs &a, const RopeTable &t, hipStream_t s) {
  PrologueArgs b = a;
  const int64_t bx = (a.N + kTokensPerBlock - 1) / kTokensPerBlock;
  b.bh_chunk = bh_chunk_for(a.BH, bx, 1024);   // about four blocks per compute unit
  const dim3 grid((unsigned)bx, (unsigned)((a.BH + b.bh_chunk - 1) / b.bh_chunk));
  hipLaunchKernelGGL(prologue_bf16_kernel, grid, dim3(kThreads), 0, s, b, t);
  return hipGetLastError();
}

hipError_t launch_prologue_fp8(const PrologueArgs &a, const RopeTable &t, hipStream_t s) {
  PrologueArgs b = a;
  const int64_t bx = (a.N + kTokensPerBlock8 - 1) / kTokensPerBlock8;
  b.bh_chunk = bh_chunk_for(a.BH, bx, 3072);   // the half-size fp8 stream: about twelve per compute unit
  const dim3 grid((unsigned)bx, (unsigned)((a.BH + b.bh_chunk - 1) / b.bh_chunk));
  hipLaunchKernelGGL(prologue_fp8_kernel, grid, dim3(kThreads), 0, s, b, t);
  return hipGetLastError();
}

}  // namespace fluxattn

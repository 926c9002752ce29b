// Non-causal joint attention O = softmax(Q K^T * scale) V on gfx950 MFMA.
//
// Dense attention over the merged text + image (+ reference) tokens is the
// dominant kernel of a FLUX-style DiT step (NVIDIA blog post "Speed up image
// generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
// "Quantized and sparse attention"); queries and keys arrive normalised and
// rotated (section "GEMM kernel optimization").
//
// Design (flash-style, one pass over K/V, scores never leave registers):
//   * A workgroup owns BR = 4 waves x 32*QB query rows of one (b,h).  Each
//     wave keeps its queries in VGPRs as the B operand of
//     v_mfma_f32_32x32x16_bf16 and computes the transposed score tile
//     S^T = K Q^T, so every lane ends up owning one query (lane % 32) and 16
//     keys per 32-key block.  The softmax row state (max, sum) is then
//     lane-local except for one exchange with lane ^ 32.
//   * O^T = V^T P^T uses the probabilities straight from registers as the B
//     operand; V^T comes from LDS.  Because keys are summed over, the kernel
//     permutes keys inside each group of 16 (swap of key bits 2 and 3) so
//     that the keys a lane holds for one MFMA step are 8 consecutive LDS
//     elements: one ds_read_b128 per operand.
//   * K and V^T tiles of BC = 64 keys are double-buffered in LDS (64 KiB):
//     the next tile is fetched into registers while the current one is
//     consumed, then written to the other buffer; one barrier per tile.
//   * Online softmax in base 2 (scale * log2 e folded into one FMA).  The
//     running max is only moved, and O and l rescaled, when some row's max
//     grows by more than 8 (log2 units), so most tiles skip the rescale;
//     probabilities stay <= 2^8 and the final O / l is unchanged.
//   * The normaliser l sums the bf16-rounded probabilities that the MFMA
//     consumes (v_dot2 with ones), so V == 1 gives exactly 1.
//   * blockIdx is remapped so that the workgroups that the dispatcher sends
//     to one XCD (blockIdx % 8) cover consecutive query tiles of the same
//     (b,h): their K/V stream is shared through that XCD's L2.
//   * fp8 (OCP E4M3) inputs are widened to bf16 on load, which is exact, and
//     the per-(b,h) scales are folded into the softmax scale (q, k) and the
//     final normalisation (v).
#include "fluxattn_internal.h"

#include <atomic>

namespace fluxattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBC = 64;                           // keys per tile
constexpr int kKTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = key
constexpr int kVTileBytes = kHeadDim * kBC * 2;   // 16 KiB, row = head dim
constexpr int kStageBytes = kKTileBytes + kVTileBytes;
constexpr int kLdsBytes = 2 * kStageBytes;        // 64 KiB

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3 codes -> four bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return make_uint2(pack_bf16(lo[0], lo[1]), pack_bf16(hi[0], hi[1]));
}

// 16 bytes = 8 consecutive head-dim elements of one row, widened to bf16.
template <bool FP8>
__device__ __forceinline__ uint4 load_chunk(const void *base, int64_t elem, bool valid) {
  if (!valid) return make_uint4(0, 0, 0, 0);
  if constexpr (FP8) {
    const uint2 r = *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(base) + elem);
    const uint2 a = e4m3x4_to_bf16x4(r.x), b = e4m3x4_to_bf16x4(r.y);
    return make_uint4(a.x, a.y, b.x, b.y);
  } else {
    return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
  }
}

// Position of key `key` (0..63 inside the tile) in a V^T row: swap bits 2, 3.
__device__ __forceinline__ int vperm(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Byte offset of the 16-byte chunk `ch` of K row `row` (XOR swizzle on 8).
__device__ __forceinline__ int k_off(int row, int ch) { return row * 256 + ((ch ^ (row & 7)) << 4); }
// Byte offset of the 16-byte chunk `ch` (8 permuted keys) of V^T row `d`.
__device__ __forceinline__ int v_off(int d, int ch) { return d * 128 + ((ch ^ (d & 7)) << 4); }

struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};

template <bool FP8>
__device__ __forceinline__ void fetch_tile(TileRegs &r, const void *K, const void *V, int64_t head_off,
                                           int kv0, int N, int tid) {
  // K: chunk idx = tid + 256 i -> key row idx / 16, head-dim chunk idx % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 4, ch = idx & 15;
    const int key = kv0 + row;
    r.k[i] = load_chunk<FP8>(K, head_off + (int64_t)key * kHeadDim + 8 * ch, key < N);
  }
  // V: lane owns keys 4*kg .. 4*kg+3 of head-dim chunk dc
  const int kg = tid & 15, dc = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kv0 + 4 * kg + i;
    r.v[i] = load_chunk<FP8>(V, head_off + (int64_t)key * kHeadDim + 8 * dc, key < N);
  }
}

__device__ __forceinline__ void store_tile(const TileRegs &r, char *stage, int tid) {
  char *ks = stage;
  char *vs = stage + kKTileBytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 4, ch = idx & 15;
    *reinterpret_cast<uint4 *>(ks + k_off(row, ch)) = r.k[i];
  }
  // Transpose 4 keys x 8 dims into 8 V^T rows of 4 (permuted, consecutive) keys.
  const int kg = tid & 15, dc = tid >> 4;
  const int kp = vperm(4 * kg);      // multiple of 4: the 4 keys stay adjacent
  const int ch = kp >> 3, within = (kp & 7) * 2;
  const uint32_t *x0 = reinterpret_cast<const uint32_t *>(&r.v[0]);
  const uint32_t *x1 = reinterpret_cast<const uint32_t *>(&r.v[1]);
  const uint32_t *x2 = reinterpret_cast<const uint32_t *>(&r.v[2]);
  const uint32_t *x3 = reinterpret_cast<const uint32_t *>(&r.v[3]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    const int w = j >> 1;
    uint2 out;
    out.x = __builtin_amdgcn_perm(x1[w], x0[w], sel);
    out.y = __builtin_amdgcn_perm(x3[w], x2[w], sel);
    const int d = 8 * dc + j;
    *reinterpret_cast<uint2 *>(vs + v_off(d, ch) + within) = out;
  }
}

__device__ __forceinline__ bf16x8_t lds_read16(const char *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}

template <int QB, bool FP8>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(ForwardArgs a) {
  constexpr int BR = kWaves * 32 * QB;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;

  // blockIdx -> (b*h, query tile); the tiles dispatched to one XCD are
  // consecutive in (b*h, tile) order.
  const int ntiles = (N + BR - 1) / BR;
  const int total = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  const int logical = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int bh = logical / ntiles;
  const int qt = logical - bh * ntiles;
  const int64_t head_off = (int64_t)bh * N * kHeadDim;

  float c = a.scale_log2;
  float o_scale = 1.f;
  if constexpr (FP8) {
    c *= a.q_scale[bh] * a.k_scale[bh];
    o_scale = a.v_scale[bh];
  }

  // Query fragments: qf[qb][kk] = Q[q][16kk + 8hi .. +8), q = row of lane.
  bf16x8_t qf[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qt * BR + (wave * QB + qb) * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 r = load_chunk<FP8>(a.q, head_off + (int64_t)q * kHeadDim + 16 * kk + 8 * hi, q < N);
      qf[qb][kk] = __builtin_bit_cast(bf16x8_t, r);
    }
  }

  f32x16_t o[QB][4];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const int T = (N + kBC - 1) / kBC;
  TileRegs regs;
  fetch_tile<FP8>(regs, a.k, a.v, head_off, 0, N, tid);
  store_tile(regs, lds, tid);
  __syncthreads();

  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (int t = 0; t < T; ++t) {
    const char *stage = lds + (t & 1) * kStageBytes;
    const char *ks = stage;
    const char *vs = stage + kKTileBytes;
    const int kv0 = t * kBC;
    if (t + 1 < T) fetch_tile<FP8>(regs, a.k, a.v, head_off, kv0 + kBC, N, tid);

    // ---- S^T = K Q^T: two 32-key blocks
    f32x16_t s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[qb][kb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf = lds_read16(ks + k_off(32 * kb + l32, 2 * kk + hi));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][kk], s[qb][kb], 0, 0, 0);
      }
    }

    // ---- online softmax; lane owns query l32 and keys 8(r/4) + 4hi + r%4
    const bool tail = kv0 + kBC > N;
    bf16x8_t pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (tail) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= N) s[qb][kb][r] = -INFINITY;
          }
      }
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qb], mx);
      const bool grow = (m_new - m_run[qb]) * c > 8.0f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = exp2f((m_run[qb] - m_new) * c);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
      }
      const float mc = m_run[qb] * c;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, r0 = 8 * (st & 1);
        bf16x8_t p;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r0 + i], c, -mc));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r0 + i + 1], c, -mc));
          bf16x2_t pr;
          pr[0] = (__bf16)e0;
          pr[1] = (__bf16)e1;
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run[qb], false);
          p[i] = pr[0];
          p[i + 1] = pr[1];
        }
        pf[qb][st] = p;
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t vf = lds_read16(vs + v_off(32 * db + l32, 2 * st + hi));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][st], o[qb][db], 0, 0, 0);
      }
    }

    if (t + 1 < T) store_tile(regs, lds + ((t + 1) & 1) * kStageBytes, tid);
    __syncthreads();
  }

  // ---- epilogue: O / l, round once to bf16; lane holds query l32,
  // head dims 32db + 8g + 4hi + (0..3)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qt * BR + (wave * QB + qb) * 32 + l32;
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const float inv = o_scale / l_tot;
    if (q < N) {
      uint16_t *dst = static_cast<uint16_t *>(a.o) + head_off + (int64_t)q * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 w;
          w.x = pack_bf16(o[qb][db][4 * g + 0] * inv, o[qb][db][4 * g + 1] * inv);
          w.y = pack_bf16(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv);
          *reinterpret_cast<uint2 *>(dst + 32 * db + 8 * g + 4 * hi) = w;
        }
    }
  }
}

template <int QB, bool FP8>
hipError_t launch(const ForwardArgs &a, hipStream_t s) {
  constexpr int BR = kWaves * 32 * QB;
  const int64_t ntiles = (a.N + BR - 1) / BR;
  const int64_t grid = ntiles * a.BH;
  // Raise the dynamic-LDS limit once per device (idempotent, so a race
  // between threads only repeats the call).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_kernel<QB, FP8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<QB, FP8>), dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const ForwardArgs &a, hipStream_t s) { return launch<1, false>(a, s); }
hipError_t launch_forward_fp8(const ForwardArgs &a, hipStream_t s) { return launch<1, true>(a, s); }

int64_t forward_grid_blocks(int64_t BH, int64_t N) {
  const int64_t BR = kWaves * 32;
  return BH * ((N + BR - 1) / BR);
}

}  // namespace fluxattn

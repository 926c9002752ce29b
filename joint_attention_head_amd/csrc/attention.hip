// Non-causal joint attention O = softmax(Q K^T * scale) V on gfx950 MFMA.
//
// Dense attention over the merged text + image (+ reference) tokens is the
// dominant kernel of a FLUX-style DiT step (NVIDIA blog post "Speed up image
// generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
// "Quantized and sparse attention"); queries and keys arrive normalised and
// rotated (section "GEMM kernel optimization").
//
// Design (flash-style single pass over K/V; scores never leave registers):
//
//  * Workgroup = 8 waves = 256 query rows of one (b,h); wave w owns 32 rows.
//    Queries stay in VGPRs as the B operand of v_mfma_f32_32x32x16_bf16 and
//    each wave computes the transposed score tile S^T = K Q^T, so a lane owns
//    one query (lane % 32) and 16 of every 32 keys: the softmax row state is
//    lane-local up to one exchange with lane ^ 32.
//  * O^T = V^T P^T takes the probabilities straight from registers as the B
//    operand.  The keys a lane holds for one MFMA step are
//    {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); since keys are summed over,
//    the V^T operand only has to list the same keys in the same order, which
//    two ds_read_b64_tr_b16 transposing reads of the row-major V tile do.
//  * Ping-pong: the waves form two groups of four, one wave of each group per
//    SIMD.  Every phase ends with a workgroup barrier; in each phase one
//    group runs its matrix half-step (QK^T of the next tile, PV of the
//    current one: 32 MFMAs) while the other runs its vector half-step (online
//    softmax of the next tile, plus its share of the K/V tile loads), so the
//    matrix cores and the VALU of every SIMD are busy at the same time.
//  * K/V tiles of 64 keys go through a 4-stage LDS ring (128 KiB).  Group 0
//    loads K tiles and group 1 V tiles, global -> VGPR in one vector
//    half-step and VGPR -> LDS two phases later.  Buffer-resource loads
//    return 0 past the end of a head, so ragged tails need no branches.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA).  The
//    running max only moves, and O and l are rescaled, when a row's max grows
//    by more than 8 (log2 units); probabilities stay <= 2^8 and O / l is
//    unchanged.  l sums the bf16-rounded probabilities the MFMA consumes.
//  * blockIdx is remapped so that the workgroups the dispatcher sends to one
//    XCD (blockIdx % 8) take consecutive query tiles of the same (b,h) and
//    share its K/V stream through that XCD's L2.
//  * fp8 (OCP E4M3) inputs are widened to bf16 on load, which is exact; the
//    per-(b,h) scales are folded into the softmax scale (q, k) and into the
//    final normalisation (v).
#include "fluxattn_internal.h"

#include <atomic>

namespace fluxattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * 32;                  // query rows per workgroup
constexpr int kBC = 64;                           // keys per tile
constexpr int kStages = 4;
constexpr int kKTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = key
constexpr int kVTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = key
constexpr int kStageBytes = kKTileBytes + kVTileBytes;
constexpr int kLdsBytes = kStages * kStageBytes;  // 128 KiB
constexpr uint32_t kRsrcWord3 = 0x00020000u;      // raw buffer, 32-bit data format

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Four E4M3 codes -> four bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(uint32_t w) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  u32x2_t r;
  r[0] = pack_bf16(lo[0], lo[1]);
  r[1] = pack_bf16(hi[0], hi[1]);
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 8 consecutive head-dim elements (element offset `elem` inside one head),
// widened to bf16; reads past the head's end return zeros.
template <bool FP8>
__device__ __forceinline__ u32x4_t load8(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  if constexpr (FP8) {
    const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(r, elem, 0, 0);
    const u32x2_t a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
    u32x4_t v;
    v[0] = a[0];
    v[1] = a[1];
    v[2] = b[0];
    v[3] = b[1];
    return v;
  } else {
    return __builtin_amdgcn_raw_buffer_load_b128(r, elem * 2, 0, 0);
  }
}

// LDS layouts.  K tile: row = key, 16 chunks of 16 bytes, chunk XOR (key & 15)
// (ds_read_b128 of 16 consecutive keys hits 16 distinct bank groups).
// V tile: row = key, chunk XOR 4*(key & 3) (the transposing reads touch 4
// rows x 4 chunks per 32 lanes).
__device__ __forceinline__ int k_off(int key, int ch) { return key * 256 + ((ch ^ (key & 15)) << 4); }
__device__ __forceinline__ int v_off(int key, int ch) { return key * 256 + ((ch ^ ((key & 3) << 2)) << 4); }

__device__ __forceinline__ bf16x8_t lds_read_b128(const char *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}

// Transposing LDS read: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte loads of lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ i16x4_t lds_read_tr(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(__attribute__((address_space(3))) const char *)p);
}

template <bool FP8>
struct Loader {
  // This thread's 4 chunks of one tile (group 0: K tile, group 1: V tile).
  u32x4_t r[4];

  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t src, int tile, int rank) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = rank + 256 * i;            // 0..1023 chunk of the tile
      const int key = tile * kBC + (idx >> 4);
      r[i] = load8<FP8>(src, (uint32_t)key * kHeadDim + 8 * (idx & 15));
    }
  }
  __device__ __forceinline__ void store(char *tile_base, bool is_v, int rank) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = rank + 256 * i;
      const int key = idx >> 4, ch = idx & 15;
      const int off = is_v ? v_off(key, ch) : k_off(key, ch);
      *reinterpret_cast<u32x4_t *>(tile_base + off) = r[i];
    }
  }
};

template <bool FP8>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(ForwardArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int simd_of_wave[kWaves];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;

  // ---- ping-pong groups: sort waves by (SIMD, wave id); alternate groups
  // along that order, so the two waves of a SIMD land in different groups.
  if (lane == 0) simd_of_wave[wave] = (int)__builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));
  __syncthreads();
  int order = 0;
  {
    const int mine = simd_of_wave[wave] * kWaves + wave;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) order += (simd_of_wave[w] * kWaves + w) < mine;
  }
  const int group = order & 1;
  const int rank = (order >> 1) * 64 + lane;   // 0..255 inside the group

  // ---- blockIdx -> (b*h, query tile), consecutive tiles per XCD
  const int ntiles = (N + kBR - 1) / kBR;
  const int total = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, q8 = total >> 3, r8 = total & 7;
  const int logical = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const int bh = logical / ntiles;
  const int qt = logical - bh * ntiles;

  constexpr int kElem = FP8 ? 1 : 2;
  const size_t head_elems = (size_t)N * kHeadDim;
  const uint32_t head_bytes = (uint32_t)(head_elems * kElem);
  const char *qbase = static_cast<const char *>(a.q) + (size_t)bh * head_elems * kElem;
  const char *kbase = static_cast<const char *>(a.k) + (size_t)bh * head_elems * kElem;
  const char *vbase = static_cast<const char *>(a.v) + (size_t)bh * head_elems * kElem;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, head_bytes);

  float c = a.scale_log2;
  float o_scale = 1.f;
  if constexpr (FP8) {
    c *= a.q_scale[bh] * a.k_scale[bh];
    o_scale = a.v_scale[bh];
  }

  const int T = (N + kBC - 1) / kBC;

  // ---- fill the first stages (all threads: group 0 K, group 1 V); all the
  // fetches are in flight before the first store waits for its data
  Loader<FP8> ld;
  const __amdgpu_buffer_rsrc_t my_src = group ? rv : rk;
  {
    Loader<FP8> pre[kStages];
#pragma unroll
    for (int j = 0; j < kStages; ++j)
      if (j < T) pre[j].fetch(my_src, j, rank);
#pragma unroll
    for (int j = 0; j < kStages; ++j)
      if (j < T) pre[j].store(lds + j * kStageBytes + group * kKTileBytes, group == 1, rank);
  }

  // ---- queries: qf[kk] = Q[q][16kk + 8hi .. +8), q = this lane's row
  const int q_row = qt * kBR + wave * 32 + l32;
  bf16x8_t qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8_t, load8<FP8>(rq, (uint32_t)q_row * kHeadDim + 16 * kk + 8 * hi));

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  f32x16_t s[2];
  bf16x8_t pf[4];
  float m_run = -INFINITY, l_run = 0.f;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // V^T operand addressing (transposing reads): lane = 16 G + j
  const int G = lane >> 4, j16 = lane & 15;
  const int v_key_lane = 4 * (G >> 1) + (j16 >> 2);           // + 16 st (+ 8)
  const int v_byte_lane = 32 * (G & 1) + 8 * (j16 & 3);         // + 64 db

  __syncthreads();

  // Phase p: group 0 runs half-step h = p, group 1 runs h = p - 1.
  //   h even: QK^T of tile h/2 (if any) and PV of tile h/2 - 1 (if any)
  //   h odd : softmax of tile (h-1)/2; store K/V tile (h+3)/2 and fetch the next
  const int n_phases = 2 * T + 2;
  for (int p = 0; p < n_phases; ++p) {
    const int h = p - group;
    if (h >= 0 && (h & 1) == 0) {
      const int jq = h >> 1, jv = jq - 1;
      if (jq < T) {
        const char *ks = lds + (jq % kStages) * kStageBytes;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const bf16x8_t kf = lds_read_b128(ks + k_off(32 * kb + l32, 2 * kk + hi));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
          }
        }
      }
      if (jv >= 0 && jv < T) {
        const char *vs = lds + (jv % kStages) * kStageBytes + kKTileBytes;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int key = 16 * st + v_key_lane;
            const int byte = 64 * db + v_byte_lane;
            const int ch = byte >> 4, within = byte & 15;
            const i16x4_t lo = lds_read_tr(vs + v_off(key, ch) + within);
            const i16x4_t hi4 = lds_read_tr(vs + v_off(key + 8, ch) + within);
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], o[db], 0, 0, 0);
          }
        }
      }
    } else if (h >= 0) {
      const int js = (h - 1) >> 1;
      if (js < T) {
        // ---- online softmax of tile js; lane owns query l32 and keys
        // 32 kb + 8 (r / 4) + 4 hi + r % 4
        if (js * kBC + kBC > N) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = js * kBC + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key >= N) s[kb][r] = -INFINITY;
            }
        }
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > 8.0f) != 0) {
          const float alpha = exp2f((m_run - m_new) * c);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        const float mc = m_run * c;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int kb = st >> 1, r0 = 8 * (st & 1);
          bf16x8_t pv;
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + i], c, -mc));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + i + 1], c, -mc));
            bf16x2_t pr;
            pr[0] = (__bf16)e0;
            pr[1] = (__bf16)e1;
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
            pv[i] = pr[0];
            pv[i + 1] = pr[1];
          }
          pf[st] = pv;
        }
      }
      // ---- K/V ring: store tile (h+3)/2 fetched two phases ago, fetch the next
      const int jw = (h + 3) >> 1;
      if (jw >= kStages && jw < T) ld.store(lds + (jw % kStages) * kStageBytes + group * kKTileBytes, group == 1, rank);
      if (jw + 1 >= kStages && jw + 1 < T) ld.fetch(my_src, jw + 1, rank);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l, one bf16 rounding; lane holds query l32 and head
  // dims 32 db + 8 g + 4 hi + (0..3); stores past the head's end are dropped
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = o_scale / l_tot;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<char *>(a.o) + (size_t)bh * head_elems * 2,
                                              (uint32_t)(head_elems * 2));
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = pack_bf16(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      w[1] = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      const uint32_t elem = (uint32_t)q_row * kHeadDim + 32 * db + 8 * g + 4 * hi;
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, elem * 2, 0, 0);
    }
}

template <bool FP8>
hipError_t launch(const ForwardArgs &a, hipStream_t s) {
  const int64_t ntiles = (a.N + kBR - 1) / kBR;
  const int64_t grid = ntiles * a.BH;
  // Raise the dynamic-LDS limit once per device (idempotent, so a race
  // between threads only repeats the call).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_kernel<FP8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<FP8>), dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const ForwardArgs &a, hipStream_t s) { return launch<false>(a, s); }
hipError_t launch_forward_fp8(const ForwardArgs &a, hipStream_t s) { return launch<true>(a, s); }

int64_t forward_grid_blocks(int64_t BH, int64_t N) { return BH * ((N + kBR - 1) / kBR); }

}  // namespace fluxattn

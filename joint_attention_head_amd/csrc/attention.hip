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
//    the V^T operand only has to list the same keys in the same order.  V
//    tiles are stored transposed in LDS (row = head dim) with bits 2 and 3
//    of the key swapped inside every group of 16, so that list is one
//    ds_read_b128 per lane.
//  * Ping-pong: the waves form two groups of four, one wave of each group per
//    SIMD.  Every phase ends with a workgroup barrier; in each phase one
//    group runs its matrix half-step (QK^T of the next tile, PV of the
//    current one: 32 MFMAs, at raised wave priority) while the other runs
//    its vector half-step (online softmax of the next tile), so the matrix
//    cores and the VALU of every SIMD are busy at the same time.
//  * K tiles and V^T tiles of 64 keys go through two 4-slot LDS rings
//    (64 KiB each).  Both groups load half of every tile at the start of
//    their matrix half-steps: bf16 K by direct global -> LDS buffer loads,
//    three tiles ahead; V (and fp8 K) global -> VGPR one iteration before
//    the transposing VGPR -> LDS store, two tiles ahead.  Buffer-resource
//    loads return 0 past the end of a head, so ragged tails need no
//    branches; the softmax masks keys >= N.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA).  The
//    running max only moves, and O and l are rescaled, when a row's max grows
//    by more than 8 (log2 units); probabilities stay <= 2^8 and O / l is
//    unchanged.  l sums the fp32 probabilities; P is rounded to bf16 for
//    the MFMA.
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
constexpr int kSlots = 4;                         // per ring (K and V^T)
constexpr int kKTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = key
constexpr int kVTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = head dim
constexpr int kVRingOffset = kSlots * kKTileBytes;
constexpr int kLdsBytes = kSlots * (kKTileBytes + kVTileBytes);  // 128 KiB
constexpr uint32_t kRsrcWord3 = 0x00020000u;      // raw buffer, 32-bit data format

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char_t;
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

// LDS layouts (per stage: K tile then V^T tile, 16 KiB each).
//  K tile : row = key (256 B), 16-byte chunk c of the head dim stored at
//           c ^ (key & 15): the 16 keys one ds_read_b128 phase touches hit 16
//           distinct bank groups.
//  V^T tile: row = head dim d (128 B = 64 keys), keys permuted inside every
//           group of 16 (bits 2 and 3 swapped) so that the 8 keys a lane
//           feeds one PV MFMA are consecutive; chunk c stored at
//           c ^ ((d >> 1) & 7).
__device__ __forceinline__ int k_off(int key, int ch) { return key * 256 + ((ch ^ (key & 15)) << 4); }
__device__ __forceinline__ int vt_off(int d, int ch) { return d * 128 + ((ch ^ ((d >> 1) & 7)) << 4); }
__device__ __forceinline__ int vperm(int key) { return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1); }

__device__ __forceinline__ bf16x8_t lds_read_b128(const char *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}

// Tile loader.  Each of the two wave groups loads half of every tile:
// keys [32 g, 32 g + 32) of its K and V^T tiles.
//  V: thread `rank` of group g owns keys 32 g + 4 kg .. +3 (kg = rank % 8)
//     at head dims 4 dq .. 4 dq + 3 (dq = rank / 8) and stores them
//     transposed into 4 V^T rows.
//  K (fp8 only, bf16 K goes straight to LDS): chunks rank and rank + 256
//     of the group's 512 16-byte K chunks, widened to bf16.
template <bool FP8>
struct Loader {
  u32x2_t v[4];
  u32x4_t k[2];

  __device__ __forceinline__ void fetch_v(__amdgpu_buffer_rsrc_t src, int tile, int g, int rank) {
    const int kg = rank & 7, dq = rank >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t elem = (uint32_t)(tile * kBC + 32 * g + 4 * kg + i) * kHeadDim + 4 * dq;
      if constexpr (FP8) {
        v[i] = e4m3x4_to_bf16x4(__builtin_amdgcn_raw_buffer_load_b32(src, elem, 0, 0));
      } else {
        v[i] = __builtin_amdgcn_raw_buffer_load_b64(src, elem * 2, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store_v(char *vt, int g, int rank) const {
    const int kg = rank & 7, dq = rank >> 3;
    const int kp = vperm(32 * g + 4 * kg);   // multiple of 4: the 4 keys stay adjacent
    const int ch = kp >> 3, within = (kp & 7) * 2;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
      const int w = jj >> 1;
      u32x2_t out;
      out[0] = __builtin_amdgcn_perm(v[1][w], v[0][w], sel);
      out[1] = __builtin_amdgcn_perm(v[3][w], v[2][w], sel);
      const int d = 4 * dq + jj;
      *reinterpret_cast<u32x2_t *>(vt + vt_off(d, ch) + within) = out;
    }
  }
  __device__ __forceinline__ void fetch_k(__amdgpu_buffer_rsrc_t src, int tile, int g, int rank) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = rank + 256 * i;
      const int row = 32 * g + (idx >> 4);
      k[i] = load8<FP8>(src, (uint32_t)(tile * kBC + row) * kHeadDim + 8 * (idx & 15));
    }
  }
  __device__ __forceinline__ void store_k(char *kt, int g, int rank) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = rank + 256 * i;
      *reinterpret_cast<u32x4_t *>(kt + k_off(32 * g + (idx >> 4), idx & 15)) = k[i];
    }
  }
};

// Raw buffer descriptor words of one head (base, no stride, `bytes`
// records, 32-bit data format); out-of-range offsets read as zero.
__device__ __forceinline__ i32x4_t rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = (int)(uint32_t)p;
  r[1] = (int)((uint32_t)(p >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = (int)kRsrcWord3;
  return r;
}

// Half a K tile straight from global memory into LDS (bf16 only): wave gw
// (0..3) of group g copies the 2 KiB of rows 32 g + 8 gw .. +8 with two
// buffer_load_dwordx4 ... lds.  Such a copy writes 16 bytes per lane to
// LDS [M0 + imm + 16 lane] from global [rsrc + voffset + imm]; both use one
// M0 and the immediates 0 and 1024.  Lane l of copy i fetches the chunk the
// K swizzle puts at its LDS slot.  Issued from inline asm so that the
// compiler does not make every later LDS read wait for it; the kernel orders
// the copies itself with vmcnt waits before its barriers.
__device__ __forceinline__ void k_half_direct(i32x4_t rk, uint32_t kt_addr, int tile, int g, int gw, int lane) {
  const int row0 = 32 * g + 8 * gw;
  uint32_t vo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = row0 + 4 * i + (lane >> 4);
    const int ch = (lane & 15) ^ (row & 15);
    const uint32_t byte = ((uint32_t)(tile * kBC + row) * kHeadDim + 8 * ch) * 2;
    vo[i] = byte - 1024u * i;   // row >= 4 i, so byte >= 1024 i
  }
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(kt_addr + 256u * row0);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
      :
      : "s"(m0), "v"(vo[0]), "v"(vo[1]), "s"(rk)
      : "memory");
}

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
  // the sort key is the same in every lane of a wave: keep it scalar
  order = __builtin_amdgcn_readfirstlane(order);
  const int group = order & 1;
  const int gw = order >> 1;                   // wave index inside the group
  const int rank = gw * 64 + lane;             // 0..255 inside the group

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
  auto k_tile = [&](int j) { return lds + (j % kSlots) * kKTileBytes; };
  auto v_tile = [&](int j) { return lds + kVRingOffset + (j % kSlots) * kVTileBytes; };
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((lds_char_t *)lds);
  const i32x4_t wk = rsrc_words(kbase, head_bytes);

  // ---- rings.  Both groups load half of every tile.  K runs kKAhead tiles
  // ahead of its first use (fp8: one tile less, through registers), V^T
  // two: K tiles 0 .. kKAhead-1 and V^T tiles 0, 1 go in first, V tile 2
  // (fp8: and K tile 2) is left in flight in the loader registers.
  constexpr int kKAhead = 3;
  Loader<FP8> ld;
  for (int j = 0; j < 2 && j < T; ++j) {
    ld.fetch_v(rv, j, group, rank);
    ld.store_v(v_tile(j), group, rank);
    if constexpr (FP8) {
      ld.fetch_k(rk, j, group, rank);
      ld.store_k(k_tile(j), group, rank);
    }
  }
  if constexpr (!FP8) {
    for (int j = 0; j < kKAhead && j < T; ++j)
      k_half_direct(wk, lds_base + (j % kSlots) * kKTileBytes, j, group, gw, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if (2 < T) {
    ld.fetch_v(rv, 2, group, rank);
    if constexpr (FP8) ld.fetch_k(rk, 2, group, rank);
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
  float m_run = -INFINITY;
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};
  const f32x16_t zero = {};

  // Matrix half-step as a 32-step software pipeline over operand fragments:
  // steps 0..15 are QK^T of tile jq (kk = s/2, 32-key block kb = s%2), steps
  // 16..31 PV of tile jv (16-key step st = (s-16)/4, head-dim block
  // db = (s-16)%4).  Fragment s+kPre is requested from LDS before MFMA s is
  // issued, and scheduling fences keep that order.
#ifndef FLUXATTN_PREFETCH
#define FLUXATTN_PREFETCH 6
#endif
  constexpr int kPre = FLUXATTN_PREFETCH;
  auto frag = [&](int step, const char *ks, const char *vs) -> bf16x8_t {
    if (step < 16) {
      const int kk = step >> 1, kb = step & 1;
      return lds_read_b128(ks + k_off(32 * kb + l32, 2 * kk + hi));
    }
    const int st = (step - 16) >> 2, db = (step - 16) & 3;
    return lds_read_b128(vs + vt_off(32 * db + l32, 2 * st + hi));
  };
  auto matrix_step = [&](int step, bf16x8_t f) {
    if (step < 16) {
      const int kk = step >> 1, kb = step & 1;
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[kk], kk ? s[kb] : zero, 0, 0, 0);
    } else {
      const int st = (step - 16) >> 2, db = (step - 16) & 3;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[st], o[db], 0, 0, 0);
    }
  };
  auto matrix_half = [&](int jq, int jv) {
    const char *ks = k_tile(jq);
    const char *vs = v_tile(jv);
    bf16x8_t ring[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) ring[i] = frag(i, ks, vs);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 0; step < 32; ++step) {
      const bf16x8_t f = ring[step % kPre];
      if (step + kPre < 32) ring[step % kPre] = frag(step + kPre, ks, vs);
      matrix_step(step, f);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto qk_only = [&](int j) {
    const char *ks = k_tile(j);
#pragma unroll
    for (int step = 0; step < 16; ++step) matrix_step(step, frag(step, ks, ks));
  };

  // Online softmax of tile j.  Lane owns query l32 and keys
  // 32 kb + 8 (r / 4) + 4 hi + r % 4 of the tile (register r of s[kb]).
  // Short dependency chains: 4 independent max chains, 4 running sums.
  auto softmax = [&](int j) {
    if (j * kBC + kBC > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBC + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= N) s[kb][r] = -INFINITY;
        }
    }
    float mq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int kb = g >> 1, r0 = 8 * (g & 1);
      float m = fmaxf(s[kb][r0], s[kb][r0 + 1]);
#pragma unroll
      for (int r = 2; r < 8; ++r) m = fmaxf(m, s[kb][r0 + r]);
      mq[g] = m;
    }
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
      mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));   // max over both half-waves
    }
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64((m_new - m_run) * c > 8.0f) != 0) {
      const float alpha = exp2f((m_run - m_new) * c);
      m_run = m_new;
#pragma unroll
      for (int g = 0; g < 4; ++g) l_part[g] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    const float mc = m_run * c;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, r0 = 8 * (st & 1);
      bf16x8_t pv8;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + i], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + i + 1], c, -mc));
        l_part[st] += e0 + e1;
        pv8[i] = (__bf16)e0;
        pv8[i + 1] = (__bf16)e1;
      }
      pf[st] = pv8;
    }
    // keep the exponentials in this (vector) half-step: without these the
    // compiler sinks them next to their MFMA consumers in the matrix one
#pragma unroll
    for (int st = 0; st < 4; ++st) asm volatile("" : "+v"(pf[st]));
#pragma unroll
    for (int g = 0; g < 4; ++g) asm volatile("" : "+v"(l_part[g]));
  };

  __syncthreads();

  // Half-steps of every wave, each followed by a workgroup barrier:
  //   QK(0) | SM(0) | rings+QK(1)+PV(0) | SM(1) | ... | rings+QK+PV(T-1)
  // Group 1 runs one barrier behind group 0, so in every phase one group is
  // in a matrix half-step and the other in a vector half-step.  A wave
  // raises its priority for its matrix half-step, so the MFMA stream is
  // fed first and the softmax of the other wave fills the gaps.
  // At the start of its matrix half-step of iteration j each group stores
  // its half of V^T tile j+2 (fetched one iteration earlier) and fetches its
  // half of tile j+3; bf16: starts copying its half of K tile j+3 and waits
  // for its K tile j+2 copies (first read in iteration j+1); fp8: stores its
  // half of K tile j+2 and fetches tile j+3.  Slot reuse: the K slot of
  // tile j+3 (j+2 for fp8) last held tile j-1 (j-2), read by QK^T in
  // iteration j-2 (j-3); the V^T slot of tile j+2 last held tile j-2, read
  // by PV in iteration j-2; the barriers between put those reads before
  // either group's matrix half-step of iteration j.
  if (group == 1) __syncthreads();
  qk_only(0);
  __syncthreads();
  for (int j = 0; j < T; ++j) {
    softmax(j);
    __syncthreads();
    __builtin_amdgcn_s_setprio(3);
    if (j + 2 < T) {
      ld.store_v(v_tile(j + 2), group, rank);
      if constexpr (FP8) ld.store_k(k_tile(j + 2), group, rank);
    }
    if (j + 3 < T) {
      ld.fetch_v(rv, j + 3, group, rank);
      if constexpr (FP8) {
        ld.fetch_k(rk, j + 3, group, rank);
      } else {
        k_half_direct(wk, lds_base + ((j + 3) % kSlots) * kKTileBytes, j + 3, group, gw, lane);
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      }
    } else if constexpr (!FP8) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    matrix_half(min(j + 1, T - 1), j);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }
  if (group == 0) __syncthreads();

  // ---- epilogue: O / l, one bf16 rounding; lane holds query l32 and head
  // dims 32 db + 8 g + 4 hi + (0..3); stores past the head's end are dropped
  float l_run = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l_run), __float_as_int(l_run), false, false);
    l_run = __int_as_float(sw[0]) + __int_as_float(sw[1]);   // both half-waves' keys
  }
  const float inv = o_scale / l_run;
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

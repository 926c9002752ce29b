// Non-causal joint attention O = softmax(Q K^T * scale) V on the gfx950
// fp8 matrix cores: OCP E4M3 queries, keys, values and probabilities,
// v_mfma_f32_32x32x64_f8f6f4 with fp32 accumulation, bf16 output.
//
// FP8 for both the QK^T and the P.V operands is the attention precision the
// NVIDIA blog post "Speed up image generation with FLUX 3 Image Klein on
// NVIDIA Blackwell GPUs" selects in section "Quantized and sparse
// attention".  The structure follows the bf16 kernel (attention.hip):
//
//  * Workgroup = 8 waves = 256 query rows of one (b,h); wave w owns 32 rows
//    and computes S^T = K Q^T (a lane owns query lane % 32 and 16 of every
//    32 keys), so the softmax row state is lane-local up to one exchange
//    with lane ^ 32.  Queries stay in VGPRs as E4M3 codes: 64 bytes a lane,
//    the B operand of two MFMAs (64 head dims each) per 32 keys.
//  * O^T = V^T P^T takes P straight from registers as the B operand: the
//    32 keys a lane holds for a 64-key tile ({32 kb + 8 m + 4 h + r},
//    h = lane / 32) become k-slots 32 h + 16 kb + 4 m + r.  V tiles sit in
//    LDS as they are in memory (row = key); four transposing byte reads
//    (ds_read_b64_tr_b8) give a lane its head dim of those keys in that
//    slot order.
//  * P is stored as e4m3(p'), p' = 2^6 p relative to the row's running
//    shift (a shift puts the row maximum at 2^6): every p' stays <= 448,
//    the largest finite E4M3 value, and values down to p = 2^-12 keep the
//    full 3-bit mantissa.  O / l is unchanged by the factor.
//  * l sums the rounded P, the values PV multiplies, on the matrix cores:
//    one 16 x 16 x 128 MFMA per tile against a constant ones operand (see
//    `lsum`), so the softmax VALU does no additions.
//  * Ping-pong: two groups of four waves, one wave of each group per SIMD;
//    in every phase one group runs its matrix half-step (PV of the current
//    tile, QK^T of the next: 8 MFMAs of 64 cycles, raised wave priority)
//    while the other runs the online softmax.
//  * K and V tiles (row = key, 128 B) arrive by direct global -> LDS copies
//    three tiles ahead; nothing passes through VGPRs.  Both rings have 4
//    slots of 8 KiB.
//  * Scales: per-(b,h) scales of q, k fold into the softmax scale and the
//    scale of v into the final normalisation.  The fused form (FUSEQ) reads
//    raw E4M3 queries, applies RMSNorm + RoPE in fp32 and re-encodes each
//    query with its own power-of-two scale, which the QK^T MFMA applies as
//    its B block scale together with the softmax scale.
//  * Work per workgroup: a list of jobs, one whole query block or, when
//    the host balances the last round, pieces of blocks split by key
//    range, as in the bf16 kernel (attn_common.h).
#include "attn_common.h"

#include <atomic>

namespace fluxattn {
namespace {

using namespace attn;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
static_assert(kThreads == kSplitThreads, "split partials are laid out per thread of a 512-thread workgroup");
constexpr int kBR = kWaves * 32;                  // query rows per workgroup
constexpr int kBC = 64;                           // keys per tile
constexpr int kSlots = 4;                         // per ring (K and V)
constexpr int kKTileBytes = kBC * kHeadDim;       // 8 KiB, row = key (128 codes)
constexpr int kVTileBytes = kBC * kHeadDim;       // 8 KiB, row = key (128 codes)
constexpr int kVRingOffset = kSlots * kKTileBytes;
constexpr int kLdsBytes = kSlots * (kKTileBytes + kVTileBytes);  // 64 KiB
// After a shift the row maximum is p' = 2^kPExp; the shift moves when some
// p' of a tile would exceed 2^kShiftAt, so every p' stays <= 2^8 < 448.
// (A lower kPExp would make shifts rarer, but sends two more binades of
// small p' to E4M3 subnormals.)
constexpr float kPExp = 6.f;
constexpr float kShiftAt = 8.f;

// LDS layouts.
//  K tile : row = key (128 B = 8 chunks of 16 B); chunk c of key r sits at
//           c ^ ((r >> 1) & 7), so the 16 keys one ds_read_b128 phase reads
//           hit 16 distinct 16-byte bank groups.
//  V tile : row = key (128 B = 8 chunks of 16 B); chunk c of key r sits at
//           c ^ vsw(r), vsw(r) made of bits 0, 1 and 3 of r.  A transposing
//           read touches 8 keys (r % 4 = 0..3 at two r / 8) x 16 bytes per
//           16 lanes and 16 keys x 32 bytes per wave; this puts every
//           16-byte piece of one pass in its own banks.  Key offsets that
//           are multiples of 16 stay immediates.
__device__ __forceinline__ int k_off(int key, int ch) { return key * 128 + ((ch ^ ((key >> 1) & 7)) << 4); }
__device__ __forceinline__ int vsw(int key) { return (key & 3) | ((key >> 1) & 4); }
__device__ __forceinline__ int v_off(int key, int ch) { return key * 128 + ((ch ^ vsw(key)) << 4); }

typedef int i32x2_t __attribute__((ext_vector_type(2)));
// PV operand: four transposing byte reads, 16 keys apart (2 KiB)
__device__ __forceinline__ i32x8_t lds_read_tr8x4(const char *p) {
  typedef __attribute__((address_space(3))) i32x2_t *lp;
  const i32x2_t a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lp)(p));
  const i32x2_t b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lp)(p + 2048));
  const i32x2_t c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lp)(p + 4096));
  const i32x2_t d = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lp)(p + 6144));
  const i32x4_t x = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const i32x4_t y = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ i32x8_t lds_frag(const char *p0, const char *p1) {
  const i32x4_t x = *reinterpret_cast<const i32x4_t *>(p0);
  const i32x4_t y = *reinterpret_cast<const i32x4_t *>(p1);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// D = C + A B on E4M3 operands.  Zero scale operands select the plain
// v_mfma_f32_32x32x64_f8f6f4 (unit scales).  The scaled encoding, even with
// unit scales, holds up the other wave's VALU while it runs: the softmax of
// the other ping-pong group then stretches by the length of this group's
// matrix half-step.
__device__ __forceinline__ f32x16_t mfma_f8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// D = C + A B, 16 x 16 x 128 on E4M3 operands (plain encoding, unit scales).
__device__ __forceinline__ f32x4_t mfma16_f8(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// D = C + 2^(sb - 127) A B: sb is this lane's E8M0 block scale of B, i.e.
// of the 32 B elements the lane holds (its column, one half of k).
__device__ __forceinline__ f32x16_t mfma_f8_bscaled(i32x8_t a, i32x8_t b, f32x16_t c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// Queries of the fused entry point: raw E4M3 Q times its scale -> RMSNorm
// over the 128 dims -> rotation of each adjacent pair -> E4M3 codes of
// Q' * g * 2^-e with g = softmax scale * log2 e * (k scale) and e the
// smallest integer that keeps every code within 448 (e = ceil(log2(amax g /
// 448))): the QK^T MFMA with B block scale 2^e then yields the base-2
// logits c*S directly, and the largest code of the query lies in (224, 448].
// Returns the E8M0 scale 127 + e in `sb`.  The lane holds dims
// 64 kk + 32 hi + (0..31); the other 64 are in lane ^ 32.
// In two parts, so that the job's first tile copies go out between them:
// load_q_issue requests the raw codes and the position ids (no wait) and
// reads the row's norm weights from the LDS table; q_transform does the
// arithmetic.
struct QueryIn {
  u32x4_t raw[4];   // raw[2 kk + t]: dims 64 kk + 32 hi + 16 t + (0..15)
  int pos[3];       // position ids of the lane's query
  float4 w[16];     // w[4 c + q]: norm weights of dims 64 (c / 2) + 32 hi + 16 (c % 2) + 4 q .. +4
};
__device__ __forceinline__ void load_q_issue(QueryIn &in, const ForwardArgs &a, const RopeLds *tab,
                                             const HeadView &vq, int q_row, int hi) {
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(vq.base, vq.bytes);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    in.raw[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rq, (uint32_t)q_row * vq.row + (uint32_t)(64 * (c >> 1) + 32 * hi + 16 * (c & 1)),
                                                0, 0));
  // rows past N belong to no token: any valid row serves, their outputs are
  // never stored
  const int tok = min(q_row, a.N - 1);
#pragma unroll
  for (int i = 0; i < 3; ++i) in.pos[i] = a.pos[3 * tok + i];
  const float *w_q = tab->wq[stream_of(a, tok)];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      in.w[4 * c + q4] = *reinterpret_cast<const float4 *>(w_q + 64 * (c >> 1) + 32 * hi + 16 * (c & 1) + 4 * q4);
}
__device__ __forceinline__ void q_transform(i32x8_t (&qf)[2], int &sb, const QueryIn &in, const ForwardArgs &a,
                                            const RopeLds *tab, int hi, float in_scale, float g) {
  const u32x4_t(&raw)[4] = in.raw;
  // E4M3 codes as float; the dequantisation scale s_q is folded into the
  // normalisation: x_deq w rstd = x w (s_q rstd), with rstd from s_q^2 sum x^2
  float x[64];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[c][w], false);
      const f32x2_t up = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[c][w], true);
      x[16 * c + 4 * w + 0] = lo[0];
      x[16 * c + 4 * w + 1] = lo[1];
      x[16 * c + 4 * w + 2] = up[0];
      x[16 * c + 4 * w + 3] = up[1];
    }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) ss = fmaf(x[i], x[i], ss);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(ss), __float_as_int(ss), false, false);
    ss = __int_as_float(sw[0]) + __int_as_float(sw[1]);   // all 128 dims of this query
  }
  const float rs = in_scale / sqrtf(ss * (in_scale * in_scale) * (1.0f / kHeadDim) + a.eps);
  const float pf[3] = {(float)in.pos[0], (float)in.pos[1], (float)in.pos[2]};
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // pairs d0 / 2 + 4 g + (0..3)
      float sn[4], cs[4];
      rotations4(tab, pf, 32 * (c >> 1) + 16 * hi + 8 * (c & 1) + 4 * g, sn, cs);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int q4 = 2 * g + qq;
        const float4 w = in.w[4 * c + q4];
        const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int i = 16 * c + 4 * q4 + 2 * m, r = 2 * qq + m;
          const float u = x[i] * (wv[2 * m] * rs);
          const float v = x[i + 1] * (wv[2 * m + 1] * rs);
          x[i] = u * cs[r] - v * sn[r];
          x[i + 1] = u * sn[r] + v * cs[r];
          amax = fmaxf(amax, fmaxf(fabsf(x[i]), fabsf(x[i + 1])));
        }
      }
    }
  }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(amax), __float_as_int(amax), false, false);
    amax = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
  }
  // e = ceil(log2 v) for v = amax g / 448 = m 2^E, m in [0.5, 1)
  const float v = amax * g * (1.0f / 448.f);
  int e = 0;
  if (v > 0.f) {
    e = __builtin_amdgcn_frexp_expf(v);
    if (__builtin_amdgcn_frexp_mantf(v) == 0.5f) e -= 1;
    e = min(max(e, -120), 120);
  }
  sb = 127 + e;
  const float inv = g * __builtin_ldexpf(1.0f, -e);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = 32 * kk + 4 * u;
      // |x * inv| <= amax g 2^-e <= 448 up to fp32 rounding, which rounds
      // back to 448
      qf[kk][u] = (int)f32x4_to_e4m3(x[i] * inv, x[i + 1] * inv, x[i + 2] * inv, x[i + 3] * inv);
    }
}

// Attention of one query block over key tiles [job.kt0, job.kt0 + job.T):
// the whole head (job.cut < 0: O is stored) or one piece of a split block.
template <bool FUSEQ, bool STRIDED>
__device__ __forceinline__ void attn_job(const ForwardArgs &a, char *lds, const RopeLds *rope, int *split_ticket,
                                         const SplitJob job, const int tid_in, const int group, const int gw) {
  // lane constants are computed per job (an opaque copy of the thread id
  // keeps them from being hoisted out of the job loop, where they would
  // overlap the fused query transform's temporaries)
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;
  // wave-uniform job fields (they address the scalar buffer descriptors)
  const int bh = __builtin_amdgcn_readfirstlane(job.bh), qt = __builtin_amdgcn_readfirstlane(job.qt);
  const int kt0 = __builtin_amdgcn_readfirstlane(job.kt0), T = __builtin_amdgcn_readfirstlane(job.T);

  const HeadView vq = head_view<STRIDED>(a.q, a.sq, 1, bh, a.H, N);
  const HeadView vk = head_view<STRIDED>(a.k, a.sk, 1, bh, a.H, N);
  const HeadView vv = head_view<STRIDED>(a.v, a.sv, 1, bh, a.H, N);
  const HeadView vo = head_view<STRIDED>(a.o, a.so, 2, bh, a.H, N);

  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((lds_char_t *)lds);

  // ---- lane constants (bytes).  Each group loads half of every tile:
  // keys [32 g, 32 g + 32).
  //  K by direct copies: wave gw of group g copies keys 32 g + 8 gw .. +8
  //     with one buffer_load_dwordx4 ... lds; lane l fetches the chunk the
  //     swizzle puts at LDS row 32 g + 8 gw + l / 8, chunk position l % 8.
  const int krow = 32 * group + 8 * gw + (lane >> 3);
  const uint32_t k_dgoff = (uint32_t)krow * vk.row + (uint32_t)(16 * ((lane & 7) ^ ((krow >> 1) & 7)));
  const uint32_t k_m0 = lds_base + 128u * (uint32_t)(32 * group + 8 * gw);
  //  V by direct copies of the same rows into the V ring, with its swizzle
  const uint32_t v_dgoff = (uint32_t)krow * vv.row + (uint32_t)(16 * ((lane & 7) ^ vsw(krow)));
  //  QK^T fragments (32 bytes = two chunks each): K (kk) row l32, chunks
  //     4 kk + 2 hi + t.  Slot and 32-key block (4 KiB) are immediates.
  uint32_t kf[2][2], vtr[4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int t = 0; t < 2; ++t) kf[kk][t] = (uint32_t)k_off(l32, 4 * kk + 2 * hi + t);
  //  PV operand by transposing byte reads.  Within 16 lanes, lane m of a
  //     ds_read_b64_tr_b8 receives byte m % 8 of the 8-byte pieces that
  //     lanes 2 j + m / 8 (j = 0..7) address.  Lane L addresses key
  //     4 (L / 32) + 8 ((L % 16) / 8) + (L % 16) / 2 % 4 (+ 16 t for read
  //     t), head dims 32 db + 16 ((L / 16) % 2) + 8 (L % 2) .. +8; so lane
  //     l receives head dim 32 db + l % 32 of the keys in the k-slot order
  //     of its P operand.
  {
    const int t16 = lane & 15;
    const int row0 = 4 * hi + 8 * (t16 >> 3) + ((t16 >> 1) & 3);
    const int dh = (lane >> 4) & 1, i2 = lane & 1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      vtr[db] = (uint32_t)(kVRingOffset + v_off(row0, 2 * db + dh) + 8 * i2);
  }

  // ---- ring traffic helpers
  auto k_dma = [&](const i32x4_t &words, uint32_t slot_bytes) __attribute__((always_inline)) {
    // the LDS address is added up here, not by the compiler: precomputed
    // sums for every slot would hold scalar registers through the loop
    asm volatile(
        "s_add_u32 m0, %0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(k_m0), "v"(k_dgoff), "s"(words), "s"(slot_bytes)
        : "memory", "scc");
  };
  auto v_dma = [&](const i32x4_t &words, uint32_t slot_bytes) __attribute__((always_inline)) {
    asm volatile(
        "s_add_u32 m0, %0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(k_m0), "v"(v_dgoff), "s"(words), "s"(kVRingOffset + slot_bytes)
        : "memory", "scc");
  };

  // ---- queries: qf[kk] = codes of dims 64 kk + 32 hi .. +32 of this
  // lane's query; c = softmax scale * log2 e * (q scale) * (k scale).
  // Requested first; the fused transform follows the first tile copies.
  const int q_row = qt * kBR + wave * 32 + l32;
  // the head's dequantisation scales, read before the tile copies go out
  // (a later read would wait for them)
  const float q_scale = a.q_scale[bh], k_scale = a.k_scale[bh], v_scale = a.v_scale[bh];
  i32x8_t qf[2];
  float qs = 1.f;
  int qsb = 127;   // fused: E8M0 B scale of the QK^T MFMAs, c folded in
  QueryIn qin;
  if constexpr (FUSEQ) {
    load_q_issue(qin, a, rope, vq, q_row, hi);
  } else {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(vq.base, vq.bytes);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t off = (uint32_t)q_row * vq.row + (uint32_t)(64 * kk + 32 * hi);
      const i32x4_t x = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      const i32x4_t y = __builtin_bit_cast(i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0));
      qf[kk] = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    qs = q_scale;
  }

  // ---- rings, before the loop: K and V tiles 0, 1, 2 in LDS, by the same
  // copies as in the loop but through the builtin, so that the compiler
  // counts them: the query transform then waits for the queries only and
  // runs while the tiles arrive.  Tile indices are clamped to T - 1 (a fixed
  // count of copies; extra ones land in slots no step reads).
  __builtin_amdgcn_sched_barrier(0);
  {
    typedef __attribute__((address_space(3))) void *lds_void_t;
    lds_char_t *dst = (lds_char_t *)lds + 128 * (32 * group + 8 * gw);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t tile = (uint32_t)(kt0 + min(j, T - 1)) * (uint32_t)kBC;   // first key
      const uint32_t skip_k = tile * vk.row, skip_v = tile * vv.row;   // the views' row pitches may differ
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(vk.base + skip_k, vk.bytes - skip_k),
                                               (lds_void_t)(dst + j * kKTileBytes), 16, k_dgoff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(vv.base + skip_v, vv.bytes - skip_v),
                                               (lds_void_t)(dst + kVRingOffset + j * kVTileBytes), 16, v_dgoff, 0,
                                               0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (FUSEQ) {
    // the transform's inputs and outputs pass through empty asm statements
    // after the copies and before their wait, which pins the transform
    // between the two
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(qin.raw[c]));
#pragma unroll
    for (int i = 0; i < 3; ++i) asm volatile("" : "+v"(qin.pos[i]));
    q_transform(qf, qsb, qin, a, rope, hi, q_scale, a.scale_log2 * k_scale);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) asm volatile("" : "+v"(qf[kk]));
    asm volatile("" : "+v"(qsb));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // unfused: x = c*S - b by one FMA per score; fused: the MFMA's B scale
  // applies c and its accumulator starts at -b (`bias`)
  const float c = a.scale_log2 * qs * k_scale;
  const float o_scale = v_scale;

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  f32x16_t s[2];
  i32x8_t pf = {};         // P^T operand: byte 16 kb + r = p' of s[kb][r]
  float b_run = 0.f;       // this row's running shift, base-2 units
  f32x16_t bias = {};      // fused: -b_run in every element
  // Row sums of the rounded P by the matrix cores: read as the B operand of
  // a 16 x 16 x 128 MFMA, the P^T operand gives column l % 16, k-block
  // l / 16 the bytes of query 16 ((l / 16) % 2) + l % 16 at k-slots
  // 32 (l / 32) ..; an A operand of ones in k-blocks of the same parity as
  // bit 2 of the row sums, in output row i, all 64 slots of query
  // 16 ((i / 4) % 2) + column, and lane l holds rows 4 (l / 16) .. +3 of
  // column l % 16: the sum of its own query, four times.
  f32x4_t lsum = {};
  i32x8_t lones;
  {
    const int v = (((lane >> 4) & 1) == ((lane >> 2) & 1)) ? 0x38383838 : 0;   // E4M3 1.0
#pragma unroll
    for (int i = 0; i < 8; ++i) lones[i] = v;
  }
  const f32x16_t zero = {};

  // Matrix half-step as an 8-step software pipeline: steps 0..3 are PV of
  // the current tile (head-dim block db = step), steps 4..7 QK^T of the
  // next tile (kk = (step-4)/2, 32-key block kb = (step-4)%2).  Operand
  // step+kPre is requested from LDS before MFMA step is issued.
  constexpr int kPre = 2;
  auto frag = [&](int step, int kslot_bytes, int vslot_bytes) __attribute__((always_inline)) -> i32x8_t {
    if (step >= 4) {
      const int kk = (step - 4) >> 1, kb = (step - 4) & 1;
      return lds_frag(lds + kf[kk][0] + (kslot_bytes + kb * 4096), lds + kf[kk][1] + (kslot_bytes + kb * 4096));
    }
    return lds_read_tr8x4(lds + vtr[step] + vslot_bytes);
  };
  auto matrix_step = [&](int step, i32x8_t f) __attribute__((always_inline)) {
    if (step >= 4) {
      const int kk = (step - 4) >> 1, kb = (step - 4) & 1;
      if constexpr (FUSEQ) {
        s[kb] = mfma_f8_bscaled(f, qf[kk], kk ? s[kb] : bias, qsb);
      } else {
        s[kb] = mfma_f8(f, qf[kk], kk ? s[kb] : zero);
      }
    } else {
      o[step] = mfma_f8(f, pf, o[step]);
    }
  };

  // Online softmax of tile j (see the header comment): x = c*S - b by one
  // FMA per score (fused: by the MFMA's scale and accumulator), p' = 2^x.
  // The lane maximum of x (16 max3) decides: when some lane's exceeds
  // kShiftAt, and on the first tile, b moves so that the row maximum lands
  // at 2^kPExp (first tile: always), with O and l rescaled.
  auto softmax = [&](int j, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value != 0;
    if constexpr (!FUSEQ) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], c, -b_run);
    }
    if ((kt0 + j) * kBC + kBC > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = (kt0 + j) * kBC + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= N) s[kb][r] = -INFINITY;
        }
    }
    auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float e0 = __builtin_amdgcn_exp2f(s[kb][4 * u + 0]);
          const float e1 = __builtin_amdgcn_exp2f(s[kb][4 * u + 1]);
          const float e2 = __builtin_amdgcn_exp2f(s[kb][4 * u + 2]);
          const float e3 = __builtin_amdgcn_exp2f(s[kb][4 * u + 3]);
          pf[4 * kb + u] = (int)f32x4_to_e4m3_over(e0, e1, e2, e3, pf[4 * kb + u]);
        }
    };
    // lane maximum of x - b (max3 chains)
    float m = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) m = fmaxf(m, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, s[1][r]);
    if (kFirst || __builtin_amdgcn_ballot_w64(m > kShiftAt) != 0) {
      float mx = m;
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
        mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));   // max over both half-waves
      }
      // first tile: any shift (mx is finite: key 0 is in the tile)
      const float d = kFirst ? mx - kPExp : fmaxf(mx - kPExp, 0.f);
      b_run += d;
      if constexpr (FUSEQ) {
#pragma unroll
        for (int i = 0; i < 16; ++i) bias[i] = -b_run;
      }
      if constexpr (!kFirst) {
        const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[i] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= d;
    }
    exps();
    // keep the exponentials in this (vector) half-step
    asm volatile("" : "+v"(pf));
  };

  // Schedule and ring reuse as in the bf16 kernel: QK^T(0), vector
  // half-step of tile 0, then per tile j a matrix half-step (PV(j),
  // QK^T(j+1)) and the vector half-step of tile j+1; group 1 runs one
  // barrier behind group 0.  Ring traffic of matrix half-step j: copy V and
  // K tile j+3 into LDS.  Both slots last held tile j-1 (read by PV(j-1) in
  // matrix half-step j-1 and by QK^T(j-1) in matrix half-step j-2): at
  // least one barrier separates those reads from either group's writes.
  // Tile indices are clamped to T-1; extra copies land in slots no later
  // step reads.  The vmcnt wait in each vector half-step retires the
  // previous matrix half-step's copies.
  constexpr int kVLoadStep = 1, kKLoadStep = 5;
  // First kPre fragments of the next matrix half-step (V slot of tile j+1,
  // K slot of tile j+2), requested at the start of the vector half-step so
  // the LDS reads overlap the softmax.  Both tiles are complete: they were
  // copied in matrix half-steps j-2 and j-1, and every wave has retired its
  // part and passed a barrier since.  The only slots written before the
  // next barrier are those of tile j+3.
  auto prefetch = [&](int kslot_bytes, int vslot_bytes, i32x8_t *ring) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) ring[i] = frag(i, kslot_bytes, vslot_bytes);
  };
  // end of the vector half-step: retire this wave's copies of the matrix
  // half-step just done, before the next barrier
  auto vector_tail = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  auto iteration = [&](int j, auto slot, i32x8_t *ring) __attribute__((always_inline)) {
    constexpr int R = decltype(slot)::value;
    constexpr int kCur = R * kKTileBytes;                       // V slot of tile j (same offset in both rings)
    constexpr int kNext = ((R + 1) % kSlots) * kKTileBytes;    // slots of tile j+1
    constexpr int kPlus3 = ((R + 3) % kSlots) * kKTileBytes;   // slots of tile j+3
    const int tn = min(j + 3, T - 1);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      const i32x8_t f = ring[step % kPre];
      if (step + kPre < 8) ring[step % kPre] = frag(step + kPre, kNext, kCur);
      matrix_step(step, f);
      if (step == 3) lsum = mfma16_f8(lones, pf, lsum);   // row sums of P(j)
      if (step == kVLoadStep) v_dma(tile_words(vv, kt0 + tn, kBC), kPlus3);
      if (step == kKLoadStep) k_dma(tile_words(vk, kt0 + tn, kBC), kPlus3);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // the QK^T MFMAs belong to this half-step: without this use the
    // compiler sinks them past the barrier into the softmax branch
    asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    __syncthreads();
    if (j + 1 < T) {
      prefetch(((R + 2) % kSlots) * kKTileBytes, kNext, ring);
      softmax(j + 1, Slot<0>{});
      vector_tail();
    }
  };

  __syncthreads();
  if (group == 1) __syncthreads();
  // QK^T(0): all four fragments requested before the first MFMA
  {
    i32x8_t r0[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r0[i] = frag(4 + i, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 4; step < 8; ++step) {
      matrix_step(step, r0[step - 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  i32x8_t ring[kPre];
  prefetch(1 * kKTileBytes, 0, ring);
  softmax(0, Slot<1>{});
  vector_tail();
  int j = 0;
  for (; j + kSlots <= T; j += kSlots) {
    iteration(j, Slot<0>{}, ring);
    iteration(j + 1, Slot<1>{}, ring);
    iteration(j + 2, Slot<2>{}, ring);
    iteration(j + 3, Slot<3>{}, ring);
  }
  if (j < T) iteration(j, Slot<0>{}, ring);
  if (j + 1 < T) iteration(j + 1, Slot<1>{}, ring);
  if (j + 2 < T) iteration(j + 2, Slot<2>{}, ring);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (group == 0) __syncthreads();

  // ---- epilogue: O * s_v / l, one bf16 rounding; lane holds query l32 and
  // head dims 32 db + 8 g + 4 hi + (0..3); stores past the head's end drop
  float l_run[1] = {lsum[0]};   // all 64 keys of every tile, rounded P
  float b_fin[1] = {b_run};
  // a piece of a split block: the piece that finishes second merges
  if (job.cut >= 0 && !split_merge<1>(a, job, o, b_fin, l_run, tid, split_ticket)) return;
  const float inv = o_scale / l_run[0];
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(vo.base, vo.bytes);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = pack_bf16(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      w[1] = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      const uint32_t off = (uint32_t)q_row * vo.row + (uint32_t)((32 * db + 8 * g + 4 * hi) * 2);
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
    }
}

template <bool FUSEQ, bool STRIDED>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_kernel(ForwardArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int simd_of_wave[kWaves];
  __shared__ int split_ticket;
  __shared__ RopeLds rope;

  const int tid = threadIdx.x;
  if constexpr (FUSEQ) rope_lds_fill(&rope, a, tid, kThreads);   // before the barrier in pingpong_order
  const int order = pingpong_order(simd_of_wave, tid >> 6, tid & 63);
  const int group = order & 1;
  const int gw = order >> 1;                   // wave index inside the group

  // ---- this workgroup's share of the (query block, key tile) pairs; the
  // range state waits in LDS (one copy per wave) while a job runs, so it
  // takes no scalar registers there
  __shared__ SplitRange range_lds[kWaves];
  SplitRange *rs = &range_lds[tid >> 6];
  {
    const SplitRange r = split_range(a, kBR, kBC, blockIdx.x, gridDim.x);
    if ((tid & 63) == 0) *rs = r;
  }
  for (;;) {
    SplitRange r = split_range_load(rs);
    SplitJob job;
    if (!split_next(r, job)) break;
    if ((tid & 63) == 0) *rs = r;
    attn_job<FUSEQ, STRIDED>(a, lds, &rope, &split_ticket, job, tid, group, gw);
  }
}

template <bool FUSEQ, bool STRIDED>
hipError_t launch(const ForwardArgs &a, hipStream_t s) {
  const int64_t grid =
      a.split_groups > 0 ? a.split_groups : std::min<int64_t>(a.whole_groups, (int64_t)((a.N + kBR - 1) / kBR) * a.BH);
  // Raise the dynamic-LDS limit once per device (idempotent, so a race
  // between threads only repeats the call).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_fp8_kernel<FUSEQ, STRIDED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<FUSEQ, STRIDED>), dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_fp8(const ForwardArgs &a, bool fused, bool strided, hipStream_t s) {
  const int v = (fused ? 2 : 0) | (strided ? 1 : 0);
  switch (v) {
    case 0: return launch<false, false>(a, s);
    case 1: return launch<false, true>(a, s);
    case 2: return launch<true, false>(a, s);
    default: return launch<true, true>(a, s);
  }
}

}  // namespace fluxattn

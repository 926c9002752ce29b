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
//  * Workgroup = 8 waves = 256 query rows of one (b,h); wave w owns 32 rows
//    as two halves of 16 (h = 0, 1).  Every product is a
//    v_mfma_f32_16x16x32_bf16: at the chip's power limit it sustains a
//    higher clock than the 32x32x16 shape, which moves more accumulator and
//    operand register bytes per flop.  Lane l works on query l % 16 of each
//    half, and on k-slots 8 g .. +8 and output rows 4 g .. +4 of every
//    MFMA, g = l / 16.
//  * S^T = K Q^T: K (16 keys x 32 dims) is the A operand, read from LDS
//    with one ds_read_b128 per lane, and the queries stay in VGPRs as the B
//    operand.  Lane l then holds, for each of its two queries, keys
//    16 kb + 4 g .. +4 of every 16-key block kb: the row state of a query
//    is spread over the four lanes l % 16 + 16 g.
//  * O^T = V^T P^T takes the probabilities straight from registers as the
//    B operand: of a 32-key block the lane's own keys {4 g .. +4} and
//    {16 + 4 g .. +4} fill its k-slots 8 g .. +8.  Since keys are summed
//    over, the V^T operand only has to list the same keys in the same
//    k-slots; two transposing reads (ds_read_b64_tr_b16) of the V tile, as
//    it is in memory (row = key), give a lane those 8 keys at its head dim.
//  * Ping-pong: the waves form two groups of four, one wave of each group per
//    SIMD.  Every phase ends with a workgroup barrier; in each phase one
//    group runs its matrix half-step (PV of the current tile, QK^T of the
//    next one: 64 MFMAs, at raised wave priority) while the other runs its
//    vector half-step (online softmax of the next tile), so the matrix cores
//    and the VALU of every SIMD are busy at the same time.
//  * The matrix half-step issues no VALU instruction: a VALU op of the MFMA
//    wave would queue behind the other wave's softmax and hold up the MFMA
//    stream.  LDS addresses are lane constants plus immediates (the loop is
//    unrolled over the four ring slots), and global loads take per-tile
//    buffer descriptors built with scalar ops.
//  * K and V tiles of 64 keys go through two 4-slot LDS rings (64 KiB
//    each).  Both groups copy half of every tile with direct global -> LDS
//    buffer loads, three tiles ahead, spread over their matrix half-steps;
//    no tile passes through VGPRs.  Buffer-resource loads return 0 past the
//    end of a head, so ragged tails need no branches; the softmax masks
//    keys >= N.
//  * Online softmax in base 2: x = c*S - b (c = scale * log2 e, b = the
//    row's running shift), then p = 2^x.  The plain form spends one FMA per
//    score on x; the fused form gets it from the MFMA, with c folded into
//    the queries and -b as the accumulator's initial value.  The row
//    maximum is only scanned when a lane's share of the tile's row sum (an
//    upper bound of every probability in it) exceeds 2^16; b then moves up
//    to the maximum if that exceeds it by more than 8, with O and l
//    rescaled.  O / l is unchanged by the shift.  l sums the fp32
//    probabilities; P is rounded to bf16 for the MFMA.
//  * blockIdx is remapped so that the workgroups the dispatcher sends to one
//    XCD (blockIdx % 8) take consecutive query tiles of the same (b,h) and
//    share its K/V stream through that XCD's L2.
//  * A workgroup runs a list of jobs (attn_common.h): the launch is a
//    persistent grid of at most one workgroup per compute unit.  Uncut,
//    each takes whole blocks of its XCD's range in turn; when the host
//    balances the last round, it takes whole blocks in launch order and then
//    an equal share of the tail's (query block, key tile) pairs, a cut
//    block's pieces being merged by whichever finishes last.
//  * A job requests its queries, then its first three tiles' copies, and
//    normalises and rotates the queries (fused form) while the tiles arrive.
// FP8 inputs run on the fp8 matrix cores instead (attention_fp8.hip).
#include "attn_common.h"

#include <atomic>

namespace fluxattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
static_assert(kThreads == kSplitThreads, "split partials are laid out per thread of a 512-thread workgroup");
constexpr int kBR = kWaves * 32;                  // query rows per workgroup
constexpr int kBC = 64;                           // keys per tile
constexpr int kSlots = 4;                         // per ring (K and V)
constexpr int kKTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = key
constexpr int kVTileBytes = kBC * kHeadDim * 2;   // 16 KiB, row = key
constexpr int kVRingOffset = kSlots * kKTileBytes;
constexpr int kLdsBytes = kSlots * (kKTileBytes + kVTileBytes);  // 128 KiB

using namespace attn;

// LDS layouts (K ring, then V ring; 16 KiB per slot).
//  K tile: row = key (256 B), 16-byte chunk c of the head dim stored at
//          c ^ (key & 15): the 16 keys one ds_read_b128 phase touches hit 16
//          distinct bank groups.
//  V tile: row = key (256 B), chunk c stored at c ^ vsw(key), vsw(key) =
//          2 (key % 8).  A transposing read touches 4 consecutive keys x 32
//          bytes (two chunks) per 16 lanes and 8 keys x 32 bytes per half
//          wave; the swizzle puts those eight 32-byte pieces in the eight
//          32-byte bank windows of a 256-byte bank row.  It depends on
//          key % 8 only, so key offsets that are multiples of 8 stay
//          immediates.
__device__ __forceinline__ int k_off(int key, int ch) { return key * 256 + ((ch ^ (key & 15)) << 4); }
__device__ __forceinline__ int vsw(int key) { return (key & 7) << 1; }
__device__ __forceinline__ int v_off(int key, int ch) { return key * 256 + ((ch ^ vsw(key)) << 4); }

__device__ __forceinline__ bf16x8_t lds_read_b128(const char *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}
typedef short i16x4_t __attribute__((ext_vector_type(4)));
// two transposing reads: elements 0..3 from p, 4..7 from p + 4096 (16 keys on)
__device__ __forceinline__ bf16x8_t lds_read_tr2(const char *p) {
  typedef __attribute__((address_space(3))) i16x4_t *lp;
  const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p));
  const i16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p + 4096));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// D = C + A B, 16 x 16 x 32, bf16 operands, fp32 accumulation.
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x combined over the four lanes l % 16 + 16 g that hold one query (max or
// sum; the same value, bit for bit, in all four: each step combines a
// pair of lanes commutatively)
__device__ __forceinline__ float quad_max(float x) {
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// Queries of the fused entry points: raw Q -> RMSNorm over the 128 dims ->
// rotation of each adjacent pair by its axis position times frequency
// (the prologue's operations) -> times c = softmax scale * log2 e -> bf16,
// so that the QK^T MFMA yields base-2 logits.  The lane holds two queries
// (q_row[h], h = 0, 1) and of each the dims 32 ks + 8 g .. +8 (ks = 0..3):
// the other 96 dims of a query are in lanes lane ^ 16, ^ 32, ^ 48.  The one
// bf16 rounding of Q' is the same as the prologue's, applied to c Q'.
// In two parts, so that the job's first tile copies go out between them:
// load_q_issue requests the raw queries and position ids (no wait) and
// reads the rows' norm weights from the LDS table; q_transform does the
// arithmetic.
struct QueryIn {
  int pos[2][3];        // position ids of the lane's two queries
  float4 w[2][4][2];    // their norm weights, dims 32 ks + 8 g .. +8
};
__device__ __forceinline__ void load_q_issue(bf16x8_t (&qf)[2][4], QueryIn &in, const ForwardArgs &a,
                                             const RopeLds *tab, const HeadView &vq, const int (&q_row)[2],
                                             int g) {
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(vq.base, vq.bytes);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t off = (uint32_t)q_row[h] * vq.row + (uint32_t)((32 * ks + 8 * g) * 2);
      qf[h][ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // rows past N belong to no token: any valid row serves, their outputs
    // are never stored
    const int tok = min(q_row[h], a.N - 1);
#pragma unroll
    for (int i = 0; i < 3; ++i) in.pos[h][i] = a.pos[3 * tok + i];
    const float *w_q = tab->wq[stream_of(a, tok)];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      in.w[h][ks][0] = *reinterpret_cast<const float4 *>(w_q + 32 * ks + 8 * g);
      in.w[h][ks][1] = *reinterpret_cast<const float4 *>(w_q + 32 * ks + 8 * g + 4);
    }
  }
}
__device__ __forceinline__ void q_transform(bf16x8_t (&qf)[2][4], const QueryIn &in, const ForwardArgs &a,
                                            const RopeLds *tab, int g) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (float)qf[h][ks][i];
        ss = fmaf(x, x, ss);
      }
    ss = quad_sum(ss);   // all 128 dims of this query
    // rstd and the logit scale c folded into the weights: Q' c = (x w rstd c)
    // rotated
    const float rs = a.scale_log2 / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
    const float pf[3] = {(float)in.pos[h][0], (float)in.pos[h][1], (float)in.pos[h][2]};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)qf[h][ks][i];
      const float4 w0 = in.w[h][ks][0], w1 = in.w[h][ks][1];
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float sn[4], cs[4];
      rotations4(tab, pf, 16 * ks + 4 * g, sn, cs);   // pairs 16 ks + 4 g + m
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float u = x[2 * m] * (w[2 * m] * rs);
        const float v = x[2 * m + 1] * (w[2 * m + 1] * rs);
        qf[h][ks][2 * m] = (__bf16)(u * cs[m] - v * sn[m]);
        qf[h][ks][2 * m + 1] = (__bf16)(u * sn[m] + v * cs[m]);
      }
    }
  }
}

template <bool FUSEQ, bool STRIDED>
__device__ __forceinline__ void attn_job(const ForwardArgs &a, char *lds, const RopeLds *rope, int *split_ticket,
                                         const SplitJob job, const int tid_in, const int group, const int gw) {
  // lane constants are computed per job (an opaque copy of the thread id
  // keeps them from being hoisted out of the job loop, where they would
  // overlap the fused query transform's temporaries)
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int N = a.N;
  // wave-uniform job fields (they address the scalar buffer descriptors)
  const int bh = __builtin_amdgcn_readfirstlane(job.bh), qt = __builtin_amdgcn_readfirstlane(job.qt);
  const int kt0 = __builtin_amdgcn_readfirstlane(job.kt0), T = __builtin_amdgcn_readfirstlane(job.T);

  // ---- per-head base pointers, token-row pitches and buffer extents
  const HeadView vq = head_view<STRIDED>(a.q, a.sq, 2, bh, a.H, N);
  // ---- queries: qf[h][ks] = Q[q_row[h]][32 ks + 8 g .. +8), the B
  // operands of QK^T, requested first (the fused transform follows the
  // first tile copies below)
  const int q_row[2] = {qt * kBR + wave * 32 + l16, qt * kBR + wave * 32 + 16 + l16};
  bf16x8_t qf[2][4];
  QueryIn qin;
  if constexpr (FUSEQ) {
    load_q_issue(qf, qin, a, rope, vq, q_row, g);
  } else {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(vq.base, vq.bytes);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t off = (uint32_t)q_row[h] * vq.row + (uint32_t)((32 * ks + 8 * g) * 2);
        qf[h][ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      }
  }

  const HeadView vk = head_view<STRIDED>(a.k, a.sk, 2, bh, a.H, N);
  const HeadView vv = head_view<STRIDED>(a.v, a.sv, 2, bh, a.H, N);
  const HeadView vo = head_view<STRIDED>(a.o, a.so, 2, bh, a.H, N);

  const float c = a.scale_log2;
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((lds_char_t *)lds);

  // ---- lane constants (bytes).  Each ping-pong group loads half of every
  // tile: keys [32 group, 32 group + 32).
  //  K by direct copies: wave gw of the group copies rows
  //     32 group + 8 gw .. +8 with two buffer_load_dwordx4 ... lds; lane l
  //     of copy i fetches the chunk the K swizzle puts at LDS slot row
  //     32 group + 8 gw + 4 i + l / 16, chunk position l % 16.
  uint32_t k_dgoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * group + 8 * gw + 4 * i + (lane >> 4);
    const int ch = (lane & 15) ^ (row & 15);
    k_dgoff[i] = (uint32_t)row * vk.row + (uint32_t)(8 * ch * 2);
  }
  const uint32_t k_m0 = lds_base + 256u * (uint32_t)(32 * group + 8 * gw);
  //  V by direct copies of the same rows into the V ring, with its swizzle:
  //     lane l fetches the chunk that lands at chunk position l % 16
  uint32_t v_dgoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * group + 8 * gw + 4 * i + (lane >> 4);
    v_dgoff[i] = (uint32_t)row * vv.row + (uint32_t)(16 * ((lane & 15) ^ vsw(row)));
  }
  //  QK^T fragments (A operand): K row l16 (+ 16 kb: immediate), chunk
  //     4 ks + g, i.e. dims 32 ks + 8 g .. +8; the slot is an immediate.
  uint32_t kf[4], vtr[8];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kf[ks] = (uint32_t)k_off(l16, 4 * ks + g);
  //  PV fragments (A operand, V^T) by transposing reads.  Within 16 lanes,
  //     lane m of a ds_read_b64_tr_b16 receives element m % 4 of the 8-byte
  //     pieces that lanes m / 4, 4 + m / 4, 8 + m / 4, 12 + m / 4 address.
  //     Lane L addresses key 4 (L / 16) + (L / 4) % 4 (+ 32 kb + 16 t: the
  //     32-key block and the read, immediates), head dims 16 db + 4 (L % 4)
  //     .. +4; so lane l receives head dim 16 db + l % 16 of keys
  //     32 kb + 16 t + 4 g + 0..3, its k-slots 8 g + 4 t .. +4.
  {
    const int row0 = 4 * g + ((lane >> 2) & 3);
    const int i4 = lane & 3;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vtr[db] = (uint32_t)(kVRingOffset + v_off(row0, 2 * db + (i4 >> 1)) + 8 * (i4 & 1));
  }

  // ---- ring traffic helpers
  // one of the two direct K copies of this wave: 1 KiB = 4 rows
  auto k_dma_one = [&](const i32x4_t &words, uint32_t slot_bytes, int i) __attribute__((always_inline)) {
    // the LDS address is added up here, not by the compiler: precomputed
    // sums for every slot would hold 16 scalar registers through the loop
    asm volatile(
        "s_add_u32 m0, %0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(k_m0), "v"(k_dgoff[i]), "s"(words), "s"(slot_bytes + 1024u * (uint32_t)i)
        : "memory", "scc");
  };
  // one of the two direct V copies of this wave
  auto v_dma_one = [&](const i32x4_t &words, uint32_t slot_bytes, int i) __attribute__((always_inline)) {
    asm volatile(
        "s_add_u32 m0, %0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(k_m0), "v"(v_dgoff[i]), "s"(words), "s"(kVRingOffset + slot_bytes + 1024u * (uint32_t)i)
        : "memory", "scc");
  };

  // ---- rings, before the loop: K and V tiles 0, 1, 2 in LDS, by the same
  // copies as in the loop but through the builtin, so that the compiler
  // counts them: the query transform then waits for the queries only and
  // runs while the tiles arrive.  Tile indices are clamped to T - 1 (a fixed
  // count of copies; extra ones land in slots no step reads).
  __builtin_amdgcn_sched_barrier(0);
  {
    typedef __attribute__((address_space(3))) void *lds_void_t;
    lds_char_t *dst = (lds_char_t *)lds + 256 * (32 * group + 8 * gw);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t tile = (uint32_t)(kt0 + min(j, T - 1)) * (uint32_t)kBC;   // first key
      const uint32_t skip_k = tile * vk.row, skip_v = tile * vv.row;   // the views' row pitches may differ
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(vk.base + skip_k, vk.bytes - skip_k);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vv.base + skip_v, vv.bytes - skip_v);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t)(dst + j * kKTileBytes + 1024 * i), 16,
                                                 k_dgoff[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t)(dst + kVRingOffset + j * kKTileBytes + 1024 * i),
                                                 16, v_dgoff[i], 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (FUSEQ) {
    // the transform's inputs and outputs pass through empty asm statements
    // after the copies and before their wait, which pins the transform
    // between the two (otherwise the compiler moves parts of it to either
    // side)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qf[h][ks]));
#pragma unroll
      for (int i = 0; i < 3; ++i) asm volatile("" : "+v"(qin.pos[h][i]));
    }
    q_transform(qf, qin, a, rope, g);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qf[h][ks]));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Accumulators, [.. + h] for the lane's query of half h:
  //  o[2 db + h]: O^T head dims 16 db + 4 g .. +4;
  //  s[2 kb + h]: S^T keys 16 kb + 4 g .. +4 of the tile (kb = 0..3);
  //  pf[2 kb + h]: P^T operand of 32-key block kb (kb = 0, 1): keys
  //      32 kb + 4 g .. +4, then 32 kb + 16 + 4 g .. +4.
  f32x4_t o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t s[8];
  bf16x8_t pf[4];
  float b_run[2] = {0.f, 0.f};        // the rows' running shifts, base-2 units
  f32x4_t bias[2] = {};               // fused: -b_run[h] in every element
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};   // [2 kb + h]: this lane's keys
  const f32x4_t zero = {};

  // Matrix half-step as a 32-step software pipeline over operand fragments,
  // each serving the MFMAs of both query halves: steps 0..15 are PV of the
  // current tile (32-key block kb = s/8, head-dim block db = s%8), steps
  // 16..31 QK^T of the next tile (dims 32 ks, ks = (s-16)/4, 16-key block
  // kb = (s-16)%4: eight accumulator chains in turn).  Fragment s+kPre is
  // requested from LDS before the MFMAs of step s are issued, and
  // scheduling fences keep that order.  The V tile of the PV steps is
  // complete before the half-step starts, so the first kPre fragments are
  // requested before the barrier.  A PV fragment is two transposing reads,
  // a QK^T fragment one ds_read_b128.
  constexpr int kPre = 6;
  auto frag = [&](int step, int kslot_bytes, int vslot_bytes) __attribute__((always_inline)) -> bf16x8_t {
    if (step >= 16) {
      const int ks = (step - 16) >> 2, kb = (step - 16) & 3;
      return lds_read_b128(lds + kf[ks] + (kslot_bytes + kb * 16 * 256));
    }
    const int kb = step >> 3, db = step & 7;
    return lds_read_tr2(lds + vtr[db] + (vslot_bytes + kb * 32 * 256));
  };
  auto matrix_step = [&](int step, bf16x8_t f) __attribute__((always_inline)) {
    if (step >= 16) {
      const int ks = (step - 16) >> 2, kb = (step - 16) & 3;
      // fused: Q' carries c and the accumulator starts at -b
#pragma unroll
      for (int h = 0; h < 2; ++h)
        s[2 * kb + h] = mfma16(f, qf[h][ks], ks ? s[2 * kb + h] : (FUSEQ ? bias[h] : zero));
    } else {
      const int kb = step >> 3, db = step & 7;
#pragma unroll
      for (int h = 0; h < 2; ++h) o[2 * db + h] = mfma16(f, pf[2 * kb + h], o[2 * db + h]);
    }
  };

  // Online softmax of tile j.  The lane holds, for query h, keys
  // 16 kb + 4 g + r of the tile in register r of s[2 kb + h]; x = c*S - b
  // (c = softmax scale * log2 e) by one FMA per score, or straight from the
  // MFMA in the fused form.  Common case: p = 2^x straight away; the row
  // maximum is only needed when some p may be large, which the lane's share
  // of the tile's row sum (>= every p in it) tells.  Then, or on the first
  // tile, b moves up to the row maximum (over the query's four lanes) when
  // that exceeds it by more than 8 (first tile: moves to it), O and l are
  // scaled by 2^-shift and p recomputed, so p <= 2^16 always and O / l is
  // unchanged.
  auto softmax = [&](int j, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value != 0;
    if constexpr (!FUSEQ) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[i][r] = fmaf(s[i][r], c, -b_run[i & 1]);
    }
    if ((kt0 + j) * kBC + kBC > N) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = (kt0 + j) * kBC + 16 * (i >> 1) + 4 * g + r;
          if (key >= N) s[i][r] = -INFINITY;
        }
    }
    float t[4];
    auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float acc;   // starts at the first pair: 0 + x is not folded (-0)
          bf16x8_t pv8;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int i = 2 * (2 * kb + half) + h;
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const float e0 = __builtin_amdgcn_exp2f(s[i][r]);
              const float e1 = __builtin_amdgcn_exp2f(s[i][r + 1]);
              acc = (half || r) ? acc + (e0 + e1) : e0 + e1;
              pv8[4 * half + r] = (__bf16)e0;
              pv8[4 * half + r + 1] = (__bf16)e1;
            }
          }
          t[2 * kb + h] = acc;
          pf[2 * kb + h] = pv8;
        }
    };
    if constexpr (!kFirst) exps();
    const float tot0 = t[0] + t[2], tot1 = t[1] + t[3];
    if (kFirst || __builtin_amdgcn_ballot_w64(!(tot0 <= 65536.f) || !(tot1 <= 65536.f)) != 0) {
      float mx[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float mq[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f32x4_t x = s[2 * kb + h];
          mq[kb] = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        }
        mx[h] = quad_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
      }
      if (kFirst || __builtin_amdgcn_ballot_w64(mx[0] > 8.0f || mx[1] > 8.0f) != 0) {
        float d[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          d[h] = kFirst ? mx[h] : fmaxf(mx[h], 0.f);
          b_run[h] += d[h];
          if constexpr (FUSEQ) {
#pragma unroll
            for (int e = 0; e < 4; ++e) bias[h][e] = -b_run[h];
          }
        }
        if constexpr (!kFirst) {
          const float alpha[2] = {__builtin_amdgcn_exp2f(-d[0]), __builtin_amdgcn_exp2f(-d[1])};
#pragma unroll
          for (int i = 0; i < 4; ++i) l_part[i] *= alpha[i & 1];
#pragma unroll
          for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[i][e] *= alpha[i & 1];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[i][r] -= d[i & 1];
        exps();
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l_part[i] += t[i];
    // keep the exponentials in this (vector) half-step: without these the
    // compiler sinks them next to their MFMA consumers in the matrix one
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pf[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(l_part[i]));
  };

  // Schedule of each wave: QK^T(0), vector half-step of tile 0, then per
  // tile j a matrix half-step (PV(j), QK^T(j+1)) followed by the vector
  // half-step of tile j+1 (softmax, first fragment reads of the next matrix
  // half-step).  Group 1 runs one barrier behind group 0, so in every phase
  // one group is in a matrix half-step and the other in a vector half-step.
  // Ring traffic of the matrix half-step of tile j: copy K and V tile j+3
  // into LDS.  Slot reuse: both slots of tile j+3 last held tile j-1, read
  // by PV(j-1) and QK^T(j-1) in matrix half-steps j-1 and j-2; at least one
  // barrier separates those reads from either group's writes.  Tile indices
  // of the copies are clamped to T-1: extra copies land in slots no later
  // step reads.  The vmcnt wait in each vector half-step retires the
  // previous matrix half-step's copies, so a tile is in LDS two barriers
  // before its first reader.
  // where in the 32-step matrix pipeline the two V and the two K copies go
  constexpr int kVLoad0 = 12, kVLoadGap = 6, kKLoad0 = 26, kKLoadGap = 3;
  // vector half-step tail: retire this wave's copies, then request the
  // first fragments of the next matrix half-step (V slot of tile j, K slot
  // of tile j+1)
  auto vector_tail = [&](int kslot_bytes, int vslot_bytes, bf16x8_t *ring) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < kPre; ++i) ring[i] = frag(i, kslot_bytes, vslot_bytes);
  };
  // Iteration j (ring slot R = j % 4): matrix half-step PV(j), QK^T(j+1)
  // with the ring traffic, then the vector half-step of tile j+1.
  auto iteration = [&](int j, auto slot, bf16x8_t *ring) __attribute__((always_inline)) {
    constexpr int R = decltype(slot)::value;
    constexpr int kCur = R * kKTileBytes;                       // V slot of tile j (same byte offset in both rings)
    constexpr int kNext = ((R + 1) % kSlots) * kKTileBytes;    // slots of tile j+1
    constexpr int kPlus3 = ((R + 3) % kSlots) * kKTileBytes;   // slots of tile j+3 (K and V)
    const int tn = min(j + 3, T - 1);
    // the vector half-step wrote no LDS, and the fragment reads it issued
    // touch a slot no wave writes before the next barrier: a plain barrier
    // that does not wait for them
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_setprio(3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 0; step < 32; ++step) {
      const bf16x8_t f = ring[step % kPre];
      if (step + kPre < 32) ring[step % kPre] = frag(step + kPre, kNext, kCur);
      matrix_step(step, f);
      if (step == kVLoad0 || step == kVLoad0 + kVLoadGap) v_dma_one(tile_words(vv, kt0 + tn, kBC), kPlus3, step == kVLoad0 ? 0 : 1);
      if (step == kKLoad0 || step == kKLoad0 + kKLoadGap) k_dma_one(tile_words(vk, kt0 + tn, kBC), kPlus3, step == kKLoad0 ? 0 : 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    if (j + 1 < T) {
      softmax(j + 1, Slot<0>{});
      vector_tail(((R + 2) % kSlots) * kKTileBytes, kNext, ring);
    }
  };

  __syncthreads();
  if (group == 1) __syncthreads();
  // QK^T(0) from slot 0, then the vector half-step of tile 0
#pragma unroll
  for (int step = 16; step < 32; ++step) matrix_step(step, frag(step, 0, 0));
  __syncthreads();
  bf16x8_t ring[kPre];
  softmax(0, Slot<1>{});
  vector_tail(1 * kKTileBytes, 0, ring);
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

  // ---- epilogue: O / l, one bf16 rounding; the lane holds head dims
  // 16 db + 4 g .. +4 of its two queries; stores past the head's end are
  // dropped
  float l_run[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) l_run[h] = quad_sum(l_part[h] + l_part[2 + h]);   // the query's four lanes
  // a piece of a split block: the piece that finishes second merges
  if (job.cut >= 0 && !split_merge<2>(a, job, o, b_run, l_run, tid, split_ticket)) return;
  const float inv[2] = {1.0f / l_run[0], 1.0f / l_run[1]};
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(vo.base, vo.bytes);
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4_t x = o[2 * db + h];
      u32x2_t w;
      w[0] = pack_bf16(x[0] * inv[h], x[1] * inv[h]);
      w[1] = pack_bf16(x[2] * inv[h], x[3] * inv[h]);
      const uint32_t off = (uint32_t)q_row[h] * vo.row + (uint32_t)((16 * db + 4 * g) * 2);
      __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
    }
}

template <bool FUSEQ, bool STRIDED>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(ForwardArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int simd_of_wave[kWaves];
  __shared__ int split_ticket;
  __shared__ RopeLds rope;

  const int tid = threadIdx.x;
  if constexpr (FUSEQ) rope_lds_fill(&rope, a, tid, kThreads);   // before the barrier in pingpong_order
  // ---- ping-pong groups: the two waves of a SIMD land in different groups
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
  const int64_t ntiles = (a.N + kBR - 1) / kBR;
  const int64_t grid = a.split_groups > 0 ? a.split_groups : std::min<int64_t>(a.whole_groups, ntiles * a.BH);
  // Raise the dynamic-LDS limit once per device (idempotent, so a race
  // between threads only repeats the call).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_kernel<FUSEQ, STRIDED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<FUSEQ, STRIDED>), dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const ForwardArgs &a, bool fused, bool strided, hipStream_t s) {
  const int v = (fused ? 2 : 0) | (strided ? 1 : 0);
  switch (v) {
    case 0: return launch<false, false>(a, s);
    case 1: return launch<false, true>(a, s);
    case 2: return launch<true, false>(a, s);
    default: return launch<true, true>(a, s);
  }
}

int64_t forward_grid_blocks(int64_t BH, int64_t N) { return BH * ((N + kBR - 1) / kBR); }
int64_t forward_key_tiles(int64_t N) { return (N + kBC - 1) / kBC; }

}  // namespace fluxattn

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
//    tiles sit in LDS as they are in memory (row = key); two transposing
//    reads (ds_read_b64_tr_b16) give a lane those 8 keys at its head dim.
//  * Ping-pong: the waves form two groups of four, one wave of each group per
//    SIMD.  Every phase ends with a workgroup barrier; in each phase one
//    group runs its matrix half-step (PV of the current tile, QK^T of the
//    next one: 32 MFMAs, at raised wave priority) while the other runs its
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
//    maximum is only scanned when the tile's row sum (an upper bound of
//    every probability in it) exceeds 2^16; b then moves up to the maximum
//    if that exceeds it by more than 8, with O and l rescaled.  O / l is
//    unchanged by the shift.  l sums the fp32 probabilities; P is rounded
//    to bf16 for the MFMA.
//  * blockIdx is remapped so that the workgroups the dispatcher sends to one
//    XCD (blockIdx % 8) take consecutive query tiles of the same (b,h) and
//    share its K/V stream through that XCD's L2.
//  * A workgroup runs a list of jobs (attn_common.h): normally one whole
//    query block; when the host balances the last round, a persistent grid
//    takes whole blocks in launch order and then an equal share of the
//    tail's (query block, key tile) pairs, a cut block's pieces being
//    merged by whichever finishes last.
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
//  V tile: row = key (256 B), chunk c stored at c ^ vsw(key), vsw taking
//          key % 4 to 0, 6, 10, 12.  A transposing read touches 4
//          consecutive keys x 32 bytes per 16 lanes and 8 keys x 64 bytes per
//          wave; the swizzle puts every 32-byte piece of one 256-byte bank
//          row in its own banks.  The swizzle only moves chunks within bits
//          1..3 of their index and depends on key % 4, so key offsets that
//          are multiples of 4 stay immediates.
__device__ __forceinline__ int k_off(int key, int ch) { return key * 256 + ((ch ^ (key & 15)) << 4); }
__device__ __forceinline__ int vsw(int key) { return (0xCA60 >> (4 * (key & 3))) & 15; }
__device__ __forceinline__ int v_off(int key, int ch) { return key * 256 + ((ch ^ vsw(key)) << 4); }

__device__ __forceinline__ bf16x8_t lds_read_b128(const char *p) {
  return *reinterpret_cast<const bf16x8_t *>(p);
}
typedef short i16x4_t __attribute__((ext_vector_type(4)));
// two transposing reads: elements 0..3 from p, 4..7 from p + 2048 (8 keys on)
__device__ __forceinline__ bf16x8_t lds_read_tr2(const char *p) {
  typedef __attribute__((address_space(3))) i16x4_t *lp;
  const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p));
  const i16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p + 2048));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Queries of the fused entry points: raw Q -> RMSNorm over the 128 dims ->
// rotation of each adjacent pair by its axis position times frequency
// (the prologue's operations, on the 64 dims this lane holds:
// 16 kk + 8 hi + i; the other 64 are in lane ^ 32) -> times c = softmax
// scale * log2 e -> bf16, so that the QK^T MFMA yields base-2 logits.  The
// one bf16 rounding of Q' is the same as the prologue's, applied to c Q'.
__device__ __forceinline__ void load_q_fused(bf16x8_t (&qf)[8], const ForwardArgs &a, const RopeLds *rope,
                                             const HeadView &vq, int q_row, int hi) {
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(vq.base, vq.bytes);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const uint32_t off = (uint32_t)q_row * vq.row + (uint32_t)((16 * kk + 8 * hi) * 2);
    qf[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
  }
  float ss = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (float)qf[kk][i];
      ss = fmaf(x, x, ss);
    }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(ss), __float_as_int(ss), false, false);
    ss = __int_as_float(sw[0]) + __int_as_float(sw[1]);   // all 128 dims of this query
  }
  // rstd and the logit scale c folded into the weights: Q' c = (x w rstd c)
  // rotated
  const float rs = a.scale_log2 / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
  // position ids of this query (rows past N belong to no token: any valid
  // row serves, their outputs are never stored)
  const int tok = min(q_row, a.N - 1);
  const float pf[3] = {(float)a.pos[3 * tok + 0], (float)a.pos[3 * tok + 1], (float)a.pos[3 * tok + 2]};
  const float *w_q = stream_weights(a, tok);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)qf[kk][i];
    const float4 w0 = *reinterpret_cast<const float4 *>(w_q + 16 * kk + 8 * hi);
    const float4 w1 = *reinterpret_cast<const float4 *>(w_q + 16 * kk + 8 * hi + 4);
    const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float sn[4], cs[4];
    rotations4(rope, pf, 8 * kk + 4 * hi, sn, cs);   // pairs 8 kk + 4 hi + m
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float u = x[2 * m] * (w[2 * m] * rs);
      const float v = x[2 * m + 1] * (w[2 * m + 1] * rs);
      qf[kk][2 * m] = (__bf16)(u * cs[m] - v * sn[m]);
      qf[kk][2 * m + 1] = (__bf16)(u * sn[m] + v * cs[m]);
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
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;
  // wave-uniform job fields (they address the scalar buffer descriptors)
  const int bh = __builtin_amdgcn_readfirstlane(job.bh), qt = __builtin_amdgcn_readfirstlane(job.qt);
  const int kt0 = __builtin_amdgcn_readfirstlane(job.kt0), T = __builtin_amdgcn_readfirstlane(job.T);

  // ---- per-head base pointers, token-row pitches and buffer extents
  const HeadView vq = head_view<STRIDED>(a.q, a.sq, 2, bh, a.H, N);
  // ---- queries: qf[kk] = Q[q][16kk + 8hi .. +8), q = this lane's row
  // (first, so the fused transform's temporaries overlap no other state)
  const int q_row = qt * kBR + wave * 32 + l32;
  bf16x8_t qf[8];
  if constexpr (FUSEQ) {
    load_q_fused(qf, a, rope, vq, q_row, hi);
  } else {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(vq.base, vq.bytes);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint32_t off = (uint32_t)q_row * vq.row + (uint32_t)((16 * kk + 8 * hi) * 2);
      qf[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
  }

  const HeadView vk = head_view<STRIDED>(a.k, a.sk, 2, bh, a.H, N);
  const HeadView vv = head_view<STRIDED>(a.v, a.sv, 2, bh, a.H, N);
  const HeadView vo = head_view<STRIDED>(a.o, a.so, 2, bh, a.H, N);

  const float c = a.scale_log2;
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((lds_char_t *)lds);

  // ---- lane constants (bytes).  Each group loads half of every tile:
  // keys [32 g, 32 g + 32).
  //  K by direct copies: wave gw of group g copies rows
  //     32 g + 8 gw .. +8 with two buffer_load_dwordx4 ... lds; lane l of
  //     copy i fetches the chunk the K swizzle puts at LDS slot row
  //     32 g + 8 gw + 4 i + l / 16, chunk position l % 16.
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
  //  MFMA fragments: K (kk) row l32, chunk 2 kk + hi; slot and 32-key
  //     block are immediates.
  uint32_t kf[8], vtr[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kf[kk] = (uint32_t)k_off(l32, 2 * kk + hi);
  //  PV operand by transposing reads.  Within 16 lanes, lane m of a
  //     ds_read_b64_tr_b16 receives element m % 4 of the 8-byte pieces that
  //     lanes m / 4, 4 + m / 4, 8 + m / 4, 12 + m / 4 address.  Lane L
  //     addresses key 4 (L / 32) + (L / 4) % 4 (+ 16 st + 8 half: slot and
  //     key offsets are immediates), head dims 32 db + 16 ((L / 16) % 2) +
  //     4 (L % 4) .. +4; so lane l receives head dim 32 db + l % 32 of keys
  //     16 st + 8 half + 4 (l / 32) + 0..3, the order of the B operand.
  {
    const int row0 = 4 * hi + ((lane >> 2) & 3);
    const int dh = (lane >> 4) & 1, i4 = lane & 3;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      vtr[db] = (uint32_t)(kVRingOffset + v_off(row0, 4 * db + 2 * dh + (i4 >> 1)) + 8 * (i4 & 1));
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

  // ---- rings, before the loop: K and V tiles 0, 1, 2 in LDS
  for (int j = 0; j < 3 && j < T; ++j) {
    const i32x4_t w = tile_words(vk, kt0 + j, kBC);
    k_dma_one(w, j * kKTileBytes, 0);
    k_dma_one(w, j * kKTileBytes, 1);
    const i32x4_t wv = tile_words(vv, kt0 + j, kBC);
    v_dma_one(wv, j * kKTileBytes, 0);
    v_dma_one(wv, j * kKTileBytes, 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  f32x16_t s[2];
  bf16x8_t pf[4];
  float b_run = 0.f;      // this row's running shift, base-2 units
  f32x16_t bias = {};     // fused: -b_run in every element
  float l_part[4] = {0.f, 0.f, 0.f, 0.f};
  const f32x16_t zero = {};

  // Matrix half-step as a 32-step software pipeline over operand fragments:
  // steps 0..15 are PV of the current tile (16-key step st = s/4, head-dim
  // block db = s%4), steps 16..31 QK^T of the next tile (kk = (s-16)/2,
  // 32-key block kb = (s-16)%2).  Fragment s+kPre is requested from LDS
  // before MFMA s is issued, and scheduling fences keep that order.  The
  // V tile of the PV steps is complete before the half-step starts, so the
  // first kPre fragments are requested before the barrier.  A PV fragment
  // is two transposing reads, a QK^T fragment one ds_read_b128.
  constexpr int kPre = 6;
  auto frag = [&](int step, int kslot_bytes, int vslot_bytes) __attribute__((always_inline)) -> bf16x8_t {
    if (step >= 16) {
      const int kk = (step - 16) >> 1, kb = (step - 16) & 1;
      return lds_read_b128(lds + kf[kk] + (kslot_bytes + kb * 32 * 256));
    }
    const int st = step >> 2, db = step & 3;
    return lds_read_tr2(lds + vtr[db] + (vslot_bytes + st * 16 * 256));
  };
  auto matrix_step = [&](int step, bf16x8_t f) __attribute__((always_inline)) {
    if (step >= 16) {
      const int kk = (step - 16) >> 1, kb = (step - 16) & 1;
      // fused: Q' carries c and the accumulator starts at -b
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[kk], kk ? s[kb] : (FUSEQ ? bias : zero), 0, 0, 0);
    } else {
      const int st = step >> 2, db = step & 3;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[st], o[db], 0, 0, 0);
    }
  };

  // Online softmax of tile j.  Lane owns query l32 and keys
  // 32 kb + 8 (r / 4) + 4 hi + r % 4 of the tile (register r of s[kb]);
  // x = c*S - b (c = softmax scale * log2 e) by one FMA per score, or
  // straight from the MFMA in the fused form.  Common case: p = 2^x
  // straight away; the row maximum is
  // only needed when some p may be large, which the tile's own row sum
  // (>= every p in it) tells.  Then, or on the first tile, b moves up to the
  // row maximum when that exceeds it by more than 8 (first tile: moves to
  // it), O and l are scaled by 2^-shift and p recomputed, so p <= 2^16
  // always and O / l is unchanged.
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
    float t[4];
    auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, r0 = 8 * (st & 1);
        float acc;   // starts at the first pair: 0 + x is not folded (-0)
        bf16x8_t pv8;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float e0 = __builtin_amdgcn_exp2f(s[kb][r0 + i]);
          const float e1 = __builtin_amdgcn_exp2f(s[kb][r0 + i + 1]);
          acc = i ? acc + (e0 + e1) : e0 + e1;
          pv8[i] = (__bf16)e0;
          pv8[i + 1] = (__bf16)e1;
        }
        t[st] = acc;
        pf[st] = pv8;
      }
    };
    if constexpr (!kFirst) exps();
    const float tot = (t[0] + t[1]) + (t[2] + t[3]);
    if (kFirst || __builtin_amdgcn_ballot_w64(!(tot <= 65536.f)) != 0) {
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
      if (kFirst || __builtin_amdgcn_ballot_w64(mx > 8.0f) != 0) {
        const float d = kFirst ? mx : fmaxf(mx, 0.f);
        b_run += d;
        if constexpr (FUSEQ) {
#pragma unroll
          for (int i = 0; i < 16; ++i) bias[i] = -b_run;
        }
        if constexpr (!kFirst) {
          const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
          for (int g = 0; g < 4; ++g) l_part[g] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] -= d;
        exps();
      }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) l_part[st] += t[st];
    // keep the exponentials in this (vector) half-step: without these the
    // compiler sinks them next to their MFMA consumers in the matrix one
#pragma unroll
    for (int st = 0; st < 4; ++st) asm volatile("" : "+v"(pf[st]));
#pragma unroll
    for (int g = 0; g < 4; ++g) asm volatile("" : "+v"(l_part[g]));
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

  // ---- epilogue: O / l, one bf16 rounding; lane holds query l32 and head
  // dims 32 db + 8 g + 4 hi + (0..3); stores past the head's end are dropped
  float l_run = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l_run), __float_as_int(l_run), false, false);
    l_run = __int_as_float(sw[0]) + __int_as_float(sw[1]);   // both half-waves' keys
  }
  // a piece of a split block: the piece that finishes second merges
  if (job.cut >= 0 && !split_merge(a, job, o, b_run, l_run, tid, split_ticket)) return;
  const float inv = 1.0f / l_run;
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
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(ForwardArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int simd_of_wave[kWaves];
  __shared__ int split_ticket;
  __shared__ RopeLds rope;

  const int tid = threadIdx.x;
  if constexpr (FUSEQ) rope_lds_fill(&rope, a, tid);   // before the barrier in pingpong_order
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
    const SplitRange r = split_range(a, kBR, kBC, xcd_logical_block(blockIdx.x, gridDim.x));
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
  const int64_t grid = a.split_groups > 0 ? a.split_groups : ntiles * a.BH;
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

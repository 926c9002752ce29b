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
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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

// ---- Key-range split.  Without a split, the launch has whole_groups
// persistent workgroups, which the dispatcher deals to the 8 XCDs round
// robin; those on XCD x take the blocks of its contiguous range (the range
// xcd_logical_block gives it) in turn.  With split_groups = G
// persistent workgroups and nb blocks, the first F = split_whole rounds
// (chosen on the host, F G < nb) go as whole blocks in launch order:
// workgroup w takes blocks w, w + G, ..., so the workgroups running at one
// time work on neighbouring blocks of the same heads and stream the same
// key tiles in step, sharing them in L2.  The remaining nb - F G blocks
// form the tail: its (query block, key tile) pairs, key tiles in order
// inside each block, are
// dealt out as G equal contiguous shares, share w = pairs
// [U w / G, U (w + 1) / G) of the tail's U to workgroup w.  A share spans
// at most two tail blocks when it is shorter than a block, and then cuts
// blocks into two or more pieces; a longer share has at most a partial
// block at each end.  A partial piece goes to slot 2w if it is the first
// job of share w, else 2w + 1.
struct SplitRange {
  int whole;          // whole blocks still to do before the tail
  int blk, stride;    // next whole block, and the step between them
  int64_t u, end;     // next pair of the tail share, end of the share
  int64_t start;      // first pair of the share
  int64_t U;          // pairs in the tail
  int base;           // first tail block
  int key_tiles, q_tiles, logical, groups;
};
struct SplitJob {
  int bh, qt;         // head and query block
  int kt0, T;         // key tiles [kt0, kt0 + T)
  int cut;            // -1: the whole block; else its index in the tail
  int slot;           // partial slot of this piece
  int w_lo, w_hi;     // shares that hold pieces of the block
  int64_t U;          // tail pairs, key tiles per block and groups: what
  int key_tiles;      // the merge needs to find the other pieces' slots
  int groups;
};

__device__ __forceinline__ SplitRange split_range(const ForwardArgs &a, int rows, int keys, int bid, int grid) {
  SplitRange r;
  r.q_tiles = (a.N + rows - 1) / rows;
  r.key_tiles = (a.N + keys - 1) / keys;
  const int logical = xcd_logical_block(bid, grid);
  r.logical = logical;
  r.blk = logical;
  r.groups = a.split_groups;
  if (a.split_groups > 0) {
    const int G = a.split_groups;
    const int nb = a.BH * r.q_tiles;
    r.whole = a.split_whole;
    r.stride = G;
    r.base = r.whole * G;
    r.U = (int64_t)(nb - r.base) * r.key_tiles;
    r.start = r.U * logical / G;
    r.u = r.start;
    r.end = r.U * (logical + 1) / G;
  } else {
    // XCD x holds blocks [x q8 + min(x, r8), + q8 + (x < r8)) and the
    // workgroups bid = x, x + 8, ... of the grid; its j-th takes the range's
    // blocks j, j + slots, ...
    const int nb = a.BH * r.q_tiles;
    const int x = bid & 7, j = bid >> 3, q8 = nb >> 3, r8 = nb & 7;
    const int count = q8 + (x < r8), slots = (grid + 7 - x) >> 3;
    r.blk = x * q8 + min(x, r8) + j;
    r.stride = slots;
    r.whole = j < count ? (count - j + slots - 1) / slots : 0;
    r.base = 0;
    r.U = r.start = r.u = r.end = 0;
  }
  return r;
}

// The range state back from LDS as wave-uniform (scalar) values.
__device__ __forceinline__ SplitRange split_range_load(const SplitRange *p) {
  auto u32 = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  auto u64 = [](int64_t v) {
    const uint64_t x = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  SplitRange r;
  r.whole = u32(p->whole);
  r.blk = u32(p->blk);
  r.stride = u32(p->stride);
  r.u = u64(p->u);
  r.end = u64(p->end);
  r.start = u64(p->start);
  r.U = u64(p->U);
  r.base = u32(p->base);
  r.key_tiles = u32(p->key_tiles);
  r.q_tiles = u32(p->q_tiles);
  r.logical = u32(p->logical);
  r.groups = u32(p->groups);
  return r;
}

// Share of tail pair u: the largest w with U w / G <= u.
__device__ __forceinline__ int split_share_of(int64_t u, int64_t U, int G) { return (int)(((u + 1) * G - 1) / U); }

// Partial slot of share w's piece of tail block b: its first job when the
// share starts inside or at the start of the block, else its last.
__device__ __forceinline__ int split_slot(int w, int b, int64_t U, int key_tiles, int G) {
  return U * w / G >= (int64_t)b * key_tiles ? 2 * w : 2 * w + 1;
}

// Next job of the workgroup (false when it is done).
__device__ __forceinline__ bool split_next(SplitRange &r, SplitJob &j) {
  int blk;
  j.cut = -1;
  j.slot = j.w_lo = j.w_hi = 0;
  j.U = r.U;
  j.key_tiles = r.key_tiles;
  j.groups = r.groups;
  if (r.whole > 0) {
    blk = r.blk;
    r.blk += r.stride;
    --r.whole;
    j.kt0 = 0;
    j.T = r.key_tiles;
  } else {
    if (r.u >= r.end) return false;
    const int b = (int)(r.u / r.key_tiles);
    j.kt0 = (int)(r.u - (int64_t)b * r.key_tiles);
    j.T = (int)min((int64_t)(r.key_tiles - j.kt0), r.end - r.u);
    r.u += j.T;
    blk = r.base + b;
    if (j.T != r.key_tiles) {
      j.cut = b;
      j.slot = r.start >= (int64_t)b * r.key_tiles ? 2 * r.logical : 2 * r.logical + 1;
      j.w_lo = split_share_of((int64_t)b * r.key_tiles, r.U, r.groups);
      j.w_hi = split_share_of((int64_t)(b + 1) * r.key_tiles - 1, r.U, r.groups);
    }
  }
  j.bh = blk / r.q_tiles;
  j.qt = blk - j.bh * r.q_tiles;
  return true;
}

// End of one piece of a cut block.  The piece stores its O accumulators
// o (unnormalised, relative to 2^b: row shift b in base-2 units) and its
// normalisers l in its slot, then counts itself in at the block.  All but
// the last to arrive return false; the last reads the other pieces and
// merges them into (o, b, l): every piece rescaled to the largest shift
// and summed in share order (whichever piece merges, the result is the
// same, bit for bit), resets the count for the next launch and returns
// true (it then stores O).  Nobody waits for anybody.
// A thread holds R query rows (1 or 2): its 64 accumulators are 16 float4
// (acc4 below), float4 i belonging to row i % R, and b[r], l[r] are row r's
// shift and normaliser.  Float4 i of every thread sits at i * 8 KiB (a
// scalar offset) + 16 * thread.
// Coherence between the workgroups (possibly on different XCDs, whose L2
// caches are not coherent with each other) comes from device-scope
// accesses to the partials and the count alone: the partial stores and
// loads carry the device-scope cache policy (sc1), the stores are retired
// (vmcnt 0) before the workgroup barrier that precedes the count, and the
// count is a device-scope atomic.  No cache-wide writeback or invalidate is
// needed, so the other workgroups' cached K and V tiles stay put.  All
// threads of the workgroup call this; it contains two workgroup barriers.
constexpr int kCPolDevice = 16;   // buffer cache policy: sc1 (device scope)

// float4 i of a thread's 64 accumulators, held as 4 x 16 or as 16 x 4 floats
__device__ __forceinline__ f32x4_t acc4(const f32x16_t (&o)[4], int i) {
  const int db = i >> 2, g = i & 3;
  return f32x4_t{o[db][4 * g + 0], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
}
__device__ __forceinline__ f32x4_t acc4(const f32x4_t (&o)[16], int i) { return o[i]; }
__device__ __forceinline__ void acc4_set(f32x16_t (&o)[4], int i, f32x4_t v) {
  const int db = i >> 2, g = i & 3;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[db][4 * g + e] = v[e];
}
__device__ __forceinline__ void acc4_set(f32x4_t (&o)[16], int i, f32x4_t v) { o[i] = v; }

template <int R, class Acc>
__device__ __forceinline__ bool split_merge(const ForwardArgs &a, const SplitJob &job, Acc &o, float (&b)[R],
                                            float (&l)[R], int tid, int *ticket) {
  static_assert(R == 1 || R == 2, "one or two rows per thread");
  constexpr uint32_t kPieceBytes = (uint32_t)(kSplitPieceFloats * 4);
  constexpr uint32_t kBLOffset = 64u * 4u * kSplitThreads;
  auto slot_rsrc = [&](int slot) {
    return make_rsrc(a.split_part + (int64_t)slot * kSplitPieceFloats, kPieceBytes);
  };
  const uint32_t t16 = (uint32_t)tid * 16u;
  {
    const __amdgpu_buffer_rsrc_t mine = slot_rsrc(job.slot);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc4(o, i)), mine, t16,
                                             (uint32_t)i * (16u * kSplitThreads), kCPolDevice);
    // (b0, l0, b1, l1)
    u32x4_t w;
    w[0] = __float_as_uint(b[0]);
    w[1] = __float_as_uint(l[0]);
    w[2] = __float_as_uint(b[R - 1]);
    w[3] = __float_as_uint(l[R - 1]);
    __builtin_amdgcn_raw_buffer_store_b128(w, mine, kBLOffset + t16, 0, kCPolDevice);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) *ticket = __hip_atomic_fetch_add(a.split_cnt + job.cut, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*ticket != job.w_hi - job.w_lo) return false;
  if (tid == 0) __hip_atomic_store(a.split_cnt + job.cut, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the largest row shifts over the pieces
  float m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) m[r] = b[r];
  for (int w = job.w_lo; w <= job.w_hi; ++w) {
    const u32x4_t blw = __builtin_amdgcn_raw_buffer_load_b128(
        slot_rsrc(split_slot(w, job.cut, job.U, job.key_tiles, job.groups)), kBLOffset + t16, 0, kCPolDevice);
#pragma unroll
    for (int r = 0; r < R; ++r) m[r] = fmaxf(m[r], __uint_as_float(blw[2 * r]));
  }
  // sum in share order, every piece (this one too) read back from its
  // slot, into o
#pragma unroll
  for (int i = 0; i < 16; ++i) acc4_set(o, i, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int r = 0; r < R; ++r) l[r] = 0.f;
  for (int w = job.w_lo; w <= job.w_hi; ++w) {
    const __amdgpu_buffer_rsrc_t piece = slot_rsrc(split_slot(w, job.cut, job.U, job.key_tiles, job.groups));
    const u32x4_t blw = __builtin_amdgcn_raw_buffer_load_b128(piece, kBLOffset + t16, 0, kCPolDevice);
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sc[r] = __builtin_amdgcn_exp2f(__uint_as_float(blw[2 * r]) - m[r]);
      l[r] = fmaf(__uint_as_float(blw[2 * r + 1]), sc[r], l[r]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(piece, t16, (uint32_t)i * (16u * kSplitThreads), kCPolDevice);
      f32x4_t y = acc4(o, i);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = fmaf(__uint_as_float(x[e]), sc[i % R], y[e]);
      acc4_set(o, i, y);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) b[r] = m[r];
  return true;
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

// Tables of the fused query prologue in LDS: the rotation rates rate[a][p]
// as in the arguments (one nonzero axis per pair), and the query norm
// weights of each stream.  Filled by the workgroup's threads before its
// first barrier.
struct alignas(16) RopeLds {
  float rate[3][kPairs];
  float wq[4][kHeadDim];
};

// Streams of the launch: those whose first token lies inside the sequence
// (the host sets the starts of absent ones past N).
__device__ __forceinline__ int stream_count(const ForwardArgs &a) {
  return 1 + (a.streams.start[1] <= a.N) + (a.streams.start[2] <= a.N) + (a.streams.start[3] <= a.N);
}

// Stream of a token.
__device__ __forceinline__ int stream_of(const ForwardArgs &a, int tok) {
  return (tok >= a.streams.start[1]) + (tok >= a.streams.start[2]) + (tok >= a.streams.start[3]);
}

__device__ __forceinline__ void rope_lds_fill(RopeLds *t, const ForwardArgs &a, int tid, int threads) {
  if (tid < kPairs) {
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) t->rate[ax][tid] = a.rope_rate[ax][tid];
  }
  const int n = stream_count(a) * kHeadDim;
  for (int i = tid; i < n; i += threads) t->wq[i / kHeadDim][i % kHeadDim] = a.w_q[i];
}

// (sin, cos) of the rotations of pairs p0 .. p0+3 (p0 a multiple of 4) of a
// token at positions pf: angle = sum over axes of pf[a] * rate[a][p] in
// revolutions (two of the three products are exactly 0, so this is the one
// product of the pair's own axis), reduced to [0, 1) for the hardware sine
// / cosine (absolute error about 1e-6 plus the fp32 rounding of the
// product, 6e-8 of it).
__device__ __forceinline__ void rotations4(const RopeLds *t, const float (&pf)[3], int p0, float (&sn)[4],
                                           float (&cs)[4]) {
  const float4 r0 = *reinterpret_cast<const float4 *>(&t->rate[0][p0]);
  const float4 r1 = *reinterpret_cast<const float4 *>(&t->rate[1][p0]);
  const float4 r2 = *reinterpret_cast<const float4 *>(&t->rate[2][p0]);
  const float a0[4] = {r0.x, r0.y, r0.z, r0.w}, a1[4] = {r1.x, r1.y, r1.z, r1.w}, a2[4] = {r2.x, r2.y, r2.z, r2.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float rev = __builtin_amdgcn_fractf(fmaf(pf[2], a2[m], fmaf(pf[1], a1[m], pf[0] * a0[m])));
    sn[m] = __builtin_amdgcn_sinf(rev);
    cs[m] = __builtin_amdgcn_cosf(rev);
  }
}

}  // namespace attn
}  // namespace fluxattn

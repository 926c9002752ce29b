// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fluxattn.h"

namespace fluxattn {

constexpr int kHeadDim = 128;
constexpr int kPairs = kHeadDim / 2;

// Per head-dimension pair p (dims 2p, 2p+1): which position axis rotates it
// and its frequency theta^(-2j/axes_a) in revolutions (divided by 2 pi in
// fp64 on the host, rounded to fp32).
struct RopeTable {
  float freq[kPairs];
  int8_t axis[kPairs];
};

// Element strides of a [B, H, N, D] view (D contiguous).
struct Strides {
  int64_t b, h;
  int32_t n;
};

// Token ranges with their own norm weights: stream s covers tokens
// [start[s], start[s+1]); unused entries hold INT32_MAX.
struct Streams {
  int32_t start[4];   // start[0] = 0
};

struct PrologueArgs {
  const void *q, *k;
  void *q_out, *k_out;
  const float *w_q, *w_k;             // [streams, D]
  const int32_t *pos;
  const float *q_scale, *k_scale;     // fp8 only
  float *q_scale_out, *k_scale_out;   // fp8 only
  int64_t BH;                         // B * H
  int32_t H;
  int32_t N;
  float eps;
  Strides sq, sk, sqo, sko;
  Streams streams;
  int32_t num_streams;
  int32_t bh_chunk;                   // (b,h) rows per block along grid.y
};

struct ForwardArgs {
  const void *q, *k, *v;
  void *o;
  const float *q_scale, *k_scale, *v_scale;  // fp8 only
  int32_t BH;
  int32_t H;
  int32_t N;
  float scale_log2;   // softmax_scale * log2(e)
  Strides sq, sk, sv, so;   // used by the strided kernels only
  Streams streams;          // fused query prologue only
  // fused query prologue only: raw q is normalised and rotated on load
  const float *w_q;
  const int32_t *pos;
  float eps;
  // pair p turns by pos[a] * rope_rate[a][p] revolutions summed over the
  // three axes a: rope_rate[a][p] = theta^(-2 j / axes[a]) / (2 pi) for the
  // axis a that pair p belongs to (index j inside it), 0 for the other two
  // (the key prologue's frequencies, in revolutions)
  float rope_rate[3][kPairs];
  // Key-range split (split_groups > 0): a persistent grid of split_groups
  // workgroups, split_whole rounds of whole blocks first, then an equal
  // contiguous share each of the remaining (query block, key tile) pairs.  A query block cut between
  // workgroups leaves one partial result per piece in split_part; the last
  // piece to finish merges them (split_cnt holds the arrival count of each
  // cut block and is left at zero).
  float *split_part;
  int32_t *split_cnt;
  int32_t split_groups;
  int32_t split_whole;      // rounds of whole blocks before the tail
  // Uncut launches (split_groups <= 0): a persistent grid of this many
  // workgroups (at most one per compute unit and per query block), each
  // taking whole blocks in turn.
  int32_t whole_groups;
};

// Partial result of one piece of a split query block: per thread of the
// 512-thread workgroup, 64 fp32 O accumulators (16 float4, stored
// [float4 index][thread]) then the row shifts b and normalisers l of the
// thread's one or two query rows (float4 (b0, l0, b1, l1) per thread).
// Two slots per workgroup: the first and the last job of its share.
constexpr int kSplitThreads = 512;
constexpr int64_t kSplitPieceFloats = (int64_t)kSplitThreads * 64 + (int64_t)kSplitThreads * 4;

// Split workspace: one int32 arrival count per tail block, in a region
// sized for the largest setting (2 * kMaxGroups counts, so that the slots
// after it never move whatever a launch's groups), then two partial slots
// per workgroup.  256-byte aligned.
constexpr int32_t kMaxGroups = 1 << 14;
constexpr uint64_t kSplitCountBytes = static_cast<uint64_t>(2) * kMaxGroups * sizeof(int32_t);
constexpr uint64_t kSplitAlign = 256;
constexpr uint64_t split_workspace_bytes_for(int64_t groups) {
  return kSplitCountBytes + static_cast<uint64_t>(groups) * 2 * kSplitPieceFloats * sizeof(float);
}

hipError_t launch_prologue_bf16(const PrologueArgs &a, const RopeTable &t,
                                hipStream_t s);
hipError_t launch_prologue_fp8(const PrologueArgs &a, const RopeTable &t,
                               hipStream_t s);
// Attention launches: bf16 inputs on the bf16 matrix cores, E4M3 inputs on
// the fp8 matrix cores (E4M3 Q, K, V and P).  fused: the Q load applies
// RMSNorm + RoPE to raw queries.  strided: q, k, v, o follow the strides in
// the arguments (else contiguous [B, H, N, D]).
hipError_t launch_forward_bf16(const ForwardArgs &a, bool fused, bool strided, hipStream_t s);
hipError_t launch_forward_fp8(const ForwardArgs &a, bool fused, bool strided, hipStream_t s);

// Query blocks (one workgroup each without a split) for B*H heads of N
// tokens, and key tiles per head.
int64_t forward_grid_blocks(int64_t BH, int64_t N);
int64_t forward_key_tiles(int64_t N);

// Keeps e for fluxattn_last_hip_error() on this thread; returns
// FLUXATTN_ERR_HIP.
fluxattn_status record_hip_error(hipError_t e);

// Every check of fluxattn_forward_fused_ex_bf16 with a split of `groups`
// workgroups except the workspace's, enqueueing nothing; on success
// *need_bytes is the split workspace the launch needs (0 when it is not
// cut).
fluxattn_status check_forward_fused_ex_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                            fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
                                            void *o, fluxattn_layout o_layout, const float *q_norm_w,
                                            const fluxattn_streams &streams, const int32_t *pos_ids, int64_t B,
                                            int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                            int32_t axes_w, float theta, float eps, float softmax_scale,
                                            int32_t groups, uint64_t *need_bytes);

}  // namespace fluxattn

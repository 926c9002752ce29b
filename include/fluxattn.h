/*
 * fluxattn — joint-attention block of FLUX-style MM-DiT image generators on
 * AMD Instinct MI355X (gfx950).
 *
 * The block, as NVIDIA's blog post "Speed up image generation with FLUX 3
 * Image Klein on NVIDIA Blackwell GPUs" describes it:
 *   - section "Running FLUX 3 inference with TensorRT LLM VisualGen": the text,
 *     noisy-target-image and optional reference-image token streams are
 *     processed separately and merged by one joint attention over all tokens;
 *   - section "GEMM kernel optimization": query/key normalisation and rotary
 *     position embedding (RoPE) follow the QKV projection;
 *   - section "Quantized and sparse attention": dense BF16 attention is the
 *     dominant kernel at 2048x2048, and FP8 queries/keys and values are a
 *     supported attention precision.
 * The pages give no formulas.  This library uses the plain readings:
 *   RMSNorm   y_d = x_d * w_d / sqrt(mean_d(x^2) + eps), one fp32 weight
 *             vector for Q and one for K, shared over batch and heads; the
 *             _ex entry points take one vector per token stream;
 *   RoPE      head dims split into contiguous (t, h, w) blocks of
 *             (axes_t, axes_h, axes_w); inside axis a's block the adjacent
 *             pair (y[2j], y[2j+1]) = (u, v) is rotated to
 *             (u cos phi - v sin phi, u sin phi + v cos phi),
 *             phi = pos_a * theta^(-2j/axes_a); V is not rotated;
 *   attention O = softmax(Q' K'^T * softmax_scale) V, non-causal, no mask.
 *
 * Conventions shared by every entry point
 *   Layout     row-major contiguous [B, H, N, D]; element (b,h,n,d) sits at
 *              ((b*H + h)*N + n)*D + d.  The _ex entry points take strided
 *              views instead (fluxattn_layout below).  pos_ids is int32
 *              [N, 3] = (t, h, w) per token, shared by all B and H.  Scales
 *              are fp32 [B, H], contiguous.
 *   Pointers   all data pointers are DEVICE pointers on the current HIP device.
 *              The caller owns every buffer, including the optional split
 *              workspace of the _ex attention forms.  The library keeps no
 *              per-call or process-wide setting, allocates nothing, frees
 *              nothing and never synchronises; work is enqueued on `stream`
 *              (a hipStream_t; NULL = null stream) and the call returns at
 *              once, so every call may be captured into a HIP graph.
 *   Shapes     D == 128; B, H, N >= 1; N <= FLUXATTN_MAX_N; axes even and
 *              summing to D; theta > 0; eps >= 0.
 *   Alignment  q/k/v/o and prologue outputs 16 bytes; pos_ids, weights and
 *              scales 4 bytes.
 *   Errors     validation order: null pointers, shape, alignment, aliasing,
 *              device (must be gfx950), then the split workspace (its plan
 *              depends on the device).  Any failure returns before anything
 *              is enqueued and leaves every output untouched.  A failed
 *              launch returns FLUXATTN_ERR_HIP (fluxattn_last_hip_error()
 *              gives the hipError_t).  Faults inside a kernel surface at the
 *              caller's next synchronisation, as with any HIP work.
 *   Numerics   inputs are not checked for NaN/Inf; a NaN spreads to the rows
 *              it touches.  Results are bitwise reproducible run to run.
 *              Launches without a split use no atomics; a split launch
 *              counts the pieces of each cut query block with one
 *              device-scope atomic counter and merges them in a fixed
 *              order, whichever piece arrives last (fluxattn_split).
 *   Threads    every entry point is re-entrant and thread-safe; calls that
 *              share a split workspace must not run at the same time.
 */
#ifndef FLUXATTN_H
#define FLUXATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLUXATTN_HEAD_DIM 128
#define FLUXATTN_MAX_N (1 << 22)

/*
 * A strided [B, H, N, D] view: element (b,h,n,d) sits at
 * b*b_stride + h*h_stride + n*n_stride + d elements past the view's pointer
 * (d is always contiguous).  Contiguous [B,H,N,D] is {H*N*D, N*D, D}; the
 * [B,N,H,D] layout a QKV projection writes is {N*H*D, D, H*D}; one of q, k,
 * v inside a packed [B,N,3,H,D] tensor is {3*N*H*D, D, 3*H*D} from that
 * tensor's pointer plus 0, H*D or 2*H*D elements.
 * Rules: strides >= 0 and, in bytes, multiples of 16; n_stride >= D (token
 * rows do not overlap) and at most 2^30 bytes; within one (b,h), row
 * ceil(N/256)*256 - 1 ends less than 2^32 bytes past row 0.  Outputs must
 * be one-to-one (no two (b,h,n,d) share an element).  Views whose
 * bounding ranges overlap are still disjoint when they share all three
 * strides, b_stride is a multiple of n_stride and they sit in separate
 * slices of each token row (as the q, k, v slices of a packed tensor do).
 */
typedef struct {
    int64_t b_stride, h_stride, n_stride;
} fluxattn_layout;

/*
 * Token streams for per-stream RMSNorm weights: the sequence is the
 * concatenation of `count` (1..4) streams, stream s holding tokens
 * [start[s], start[s+1]) (the last runs to N); weight row s applies to
 * them.  start[0] == 0, starts non-decreasing and <= N (an empty stream is
 * allowed); entries past count are ignored.  FLUX: text then image (then
 * reference image) tokens, each stream with its own norm weights (blog post
 * above, section "Running FLUX 3 inference with TensorRT LLM VisualGen").
 */
typedef struct {
    int32_t count;
    int32_t start[4];
} fluxattn_streams;

/*
 * Key-range split of one attention launch (an execution choice: the function
 * computed is the one each entry point describes).  A launch normally runs
 * at most one persistent workgroup per compute unit, each computing whole
 * 256-query blocks of each (b,h) in turn, in rounds of one block per
 * compute unit, and its last round can leave compute units idle.  A split
 * launch instead runs G persistent workgroups: all but the
 * last one or two rounds of blocks go whole, in launch order, and the
 * remaining blocks' (query block, 64-key tile) pairs, in (b, h, query
 * block, key tile) order, are dealt out as G equal contiguous shares.  A
 * block whose keys fall in several shares is computed in pieces; each piece
 * leaves its fp32 partial O, row shift and normaliser in the workspace, and
 * the piece that arrives last merges them in share order and stores O.
 * Results differ from the uncut launch by the P roundings (each piece's P
 * is relative to its own running shift) and fp32 summation order, and are
 * deterministic.
 *   groups     0: G = the device's compute units; the launch is cut with
 *                 at least two rounds of blocks when whole blocks would
 *                 leave more than 3% of the last round idle, and between
 *                 one and two rounds when the second round would be less
 *                 than 7/12 full (one whole round, then the rest cut);
 *              > 0 (at most 16384): G = groups, at most one per key tile of
 *                 the cut blocks; always cut (with more workgroups than
 *                 blocks, blocks are cut into several pieces);
 *              < 0: never cut (the same as passing no fluxattn_split).
 *   workspace  device memory of the caller, 256-byte aligned, at least
 *              fluxattn_split_workspace_bytes() long for the launch, apart
 *              from every other buffer of the call, and all zero before
 *              its first use (for example one hipMemset after allocation).
 *              A launch leaves the arrival counts at its start zero again,
 *              so a workspace serves any number of launches, with any
 *              groups, as long as they do not overlap in time (one stream,
 *              or ordered by events).  NULL is fine for a launch that is
 *              not cut (fluxattn_split_workspace_bytes() == 0).
 *   workspace_bytes  its size.
 * A missing, short, misaligned or overlapping workspace for a launch that
 * is cut returns FLUXATTN_ERR_WORKSPACE.
 */
typedef struct {
    int32_t groups;
    void *workspace;
    uint64_t workspace_bytes;
} fluxattn_split;

typedef enum {
    FLUXATTN_OK = 0,
    FLUXATTN_ERR_NULL_POINTER = 1,  /* a required pointer is NULL            */
    FLUXATTN_ERR_INVALID_SHAPE = 2, /* B/H/N/D/axes/theta/eps out of range   */
    FLUXATTN_ERR_MISALIGNED = 3,    /* a pointer breaks the alignment rule   */
    FLUXATTN_ERR_ALIASING = 4,      /* an output overlaps a buffer it may not */
    FLUXATTN_ERR_NO_DEVICE = 5,     /* no HIP device, or it is not gfx950    */
    FLUXATTN_ERR_HIP = 6,           /* a HIP call (launch) failed            */
    FLUXATTN_ERR_WORKSPACE = 7      /* split workspace missing, too small,
                                       misaligned or overlapping a buffer  */
} fluxattn_status;

/*
 * Fused per-head RMSNorm + 3-axis RoPE on queries and keys, bf16.
 * (blog post above, section "GEMM kernel optimization".)
 *   q, k          bf16 [B,H,N,D] inputs.
 *   q_out, k_out  bf16 [B,H,N,D] outputs, round-to-nearest-even.  q_out may
 *                 equal q and k_out may equal k (in place); any other
 *                 overlap between an output and another buffer is
 *                 FLUXATTN_ERR_ALIASING.
 *   q_norm_w, k_norm_w  fp32 [D] RMSNorm weights.
 *   pos_ids       int32 [N,3] (t,h,w) token positions.
 *   axes_*, theta RoPE axis split and base (FLUX: 16, 56, 56 and 1e4).
 *   eps           RMSNorm epsilon (FLUX: 1e-6), inside the square root.
 * Keys only: q, q_out and q_norm_w all NULL processes k alone (the form
 * the fused attention entry points below pair with); a NULL among them
 * otherwise is FLUXATTN_ERR_NULL_POINTER.
 * Rotation angles are evaluated in fp32 in revolutions, id times the
 * frequency divided by 2 pi (computed in fp64 on the host, rounded to
 * fp32), reduced to one turn and passed to the hardware sine and cosine
 * (absolute error about 1e-6 rad plus 6e-8 of the angle), the same
 * rotation the fused attention entry points apply to the queries; sums of
 * squares are fp32.
 */
fluxattn_status fluxattn_qk_norm_rope_bf16(
    const void *q, const void *k, void *q_out, void *k_out,
    const float *q_norm_w, const float *k_norm_w, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    void *stream);

/*
 * The same prologue on OCP FP8 E4M3 (e4m3fn: bias 7, max 448, no Inf)
 * inputs with per-(b,h) dequantisation scales: x = e4m3(code) * scale[b,h].
 * (blog post above, sections "GEMM kernel optimization" and "Quantized and
 * sparse attention".)
 *   q, k                    uint8 E4M3 codes [B,H,N,D].
 *   q_scale, k_scale        fp32 [B,H] input scales.
 *   q_out, k_out            uint8 E4M3 codes [B,H,N,D]; may equal q / k.
 *   q_scale_out, k_scale_out fp32 [B,H], written by the kernel with
 *                 sqrt(D) * max|w| / 448 for the matching weight vector.
 *                 Every prologue output is bounded by sqrt(D) * max|w| in
 *                 magnitude, so the encode never saturates.
 * Other arguments as in fluxattn_qk_norm_rope_bf16; keys only when q,
 * q_scale, q_out, q_scale_out and q_norm_w are all NULL.
 */
fluxattn_status fluxattn_qk_norm_rope_fp8(
    const uint8_t *q, const uint8_t *k, const float *q_scale,
    const float *k_scale, uint8_t *q_out, uint8_t *k_out, float *q_scale_out,
    float *k_scale_out, const float *q_norm_w, const float *k_norm_w,
    const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    void *stream);

/*
 * Non-causal joint attention O = softmax(Q K^T * softmax_scale) V over all N
 * tokens of each (b,h), bf16 in and out.  (blog post above, sections
 * "Running FLUX 3 inference with TensorRT LLM VisualGen" and "Quantized and
 * sparse attention".)
 *   q, k, v   bf16 [B,H,N,D] (q and k normally come out of the prologue).
 *   o         bf16 [B,H,N,D] output; must not overlap q, k or v.
 *   softmax_scale  <= 0 selects 1/sqrt(D).
 * Scores and the softmax run in fp32 (exponentials in base 2 with the scale
 * folded in); the normaliser sums the fp32 probabilities, which are then
 * rounded to bf16 for the P.V product; O is accumulated in fp32, divided by
 * the normaliser and rounded once to bf16.  The N x N score matrix is never
 * stored.  Deterministic: the same inputs give bitwise the same output.
 */
fluxattn_status fluxattn_forward_bf16(
    const void *q, const void *k, const void *v, void *o,
    int64_t B, int64_t H, int64_t N, int64_t D, float softmax_scale,
    void *stream);

/*
 * Joint attention on E4M3 queries, keys and values with per-(b,h) scales:
 * Q = e4m3(q)*q_scale[b,h], and likewise K and V.  Output o is bf16
 * [B,H,N,D] and must not overlap q, k or v.  (blog post above, section
 * "Quantized and sparse attention": FP8 for both the QK and the V operands.)
 * Q K^T and P.V run on the fp8 matrix cores with fp32 accumulation; P is
 * encoded as E4M3 of 2^6 p relative to a running shift of each row (so every
 * code stays <= 2^8); the normaliser sums those E4M3 values, the ones P.V
 * multiplies; O is divided by it, times v_scale, and rounded once to bf16.
 * Deterministic.
 */
fluxattn_status fluxattn_forward_fp8(
    const uint8_t *q, const uint8_t *k, const uint8_t *v,
    const float *q_scale, const float *k_scale, const float *v_scale,
    void *o, int64_t B, int64_t H, int64_t N, int64_t D, float softmax_scale,
    void *stream);

/*
 * Attention on raw (pre-norm) queries: the kernel's query load applies the
 * queries' RMSNorm + RoPE in registers, so Q' never goes to memory; k must
 * already hold K' (e.g. from the keys-only prologue above).  (blog post
 * above, section "GEMM kernel optimization": the pages fuse this step into
 * the QKV projection's epilogue; here it is fused into its consumer.)
 *   q         bf16 [B,H,N,D] raw queries.
 *   k, v      bf16 [B,H,N,D] prepared keys, values.
 *   o         bf16 [B,H,N,D] output; must not overlap any input.
 *   q_norm_w  fp32 [D] query RMSNorm weights, 16-byte aligned.
 *   pos_ids, axes_*, theta, eps  as in fluxattn_qk_norm_rope_bf16.
 *   softmax_scale  as in fluxattn_forward_bf16.
 * Q' is computed in fp32, multiplied by c = softmax scale * log2 e and
 * rounded to bf16 once (the prologue rounds Q' itself once), so the QK^T
 * product yields base-2 logits directly.  The rotation rates are the
 * prologue's frequencies theta^(-2j/axes_a) computed on the host and
 * expressed in revolutions (divided by 2 pi, rounded to fp32); each angle
 * pos * rate is reduced to one revolution and goes through the hardware
 * sine / cosine (absolute error about 1e-6 + 1.2e-7 |angle| rad, the fp32
 * rounding of the rate and of the product).  Numerics
 * otherwise as fluxattn_forward_bf16.
 */
fluxattn_status fluxattn_forward_fused_bf16(
    const void *q, const void *k, const void *v, void *o,
    const float *q_norm_w, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, void *stream);

/*
 * fp8 form: E4M3 q (raw), k (prepared), v with fp32 [B,H] scales; the
 * queries are dequantised, normalised and rotated in fp32, then re-encoded
 * in E4M3 per query: codes of Q' * g / 2^e with g = softmax scale * log2 e *
 * k_scale and e the smallest integer keeping every code within 448; the
 * QK^T product applies 2^e as its block scale.  Numerics otherwise as
 * fluxattn_forward_fp8.  Output bf16.
 */
fluxattn_status fluxattn_forward_fused_fp8(
    const uint8_t *q, const uint8_t *k, const uint8_t *v,
    const float *q_scale, const float *k_scale, const float *v_scale,
    void *o, const float *q_norm_w, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, void *stream);

/*
 * The whole block in two launches: the keys-only prologue into k_work,
 * then fluxattn_forward_fused_bf16 on the raw queries.
 *   q, k, v    bf16 [B,H,N,D]: raw (pre-norm) queries and keys, values.
 *   k_work     bf16 [B,H,N,D], receives K'; may equal k (in place), must
 *              not overlap any other buffer.
 *   o          bf16 [B,H,N,D] output; must not overlap any other buffer.
 *   q_norm_w   fp32 [D], 16-byte aligned; k_norm_w fp32 [D].
 *   Other arguments as in fluxattn_qk_norm_rope_bf16 and
 *   fluxattn_forward_bf16.  Results match those two calls up to fp32
 *   summation order and the query rotation, computed as in
 *   fluxattn_forward_fused_bf16.
 */
fluxattn_status fluxattn_joint_attention_bf16(
    const void *q, const void *k, const void *v, void *k_work, void *o,
    const float *q_norm_w, const float *k_norm_w, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, void *stream);

/*
 * fp8 form of fluxattn_joint_attention_bf16: E4M3 q, k, v with fp32 [B,H]
 * scales.  The fp8 key prologue writes k_work (E4M3) and k_scale_work
 * (fp32 [B,H], must not overlap k_scale); the queries are dequantised,
 * normalised and rotated in the attention kernel and re-encoded in E4M3 per
 * query, as in fluxattn_forward_fused_fp8.  Output bf16.
 */
fluxattn_status fluxattn_joint_attention_fp8(
    const uint8_t *q, const uint8_t *k, const uint8_t *v,
    const float *q_scale, const float *k_scale, const float *v_scale,
    uint8_t *k_work, float *k_scale_work, void *o,
    const float *q_norm_w, const float *k_norm_w, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, void *stream);

/*
 * Strided, multi-stream forms.  Each takes a fluxattn_layout after every
 * [B,H,N,D] tensor (rules above) and, where norm weights appear, a
 * fluxattn_streams with q_norm_w / k_norm_w as fp32 [streams.count, D]
 * (one row per stream).  The attention forms (forward, forward_fused,
 * joint_attention) also take an optional key-range split (fluxattn_split
 * above; NULL = uncut).  Everything else, including aliasing (in place
 * means the same pointer and the same layout), is as in the contiguous
 * entry point of the same name, which equals its _ex form with contiguous
 * layouts, one stream and no split.  Invalid layouts, streams or split
 * groups give FLUXATTN_ERR_INVALID_SHAPE.  For the fp8 prologue, q_scale_out /
 * k_scale_out are sqrt(D) * max|w| / 448 with the maximum over all
 * streams' rows.  k_work of the joint forms is contiguous [B,H,N,D] and
 * may equal k only when k is contiguous too.
 */
fluxattn_status fluxattn_qk_norm_rope_ex_bf16(
    const void *q, fluxattn_layout q_layout, const void *k,
    fluxattn_layout k_layout, void *q_out, fluxattn_layout q_out_layout,
    void *k_out, fluxattn_layout k_out_layout, const float *q_norm_w,
    const float *k_norm_w, fluxattn_streams streams, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    void *stream);

fluxattn_status fluxattn_qk_norm_rope_ex_fp8(
    const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
    fluxattn_layout k_layout, const float *q_scale, const float *k_scale,
    uint8_t *q_out, fluxattn_layout q_out_layout, uint8_t *k_out,
    fluxattn_layout k_out_layout, float *q_scale_out, float *k_scale_out,
    const float *q_norm_w, const float *k_norm_w, fluxattn_streams streams,
    const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    void *stream);

fluxattn_status fluxattn_forward_ex_bf16(
    const void *q, fluxattn_layout q_layout, const void *k,
    fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
    void *o, fluxattn_layout o_layout, int64_t B, int64_t H, int64_t N,
    int64_t D, float softmax_scale, const fluxattn_split *split, void *stream);

fluxattn_status fluxattn_forward_ex_fp8(
    const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
    fluxattn_layout k_layout, const uint8_t *v, fluxattn_layout v_layout,
    const float *q_scale, const float *k_scale, const float *v_scale,
    void *o, fluxattn_layout o_layout, int64_t B, int64_t H, int64_t N,
    int64_t D, float softmax_scale, const fluxattn_split *split, void *stream);

/*
 * Attention on raw queries (fluxattn_forward_fused_bf16 / _fp8) over
 * strided views, with per-stream query norm weights and an optional split.
 */
fluxattn_status fluxattn_forward_fused_ex_bf16(
    const void *q, fluxattn_layout q_layout, const void *k,
    fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
    void *o, fluxattn_layout o_layout, const float *q_norm_w,
    fluxattn_streams streams, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, const fluxattn_split *split, void *stream);

fluxattn_status fluxattn_forward_fused_ex_fp8(
    const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
    fluxattn_layout k_layout, const uint8_t *v, fluxattn_layout v_layout,
    const float *q_scale, const float *k_scale, const float *v_scale,
    void *o, fluxattn_layout o_layout, const float *q_norm_w,
    fluxattn_streams streams, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, const fluxattn_split *split, void *stream);

fluxattn_status fluxattn_joint_attention_ex_bf16(
    const void *q, fluxattn_layout q_layout, const void *k,
    fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
    void *k_work, void *o, fluxattn_layout o_layout, const float *q_norm_w,
    const float *k_norm_w, fluxattn_streams streams, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, const fluxattn_split *split, void *stream);

fluxattn_status fluxattn_joint_attention_ex_fp8(
    const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
    fluxattn_layout k_layout, const uint8_t *v, fluxattn_layout v_layout,
    const float *q_scale, const float *k_scale, const float *v_scale,
    uint8_t *k_work, float *k_scale_work, void *o, fluxattn_layout o_layout,
    const float *q_norm_w, const float *k_norm_w, fluxattn_streams streams,
    const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, const fluxattn_split *split, void *stream);

/*
 * Bytes of split workspace (fluxattn_split above) that an attention launch
 * over B*H heads of N tokens needs with this groups setting: 0 when the
 * launch would not be cut.  Host-only: enqueues nothing.  groups == 0
 * depends on the current device's compute units and returns
 * FLUXATTN_ERR_NO_DEVICE without a gfx950 device.  A launch with
 * groups > 0 needs 128 KiB plus about 264 KiB per workgroup.
 */
fluxattn_status fluxattn_split_workspace_bytes(
    int64_t B, int64_t H, int64_t N, int64_t D, int32_t groups,
    uint64_t *bytes);

/*
 * fluxattn_forward_fused_ex_bf16 with a split of `groups` workgroups
 * (fluxattn_split.groups) whose workspace is a static array of the library
 * instead of caller memory: for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid it).
 *   Limit: a split of at most 256 workgroups (68.1 MiB, one per compute unit
 *          of an MI355X, the default setting's launch there); a launch
 *          whose split would need more returns FLUXATTN_ERR_WORKSPACE
 *          before anything is enqueued.  Launches that are not cut use no
 *          scratch.
 *   Memory: each device this entry point runs on holds its own copy of the
 *          array until the process ends; the first call on a device looks
 *          it up and clears its arrival counts on `stream` (a caller that
 *          captures graphs makes that first call before capturing).
 *   Threads: every call on one device shares that device's array, which
 *          keeps the last call's partial results; calls that overlap in
 *          time on one device race (one stream, or order them by events).
 * Arguments, checks, numerics and errors are those of
 * fluxattn_forward_fused_ex_bf16 (validation runs before anything is
 * enqueued); results are bitwise those of that entry point with the same
 * groups.
 */
fluxattn_status fluxattn_forward_fused_noalloc_bf16(
    const void *q, fluxattn_layout q_layout, const void *k,
    fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
    void *o, fluxattn_layout o_layout, const float *q_norm_w,
    fluxattn_streams streams, const int32_t *pos_ids,
    int64_t B, int64_t H, int64_t N, int64_t D,
    int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta, float eps,
    float softmax_scale, int32_t groups, void *stream);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char *fluxattn_status_string(fluxattn_status s);

/* hipError_t of this thread's most recent FLUXATTN_ERR_HIP (0 if none). */
int fluxattn_last_hip_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int fluxattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLUXATTN_H */

// C ABI of libfluxattn: argument validation, device check and launches.
// Every check runs on the host before anything is enqueued, so a rejected
// call leaves all outputs untouched and needs no GPU work to report.
#include <math.h>
#include <string.h>

#include <atomic>

#include "fluxattn.h"
#include "fluxattn_internal.h"

using namespace fluxattn;

namespace {

thread_local int g_last_hip_error = 0;

fluxattn_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return FLUXATTN_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range span(const void *p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// An output must either coincide exactly with its own input (in place) or
// overlap nothing else.
bool output_ok(Range out, Range own_in, const Range *others, int n_others) {
  if (overlap(out, own_in) && !(out.lo == own_in.lo && out.hi == own_in.hi)) return false;
  for (int i = 0; i < n_others; ++i)
    if (overlap(out, others[i])) return false;
  return true;
}

bool shape_ok(int64_t B, int64_t H, int64_t N, int64_t D) {
  if (B < 1 || H < 1 || N < 1 || D != kHeadDim) return false;
  if (N > FLUXATTN_MAX_N) return false;
  if (B > (int64_t(1) << 20) || H > (int64_t(1) << 20)) return false;
  const int64_t BH = B * H;
  if (BH > (int64_t(1) << 30)) return false;
  // element count must stay well inside int64, workgroup counts inside int32
  if (BH > (int64_t(1) << 62) / (N * D)) return false;
  if (forward_grid_blocks(BH, N) > 0x7fffffffLL) return false;
  return true;
}

bool rope_ok(int32_t at, int32_t ah, int32_t aw, float theta, float eps) {
  if (at < 0 || ah < 0 || aw < 0) return false;
  if ((at | ah | aw) & 1) return false;
  if (at + ah + aw != kHeadDim) return false;
  if (!(theta > 0.f) || !isfinite(theta)) return false;
  if (!(eps >= 0.f) || !isfinite(eps)) return false;
  return true;
}

// gfx950 check, cached per device (arch never changes for a device id).
fluxattn_status device_ok() {
  static std::atomic<int> cache[64];  // 0 unknown, 1 ok, 2 wrong arch
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FLUXATTN_ERR_NO_DEVICE;
  }
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return FLUXATTN_OK;
    if (c == 2) return FLUXATTN_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return FLUXATTN_ERR_NO_DEVICE;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FLUXATTN_OK : FLUXATTN_ERR_NO_DEVICE;
}

RopeTable make_rope_table(int32_t at, int32_t ah, int32_t aw, float theta) {
  RopeTable t;
  const int32_t dims[3] = {at, ah, aw};
  int pair = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < dims[a] / 2; ++j, ++pair) {
      t.freq[pair] = static_cast<float>(pow(static_cast<double>(theta), -2.0 * j / dims[a]));
      t.axis[pair] = static_cast<int8_t>(a);
    }
  return t;
}

template <bool FP8>
fluxattn_status prologue_impl(const void *q, const void *k, const float *q_scale, const float *k_scale,
                              void *q_out, void *k_out, float *q_scale_out, float *k_scale_out,
                              const float *q_norm_w, const float *k_norm_w, const int32_t *pos_ids,
                              int64_t B, int64_t H, int64_t N, int64_t D, int32_t at, int32_t ah,
                              int32_t aw, float theta, float eps, void *stream) {
  // q == NULL: keys only (q_out, q_norm_w and the fp8 q scales must then be NULL too)
  const bool has_q = q != nullptr;
  if (!has_q && (q_out || q_norm_w || (FP8 && (q_scale || q_scale_out)))) return FLUXATTN_ERR_NULL_POINTER;
  if (!k || !k_out || !k_norm_w || !pos_ids) return FLUXATTN_ERR_NULL_POINTER;
  if (has_q && (!q_out || !q_norm_w)) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!k_scale || !k_scale_out)) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && has_q && (!q_scale || !q_scale_out)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || !rope_ok(at, ah, aw, theta, eps)) return FLUXATTN_ERR_INVALID_SHAPE;
  // (aligned() of a NULL pointer holds)
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) ||
      !aligned(q_norm_w, 4) || !aligned(k_norm_w, 4) || !aligned(pos_ids, 4))
    return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(q_scale_out, 4) ||
              !aligned(k_scale_out, 4)))
    return FLUXATTN_ERR_MISALIGNED;

  const int64_t BH = B * H;
  const int64_t tensor_bytes = BH * N * D * (FP8 ? 1 : 2);
  const Range none = {0, 0};
  auto sp = [](const void *p, int64_t bytes) { return p ? span(p, bytes) : Range{0, 0}; };
  const Range rq = sp(q, tensor_bytes), rk = span(k, tensor_bytes);
  const Range rqo = sp(q_out, tensor_bytes), rko = span(k_out, tensor_bytes);
  const Range rwq = sp(q_norm_w, D * 4), rwk = span(k_norm_w, D * 4), rp = span(pos_ids, N * 12);
  Range rsq = none, rsk = none, rsqo = none, rsko = none;
  if (FP8) {
    rsq = sp(q_scale, BH * 4);
    rsk = span(k_scale, BH * 4);
    rsqo = sp(q_scale_out, BH * 4);
    rsko = span(k_scale_out, BH * 4);
  }
  {
    const Range oq[] = {rk, rko, rwq, rwk, rp, rsq, rsk, rsqo, rsko};
    const Range ok[] = {rq, rqo, rwq, rwk, rp, rsq, rsk, rsqo, rsko};
    if ((has_q && !output_ok(rqo, rq, oq, FP8 ? 9 : 5)) || !output_ok(rko, rk, ok, FP8 ? 9 : 5))
      return FLUXATTN_ERR_ALIASING;
    if (FP8) {
      const Range os[] = {rq, rk, rqo, rko, rwq, rwk, rp, rsq, rsk, rsko};
      const Range ok2[] = {rq, rk, rqo, rko, rwq, rwk, rp, rsq, rsk, rsqo};
      if ((has_q && !output_ok(rsqo, none, os, 10)) || !output_ok(rsko, none, ok2, 10))
        return FLUXATTN_ERR_ALIASING;
    }
  }
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;

  PrologueArgs a{};
  a.q = q;
  a.k = k;
  a.q_out = q_out;
  a.k_out = k_out;
  a.w_q = q_norm_w;
  a.w_k = k_norm_w;
  a.pos = pos_ids;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.q_scale_out = q_scale_out;
  a.k_scale_out = k_scale_out;
  a.BH = BH;
  a.N = static_cast<int32_t>(N);
  a.eps = eps;
  const RopeTable t = make_rope_table(at, ah, aw, theta);
  const hipError_t e = FP8 ? launch_prologue_fp8(a, t, static_cast<hipStream_t>(stream))
                           : launch_prologue_bf16(a, t, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLUXATTN_OK : hip_fail(e);
}

template <bool FP8>
fluxattn_status forward_impl(const void *q, const void *k, const void *v, const float *q_scale,
                             const float *k_scale, const float *v_scale, void *o, int64_t B, int64_t H,
                             int64_t N, int64_t D, float softmax_scale, void *stream) {
  if (!q || !k || !v || !o) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!q_scale || !k_scale || !v_scale)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D)) return FLUXATTN_ERR_INVALID_SHAPE;
  if (!(softmax_scale <= 0.f) && !(softmax_scale > 0.f && isfinite(softmax_scale)))
    return FLUXATTN_ERR_INVALID_SHAPE;  // NaN or +inf
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return FLUXATTN_ERR_MISALIGNED;
  const int64_t BH = B * H;
  const int64_t in_bytes = BH * N * D * (FP8 ? 1 : 2);
  const Range ro = span(o, BH * N * D * 2);
  const Range none = {0, 0};
  Range others[6] = {span(q, in_bytes), span(k, in_bytes), span(v, in_bytes), none, none, none};
  if (FP8) {
    others[3] = span(q_scale, BH * 4);
    others[4] = span(k_scale, BH * 4);
    others[5] = span(v_scale, BH * 4);
  }
  if (!output_ok(ro, none, others, FP8 ? 6 : 3)) return FLUXATTN_ERR_ALIASING;
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;

  const double scale = softmax_scale > 0.f ? static_cast<double>(softmax_scale) : 1.0 / sqrt(static_cast<double>(D));
  ForwardArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.BH = static_cast<int32_t>(BH);
  a.N = static_cast<int32_t>(N);
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);  // * log2(e)
  const hipError_t e = FP8 ? launch_forward_fp8(a, static_cast<hipStream_t>(stream))
                           : launch_forward_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLUXATTN_OK : hip_fail(e);
}

// Attention whose Q load normalises and rotates raw queries (K already
// prepared).
template <bool FP8>
fluxattn_status fused_impl(const void *q, const void *k, const void *v, const float *q_scale,
                           const float *k_scale, const float *v_scale, void *o, const float *q_norm_w,
                           const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D, int32_t at,
                           int32_t ah, int32_t aw, float theta, float eps, float softmax_scale, void *stream) {
  if (!q || !k || !v || !o || !q_norm_w || !pos_ids) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!q_scale || !k_scale || !v_scale)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || !rope_ok(at, ah, aw, theta, eps)) return FLUXATTN_ERR_INVALID_SHAPE;
  if (!(softmax_scale <= 0.f) && !(softmax_scale > 0.f && isfinite(softmax_scale)))
    return FLUXATTN_ERR_INVALID_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(q_norm_w, 16) ||
      !aligned(pos_ids, 4))
    return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))) return FLUXATTN_ERR_MISALIGNED;
  const int64_t BH = B * H;
  const int64_t in_bytes = BH * N * D * (FP8 ? 1 : 2);
  const Range none = {0, 0};
  Range others[8] = {span(q, in_bytes), span(k, in_bytes), span(v, in_bytes), span(q_norm_w, D * 4),
                     span(pos_ids, N * 12), none, none, none};
  if (FP8) {
    others[5] = span(q_scale, BH * 4);
    others[6] = span(k_scale, BH * 4);
    others[7] = span(v_scale, BH * 4);
  }
  if (!output_ok(span(o, BH * N * D * 2), none, others, 8)) return FLUXATTN_ERR_ALIASING;
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;

  const double scale = softmax_scale > 0.f ? static_cast<double>(softmax_scale) : 1.0 / sqrt(static_cast<double>(D));
  ForwardArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.BH = static_cast<int32_t>(BH);
  a.N = static_cast<int32_t>(N);
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  a.w_q = q_norm_w;
  a.pos = pos_ids;
  a.eps = eps;
  const int32_t dims[3] = {at, ah, aw};
  a.rope_first[0] = 0;
  for (int i = 0; i < 3; ++i) {
    a.rope_first[i + 1] = a.rope_first[i] + dims[i] / 2;
    a.rope_log2_step[i] = dims[i] > 0 ? static_cast<float>(-2.0 * log2(static_cast<double>(theta)) / dims[i]) : 0.f;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = FP8 ? launch_forward_fused_fp8(a, st) : launch_forward_fused_bf16(a, st);
  return e == hipSuccess ? FLUXATTN_OK : hip_fail(e);
}

// The whole block: keys' prologue into k_work, then the fused attention.
template <bool FP8>
fluxattn_status joint_impl(const void *q, const void *k, const void *v, const float *q_scale,
                           const float *k_scale, const float *v_scale, void *k_work, float *k_scale_work,
                           void *o, const float *q_norm_w, const float *k_norm_w, const int32_t *pos_ids,
                           int64_t B, int64_t H, int64_t N, int64_t D, int32_t at, int32_t ah, int32_t aw,
                           float theta, float eps, float softmax_scale, void *stream) {
  if (!q || !k || !v || !k_work || !o || !q_norm_w || !k_norm_w || !pos_ids) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!q_scale || !k_scale || !v_scale || !k_scale_work)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || !rope_ok(at, ah, aw, theta, eps)) return FLUXATTN_ERR_INVALID_SHAPE;
  if (!(softmax_scale <= 0.f) && !(softmax_scale > 0.f && isfinite(softmax_scale)))
    return FLUXATTN_ERR_INVALID_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_work, 16) || !aligned(o, 16) ||
      !aligned(q_norm_w, 16) || !aligned(k_norm_w, 4) || !aligned(pos_ids, 4))
    return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(k_scale_work, 4)))
    return FLUXATTN_ERR_MISALIGNED;

  const int64_t BH = B * H;
  const int64_t in_bytes = BH * N * D * (FP8 ? 1 : 2);
  const Range none = {0, 0};
  const Range rq = span(q, in_bytes), rk = span(k, in_bytes), rv = span(v, in_bytes);
  const Range rkw = span(k_work, in_bytes), ro = span(o, BH * N * D * 2);
  const Range rwq = span(q_norm_w, D * 4), rwk = span(k_norm_w, D * 4), rp = span(pos_ids, N * 12);
  Range rsq = none, rsk = none, rsv = none, rskw = none;
  if (FP8) {
    rsq = span(q_scale, BH * 4);
    rsk = span(k_scale, BH * 4);
    rsv = span(v_scale, BH * 4);
    rskw = span(k_scale_work, BH * 4);
  }
  {
    // k_work: exactly k (in place) or apart from everything else
    const Range kw_others[] = {rq, rv, ro, rwq, rwk, rp, rsq, rsk, rsv, rskw};
    if (!output_ok(rkw, rk, kw_others, 10)) return FLUXATTN_ERR_ALIASING;
    const Range o_others[] = {rq, rk, rv, rkw, rwq, rwk, rp, rsq, rsk, rsv, rskw};
    if (!output_ok(ro, none, o_others, 11)) return FLUXATTN_ERR_ALIASING;
    if (FP8) {
      const Range s_others[] = {rq, rk, rv, rkw, ro, rwq, rwk, rp, rsq, rsk, rsv};
      if (!output_ok(rskw, none, s_others, 11)) return FLUXATTN_ERR_ALIASING;
    }
  }
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;
  // both calls below re-validate a subset of the above and cannot fail it
  fluxattn_status s = prologue_impl<FP8>(nullptr, k, nullptr, k_scale, nullptr, k_work, nullptr, k_scale_work,
                                         nullptr, k_norm_w, pos_ids, B, H, N, D, at, ah, aw, theta, eps, stream);
  if (s != FLUXATTN_OK) return s;
  return fused_impl<FP8>(q, k_work, v, q_scale, k_scale_work, v_scale, o, q_norm_w, pos_ids, B, H, N, D, at, ah,
                         aw, theta, eps, softmax_scale, stream);
}

}  // namespace

extern "C" {

fluxattn_status fluxattn_qk_norm_rope_bf16(const void *q, const void *k, void *q_out, void *k_out,
                                           const float *q_norm_w, const float *k_norm_w,
                                           const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                           int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                           float theta, float eps, void *stream) {
  return prologue_impl<false>(q, k, nullptr, nullptr, q_out, k_out, nullptr, nullptr, q_norm_w, k_norm_w,
                              pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, stream);
}

fluxattn_status fluxattn_qk_norm_rope_fp8(const uint8_t *q, const uint8_t *k, const float *q_scale,
                                          const float *k_scale, uint8_t *q_out, uint8_t *k_out,
                                          float *q_scale_out, float *k_scale_out, const float *q_norm_w,
                                          const float *k_norm_w, const int32_t *pos_ids, int64_t B,
                                          int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                          int32_t axes_w, float theta, float eps, void *stream) {
  return prologue_impl<true>(q, k, q_scale, k_scale, q_out, k_out, q_scale_out, k_scale_out, q_norm_w,
                             k_norm_w, pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, stream);
}

fluxattn_status fluxattn_forward_bf16(const void *q, const void *k, const void *v, void *o, int64_t B,
                                      int64_t H, int64_t N, int64_t D, float softmax_scale, void *stream) {
  return forward_impl<false>(q, k, v, nullptr, nullptr, nullptr, o, B, H, N, D, softmax_scale, stream);
}

fluxattn_status fluxattn_forward_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                                     const float *q_scale, const float *k_scale, const float *v_scale,
                                     void *o, int64_t B, int64_t H, int64_t N, int64_t D,
                                     float softmax_scale, void *stream) {
  return forward_impl<true>(q, k, v, q_scale, k_scale, v_scale, o, B, H, N, D, softmax_scale, stream);
}

fluxattn_status fluxattn_forward_fused_bf16(const void *q, const void *k, const void *v, void *o,
                                            const float *q_norm_w, const int32_t *pos_ids, int64_t B,
                                            int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                            int32_t axes_w, float theta, float eps, float softmax_scale,
                                            void *stream) {
  return fused_impl<false>(q, k, v, nullptr, nullptr, nullptr, o, q_norm_w, pos_ids, B, H, N, D, axes_t, axes_h,
                           axes_w, theta, eps, softmax_scale, stream);
}

fluxattn_status fluxattn_forward_fused_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                                           const float *q_scale, const float *k_scale, const float *v_scale,
                                           void *o, const float *q_norm_w, const int32_t *pos_ids, int64_t B,
                                           int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                           int32_t axes_w, float theta, float eps, float softmax_scale,
                                           void *stream) {
  return fused_impl<true>(q, k, v, q_scale, k_scale, v_scale, o, q_norm_w, pos_ids, B, H, N, D, axes_t, axes_h,
                          axes_w, theta, eps, softmax_scale, stream);
}

fluxattn_status fluxattn_joint_attention_bf16(const void *q, const void *k, const void *v, void *k_work,
                                              void *o, const float *q_norm_w, const float *k_norm_w,
                                              const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                              int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                              float theta, float eps, float softmax_scale, void *stream) {
  return joint_impl<false>(q, k, v, nullptr, nullptr, nullptr, k_work, nullptr, o, q_norm_w, k_norm_w, pos_ids,
                           B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, stream);
}

fluxattn_status fluxattn_joint_attention_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                                             const float *q_scale, const float *k_scale,
                                             const float *v_scale, uint8_t *k_work, float *k_scale_work,
                                             void *o, const float *q_norm_w, const float *k_norm_w,
                                             const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                             int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                             float theta, float eps, float softmax_scale, void *stream) {
  return joint_impl<true>(q, k, v, q_scale, k_scale, v_scale, k_work, k_scale_work, o, q_norm_w, k_norm_w,
                          pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, stream);
}

const char *fluxattn_status_string(fluxattn_status s) {
  switch (s) {
    case FLUXATTN_OK: return "ok";
    case FLUXATTN_ERR_NULL_POINTER: return "null pointer";
    case FLUXATTN_ERR_INVALID_SHAPE: return "invalid shape or parameter";
    case FLUXATTN_ERR_MISALIGNED: return "misaligned pointer";
    case FLUXATTN_ERR_ALIASING: return "output overlaps another buffer";
    case FLUXATTN_ERR_NO_DEVICE: return "no gfx950 HIP device";
    case FLUXATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int fluxattn_last_hip_error(void) { return g_last_hip_error; }

int fluxattn_version(void) { return 110; }

}  // extern "C"

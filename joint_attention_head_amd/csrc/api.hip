// C ABI of libfluxattn: argument validation, device check and launches.
// Every check runs on the host before anything is enqueued, so a rejected
// call leaves all outputs untouched and needs no GPU work to report.
#include <math.h>
#include <string.h>

#include <algorithm>
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
  if (!p) return {0, 0};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// ---- shapes and parameters

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

bool scale_ok(float softmax_scale) {
  return softmax_scale <= 0.f || (softmax_scale > 0.f && isfinite(softmax_scale));  // rejects NaN, +inf
}

// Norm-weight streams: 1..4 token ranges starting at 0, non-decreasing
// starts within [0, N].
bool streams_ok(const fluxattn_streams &s, int64_t N) {
  if (s.count < 1 || s.count > 4 || s.start[0] != 0) return false;
  for (int i = 1; i < s.count; ++i)
    if (s.start[i] < s.start[i - 1] || s.start[i] > N) return false;
  return true;
}

Streams to_streams(const fluxattn_streams &s) {
  Streams r;
  for (int i = 0; i < 4; ++i) r.start[i] = i < s.count ? s.start[i] : 0x7fffffff;
  return r;
}

// ---- strided [B, H, N, D] views (d contiguous)

struct View {
  const void *p;
  int64_t sb, sh, sn;  // element strides
};

View contiguous(const void *p, int64_t H, int64_t N, int64_t D) { return {p, H * N * D, N * D, D}; }
View view_of(const void *p, const fluxattn_layout &l) { return {p, l.b_stride, l.h_stride, l.n_stride}; }

bool is_contiguous(const View &v, int64_t H, int64_t N, int64_t D) {
  return v.sb == H * N * D && v.sh == N * D && v.sn == D;
}

// Strides are non-negative and keep every row 16-byte aligned; token rows
// do not overlap (rows past N then lie past a head's last row, where the
// attention kernel's bounded loads read zeros and its stores drop) and the
// token stride fits the kernels' 32-bit row pitch.
bool strides_ok(const View &v, int64_t D, int esize) {
  if (v.sb < 0 || v.sh < 0 || v.sn < D) return false;
  if ((v.sb * esize) % 16 || (v.sh * esize) % 16 || (v.sn * esize) % 16) return false;
  return v.sn * esize <= (int64_t(1) << 30);
}

// Elements from a view's first to past its last element.
int64_t extent_elems(const View &v, int64_t B, int64_t H, int64_t N, int64_t D) {
  return (B - 1) * v.sb + (H - 1) * v.sh + (N - 1) * v.sn + D;
}
Range extent(const View &v, int64_t B, int64_t H, int64_t N, int64_t D, int esize) {
  return span(v.p, extent_elems(v, B, H, N, D) * esize);
}

// The attention kernel addresses a head through 32-bit buffer offsets and
// walks query rows in blocks of 256: every row of the last block, padded
// past N, must still have an offset below 2^32 so that no offset wraps back
// into the head.
bool head_fits(const View &v, int64_t N, int64_t D, int esize) {
  const int64_t rows = (N + 255) / 256 * 256;
  return ((rows - 1) * v.sn + D) * esize < (int64_t(1) << 32);
}

// Distinct (b, h, n, d) reach distinct elements (needed for outputs).
bool injective(const View &v, int64_t B, int64_t H, int64_t N, int64_t D) {
  struct Dim {
    int64_t stride, count;
  } dims[3] = {{v.sb, B}, {v.sh, H}, {v.sn, N}};
  std::sort(dims, dims + 3, [](const Dim &a, const Dim &b) { return a.stride < b.stride; });
  int64_t need = D;  // the next dimension must step past everything before it
  for (const Dim &d : dims) {
    if (d.count == 1) continue;
    if (d.stride < need) return false;
    need = d.stride * d.count;
  }
  return true;
}

bool same_view(const View &a, const View &b) {
  return a.p == b.p && a.sb == b.sb && a.sh == b.sh && a.sn == b.sn;
}

// No element in common.  Views whose extents overlap are still disjoint if
// they share strides and interleave inside token rows, like the q, k and v
// views of a packed [B, N, 3, H, D] tensor.
bool disjoint(const View &a, const View &b, int64_t B, int64_t H, int64_t N, int64_t D, int esize) {
  if (!a.p || !b.p) return true;
  if (!overlap(extent(a, B, H, N, D, esize), extent(b, B, H, N, D, esize))) return true;
  if (a.sb != b.sb || a.sh != b.sh || a.sn != b.sn) return false;
  const int64_t diff = static_cast<int64_t>(reinterpret_cast<uintptr_t>(b.p) - reinterpret_cast<uintptr_t>(a.p));
  if (diff % esize) return false;
  const int64_t delta = diff / esize;
  const int64_t foot = (H - 1) * a.sh + D;  // elements of one token row of a view
  if (a.sn < foot) return false;
  if (B > 1 && a.sb % a.sn) return false;
  const int64_t r = ((delta % a.sn) + a.sn) % a.sn;
  return r >= foot && r + foot <= a.sn;
}

// ---- key-range split of the forward launches

int32_t compute_units(int dev) {
  static std::atomic<int32_t> cache[64];
  if (dev >= 0 && dev < 64) {
    const int32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Persistent workgroups of a launch over nb query blocks of key_tiles key
// tiles each (groups == 0: the launch runs uncut), and the rounds of whole
// blocks before the tail.  setting: the caller's groups (0: `cus`
// workgroups, cut only with at least two rounds of blocks and more than 3%
// of the last round idle; > 0: that many, always cut; < 0: never).
struct SplitPlan {
  int64_t groups = 0, whole = 0;
};

SplitPlan split_plan_for(int64_t nb, int64_t key_tiles, int32_t setting, int32_t cus) {
  SplitPlan p;
  if (setting < 0 || nb < 1) return p;
  int64_t groups = setting > 0 ? setting : cus;
  if (groups < 2) return p;
  if (setting == 0) {
    // at most one round: never cut (the per-job start-up and the merges
    // outweigh the idle units: N = 1536 runs 19% (bf16) and 26% (fp8)
    // slower cut)
    if (nb <= groups) return p;
    if (nb < 2 * groups) {
      // one to two rounds: one whole round, then the rest cut, when the
      // second round would be less than 7/12 full (its shares stream keys
      // out of step, and a part-empty round runs at a higher clock; at
      // N = 4608 cutting measured +18% at 27% full, +2.5% at 55%, -1.2% at
      // 62% and -2.6% at 69%)
      if ((nb - groups) * 12 >= groups * 7) return p;
    } else {
      // whole rounds, then a tail: cut when whole blocks would leave more
      // than 3% of the last round idle
      const int64_t rounds = (nb + groups - 1) / groups;
      if (nb * 100 >= rounds * groups * 97) return p;
    }
  }
  // all but the last one or two rounds whole (the default setting keeps
  // one whole round between one and two rounds); every share holds at
  // least one pair of the tail (the merge reads a slot of every share
  // between a block's first and last)
  const int64_t whole = nb >= 2 * groups ? nb / groups - 1 : (setting == 0 ? 1 : 0);
  const int64_t tail = nb - whole * groups;
  groups = std::min<int64_t>(groups, tail * key_tiles);
  if (groups < 2 || (setting == 0 && nb == groups)) return p;
  p.groups = groups;
  p.whole = whole;
  return p;
}

// Split workspace layout: one arrival count per tail block (fewer than
// 2 * groups of them), then two partial slots per workgroup.  The count
// region has the size for the largest setting whatever the launch's groups,
// so that the slots never move: launches with different group counts may
// share a workspace, and a slot written by one must not land on counts
// another expects at zero.
uint64_t split_bytes(int64_t groups) { return groups > 0 ? split_workspace_bytes_for(groups) : 0; }

// The split setting of a call: NULL means never cut.
int32_t split_setting(const fluxattn_split *sp) { return sp ? sp->groups : -1; }

bool split_setting_ok(const fluxattn_split *sp) { return !sp || sp->groups <= kMaxGroups; }

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

// Axis and frequency theta^(-2j/axes_a), in revolutions, of every pair.
RopeTable make_rope_table(int32_t at, int32_t ah, int32_t aw, float theta) {
  RopeTable t;
  const int32_t dims[3] = {at, ah, aw};
  int pair = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < dims[a] / 2; ++j, ++pair) {
      t.freq[pair] = static_cast<float>(pow(static_cast<double>(theta), -2.0 * j / dims[a]) / 6.283185307179586);
      t.axis[pair] = static_cast<int8_t>(a);
    }
  return t;
}

// A buffer that is not a [B,H,N,D] view (weights, ids, scales), as a view
// whose single row spans it: disjoint() then compares extents only.
struct Plain {
  const void *p;
  int64_t bytes;
};

bool apart(const View &v, int64_t B, int64_t H, int64_t N, int64_t D, int esize, const Plain *plains, int n) {
  const Range r = extent(v, B, H, N, D, esize);
  for (int i = 0; i < n; ++i)
    if (overlap(r, span(plains[i].p, plains[i].bytes))) return false;
  return true;
}

// ---- the prologue: RMSNorm + RoPE of q and k views (q may be absent)

template <bool FP8>
fluxattn_status prologue_core(View q, View k, const float *q_scale, const float *k_scale, View qo, View ko,
                              float *q_scale_out, float *k_scale_out, const float *q_norm_w,
                              const float *k_norm_w, const fluxattn_streams &streams, const int32_t *pos_ids,
                              int64_t B, int64_t H, int64_t N, int64_t D, int32_t at, int32_t ah, int32_t aw,
                              float theta, float eps, void *stream) {
  constexpr int E = FP8 ? 1 : 2;
  // q == NULL: keys only (q_out, q_norm_w and the fp8 q scales must then be NULL too)
  const bool has_q = q.p != nullptr;
  if (!has_q && (qo.p || q_norm_w || (FP8 && (q_scale || q_scale_out)))) return FLUXATTN_ERR_NULL_POINTER;
  if (!k.p || !ko.p || !k_norm_w || !pos_ids) return FLUXATTN_ERR_NULL_POINTER;
  if (has_q && (!qo.p || !q_norm_w)) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!k_scale || !k_scale_out)) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && has_q && (!q_scale || !q_scale_out)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || !rope_ok(at, ah, aw, theta, eps) || !streams_ok(streams, N))
    return FLUXATTN_ERR_INVALID_SHAPE;
  for (const View *v : {&q, &k, &qo, &ko})
    if (v->p && (!strides_ok(*v, D, E) || !head_fits(*v, N, D, E))) return FLUXATTN_ERR_INVALID_SHAPE;
  if ((has_q && !injective(qo, B, H, N, D)) || !injective(ko, B, H, N, D)) return FLUXATTN_ERR_INVALID_SHAPE;
  // (aligned() of a NULL pointer holds)
  if (!aligned(q.p, 16) || !aligned(k.p, 16) || !aligned(qo.p, 16) || !aligned(ko.p, 16) ||
      !aligned(q_norm_w, 4) || !aligned(k_norm_w, 4) || !aligned(pos_ids, 4))
    return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(q_scale_out, 4) ||
              !aligned(k_scale_out, 4)))
    return FLUXATTN_ERR_MISALIGNED;

  const int64_t BH = B * H;
  const int64_t S = streams.count;
  const Plain plains[] = {{q_norm_w, S * D * 4}, {k_norm_w, S * D * 4}, {pos_ids, N * 12}, {q_scale, BH * 4},
                          {k_scale, BH * 4},     {q_scale_out, BH * 4}, {k_scale_out, BH * 4}};
  // outputs: exactly their own input (in place) or apart from it; apart from
  // the other tensors and every plain buffer (a scale output is checked
  // against all others but itself)
  if (has_q) {
    if (!same_view(qo, q) && !disjoint(qo, q, B, H, N, D, E)) return FLUXATTN_ERR_ALIASING;
    if (!disjoint(qo, k, B, H, N, D, E) || !disjoint(qo, ko, B, H, N, D, E)) return FLUXATTN_ERR_ALIASING;
    if (!apart(qo, B, H, N, D, E, plains, 7)) return FLUXATTN_ERR_ALIASING;
  }
  if (!same_view(ko, k) && !disjoint(ko, k, B, H, N, D, E)) return FLUXATTN_ERR_ALIASING;
  if (!disjoint(ko, q, B, H, N, D, E)) return FLUXATTN_ERR_ALIASING;
  if (!apart(ko, B, H, N, D, E, plains, 7)) return FLUXATTN_ERR_ALIASING;
  if (FP8) {
    const Range tensors[] = {extent(q, B, H, N, D, E), extent(k, B, H, N, D, E), extent(qo, B, H, N, D, E),
                             extent(ko, B, H, N, D, E)};
    for (int o = 5; o < 7; ++o) {
      if (!plains[o].p) continue;
      const Range r = span(plains[o].p, plains[o].bytes);
      for (const Range &t : tensors)
        if (overlap(r, t)) return FLUXATTN_ERR_ALIASING;
      for (int i = 0; i < 7; ++i)
        if (i != o && overlap(r, span(plains[i].p, plains[i].bytes))) return FLUXATTN_ERR_ALIASING;
    }
  }
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;

  PrologueArgs a{};
  a.q = q.p;
  a.k = k.p;
  a.q_out = const_cast<void *>(qo.p);
  a.k_out = const_cast<void *>(ko.p);
  a.w_q = q_norm_w;
  a.w_k = k_norm_w;
  a.pos = pos_ids;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.q_scale_out = q_scale_out;
  a.k_scale_out = k_scale_out;
  a.BH = BH;
  a.H = static_cast<int32_t>(H);
  a.N = static_cast<int32_t>(N);
  a.eps = eps;
  auto st = [](const View &v) { return Strides{v.sb, v.sh, static_cast<int32_t>(v.sn)}; };
  a.sq = st(q);
  a.sk = st(k);
  a.sqo = st(qo);
  a.sko = st(ko);
  a.streams = to_streams(streams);
  a.num_streams = streams.count;
  const RopeTable t = make_rope_table(at, ah, aw, theta);
  const hipError_t e = FP8 ? launch_prologue_fp8(a, t, static_cast<hipStream_t>(stream))
                           : launch_prologue_bf16(a, t, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLUXATTN_OK : hip_fail(e);
}

// ---- attention (fused: q is raw and gets RMSNorm + RoPE on load)

// Validation, the split plan and the kernel arguments of one attention
// launch; nothing is enqueued.  `others` are further buffers of the calling
// entry point that the split workspace must not overlap.
template <bool FP8>
fluxattn_status forward_prepare(View q, View k, View v, const float *q_scale, const float *k_scale,
                                const float *v_scale, View o, int64_t B, int64_t H, int64_t N, int64_t D,
                                float softmax_scale, bool fused, const float *q_norm_w,
                                const fluxattn_streams &streams, const int32_t *pos_ids, int32_t at, int32_t ah,
                                int32_t aw, float theta, float eps, const fluxattn_split *split,
                                const Range *others, int n_others, ForwardArgs &a, bool &strided,
                                uint64_t *need_out = nullptr) {
  constexpr int E = FP8 ? 1 : 2;
  if (!q.p || !k.p || !v.p || !o.p) return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!q_scale || !k_scale || !v_scale)) return FLUXATTN_ERR_NULL_POINTER;
  if (fused && (!q_norm_w || !pos_ids)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || !scale_ok(softmax_scale) || !split_setting_ok(split))
    return FLUXATTN_ERR_INVALID_SHAPE;
  if (fused && (!rope_ok(at, ah, aw, theta, eps) || !streams_ok(streams, N))) return FLUXATTN_ERR_INVALID_SHAPE;
  for (const View *w : {&q, &k, &v})
    if (!strides_ok(*w, D, E) || !head_fits(*w, N, D, E)) return FLUXATTN_ERR_INVALID_SHAPE;
  if (!strides_ok(o, D, 2) || !head_fits(o, N, D, 2) || !injective(o, B, H, N, D)) return FLUXATTN_ERR_INVALID_SHAPE;
  if (!aligned(q.p, 16) || !aligned(k.p, 16) || !aligned(v.p, 16) || !aligned(o.p, 16))
    return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))) return FLUXATTN_ERR_MISALIGNED;
  if (fused && (!aligned(q_norm_w, 16) || !aligned(pos_ids, 4))) return FLUXATTN_ERR_MISALIGNED;
  const int64_t BH = B * H;
  const Range ro = extent(o, B, H, N, D, 2);
  for (const View *w : {&q, &k, &v})
    if (overlap(ro, extent(*w, B, H, N, D, E))) return FLUXATTN_ERR_ALIASING;
  const Plain plains[] = {{q_scale, BH * 4}, {k_scale, BH * 4}, {v_scale, BH * 4},
                          {fused ? q_norm_w : nullptr, streams.count * D * 4}, {fused ? pos_ids : nullptr, N * 12}};
  if (!apart(o, B, H, N, D, 2, plains, 5)) return FLUXATTN_ERR_ALIASING;
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;

  // the split plan and the uncut launch's grid depend on the device's
  // compute units, so the workspace is checked after the device
  const int32_t setting = split_setting(split);
  int32_t cus = 0;
  {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) {
      (void)hipGetLastError();
      return FLUXATTN_ERR_NO_DEVICE;
    }
    cus = compute_units(d);
  }
  const int64_t nb = forward_grid_blocks(BH, N);
  const SplitPlan plan = split_plan_for(nb, forward_key_tiles(N), setting, cus);
  const int64_t groups = plan.groups;
  if (need_out) {
    // validation only: report the workspace the launch needs
    *need_out = split_bytes(groups);
    return FLUXATTN_OK;
  }
  if (groups > 0) {
    const uint64_t need = split_bytes(groups);
    if (!split->workspace || split->workspace_bytes < need || !aligned(split->workspace, kSplitAlign))
      return FLUXATTN_ERR_WORKSPACE;
    const Range ws = span(split->workspace, static_cast<int64_t>(need));
    for (const View *w : {&q, &k, &v})
      if (overlap(ws, extent(*w, B, H, N, D, E))) return FLUXATTN_ERR_WORKSPACE;
    if (overlap(ws, ro)) return FLUXATTN_ERR_WORKSPACE;
    for (const Plain &pl : plains)
      if (overlap(ws, span(pl.p, pl.bytes))) return FLUXATTN_ERR_WORKSPACE;
    for (int i = 0; i < n_others; ++i)
      if (overlap(ws, others[i])) return FLUXATTN_ERR_WORKSPACE;
  }

  const double scale = softmax_scale > 0.f ? static_cast<double>(softmax_scale) : 1.0 / sqrt(static_cast<double>(D));
  a = ForwardArgs{};
  a.q = q.p;
  a.k = k.p;
  a.v = v.p;
  a.o = const_cast<void *>(o.p);
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.BH = static_cast<int32_t>(BH);
  a.H = static_cast<int32_t>(H);
  a.N = static_cast<int32_t>(N);
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);  // * log2(e)
  auto st = [](const View &w) { return Strides{w.sb, w.sh, static_cast<int32_t>(w.sn)}; };
  a.sq = st(q);
  a.sk = st(k);
  a.sv = st(v);
  a.so = st(o);
  if (fused) {
    a.w_q = q_norm_w;
    a.pos = pos_ids;
    a.eps = eps;
    a.streams = to_streams(streams);
    // the key prologue's frequencies (make_rope_table), in revolutions
    const int32_t dims[3] = {at, ah, aw};
    int pair = 0;
    for (int ax = 0; ax < 3; ++ax)
      for (int j = 0; j < dims[ax] / 2; ++j, ++pair) {
        for (int b = 0; b < 3; ++b)
          a.rope_rate[b][pair] =
              b == ax ? static_cast<float>(pow(static_cast<double>(theta), -2.0 * j / dims[ax]) / 6.283185307179586)
                      : 0.f;
      }
  }
  if (groups > 0) {
    a.split_cnt = static_cast<int32_t *>(split->workspace);
    a.split_part = reinterpret_cast<float *>(static_cast<char *>(split->workspace) + kSplitCountBytes);
    a.split_groups = static_cast<int32_t>(groups);
    a.split_whole = static_cast<int32_t>(plan.whole);
  }
  // uncut: one persistent workgroup per compute unit (or per block)
  a.whole_groups = static_cast<int32_t>(cus > 0 ? std::min<int64_t>(nb, cus) : nb);
  strided = !(is_contiguous(q, H, N, D) && is_contiguous(k, H, N, D) && is_contiguous(v, H, N, D) &&
              is_contiguous(o, H, N, D));
  return FLUXATTN_OK;
}

template <bool FP8>
fluxattn_status forward_launch(const ForwardArgs &a, bool fused, bool strided, void *stream) {
  const hipError_t e = FP8 ? launch_forward_fp8(a, fused, strided, static_cast<hipStream_t>(stream))
                           : launch_forward_bf16(a, fused, strided, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLUXATTN_OK : hip_fail(e);
}

template <bool FP8>
fluxattn_status forward_core(View q, View k, View v, const float *q_scale, const float *k_scale,
                             const float *v_scale, View o, int64_t B, int64_t H, int64_t N, int64_t D,
                             float softmax_scale, bool fused, const float *q_norm_w,
                             const fluxattn_streams &streams, const int32_t *pos_ids, int32_t at, int32_t ah,
                             int32_t aw, float theta, float eps, const fluxattn_split *split, void *stream) {
  ForwardArgs a;
  bool strided = false;
  const fluxattn_status s =
      forward_prepare<FP8>(q, k, v, q_scale, k_scale, v_scale, o, B, H, N, D, softmax_scale, fused, q_norm_w, streams,
                           pos_ids, at, ah, aw, theta, eps, split, nullptr, 0, a, strided);
  if (s != FLUXATTN_OK) return s;
  return forward_launch<FP8>(a, fused, strided, stream);
}

// ---- the whole block: keys-only prologue into k_work (contiguous), then
// the fused attention

template <bool FP8>
fluxattn_status joint_core(View q, View k, View v, const float *q_scale, const float *k_scale,
                           const float *v_scale, void *k_work, float *k_scale_work, View o,
                           const float *q_norm_w, const float *k_norm_w, const fluxattn_streams &streams,
                           const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D, int32_t at,
                           int32_t ah, int32_t aw, float theta, float eps, float softmax_scale,
                           const fluxattn_split *split, void *stream) {
  constexpr int E = FP8 ? 1 : 2;
  if (!q.p || !k.p || !v.p || !k_work || !o.p || !q_norm_w || !k_norm_w || !pos_ids)
    return FLUXATTN_ERR_NULL_POINTER;
  if (FP8 && (!q_scale || !k_scale || !v_scale || !k_scale_work)) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || !rope_ok(at, ah, aw, theta, eps) || !scale_ok(softmax_scale) ||
      !streams_ok(streams, N) || !split_setting_ok(split))
    return FLUXATTN_ERR_INVALID_SHAPE;
  View kw = contiguous(k_work, H, N, D);
  for (const View *w : {&q, &k, &v})
    if (!strides_ok(*w, D, E) || !head_fits(*w, N, D, E)) return FLUXATTN_ERR_INVALID_SHAPE;
  if (!strides_ok(o, D, 2) || !head_fits(o, N, D, 2) || !injective(o, B, H, N, D) || !head_fits(kw, N, D, E))
    return FLUXATTN_ERR_INVALID_SHAPE;
  if (!aligned(q.p, 16) || !aligned(k.p, 16) || !aligned(v.p, 16) || !aligned(k_work, 16) || !aligned(o.p, 16) ||
      !aligned(q_norm_w, 16) || !aligned(k_norm_w, 4) || !aligned(pos_ids, 4))
    return FLUXATTN_ERR_MISALIGNED;
  if (FP8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(k_scale_work, 4)))
    return FLUXATTN_ERR_MISALIGNED;

  const int64_t BH = B * H;
  const int64_t S = streams.count;
  const Plain plains[] = {{q_norm_w, S * D * 4}, {k_norm_w, S * D * 4}, {pos_ids, N * 12}, {q_scale, BH * 4},
                          {k_scale, BH * 4},     {v_scale, BH * 4},     {k_scale_work, BH * 4}};
  // k_work: exactly k (in place) or apart from everything else
  if (!same_view(kw, k) && !disjoint(kw, k, B, H, N, D, E)) return FLUXATTN_ERR_ALIASING;
  if (!disjoint(kw, q, B, H, N, D, E) || !disjoint(kw, v, B, H, N, D, E)) return FLUXATTN_ERR_ALIASING;
  if (overlap(extent(kw, B, H, N, D, E), extent(o, B, H, N, D, 2)) || !apart(kw, B, H, N, D, E, plains, 7))
    return FLUXATTN_ERR_ALIASING;
  // o: apart from every input and k_work
  for (const View *w : {&q, &k, &v})
    if (overlap(extent(o, B, H, N, D, 2), extent(*w, B, H, N, D, E))) return FLUXATTN_ERR_ALIASING;
  if (!apart(o, B, H, N, D, 2, plains, 7)) return FLUXATTN_ERR_ALIASING;
  if (FP8) {
    // the new key scales: apart from all other buffers
    const Range r = span(k_scale_work, BH * 4);
    for (const View *w : {&q, &k, &v, &kw})
      if (overlap(r, extent(*w, B, H, N, D, E))) return FLUXATTN_ERR_ALIASING;
    if (overlap(r, extent(o, B, H, N, D, 2))) return FLUXATTN_ERR_ALIASING;
    for (int i = 0; i < 6; ++i)
      if (overlap(r, span(plains[i].p, plains[i].bytes))) return FLUXATTN_ERR_ALIASING;
  }
  const fluxattn_status dev = device_ok();
  if (dev != FLUXATTN_OK) return dev;
  // the attention launch (and its split workspace, which must not overlap
  // the raw keys and their weights either) is checked before the prologue
  // is enqueued; both calls re-validate a subset of the above and cannot
  // fail it
  const Range others[] = {extent(k, B, H, N, D, E), span(k_norm_w, S * D * 4)};
  ForwardArgs fa;
  bool strided = false;
  fluxattn_status s =
      forward_prepare<FP8>(q, kw, v, q_scale, k_scale_work, v_scale, o, B, H, N, D, softmax_scale, true, q_norm_w,
                           streams, pos_ids, at, ah, aw, theta, eps, split, others, 2, fa, strided);
  if (s != FLUXATTN_OK) return s;
  s = prologue_core<FP8>(View{}, k, nullptr, k_scale, View{}, kw, nullptr, k_scale_work, nullptr, k_norm_w, streams,
                         pos_ids, B, H, N, D, at, ah, aw, theta, eps, stream);
  if (s != FLUXATTN_OK) return s;
  return forward_launch<FP8>(fa, true, strided, stream);
}

const fluxattn_streams kOneStream = {1, {0, 0, 0, 0}};

}  // namespace

namespace fluxattn {

fluxattn_status record_hip_error(hipError_t e) { return hip_fail(e); }

fluxattn_status check_forward_fused_ex_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                            fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
                                            void *o, fluxattn_layout o_layout, const float *q_norm_w,
                                            const fluxattn_streams &streams, const int32_t *pos_ids, int64_t B,
                                            int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                            int32_t axes_w, float theta, float eps, float softmax_scale,
                                            int32_t groups, uint64_t *need_bytes) {
  const fluxattn_split sp = {groups, nullptr, 0};
  ForwardArgs a;
  bool strided = false;
  return forward_prepare<false>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), nullptr, nullptr,
                                nullptr, view_of(o, o_layout), B, H, N, D, softmax_scale, true, q_norm_w, streams,
                                pos_ids, axes_t, axes_h, axes_w, theta, eps, &sp, nullptr, 0, a, strided,
                                need_bytes);
}

}  // namespace fluxattn

extern "C" {

fluxattn_status fluxattn_qk_norm_rope_bf16(const void *q, const void *k, void *q_out, void *k_out,
                                           const float *q_norm_w, const float *k_norm_w,
                                           const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                           int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                           float theta, float eps, void *stream) {
  return prologue_core<false>(contiguous(q, H, N, D), contiguous(k, H, N, D), nullptr, nullptr,
                              contiguous(q_out, H, N, D), contiguous(k_out, H, N, D), nullptr, nullptr, q_norm_w,
                              k_norm_w, kOneStream, pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, stream);
}

fluxattn_status fluxattn_qk_norm_rope_fp8(const uint8_t *q, const uint8_t *k, const float *q_scale,
                                          const float *k_scale, uint8_t *q_out, uint8_t *k_out,
                                          float *q_scale_out, float *k_scale_out, const float *q_norm_w,
                                          const float *k_norm_w, const int32_t *pos_ids, int64_t B,
                                          int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                          int32_t axes_w, float theta, float eps, void *stream) {
  return prologue_core<true>(contiguous(q, H, N, D), contiguous(k, H, N, D), q_scale, k_scale,
                             contiguous(q_out, H, N, D), contiguous(k_out, H, N, D), q_scale_out, k_scale_out,
                             q_norm_w, k_norm_w, kOneStream, pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta,
                             eps, stream);
}

fluxattn_status fluxattn_qk_norm_rope_ex_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                              fluxattn_layout k_layout, void *q_out, fluxattn_layout q_out_layout,
                                              void *k_out, fluxattn_layout k_out_layout, const float *q_norm_w,
                                              const float *k_norm_w, fluxattn_streams streams,
                                              const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D,
                                              int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta,
                                              float eps, void *stream) {
  return prologue_core<false>(view_of(q, q_layout), view_of(k, k_layout), nullptr, nullptr,
                              view_of(q_out, q_out_layout), view_of(k_out, k_out_layout), nullptr, nullptr, q_norm_w,
                              k_norm_w, streams, pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, stream);
}

fluxattn_status fluxattn_qk_norm_rope_ex_fp8(const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
                                             fluxattn_layout k_layout, const float *q_scale, const float *k_scale,
                                             uint8_t *q_out, fluxattn_layout q_out_layout, uint8_t *k_out,
                                             fluxattn_layout k_out_layout, float *q_scale_out, float *k_scale_out,
                                             const float *q_norm_w, const float *k_norm_w,
                                             fluxattn_streams streams, const int32_t *pos_ids, int64_t B,
                                             int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                             int32_t axes_w, float theta, float eps, void *stream) {
  return prologue_core<true>(view_of(q, q_layout), view_of(k, k_layout), q_scale, k_scale,
                             view_of(q_out, q_out_layout), view_of(k_out, k_out_layout), q_scale_out, k_scale_out,
                             q_norm_w, k_norm_w, streams, pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps,
                             stream);
}

fluxattn_status fluxattn_forward_bf16(const void *q, const void *k, const void *v, void *o, int64_t B,
                                      int64_t H, int64_t N, int64_t D, float softmax_scale, void *stream) {
  return forward_core<false>(contiguous(q, H, N, D), contiguous(k, H, N, D), contiguous(v, H, N, D), nullptr,
                             nullptr, nullptr, contiguous(o, H, N, D), B, H, N, D, softmax_scale, false, nullptr,
                             kOneStream, nullptr, 0, 0, 0, 0.f, 0.f, nullptr, stream);
}

fluxattn_status fluxattn_forward_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                                     const float *q_scale, const float *k_scale, const float *v_scale,
                                     void *o, int64_t B, int64_t H, int64_t N, int64_t D,
                                     float softmax_scale, void *stream) {
  return forward_core<true>(contiguous(q, H, N, D), contiguous(k, H, N, D), contiguous(v, H, N, D), q_scale,
                            k_scale, v_scale, contiguous(o, H, N, D), B, H, N, D, softmax_scale, false, nullptr,
                            kOneStream, nullptr, 0, 0, 0, 0.f, 0.f, nullptr, stream);
}

fluxattn_status fluxattn_forward_ex_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                         fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
                                         void *o, fluxattn_layout o_layout, int64_t B, int64_t H, int64_t N,
                                         int64_t D, float softmax_scale, const fluxattn_split *split,
                                         void *stream) {
  return forward_core<false>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), nullptr, nullptr,
                             nullptr, view_of(o, o_layout), B, H, N, D, softmax_scale, false, nullptr, kOneStream,
                             nullptr, 0, 0, 0, 0.f, 0.f, split, stream);
}

fluxattn_status fluxattn_forward_ex_fp8(const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
                                        fluxattn_layout k_layout, const uint8_t *v, fluxattn_layout v_layout,
                                        const float *q_scale, const float *k_scale, const float *v_scale, void *o,
                                        fluxattn_layout o_layout, int64_t B, int64_t H, int64_t N, int64_t D,
                                        float softmax_scale, const fluxattn_split *split, void *stream) {
  return forward_core<true>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), q_scale, k_scale,
                            v_scale, view_of(o, o_layout), B, H, N, D, softmax_scale, false, nullptr, kOneStream,
                            nullptr, 0, 0, 0, 0.f, 0.f, split, stream);
}

fluxattn_status fluxattn_forward_fused_bf16(const void *q, const void *k, const void *v, void *o,
                                            const float *q_norm_w, const int32_t *pos_ids, int64_t B,
                                            int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                            int32_t axes_w, float theta, float eps, float softmax_scale,
                                            void *stream) {
  return forward_core<false>(contiguous(q, H, N, D), contiguous(k, H, N, D), contiguous(v, H, N, D), nullptr,
                             nullptr, nullptr, contiguous(o, H, N, D), B, H, N, D, softmax_scale, true, q_norm_w,
                             kOneStream, pos_ids, axes_t, axes_h, axes_w, theta, eps, nullptr, stream);
}

fluxattn_status fluxattn_forward_fused_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                                           const float *q_scale, const float *k_scale, const float *v_scale,
                                           void *o, const float *q_norm_w, const int32_t *pos_ids, int64_t B,
                                           int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                           int32_t axes_w, float theta, float eps, float softmax_scale,
                                           void *stream) {
  return forward_core<true>(contiguous(q, H, N, D), contiguous(k, H, N, D), contiguous(v, H, N, D), q_scale,
                            k_scale, v_scale, contiguous(o, H, N, D), B, H, N, D, softmax_scale, true, q_norm_w,
                            kOneStream, pos_ids, axes_t, axes_h, axes_w, theta, eps, nullptr, stream);
}

fluxattn_status fluxattn_joint_attention_bf16(const void *q, const void *k, const void *v, void *k_work,
                                              void *o, const float *q_norm_w, const float *k_norm_w,
                                              const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                              int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                              float theta, float eps, float softmax_scale, void *stream) {
  return joint_core<false>(contiguous(q, H, N, D), contiguous(k, H, N, D), contiguous(v, H, N, D), nullptr, nullptr,
                           nullptr, k_work, nullptr, contiguous(o, H, N, D), q_norm_w, k_norm_w, kOneStream, pos_ids,
                           B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, nullptr, stream);
}

fluxattn_status fluxattn_joint_attention_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                                             const float *q_scale, const float *k_scale,
                                             const float *v_scale, uint8_t *k_work, float *k_scale_work,
                                             void *o, const float *q_norm_w, const float *k_norm_w,
                                             const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                             int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                             float theta, float eps, float softmax_scale, void *stream) {
  return joint_core<true>(contiguous(q, H, N, D), contiguous(k, H, N, D), contiguous(v, H, N, D), q_scale, k_scale,
                          v_scale, k_work, k_scale_work, contiguous(o, H, N, D), q_norm_w, k_norm_w, kOneStream,
                          pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, nullptr, stream);
}

fluxattn_status fluxattn_joint_attention_ex_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                                 fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
                                                 void *k_work, void *o, fluxattn_layout o_layout,
                                                 const float *q_norm_w, const float *k_norm_w,
                                                 fluxattn_streams streams, const int32_t *pos_ids, int64_t B,
                                                 int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                                 int32_t axes_w, float theta, float eps, float softmax_scale,
                                                 const fluxattn_split *split, void *stream) {
  return joint_core<false>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), nullptr, nullptr,
                           nullptr, k_work, nullptr, view_of(o, o_layout), q_norm_w, k_norm_w, streams, pos_ids, B, H,
                           N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, split, stream);
}

fluxattn_status fluxattn_joint_attention_ex_fp8(const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
                                                fluxattn_layout k_layout, const uint8_t *v, fluxattn_layout v_layout,
                                                const float *q_scale, const float *k_scale, const float *v_scale,
                                                uint8_t *k_work, float *k_scale_work, void *o,
                                                fluxattn_layout o_layout, const float *q_norm_w,
                                                const float *k_norm_w, fluxattn_streams streams,
                                                const int32_t *pos_ids, int64_t B, int64_t H, int64_t N, int64_t D,
                                                int32_t axes_t, int32_t axes_h, int32_t axes_w, float theta,
                                                float eps, float softmax_scale, const fluxattn_split *split,
                                                void *stream) {
  return joint_core<true>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), q_scale, k_scale,
                          v_scale, k_work, k_scale_work, view_of(o, o_layout), q_norm_w, k_norm_w, streams, pos_ids,
                          B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, split, stream);
}

fluxattn_status fluxattn_forward_fused_ex_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                               fluxattn_layout k_layout, const void *v, fluxattn_layout v_layout,
                                               void *o, fluxattn_layout o_layout, const float *q_norm_w,
                                               fluxattn_streams streams, const int32_t *pos_ids, int64_t B,
                                               int64_t H, int64_t N, int64_t D, int32_t axes_t, int32_t axes_h,
                                               int32_t axes_w, float theta, float eps, float softmax_scale,
                                               const fluxattn_split *split, void *stream) {
  return forward_core<false>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), nullptr, nullptr,
                             nullptr, view_of(o, o_layout), B, H, N, D, softmax_scale, true, q_norm_w, streams,
                             pos_ids, axes_t, axes_h, axes_w, theta, eps, split, stream);
}

fluxattn_status fluxattn_forward_fused_ex_fp8(const uint8_t *q, fluxattn_layout q_layout, const uint8_t *k,
                                              fluxattn_layout k_layout, const uint8_t *v, fluxattn_layout v_layout,
                                              const float *q_scale, const float *k_scale, const float *v_scale,
                                              void *o, fluxattn_layout o_layout, const float *q_norm_w,
                                              fluxattn_streams streams, const int32_t *pos_ids, int64_t B, int64_t H,
                                              int64_t N, int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                              float theta, float eps, float softmax_scale,
                                              const fluxattn_split *split, void *stream) {
  return forward_core<true>(view_of(q, q_layout), view_of(k, k_layout), view_of(v, v_layout), q_scale, k_scale,
                            v_scale, view_of(o, o_layout), B, H, N, D, softmax_scale, true, q_norm_w, streams, pos_ids,
                            axes_t, axes_h, axes_w, theta, eps, split, stream);
}

fluxattn_status fluxattn_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t groups,
                                               uint64_t *bytes) {
  if (!bytes) return FLUXATTN_ERR_NULL_POINTER;
  if (!shape_ok(B, H, N, D) || groups > kMaxGroups) return FLUXATTN_ERR_INVALID_SHAPE;
  int32_t cus = 0;
  if (groups == 0) {
    const fluxattn_status dev = device_ok();
    if (dev != FLUXATTN_OK) return dev;
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) {
      (void)hipGetLastError();
      return FLUXATTN_ERR_NO_DEVICE;
    }
    cus = compute_units(d);
  }
  *bytes = split_bytes(split_plan_for(forward_grid_blocks(B * H, N), forward_key_tiles(N), groups, cus).groups);
  return FLUXATTN_OK;
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
    case FLUXATTN_ERR_WORKSPACE: return "split workspace missing, too small, misaligned or overlapping";
  }
  return "unknown status";
}

int fluxattn_last_hip_error(void) { return g_last_hip_error; }

int fluxattn_version(void) { return 20000; }

}  // extern "C"

// fluxattn_forward_fused_noalloc_bf16: the fused bf16 attention with the
// key-range split, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops).  Its split workspace is a static device
// array of this file instead of caller memory; everything else is
// fluxattn_forward_fused_ex_bf16.
#include <atomic>
#include <mutex>

#include "fluxattn.h"
#include "fluxattn_internal.h"

using namespace fluxattn;

namespace {

// Room for a split over 256 workgroups, one per compute unit of an MI355X
// (the default setting's launch there): 128 KiB of arrival counts and two
// 136 KiB partial slots per workgroup, 68.1 MiB.  Every GPU the library runs
// this entry point on holds its own copy until the process ends.
constexpr int32_t kScratchGroups = 256;
constexpr uint64_t kScratchBytes = split_workspace_bytes_for(kScratchGroups);

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of each GPU's copy (0 until the first call on that device
// has looked it up and cleared its arrival counts).
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch[kMaxDevices];
std::mutex g_setup_mu;

__global__ void clear_counts_kernel(int32_t *counts, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) counts[i] = 0;
}

// Set-up on the current device: look the array up (host code must use
// this address, never the array's name) and clear its arrival counts on
// `s`, ahead of the first launch that uses it.  The counts are zero from
// static initialisation already; every split launch leaves them at zero.
hipError_t scratch_for_device(int dev, hipStream_t s, void **out) {
  uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) {
    *out = reinterpret_cast<void *>(p);
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_setup_mu);
  p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    constexpr int n = static_cast<int>(kSplitCountBytes / sizeof(int32_t));
    hipLaunchKernelGGL(clear_counts_kernel, dim3(32), dim3(256), 0, s, static_cast<int32_t *>(ptr), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    p = reinterpret_cast<uintptr_t>(ptr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = reinterpret_cast<void *>(p);
  return hipSuccess;
}

}  // namespace

extern "C" {

fluxattn_status fluxattn_forward_fused_noalloc_bf16(const void *q, fluxattn_layout q_layout, const void *k,
                                                    fluxattn_layout k_layout, const void *v,
                                                    fluxattn_layout v_layout, void *o, fluxattn_layout o_layout,
                                                    const float *q_norm_w, fluxattn_streams streams,
                                                    const int32_t *pos_ids, int64_t B, int64_t H, int64_t N,
                                                    int64_t D, int32_t axes_t, int32_t axes_h, int32_t axes_w,
                                                    float theta, float eps, float softmax_scale, int32_t groups,
                                                    void *stream) {
  // every check of the workspace-taking entry point but the workspace's,
  // and the bytes the launch's split needs
  uint64_t need = 0;
  fluxattn_status st = check_forward_fused_ex_bf16(q, q_layout, k, k_layout, v, v_layout, o, o_layout, q_norm_w,
                                                   streams, pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps,
                                                   softmax_scale, groups, &need);
  if (st != FLUXATTN_OK) return st;
  if (need > kScratchBytes) return FLUXATTN_ERR_WORKSPACE;   // more than 256 workgroups
  if (need == 0)   // not cut: no scratch at all
    return fluxattn_forward_fused_ex_bf16(q, q_layout, k, k_layout, v, v_layout, o, o_layout, q_norm_w, streams,
                                          pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale,
                                          nullptr, stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FLUXATTN_ERR_NO_DEVICE;
  }
  void *ws = nullptr;
  e = scratch_for_device(dev, static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) return record_hip_error(e);
  const fluxattn_split sp = {groups, ws, kScratchBytes};
  return fluxattn_forward_fused_ex_bf16(q, q_layout, k, k_layout, v, v_layout, o, o_layout, q_norm_w, streams,
                                        pos_ids, B, H, N, D, axes_t, axes_h, axes_w, theta, eps, softmax_scale, &sp,
                                        stream);
}

}  // extern "C"

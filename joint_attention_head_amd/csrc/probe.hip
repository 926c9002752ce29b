// fluxattn_probe_mfma: the practical matrix-core rate of the chip, as the
// context of the attention kernels' roofline fractions.  Every SIMD runs two
// waves (the attention kernels' occupancy) issuing back-to-back MFMAs of one
// shape (bf16 32x32x16, E4M3 32x32x64 as the fp8 kernel, bf16 16x16x32 as
// the bf16 kernel) on register operands: independent accumulator chains
// (four of the 32x32 shapes, eight of the 16x16 one), and A and B operands
// taken in turn from eight pseudo-random fragments each, so the operand data
// changes from one MFMA to the next as it does in attention.  Nothing else
// runs, so the rate it reaches is what the matrix cores deliver at the clock
// the power limit allows for this work alone.
#include <string.h>

#include "fluxattn.h"
#include "fluxattn_internal.h"
#include "fluxattn_probe.h"

namespace fluxattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kFrags = 8;
constexpr int kChains = 4;

// A well-mixed 32-bit hash (the finaliser of splitmix32-style generators).
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 value of magnitude in [2^-2, 2^2) with a random sign and mantissa.
__device__ __forceinline__ __bf16 rand_bf16(uint32_t h) {
  const uint16_t bits = (uint16_t)(((h & 1u) << 15) | ((125u + ((h >> 1) & 3u)) << 7) | ((h >> 3) & 0x7fu));
  return __builtin_bit_cast(__bf16, bits);
}

// E4M3 code of magnitude in [2^-3, 2^4] with a random sign (never NaN).
__device__ __forceinline__ uint32_t rand_e4m3(uint32_t h) {
  return ((h & 1u) << 7) | ((4u + ((h >> 1) & 7u)) << 3) | ((h >> 4) & 7u);
}

__global__ __launch_bounds__(kWaves * 64) void probe_bf16_kernel(int64_t iterations, float *sink) {
  const uint32_t seed = (blockIdx.x * blockDim.x + threadIdx.x) * 0x9e3779b9u;
  bf16x8_t a[kFrags], b[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[f][e] = rand_bf16(mix32(seed + 16u * f + e));
      b[f][e] = rand_bf16(mix32(seed + 16u * f + e + 8u + 0x5bd1e995u));
    }
  f32x16_t acc[kChains] = {};
  for (int64_t it = 0; it < iterations; ++it) {
#pragma unroll
    for (int k = 0; k < kFrags; ++k)
      acc[k % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + 3) % kFrags], acc[k % kChains], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * kWaves + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(kWaves * 64) void probe_fp8_kernel(int64_t iterations, float *sink) {
  const uint32_t seed = (blockIdx.x * blockDim.x + threadIdx.x) * 0x9e3779b9u;
  i32x8_t a[kFrags], b[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t wa = 0, wb = 0;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        wa |= rand_e4m3(mix32(seed + 64u * f + 4u * e + y)) << (8 * y);
        wb |= rand_e4m3(mix32(seed + 64u * f + 4u * e + y + 0x5bd1e995u)) << (8 * y);
      }
      a[f][e] = (int)wa;
      b[f][e] = (int)wb;
    }
  f32x16_t acc[kChains] = {};
  for (int64_t it = 0; it < iterations; ++it) {
#pragma unroll
    for (int k = 0; k < kFrags; ++k)
      acc[k % kChains] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k], b[(k + 3) % kFrags], acc[k % kChains],
                                                                         0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * kWaves + (threadIdx.x >> 6)] = s;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16 MFMAs of 16 x 16 x 32 per round (the flops of 8 of 32 x 32 x 16), eight
// accumulator chains
__global__ __launch_bounds__(kWaves * 64) void probe_bf16_16_kernel(int64_t iterations, float *sink) {
  const uint32_t seed = (blockIdx.x * blockDim.x + threadIdx.x) * 0x9e3779b9u;
  bf16x8_t a[kFrags], b[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[f][e] = rand_bf16(mix32(seed + 16u * f + e));
      b[f][e] = rand_bf16(mix32(seed + 16u * f + e + 8u + 0x5bd1e995u));
    }
  f32x4_t acc[8] = {};
  for (int64_t it = 0; it < iterations; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int k = 0; k < kFrags; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], b[(k + 3 + r) % kFrags], acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[c][e];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * kWaves + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace fluxattn

using namespace fluxattn;

extern "C" {

fluxattn_status fluxattn_probe_mfma(int32_t kind, int64_t iterations, int32_t workgroups, float *sink,
                                    double *flops, void *stream) {
  if (!sink || !flops) return FLUXATTN_ERR_NULL_POINTER;
  if ((kind < 0 || kind > 2) || iterations < 1 || iterations > (int64_t(1) << 40) || workgroups < 1 ||
      workgroups > (1 << 20))
    return FLUXATTN_ERR_INVALID_SHAPE;
  if (reinterpret_cast<uintptr_t>(sink) & 3) return FLUXATTN_ERR_MISALIGNED;
  int dev = -1;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    (void)hipGetLastError();
    return FLUXATTN_ERR_NO_DEVICE;
  }
  // flop per round and wave: 8 MFMAs of 2 * 32 * 32 * k, k = 16 (bf16) or
  // 64 (E4M3), or 16 of 2 * 16 * 16 * 32 (bf16, the same as kind 0)
  const double per_round = kind == 1 ? 8 * 2.0 * 32 * 32 * 64 : 8 * 2.0 * 32 * 32 * 16;
  *flops = per_round * static_cast<double>(iterations) * kWaves * workgroups;
  if (kind == 2)
    hipLaunchKernelGGL(probe_bf16_16_kernel, dim3(workgroups), dim3(kWaves * 64), 0, static_cast<hipStream_t>(stream),
                       iterations, sink);
  else if (kind == 0)
    hipLaunchKernelGGL(probe_bf16_kernel, dim3(workgroups), dim3(kWaves * 64), 0, static_cast<hipStream_t>(stream),
                       iterations, sink);
  else
    hipLaunchKernelGGL(probe_fp8_kernel, dim3(workgroups), dim3(kWaves * 64), 0, static_cast<hipStream_t>(stream),
                       iterations, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FLUXATTN_OK : record_hip_error(e);
}

}  // extern "C"

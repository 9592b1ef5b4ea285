// Device-side helpers shared by the gfx950 kernels of the ladder decode/prefill path.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ladder {

// bf16 is carried as its 16-bit pattern; its value is the fp32 with those upper bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Elements of a weight type per 16-byte vector load.
template <typename WT> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<uint16_t> { static constexpr int N = 8; };

// Unpack one 16-byte chunk of weights into fp32.
__device__ __forceinline__ void unpack16(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void unpack16(const uint4& v, float (&f)[4]) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename WT> __device__ __forceinline__ float load_w(const WT* p);
template <> __device__ __forceinline__ float load_w<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_w<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename WT> __device__ __forceinline__ void store_w(WT* p, float v);
template <> __device__ __forceinline__ void store_w<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_w<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Launch timing (measurement aid).  While armed, the decode-path launches go through
// hipExtLaunchKernelGGL: the first one records `start` when its dispatch begins, every
// one records `stop` when its dispatch ends, so the pair spans exactly the kernels
// launched between arming and disarming.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool armed = false;
};
LaunchEvents& launch_events();   // this host thread's

template <typename F, typename... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, Args... args) {
  LaunchEvents& le = launch_events();
  if (le.armed) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, le.start, le.stop, 0, args...);
    le.start = nullptr;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

}  // namespace ladder

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

// RoPE rotation of the adjacent pair (a, b) by the angle of cosine c and sine s,
// a' = a c - b s and b' = a s + b c, each with one fused multiply-add in a fixed order so
// that every kernel that rotates rounds the same way.
__device__ __forceinline__ void rope_rot(float& a, float& b, float c, float s) {
  const float r0 = fmaf(a, c, -(b * s));
  const float r1 = fmaf(a, s, b * c);
  a = r0;
  b = r1;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// fp16 operands of the matrix cores.  A pair hi = fp16(v), lo = fp16(v - hi) carries
// about 22 significant bits of an fp32 value; bf16 values convert to fp16 exactly for
// |v| in [2^-17, 65504].
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void split_h2(float a, float b, uint32_t& hi, uint32_t& lo) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 h = {(_Float16)a, (_Float16)b};
  const h2 l = {(_Float16)(a - (float)h[0]), (_Float16)(b - (float)h[1])};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// bf16 operands of the matrix cores: a pair hi = bf16(a), lo = bf16(a - hi) carries about
// 16 significant bits of an fp32 value over fp32's exponent range.  Both conversions are
// gfx950's packed v_cvt_pk_bf16_f32 (round to nearest even).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split_bf2(float a, float b, uint32_t& hi, uint32_t& lo) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 h = {(__bf16)a, (__bf16)b};
  const bf2 l = {(__bf16)(a - (float)h[0]), (__bf16)(b - (float)h[1])};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// 8 bf16 (one 16-byte chunk) -> 8 fp16
__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4& v) {
  return make_uint4(pack_h2(bf16_lo(v.x), bf16_hi(v.x)), pack_h2(bf16_lo(v.y), bf16_hi(v.y)),
                    pack_h2(bf16_lo(v.z), bf16_hi(v.z)), pack_h2(bf16_lo(v.w), bf16_hi(v.w)));
}

__device__ __forceinline__ void wave_stores_done_fwd() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xF70);               // vmcnt(0): this wave's stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Coherent (agent-scope) accesses for data that one workgroup writes and another reads
// within a kernel: they bypass the per-XCD caches, so publishing them needs no L2
// write-back, only that the stores have completed.
// Device memory through a pointer the compiler cannot trace to a kernel argument (read
// from a table in memory, say) would be accessed with flat instructions, which count in
// both the vector-memory and the LDS counters, so every use of a load waits for all
// outstanding loads.  Every pointer given to gbl() addresses device memory.
#define LADDER_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const LADDER_GLOBAL T* gbl(const T* p) { return (const LADDER_GLOBAL T*)p; }
template <typename T>
__device__ __forceinline__ LADDER_GLOBAL T* gbl(T* p) { return (LADDER_GLOBAL T*)p; }
typedef float gf32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int gu32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ldg4(const float* p) {
  const gf32x4 v = *(const LADDER_GLOBAL gf32x4*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldg4u(const void* p) {
  const gu32x4 v = *(const LADDER_GLOBAL gu32x4*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Streaming (nontemporal) 16-byte load for data read once per pass, such as weight rows:
// the line is not kept in the caches, which streams ~15% faster than an ordinary load.
__device__ __forceinline__ uint4 ldg4u_nt(const void* p) {
  const gu32x4 v = __builtin_nontemporal_load((const LADDER_GLOBAL gu32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stg4(float* p, const float4& v) {
  gf32x4 w;
  w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
  *(LADDER_GLOBAL gf32x4*)p = w;
}

__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(gbl(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(gbl(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(gbl(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(gbl(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ld_coh4(const float* p) {
  return make_float4(ld_coh(p), ld_coh(p + 1), ld_coh(p + 2), ld_coh(p + 3));
}
__device__ __forceinline__ void st_coh4(float* p, float4 v) {
  st_coh(p, v.x); st_coh(p + 1, v.y); st_coh(p + 2, v.z); st_coh(p + 3, v.w);
}

// Arrival of a workgroup whose cross-workgroup writes were all coherent stores: once
// every wave's stores have completed it counts itself; the last of `total` resets the
// count and publishes `epoch` in *flag.
__device__ __forceinline__ void wg_arrive_coh(int* cnt, int* flag, int total, int epoch) {
  wave_stores_done_fwd();
  __syncthreads();
  if (threadIdx.x == 0 && __hip_atomic_fetch_add(gbl(cnt), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1) {
    __hip_atomic_store(gbl(cnt), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gbl(flag), epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait (one thread polls, bounded) until *flag == epoch; the data behind it is read with
// coherent loads, so no invalidate is needed.  A poll that gives up sets *err.
__device__ __forceinline__ void wg_wait_coh(const int* flag, int epoch, int* err) {
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(gbl(flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins == (1u << 19)) {          // far beyond any real wait
        __hip_atomic_fetch_or(gbl(err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      // another wait already gave up: the results are void, so do not wait again
      if ((spins & 1023u) == 0 && __hip_atomic_load(gbl(err), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
    }
  }
  __syncthreads();
}

// Progress words: every producer workgroup owns one 32-bit word and stores a code that
// only grows (step epoch, layer, phase) when it has finished a phase; "all producers
// passed phase X" is min over the words >= code(X).  Unlike one shared counter, the
// producers' updates are independent stores, so none waits behind the others' atomics.
__device__ __forceinline__ void prog_publish(uint32_t* word, uint32_t code) {
  wave_stores_done_fwd();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(gbl(word), code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every word of prog[0..n) has reached `code` (wrap-safe comparison); the
// whole workgroup polls, one word per thread and round.  Bounded: after 2^16 rounds it
// sets *err and returns; it also returns once another wait has set *err.  Every exit is
// taken by the whole workgroup together.
__device__ __forceinline__ void prog_wait(const uint32_t* prog, int n, uint32_t code, int* err) {
  unsigned rounds = 0;
  for (;;) {
    int ok = 1;
    for (int i = threadIdx.x; i < n; i += blockDim.x)
      ok &= (int)(__hip_atomic_load(gbl(prog) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - code) >= 0;
    if (__syncthreads_and(ok)) return;
    if ((++rounds & 255u) == 0) {
      int bail = rounds >= (1u << 16);
      if (threadIdx.x == 0) {
        if (bail) __hip_atomic_fetch_or(gbl(err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else bail = __hip_atomic_load(gbl(err), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      }
      if (__syncthreads_or(bail)) return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Cross-workgroup synchronisation inside one kernel, with one L2 write-back or
// invalidate per workgroup (not one per wave): every wave first waits for its own global
// stores to complete (they are then in its XCD's L2), the workgroup meets at a barrier,
// and one thread performs the agent-scope release (L2 write-back) or acquire (L1/L2
// invalidate) for all of them.
__device__ __forceinline__ void wave_stores_done() { wave_stores_done_fwd(); }

// A producer workgroup, after its writes, counts itself; the last of `total` publishes
// the step's epoch in *flag.
__device__ __forceinline__ void wg_signal(int* cnt, int* flag, int total, int epoch) {
  wave_stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (atomicAdd(cnt, 1) == total - 1) {
      __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
      __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// A consumer waits (one thread polls, bounded) until *flag == epoch, then acquires; on a
// poll that gives up it sets *err and goes on, so every wave still ends.
__device__ __forceinline__ void wg_wait(const int* flag, int epoch, int* err) {
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == (1u << 18)) {          // ~14 ms: far beyond any real wait
        atomicOr(err, 1);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

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

// Small memory-bound kernels of the prefill path and the decode step prologue.
#include <climits>

#include "common.hpp"
#include "kernels.h"

namespace ladder {

LaunchEvents& launch_events() {
  static thread_local LaunchEvents le;
  return le;
}

void launch_events_arm(hipEvent_t start, hipEvent_t stop) {
  LaunchEvents& le = launch_events();
  le.start = start;
  le.stop = stop;
  le.armed = true;
}

void launch_events_disarm() { launch_events() = LaunchEvents{}; }

// x[m][:] = E[ids[m]][:] in fp32.  Ids outside [0, V) are clamped so a bad id cannot
// read outside the table.
template <typename WT>
__device__ __forceinline__ void embed_row(const WT* table, int V, int H, int id, float* x) {
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const WT* row = table + (size_t)id * H;
  constexpr int VEC = Vec<WT>::N;                   // 16-byte vectors: 8 bf16 or 4 fp32
  if (H % VEC == 0) {
    const int nv = H / VEC;
    for (int v0 = threadIdx.x; v0 < nv; v0 += 4 * 256) {
      uint4 r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {                 // the four loads in flight together
        const int v = v0 + 256 * k;
        r[k] = v < nv ? *(const uint4*)(row + (size_t)v * VEC) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = v0 + 256 * k;
        if (v < nv) {
          float f[VEC];
          unpack16(r[k], f);
#pragma unroll
          for (int e = 0; e < VEC; e += 4)
            *(float4*)(x + (size_t)v * VEC + e) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < H; i += 256) x[i] = load_w<WT>(row + i);
  }
}

template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel(const WT* table, int V, int H, const int* ids, float* x) {
  const int m = blockIdx.x;
  embed_row<WT>(table, V, H, ids[m], x + (size_t)m * H);
}

template <typename WT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int ldx, const WT* gain, float eps, int H,
                                                      float* out) {
  __shared__ float part[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)m * ldx;
  float s = 0.f;
  if (H % 4 == 0 && ldx % 4 == 0) {              // 16-byte loads and stores
    const int n4 = H / 4;
    for (int i = tid; i < n4; i += 256) {
      const float4 v = *(const float4*)(xr + 4 * i);
      s = fmaf(v.x, v.x, s);
      s = fmaf(v.y, v.y, s);
      s = fmaf(v.z, v.z, s);
      s = fmaf(v.w, v.w, s);
    }
  } else {
    for (int i = tid; i < H; i += 256) s = fmaf(xr[i], xr[i], s);
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  if (H % 4 == 0 && ldx % 4 == 0) {
    const int n4 = H / 4;
    for (int i = tid; i < n4; i += 256) {
      const float4 v = *(const float4*)(xr + 4 * i);
      *(float4*)(out + (size_t)m * H + 4 * i) =
          make_float4(v.x * inv * load_w<WT>(gain + 4 * i), v.y * inv * load_w<WT>(gain + 4 * i + 1),
                      v.z * inv * load_w<WT>(gain + 4 * i + 2), v.w * inv * load_w<WT>(gain + 4 * i + 3));
    }
  } else {
    for (int i = tid; i < H; i += 256) out[(size_t)m * H + i] = xr[i] * inv * load_w<WT>(gain + i);
  }
}

// rmsnorm_kernel's output (bf16 gains, H and ldx multiples of 4) split into bf16 pairs
// hi = bf16(y), lo = bf16(y - hi), 16 bytes per 4 columns: their 4 hi, then their 4 lo.
// V > 0: the row is read once into registers (V float4 per thread, H <= 1024 V); V = 0: a
// second pass re-reads it.  The same sums in the same order either way.
template <int V>
__global__ __launch_bounds__(256) void rmsnorm_pairs_kernel(const float* x, int ldx, const uint16_t* gain, float eps,
                                                            int H, uint16_t* out) {
  __shared__ float part[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)m * ldx;
  const int n4 = H / 4;
  float4 r[V > 0 ? V : 1];
  float s = 0.f;
  if constexpr (V > 0) {
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int i = tid + 256 * k;
      r[k] = i < n4 ? ldg4(xr + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
      if (tid + 256 * k < n4) {
        s = fmaf(r[k].x, r[k].x, s);
        s = fmaf(r[k].y, r[k].y, s);
        s = fmaf(r[k].z, r[k].z, s);
        s = fmaf(r[k].w, r[k].w, s);
      }
    }
  } else {
    for (int i = tid; i < n4; i += 256) {
      const float4 v = *(const float4*)(xr + 4 * i);
      s = fmaf(v.x, v.x, s);
      s = fmaf(v.y, v.y, s);
      s = fmaf(v.z, v.z, s);
      s = fmaf(v.w, v.w, s);
    }
  }
  s = wave_sum(s);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  uint4* o = (uint4*)(out + (size_t)m * 2 * H);
  auto emit = [&](int i, const float4& v) {
    const float y0 = v.x * inv * load_w<uint16_t>(gain + 4 * i), y1 = v.y * inv * load_w<uint16_t>(gain + 4 * i + 1);
    const float y2 = v.z * inv * load_w<uint16_t>(gain + 4 * i + 2), y3 = v.w * inv * load_w<uint16_t>(gain + 4 * i + 3);
    uint32_t h0, l0, h1, l1;
    split_bf2(y0, y1, h0, l0);
    split_bf2(y2, y3, h1, l1);
    o[i] = make_uint4(h0, h1, l0, l1);
  };
  if constexpr (V > 0) {
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (tid + 256 * k < n4) emit(tid + 256 * k, r[k]);
  } else {
    for (int i = tid; i < n4; i += 256) emit(i, *(const float4*)(xr + 4 * i));
  }
}

// Row m = b*T + t of qkv holds token t of sequence b at position start_pos + t.
template <typename WT>
__global__ __launch_bounds__(256) void rope_kv_kernel(const float* qkv, int T, int start_pos, const int* d_pos, int nq,
                                                      int nkv, int hd, const float* rope_cos, const float* rope_sin,
                                                      float* q_out, WT* k_cache, WT* v_cache, int max_seq) {
  const int m = blockIdx.x;
  const int b = m / T, t = m % T, pos = (d_pos ? *d_pos : start_pos) + t;
  const int qr = nq * hd, kr = nkv * hd, half = hd / 2;
  const float* row = qkv + (size_t)m * (qr + 2 * kr);
  for (int i = threadIdx.x; i < (qr + kr) / 2; i += 256) {
    const int n = 2 * i;
    const int d = (n < qr ? n : n - qr) % hd;
    const float c = rope_cos[(size_t)pos * half + d / 2], s = rope_sin[(size_t)pos * half + d / 2];
    float r0 = row[n], r1 = row[n + 1];
    rope_rot(r0, r1, c, s);
    if (n < qr) {
      q_out[(size_t)m * qr + n] = r0;
      q_out[(size_t)m * qr + n + 1] = r1;
    } else {
      const int kvh = (n - qr) / hd;
      WT* dst = k_cache + (((size_t)b * nkv + kvh) * max_seq + pos) * hd + d;
      store_w<WT>(dst, r0);
      store_w<WT>(dst + 1, r1);
    }
  }
  for (int i = threadIdx.x; i < kr; i += 256) {
    const int kvh = i / hd, d = i % hd;
    store_w<WT>(v_cache + (((size_t)b * nkv + kvh) * max_seq + pos) * hd + d, row[qr + kr + i]);
  }
}

__global__ __launch_bounds__(256) void swiglu_kernel(const float* gu, size_t total, int F, float* a) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const size_t m = i / F, n = i % F;
    const float g = gu[m * 2 * F + 2 * n], u = gu[m * 2 * F + 2 * n + 1];
    a[i] = silu(g) * u;
  }
}

__global__ __launch_bounds__(256) void add_kernel(const float* x, const float* y, float* out, size_t n) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) out[i] = x[i] + y[i];
}

// One decode step's prologue: workgroup b embeds token ids_src[b] into x row b;
// workgroup 0 also keeps the ids, sets the position and bumps the step's epoch.
template <typename WT>
__global__ __launch_bounds__(256) void decode_prologue_kernel(const int* ids_src, int* ids_dst, int B, int* d_pos,
                                                              int pos, int* d_epoch, const WT* table, int V, int H,
                                                              float* x) {
  const int b = blockIdx.x;
  if (b == 0) {
    const int i = threadIdx.x;
    if (i < B) ids_dst[i] = ids_src[i];
    if (i == 0) {
      *d_pos = pos;
      if (d_epoch) *d_epoch += 1;
    }
  }
  embed_row<WT>(table, V, H, ids_src[b], x + (size_t)b * H);
}

// Streaming read of n 16-byte vectors, each workgroup a contiguous share, with
// nontemporal loads (the ones the weight streams use): the measured HBM read ceiling of
// the part.  The sum only keeps the loads alive.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n, int iters,
                                                         float* sink) {
  const size_t base = (size_t)blockIdx.x * iters * 1024;
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    uint4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t i = base + ((size_t)it * 4 + k) * 256 + threadIdx.x;
      v[k] = i < n ? ldg4u_nt(p + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += __uint_as_float(v[k].x ^ v[k].y ^ v[k].z ^ v[k].w);
  }
  if (acc == 1.0f) sink[blockIdx.x] = acc;            // practically never
}

__global__ void epoch_bump_kernel(int* d_epoch) {
  if (threadIdx.x == 0) *d_epoch += 1;
}

static unsigned grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  return (unsigned)(g < 1 ? 1 : g);
}

hipError_t launch_embed(int wdtype, const void* table, int V, int H, const int* ids, int M, float* x, hipStream_t s) {
  if (wdtype == W_BF16) hipLaunchKernelGGL(embed_kernel<uint16_t>, dim3(M), dim3(256), 0, s, (const uint16_t*)table, V, H, ids, x);
  else hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, s, (const float*)table, V, H, ids, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int wdtype, const float* x, int ldx, const void* gain, float eps, int M, int H,
                          float* out, hipStream_t s) {
  if (wdtype == W_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, dim3(M), dim3(256), 0, s, x, ldx, (const uint16_t*)gain, eps, H, out);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(M), dim3(256), 0, s, x, ldx, (const float*)gain, eps, H, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_pairs(const float* x, int ldx, const void* gain, float eps, int M, int H, void* out,
                                hipStream_t s) {
  if (M < 1 || H < 4 || H % 4 != 0 || ldx % 4 != 0) return hipErrorInvalidValue;
  if (H <= 8192)
    hipLaunchKernelGGL(rmsnorm_pairs_kernel<8>, dim3(M), dim3(256), 0, s, x, ldx, (const uint16_t*)gain, eps, H,
                       (uint16_t*)out);
  else if (H <= 16384)
    hipLaunchKernelGGL(rmsnorm_pairs_kernel<16>, dim3(M), dim3(256), 0, s, x, ldx, (const uint16_t*)gain, eps, H,
                       (uint16_t*)out);
  else
    hipLaunchKernelGGL(rmsnorm_pairs_kernel<0>, dim3(M), dim3(256), 0, s, x, ldx, (const uint16_t*)gain, eps, H,
                       (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_rope_kv(int wdtype, const float* qkv, int B, int T, int start_pos, const int* d_pos, int nq, int nkv, int hd,
                          const float* rope_cos, const float* rope_sin, float* q_out,
                          void* k_cache, void* v_cache, int max_seq, hipStream_t s) {
  if (wdtype == W_BF16)
    hipLaunchKernelGGL(rope_kv_kernel<uint16_t>, dim3(B * T), dim3(256), 0, s, qkv, T, start_pos, d_pos, nq, nkv, hd,
                       rope_cos, rope_sin, q_out, (uint16_t*)k_cache, (uint16_t*)v_cache, max_seq);
  else
    hipLaunchKernelGGL(rope_kv_kernel<float>, dim3(B * T), dim3(256), 0, s, qkv, T, start_pos, d_pos, nq, nkv, hd,
                       rope_cos, rope_sin, q_out, (float*)k_cache, (float*)v_cache, max_seq);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* gu, int M, int F, float* a, hipStream_t s) {
  const size_t total = (size_t)M * F;
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(total)), dim3(256), 0, s, gu, total, F, a);
  return hipGetLastError();
}

hipError_t launch_epoch_bump(int* d_epoch, hipStream_t s) {
  hipLaunchKernelGGL(epoch_bump_kernel, dim3(1), dim3(64), 0, s, d_epoch);
  return hipGetLastError();
}

hipError_t launch_add(const float* x, const float* y, float* out, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(add_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, y, out, n);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, size_t bytes, int grid, float* sink, hipStream_t s) {
  const size_t n = bytes / 16;
  if (grid < 1 || n == 0) return hipErrorInvalidValue;
  const size_t per = (n + grid - 1) / grid;
  const int iters = (int)((per + 1023) / 1024);
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, s, (const uint4*)buf, n, iters, sink);
  return hipGetLastError();
}

hipError_t launch_decode_prologue(const int* ids_src, int* ids_dst, int B, int* d_pos, int pos, int* d_epoch,
                                  int wdtype, const void* table, int V, int H, float* x, hipStream_t s) {
  if (B < 1 || B > 256) return hipErrorInvalidValue;
  if (wdtype == W_BF16)
    hipLaunchKernelGGL(decode_prologue_kernel<uint16_t>, dim3(B), dim3(256), 0, s, ids_src, ids_dst, B, d_pos, pos,
                       d_epoch, (const uint16_t*)table, V, H, x);
  else
    hipLaunchKernelGGL(decode_prologue_kernel<float>, dim3(B), dim3(256), 0, s, ids_src, ids_dst, B, d_pos, pos,
                       d_epoch, (const float*)table, V, H, x);
  return hipGetLastError();
}

// next[b] = index of the first maximum of x[b][0..V) (one workgroup per row).
__global__ __launch_bounds__(256) void argmax_rows_kernel(const float* x, int V, int ld, int* next) {
  __shared__ float rv[256];
  __shared__ int ri[256];
  const int tid = threadIdx.x, b = blockIdx.x;
  const float* row = x + (size_t)b * ld;
  float best = -INFINITY;
  int idx = INT_MAX;
  for (int i = tid; i < V; i += 256) {
    const float v = row[i];
    if (v > best) { best = v; idx = i; }        // i grows: the first maximum of this thread's entries
  }
  rv[tid] = best;
  ri[tid] = idx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      const float v = rv[tid + o];
      const int i = ri[tid + o];
      if (v > rv[tid] || (v == rv[tid] && i < ri[tid])) { rv[tid] = v; ri[tid] = i; }
    }
    __syncthreads();
  }
  if (tid == 0) next[b] = ri[0] == INT_MAX ? 0 : ri[0];
}

hipError_t launch_argmax_rows(const float* x, int B, int V, int ld, int* next, hipStream_t s) {
  if (!x || !next || B < 1 || V < 1 || ld < V) return hipErrorInvalidValue;
  launch_timed(argmax_rows_kernel, dim3(B), dim3(256), 0, s, x, V, ld, next);
  return hipGetLastError();
}

}  // namespace ladder

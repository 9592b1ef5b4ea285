// Grouped-query causal softmax attention over the KV cache.
//
// Decode (one new token per sequence): the keys 0..pos of one (sequence, kv head)
// are split into n_split contiguous chunks, one workgroup each.  A workgroup stages
// 64-key tiles of K and V in LDS once and serves all G = nq/nkv query heads that
// share that kv head (the GQA map: query head h reads kv head h / G), keeping a
// running max / sum / accumulator per head (online softmax).  The last workgroup of
// a (sequence, kv head) merges the chunks with their log-sum-exp weights, in chunk
// order, so results do not depend on scheduling.
//
// Prefill (T tokens per sequence starting at start_pos): one workgroup per 32-query
// tile of one head walks the causally visible 64-key tiles with the same online
// softmax.
#include "common.hpp"
#include "kernels.h"

namespace ladder {

constexpr int kKeyTile = 64;
constexpr int kMaxGroup = 16;

template <typename WT, int HD>
__device__ __forceinline__ void stage_rows(float (*dst)[HD + 4], const WT* src, int n_rows, int tid) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int VPR = HD / VEC;                       // 16-byte vectors per row
  for (int i = tid; i < kKeyTile * VPR; i += 256) {
    const int r = i / VPR, c = (i % VPR) * VEC;
    float f[VEC];
    if (r < n_rows) {
      unpack16(*(const uint4*)(src + (size_t)r * HD + c), f);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[r][c + e] = f[e];
  }
}

template <typename WT, int HD>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeParams p) {
  __shared__ float qs[kMaxGroup][HD];
  __shared__ float ks[kKeyTile][HD + 4];
  __shared__ float vs[kKeyTile][HD + 4];
  __shared__ float ps[kMaxGroup][kKeyTile];
  __shared__ float alpha[kMaxGroup];
  __shared__ float m_run[kMaxGroup];
  __shared__ float l_run[kMaxGroup];
  __shared__ int is_last;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.nq / p.nkv;
  const int len = *p.d_pos + 1;
  const int chunk = (len + p.n_split - 1) / p.n_split;
  const int start = s * chunk;
  const int end = min(len, start + chunk);
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t kv_base = ((size_t)b * p.nkv + kvh) * p.max_seq * HD;
  const WT* kc = (const WT*)p.k_cache + kv_base;
  const WT* vc = (const WT*)p.v_cache + kv_base;

  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i % HD;
    qs[h][d] = p.q[(size_t)b * p.nq * HD + (size_t)(kvh * G + h) * HD + d];
  }
  if (tid < G) { m_run[tid] = -INFINITY; l_run[tid] = 0.f; }
  constexpr int kMaxOwn = kMaxGroup * HD / 256;
  float acc[kMaxOwn];
#pragma unroll
  for (int k = 0; k < kMaxOwn; ++k) acc[k] = 0.f;
  __syncthreads();

  for (int t0 = start; t0 < end; t0 += kKeyTile) {
    const int n = min(kKeyTile, end - t0);
    stage_rows<WT, HD>(ks, kc + (size_t)t0 * HD, n, tid);
    stage_rows<WT, HD>(vs, vc + (size_t)t0 * HD, n, tid);
    __syncthreads();
    for (int i = tid; i < G * kKeyTile; i += 256) {
      const int h = i / kKeyTile, j = i % kKeyTile;
      float dot = 0.f;
      if (j < n) {
#pragma unroll 8
        for (int d = 0; d < HD; ++d) dot = fmaf(qs[h][d], ks[j][d], dot);
        ps[h][j] = dot * scale;
      } else {
        ps[h][j] = -INFINITY;
      }
    }
    __syncthreads();
    for (int h = wid; h < G; h += 4) {
      const float sc = ps[h][lane];
      const float m_new = fmaxf(m_run[h], wave_max(sc));
      const float e = lane < n ? expf(sc - m_new) : 0.f;
      const float sum = wave_sum(e);
      ps[h][lane] = e;
      if (lane == 0) {
        const float a = expf(m_run[h] - m_new);
        alpha[h] = a;
        l_run[h] = l_run[h] * a + sum;
        m_run[h] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxOwn; ++k) {
      const int i = tid + k * 256;
      if (i < G * HD) {
        const int h = i / HD, d = i % HD;
        float a = acc[k] * alpha[h];
        for (int j = 0; j < n; ++j) a = fmaf(ps[h][j], vs[j][d], a);
        acc[k] = a;
      }
    }
    __syncthreads();
  }

  // this chunk's (max, sum, unnormalised accumulator) per query head
  const size_t stride = HD + 2;
#pragma unroll
  for (int k = 0; k < kMaxOwn; ++k) {
    const int i = tid + k * 256;
    if (i < G * HD) {
      const int h = i / HD, d = i % HD;
      float* dst = p.part + (((size_t)b * p.nq + kvh * G + h) * p.n_split + s) * stride;
      dst[2 + d] = acc[k];
      if (d == 0) { dst[0] = m_run[h]; dst[1] = l_run[h]; }
    }
  }
  __threadfence();
  __syncthreads();
  int* counter = p.counters + (size_t)b * p.nkv + kvh;
  if (tid == 0) is_last = (atomicAdd(counter, 1) == p.n_split - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i % HD;
    const float* src = p.part + (((size_t)b * p.nq + kvh * G + h) * p.n_split) * stride;
    float M = -INFINITY;
    for (int q = 0; q < p.n_split; ++q) M = fmaxf(M, src[q * stride]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
      for (int q = 0; q < p.n_split; ++q) {
        const float w = expf(src[q * stride] - M);
        L = fmaf(src[q * stride + 1], w, L);
        o = fmaf(src[q * stride + 2 + d], w, o);
      }
    }
    p.out[(size_t)b * p.nq * HD + (size_t)(kvh * G + h) * HD + d] = L > 0.f ? o / L : 0.f;
  }
  if (tid == 0) *counter = 0;
}

int attn_decode_splits(int max_seq) {
  int n = (max_seq + kKeyTile - 1) / kKeyTile;
  if (n < 1) n = 1;
  if (n > 32) n = 32;
  return n;
}

hipError_t launch_attn_decode(const AttnDecodeParams& p, hipStream_t s) {
  if (p.nkv < 1 || p.nq % p.nkv != 0 || p.nq / p.nkv > kMaxGroup) return hipErrorInvalidValue;
  dim3 grid(p.n_split, p.nkv, p.B);
  if (p.hd == 128) {
    if (p.wdtype == W_BF16) hipLaunchKernelGGL((attn_decode_kernel<uint16_t, 128>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_decode_kernel<float, 128>), grid, dim3(256), 0, s, p);
  } else if (p.hd == 64) {
    if (p.wdtype == W_BF16) hipLaunchKernelGGL((attn_decode_kernel<uint16_t, 64>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_decode_kernel<float, 64>), grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ prefill

constexpr int kQTile = 32;

template <typename WT, int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnPrefillParams p) {
  __shared__ float qs[kQTile][HD + 4];
  __shared__ float ks[kKeyTile][HD + 4];
  __shared__ float vs[kKeyTile][HD + 4];
  __shared__ float ss[kQTile][kKeyTile + 1];

  const int tid = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = p.nq / p.nkv, kvh = h / G;
  const int qi = tid >> 3, sub = tid & 7;          // 8 threads per query row
  const int t = qt * kQTile + qi;                  // token index within the chunk
  const bool qvalid = t < p.T;
  const int qpos = p.start_pos + t;
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t kv_base = ((size_t)b * p.nkv + kvh) * p.max_seq * HD;
  const WT* kc = (const WT*)p.k_cache + kv_base;
  const WT* vc = (const WT*)p.v_cache + kv_base;
  const size_t qld = (size_t)p.nq * HD;

  for (int i = tid; i < kQTile * HD; i += 256) {
    const int r = i / HD, d = i % HD;
    const int tt = qt * kQTile + r;
    qs[r][d] = tt < p.T ? p.q[((size_t)b * p.T + tt) * qld + (size_t)h * HD + d] : 0.f;
  }
  constexpr int DPT = HD / 8;                      // output dims per thread
  float acc[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) acc[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int last_t = min(p.T, (qt + 1) * kQTile) - 1;
  const int n_keys = p.start_pos + last_t + 1;     // keys visible to the last query of the tile
  for (int k0 = 0; k0 < n_keys; k0 += kKeyTile) {
    const int n = min(kKeyTile, n_keys - k0);
    __syncthreads();
    stage_rows<WT, HD>(ks, kc + (size_t)k0 * HD, n, tid);
    stage_rows<WT, HD>(vs, vc + (size_t)k0 * HD, n, tid);
    __syncthreads();
    float sc[kKeyTile / 8];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kKeyTile / 8; ++k) {
      const int j = sub + 8 * k;
      const int kp = k0 + j;
      float dot = -INFINITY;
      if (j < n && kp <= qpos) {
        float a = 0.f;
#pragma unroll 8
        for (int d = 0; d < HD; ++d) a = fmaf(qs[qi][d], ks[j][d], a);
        dot = a * scale;
      }
      sc[k] = dot;
      mx = fmaxf(mx, dot);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    const float m_new = fmaxf(m_run, mx);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kKeyTile / 8; ++k) {
      const float e = sc[k] == -INFINITY ? 0.f : expf(sc[k] - m_new);
      ss[qi][sub + 8 * k] = e;
      sum += e;
    }
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    sum += __shfl_xor(sum, 4, 64);
    const float a = m_new == -INFINITY ? 0.f : expf(m_run - m_new);
    l_run = l_run * a + sum;
    m_run = m_new;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < DPT; ++k) acc[k] *= a;
    for (int j = 0; j < n; ++j) {
      const float pj = ss[qi][j];
#pragma unroll
      for (int k = 0; k < DPT; ++k) acc[k] = fmaf(pj, vs[j][sub * DPT + k], acc[k]);
    }
  }
  if (!qvalid) return;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  const size_t o = ((size_t)b * p.T + t) * qld + (size_t)h * HD + sub * DPT;
  if (p.out_bf16) {
    uint16_t* dst = (uint16_t*)p.out + o;
#pragma unroll
    for (int k = 0; k < DPT; ++k) dst[k] = f32_to_bf16(acc[k] * inv);
  } else {
    float* dst = (float*)p.out + o;
#pragma unroll
    for (int k = 0; k < DPT; ++k) dst[k] = acc[k] * inv;
  }
}

hipError_t launch_attn_prefill(const AttnPrefillParams& p, hipStream_t s) {
  if (p.nkv < 1 || p.nq % p.nkv != 0) return hipErrorInvalidValue;
  dim3 grid((p.T + kQTile - 1) / kQTile, p.nq, p.B);
  if (p.hd == 128) {
    if (p.wdtype == W_BF16) hipLaunchKernelGGL((attn_prefill_kernel<uint16_t, 128>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_prefill_kernel<float, 128>), grid, dim3(256), 0, s, p);
  } else if (p.hd == 64) {
    if (p.wdtype == W_BF16) hipLaunchKernelGGL((attn_prefill_kernel<uint16_t, 64>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_prefill_kernel<float, 64>), grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ladder

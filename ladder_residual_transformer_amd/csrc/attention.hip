// Grouped-query causal softmax attention over the KV cache.
//
// Decode (one new token per sequence): split-KV workgroups of attn_decode.hpp.
//
// Prefill (T tokens per sequence starting at start_pos): one workgroup per 32-query
// tile of one head walks the causally visible 64-key tiles with the same online
// softmax.
#include "attn_decode.hpp"
#include "common.hpp"
#include "kernels.h"

namespace ladder {

constexpr int kKeyTile = 64;      // prefill key tile

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

template <typename WT, int HD, int HPW>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeParams p) {
  __shared__ AttnLds<WT, HD> L;
  attn_decode_block<WT, HD, HPW>(p, blockIdx.x, L);
}

// Chunks per (sequence, kv head): one 64-key tile each at full length, at most 16 (the
// merge then reads every chunk of a head slice in one round of loads).
int attn_decode_splits(int max_seq) {
  int n = (max_seq + kAttnKeyTile - 1) / kAttnKeyTile;
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  return n;
}

template <typename WT, int HD>
hipError_t attn_decode_go(const AttnDecodeParams& p, hipStream_t s) {
  dim3 grid(p.n_split * p.nkv * p.B);
  switch (attn_hpw(p.nq / p.nkv)) {
    case 1: hipLaunchKernelGGL((attn_decode_kernel<WT, HD, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((attn_decode_kernel<WT, HD, 2>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((attn_decode_kernel<WT, HD, 4>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnDecodeParams& p, hipStream_t s) {
  if (p.nkv < 1 || p.nq % p.nkv != 0 || p.nq / p.nkv > kAttnMaxGroup || p.n_split > kAttnMaxSplits)
    return hipErrorInvalidValue;
  if (p.hd == 128) return p.wdtype == W_BF16 ? attn_decode_go<uint16_t, 128>(p, s) : attn_decode_go<float, 128>(p, s);
  if (p.hd == 64) return p.wdtype == W_BF16 ? attn_decode_go<uint16_t, 64>(p, s) : attn_decode_go<float, 64>(p, s);
  return hipErrorInvalidValue;
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

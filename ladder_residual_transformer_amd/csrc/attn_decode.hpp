// One workgroup of split-KV grouped-query decode attention (device code shared by the
// stand-alone attention kernel and the fused attention + down-projection kernel).
//
// Workgroup (s, kvh, b) owns keys [s*chunk, min(len, (s+1)*chunk)) of kv head kvh of
// sequence b, with len = pos + 1.  Keys are processed in 64-key tiles; the K and V
// rows of the next tile are loaded into registers while the current one is used, so
// a chunk of one tile costs a single memory round trip.  A tile sits in LDS in its
// stored type with an odd row stride in dwords, so lane j can read row j without bank
// conflicts.
//
// Each wave works on its own query heads (wave w owns heads w, w+4, ...; all G =
// nq/nkv heads share the kv head, query head h reading kv head h / G).  For a tile the
// wave scores key j in lane j, updates the heads' running max and sum (online
// softmax), and then accumulates P.V with lane l owning output dimensions
// l*DPL .. l*DPL+DPL-1, taking key j's weight from lane j with a lane broadcast.  Every
// loop bound is a compile-time constant (heads per wave HPW is a template parameter;
// missing heads compute on a clamped index and are not stored), so the loops stay
// branch-free.  Each workgroup writes its (max, sum, accumulator); the last workgroup
// of a (sequence, kv head), found with an atomic ticket, merges the chunks in chunk
// order with their log-sum-exp weights, so the result does not depend on scheduling.
#pragma once
#include "common.hpp"
#include "kernels.h"

namespace ladder {

constexpr int kAttnKeyTile = 64;
constexpr int kAttnMaxGroup = 16;
constexpr int kAttnMaxSplits = 32;

template <typename WT, int HD>
struct AttnLds {
  static constexpr int RW = HD * (int)sizeof(WT) / 4 + 1;   // dwords per staged row (odd)
  __attribute__((aligned(16))) float qs[kAttnMaxGroup][HD];
  uint32_t ks[kAttnKeyTile][RW];
  uint32_t vs[kAttnKeyTile][RW];
  float wsc[kAttnMaxGroup][kAttnMaxSplits];
  float lsc[kAttnMaxGroup][kAttnMaxSplits];
  float linv[kAttnMaxGroup];
  int is_last;
};

// element e of a staged row
template <typename WT> __device__ __forceinline__ float attn_elem(const uint32_t* row, int e);
template <> __device__ __forceinline__ float attn_elem<uint16_t>(const uint32_t* row, int e) {
  const uint32_t w = row[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}
template <> __device__ __forceinline__ float attn_elem<float>(const uint32_t* row, int e) {
  return __uint_as_float(row[e]);
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Heads per wave for a group of G query heads per kv head.
__host__ __device__ constexpr int attn_hpw(int G) { return G <= 4 ? 1 : (G <= 8 ? 2 : 4); }

// Requires blockDim.x == 256 and G <= 4 * HPW.  `blk` enumerates (s, kvh, b), s fastest.
template <typename WT, int HD, int HPW>
__device__ void attn_decode_block(const AttnDecodeParams& p, int blk, AttnLds<WT, HD>& L) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int VPR = HD / VEC;                          // 16-byte vectors per row
  constexpr int VPT = kAttnKeyTile * VPR / 256;          // per thread per tile, K and V each
  constexpr int DPL = HD / 64;                           // output dims per lane
  static_assert(VPT >= 1 && kAttnKeyTile * VPR % 256 == 0 && HD % 64 == 0, "tile shape");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blk % p.n_split;
  const int kvh = (blk / p.n_split) % p.nkv;
  const int b = blk / (p.n_split * p.nkv);
  const int G = p.nq / p.nkv;
  const int len = *p.d_pos + 1;
  const int chunk = (len + p.n_split - 1) / p.n_split;
  const int start = s * chunk;
  const int end = min(len, start + chunk);
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t kv_base = ((size_t)b * p.nkv + kvh) * p.max_seq * HD;
  const WT* kc = (const WT*)p.k_cache + kv_base;
  const WT* vc = (const WT*)p.v_cache + kv_base;

  uint4 kr[VPT], vr[VPT];
  // unconditional loads: rows past the chunk end repeat its last key (never used)
  auto load_tile = [&](int t0) {
    const int last = end - 1 - t0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + 256 * i, r = min(idx / VPR, last), c = (idx % VPR) * VEC;
      kr[i] = *(const uint4*)(kc + (size_t)(t0 + r) * HD + c);
      vr[i] = *(const uint4*)(vc + (size_t)(t0 + r) * HD + c);
    }
  };
  if (start < end) load_tile(start);
  for (int i = tid; i < G * HD; i += 256) {
    const int h = i / HD, d = i % HD;
    L.qs[h][d] = p.q[(size_t)b * p.nq * HD + (size_t)(kvh * G + h) * HD + d];
  }

  int hc[HPW];                                           // this wave's heads, clamped to G-1
#pragma unroll
  for (int k = 0; k < HPW; ++k) hc[k] = min(wid + 4 * k, G - 1);
  float m_run[HPW], l_run[HPW], acc[HPW][DPL];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[k][e] = 0.f;
  }

  for (int t0 = start; t0 < end; t0 += kAttnKeyTile) {
    const int n = min(kAttnKeyTile, end - t0);
    if (t0 > start) __syncthreads();                     // previous tile fully consumed
    // registers -> LDS (4 dwords per 16-byte vector; odd row stride keeps rows apart)
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + 256 * i, r = idx / VPR, cw = (idx % VPR) * 4;
      L.ks[r][cw] = kr[i].x; L.ks[r][cw + 1] = kr[i].y; L.ks[r][cw + 2] = kr[i].z; L.ks[r][cw + 3] = kr[i].w;
      L.vs[r][cw] = vr[i].x; L.vs[r][cw + 1] = vr[i].y; L.vs[r][cw + 2] = vr[i].z; L.vs[r][cw + 3] = vr[i].w;
    }
    __syncthreads();
    if (t0 + kAttnKeyTile < end) load_tile(t0 + kAttnKeyTile);     // next tile in flight

    // scores: lane = key
    float sc[HPW];
#pragma unroll
    for (int k = 0; k < HPW; ++k) sc[k] = 0.f;
    const uint32_t* krow = L.ks[lane];
#pragma unroll
    for (int d = 0; d < HD; d += 4) {               // 4 dims per step: one 16-byte q read per head
      float kv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[e] = attn_elem<WT>(krow, d + e);
#pragma unroll
      for (int k = 0; k < HPW; ++k) {
        const float4 q4 = *reinterpret_cast<const float4*>(&L.qs[hc[k]][d]);
        sc[k] = fmaf(q4.x, kv[0], sc[k]);
        sc[k] = fmaf(q4.y, kv[1], sc[k]);
        sc[k] = fmaf(q4.z, kv[2], sc[k]);
        sc[k] = fmaf(q4.w, kv[3], sc[k]);
      }
    }
    // online softmax per head, then P.V with lane = output dims
    float pj[HPW];
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
      const float sv = lane < n ? sc[k] * scale : -INFINITY;
      const float m_new = fmaxf(m_run[k], wave_max(sv));
      pj[k] = lane < n ? expf(sv - m_new) : 0.f;
      const float a = expf(m_run[k] - m_new);
      l_run[k] = l_run[k] * a + wave_sum(pj[k]);
      m_run[k] = m_new;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[k][e] *= a;
    }
#pragma unroll 4
    for (int j = 0; j < n; ++j) {
      float v[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[e] = attn_elem<WT>(L.vs[j], lane * DPL + e);
#pragma unroll
      for (int k = 0; k < HPW; ++k) {
        const float w = lane_bcast(pj[k], j);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[k][e] = fmaf(w, v[e], acc[k][e]);
      }
    }
  }

  // this chunk's (max, sum, unnormalised accumulator) per query head; records of HD + 4
  // floats: max, sum, two unused, then the accumulator 16-byte aligned
  const size_t stride = HD + 4;
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = wid + 4 * k;
    if (h < G) {
      float* dst = p.part + (((size_t)b * p.nq + kvh * G + h) * p.n_split + s) * stride;
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[4 + lane * DPL + e] = acc[k][e];
      if (lane == 0) { dst[0] = m_run[k]; dst[1] = l_run[k]; }
    }
  }
  __threadfence();
  __syncthreads();
  int* counter = p.counters + (size_t)b * p.nkv + kvh;
  if (tid == 0) L.is_last = (atomicAdd(counter, 1) == p.n_split - 1);
  __syncthreads();
  if (!L.is_last) return;
  __threadfence();
  // merge: per head M = max_s m_s, w_s = e^{m_s - M}, L = sum_s l_s w_s,
  // o[d] = sum_s acc_s[d] w_s / L, summed in chunk order
  const float* base = p.part + ((size_t)b * p.nq + kvh * G) * p.n_split * stride;
  for (int i = tid; i < G * p.n_split; i += 256) {
    const int h = i / p.n_split, q = i % p.n_split;
    const float* src = base + ((size_t)h * p.n_split + q) * stride;
    L.wsc[h][q] = src[0];
    L.lsc[h][q] = src[1];
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int q = 0; q < p.n_split; ++q) M = fmaxf(M, L.wsc[tid][q]);
    float Ls = 0.f;
    for (int q = 0; q < p.n_split; ++q) {
      const float w = M == -INFINITY ? 0.f : expf(L.wsc[tid][q] - M);
      L.wsc[tid][q] = w;
      Ls = fmaf(L.lsc[tid][q], w, Ls);
    }
    L.linv[tid] = Ls > 0.f ? 1.0f / Ls : 0.f;
  }
  __syncthreads();
  // one thread per (head, 4 dims); all of a group's 16 chunk loads are issued together
  constexpr int QG = 16;
  for (int i = tid; i < G * (HD / 4); i += 256) {
    const int h = i / (HD / 4), d4 = (i % (HD / 4)) * 4;
    const float* src = base + (size_t)h * p.n_split * stride + 4 + d4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < p.n_split; q0 += QG) {
      float4 a[QG];
#pragma unroll
      for (int q = 0; q < QG; ++q) a[q] = *(const float4*)(src + (size_t)min(q0 + q, p.n_split - 1) * stride);
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        const float w = q0 + q < p.n_split ? L.wsc[h][q0 + q] : 0.f;
        o.x = fmaf(a[q].x, w, o.x);
        o.y = fmaf(a[q].y, w, o.y);
        o.z = fmaf(a[q].z, w, o.z);
        o.w = fmaf(a[q].w, w, o.w);
      }
    }
    const float li = L.linv[h];
    *(float4*)(p.out + (size_t)b * p.nq * HD + (size_t)(kvh * G + h) * HD + d4) =
        make_float4(o.x * li, o.y * li, o.z * li, o.w * li);
  }
  if (tid == 0) *counter = 0;
}

}  // namespace ladder

// Grouped-query causal softmax attention over the KV cache.
//
// Decode (one new token per sequence): split-KV workgroups of attn_decode.hpp.
//
// Prefill (T tokens per sequence starting at start_pos), causal, online softmax:
//   bf16 models: matrix cores.  A workgroup owns 128 queries of one head, a wave 32 of
//     them; S^T = K.Q^T and O^T += V^T.P^T run as v_mfma_f32_32x32x16_f16 with the
//     stored bf16 K/V converted exactly to fp16 in LDS, and q and the probabilities p
//     each carried as an fp16 pair (hi + lo, about 22 significant bits, two MFMAs per
//     product); fp32 accumulation and fp32 softmax statistics.
//   fp32 models: a VALU kernel, one workgroup per 32-query tile of one head.
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

// Key chunks per sequence and kv head: one 64-key tile each up to 16 chunks (beyond 16,
// the merge's inputs cost more than the shorter chunks save on the 70B shard's decode).
int attn_decode_splits(int max_seq) {
  int n = (max_seq + kAttnKeyTile - 1) / kAttnKeyTile;
  if (n < 1) n = 1;
  if (n > kAttnDefaultSplits) n = kAttnDefaultSplits;
  return n;
}

template <typename WT, int HD>
hipError_t attn_decode_go(const AttnDecodeParams& p, hipStream_t s) {
  dim3 grid(p.n_split * p.nkv * p.B);
  switch (attn_hpw(p.nq / p.nkv)) {
    case 1: launch_timed(attn_decode_kernel<WT, HD, 1>, grid, dim3(256), 0, s, p); break;
    case 2: launch_timed(attn_decode_kernel<WT, HD, 2>, grid, dim3(256), 0, s, p); break;
    default: launch_timed(attn_decode_kernel<WT, HD, 4>, grid, dim3(256), 0, s, p); break;
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
  float* dst = p.out + o;
#pragma unroll
  for (int k = 0; k < DPT; ++k) dst[k] = acc[k] * inv;
}


// ------------------------------------------------- prefill, bf16 models (MFMA)

constexpr int kPqWave = 32;                  // queries per wave
constexpr int kPqTile = 4 * kPqWave;         // queries per workgroup
constexpr int kPkTile = 64;                  // keys per LDS tile

template <int HD>
struct PrefillLds {
  uint16_t ks[kPkTile][HD + 8];     // K tile, row = key (fp16)
  uint16_t vt[HD][kPkTile + 8];     // V tile transposed, row = head dim (fp16), keys at vt_col
};
static_assert(kPkTile == kAttnKeyTile, "vt_col permutes the 16 key groups of a 64-key row");

// MFMA 32x32x16 operand/result layout (lane l): A row l%32, B column l%32, k-slots
// 8*(l/32)..+8; C column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for result r = 0..15.
template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_mfma_kernel(AttnPrefillParams p) {
  __shared__ __attribute__((aligned(16))) PrefillLds<HD> L;
  constexpr int NST = HD / 16;               // 16-dim steps of S = K.Q^T
  constexpr int NDB = HD / 32;               // 32-dim blocks of O^T
  constexpr int CPR = HD / 8;                // 16-byte chunks per K/V row
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int n_qt = (p.T + kPqTile - 1) / kPqTile;
  const int NC = p.nchunk;                     // key chunks per query tile (1: no split)
  const int qt = n_qt - 1 - (int)blockIdx.x / NC;   // longest causal ranges first
  const int chunk = (int)blockIdx.x % NC;
  const int h = blockIdx.y, b = blockIdx.z;
  const int G = p.nq / p.nkv, kvh = h / G;
  const size_t kv_base = ((size_t)b * p.nkv + kvh) * p.max_seq * HD;
  const uint16_t* kc = (const uint16_t*)p.k_cache + kv_base;
  const uint16_t* vc = (const uint16_t*)p.v_cache + kv_base;
  const size_t qld = (size_t)p.nq * HD;

  // this lane's query (column of S^T); rows past T reuse the last valid token so every
  // key they touch is written, and write nothing
  const int t_raw = qt * kPqTile + w * kPqWave + col;
  const int t_q = t_raw < p.T ? t_raw : p.T - 1;
  const int qpos = p.start_pos + t_q;
  const int wave_last = p.start_pos + min(p.T - 1, qt * kPqTile + w * kPqWave + kPqWave - 1);
  const int n_keys = p.start_pos + min(p.T, (qt + 1) * kPqTile);   // keys of the query tile
  // this workgroup's keys [k_lo, k_hi): all of them, or one chunk of them
  const int k_lo = NC > 1 ? chunk * p.kchunk : 0;
  if (k_lo >= n_keys) return;                  // whole workgroup: the tile has fewer chunks
  const int k_hi = NC > 1 ? min(n_keys, k_lo + p.kchunk) : n_keys;
  const int tile_chunks = NC > 1 ? (n_keys + p.kchunk - 1) / p.kchunk : 1;
  const int n_kt = (k_hi - k_lo + kPkTile - 1) / kPkTile;

  // Q^T operand as fp16 pairs: step s holds dims 16s + 8*half .. +8 of this lane's query
  half8 qh[NST], ql[NST];
  {
    const float* qrow = p.q + ((size_t)b * p.T + t_q) * qld + (size_t)h * HD;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const float4 a = *(const float4*)(qrow + 16 * s + 8 * half);
      const float4 c = *(const float4*)(qrow + 16 * s + 8 * half + 4);
      uint4 hi, lo;
      split_h2(a.x, a.y, hi.x, lo.x);
      split_h2(a.z, a.w, hi.y, lo.y);
      split_h2(c.x, c.y, hi.z, lo.z);
      split_h2(c.z, c.w, hi.w, lo.w);
      qh[s] = __builtin_bit_cast(half8, hi);
      ql[s] = __builtin_bit_cast(half8, lo);
    }
  }

  // K/V tile loads: thread moves K chunks (row, c) and V chunk pairs (rows 2j, 2j+1)
  constexpr int KCH = kPkTile * CPR / 256;          // K chunks per thread
  constexpr int VPAIR = (kPkTile / 2) * CPR / 256;  // V row pairs per thread
  uint4 kr[KCH], vr[VPAIR][2];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + 256 * i, r = e / CPR, c = e % CPR;
      const int kp = k0 + r;
      kr[i] = kp < k_hi ? *(const uint4*)(kc + (size_t)kp * HD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < VPAIR; ++i) {
      const int e = tid + 256 * i, j = e / CPR, c = e % CPR;
      const int kp = k0 + 2 * j;
      vr[i][0] = kp < k_hi ? *(const uint4*)(vc + (size_t)kp * HD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
      vr[i][1] = kp + 1 < k_hi ? *(const uint4*)(vc + (size_t)(kp + 1) * HD + c * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + 256 * i, r = e / CPR, c = e % CPR;
      *(uint4*)&L.ks[r][c * 8] = bf16x8_to_f16x8(kr[i]);
    }
#pragma unroll
    for (int i = 0; i < VPAIR; ++i) {
      const int e = tid + 256 * i, j = e / CPR, c = e % CPR;
      const uint32_t* v0 = (const uint32_t*)&vr[i][0];
      const uint32_t* v1 = (const uint32_t*)&vr[i][1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *(uint32_t*)&L.vt[c * 8 + 2 * q][vt_col(c * 8, 2 * j)] = pack_h2(bf16_lo(v0[q]), bf16_lo(v1[q]));
        *(uint32_t*)&L.vt[c * 8 + 2 * q + 1][vt_col(c * 8, 2 * j)] = pack_h2(bf16_hi(v0[q]), bf16_hi(v1[q]));
      }
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  const float c2 = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(hd)
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(k_lo);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = k_lo + kt * kPkTile;
    __syncthreads();                 // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(k0 + kPkTile);
    if (k0 > wave_last) continue;    // no visible key for this wave (uniform)

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const half8 a = *(const half8*)&L.ks[kb * 32 + col][16 * st + 8 * half];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, ql[st], s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qh[st], s[kb], 0, 0, 0);
      }
    }
    // causal mask, running max over this lane's 32 keys and its partner lane's 32
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kp = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (kp > qpos) s[kb][r] = -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // finite from the first tile on without a split (key 0 is visible to every query); a
    // later key chunk may hold no visible key yet for this lane's query
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f((m_run - m_new) * c2);
    m_run = m_new;
    const float mc = m_new == -INFINITY ? 0.f : m_new * c2;
    float ls = 0.f;
    uint32_t ph[2][8], pl[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = exp2f(fmaf(s[kb][r], c2, -mc));
        const float e1 = exp2f(fmaf(s[kb][r + 1], c2, -mc));
        ls += e0 + e1;
        split_h2(e0, e1, ph[kb][r >> 1], pl[kb][r >> 1]);
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    // O^T += V^T . P^T over 16-key steps; step t of block kb takes this lane's results
    // 8*(t&1) .. +8, i.e. keys 16*t' + 4*half + {0..3, 8..11} with t' = 2*kb + (t&1)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, sub = t & 1;
      const half8 pfh = __builtin_bit_cast(half8, make_uint4(ph[kb][4 * sub], ph[kb][4 * sub + 1],
                                                             ph[kb][4 * sub + 2], ph[kb][4 * sub + 3]));
      const half8 pfl = __builtin_bit_cast(half8, make_uint4(pl[kb][4 * sub], pl[kb][4 * sub + 1],
                                                             pl[kb][4 * sub + 2], pl[kb][4 * sub + 3]));
      const int kbase = 16 * t + 4 * half;
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const uint16_t* vrow = &L.vt[d * 32 + col][0];
        const uint2 lo = *(const uint2*)(vrow + vt_col(d * 32 + col, kbase));
        const uint2 hi = *(const uint2*)(vrow + vt_col(d * 32 + col, kbase + 8));
        const half8 vf = __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pfl, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pfh, o[d], 0, 0, 0);
      }
    }
  }
  l_run += __shfl_xor(l_run, 32, 64);
  if (t_raw >= p.T) return;
  if (tile_chunks > 1) {
    // chunk record: max (raw score units), sum, two unused, unnormalized accumulator
    float* rec = p.part + ((((size_t)b * p.nq + h) * p.T + t_raw) * NC + chunk) * (HD + 4);
    if (half == 0) {
      rec[0] = m_run;
      rec[1] = l_run;
    }
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = d * 32 + 8 * g + 4 * half;
        *(float4*)(rec + 4 + dim) = make_float4(o[d][4 * g], o[d][4 * g + 1], o[d][4 * g + 2], o[d][4 * g + 3]);
      }
    return;
  }
  const float inv = 1.0f / l_run;
  float* dst = p.out + ((size_t)b * p.T + t_raw) * qld + (size_t)h * HD;
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = d * 32 + 8 * g + 4 * half;
      *(float4*)(dst + dim) = make_float4(o[d][4 * g] * inv, o[d][4 * g + 1] * inv,
                                          o[d][4 * g + 2] * inv, o[d][4 * g + 3] * inv);
    }
}

// Combines the chunk records of the query tiles that were split: per (sequence, head,
// query) M = max_c m_c, w_c = 2^((m_c - M) log2(e)/sqrt(hd)), out = sum_c w_c acc_c /
// sum_c w_c l_c, in chunk order.  One thread per 4 output dimensions.
template <int HD>
__global__ __launch_bounds__(256) void attn_prefill_merge_kernel(AttnPrefillParams p) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int e = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int t = e / (HD / 4), d4 = (e % (HD / 4)) * 4;
  if (t >= p.T) return;
  const int qt = t / kPqTile;
  const int n_keys = p.start_pos + min(p.T, (qt + 1) * kPqTile);
  const int nc = (n_keys + p.kchunk - 1) / p.kchunk;
  if (nc <= 1) return;                         // written by its only workgroup
  const float c2 = 1.4426950408889634f / sqrtf((float)HD);
  const float* rec = p.part + (((size_t)b * p.nq + h) * p.T + t) * p.nchunk * (HD + 4);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, rec[(size_t)c * (HD + 4)]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < nc; ++c) {
    const float* r = rec + (size_t)c * (HD + 4);
    const float w = r[0] == -INFINITY ? 0.f : exp2f((r[0] - M) * c2);
    L = fmaf(r[1], w, L);
    const float4 a = *(const float4*)(r + 4 + d4);
    acc.x = fmaf(a.x, w, acc.x);
    acc.y = fmaf(a.y, w, acc.y);
    acc.z = fmaf(a.z, w, acc.z);
    acc.w = fmaf(a.w, w, acc.w);
  }
  const float inv = 1.0f / L;
  float* dst = p.out + ((size_t)b * p.T + t) * ((size_t)p.nq * HD) + (size_t)h * HD + d4;
  *(float4*)dst = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

hipError_t launch_attn_prefill(const AttnPrefillParams& p_in, hipStream_t s) {
  AttnPrefillParams p = p_in;
  if (p.nkv < 1 || p.nq % p.nkv != 0 || p.T < 1) return hipErrorInvalidValue;
  if (p.wdtype == W_BF16) {
    if (p.hd != 128 && p.hd != 64) return hipErrorInvalidValue;
    // few query tiles (one prompt of ~1k tokens: 8 tiles per head): cut each tile's keys
    // into at most kAttnPrefillMaxChunks chunks of >= 256 keys, so that the longest causal
    // range no longer sets the launch's duration alone
    const int n_qt = (p.T + kPqTile - 1) / kPqTile;
    p.nchunk = 1;
    p.kchunk = 0;
    if (p.part && (long long)n_qt * p.nq * p.B < 256) {
      const int n_keys_max = p.start_pos + p.T;
      int ck = (n_keys_max + kAttnPrefillMaxChunks - 1) / kAttnPrefillMaxChunks;
      ck = (ck + kPkTile - 1) / kPkTile * kPkTile;
      if (ck < 256) ck = 256;
      const int nc = (n_keys_max + ck - 1) / ck;
      if (nc > 1 && (size_t)p.B * p.nq * p.T * nc * (p.hd + 4) <= p.part_floats) {
        p.nchunk = nc;
        p.kchunk = ck;
      }
    }
    dim3 grid(n_qt * p.nchunk, p.nq, p.B);
    if (p.hd == 128) hipLaunchKernelGGL(attn_prefill_mfma_kernel<128>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(attn_prefill_mfma_kernel<64>, grid, dim3(256), 0, s, p);
    if (p.nchunk > 1) {
      dim3 mg((p.T * (p.hd / 4) + 255) / 256, p.nq, p.B);
      if (p.hd == 128) hipLaunchKernelGGL(attn_prefill_merge_kernel<128>, mg, dim3(256), 0, s, p);
      else hipLaunchKernelGGL(attn_prefill_merge_kernel<64>, mg, dim3(256), 0, s, p);
    }
    return hipGetLastError();
  }
  dim3 grid((p.T + kQTile - 1) / kQTile, p.nq, p.B);
  if (p.hd == 128) hipLaunchKernelGGL((attn_prefill_kernel<float, 128>), grid, dim3(256), 0, s, p);
  else if (p.hd == 64) hipLaunchKernelGGL((attn_prefill_kernel<float, 64>), grid, dim3(256), 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ladder

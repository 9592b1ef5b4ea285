// Stochastic next-token draw from the LM head's logits (the optional alternative to the
// greedy argmax).
//
// The draw follows the inference code's `logits_to_probs` / `multinomial_sample_one_no_sync`
// / `sample` (function names on the codewithpapers record of the method's pages), read
// as: logits divided by a temperature T, optionally cut to the top k (every logit >= the
// k-th largest is kept), one token drawn from the softmax of the kept ones by the
// exponential race, which in log form is the Gumbel-max rule
//   token = argmax over kept i of  z_i / T - log(-log U_i),
// so no normalisation, no cumulative sum and no host synchronisation are needed.
//
// U_i comes from Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, SC 2011): the
// counter (i / 4, b, pos, 0) under the key (seed low word, seed high word) gives four
// 32-bit words, entry i takes word i % 4 and U = (2 (word >> 9) + 1) 2^-24, an exact
// float in (0, 1).  A draw is a function of (seed, position, sequence, vocabulary entry)
// only, so a replayed graph draws the same tokens for the same positions.
//
// One workgroup per sequence.  Rows of up to kSampleLdsFloats logits are first copied
// into LDS with independent loads (every later pass reads LDS); longer rows are read
// from global memory in each pass.  The top-k threshold is found by a radix select over
// the order-preserving 32-bit keys of the logits, 8 bits per pass (4 passes over the
// row, histograms in LDS); the draw is one more pass computing the Gumbel scores of the
// kept entries and a workgroup argmax (lowest index on equal scores).
#include <climits>

#include "common.hpp"
#include "kernels.h"

namespace ladder {

namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;   // round multipliers
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;   // key increments

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint32_t hi0 = __umulhi(kPhiloxM0, c.x), lo0 = kPhiloxM0 * c.x;
    const uint32_t hi1 = __umulhi(kPhiloxM1, c.z), lo1 = kPhiloxM1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Larger float -> larger unsigned key (finite values).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSampleLdsFloats = 32768;   // 128 KB of LDS: rows up to this many logits are staged

template <bool STAGED>
__global__ __launch_bounds__(256) void sample_kernel(SampleParams p) {
  extern __shared__ float zs[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_digit, sel_rank;
  __shared__ float rv[256];
  __shared__ int ri[256];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int V = p.V;
  const float* zg = p.logits + (size_t)b * p.ldl;
  if constexpr (STAGED) {
#pragma unroll 8
    for (int i = tid; i < V; i += 256) zs[i] = zg[i];
    __syncthreads();
  }
  const float* z = STAGED ? zs : zg;

  // ---- top-k threshold: key of the k-th largest logit (0 keeps everything)
  uint32_t thr = 0;
  if (p.top_k > 0 && p.top_k < V) {
    uint32_t prefix = 0, mask = 0, k = (uint32_t)p.top_k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < V; i += 256) {
        const uint32_t key = order_key(z[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        // the digit d holding the k-th largest among the keys that match the prefix
        uint32_t above = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (above + hist[d] >= k) break;
          above += hist[d];
        }
        sel_digit = (uint32_t)d;
        sel_rank = k - above;
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      mask |= 255u << shift;
      k = sel_rank;
      __syncthreads();                          // before hist is cleared again
    }
    thr = prefix;
  }

  // ---- Gumbel-max draw over the kept entries
  const int pos = p.d_pos ? *gbl(p.d_pos) : p.pos;
  float best = -INFINITY;
  int bidx = INT_MAX;
  for (int j = tid; j < (V + 3) / 4; j += 256) {
    const uint4 w = philox4x32_10(make_uint4((uint32_t)j, (uint32_t)b, (uint32_t)pos, 0u), p.seed_lo, p.seed_hi);
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * j + e;
      if (i < V) {
        const float zi = z[i];
        if (order_key(zi) >= thr) {
          const float u = (float)((words[e] >> 9) * 2u + 1u) * 0x1p-24f;
          const float s = zi / p.temperature - logf(-logf(u));
          if (s > best || (s == best && i < bidx)) {
            best = s;
            bidx = i;
          }
        }
      }
    }
  }
  rv[tid] = best;
  ri[tid] = bidx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      const float v = rv[tid + o];
      const int i = ri[tid + o];
      if (v > rv[tid] || (v == rv[tid] && i < ri[tid])) {
        rv[tid] = v;
        ri[tid] = i;
      }
    }
    __syncthreads();
  }
  if (tid == 0) p.next[b] = ri[0] == INT_MAX ? 0 : ri[0];
}

}  // namespace

hipError_t launch_sample(const SampleParams& p, hipStream_t s) {
  if (!p.logits || !p.next || p.B < 1 || p.V < 1 || p.ldl < p.V || !(p.temperature > 0.f) ||
      !(p.temperature < INFINITY) || p.top_k < 0)
    return hipErrorInvalidValue;
  if (p.V <= kSampleLdsFloats) {
    const size_t lds = (size_t)p.V * sizeof(float);
    static bool attr = false;
    if (!attr) {
      const hipError_t e = hipFuncSetAttribute((const void*)sample_kernel<true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kSampleLdsFloats * (int)sizeof(float));
      if (e != hipSuccess) return e;
      attr = true;
    }
    launch_timed(sample_kernel<true>, dim3(p.B), dim3(256), (uint32_t)lds, s, p);
  } else {
    launch_timed(sample_kernel<false>, dim3(p.B), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ladder

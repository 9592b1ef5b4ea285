// Prefill projections C[M][N] = (R) + A[M][K] . W^T with M = batch x tokens.
//
// bf16 models: a dense contraction, so it runs on the CDNA4 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  A arrives in fp32 and is split on
// its way into LDS into a pair of bf16 values, hi = bf16(a) and lo = bf16(a - hi) (the
// prefill projections fed by an RMSNorm get A already split by the RMSNorm kernel: 50.0
// against 52.1 ms for the 70B shard's 1024-token prefill, since each of the 56 column
// tiles of its gate/up GEMM would otherwise split the same rows again),
// which together carry about 16 significant bits over fp32's range; the stored bf16
// weights feed the matrix cores as they are.  Each product is then two MFMAs, hi.W and
// lo.W, into one fp32 accumulator: a single 16-bit rounding of the activations perturbs
// every module input by up to 2^-9 (bf16) or 2^-12 (fp16) relative, and a CPU emulation
// of the 70B-shape shard (80 ladder layers) carries one rounding to 5.3e-2 (bf16) or
// 1.25e-2 (fp16) in the logits, above the 1e-2 bar, while a bf16 or fp16 pair stays at
// the ~5e-3 that any 2^-22 perturbation reaches at that depth.
//
// Tiling: a workgroup of 4 waves owns a 128x128 tile of C (2x2 waves of 64x64, i.e.
// 4x4 MFMA tiles each; 32x128 or 64x128 tiles for at most 32 or 64 rows, as in a decode
// step of a large batch, where 128-row tiles would be mostly padding; 64x64 tiles when
// 128x128 ones would leave CUs idle) and walks K
// in steps of 32 through double-buffered LDS with padded rows.  The global loads run
// kStages steps ahead of the MFMAs in a ring of register buffers (a step's MFMA work,
// ~0.2-0.4 us per workgroup, is well below the latency of a global load under a full
// device's traffic, so one step of prefetch leaves the matrix cores waiting).
// Optional epilogues: a residual add, or SwiGLU over interleaved gate/up columns.
// Optional RMSNorm (split launches of a decode step): RMSNorm(x) W^T = (x * g) W^T / rms(x)
// row by row, so A is the raw residual row, it is multiplied by the gain on its way into
// LDS, the workgroups of the first column tile add up each row's squares over their K
// slice, and the reduction divides each row's sums by its rms.  The raw rows pass through
// the bf16 pairs unnormalized, which hold fp32's exponent range.
// Workgroups are dealt to the 8 XCDs round robin, so the tile list (M fastest) is cut
// into 8 contiguous runs and run x goes to XCD x: workgroups that share a weight tile
// run together on one XCD and read it once into that XCD's L2.
// Split K: when a projection has too few 128x128 tiles to fill the device (the QKV
// projection of a narrow shard: 80 tiles at M 1024), S workgroups share each tile, each
// over K/S, and store fp32 partial tiles; a reduction kernel sums them in slice order
// (deterministic) and applies the epilogue.
//
// fp32 models (small correctness-only models): a plain LDS-tiled VALU GEMM.
#include <type_traits>

#include "attn_decode.hpp"
#include "common.hpp"
#include "kernels.h"

namespace ladder {

template <int N>
using IC = std::integral_constant<int, N>;

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

template <typename WT>
__device__ __forceinline__ const WT* gemm_row(const RowSrc& s, int r, int K) {
  if (s.interleave) return (const WT*)s.m[r & 1] + (size_t)(r >> 1) * K;
  if (r < s.n0) return (const WT*)s.m[0] + (size_t)r * K;
  if (r < s.n1) return (const WT*)s.m[1] + (size_t)(r - s.n0) * K;
  return (const WT*)s.m[2] + (size_t)(r - s.n1) * K;
}

constexpr int BK = 32;
// LDS operand tiles hold rows of BK = 32 bf16 (four 16-byte chunks) without padding; chunk c
// of row r sits at position c ^ ((r / 4) % 4).  Then a pass of 16-byte or 8-byte staging
// writes (4 rows of 64 bytes) and a pass of 16-byte MFMA operand reads (16 rows, one chunk
// each) both cover every bank once; with rows padded to 40 bf16 the writes conflicted
// 2-way (half of the LDS cycles of the prefill GEMMs were bank conflicts).
__device__ __forceinline__ int gsw(int r, int chunk) { return 8 * (chunk ^ ((r >> 2) & 3)); }
constexpr int kXcds = 8;
constexpr int kStages = 4;   // K steps whose global loads are in flight (even: LDS buffers alternate)

// TM x TN workgroup tile (128x128, or 64x64 when the big tiles would not fill the
// device), 4 waves of (TM/2) x (TN/2), i.e. (TM/32) x (TN/32) MFMA tiles of 16x16 each.
// Slice s of S covers K steps [s * nst / S, (s + 1) * nst / S) of the nst = K / 32; with more than one
// slice the raw partial tile goes to p.ws[slice][M][N].
// Register caps: two waves per SIMD for 128-row tiles (two workgroups per CU instead of
// one) and for 64-row tiles with the folded RMSNorm, three for the other 64-row tiles and
// four for 32-row tiles; each the tightest that keeps the four-stage ring in registers
// without spills.  With the caps and the unconditional loads (the ring actually in
// flight): the 70B shard's 1024-token prefill 51.0 against 54.3 ms, batch-64 decode 4991
// against 4817 tok/s on the 70B shard and 2313 against 2132 on the 405B shard.
// APAIR: A arrives already split into bf16 pairs (p.a_pairs: 16 bytes per 4 columns, their
// 4 hi then their 4 lo values) and goes into LDS as it is (the split is done once by A's
// producer instead of once per column tile).
// One workgroup's tile (tile, slice of S) of problem p.
template <int TM, int TN, bool NORM, bool APAIR>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int tile, int slice, int S, int n_tiles_m, int nst) {
  static_assert(!(NORM && APAIR), "the folded RMSNorm takes fp32 rows");
  constexpr int FM = TM / 32, FN = TN / 32;       // MFMA tiles per wave
  constexpr int AV = TM * BK / 4 / 256;           // float4 of A per thread per K step
  constexpr int BV = TN * BK / 8 / 256;           // 16-byte W chunks per thread per K step
  static_assert(AV >= 1 && BV >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t Ah[2][TM][BK];
  __shared__ __attribute__((aligned(16))) uint16_t Al[2][TM][BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TN][BK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = (tile % n_tiles_m) * TM, n0 = (tile / n_tiles_m) * TN;
  const int st0 = slice * nst / S;
  const int kbase = st0 * BK;
  const float* A = (const float*)p.A + kbase;
  const uint16_t* Ap = (const uint16_t*)p.A + 2 * kbase;                      // APAIR

  // per K step a thread moves AV float4 of A (rows c/8, columns 4*(c%8)) and BV 16-byte
  // chunks of W (rows c/4, columns 8*(c%4)).  Rows past M (N) read row M-1 (N-1): they
  // only feed output rows (columns) that are never stored, and every load is
  // unconditional, so that the wait before each step's LDS stores covers that step's
  // loads only (with loads under branches the compiler waits for all of them, and the
  // ring holds nothing in flight).
  const float* arow[AV];
  const uint16_t* aprow[AV];   // APAIR
  const uint16_t* brow[BV];
  int ar[AV], ac[AV], br[BV], bc[BV];
#pragma unroll
  for (int i = 0; i < AV; ++i) {
    const int c = tid + 256 * i;
    ar[i] = c >> 3;
    ac[i] = (c & 7) * 4;
    const int m = m0 + ar[i];
    if constexpr (APAIR) aprow[i] = Ap + 2 * ((size_t)min(m, p.M - 1) * p.lda + ac[i]);
    else arow[i] = A + (size_t)min(m, p.M - 1) * p.lda + ac[i];
  }
#pragma unroll
  for (int i = 0; i < BV; ++i) {
    const int c = tid + 256 * i;
    br[i] = c >> 2;
    bc[i] = (c & 3) * 8;
    const int n = n0 + br[i];
    brow[i] = gemm_row<uint16_t>(p.rows, min(n, p.N - 1), p.K) + kbase + bc[i];
  }
  // register ring: stage st holds the global loads of one K step
  float4 ra[kStages][AV];
  uint4 rp[kStages][AV];       // APAIR: 4 bf16 of the hi plane (x, y), 4 of the lo plane (z, w)
  uint4 rb[kStages][BV];
  uint2 rg[kStages][AV];                          // NORM: the gain of each A float4 (4 x bf16)
  const uint16_t* gain = NORM ? (const uint16_t*)p.gain + kbase : nullptr;
  const bool sum_sq = NORM && tile < n_tiles_m;   // the first column tile adds up the squares
  float sq[AV];
#pragma unroll
  for (int i = 0; i < AV; ++i) sq[i] = 0.f;
  const int nk = (slice + 1) * nst / S - st0;
  const int nkp = (nk + kStages - 1) / kStages * kStages;   // steps padded to whole ring turns
  // Stage indices are compile-time constants (std::integral_constant), so that the ring
  // stays in registers.  Step kt's loads into stage ST (steps past the slice load its last
  // step again).
  auto gload = [&](auto STC, int kt) {
    constexpr int st = decltype(STC)::value;
    const int k0 = min(kt, nk - 1) * BK;
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      if constexpr (APAIR) {
        rp[st][i] = ldg4u(aprow[i] + 2 * k0);
        continue;
      }
      ra[st][i] = ldg4(arow[i] + k0);
      if constexpr (NORM) rg[st][i] = *(const uint2*)(gain + k0 + ac[i]);
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) rb[st][i] = ldg4u(brow[i] + k0);
  };
  // stage st (step kt) into LDS buffer buf; the A of a padding step (kt >= nk) is zero,
  // so that its products add nothing
  auto sstore = [&](auto STC, int buf, int kt) {
    constexpr int st = decltype(STC)::value;
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      if constexpr (APAIR) {
        const uint4 v = kt >= nk ? make_uint4(0u, 0u, 0u, 0u) : rp[st][i];
        const int ak = gsw(ar[i], ac[i] >> 3) + (ac[i] & 7);
        *(uint2*)&Ah[buf][ar[i]][ak] = make_uint2(v.x, v.y);
        *(uint2*)&Al[buf][ar[i]][ak] = make_uint2(v.z, v.w);
        continue;
      }
      if (kt >= nk) ra[st][i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (NORM) {
        float4& a = ra[st][i];
        if (sum_sq) {
          sq[i] = fmaf(a.x, a.x, sq[i]);
          sq[i] = fmaf(a.y, a.y, sq[i]);
          sq[i] = fmaf(a.z, a.z, sq[i]);
          sq[i] = fmaf(a.w, a.w, sq[i]);
        }
        const uint2 g = rg[st][i];
        a.x *= __uint_as_float(g.x << 16);
        a.y *= __uint_as_float(g.x & 0xffff0000u);
        a.z *= __uint_as_float(g.y << 16);
        a.w *= __uint_as_float(g.y & 0xffff0000u);
      }
      uint32_t h0, l0, h1, l1;
      split_bf2(ra[st][i].x, ra[st][i].y, h0, l0);
      split_bf2(ra[st][i].z, ra[st][i].w, h1, l1);
      const int ak = gsw(ar[i], ac[i] >> 3) + (ac[i] & 7);
      *(uint2*)&Ah[buf][ar[i]][ak] = make_uint2(h0, h1);
      *(uint2*)&Al[buf][ar[i]][ak] = make_uint2(l0, l1);
    }
#pragma unroll
    for (int i = 0; i < BV; ++i) *(uint4*)&Bs[buf][br[i]][gsw(br[i], bc[i] >> 3)] = rb[st][i];
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: steps 0 .. kStages-1 in flight, step 0 into LDS buffer 0, then stage 0
  // refilled with step kStages
  static_assert(kStages == 4, "the ring below is written out for four stages");
  gload(IC<0>{}, 0);
  gload(IC<1>{}, 1);
  gload(IC<2>{}, 2);
  gload(IC<3>{}, 3);
  sstore(IC<0>{}, 0, 0);
  gload(IC<0>{}, kStages);
  __syncthreads();
  // 16x16x32 fragments: lane holds row (A) / column (W) lane%16, k = 8*(lane/16) .. +8
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  // step kt reads LDS buffer kt & 1 and register stage kt % kStages holds (in flight)
  // step kt + kStages; after the MFMAs, step kt + 1 goes from its stage into the other
  // LDS buffer and that stage is refilled with step kt + 1 + kStages
  auto step = [&](auto UC, int kt) {
    constexpr int u = decltype(UC)::value;
      {
        constexpr int cur = u & 1;
        bf16x8 ah[FM], al[FM], b[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * (TM / 2) + i * 16 + fr;
          ah[i] = *(const bf16x8*)&Ah[cur][r][gsw(r, fk >> 3)];
          al[i] = *(const bf16x8*)&Al[cur][r][gsw(r, fk >> 3)];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * (TN / 2) + j * 16 + fr;
          b[j] = *(const bf16x8*)&Bs[cur][r][gsw(r, fk >> 3)];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], b[j], acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], b[j], acc[i][j], 0, 0, 0);
          }
        // (after the last step too: the stores go to the idle buffer, the loads repeat the
        // last step, and nothing reads either)
        using Nxt = IC<(u + 1) % kStages>;
        sstore(Nxt{}, cur ^ 1, kt + 1);
        gload(Nxt{}, kt + 1 + kStages);
        __syncthreads();
      }
  };
  for (int k0 = 0; k0 < nkp; k0 += kStages) {
    step(IC<0>{}, k0);
    step(IC<1>{}, k0 + 1);
    step(IC<2>{}, k0 + 2);
    step(IC<3>{}, k0 + 3);
  }

  if (sum_sq) {
    // the 8 threads of a row (consecutive lanes) hold its squares over 4 columns of each
    // K step; the slice's sum of row m goes to ws[S*M*N + slice*M + m]
#pragma unroll
    for (int i = 0; i < AV; ++i) {
      float v = sq[i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      const int row = m0 + ar[i];
      if ((tid & 7) == 0 && row < p.M)
        p.ws[(size_t)S * p.M * p.N + (size_t)slice * p.M + row] = v;
    }
  }

  // C fragment: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile.
  // SwiGLU: columns 2n (gate) and 2n+1 (up) sit in neighbouring lanes; the even lane
  // writes a[row][n] = silu(gate) * up.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * (TN / 2) + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * (TM / 2) + i * 16 + (lane >> 4) * 4 + r;
        float v = acc[i][j][r];
        if (S > 1) {
          if (row < p.M && col < p.N) p.ws[((size_t)slice * p.M + row) * p.N + col] = v;
        } else if (p.swiglu) {
          const float up = __shfl_xor(v, 1, 64);
          const float y = silu(v) * up;
          if (p.c_pairs) {
            // the output as bf16 pairs: lanes fr = 0 and 8 of each row gather the values of
            // the three even lanes after them (four consecutive outputs) and store one group
            const float y1 = __shfl(y, lane + 2, 64), y2 = __shfl(y, lane + 4, 64), y3 = __shfl(y, lane + 6, 64);
            if ((fr & 7) == 0 && row < p.M && col < p.N) {
              uint32_t h0, l0, h1, l1;
              split_bf2(y, y1, h0, l0);
              split_bf2(y2, y3, h1, l1);
              *(uint4*)((uint16_t*)p.C + 2 * ((size_t)row * p.ldc + (col >> 1))) = make_uint4(h0, h1, l0, l1);
            }
          } else if (!(col & 1) && row < p.M && col < p.N) {
            p.C[(size_t)row * p.ldc + (col >> 1)] = y;
          }
        } else if (row < p.M && col < p.N) {
          if (p.res) v = p.res[(size_t)row * p.ldr + col] + v;
          p.C[(size_t)row * p.ldc + col] = v;
        }
      }
    }
}

template <int TM, int TN, bool NORM = false, bool APAIR = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TM == 128 || (TM == 64 && NORM) ? 2 : TM == 64 ? 3 : 4)))
void gemm_bf16x2_kernel(GemmParams p, int n_tiles_m, int n_tiles, int per_xcd, int nst) {
  const int tile = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (tile >= n_tiles) return;
  gemm_tile<TM, TN, NORM, APAIR>(p, tile, blockIdx.y, gridDim.y, n_tiles_m, nst);
}

// Two split-K problems of one row tile (64 rows) in one launch: items [0, items0) are the
// first problem's (column run x of its tile list on XCD x, then slice), the rest the
// second's; each problem's tiles, slices and partials are those of its own launch, and
// one reduction launch then serves both.
struct GemmPairArgs {
  GemmParams p[2];
  int n_tiles[2], per_xcd[2], S[2], nst[2];
  int items0;
};

template <bool NORM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NORM ? 2 : 3)))
void gemm_pair_kernel(GemmPairArgs a) {
  int b = (int)blockIdx.x;
  const int q = b >= a.items0 ? 1 : 0;
  if (q) b -= a.items0;
  const int W = a.per_xcd[q] * kXcds;
  const int x = b % W;
  const int tile = (x % kXcds) * a.per_xcd[q] + x / kXcds;
  if (tile >= a.n_tiles[q]) return;
  gemm_tile<64, 128, NORM, false>(a.p[q], tile, b / W, a.S[q], 1, a.nst[q]);
}

// C = (res +) sum over the S slices of ws[s] in slice order, or with swiglu
// C[m][n] = silu(g) * u of the summed columns 2n, 2n+1.  One thread per output element.
__device__ __forceinline__ void splitk_reduce(const GemmParams& p, int S, size_t e) {
  const int NO = p.swiglu ? p.N / 2 : p.N;
  if (e >= (size_t)p.M * NO) return;
  const int m = (int)(e / NO), n = (int)(e % NO);
  const size_t plane = (size_t)p.M * p.N;
  float inv = 1.f;                                 // fused RMSNorm: 1 / rms of row m
  if (p.gain) {
    const float* q = p.ws + (size_t)S * plane + m;
    float t = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) t += q[(size_t)s * p.M];
    inv = 1.0f / sqrtf(t / (float)p.K + p.eps);
  }
  if (p.swiglu) {
    const float* w = p.ws + (size_t)m * p.N + 2 * n;
    float g = 0.f, u = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      g += w[s * plane];
      u += w[s * plane + 1];
    }
    if (p.gain) {
      g *= inv;
      u *= inv;
    }
    p.C[(size_t)m * p.ldc + n] = silu(g) * u;
  } else {
    const float* w = p.ws + (size_t)m * p.N + n;
    float v = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) v += w[s * plane];
    if (p.gain) v *= inv;
    if (p.res) v = p.res[(size_t)m * p.ldr + n] + v;
    p.C[(size_t)m * p.ldc + n] = v;
  }
}

// The reduction of a decode step's QKV projection with rope_kv's epilogue (bf16 caches): a
// thread sums the partials of two neighbouring outputs (n even) as splitk_reduce does, then
// rotates the q and k pairs (d, d + 1) and writes q to rope_q, k and v to the caches at
// position *d_pos, with rope_kv's arithmetic on the same fp32 values.
__device__ __forceinline__ void splitk_reduce_rope(const GemmParams& p, int S, size_t e) {
  const int NP = p.N / 2;
  if (e >= (size_t)p.M * NP) return;
  const int m = (int)(e / NP), n = 2 * (int)(e % NP);
  const size_t plane = (size_t)p.M * p.N;
  float inv = 1.f;
  if (p.gain) {
    const float* q = p.ws + (size_t)S * plane + m;
    float t = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) t += q[(size_t)s * p.M];
    inv = 1.0f / sqrtf(t / (float)p.K + p.eps);
  }
  const float* w = p.ws + (size_t)m * p.N + n;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    v0 += w[s * plane];
    v1 += w[s * plane + 1];
  }
  if (p.gain) {
    v0 *= inv;
    v1 *= inv;
  }
  const int qr = p.nq * p.hd, kr = p.nkv * p.hd, pos = *gbl(p.d_pos);
  uint16_t* dst;
  if (n < qr + kr) {
    const int d = (n < qr ? n : n - qr) % p.hd;
    const float c = p.rope_cos[(size_t)pos * (p.hd / 2) + d / 2], sn = p.rope_sin[(size_t)pos * (p.hd / 2) + d / 2];
    rope_rot(v0, v1, c, sn);
    if (n < qr) {
      p.rope_q[(size_t)m * qr + n] = v0;
      p.rope_q[(size_t)m * qr + n + 1] = v1;
      return;
    }
    dst = (uint16_t*)p.k_cache + (((size_t)m * p.nkv + (n - qr) / p.hd) * p.max_seq + pos) * p.hd + d;
  } else {
    const int i = n - qr - kr;
    dst = (uint16_t*)p.v_cache + (((size_t)m * p.nkv + i / p.hd) * p.max_seq + pos) * p.hd + i % p.hd;
  }
  store_w<uint16_t>(dst, v0);
  store_w<uint16_t>(dst + 1, v1);
}

__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(GemmParams p, int S) {
  splitk_reduce(p, S, (size_t)blockIdx.x * 256 + threadIdx.x);
}

// The reductions of a pair launch in one launch: blocks [0, blocks0) reduce problem a
// (with the RoPE + KV epilogue where a.rope_q is set).
__global__ __launch_bounds__(256) void gemm_splitk_reduce_pair_kernel(GemmParams a, int Sa, GemmParams b, int Sb,
                                                                      int blocks0) {
  const int bi = (int)blockIdx.x;
  if (bi >= blocks0) splitk_reduce(b, Sb, (size_t)(bi - blocks0) * 256 + threadIdx.x);
  else if (a.rope_q) splitk_reduce_rope(a, Sa, (size_t)bi * 256 + threadIdx.x);
  else splitk_reduce(a, Sa, (size_t)bi * 256 + threadIdx.x);
}

// A chained pair with the decode attention that feeds its first problem in the same launch:
// blocks [0, n_attn) run the split-KV attention (coherent records and output, and the
// completion signal at.done_flag = step epoch after the last merge), the next ones the
// second problem (the down projection, which needs no attention), the last ones the first
// problem (O), whose workgroups wait for the signal before loading their A (the attention
// output: nothing in the launch reads it earlier, so no cache holds a stale copy).  The
// attention workgroups come first in dispatch order and wait for nothing.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_attn_chain_kernel(GemmPairArgs g, AttnDecodeParams at, int n_attn, int* err) {
  __shared__ AttnLds<uint16_t, HD> L;
  int b = (int)blockIdx.x;
  if (b < n_attn) {
    attn_decode_block_mfma<HD, true>(at, b, L);
    return;
  }
  b -= n_attn;
  const int items1 = g.per_xcd[1] * kXcds * g.S[1];
  int q = 1;
  if (b >= items1) {
    q = 0;
    b -= items1;
    wg_wait_coh(at.done_flag, *gbl(at.d_epoch), err);
  }
  const int W = g.per_xcd[q] * kXcds;
  const int x = b % W;
  const int tile = (x % kXcds) * g.per_xcd[q] + x / kXcds;
  if (tile >= g.n_tiles[q]) return;
  gemm_tile<64, 128, false, false>(g.p[q], tile, b / W, g.S[q], 1, g.nst[q]);
}

// The reduction of a chained pair (a: the O projection with its residual, b: the down
// projection whose residual is a's output): per element x1 = res + sum(a) written to a.C,
// then x1 + sum(b) to b.C, each sum in slice order as splitk_reduce adds it.
__global__ __launch_bounds__(256) void gemm_splitk_reduce_chain_kernel(GemmParams a, int Sa, GemmParams b, int Sb) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)a.M * a.N) return;
  const int m = (int)(e / a.N), n = (int)(e % a.N);
  const size_t plane = (size_t)a.M * a.N;
  const float* wa = a.ws + (size_t)m * a.N + n;
  float o = 0.f;
#pragma unroll 8
  for (int s = 0; s < Sa; ++s) o += wa[s * plane];
  const float x1 = a.res[(size_t)m * a.ldr + n] + o;
  a.C[(size_t)m * a.ldc + n] = x1;
  const float* wb = b.ws + (size_t)m * b.N + n;
  float d = 0.f;
#pragma unroll 8
  for (int s = 0; s < Sb; ++s) d += wb[s * plane];
  b.C[(size_t)m * b.ldc + n] = x1 + d;
}

constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * FT, n0 = blockIdx.x * FT;
  const float* A = (const float*)p.A;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += FK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / FK, kk = e % FK;
      const int m = m0 + r, n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < p.M && k < p.K) ? A[(size_t)m * p.lda + k] : 0.f;
      Bs[kk][r] = (n < p.N && k < p.K) ? gemm_row<float>(p.rows, n, p.K)[k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < p.M && col < p.N) {
        float v = acc[i][j];
        if (p.res) v = p.res[(size_t)row * p.ldr + col] + v;
        p.C[(size_t)row * p.ldc + col] = v;
      }
    }
}

// Row tile height of a bf16 launch: 32 / 64 rows for at most 32 / 64 rows, else 128.
static int gemm_tile_rows(const GemmParams& p) { return p.M <= 32 ? 32 : p.M <= 64 ? 64 : 128; }

int gemm_splits(const GemmParams& p) {
  if (p.wdtype != W_BF16 || !p.ws || p.M < 1 || p.N < 1 || p.K < 1) return 1;
  // the fewest slices that give one round of workgroups (half a round for the 32- and
  // 64-row tiles: decode steps, whose projections mostly run two to a launch); at most 32
  // slices (64 made the 10-tile QKV projection of a 70B shard's decode step
  // slower: slices of 4 K steps and 64 partials per output); each slice at least kStages
  // steps long, partials (and the fused norm's row sums) within the workspace
  const int tmr = gemm_tile_rows(p);
  const int big = ((p.M + tmr - 1) / tmr) * ((p.N + 127) / 128);
  // (slices of unequal length, as many as fill one round at the register caps' occupancy,
  // measured 5057 against 4926 tok/s at batch 64 on the 70B shard but 2257 against 2297 on
  // the 405B shard and a slower prefill: not taken)
  // (for the 32- and 64-row tiles two rounds, so that more weight streams are in flight,
  // was the rule before their projections ran in pairs; tok/s on the 70B shard at batch
  // 64 / 32 / 24 and on the 405B shard at batch 64, two rounds -> one -> half: 5848 ->
  // 6729 -> 7231, 3467 -> 3687 -> 4027, 2682 -> 2872 -> 3097, 2680 -> 2877 -> 2989; a
  // quarter round: 6057, 3256, 2477, 2311)
  const int fill = tmr < 128 ? 128 : 256;
  int S = 1;
  if (big < 256) {   // (under a round of tiles: at least two slices, or none)
    for (int c = 2; c <= 32; c *= 2) {
      const size_t ws = (size_t)c * p.M * p.N + (p.gain ? (size_t)c * p.M : 0);
      if (p.K % (c * BK) != 0 || p.K / c < kStages * BK || ws > p.ws_floats) break;
      if ((long long)big * c >= fill) {
        S = c;
        break;
      }
    }
  }
  return S;
}

// The fused RMSNorm: split launches of the 32- and 64-row tiles (decode steps of up to 64
// sequences); it saves the two RMSNorm launches per layer: 4794 against 4483 tok/s at
// batch 64 on the 70B shard, 2129 against 1958 on the 405B shard (both measured before the
// register caps below).  The 128-row tiles keep the RMSNorm kernel.
bool gemm_takes_pairs(const GemmParams& p) {
  return p.wdtype == W_BF16 && !p.gain && !p.A2 && p.M > 64 && p.K % BK == 0 && p.lda % 4 == 0 &&
         (!p.swiglu || (p.N % 2 == 0 && !p.res));
}

bool gemm_writes_pairs(const GemmParams& p) {
  return p.wdtype == W_BF16 && p.swiglu && !p.gain && !p.A2 && !p.res && p.M > 64 && p.N % 16 == 0 &&
         p.ldc % 4 == 0 && p.K % BK == 0 && p.lda % 4 == 0 && gemm_splits(p) == 1;
}

bool gemm_norm_fusable(const GemmParams& p) {
  if (skinny_supported(p)) return true;
  return p.wdtype == W_BF16 && p.M <= 64 && p.lda % 4 == 0 && p.K % BK == 0 && gemm_splits(p) > 1;
}

bool gemm_pair_ok(const GemmParams& a, const GemmParams& b) {
  auto one = [](const GemmParams& p) {
    return p.wdtype == W_BF16 && !p.A2 && !p.a_pairs && !p.c_pairs && p.M > 32 &&
           p.M <= 64 && p.K % BK == 0 && p.lda % 4 == 0 && (!p.swiglu || (p.N % 2 == 0 && !p.res)) && p.ws &&
           gemm_splits(p) > 1 && !skinny_supported(p);
  };
  // a.rope_q: the first problem is a decode step's QKV projection whose reduction runs
  // rope_kv's epilogue (bf16 caches, the skinny launches' conditions on the rope fields)
  const bool rope_ok = !a.rope_q || (!a.swiglu && !a.res && a.k_cache && a.v_cache && a.rope_cos && a.rope_sin &&
                                     a.d_pos && a.hd >= 2 && a.hd % 2 == 0 && a.nq >= 1 && a.nkv >= 1 &&
                                     a.max_seq >= 1 && a.N == (a.nq + 2 * a.nkv) * a.hd);
  return one(a) && one(b) && !b.rope_q && rope_ok && a.M == b.M && (a.gain != nullptr) == (b.gain != nullptr) &&
         a.ws != b.ws;
}

hipError_t launch_gemm_pair(const GemmParams& a, const GemmParams& b, hipStream_t s) {
  if (!gemm_pair_ok(a, b)) return hipErrorInvalidValue;
  GemmPairArgs g{};
  const GemmParams* q[2] = {&a, &b};
  int items = 0;
  for (int i = 0; i < 2; ++i) {
    const GemmParams& p = *q[i];
    g.p[i] = p;
    g.n_tiles[i] = (p.N + 127) / 128;
    g.per_xcd[i] = (g.n_tiles[i] + kXcds - 1) / kXcds;
    g.S[i] = gemm_splits(p);
    g.nst[i] = p.K / BK;
    if (i == 0) g.items0 = g.per_xcd[0] * kXcds * g.S[0];
    items += g.per_xcd[i] * kXcds * g.S[i];
  }
  if (a.gain) launch_timed(gemm_pair_kernel<true>, dim3(items), dim3(256), 0, s, g);
  else launch_timed(gemm_pair_kernel<false>, dim3(items), dim3(256), 0, s, g);
  unsigned blocks[2];
  for (int i = 0; i < 2; ++i) {
    const GemmParams& p = *q[i];
    blocks[i] = (unsigned)(((size_t)p.M * (p.swiglu || (i == 0 && p.rope_q) ? p.N / 2 : p.N) + 255) / 256);
  }
  launch_timed(gemm_splitk_reduce_pair_kernel, dim3(blocks[0] + blocks[1]), dim3(256), 0, s, a, g.S[0], b, g.S[1],
               (int)blocks[0]);
  return hipGetLastError();
}

bool gemm_chain_ok(const GemmParams& a, const GemmParams& b) {
  return !a.rope_q && !b.rope_q && !a.gain && !b.gain && !a.swiglu && !b.swiglu && gemm_pair_ok(a, b) &&
         a.N == b.N && a.res && a.C && b.res == a.C && b.ldr == a.ldc && b.C && b.C != a.C && a.ws != b.ws;
}

hipError_t launch_gemm_chain(const GemmParams& a, const GemmParams& b, hipStream_t s) {
  if (!gemm_chain_ok(a, b)) return hipErrorInvalidValue;
  GemmPairArgs g{};
  const GemmParams* q[2] = {&a, &b};
  int items = 0;
  for (int i = 0; i < 2; ++i) {
    const GemmParams& p = *q[i];
    g.p[i] = p;
    g.n_tiles[i] = (p.N + 127) / 128;
    g.per_xcd[i] = (g.n_tiles[i] + kXcds - 1) / kXcds;
    g.S[i] = gemm_splits(p);
    g.nst[i] = p.K / BK;
    if (i == 0) g.items0 = g.per_xcd[0] * kXcds * g.S[0];
    items += g.per_xcd[i] * kXcds * g.S[i];
  }
  launch_timed(gemm_pair_kernel<false>, dim3(items), dim3(256), 0, s, g);
  launch_timed(gemm_splitk_reduce_chain_kernel, dim3((unsigned)(((size_t)a.M * a.N + 255) / 256)), dim3(256), 0, s, a,
               g.S[0], b, g.S[1]);
  return hipGetLastError();
}

bool gemm_attn_chain_ok(const AttnDecodeParams& at, const GemmParams& a, const GemmParams& b) {
  return gemm_chain_ok(a, b) && at.wdtype == W_BF16 && (at.hd == 64 || at.hd == 128) && at.nkv >= 1 &&
         at.nq % at.nkv == 0 && at.nq / at.nkv <= kAttnMaxGroup && at.n_split >= 1 && at.n_split <= kAttnMaxSplits &&
         at.B == a.M && at.out == a.A && !a.a_pairs && at.done_cnt && at.done_flag && at.d_epoch && at.part &&
         at.counters && at.q && at.d_pos;
}

hipError_t launch_gemm_attn_chain(const AttnDecodeParams& at, const GemmParams& a, const GemmParams& b, int* err,
                                  hipStream_t s) {
  if (!gemm_attn_chain_ok(at, a, b) || !err) return hipErrorInvalidValue;
  GemmPairArgs g{};
  const GemmParams* q[2] = {&a, &b};
  int items = 0;
  for (int i = 0; i < 2; ++i) {
    const GemmParams& p = *q[i];
    g.p[i] = p;
    g.n_tiles[i] = (p.N + 127) / 128;
    g.per_xcd[i] = (g.n_tiles[i] + kXcds - 1) / kXcds;
    g.S[i] = gemm_splits(p);
    g.nst[i] = p.K / BK;
    items += g.per_xcd[i] * kXcds * g.S[i];
  }
  g.items0 = 0;   // (unused: the kernel takes the second problem first)
  const int n_attn = at.n_split * at.nkv * at.B;
  if (at.hd == 128)
    launch_timed(gemm_attn_chain_kernel<128>, dim3(n_attn + items), dim3(256), 0, s, g, at, n_attn, err);
  else
    launch_timed(gemm_attn_chain_kernel<64>, dim3(n_attn + items), dim3(256), 0, s, g, at, n_attn, err);
  launch_timed(gemm_splitk_reduce_chain_kernel, dim3((unsigned)(((size_t)a.M * a.N + 255) / 256)), dim3(256), 0, s, a,
               g.S[0], b, g.S[1]);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.M < 1 || p.N < 1 || p.K < 1) return hipErrorInvalidValue;
  // (bf16 pairs in or out: the tiled kernel, for more than 64 rows)
  if (!p.a_pairs && !p.c_pairs && skinny_supported(p)) return launch_skinny(p, s);
  if (p.A2) return hipErrorInvalidValue;   // a second K part: skinny launches only
  if (p.a_pairs && !gemm_takes_pairs(p)) return hipErrorInvalidValue;
  if (p.c_pairs && !gemm_writes_pairs(p)) return hipErrorInvalidValue;
  if (p.wdtype == W_BF16) {
    if (p.K % BK != 0 || p.lda % 4 != 0 || (p.swiglu && (p.N % 2 != 0 || p.res))) return hipErrorInvalidValue;
    // 128x128 tiles (32x128 / 64x128 for at most 32 / 64 rows) when they give the device at
    // least one round of work; else the same tiles with K split (gemm_splits); else 64x64
    const int tmr = gemm_tile_rows(p);
    const int big = ((p.M + tmr - 1) / tmr) * ((p.N + 127) / 128);
    const int S = gemm_splits(p);
    if (p.gain && (S < 2 || tmr > 64)) return hipErrorInvalidValue;   // see gemm_norm_fusable
    if (big >= 256 || S > 1) {
      const int tm = (p.M + tmr - 1) / tmr, tiles = big, per = (tiles + kXcds - 1) / kXcds;
      const dim3 grid(per * kXcds, S);
      if (tmr == 32)
        launch_timed(p.gain ? gemm_bf16x2_kernel<32, 128, true> : gemm_bf16x2_kernel<32, 128>, grid, dim3(256), 0, s, p,
                     tm, tiles, per, p.K / BK);
      else if (tmr == 64)
        launch_timed(p.gain ? gemm_bf16x2_kernel<64, 128, true> : gemm_bf16x2_kernel<64, 128>, grid, dim3(256), 0, s,
                     p, tm, tiles, per, p.K / BK);
      else
        launch_timed(p.a_pairs ? gemm_bf16x2_kernel<128, 128, false, true> : gemm_bf16x2_kernel<128, 128>, grid,
                     dim3(256), 0, s, p, tm, tiles, per, p.K / BK);
      if (S > 1) {
        const size_t n_out = (size_t)p.M * (p.swiglu ? p.N / 2 : p.N);
        launch_timed(gemm_splitk_reduce_kernel, dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s, p, S);
      }
    } else {
      const int tm = (p.M + 63) / 64, tiles = tm * ((p.N + 63) / 64), per = (tiles + kXcds - 1) / kXcds;
      launch_timed(p.a_pairs ? gemm_bf16x2_kernel<64, 64, false, true> : gemm_bf16x2_kernel<64, 64>, dim3(per * kXcds),
                   dim3(256), 0, s, p, tm, tiles, per, p.K / BK);
    }
  } else if (p.swiglu || p.gain) {
    return hipErrorInvalidValue;
  } else {
    dim3 grid((p.N + FT - 1) / FT, (p.M + FT - 1) / FT);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ladder

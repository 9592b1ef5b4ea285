// Prefill projections C[M][N] = (R) + A[M][K] . W^T with M = batch x tokens.
//
// bf16: a dense contraction, so it runs on the CDNA4 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate).  A workgroup of 4 waves owns a
// 128x128 tile of C (2x2 waves of 64x64, i.e. 4x4 MFMA tiles each); A and W tiles of
// 128x64 are staged through double-buffered LDS with padded rows so the fragment
// reads of a wave do not collide on banks; the next K step's global loads are in
// flight while the current one is multiplied.
//
// fp32 (small correctness-only models): a plain LDS-tiled VALU GEMM.
#include "common.hpp"
#include "kernels.h"

namespace ladder {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

template <typename WT>
__device__ __forceinline__ const WT* gemm_row(const RowSrc& s, int r, int K) {
  if (s.interleave) return (const WT*)s.m[r & 1] + (size_t)(r >> 1) * K;
  if (r < s.n0) return (const WT*)s.m[0] + (size_t)r * K;
  if (r < s.n1) return (const WT*)s.m[1] + (size_t)(r - s.n0) * K;
  return (const WT*)s.m[2] + (size_t)(r - s.n1) * K;
}

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;

__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const uint16_t* A = (const uint16_t*)p.A;

  // each thread moves 4 16-byte chunks of A and of W per K step
  const uint16_t* arow[4];
  const uint16_t* brow[4];
  int srow[4], scol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    srow[i] = c >> 3;
    scol[i] = (c & 7) * 8;
    const int m = m0 + srow[i], n = n0 + srow[i];
    arow[i] = m < p.M ? A + (size_t)m * p.lda + scol[i] : nullptr;
    brow[i] = n < p.N ? gemm_row<uint16_t>(p.rows, n, p.K) + scol[i] : nullptr;
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = arow[i] ? *(const uint4*)(arow[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
      rb[i] = brow[i] ? *(const uint4*)(brow[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(uint4*)&As[buf][srow[i]][scol[i]] = ra[i];
      *(uint4*)&Bs[buf][srow[i]][scol[i]] = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)&As[cur][wm * 64 + i * 16 + fr][ks + fk];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8*)&Bs[cur][wn * 64 + j * 16 + fr][ks + fk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // C fragment: lane holds rows 4*(lane/16)+r, column lane%16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + fr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (row < p.M && col < p.N) {
          float v = acc[i][j][r];
          if (p.res) v = p.res[(size_t)row * p.ldr + col] + v;
          p.C[(size_t)row * p.ldc + col] = v;
        }
      }
    }
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

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.M < 1 || p.N < 1 || p.K < 1) return hipErrorInvalidValue;
  if (p.wdtype == W_BF16) {
    if (p.K % BK != 0) return hipErrorInvalidValue;
    dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM);
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, s, p);
  } else {
    dim3 grid((p.N + FT - 1) / FT, (p.M + FT - 1) / FT);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ladder

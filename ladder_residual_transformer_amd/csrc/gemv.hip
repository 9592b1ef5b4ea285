// Decode-time projections: bandwidth-bound GEMV y[b][n] = sum_k W[n][k] * u[b][k] for
// batch 1..16, with the module's RMSNorm folded into the prologue and the module's
// tail (RoPE + KV append, SwiGLU, ladder residual add, logits + argmax) in the epilogue.
//
// Layout per block: NT threads own fixed slices of K (VPT 16-byte vectors each), so
// the normalised input u lives in registers for the whole kernel and every weight
// byte is read once with a coalesced 16-byte load.  A block walks row tiles of ROWS
// rows (grid-stride), accumulates in fp32, reduces across its waves through LDS in a
// fixed order (results are bitwise reproducible), and runs the epilogue on the tile.
// When B is large the K dimension is split over blockIdx.y; the last block to finish
// a tile (atomic ticket) sums the slices in slice order and runs the epilogue.
//
// RMSNorm is applied as y = inv_rms * (W . (x * g)), with inv_rms = 1/sqrt(mean(x^2)+eps)
// computed from the same x the block loads.
#include <climits>

#include "common.hpp"
#include "kernels.h"

namespace ladder {

template <typename WT>
__device__ __forceinline__ const WT* row_ptr(const RowSrc& s, int r, int K) {
  if (s.interleave) return (const WT*)s.m[r & 1] + (size_t)(r >> 1) * K;
  if (r < s.n0) return (const WT*)s.m[0] + (size_t)r * K;
  if (r < s.n1) return (const WT*)s.m[1] + (size_t)(r - s.n0) * K;
  return (const WT*)s.m[2] + (size_t)(r - s.n1) * K;
}

template <typename WT, int BT, int ROWS>
__device__ void gemv_epilogue(const GemvParams& p, int row0, const float* fin, const float* inv,
                              int tid, int nt, float* bv, int* bi) {
  const int B = p.B;
  switch (p.epi) {
    case EPI_STORE:
    case EPI_ADD:
    case EPI_LOGITS: {
      for (int i = tid; i < ROWS * BT; i += nt) {
        const int r = i / BT, b = i % BT, n = row0 + r;
        if (n >= p.N || b >= B) continue;
        float y = fin[i] * inv[b];
        if (p.epi == EPI_ADD) y = p.xres[(size_t)b * p.ldr + n] + y;
        p.out[(size_t)b * p.ldo + n] = y;
      }
      if (p.epi == EPI_LOGITS && tid < B && tid < BT) {
        const int b = tid;
        float best = bv[b];
        int idx = bi[b];
        for (int r = 0; r < ROWS; ++r) {
          const int n = row0 + r;
          if (n >= p.N) break;
          const float y = fin[r * BT + b] * inv[b];
          if (y > best) { best = y; idx = n; }
        }
        bv[b] = best;
        bi[b] = idx;
      }
      break;
    }
    case EPI_ADD2: {
      for (int i = tid; i < ROWS * BT; i += nt) {
        const int r = i / BT, b = i % BT, n = row0 + r;
        if (n >= p.N || b >= B) continue;
        const float t = p.xres[(size_t)b * p.ldr + n] + fin[i] * inv[b];
        p.out[(size_t)b * p.ldo + n] = t;
        p.out2[(size_t)b * p.ldo + n] = t + p.add2[(size_t)b * p.ldo + n];
      }
      break;
    }
    case EPI_GATEUP_SWIGLU: {
      for (int i = tid; i < (ROWS / 2) * BT; i += nt) {
        const int r = 2 * (i / BT), b = i % BT, n = row0 + r;
        if (n >= p.N || b >= B) continue;
        const float g = fin[r * BT + b] * inv[b];
        const float up = fin[(r + 1) * BT + b] * inv[b];
        p.out[(size_t)b * p.ldo + (n >> 1)] = silu(g) * up;
      }
      break;
    }
    case EPI_QKV_ROPE: {
      const int pos = *p.d_pos;
      const int half = p.head_dim >> 1;
      for (int i = tid; i < (ROWS / 2) * BT; i += nt) {
        const int r = 2 * (i / BT), b = i % BT, n = row0 + r;
        if (n >= p.N || b >= B) continue;
        float y0 = fin[r * BT + b] * inv[b];
        float y1 = fin[(r + 1) * BT + b] * inv[b];
        if (n < p.q_rows + p.kv_rows) {           // q or k: rotate the adjacent pair
          const int d = (n < p.q_rows ? n : n - p.q_rows) % p.head_dim;
          const float c = p.rope_cos[(size_t)pos * half + (d >> 1)];
          const float s = p.rope_sin[(size_t)pos * half + (d >> 1)];
          rope_rot(y0, y1, c, s);
        }
        if (n < p.q_rows) {
          p.out[(size_t)b * p.ldo + n] = y0;
          p.out[(size_t)b * p.ldo + n + 1] = y1;
        } else {
          const bool isk = n < p.q_rows + p.kv_rows;
          const int rr = isk ? n - p.q_rows : n - p.q_rows - p.kv_rows;
          const int kvh = rr / p.head_dim, d = rr % p.head_dim;
          WT* cache = (WT*)(isk ? p.k_cache : p.v_cache);
          const size_t off = (((size_t)b * p.n_kv + kvh) * p.max_seq + pos) * p.head_dim + d;
          store_w<WT>(cache + off, y0);
          store_w<WT>(cache + off + 1, y1);
        }
      }
      break;
    }
    default:
      break;
  }
}

template <typename WT, int BT, int NT, int VPT, int ROWS>
__global__ __launch_bounds__(NT) void gemv_kernel(GemvParams p) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int NW = NT / 64;
  constexpr int KS = NT * VPT * VEC;
  __shared__ float red[NW][ROWS * BT];
  __shared__ float fin[ROWS * BT];
  __shared__ float sqw[NW][BT];
  __shared__ float slice_sq[BT];
  __shared__ float inv[BT];
  __shared__ float inv2[BT];
  __shared__ float bv[BT];
  __shared__ int bi[BT];
  __shared__ int is_last;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blockIdx.y, S = gridDim.y;
  const int k0 = s * KS;
  const int ntiles = (p.N + ROWS - 1) / ROWS;
  const bool norm = p.gain != nullptr;

  int koff[VPT];
  bool kvalid[VPT];
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    koff[v] = k0 + (tid + v * NT) * VEC;
    kvalid[v] = koff[v] < p.K;
  }
  // Weight loads do not depend on the input, so the first tile's are issued before
  // the prologue and every later tile's right after the previous tile's FMAs: the
  // prologue, the cross-wave reduction and the epilogue run under their latency.
  uint4 w[ROWS][VPT];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int n = tile * ROWS + r;
      const WT* rp = row_ptr<WT>(p.rows, n < p.N ? n : p.N - 1, p.K);
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        if (kvalid[v] && n < p.N) w[r][v] = *(const uint4*)(rp + koff[v]);
        else w[r][v] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  if (blockIdx.x < ntiles) load_tile(blockIdx.x);

  // ---- prologue: this thread's slice of u = x (* g), and sum of squares
  float u[BT][VPT][VEC];
  float sq[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    sq[b] = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) u[b][v][e] = 0.f;
      if (b < p.B && kvalid[v]) {
        const float* xp = p.x + (size_t)b * p.ldx + koff[v];
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const float4 t = *(const float4*)(xp + e);
          u[b][v][e] = t.x; u[b][v][e + 1] = t.y; u[b][v][e + 2] = t.z; u[b][v][e + 3] = t.w;
        }
        if (norm) {
          float g[VEC];
          unpack16(*(const uint4*)((const WT*)p.gain + koff[v]), g);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            sq[b] = fmaf(u[b][v][e], u[b][v][e], sq[b]);
            u[b][v][e] *= g[e];
          }
        }
      }
    }
  }
  if (norm) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const float t = wave_sum(sq[b]);
      if (lane == 0) sqw[wid][b] = t;
    }
  }
  if (tid < BT) { bv[tid] = -INFINITY; bi[tid] = INT_MAX; }
  __syncthreads();
  if (tid < BT) {
    float t = 0.f;
    if (norm)
      for (int q = 0; q < NW; ++q) t += sqw[q][tid];
    slice_sq[tid] = t;
    inv[tid] = norm ? 1.0f / sqrtf(t / (float)p.K + p.eps) : 1.0f;
  }
  __syncthreads();

  // ---- stream row tiles
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int row0 = tile * ROWS;
    float acc[ROWS][BT];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        float wf[VEC];
        unpack16(w[r][v], wf);
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[r][b] = fmaf(wf[e], u[b][v][e], acc[r][b]);
      }
    }
    if (tile + (int)gridDim.x < ntiles) load_tile(tile + gridDim.x);
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const float t = wave_sum(acc[r][b]);
        if (lane == 0) red[wid][r * BT + b] = t;
      }
    __syncthreads();
    if (tid < ROWS * BT) {
      float t = 0.f;
      for (int q = 0; q < NW; ++q) t += red[q][tid];
      fin[tid] = t;
    }
    __syncthreads();

    if (S == 1) {
      gemv_epilogue<WT, BT, ROWS>(p, row0, fin, inv, tid, NT, bv, bi);
    } else {
      if (tid < ROWS * BT) {
        const int r = tid / BT, b = tid % BT, n = row0 + r;
        if (n < p.N && b < p.B) p.part[((size_t)s * p.B + b) * p.N + n] = fin[tid];
      }
      if (tid < BT) p.part_sq[((size_t)tile * S + s) * BT + tid] = slice_sq[tid];
      __threadfence();
      __syncthreads();
      if (tid == 0) is_last = (atomicAdd(&p.counters[tile], 1) == S - 1);
      __syncthreads();
      if (is_last) {
        __threadfence();
        if (tid < ROWS * BT) {
          const int r = tid / BT, b = tid % BT, n = row0 + r;
          float t = 0.f;
          if (n < p.N && b < p.B)
            for (int q = 0; q < S; ++q) t += p.part[((size_t)q * p.B + b) * p.N + n];
          fin[tid] = t;
        }
        if (tid < BT) {
          float t = 0.f;
          for (int q = 0; q < S; ++q) t += p.part_sq[((size_t)tile * S + q) * BT + tid];
          inv2[tid] = norm ? 1.0f / sqrtf(t / (float)p.K + p.eps) : 1.0f;
        }
        if (tid == 0) p.counters[tile] = 0;
        __syncthreads();
        gemv_epilogue<WT, BT, ROWS>(p, row0, fin, inv2, tid, NT, bv, bi);
      }
    }
    __syncthreads();
  }

  // ---- greedy argmax across blocks (lowest index among equal maxima)
  if (p.epi == EPI_LOGITS) {
    const int blk = blockIdx.y * gridDim.x + blockIdx.x, nblk = gridDim.x * gridDim.y;
    if (tid < BT) {
      p.best_val[(size_t)blk * BT + tid] = bv[tid];
      p.best_idx[(size_t)blk * BT + tid] = bi[tid];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(p.arg_counter, 1) == nblk - 1);
    __syncthreads();
    if (is_last) {
      __threadfence();
      // each thread scans a strided subset of the block results, then a tree in LDS;
      // ties resolve to the lower index at every level, so the result is the global
      // first maximum whatever the scan order
      __shared__ float rv[NT];
      __shared__ int ri[NT];
      for (int b = 0; b < p.B && b < BT; ++b) {
        float best = -INFINITY;
        int idx = INT_MAX;
        for (int q = tid; q < nblk; q += NT) {
          const float v = p.best_val[(size_t)q * BT + b];
          const int i = p.best_idx[(size_t)q * BT + b];
          if (v > best || (v == best && i < idx)) { best = v; idx = i; }
        }
        rv[tid] = best;
        ri[tid] = idx;
        __syncthreads();
        for (int o = NT / 2; o > 0; o >>= 1) {
          if (tid < o) {
            const float v = rv[tid + o];
            const int i = ri[tid + o];
            if (v > rv[tid] || (v == rv[tid] && i < ri[tid])) { rv[tid] = v; ri[tid] = i; }
          }
          __syncthreads();
        }
        if (tid == 0) p.next_out[b] = ri[0] == INT_MAX ? 0 : ri[0];
        __syncthreads();
      }
      if (tid == 0) *p.arg_counter = 0;
    }
  }
}

// ------------------------------------------------------------------ host side

namespace {

constexpr int rows_for(int vpt, int bt) {
  int r = 16 / vpt;
  if (r < 2) r = 2;
  int cap = 64 / bt;
  if (cap < 2) cap = 2;
  return r > cap ? cap : r;
}

constexpr int kMaxBlocks = 1024;

constexpr int vpt_cap(int bt, int vec);

struct Pick { int bt, nt, vpt, rows, S, gx; };

Pick pick(int wdtype, int N, int K, int B) {
  Pick k{};
  const int VEC = wdtype == W_BF16 ? 8 : 4;
  k.bt = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16;
  const int nvec = K / VEC;
  const int vpt_max = vpt_cap(k.bt, VEC);
  if (nvec <= 64) { k.nt = 64; k.vpt = 1; }
  else if (nvec <= 128) { k.nt = 128; k.vpt = 1; }
  else {
    k.nt = 256;
    const int need = (nvec + 255) / 256;
    int v = 1;
    while (v < need && v < vpt_max) v <<= 1;
    k.vpt = v;
  }
  k.S = (nvec + k.nt * k.vpt - 1) / (k.nt * k.vpt);
  k.rows = rows_for(k.vpt, k.bt);
  const int tiles = (N + k.rows - 1) / k.rows;
  int cap = kMaxBlocks / k.S;
  if (cap < 1) cap = 1;
  k.gx = tiles < cap ? tiles : cap;
  return k;
}

template <typename WT, int BT, int NT, int VPT>
hipError_t go(const GemvParams& p, const Pick& k, hipStream_t s) {
  constexpr int ROWS = rows_for(VPT, BT);
  launch_timed(gemv_kernel<WT, BT, NT, VPT, ROWS>, dim3(k.gx, k.S), dim3(NT), 0, s, p);
  return hipGetLastError();
}

constexpr int vpt_cap(int bt, int vec) {
  int v = 64 / (vec * bt);
  return v < 1 ? 1 : (v > 8 ? 8 : v);
}

// Only the (threads, vectors-per-thread) shapes pick() can choose for this batch tile
// are instantiated; the thread's slice of u stays within 64 fp32 registers per row.
template <typename WT, int BT>
hipError_t go_bt(const GemvParams& p, const Pick& k, hipStream_t s) {
  constexpr int CAP = vpt_cap(BT, Vec<WT>::N);
  if (k.nt == 64) return go<WT, BT, 64, 1>(p, k, s);
  if (k.nt == 128) return go<WT, BT, 128, 1>(p, k, s);
  if constexpr (CAP >= 8) { if (k.vpt == 8) return go<WT, BT, 256, 8>(p, k, s); }
  if constexpr (CAP >= 4) { if (k.vpt == 4) return go<WT, BT, 256, 4>(p, k, s); }
  if constexpr (CAP >= 2) { if (k.vpt == 2) return go<WT, BT, 256, 2>(p, k, s); }
  return go<WT, BT, 256, 1>(p, k, s);
}

template <typename WT>
hipError_t go_wt(const GemvParams& p, const Pick& k, hipStream_t s) {
  switch (k.bt) {
    case 1: return go_bt<WT, 1>(p, k, s);
    case 2: return go_bt<WT, 2>(p, k, s);
    case 4: return go_bt<WT, 4>(p, k, s);
    case 8: return go_bt<WT, 8>(p, k, s);
    default: return go_bt<WT, 16>(p, k, s);
  }
}

}  // namespace

GemvWorkspaceReq gemv_workspace(int wdtype, int N, int K, int B) {
  const Pick k = pick(wdtype, N, K, B);
  GemvWorkspaceReq r{};
  const size_t tiles = (size_t)(N + k.rows - 1) / k.rows;
  if (k.S > 1) {
    r.part_floats = (size_t)k.S * B * N;
    r.part_sq_floats = tiles * k.S * k.bt;
    r.counters = tiles;
  }
  r.best = (size_t)k.gx * k.S * k.bt;
  return r;
}

hipError_t launch_gemv(const GemvParams& p, hipStream_t s) {
  if (p.B < 1 || p.B > 16 || p.N < 1 || p.K < 1) return hipErrorInvalidValue;
  const Pick k = pick(p.wdtype, p.N, p.K, p.B);
  if (p.wdtype == W_BF16) return go_wt<uint16_t>(p, k, s);
  return go_wt<float>(p, k, s);
}

}  // namespace ladder

// Device code of the row-wave decode GEMV (batch 1..4): one pass of a workgroup over a
// range of row pairs of one projection, with RMSNorm of its input fused, shared by the
// projection launches and the persistent decode-step kernel.
//
// A workgroup (4 waves) owns a contiguous range of row pairs.  It first stages its input
// u = x (* RMSNorm gain) for all batch rows in LDS as fp32 together with
// inv_rms = 1/sqrt(mean(x^2)+eps); every wave then streams whole row pairs: lane l reads
// the 16-byte vectors l, l+64, ... of both rows (coalesced, each weight byte read once),
// multiplies them with u from LDS in fp32, and a wave reduction gives the two dot
// products.  There is no barrier inside the row loop, and the next pair's weight loads
// are issued before the current pair's reduction and epilogue, so their latency
// overlaps.  A row's result depends only on K and the lane mapping, never on which
// workgroup computed it, so every launch shape gives bitwise identical values.
#pragma once
#include <climits>

#include "attn_decode.hpp"
#include "common.hpp"
#include "kernels.h"

namespace ladder {

template <typename WT>
__device__ __forceinline__ const WT* rw_row_ptr(const RowSrc& s, int r, int K) {
  // all three bases are read unconditionally and selected as values: a params struct
  // built in registers then stays in registers
  const WT* m0 = (const WT*)s.m[0];
  const WT* m1 = (const WT*)s.m[1];
  const WT* m2 = (const WT*)s.m[2];
  if (s.interleave) return ((r & 1) ? m1 : m0) + (size_t)(r >> 1) * K;
  const WT* base = r < s.n0 ? m0 : r < s.n1 ? m1 : m2;
  const int off = r < s.n0 ? r : r < s.n1 ? r - s.n0 : r - s.n1;
  return base + (size_t)off * K;
}

// Epilogue of one row pair (rows n0 = 2*pair, n0+1) for batch row b.
template <typename WT>
__device__ __forceinline__ void rw_epilogue(const GemvParams& p, int pair, int b, float y0, float y1, float inv,
                                            float& best, int& bidx) {
  const int n0 = 2 * pair, n1 = n0 + 1;
  const bool v1 = n1 < p.N;
  switch (p.epi) {
    case EPI_STORE:
    case EPI_LOGITS: {
      y0 *= inv;
      y1 *= inv;
      p.out[(size_t)b * p.ldo + n0] = y0;
      if (v1) p.out[(size_t)b * p.ldo + n1] = y1;
      if (p.epi == EPI_LOGITS) {
        if (y0 > best) { best = y0; bidx = n0; }
        if (v1 && y1 > best) { best = y1; bidx = n1; }
      }
      break;
    }
    case EPI_ADD: {
      p.out[(size_t)b * p.ldo + n0] = p.xres[(size_t)b * p.ldr + n0] + y0 * inv;
      if (v1) p.out[(size_t)b * p.ldo + n1] = p.xres[(size_t)b * p.ldr + n1] + y1 * inv;
      break;
    }
    case EPI_ADD2: {
      const float t0 = p.xres[(size_t)b * p.ldr + n0] + y0 * inv;
      p.out[(size_t)b * p.ldo + n0] = t0;
      p.out2[(size_t)b * p.ldo + n0] = t0 + p.add2[(size_t)b * p.ldo + n0];
      if (v1) {
        const float t1 = p.xres[(size_t)b * p.ldr + n1] + y1 * inv;
        p.out[(size_t)b * p.ldo + n1] = t1;
        p.out2[(size_t)b * p.ldo + n1] = t1 + p.add2[(size_t)b * p.ldo + n1];
      }
      break;
    }
    case EPI_GATEUP_SWIGLU:
      p.out[(size_t)b * p.ldo + pair] = silu(y0 * inv) * (y1 * inv);
      break;
    case EPI_QKV_ROPE: {
      y0 *= inv;
      y1 *= inv;
      const int pos = *gbl(p.d_pos);
      if (n0 < p.q_rows + p.kv_rows) {              // q or k: rotate the adjacent pair
        const int d = (n0 < p.q_rows ? n0 : n0 - p.q_rows) % p.head_dim;
        const int half = p.head_dim >> 1;
        const float c = gbl(p.rope_cos)[(size_t)pos * half + (d >> 1)];
        const float s = gbl(p.rope_sin)[(size_t)pos * half + (d >> 1)];
        rope_rot(y0, y1, c, s);
      }
      if (n0 < p.q_rows) {
        p.out[(size_t)b * p.ldo + n0] = y0;
        p.out[(size_t)b * p.ldo + n1] = y1;
      } else {
        const bool isk = n0 < p.q_rows + p.kv_rows;
        const int rr = isk ? n0 - p.q_rows : n0 - p.q_rows - p.kv_rows;
        const int kvh = rr / p.head_dim, d = rr % p.head_dim;
        WT* cache = (WT*)(isk ? p.k_cache : p.v_cache);
        const size_t off = (((size_t)b * p.n_kv + kvh) * p.max_seq + pos) * p.head_dim + d;
        store_w<WT>(cache + off, y0);
        store_w<WT>(cache + off + 1, y1);
      }
      break;
    }
    default:
      break;
  }
}

// Epilogue of one row pair for data read by other workgroups of the same kernel:
// coherent stores (the K/V row as one 32-bit word per rotated pair).
template <typename WT>
__device__ __forceinline__ void rw_epilogue_coh(const GemvParams& p, int pair, int b, float y0, float y1, float inv) {
  const int n0 = 2 * pair;
  switch (p.epi) {
    case EPI_GATEUP_SWIGLU:
      st_coh(p.out + (size_t)b * p.ldo + pair, silu(y0 * inv) * (y1 * inv));
      break;
    case EPI_QKV_ROPE: {
      y0 *= inv;
      y1 *= inv;
      const int pos = *gbl(p.d_pos);
      if (n0 < p.q_rows + p.kv_rows) {
        const int d = (n0 < p.q_rows ? n0 : n0 - p.q_rows) % p.head_dim;
        const int half = p.head_dim >> 1;
        const float c = gbl(p.rope_cos)[(size_t)pos * half + (d >> 1)];
        const float s = gbl(p.rope_sin)[(size_t)pos * half + (d >> 1)];
        rope_rot(y0, y1, c, s);
      }
      if (n0 < p.q_rows) {
        st_coh(p.out + (size_t)b * p.ldo + n0, y0);
        st_coh(p.out + (size_t)b * p.ldo + n0 + 1, y1);
      } else {
        const bool isk = n0 < p.q_rows + p.kv_rows;
        const int rr = isk ? n0 - p.q_rows : n0 - p.q_rows - p.kv_rows;
        const int kvh = rr / p.head_dim, d = rr % p.head_dim;
        WT* cache = (WT*)(isk ? p.k_cache : p.v_cache);
        const size_t off = (((size_t)b * p.n_kv + kvh) * p.max_seq + pos) * p.head_dim + d;
        if constexpr (sizeof(WT) == 2) {
          st_coh((uint32_t*)(cache + off), (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16));
        } else {
          st_coh((float*)(cache + off), y0);
          st_coh((float*)(cache + off) + 1, y1);
        }
      }
      break;
    }
    default:
      break;
  }
}

// What a pass waits for after issuing its first weight unit: nothing, a flag reaching
// an epoch, or progress words reaching a code (see prog_wait).
struct RwWait {
  const int* flag = nullptr;
  int epoch = 0;
  const uint32_t* prog = nullptr;
  int nprog = 0;
  uint32_t code = 0;
  int* err = nullptr;
};

struct RwShared {
  float sqw[4][4];
  float inv[4];
  float wbv[4][4];
  int wbi[4][4];
};

// where a pass puts its rows
// RW_OUT_ADD2_LDSRES: t = res + rows, out = t, out2 = t + dres; res (the residual rows,
// LDS) becomes out2; coherent stores.
enum { RW_OUT_EPI = 0, RW_OUT_LDS = 1, RW_OUT_ADD2_LDS = 2, RW_OUT_ADD2_LDSRES = 3 };

// Vectors of 16 bytes per lane per unit of the row-wave GEMV; a unit covers 64 * kRwVpl
// vectors of two rows.  Fixed, because the chunking is part of the arithmetic.
constexpr int kRwVpl = 4;

// LDS floats of the partial sums of a pass over n_pairs row pairs of K inputs.
__host__ __device__ inline size_t rw_part_floats(int n_pairs, int K, int vec, int BT) {
  const int nvec = K / vec;
  const int nchunk = (nvec + 64 * kRwVpl - 1) / (64 * kRwVpl);
  return (size_t)(n_pairs > 0 ? n_pairs : 0) * nchunk * 2 * BT;
}

// One pass of the row-wave GEMV over row pairs [pr0, pr1) of problem p (this
// workgroup's share).  OUT: the problem's own epilogue; the rows (times inv_rms) into
// dres[row - 2*pr0][b]; or EPI_ADD2 with dres in place of add2.  part: LDS scratch of
// rw_part_floats(pr1 - pr0, p.K, ...) floats.  wt: if it names a flag
// or progress words, the first weight unit is issued, then the workgroup waits for the
// signal before it stages the input.  COH: the outputs are read by other workgroups of
// the same kernel (coherent stores, coherent waits); the input is read with ordinary
// loads, so it must live at addresses that nothing in the kernel read before the
// producers' signal (a cached copy would be stale).
template <typename WT, int BT, int VPL, int OUT, bool COH = false>
__device__ __forceinline__ void rw_pass(const GemvParams& p, int pr0, int pr1, int lb, float* u, float* dres,
                                        const RwWait& wt, RwShared& sh, float* part, float* res = nullptr,
                                        uint4* wpre = nullptr) {
  constexpr int VEC = Vec<WT>::N;
  constexpr int CHUNK = 64 * VPL;                 // vectors of a row one wave covers per step
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int K = p.K, B = p.B;
  const int nvec = K / VEC;
  const int nchunk = (nvec + CHUNK - 1) / CHUNK;

  // The workgroup's work is (pair, chunk) units, unit j*nchunk + c being chunk c (CHUNK
  // vectors of 16 bytes) of pair pr0 + j; wave w takes units w, w+4, w+8, ... so that
  // its share differs from the others' by at most one unit.  Two register buffers form
  // a pipeline: the loads of the wave's next unit are in flight while its current one is
  // multiplied.  Each unit's two partial dot products per batch row go to part[] (LDS);
  // after a barrier every (pair, batch row) sums its chunks in chunk order and runs the
  // epilogue.  The sums depend only on K and CHUNK, so every launch shape and schedule
  // gives the same bits.  Loads are unconditional (addresses clamped into the matrix) so
  // that no branch separates a load from its use; lanes past the end of a row read the
  // zero pad of u instead, and a missing odd row is discarded by the epilogue.
  const int n_pairs = pr1 > pr0 ? pr1 - pr0 : 0;
  const int total_units = n_pairs * nchunk;
  const int n_units = total_units > wid ? (total_units - wid + 3) / 4 : 0;
  uint4 wa[2][VPL], wb[2][VPL];
  // Every load is issued unconditionally: a unit index past the wave's last unit loads
  // one vector of a valid row for all lanes (a dummy, never used), so that no branch
  // separates a load from its use and the compiler keeps both buffers in flight (with a
  // conditional load it waits for every outstanding load before issuing the next unit).
  const int pclamp = min(pr0, (p.N + 1) / 2 - 1);
  auto load_unit = [&](uint4 (&w)[2][VPL], int i) {
    const bool real = i < n_units;
    const int un = real ? wid + 4 * i : 0;
    const int pair = real ? pr0 + un / nchunk : pclamp, c = un % nchunk;
    const int n0 = 2 * pair;
    const WT* r0 = rw_row_ptr<WT>(p.rows, n0, K);
    const WT* r1 = rw_row_ptr<WT>(p.rows, min(n0 + 1, p.N - 1), K);
    const int li = real ? lane : 0, vs = real ? 64 : 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = min(c * CHUNK + li + vs * v, nvec - 1);
      w[0][v] = ldg4u_nt(r0 + (size_t)vi * VEC);
      w[1][v] = ldg4u_nt(r1 + (size_t)vi * VEC);
    }
  };
  const int ustride = K + VEC;                     // u rows carry a zero pad of VEC floats

  // wpre (LDS, with a wait): before waiting, each wave copies all of its units into LDS by
  // direct global-to-LDS loads (slot s of unit un, row r: 64 lanes x 16 B at
  // wpre + ((un * spu + s) * 2 + r) * 64), and computes them from there afterwards
  const int spu = nvec < 64 * VPL ? (nvec + 63) / 64 : VPL;
  const bool waits = wt.flag != nullptr || wt.prog != nullptr;
  if (waits && wpre) {
    for (int i = 0; i < n_units; ++i) {
      const int un = wid + 4 * i;
      const int pair = pr0 + un / nchunk, c = un % nchunk;
      const WT* r0 = rw_row_ptr<WT>(p.rows, 2 * pair, K);
      const WT* r1 = rw_row_ptr<WT>(p.rows, min(2 * pair + 1, p.N - 1), K);
      for (int v = 0; v < spu; ++v) {
        const int vi = min(c * CHUNK + lane + 64 * v, nvec - 1);
        uint4* slot = wpre + ((size_t)(un * spu + v) * 2) * 64;
        __builtin_amdgcn_global_load_lds((const void*)(r0 + (size_t)vi * VEC),
                                         (__attribute__((address_space(3))) void*)slot, 16, 0, 2);
        __builtin_amdgcn_global_load_lds((const void*)(r1 + (size_t)vi * VEC),
                                         (__attribute__((address_space(3))) void*)(slot + 64), 16, 0, 2);
      }
    }
  }
  if (waits) {
    if (!wpre) {
      load_unit(wa, 0);
      load_unit(wb, 1);
    }
    if (wt.prog) prog_wait(wt.prog, wt.nprog, wt.code, wt.err);
    else if constexpr (COH) wg_wait_coh(wt.flag, wt.epoch, wt.err);
    else wg_wait(wt.flag, wt.epoch, wt.err);
  }
  // ---- prologue: u = x (* g) for every batch row, and inv_rms.  For one batch row and
  // K <= 256*4*VEC the input loads are issued before the first weight unit, so the
  // in-order completion of loads does not make the prologue wait for the weights.
  const bool norm = p.gain != nullptr;
  if (tid < B * VEC) u[(tid / VEC) * ustride + K + tid % VEC] = 0.f;
  if (BT == 1 && nvec <= 256 * 4) {
    float4 xr[4][VEC / 4];
    uint4 gr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = min(tid + 256 * i, nvec - 1);
#pragma unroll
      for (int e = 0; e < VEC / 4; ++e)
        xr[i][e] = ldg4(p.x + (size_t)v * VEC + 4 * e);
      gr[i] = norm ? ldg4u((const WT*)p.gain + (size_t)v * VEC) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (!waits) {
      load_unit(wa, 0);
      load_unit(wb, 1);
    }
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + 256 * i;
      if (v < nvec) {
        float xv[VEC], g[VEC];
#pragma unroll
        for (int e = 0; e < VEC / 4; ++e) {
          xv[4 * e] = xr[i][e].x; xv[4 * e + 1] = xr[i][e].y; xv[4 * e + 2] = xr[i][e].z; xv[4 * e + 3] = xr[i][e].w;
        }
        if (norm) {
          unpack16(gr[i], g);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            sq = fmaf(xv[e], xv[e], sq);
            xv[e] *= g[e];
          }
        }
        float* up = u + (size_t)v * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) *(float4*)(up + e) = make_float4(xv[e], xv[e + 1], xv[e + 2], xv[e + 3]);
      }
    }
    sq = wave_sum(sq);
    if (lane == 0) sh.sqw[wid][0] = sq;
  } else {
    if (!waits) {
      load_unit(wa, 0);
      load_unit(wb, 1);
    }
    for (int b = 0; b < BT; ++b) {
      float sq = 0.f;
      if (b < B) {
        for (int v = tid; v < nvec; v += 256) {
          const float* xg = p.x + (size_t)b * p.ldx + (size_t)v * VEC;
          float xv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; e += 4) {
            const float4 t = ldg4(xg + e);
            xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
          }
          if (norm) {
            float g[VEC];
            unpack16(ldg4u((const WT*)p.gain + (size_t)v * VEC), g);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              sq = fmaf(xv[e], xv[e], sq);
              xv[e] *= g[e];
            }
          }
          float* up = u + (size_t)b * ustride + (size_t)v * VEC;
#pragma unroll
          for (int e = 0; e < VEC; e += 4) *(float4*)(up + e) = make_float4(xv[e], xv[e + 1], xv[e + 2], xv[e + 3]);
        }
      }
      sq = wave_sum(sq);
      if (lane == 0) sh.sqw[wid][b] = sq;
    }
  }
  __syncthreads();
  if (tid < BT) {
    const float t = ((sh.sqw[0][tid] + sh.sqw[1][tid]) + sh.sqw[2][tid]) + sh.sqw[3][tid];
    sh.inv[tid] = norm ? 1.0f / sqrtf(t / (float)K + p.eps) : 1.0f;
  }
  __syncthreads();
  float inv_b[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) inv_b[b] = sh.inv[b];

  // ---- units
  auto compute_unit = [&](const uint4 (&w)[2][VPL], int i) {
    const int un = wid + 4 * i;
    const int c = un % nchunk;
    float acc[2][BT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = c * CHUNK + lane + 64 * v;
      const int ui = (vi < nvec ? vi : nvec) * VEC;    // past the row end: the zero pad
      float w0[VEC], w1[VEC];
      unpack16(w[0][v], w0);
      unpack16(w[1][v], w1);
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if (b < B) {
          const float* up = u + (size_t)b * ustride + ui;
          float uv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; e += 4) {
            const float4 t = *(const float4*)(up + e);
            uv[e] = t.x; uv[e + 1] = t.y; uv[e + 2] = t.z; uv[e + 3] = t.w;
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            acc[0][b] = fmaf(w0[e], uv[e], acc[0][b]);
            acc[1][b] = fmaf(w1[e], uv[e], acc[1][b]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const float y = wave_sum(acc[r][b]);
        if (lane == 0 && i < n_units) part[((size_t)un * 2 + r) * BT + b] = y;
      }
  };
  if (waits && wpre) {
    wave_stores_done_fwd();                        // this wave's copies have landed
    for (int i = 0; i < n_units; ++i) {
      const int un = wid + 4 * i;
      uint4 w[2][VPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if (v < spu) {
          const uint4* slot = wpre + ((size_t)(un * spu + v) * 2) * 64;
          w[0][v] = slot[lane];
          w[1][v] = slot[64 + lane];
        } else {
          w[0][v] = make_uint4(0u, 0u, 0u, 0u);    // past every row end (u reads the zero pad)
          w[1][v] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      compute_unit(w, i);
    }
  } else {
    // units i and i + 1 are in flight at the top of each iteration; a past-the-end unit
    // is computed on its dummy load and its sums are dropped
    for (int i = 0; i < n_units; i += 2) {
      compute_unit(wa, i);
      load_unit(wa, i + 2);
      compute_unit(wb, i + 1);
      load_unit(wb, i + 3);
    }
  }
  __syncthreads();

  // ---- epilogues: thread t finishes pair pr0 + t / BT for batch row t % BT
  float best = -INFINITY;
  int bidx = INT_MAX;
  for (int t = tid; t < n_pairs * BT; t += 256) {
    const int j = t / BT, b = t % BT;
    if (b >= B) continue;
    const int pair = pr0 + j;
    float y0 = 0.f, y1 = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      y0 += part[((size_t)(j * nchunk + c) * 2 + 0) * BT + b];
      y1 += part[((size_t)(j * nchunk + c) * 2 + 1) * BT + b];
    }
    if constexpr (OUT == RW_OUT_EPI) {
      if constexpr (COH) rw_epilogue_coh<WT>(p, pair, b, y0, y1, inv_b[b]);
      else rw_epilogue<WT>(p, pair, b, y0, y1, inv_b[b], best, bidx);
    } else if constexpr (OUT == RW_OUT_LDS) {
      const int r = 2 * j;
      dres[r * BT + b] = y0 * inv_b[b];
      dres[(r + 1) * BT + b] = y1 * inv_b[b];
    } else if constexpr (OUT == RW_OUT_ADD2_LDSRES) {
      const int r = 2 * j, n0 = 2 * pair;
      const float t0 = res[r * BT + b] + y0 * inv_b[b];
      const float s0 = t0 + dres[r * BT + b];
      res[r * BT + b] = s0;
      st_coh(p.out + (size_t)b * p.ldo + n0, t0);
      st_coh(p.out2 + (size_t)b * p.ldo + n0, s0);
      if (n0 + 1 < p.N) {
        const float t1 = res[(r + 1) * BT + b] + y1 * inv_b[b];
        const float s1 = t1 + dres[(r + 1) * BT + b];
        res[(r + 1) * BT + b] = s1;
        st_coh(p.out + (size_t)b * p.ldo + n0 + 1, t1);
        st_coh(p.out2 + (size_t)b * p.ldo + n0 + 1, s1);
      }
    } else if constexpr (COH) {                    // EPI_ADD2, second addend from dres
      const int r = 2 * j, n0 = 2 * pair;
      const float t0 = ld_coh(p.xres + (size_t)b * p.ldr + n0) + y0 * inv_b[b];
      st_coh(p.out + (size_t)b * p.ldo + n0, t0);
      st_coh(p.out2 + (size_t)b * p.ldo + n0, t0 + dres[r * BT + b]);
      if (n0 + 1 < p.N) {
        const float t1 = ld_coh(p.xres + (size_t)b * p.ldr + n0 + 1) + y1 * inv_b[b];
        st_coh(p.out + (size_t)b * p.ldo + n0 + 1, t1);
        st_coh(p.out2 + (size_t)b * p.ldo + n0 + 1, t1 + dres[(r + 1) * BT + b]);
      }
    } else {
      const int r = 2 * j, n0 = 2 * pair;
      const float t0 = p.xres[(size_t)b * p.ldr + n0] + y0 * inv_b[b];
      p.out[(size_t)b * p.ldo + n0] = t0;
      p.out2[(size_t)b * p.ldo + n0] = t0 + dres[r * BT + b];
      if (n0 + 1 < p.N) {
        const float t1 = p.xres[(size_t)b * p.ldr + n0 + 1] + y1 * inv_b[b];
        p.out[(size_t)b * p.ldo + n0 + 1] = t1;
        p.out2[(size_t)b * p.ldo + n0 + 1] = t1 + dres[(r + 1) * BT + b];
      }
    }
  }

  if (OUT == RW_OUT_EPI && p.epi == EPI_LOGITS) {
    // per-block greedy candidate (lowest index among equal maxima), merged by
    // argmax_finalize: lanes l and l ^ o (o a multiple of BT) hold the same batch row
#pragma unroll
    for (int o = 32; o >= BT; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bidx, o, 64);
      if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    }
    if (lane < BT) { sh.wbv[wid][lane] = best; sh.wbi[wid][lane] = bidx; }
    __syncthreads();
    if (tid < BT) {
      float bb = sh.wbv[0][tid];
      int ii = sh.wbi[0][tid];
      for (int q = 1; q < 4; ++q)
        if (sh.wbv[q][tid] > bb || (sh.wbv[q][tid] == bb && sh.wbi[q][tid] < ii)) { bb = sh.wbv[q][tid]; ii = sh.wbi[q][tid]; }
      p.best_val[(size_t)lb * BT + tid] = bb;
      p.best_idx[(size_t)lb * BT + tid] = ii;
    }
  }
}

}  // namespace ladder

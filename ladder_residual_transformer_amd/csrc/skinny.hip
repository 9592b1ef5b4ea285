// Skinny projections C[M][N] = (R) + A[M][K] . W^T for M <= 32 rows (a decode step of a
// batch beyond the row-wave GEMV, or a short prefill chunk), bf16 weights.
//
// The work is weight streaming: every weight row is read once, the M activation rows are
// small.  A workgroup owns a tile of 128 weight rows and one slice of K; its four waves own
// 32 rows each (two 16-row MFMA tiles).  Weights are read with coalesced nontemporal
// 16-byte loads, each instruction covering 2 rows x 512 contiguous bytes (4 x 256 for the
// 128-wide chunks): loading them straight in the A-operand layout of
// v_mfma_f32_16x16x32_bf16 (16 rows x 64 bytes per instruction) streamed at ~5.0 TB/s
// against ~6.5 for this pattern on the part.  Each wave then passes a 16-row unit through
// an LDS buffer of its own (16-byte pieces at XOR-swizzled slots, so that neither the
// writes nor the operand reads conflict on a bank) and reads the A operands back: lane l
// holds row l % 16, eight consecutive k at 8 (l / 16) of each 32-wide K step.  The weights
// of the next K chunk are in flight while the current one is multiplied.  The activations
// of a chunk are staged in LDS (double-buffered) as bf16 pairs hi = bf16(a),
// lo = bf16(a - hi) with the RMSNorm gain folded in where asked; each product is two MFMAs,
// lo.W then hi.W, into one fp32 accumulator.  The rows of the pairs are padded so that the
// B-operand reads of a wave cover every LDS bank once.
//
// K is cut into slices, a function of the problem's own shape only; each slice writes its
// fp32 partial tile (and, with the RMSNorm fold, its rows' sums of squares) to the
// workspace with coherent stores, and the last workgroup of a tile to arrive (ticket) sums
// the partials in slice order and runs the epilogue: 1/rms scaling, SwiGLU, the residual
// add, or for a problem of two K parts (the O and down projections of a ladder layer, over
// the attention and the SwiGLU outputs) C = R + A.W^T then C2 = C + A2.W2^T.  A launch may
// hold two problems (QKV and gate/up of a ladder layer); each gives the bits of its own
// launch, and the result does not depend on the arrival order.
#include <type_traits>

#include "attn_decode.hpp"
#include "common.hpp"
#include "kernels.h"

namespace ladder {

namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kSkRows = 128;        // weight rows per tile
constexpr int kSkXcds = 8;
constexpr int kSkMaxM = 32;
// K slices of a problem at most: the epilogue loads every slice of each of a thread's
// items (M / 8 at most) in one round, 32 partial float4s, and one sum of squares per thread
constexpr int sk_max_slices(int M) { return M <= 16 ? 16 : 8; }

// Coherent (agent-scope) 16-byte accesses as two 8-byte atomics: the partial tiles cross
// workgroups (and XCDs) within the launch.
__device__ __forceinline__ void st_coh16(float* p, float4 v) {
  unsigned long long* q = (unsigned long long*)p;
  __hip_atomic_store(gbl(q), __builtin_bit_cast(unsigned long long, make_float2(v.x, v.y)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(gbl(q + 1), __builtin_bit_cast(unsigned long long, make_float2(v.z, v.w)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ld_coh16(const float* p) {
  const unsigned long long* q = (const unsigned long long*)p;
  const float2 a = __builtin_bit_cast(float2, __hip_atomic_load(gbl(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const float2 b =
      __builtin_bit_cast(float2, __hip_atomic_load(gbl(q + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return make_float4(a.x, a.y, b.x, b.y);
}

template <int MT>
struct Sk {
  static constexpr int KC = MT == 1 ? 256 : 128;   // k per chunk
  static constexpr int EPL = KC / 32;              // 16-byte weight loads per lane per 16-row unit
  static constexpr int LPR = KC / 8;               // lanes per weight row in a load instruction
  static constexpr int RPI = 64 / LPR;             // weight rows per load instruction
  static constexpr int LDX = KC + 8;               // bf16 per LDS activation row (16 bytes of pad)
  static constexpr int ROWS = MT * 16;             // activation rows staged (M padded)
  static constexpr int XV = ROWS * KC / 4 / 256;   // float4 of activations per thread per chunk
  static constexpr int TPR = KC / 4;               // threads per activation row in the staging
};
static_assert(Sk<1>::EPL * Sk<1>::RPI == 16 && Sk<2>::EPL * Sk<2>::RPI == 16, "a unit is 16 rows");

// Row r of the virtual weight matrix (selects, not an indexed load of the argument block).
__device__ __forceinline__ const uint16_t* sk_row(const RowSrc& s, int r, int K) {
  const uint16_t* m0 = (const uint16_t*)s.m[0];
  const uint16_t* m1 = (const uint16_t*)s.m[1];
  const uint16_t* m2 = (const uint16_t*)s.m[2];
  if (s.interleave) return ((r & 1) ? m1 : m0) + (size_t)(r >> 1) * K;
  const uint16_t* base = r < s.n0 ? m0 : r < s.n1 ? m1 : m2;
  const int i = r < s.n0 ? r : r < s.n1 ? r - s.n0 : r - s.n1;
  return base + (size_t)i * K;
}

// A problem of a launch: its parameters, tiles, slices of each K part and K per slice.
struct SkProb {
  GemmParams g;
  int nt, S0, S1, ks0, ks1;
};
struct SkArgs {
  SkProb p[2];
  int items0, items, per_xcd;   // work items of problem 0, of the launch
  // The decode attention in the launch (HDA != 0): blocks [0, items0) are the QKV items,
  // blocks [items0, items0 + n_attn) run split-KV attention workgroups, which wait until
  // every QKV tile's last workgroup has published `code` (epoch * kSeqCodeStride + tag) in
  // prog[tile] after its coherent q and K/V stores, and the remaining blocks are the
  // second problem's items, per1 per XCD.
  AttnDecodeParams at;
  int n_attn, per1, tag;
  uint32_t* prog;
  int* err;
};

// NORM: RMSNorm folded in (A the raw rows, multiplied by the gain on the way into LDS).
// HDA: head dimension of the attention in the launch (0: none).
template <int MT, bool NORM, int HDA = 0>
__global__ __launch_bounds__(256, 2) void skinny_kernel(SkArgs args) {
  using C = Sk<MT>;
  struct SkL {
    uint16_t xs[2][2][C::ROWS * C::LDX];   // [buffer][hi, lo][row][k]
    uint16_t wt[4][16 * C::KC];            // per wave: one 16-row unit
  };
  constexpr size_t kAttB = HDA ? sizeof(AttnLds<uint16_t, HDA ? HDA : 64>) : 0;
  __shared__ __align__(16) char lds_u[sizeof(SkL) > kAttB ? sizeof(SkL) : kAttB];
  int item0;
  if constexpr (HDA != 0) {
    const int bi = (int)blockIdx.x;
    if (bi < args.items0) {
      item0 = bi;
    } else if (bi < args.items0 + args.n_attn) {
      const uint32_t code = (uint32_t)*gbl(args.at.d_epoch) * kSeqCodeStride + (uint32_t)args.tag;
      attn_decode_block_mfma<HDA, true>(args.at, bi - args.items0, *reinterpret_cast<AttnLds<uint16_t, HDA>*>(lds_u),
                                        args.prog, args.p[0].nt, code, args.err);
      return;
    } else {
      const int li = bi - args.items0 - args.n_attn;
      const int it = (li % kSkXcds) * args.per1 + li / kSkXcds;
      if (it >= args.items - args.items0) return;
      item0 = args.items0 + it;
    }
  } else {
    item0 = (int)(blockIdx.x % kSkXcds) * args.per_xcd + (int)(blockIdx.x / kSkXcds);
    if (item0 >= args.items) return;
  }
  const bool second = item0 >= args.items0;
  const SkProb& P = second ? args.p[1] : args.p[0];
  const GemmParams& p = P.g;
  const int item = item0 - (second ? args.items0 : 0);
  const int nt = P.nt, S0 = P.S0, S = P.S0 + P.S1;
  const int slice = item / nt, tile = item % nt;
  // the K part this slice belongs to
  const bool part1 = slice >= S0;
  const int K = part1 ? p.K2 : p.K, ks = part1 ? P.ks1 : P.ks0, lda = part1 ? p.lda2 : p.lda;
  const float* A = (const float*)(part1 ? p.A2 : p.A);
  RowSrc rows;
#pragma unroll
  for (int i = 0; i < 3; ++i) rows.m[i] = part1 ? p.rows2.m[i] : p.rows.m[i];
  rows.n0 = part1 ? p.rows2.n0 : p.rows.n0;
  rows.n1 = part1 ? p.rows2.n1 : p.rows.n1;
  rows.interleave = part1 ? p.rows2.interleave : p.rows.interleave;
  const int kbeg = (part1 ? slice - S0 : slice) * ks, kend = min(K, kbeg + ks);
  const int nch = (kend - kbeg + C::KC - 1) / C::KC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rpos = p.rope_q ? *gbl(p.d_pos) : 0;   // RoPE epilogue: the position (used at the end)
  // attention in the launch: the code the QKV tiles publish
  const uint32_t pcode = HDA != 0 && p.rope_q ? (uint32_t)*gbl(args.at.d_epoch) * kSeqCodeStride + (uint32_t)args.tag : 0u;

  auto& xs = reinterpret_cast<SkL*>(lds_u)->xs;
  auto& wt = reinterpret_cast<SkL*>(lds_u)->wt;
  __shared__ float inv_s[kSkMaxM];
  __shared__ int last_s;

  // ---- weights: load i of row tile rt covers unit rows i*RPI + lane/LPR (of the wave's
  // rows tile*128 + 32*wave + 16*rt + ...), 16-byte piece lane % LPR of the chunk
  const int r16 = lane & 15, g = lane >> 4;
  const int lrow = lane / C::LPR, lkb = lane % C::LPR;
  // The rows of a 16-row unit lie in one matrix of the row source (its segment bounds are
  // multiples of 16, and N too), so each lane's rows are one pointer plus i times a fixed
  // stride.  A unit past N reads the last unit instead (its results are never stored).
  const uint16_t* wp[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int u0 = min(tile * kSkRows + 32 * wave + 16 * rt, p.N - 16);
    wp[rt] = sk_row(rows, u0 + lrow, K);
  }
  const size_t wstride = (size_t)(rows.interleave ? C::RPI / 2 : C::RPI) * K;
  // Ring of two units in registers: slot rt holds row tile rt of the chunk being
  // multiplied, and is refilled with the next chunk's row tile rt right after its use.
  uint4 w[2][C::EPL];
  auto wload = [&](auto RT, int c) {
    constexpr int rt = decltype(RT)::value;
    const int k = min(kbeg + c * C::KC + 8 * lkb, K - 8);   // past K: a valid vector, met by zero activations
#pragma unroll
    for (int i = 0; i < C::EPL; ++i) w[rt][i] = ldg4u_nt(wp[rt] + i * wstride + k);
  };
  // unit row r, 16-byte piece kb sits at slot kb ^ (r % 16) of row r in the wave's buffer
  uint16_t* wtw = wt[wave];

  // ---- activations: thread covers row (tid + 256 i) / TPR, float4 column (tid + 256 i) % TPR
  const uint16_t* gain = (const uint16_t*)p.gain;
  float4 xr[C::XV];
  uint2 gr[C::XV];         // NORM: the gain of each float4 (4 x bf16), loaded with it
  float sq[C::XV];
#pragma unroll
  for (int i = 0; i < C::XV; ++i) sq[i] = 0.f;
  auto xload = [&](int c) {
    const int cc = min(c, nch - 1);
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      const int f = tid + 256 * i, row = f / C::TPR, k = min(kbeg + cc * C::KC + 4 * (f % C::TPR), K - 4);
      xr[i] = *(const float4*)(A + (size_t)min(row, p.M - 1) * lda + k);
      if constexpr (NORM) gr[i] = *(const uint2*)(gain + k);
    }
  };
  auto xstore = [&](int buf, int c) {
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      const int f = tid + 256 * i, row = f / C::TPR, kk = 4 * (f % C::TPR);
      const int k = kbeg + c * C::KC + kk;
      float4 a = xr[i];
      if (row >= p.M || k >= kend) a = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (NORM) {
        sq[i] += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
        const uint2 gv = gr[i];
        a.x *= __uint_as_float(gv.x << 16);
        a.y *= __uint_as_float(gv.x & 0xffff0000u);
        a.z *= __uint_as_float(gv.y << 16);
        a.w *= __uint_as_float(gv.y & 0xffff0000u);
      }
      uint32_t h0, l0, h1, l1;
      split_bf2(a.x, a.y, h0, l0);
      split_bf2(a.z, a.w, h1, l1);
      *(uint2*)&xs[buf][0][row * C::LDX + kk] = make_uint2(h0, h1);
      *(uint2*)&xs[buf][1][row * C::LDX + kk] = make_uint2(l0, l1);
    }
  };

  f32x4 acc[2][MT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk: multiply each row tile's unit by the activations of LDS buffer c & 1; with
  // PF (every chunk but the last) refill the unit's slot with the next chunk right after
  // its use, then stage the next chunk's activations and load the ones after it.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto unit = [&](auto RT, int cur) {
    constexpr int rt = decltype(RT)::value;
    // the unit through the wave's LDS buffer: coalesced pieces in, A operands out (one
    // wave's LDS accesses complete in order, so no barrier is needed)
#pragma unroll
    for (int i = 0; i < C::EPL; ++i) {
      const int r = i * C::RPI + lrow;
      *(uint4*)&wtw[r * C::KC + 8 * (lkb ^ (r & 15))] = w[rt][i];
    }
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) {
      const bf16x8 a = *(const bf16x8*)&wtw[r16 * C::KC + 8 * ((4 * e + g) ^ r16)];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int xo = (mt * 16 + r16) * C::LDX + 32 * e + 8 * g;
        const bf16x8 xh = *(const bf16x8*)&xs[cur][0][xo];
        const bf16x8 xl = *(const bf16x8*)&xs[cur][1][xo];
        acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xl, acc[rt][mt], 0, 0, 0);
        acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xh, acc[rt][mt], 0, 0, 0);
      }
    }
  };
  auto chunk = [&](auto PF, int c) {
    constexpr bool pf = decltype(PF)::value;
    const int cur = c & 1;
    unit(I0{}, cur);
    if constexpr (pf) wload(I0{}, c + 1);
    unit(I1{}, cur);
    if constexpr (pf) {
      wload(I1{}, c + 1);
      xstore(cur ^ 1, c + 1);
      xload(c + 2);
    }
    __syncthreads();
  };

  // prologue: activations of chunk 0 first (they gate the first product), then the
  // weights of chunk 0, then the activations of chunk 1
  xload(0);
  wload(I0{}, 0);
  wload(I1{}, 0);
  xstore(0, 0);
  xload(1);
  __syncthreads();
  for (int c = 0; c + 1 < nch; ++c) chunk(std::true_type{}, c);
  chunk(std::false_type{}, nch - 1);

  // ---- partial tile: lane holds rows n = 4 (lane/16) + j, column m = lane % 16
  const size_t plane = (size_t)p.M * p.N;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int n = tile * kSkRows + 32 * wave + 16 * rt + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      if (m < p.M && n < p.N)
        st_coh16(p.ws + slice * plane + (size_t)m * p.N + n,
                 make_float4(acc[rt][mt][0], acc[rt][mt][1], acc[rt][mt][2], acc[rt][mt][3]));
    }
  }
  float* sqs = p.ws + (size_t)S * plane;   // [ntiles][S][M] sums of squares of the raw rows
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < C::XV; ++i) {
      float v = sq[i];
#pragma unroll
      for (int o = C::TPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      const int row = (tid + 256 * i) / C::TPR;
      if ((tid % C::TPR) == 0 && row < p.M) st_coh(sqs + ((size_t)tile * S + slice) * p.M + row, v);
    }
  }
  // The partials are coherent stores (they bypass the per-XCD caches): once every wave's
  // stores have completed the workgroup takes its ticket, and the last one reads them back
  // with coherent loads; no cache write-back or invalidate is needed.
  wave_stores_done_fwd();
  __syncthreads();
  if (tid == 0)
    last_s = __hip_atomic_fetch_add(gbl(p.cnt + tile), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!last_s) return;

  // ---- epilogue: thread item = (row m, 4 consecutive columns n), items tid + 256 jj.
  // Every partial of the thread's items and one row's sum of squares of one slice are
  // loaded in one round (one memory round trip); each item's slices are then added in
  // slice order (part 0, then part 1).
  constexpr int IPT = MT == 1 ? 2 : 4, SM = MT == 1 ? 16 : 8;   // items per thread, slices
  const int n_base = tile * kSkRows;
  const int n_items = p.M * (kSkRows / 4);
  float4 t[IPT][SM];
  float4 rcs[IPT];   // RoPE epilogue: cos and sin of the item's two pairs (c0, s0, c1, s1)
  const int rq = p.nq * p.hd, rk = p.nkv * p.hd;
#pragma unroll
  for (int jj = 0; jj < IPT; ++jj) {
    const int it = tid + 256 * jj;
    const int m = it / (kSkRows / 4), n = n_base + 4 * (it % (kSkRows / 4));
    const bool ok = it < n_items && n < p.N;
#pragma unroll
    for (int q = 0; q < SM; ++q)
      if (ok && q < S) t[jj][q] = ld_coh16(p.ws + q * plane + (size_t)m * p.N + n);
    rcs[jj] = make_float4(1.f, 0.f, 1.f, 0.f);
    if (p.rope_q && ok && n < rq + rk) {
      const int d = (n < rq ? n : n - rq) % p.hd;
      const size_t at = (size_t)rpos * (p.hd / 2) + d / 2;
      const float2 c = *(const float2*)(p.rope_cos + at), sn = *(const float2*)(p.rope_sin + at);
      rcs[jj] = make_float4(c.x, sn.x, c.y, sn.y);
    }
  }
  float* red = (float*)&xs[0][0][0];   // the staging buffers are free now
  if constexpr (NORM) {
    // row tid % M's sum of squares of slice tid / M, added in slice order below
    const float v = tid < S * p.M ? ld_coh(sqs + (size_t)tile * S * p.M + tid) : 0.f;
    if (tid < S * p.M) red[tid] = v;
    __syncthreads();
    if (tid < p.M) {
      float sum = 0.f;
      for (int q = 0; q < S; ++q) sum += red[q * p.M + tid];
      inv_s[tid] = 1.0f / sqrtf(sum / (float)p.K + p.eps);
    }
  } else if (tid < p.M) {
    inv_s[tid] = 1.f;
  }
  if (tid == 0) __hip_atomic_store(gbl(p.cnt + tile), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();

#pragma unroll
  for (int jj = 0; jj < IPT; ++jj) {
    const int it = tid + 256 * jj;
    const int m = it / (kSkRows / 4), n = n_base + 4 * (it % (kSkRows / 4));
    if (it >= n_items || n >= p.N) continue;
    float4 v0 = t[jj][0], v1 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 1; q < SM; ++q) {
      if (q >= S) continue;
      if (q < S0) {
        v0.x += t[jj][q].x; v0.y += t[jj][q].y; v0.z += t[jj][q].z; v0.w += t[jj][q].w;
      } else if (q == S0) {
        v1 = t[jj][q];
      } else {
        v1.x += t[jj][q].x; v1.y += t[jj][q].y; v1.z += t[jj][q].z; v1.w += t[jj][q].w;
      }
    }
    const float inv = inv_s[m];
    float4 o = make_float4(v0.x * inv, v0.y * inv, v0.z * inv, v0.w * inv);
    if (p.rope_q) {
      // rope_kv's arithmetic on the same fp32 values: rotate the q and k pairs (d, d + 1),
      // q to rope_q, k and v rounded to bf16 into the caches
      if (n < rq + rk) {
        rope_rot(o.x, o.y, rcs[jj].x, rcs[jj].y);
        rope_rot(o.z, o.w, rcs[jj].z, rcs[jj].w);
      }
      // with the attention in the launch its readers are other workgroups: coherent stores
      if (n < rq) {
        float* dq = p.rope_q + (size_t)m * rq + n;
        if constexpr (HDA != 0) st_coh16(dq, o);
        else *(float4*)dq = o;
      } else {
        const bool isk = n < rq + rk;
        const int r = isk ? n - rq : n - rq - rk, kvh = r / p.hd, d = r % p.hd;
        uint16_t* cache = (uint16_t*)(isk ? p.k_cache : p.v_cache);
        uint2* dc = (uint2*)(cache + (((size_t)m * p.nkv + kvh) * p.max_seq + rpos) * p.hd + d);
        const uint2 v = make_uint2((uint32_t)f32_to_bf16(o.x) | ((uint32_t)f32_to_bf16(o.y) << 16),
                                   (uint32_t)f32_to_bf16(o.z) | ((uint32_t)f32_to_bf16(o.w) << 16));
        if constexpr (HDA != 0)
          __hip_atomic_store(gbl((unsigned long long*)dc), __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else *dc = v;
      }
    } else if (p.swiglu) {
      *(float2*)(p.C + (size_t)m * p.ldc + n / 2) = make_float2(silu(o.x) * o.y, silu(o.z) * o.w);
    } else {
      if (p.res) {
        const float4 r = *(const float4*)(p.res + (size_t)m * p.ldr + n);
        o.x = r.x + o.x; o.y = r.y + o.y; o.z = r.z + o.z; o.w = r.w + o.w;
      }
      *(float4*)(p.C + (size_t)m * p.ldc + n) = o;
      if (S > S0)   // two parts: C2 = C + the part-1 sum
        *(float4*)(p.C2 + (size_t)m * p.ldc + n) = make_float4(o.x + v1.x, o.y + v1.y, o.z + v1.z, o.w + v1.w);
    }
  }
  // the QKV tile's q and K/V rows are in memory: tell the attention workgroups
  if constexpr (HDA != 0)
    if (p.rope_q) prog_publish(args.prog + tile, pcode);
}

// Slices of one K part: about 128 workgroups for its tiles (half a round: the projections
// run two to a launch, or two K parts to a problem), at least two whole chunks per slice
// (so that a workgroup has a chunk in flight while it multiplies one); a function of the
// shape only, so a problem gives the same bits in every launch.  (Aimed at 512 / 192 /
// 96 / 64 workgroups, the 70B shard decoded 1459 / 1452 / 1335 / 1170 tok/s at batch 8
// against 1534 at 128; at 512 / 256 / 192 / 96 / 64, 2566 / 2532 / 2468 / 2511 / 2217 at
// batch 16 against 2774.)
void sk_part_plan(int M, int N, int K, int* S, int* ks) {
  const int KC = M <= 16 ? 256 : 128;
  const int nt = (N + kSkRows - 1) / kSkRows;
  const int nkc = (K + KC - 1) / KC;
  const int s = std::max(1, std::min(std::min(nkc / 2, sk_max_slices(M)), (128 + nt - 1) / nt));
  const int k = (nkc + s - 1) / s * KC;
  *S = (K + k - 1) / k;
  *ks = k;
}

SkProb sk_prob(const GemmParams& p) {
  SkProb q{};
  q.g = p;
  q.nt = (p.N + kSkRows - 1) / kSkRows;
  sk_part_plan(p.M, p.N, p.K, &q.S0, &q.ks0);
  if (p.A2) sk_part_plan(p.M, p.N, p.K2, &q.S1, &q.ks1);
  return q;
}

size_t sk_need(const SkProb& q) {
  const size_t S = (size_t)q.S0 + q.S1;
  return S * q.g.M * q.g.N + (size_t)q.nt * S * q.g.M;
}

// Row sources whose 16-row units each lie in one matrix: interleaved, or segment bounds
// that are multiples of 16.
bool sk_rows_ok(const RowSrc& r) { return r.interleave || (r.n0 % 16 == 0 && r.n1 % 16 == 0); }

bool sk_ok(const GemmParams& p) {
  if (p.wdtype != W_BF16 || p.M < 1 || p.M > kSkMaxM || !p.cnt || !p.ws || p.N % 16 || p.K % 64 || p.lda % 4 ||
      !sk_rows_ok(p.rows) || (p.A2 && !sk_rows_ok(p.rows2)) ||
      (p.res && p.ldr % 4) || (!p.swiglu && p.ldc % 4) || (p.swiglu && (p.ldc % 2 || p.res)))
    return false;
  if (p.A2 && (p.gain || p.swiglu || !p.res || !p.C2 || p.K2 < 64 || p.K2 % 64 || p.lda2 % 4)) return false;
  if (p.rope_q && (p.swiglu || p.res || p.A2 || !p.k_cache || !p.v_cache || !p.rope_cos || !p.rope_sin || !p.d_pos ||
                   p.hd < 4 || p.hd % 4 || p.nq < 1 || p.nkv < 1 || p.max_seq < 1 ||
                   p.N != (p.nq + 2 * p.nkv) * p.hd))
    return false;
  const SkProb q = sk_prob(p);
  return q.S0 + q.S1 <= sk_max_slices(p.M) && q.nt <= kSkinnyMaxTiles && sk_need(q) <= p.ws_floats;
}

hipError_t sk_launch(const SkProb* q, int np, hipStream_t s) {
  SkArgs a{};
  a.p[0] = q[0];
  a.p[1] = np > 1 ? q[1] : q[0];
  a.items0 = q[0].nt * (q[0].S0 + q[0].S1);
  a.items = a.items0 + (np > 1 ? q[1].nt * (q[1].S0 + q[1].S1) : 0);
  a.per_xcd = (a.items + kSkXcds - 1) / kSkXcds;
  const dim3 grid(a.per_xcd * kSkXcds), block(256);
  const bool norm = q[0].g.gain != nullptr;
  if (q[0].g.M <= 16) launch_timed(norm ? skinny_kernel<1, true> : skinny_kernel<1, false>, grid, block, 0, s, a);
  else launch_timed(norm ? skinny_kernel<2, true> : skinny_kernel<2, false>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool skinny_supported(const GemmParams& p) { return sk_ok(p); }

size_t skinny_ws_floats(const GemmParams& p) { return sk_need(sk_prob(p)); }

hipError_t launch_skinny(const GemmParams& p, hipStream_t s) {
  if (!sk_ok(p)) return hipErrorInvalidValue;
  const SkProb q = sk_prob(p);
  return sk_launch(&q, 1, s);
}

bool skinny_pair_supported(const GemmParams& a, const GemmParams& b) {
  return sk_ok(a) && sk_ok(b) && a.M == b.M && (a.gain != nullptr) == (b.gain != nullptr);
}

bool skinny_pair_attn_supported(const GemmParams& a, const GemmParams& b, const AttnDecodeParams& at) {
  if (!skinny_pair_supported(a, b) || !a.rope_q || !a.gain || b.rope_q) return false;
  const int nt = (a.N + kSkRows - 1) / kSkRows;
  return nt <= kSeqProgWords && at.wdtype == W_BF16 && at.q == a.rope_q && at.k_cache == a.k_cache &&
         at.v_cache == a.v_cache && at.d_pos == a.d_pos && at.B == a.M && at.nq == a.nq && at.nkv == a.nkv &&
         at.hd == a.hd && at.max_seq == a.max_seq && (at.hd == 64 || at.hd == 128) && at.nq % at.nkv == 0 &&
         at.nq / at.nkv <= kAttnMaxGroup && at.n_split >= 1 && at.n_split <= kAttnMaxSplits && at.part &&
         at.counters && at.out && at.d_epoch && !at.done_flag;
}

hipError_t launch_skinny_pair_attn(const GemmParams& a, const GemmParams& b, const AttnDecodeParams& at,
                                   uint32_t* prog, int tag, int* err, hipStream_t s) {
  if (!skinny_pair_attn_supported(a, b, at) || !prog || !err || tag < 1 || tag >= (int)kSeqCodeStride)
    return hipErrorInvalidValue;
  const SkProb q[2] = {sk_prob(a), sk_prob(b)};
  SkArgs g{};
  g.p[0] = q[0];
  g.p[1] = q[1];
  g.items0 = q[0].nt * (q[0].S0 + q[0].S1);
  g.items = g.items0 + q[1].nt * (q[1].S0 + q[1].S1);
  g.per_xcd = 0;
  g.at = at;
  g.n_attn = at.n_split * at.nkv * at.B;
  g.per1 = (g.items - g.items0 + kSkXcds - 1) / kSkXcds;
  g.tag = tag;
  g.prog = prog;
  g.err = err;
  const dim3 grid(g.items0 + g.n_attn + g.per1 * kSkXcds), block(256);
  if (a.M <= 16)
    launch_timed(at.hd == 128 ? skinny_kernel<1, true, 128> : skinny_kernel<1, true, 64>, grid, block, 0, s, g);
  else
    launch_timed(at.hd == 128 ? skinny_kernel<2, true, 128> : skinny_kernel<2, true, 64>, grid, block, 0, s, g);
  return hipGetLastError();
}

hipError_t launch_skinny_pair(const GemmParams& a, const GemmParams& b, hipStream_t s) {
  if (!skinny_pair_supported(a, b)) return hipErrorInvalidValue;
  const SkProb q[2] = {sk_prob(a), sk_prob(b)};
  return sk_launch(q, 2, s);
}

}  // namespace ladder

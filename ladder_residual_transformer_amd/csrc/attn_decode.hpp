// One workgroup of split-KV grouped-query decode attention (device code shared by the
// stand-alone attention kernel and the fused attention + down-projection kernel).
//
// Workgroup (s, kvh, b) owns keys [s*chunk, min(len, (s+1)*chunk)) of kv head kvh of
// sequence b, with len = pos + 1 and chunk a whole number of 64-key tiles (the smallest
// that covers len with n_split chunks); workgroups past the last active chunk leave at
// once.  All G = nq/nkv query heads of the kv head (query head h reads kv head h / G)
// are handled by the workgroup, which keeps a running (max, sum, accumulator) per head
// over its tiles (online softmax).  The K and V rows of the next tile are loaded into
// registers while the current one is used, so a chunk of one tile costs a single memory
// round trip.
//
// bf16 caches (matrix cores): each wave scores 16 keys of the tile against all heads
// with v_mfma_f32_16x16x32_f16 (S^T = K.Q^T, K converted exactly to fp16, q carried as
// an fp16 pair hi + lo); the tile's max and sum per head go through LDS; the
// probabilities, as fp16 pairs in LDS (P^T), multiply the transposed V tile with
// v_mfma_f32_16x16x16_f16, each wave owning a quarter of the output dimensions.
//
// fp32 caches (VALU): each wave works on its own query heads (wave w owns heads w,
// w+4, ...; HPW heads per wave); it scores key j in lane j and accumulates P.V with lane
// l owning output dimensions l*DPL .. l*DPL+DPL-1, taking key j's weight from lane j.
//
// Each workgroup writes its (max, sum, accumulator); the last workgroup of a
// (sequence, kv head), found with an atomic ticket, merges the chunks in chunk order
// with their log-sum-exp weights, so the result does not depend on scheduling.  The
// merge stages the chunks' (max, sum) pairs in LDS while each thread's first 16
// accumulator loads are already in flight (one round trip for up to 16 chunks).
#pragma once
#include "common.hpp"
#include "kernels.h"

namespace ladder {

constexpr int kAttnKeyTile = 64;
constexpr int kAttnMaxGroup = 16;
constexpr int kAttnMaxSplits = 32;
constexpr int kAttnDefaultSplits = 16;   // chunks the decode path uses (at most kAttnMaxSplits)

// fp32 caches
template <typename WT, int HD>
struct AttnLds {
  static constexpr int RW = HD * (int)sizeof(WT) / 4 + 1;   // dwords per staged row (odd)
  __attribute__((aligned(16))) float qs[kAttnMaxGroup][HD];
  uint32_t ks[kAttnKeyTile][RW];
  uint32_t vs[kAttnKeyTile][RW];
  float wsc[kAttnMaxGroup][kAttnMaxSplits];   // merge: chunk maxima, then weights
  float lsc[kAttnMaxGroup][kAttnMaxSplits];   // merge: chunk sums
  float linv[kAttnMaxGroup];
  int is_last;
};

// bf16 caches: fp16 tiles for the matrix cores; rows padded by 16 bytes
template <int HD>
struct AttnLds<uint16_t, HD> {
  __attribute__((aligned(16))) uint16_t ks[kAttnKeyTile][HD + 8];   // K, row = key
  __attribute__((aligned(16))) uint16_t vt[HD][kAttnKeyTile + 8];   // V^T, row = head dim
  // P^T hi and lo, row = head; rows of 68 halves (34 dwords): the 16 rows a pass of 8-byte
  // accesses touches start 2 banks apart (with 72 halves, rows r and r + 8 shared banks)
  __attribute__((aligned(16))) uint16_t pth[16][kAttnKeyTile + 4];
  __attribute__((aligned(16))) uint16_t ptl[16][kAttnKeyTile + 4];
  float wmax[4][16];                                               // per wave and head
  float wsum[4][16];
  float wsc[kAttnMaxGroup][kAttnMaxSplits];
  float lsc[kAttnMaxGroup][kAttnMaxSplits];
  float linv[kAttnMaxGroup];
  int is_last;
};

// Position of key k in row `dim` of the V^T tile: the 4-key groups of a row are permuted by
// XOR with (dim / 8) % 16.  The transposing stores of a wave write one key pair into 16
// rows 8 apart, whose unpermuted row starts (72 halves apart) all fall in one LDS bank (a
// 16-way conflict, three quarters of the attention's LDS cycles); permuted, they spread
// over the banks.  Reads of 4 keys (one group) stay contiguous.
__device__ __forceinline__ int vt_col(int dim, int k) { return ((((k >> 2) ^ (dim >> 3)) & 15) << 2) | (k & 3); }

// Keys per chunk at length len: whole tiles, the fewest that cover len with n_split chunks.
__host__ __device__ inline int attn_chunk(int len, int n_split) {
  const int per = (len + n_split - 1) / n_split;
  return (per + kAttnKeyTile - 1) / kAttnKeyTile * kAttnKeyTile;
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Heads per wave of the fp32 path for a group of G query heads per kv head.
__host__ __device__ constexpr int attn_hpw(int G) { return G <= 4 ? 1 : (G <= 8 ? 2 : 4); }

// Record of one chunk and query head: max of score/sqrt(hd), sum of e^(score/sqrt(hd) -
// max), two unused, then the accumulator (16-byte aligned).
template <int HD> constexpr size_t attn_rec() { return HD + 4; }

// Merge of the n_act chunk records of (sequence b, kv head kvh) into the attention
// output, then (if p.done_flag) the completion signal.  COH: records, output and signal
// use coherent accesses (no cache write-back or invalidate is needed).  The counter of
// the chunks' tickets is reset for the next use.
template <int HD, bool COH = false, typename Lds>
__device__ void attn_merge(const AttnDecodeParams& p, int b, int kvh, int G, int n_act, Lds& L) {
  const int tid = threadIdx.x;
  const size_t stride = attn_rec<HD>();
  int* counter = p.counters + (size_t)b * p.nkv + kvh;
  // merge: per head M = max_s m_s, w_s = e^{m_s - M}, L = sum_s l_s w_s,
  // o[d] = sum_s acc_s[d] w_s / L, summed in chunk order.  Thread i owns (head, 4 dims)
  // item i (G*HD/4 <= 256 items for G*HD <= 1024; larger groups loop).
  constexpr int QG = 16;
  const float* base = p.part + ((size_t)b * p.nq + kvh * G) * p.n_split * stride;
  const int n_items = G * (HD / 4);
  float4 a0[QG];
  {
    const int i = min(tid, n_items - 1), h = i / (HD / 4), d4 = (i % (HD / 4)) * 4;
    const float* src = base + (size_t)h * p.n_split * stride + 4 + d4;
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const float* rec = src + (size_t)min(q, n_act - 1) * stride;
      a0[q] = COH ? ld_coh4(rec) : ldg4(rec);
    }
  }
  for (int i = tid; i < G * n_act; i += 256) {
    const int h = i / n_act, q = i % n_act;
    const float* rec = base + ((size_t)h * p.n_split + q) * stride;
    L.wsc[h][q] = COH ? ld_coh(rec) : gbl(rec)[0];
    L.lsc[h][q] = COH ? ld_coh(rec + 1) : gbl(rec)[1];
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int q = 0; q < n_act; ++q) M = fmaxf(M, L.wsc[tid][q]);
    float Ls = 0.f;
    for (int q = 0; q < n_act; ++q) {
      const float w = expf(L.wsc[tid][q] - M);
      L.wsc[tid][q] = w;
      Ls = fmaf(L.lsc[tid][q], w, Ls);
    }
    L.linv[tid] = 1.0f / Ls;
  }
  __syncthreads();
  for (int i = tid; i < n_items; i += 256) {
    const int h = i / (HD / 4), d4 = (i % (HD / 4)) * 4;
    const float* src = base + (size_t)h * p.n_split * stride + 4 + d4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < n_act; q0 += QG) {
      if (i != tid || q0 > 0) {
#pragma unroll
        for (int q = 0; q < QG; ++q) {
          const float* rec = src + (size_t)min(q0 + q, n_act - 1) * stride;
          a0[q] = COH ? ld_coh4(rec) : ldg4(rec);
        }
      }
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        if (q0 + q < n_act) {
          const float w = L.wsc[h][q0 + q];
          o.x = fmaf(a0[q].x, w, o.x);
          o.y = fmaf(a0[q].y, w, o.y);
          o.z = fmaf(a0[q].z, w, o.z);
          o.w = fmaf(a0[q].w, w, o.w);
        }
      }
    }
    const float li = L.linv[h];
    float* dst = p.out + (size_t)b * p.nq * HD + (size_t)(kvh * G + h) * HD + d4;
    const float4 r = make_float4(o.x * li, o.y * li, o.z * li, o.w * li);
    if (COH) st_coh4(dst, r);
    else stg4(dst, r);
  }
  if (tid == 0) {
    if (COH) __hip_atomic_store(gbl(counter), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *gbl(counter) = 0;
  }
  // completion signal: the last of the B*nkv merges publishes the step's epoch
  if (p.done_flag) {
    if (COH) wg_arrive_coh(p.done_cnt, p.done_flag, p.B * p.nkv, *gbl(p.d_epoch));
    else wg_signal(p.done_cnt, p.done_flag, p.B * p.nkv, *gbl(p.d_epoch));
  }
}

// Ticket and merge, after this workgroup has written its records (G heads of one chunk):
// the last chunk's workgroup merges (attn_merge).
template <int HD, bool COH = false, typename Lds>
__device__ void attn_finish(const AttnDecodeParams& p, int b, int kvh, int G, int n_act, Lds& L) {
  const int tid = threadIdx.x;
  // release this chunk's records, take a ticket; the last one acquires everybody's
  wave_stores_done();
  __syncthreads();
  int* counter = p.counters + (size_t)b * p.nkv + kvh;
  if (tid == 0) {
    if (!COH) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = __hip_atomic_fetch_add(gbl(counter), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_act - 1;
    if (!COH && last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    L.is_last = last;
  }
  __syncthreads();
  if (!L.is_last) return;
  attn_merge<HD, COH>(p, b, kvh, G, n_act, L);
}

// ----------------------------------------------------------------- bf16 (MFMA)
//
// MFMA 16x16x32 f16: lane l supplies A row l%16 and B column l%16 with k-slots
// 8*(l/16) .. +8; 16x16x16 f16: the same rows/columns with k-slots 4*(l/16) .. +4.  The
// result holds column l%16, rows 4*(l/16) + i, i = 0..3.
// wprog (COH only, nullable): q and the newest K/V row are written by other workgroups of
// the same launch, which publish wcode in wprog[0..wn) when done; the first tile's older
// rows are loaded before the wait (they come from earlier steps), the rest after it.
// Poll of the tagged QKV outputs of one kv group (batch 1): entry e of the group (its G
// query heads' rows, then its K row, then its V row) is the 64-bit word (tag << 32 |
// value bits) at tagged[row]; once every entry of the group carries `code`, the values are
// in stage[(G + 2) * HD].  Bounded: a poll that gives up sets *err.
template <int HD>
__device__ __forceinline__ void tagged_poll(const unsigned long long* tagged, int qrows, int kvrows, int kvh, int G,
                                            uint32_t code, float* stage, int* err) {
  const int n = (G + 2) * HD;
  constexpr int PER = 18 * HD / 256 + 1;       // entries per thread for G <= 16
  int pending = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if ((int)threadIdx.x + 256 * k < n) pending |= 1 << k;
  for (unsigned rounds = 0;; ++rounds) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (pending & (1 << k)) {
        const int e = (int)threadIdx.x + 256 * k;
        const int row = e < G * HD ? kvh * G * HD + e
                        : e < (G + 1) * HD ? qrows + kvh * HD + (e - G * HD)
                                           : qrows + kvrows + kvh * HD + (e - (G + 1) * HD);
        const unsigned long long w =
            __hip_atomic_load(gbl(tagged) + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == code) {
          stage[e] = __uint_as_float((uint32_t)w);
          pending &= ~(1 << k);
        }
      }
    }
    if (__syncthreads_and(pending == 0)) return;
    if (rounds == (1u << 16)) {
      if (threadIdx.x == 0) __hip_atomic_fetch_or(gbl(err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// MERGE false: the workgroup only writes its chunk's records (no ticket, no merge); a
// later launch merges them with attn_merge.  TAGGED (batch 1, COH): q and the newest K/V
// row come from the tagged QKV outputs of this launch (tagged_poll with code wcode, staged
// in tstage) instead of a progress-word wait and loads.
template <int HD, bool COH = false, bool MERGE = true, bool TAGGED = false>
__device__ void attn_decode_block_mfma(const AttnDecodeParams& p, int blk, AttnLds<uint16_t, HD>& L,
                                       const uint32_t* wprog = nullptr, int wn = 0, uint32_t wcode = 0,
                                       int* werr = nullptr, const unsigned long long* tagged = nullptr,
                                       float* tstage = nullptr) {
  static_assert(!TAGGED || COH, "the tagged hand-over reads rows written in the same launch");
  constexpr int T = kAttnKeyTile;
  constexpr int CPR = HD / 8;                  // 16-byte chunks per K/V row
  constexpr int KCH = T * CPR / 256;           // K chunks per thread per tile
  constexpr int VPAIR = (T / 2) * CPR / 256;   // V row pairs per thread per tile
  constexpr int NST = HD / 32;                 // 32-dim steps of the scores
  constexpr int DPW = HD / 4;                  // output dims per wave
  constexpr int NDB = DPW / 16;                // 16-dim blocks per wave
  static_assert(KCH >= 1 && VPAIR >= 1 && NDB >= 1 && T == 64, "tile shape");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int s = blk % p.n_split;
  const int kvh = (blk / p.n_split) % p.nkv;
  const int b = blk / (p.n_split * p.nkv);
  const int G = p.nq / p.nkv;
  const int len = *gbl(p.d_pos) + 1;
  const int chunk = attn_chunk(len, p.n_split);
  const int n_act = (len + chunk - 1) / chunk;             // chunks holding keys
  if (s >= n_act) return;                                  // whole workgroup: nothing to do
  const int start = s * chunk;
  const int end = min(len, start + chunk);
  const bool pre = COH && (wprog != nullptr || TAGGED);
  bool defer = pre;                            // the newest row is not loaded before the wait
  const size_t kv_base = ((size_t)b * p.nkv + kvh) * p.max_seq * HD;
  const uint16_t* kc = (const uint16_t*)p.k_cache + kv_base;
  const uint16_t* vc = (const uint16_t*)p.v_cache + kv_base;

  // tile loads; rows past the chunk end repeat its last key (masked, weight 0).  COH: the
  // newest row (position len-1) was written in this kernel and is read coherently (q is
  // read with ordinary loads: its producer gives it an address of its own per layer).
  uint4 kr[KCH], vr[VPAIR][2];
  // TAGGED: the newest row's 8 values at dimension c from the staged K (which 0) or V (1)
  // row, rounded to bf16 as the cache holds them
  auto tagged_row = [&](int which, int c) -> uint4 {
    const float* v = tstage + (G + which) * HD + c;
    auto pk = [&](int e) { return (uint32_t)f32_to_bf16(v[e]) | ((uint32_t)f32_to_bf16(v[e + 1]) << 16); };
    return make_uint4(pk(0), pk(2), pk(4), pk(6));
  };
  auto ld_row = [&](const uint16_t* base, int r, int c) -> uint4 {
    const uint16_t* a = base + (size_t)r * HD + c;
    if (COH && r == len - 1) {
      if (defer) return make_uint4(0u, 0u, 0u, 0u);      // not written yet: loaded after the wait
      if constexpr (TAGGED) return tagged_row(base == kc ? 0 : 1, c);
      const uint32_t* w = (const uint32_t*)a;
      return make_uint4(ld_coh(w), ld_coh(w + 1), ld_coh(w + 2), ld_coh(w + 3));
    }
    return ldg4u(a);
  };
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + 256 * i, r = min(t0 + e / CPR, end - 1), c = (e % CPR) * 8;
      kr[i] = ld_row(kc, r, c);
    }
#pragma unroll
    for (int i = 0; i < VPAIR; ++i) {
      const int e = tid + 256 * i, j = e / CPR, c = (e % CPR) * 8;
      const int r0 = min(t0 + 2 * j, end - 1), r1 = min(t0 + 2 * j + 1, end - 1);
      vr[i][0] = ld_row(vc, r0, c);
      vr[i][1] = ld_row(vc, r1, c);
    }
  };
  load_tile(start);
  if (TAGGED) {
    tagged_poll<HD>(tagged, p.nq * HD, p.nkv * HD, kvh, G, wcode, tstage, werr);
    defer = false;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + 256 * i, r = min(start + e / CPR, end - 1), c = (e % CPR) * 8;
      if (r == len - 1) kr[i] = tagged_row(0, c);
    }
#pragma unroll
    for (int i = 0; i < VPAIR; ++i) {
      const int e = tid + 256 * i, j = e / CPR, c = (e % CPR) * 8;
      if (min(start + 2 * j, end - 1) == len - 1) vr[i][0] = tagged_row(1, c);
      if (min(start + 2 * j + 1, end - 1) == len - 1) vr[i][1] = tagged_row(1, c);
    }
  } else if (pre) {
    prog_wait(wprog, wn, wcode, werr);
    defer = false;                             // later tiles load the newest row themselves
    // the newest row of the first tile (if it holds it), coherently
    auto ld_new = [&](const uint16_t* base, int c) -> uint4 {
      const uint32_t* w = (const uint32_t*)(base + (size_t)(len - 1) * HD + c);
      return make_uint4(ld_coh(w), ld_coh(w + 1), ld_coh(w + 2), ld_coh(w + 3));
    };
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int e = tid + 256 * i, r = min(start + e / CPR, end - 1), c = (e % CPR) * 8;
      if (r == len - 1) kr[i] = ld_new(kc, c);
    }
#pragma unroll
    for (int i = 0; i < VPAIR; ++i) {
      const int e = tid + 256 * i, j = e / CPR, c = (e % CPR) * 8;
      if (min(start + 2 * j, end - 1) == len - 1) vr[i][0] = ld_new(vc, c);
      if (min(start + 2 * j + 1, end - 1) == len - 1) vr[i][1] = ld_new(vc, c);
    }
  }

  // Q^T operand as fp16 pairs: column = head (zero past the group), step st holds dims
  // 32*st + 8*grp .. +8
  half8 qh[NST], ql[NST];
  {
    const float* qrow = p.q + (size_t)b * p.nq * HD + (size_t)(kvh * G + min(col, G - 1)) * HD;
    const float qz = col < G ? 1.f : 0.f;
    const float* qst = tstage + (size_t)min(col, G - 1) * HD;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const float4 x = TAGGED ? *(const float4*)(qst + 32 * st + 8 * grp) : ldg4(qrow + 32 * st + 8 * grp);
      const float4 y = TAGGED ? *(const float4*)(qst + 32 * st + 8 * grp + 4) : ldg4(qrow + 32 * st + 8 * grp + 4);
      uint4 hi, lo;
      split_h2(x.x * qz, x.y * qz, hi.x, lo.x);
      split_h2(x.z * qz, x.w * qz, hi.y, lo.y);
      split_h2(y.x * qz, y.y * qz, hi.z, lo.z);
      split_h2(y.z * qz, y.w * qz, hi.w, lo.w);
      qh[st] = __builtin_bit_cast(half8, hi);
      ql[st] = __builtin_bit_cast(half8, lo);
    }
  }
  const float c2 = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)
  float m_run = -INFINITY, l_run = 0.f;                      // of head `col`
  f32x4v o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x4v{0.f, 0.f, 0.f, 0.f};

  for (int t0 = start; t0 < end; t0 += T) {
    __syncthreads();                                       // previous tile consumed
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
    __syncthreads();
    if (t0 + T < end) load_tile(t0 + T);                   // next tile in flight

    // S^T for this wave's keys 16w .. 16w+15: the lane holds keys 16w + 4*grp + i of head col
    f32x4v sc = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const half8 a = *(const half8*)&L.ks[16 * w + col][32 * st + 8 * grp];
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[st], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[st], sc, 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (t0 + 16 * w + 4 * grp + i >= end) sc[i] = -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (grp == 0) L.wmax[w][col] = mx;
    __syncthreads();
    const float mt = fmaxf(fmaxf(L.wmax[0][col], L.wmax[1][col]), fmaxf(L.wmax[2][col], L.wmax[3][col]));
    const float m_new = fmaxf(m_run, mt);                  // finite: key t0 is in the tile
    const float alpha = exp2f((m_run - m_new) * c2);
    m_run = m_new;
    const float mc = m_new * c2;
    float e[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = exp2f(fmaf(sc[i], c2, -mc));
      ps += e[i];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    if (grp == 0) L.wsum[w][col] = ps;
    uint32_t h01, l01, h23, l23;
    split_h2(e[0], e[1], h01, l01);
    split_h2(e[2], e[3], h23, l23);
    *(uint2*)&L.pth[col][16 * w + 4 * grp] = make_uint2(h01, h23);
    *(uint2*)&L.ptl[col][16 * w + 4 * grp] = make_uint2(l01, l23);
    __syncthreads();
    l_run = l_run * alpha + ((L.wsum[0][col] + L.wsum[1][col]) + (L.wsum[2][col] + L.wsum[3][col]));
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] *= alpha;
    // O^T += V^T . P^T over 16-key steps; this wave's dims w*DPW + 16*d + (0..15)
#pragma unroll
    for (int ks = 0; ks < T / 16; ++ks) {
      const half4 bh = __builtin_bit_cast(half4, *(const uint2*)&L.pth[col][16 * ks + 4 * grp]);
      const half4 bl = __builtin_bit_cast(half4, *(const uint2*)&L.ptl[col][16 * ks + 4 * grp]);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const int vr = w * DPW + 16 * d + col;
        const half4 av = __builtin_bit_cast(half4, *(const uint2*)&L.vt[vr][vt_col(vr, 16 * ks + 4 * grp)]);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bl, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, bh, o[d], 0, 0, 0);
      }
    }
  }

  // records: the lane holds dims w*DPW + 16*d + 4*grp + (0..3) of head col
  if (col < G) {
    float* dst = p.part + (((size_t)b * p.nq + kvh * G + col) * p.n_split + s) * attn_rec<HD>();
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const float4 v = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
      if (COH) st_coh4(dst + 4 + w * DPW + 16 * d + 4 * grp, v);
      else stg4(dst + 4 + w * DPW + 16 * d + 4 * grp, v);
    }
    // the record's max is in the merge's units, score / sqrt(hd) (m_run is a raw score)
    if (w == 0 && grp == 0) {
      const float mr = m_run * (1.0f / sqrtf((float)HD));
      if (COH) { st_coh(dst, mr); st_coh(dst + 1, l_run); }
      else { gbl(dst)[0] = mr; gbl(dst)[1] = l_run; }
    }
  }
  if constexpr (MERGE) attn_finish<HD, COH>(p, b, kvh, G, n_act, L);
}

// Chunks holding keys of a decode attention at the current position (the workgroups of
// chunks past them leave at once).
__device__ __forceinline__ int attn_active_chunks(const AttnDecodeParams& p) {
  const int len = *gbl(p.d_pos) + 1;
  const int chunk = attn_chunk(len, p.n_split);
  return (len + chunk - 1) / chunk;
}

// ----------------------------------------------------------------- fp32 (VALU)

template <int HD, int HPW>
__device__ void attn_decode_block_valu(const AttnDecodeParams& p, int blk, AttnLds<float, HD>& L) {
  constexpr int VEC = Vec<float>::N;
  constexpr int VPR = HD / VEC;                          // 16-byte vectors per row
  constexpr int VPT = kAttnKeyTile * VPR / 256;          // per thread per tile, K and V each
  constexpr int DPL = HD / 64;                           // output dims per lane
  static_assert(VPT >= 1 && kAttnKeyTile * VPR % 256 == 0 && HD % 64 == 0, "tile shape");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blk % p.n_split;
  const int kvh = (blk / p.n_split) % p.nkv;
  const int b = blk / (p.n_split * p.nkv);
  const int G = p.nq / p.nkv;
  const int len = *gbl(p.d_pos) + 1;
  const int chunk = attn_chunk(len, p.n_split);
  const int n_act = (len + chunk - 1) / chunk;
  if (s >= n_act) return;
  const int start = s * chunk;
  const int end = min(len, start + chunk);
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t kv_base = ((size_t)b * p.nkv + kvh) * p.max_seq * HD;
  const float* kc = (const float*)p.k_cache + kv_base;
  const float* vc = (const float*)p.v_cache + kv_base;

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
  load_tile(start);
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
#pragma unroll 4
    for (int d = 0; d < HD; d += 4) {               // 4 dims per step: one 16-byte q read per head
#pragma unroll
      for (int k = 0; k < HPW; ++k) {
        const float4 q4 = *reinterpret_cast<const float4*>(&L.qs[hc[k]][d]);
        sc[k] = fmaf(q4.x, __uint_as_float(krow[d]), sc[k]);
        sc[k] = fmaf(q4.y, __uint_as_float(krow[d + 1]), sc[k]);
        sc[k] = fmaf(q4.z, __uint_as_float(krow[d + 2]), sc[k]);
        sc[k] = fmaf(q4.w, __uint_as_float(krow[d + 3]), sc[k]);
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
      for (int e = 0; e < DPL; ++e) v[e] = __uint_as_float(L.vs[j][lane * DPL + e]);
#pragma unroll
      for (int k = 0; k < HPW; ++k) {
        const float w = lane_bcast(pj[k], j);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[k][e] = fmaf(w, v[e], acc[k][e]);
      }
    }
  }

#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int h = wid + 4 * k;
    if (h < G) {
      float* dst = p.part + (((size_t)b * p.nq + kvh * G + h) * p.n_split + s) * attn_rec<HD>();
#pragma unroll
      for (int e = 0; e < DPL; ++e) dst[4 + lane * DPL + e] = acc[k][e];
      if (lane == 0) { dst[0] = m_run[k]; dst[1] = l_run[k]; }
    }
  }
  attn_finish<HD>(p, b, kvh, G, n_act, L);
}

// Requires blockDim.x == 256 and G <= 16 (fp32: G <= 4 * HPW).  `blk` enumerates
// (s, kvh, b), s fastest.
template <typename WT, int HD, int HPW>
__device__ void attn_decode_block(const AttnDecodeParams& p, int blk, AttnLds<WT, HD>& L) {
  if constexpr (sizeof(WT) == 2) attn_decode_block_mfma<HD>(p, blk, L);
  else attn_decode_block_valu<HD, HPW>(p, blk, L);
}

}  // namespace ladder

// Decode projections of one ladder layer at batch 1 as two streaming launches:
//
//   front: [RMSNorm + QKV + RoPE + KV append, then RMSNorm + gate/up + SwiGLU, in every
//           workgroup | split-KV GQA attention once every QKV share is done]
//   back:  [down rows, then the same O rows, x_{2l+1} = x_{2l} + o, x_{2l+2} = x_{2l+1} + d]
//
// Each projection workgroup streams its share of the layer's weights as one sequence of
// units (a unit is a row pair by a chunk of 64 x 4 sixteen-byte vectors, dealt round-robin
// to the four waves, as in the row-wave GEMV of gemv_rw.hpp).  A wave keeps NB units in
// flight in a ring of registers: after computing a unit it issues the loads of the unit
// NB positions later, which near the end of a pass is a unit of the next pass, so HBM
// stays busy across the pass boundary (the epilogue of the finished pass, the QKV signal
// to the attention workgroups, the restaging of an input).  Every load is issued
// unconditionally (a position past the last unit loads one vector of a valid row for all
// lanes and is never used), so no branch separates a load from its use and the compiler
// counts the outstanding loads exactly.  Both inputs of a launch are staged in LDS once,
// up front, when they fit; otherwise (hidden 16384) the second input is restaged at the
// boundary while the next pass's units are already in flight.  Only wave 0 runs the QKV
// epilogue and publishes: the other waves go on streaming.
//
// The per-row arithmetic (chunking, lane mapping, the order of every sum, the RMSNorm
// prologue and the epilogues) is that of gemv_rw.hpp at batch 1, so the results are
// bitwise those of every other decode schedule.
#include "gemv_rw.hpp"

namespace ladder {

namespace {

constexpr int kSv = kRwVpl;              // 16-byte vectors per lane per unit
constexpr int kSChunk = 64 * kSv;        // vectors of a row per unit
constexpr int kSVec = 8;                 // bf16 per 16-byte vector
constexpr int kMergeChunks = 16;         // key chunks of a decode attention merged in the back launch
constexpr int kMergeHeads = 64;          // query heads of one sequence it merges

// One workgroup's pass over row pairs [pr0, pr0 + np) of a virtual bf16 matrix [N][K].
struct SPass {
  RowSrc rows;
  int N, K, nvec, nchunk, pr0, nunits;   // nunits = np * nchunk
  int uoff, poff;                        // LDS byte offsets: staged input (K + 8 floats), partial sums
};

__device__ __forceinline__ SPass spass(const GemvParams& p, int pr0, int pr1, int uoff, int poff) {
  SPass s;
  s.rows = p.rows;
  s.N = p.N;
  s.K = p.K;
  s.nvec = p.K / kSVec;
  s.nchunk = (s.nvec + kSChunk - 1) / kSChunk;
  s.pr0 = pr0;
  s.nunits = (pr1 > pr0 ? pr1 - pr0 : 0) * s.nchunk;
  s.uoff = uoff;
  s.poff = poff;
  return s;
}

// Field-wise choice between two passes (the values stay in registers).
__device__ __forceinline__ SPass pick(bool first, const SPass& a, const SPass& b) {
  SPass s;
  s.rows.m[0] = first ? a.rows.m[0] : b.rows.m[0];
  s.rows.m[1] = first ? a.rows.m[1] : b.rows.m[1];
  s.rows.m[2] = first ? a.rows.m[2] : b.rows.m[2];
  s.rows.n0 = first ? a.rows.n0 : b.rows.n0;
  s.rows.n1 = first ? a.rows.n1 : b.rows.n1;
  s.rows.interleave = first ? a.rows.interleave : b.rows.interleave;
  s.N = first ? a.N : b.N;
  s.K = first ? a.K : b.K;
  s.nvec = first ? a.nvec : b.nvec;
  s.nchunk = first ? a.nchunk : b.nchunk;
  s.pr0 = first ? a.pr0 : b.pr0;
  s.nunits = first ? a.nunits : b.nunits;
  s.uoff = first ? a.uoff : b.uoff;
  s.poff = first ? a.poff : b.poff;
  return s;
}

typedef uint4 SUnit[2][kSv];

// Issue the loads of the workgroup's unit un_in of pass s (real), or of one vector of a
// valid row for every lane (not real).
__device__ __forceinline__ void sload(const SPass& s, int un_in, bool real, int lane, SUnit& w) {
  const int un = real ? un_in : 0;
  const int pmax = (s.N + 1) / 2 - 1;
  const int pair = real ? s.pr0 + un / s.nchunk : min(s.pr0, pmax);
  const int c = un % s.nchunk;
  const int n0 = 2 * pair;
  const uint16_t* r0 = rw_row_ptr<uint16_t>(s.rows, n0, s.K);
  const uint16_t* r1 = rw_row_ptr<uint16_t>(s.rows, min(n0 + 1, s.N - 1), s.K);
  const int li = real ? lane : 0, vs = real ? 64 : 0;
#pragma unroll
  for (int v = 0; v < kSv; ++v) {
    const int vi = min(c * kSChunk + li + vs * v, s.nvec - 1);
    w[0][v] = ldg4u_nt(r0 + (size_t)vi * kSVec);
    w[1][v] = ldg4u_nt(r1 + (size_t)vi * kSVec);
  }
}

// Dot products of the workgroup's unit un with the staged input; the two sums go to the
// pass's partials when the unit is real.  Same arithmetic as the row-wave GEMV.
__device__ __forceinline__ void scompute(const SPass& s, int un, bool real, int lane, const SUnit& w, char* lds) {
  const int c = un % s.nchunk;
  const float* u = reinterpret_cast<const float*>(lds + s.uoff);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int v = 0; v < kSv; ++v) {
    const int vi = c * kSChunk + lane + 64 * v;
    const int ui = (vi < s.nvec ? vi : s.nvec) * kSVec;   // past the row end: the zero pad
    float w0[8], w1[8], uv[8];
    unpack16(w[0][v], w0);
    unpack16(w[1][v], w1);
    const float4 ta = *reinterpret_cast<const float4*>(u + ui);
    const float4 tb = *reinterpret_cast<const float4*>(u + ui + 4);
    uv[0] = ta.x; uv[1] = ta.y; uv[2] = ta.z; uv[3] = ta.w;
    uv[4] = tb.x; uv[5] = tb.y; uv[6] = tb.z; uv[7] = tb.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a0 = fmaf(w0[e], uv[e], a0);
      a1 = fmaf(w1[e], uv[e], a1);
    }
  }
  const float y0 = wave_sum(a0);
  const float y1 = wave_sum(a1);
  if (lane == 0 && real) {
    float* part = reinterpret_cast<float*>(lds + s.poff);
    part[un * 2] = y0;
    part[un * 2 + 1] = y1;
  }
}

// Unit numbering within a workgroup's pass: all four waves round-robin (i-th unit of
// wave w is w + 4i), or the three waves 1..3 (i-th unit of wave w is w - 1 + 3i).
struct UI4 {
  __device__ static int unit(int i, int wid) { return wid + 4 * i; }
  __device__ static int count(int n, int wid) { return n > wid ? (n - wid + 3) / 4 : 0; }
};
struct UI3 {
  __device__ static int unit(int i, int wid) { return wid - 1 + 3 * i; }
  __device__ static int count(int n, int wid) { return wid >= 1 && n > wid - 1 ? (n - wid + 3) / 3 : 0; }
};

// Position q (>= 0) of the wave's unit sequence counted from the start of pass a (nua
// units) followed by pass b (nub units; none unless has_b): issue its loads.
template <typename UA, typename UB>
__device__ __forceinline__ void sload_pos(const SPass& a, int nua, const SPass& b, int nub, bool has_b, int q,
                                          int wid, int lane, SUnit& w) {
  const bool in_a = q < nua;
  const int j = in_a ? q : q - nua;
  const bool real = in_a || (has_b && j < nub);
  sload(pick(in_a, a, b), in_a ? UA::unit(j, wid) : UB::unit(j, wid), real, lane, w);
}

template <int NB>
struct SRing {
  SUnit w[NB];
};

__device__ __forceinline__ void scopy(SUnit& d, const SUnit& s) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int v = 0; v < kSv; ++v) d[r][v] = s[r][v];
}

// new w[k] = old w[(k + r) % NB], 0 <= r < NB (register moves; each waits for its load)
template <int NB>
__device__ __forceinline__ void srotate(SRing<NB>& R, int r) {
  static_assert(NB >= 1 && NB <= 3, "ring of one to three units");
  if constexpr (NB == 2) {
    if (r == 1) {
      SUnit t;
      scopy(t, R.w[0]);
      scopy(R.w[0], R.w[1]);
      scopy(R.w[1], t);
    }
  } else if constexpr (NB == 3) {
    if (r == 1) {
      SUnit t;
      scopy(t, R.w[0]);
      scopy(R.w[0], R.w[1]);
      scopy(R.w[1], R.w[2]);
      scopy(R.w[2], t);
    } else if (r == 2) {
      SUnit t0, t1;
      scopy(t0, R.w[0]);
      scopy(t1, R.w[1]);
      scopy(R.w[0], R.w[2]);
      scopy(R.w[1], t0);
      scopy(R.w[2], t1);
    }
  }
}

// Stream the units of pass a (unit i at position i of the wave's sequence, wave unit
// index `ui(i)`), unit i in slot i % NB on entry; behind them the loads continue into
// pass b (has_b) or are dummies.  The caller rotates the ring by nua % NB before the
// next pass.
template <int NB, typename UA, typename UB>
__device__ __forceinline__ void sstream(const SPass& a, int nua, const SPass& b, int nub, bool has_b, SRing<NB>& R,
                                        int wid, int lane, char* lds) {
  int i = 0;
  for (; i + NB <= nua; i += NB) {
#pragma unroll
    for (int d = 0; d < NB; ++d) {
      scompute(a, UA::unit(i + d, wid), true, lane, R.w[d], lds);
      sload_pos<UA, UB>(a, nua, b, nub, has_b, i + d + NB, wid, lane, R.w[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < NB - 1; ++d) {
    if (i + d < nua) {
      scompute(a, UA::unit(i + d, wid), true, lane, R.w[d], lds);
      sload_pos<UA, UB>(a, nua, b, nub, has_b, i + d + NB, wid, lane, R.w[d]);
    }
  }
}

// Staged input of one batch row of K <= 8192 inputs: the loads of x (and the gain) are
// issued first, the values are written once they have arrived.
struct SStageRegs {
  float4 xr[4][2];
  uint4 gr[4];
};

__device__ __forceinline__ void sstage_issue(const float* x, const void* gain, int K, SStageRegs& r) {
  const int tid = threadIdx.x;
  const int nvec = K / kSVec;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v = min(tid + 256 * k, nvec - 1);
    r.xr[k][0] = ldg4(x + (size_t)v * kSVec);
    r.xr[k][1] = ldg4(x + (size_t)v * kSVec + 4);
    r.gr[k] = gain ? ldg4u((const uint16_t*)gain + (size_t)v * kSVec) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// u = x (* gain) at LDS offset uoff with a zero pad of 8, and this wave's sum of squares
// in sqw[wid] (gain set).  Per-thread order of the sums is that of the row-wave prologue
// (vectors tid, tid + 256, ...).
__device__ __forceinline__ void sstage_finish(const SStageRegs& r, const void* gain, int K, char* lds, int uoff,
                                              float* sqw) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nvec = K / kSVec;
  float* u = reinterpret_cast<float*>(lds + uoff);
  if (tid < kSVec) u[K + tid] = 0.f;
  float sq = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v = tid + 256 * k;
    if (v < nvec) {
      float xv[8] = {r.xr[k][0].x, r.xr[k][0].y, r.xr[k][0].z, r.xr[k][0].w,
                     r.xr[k][1].x, r.xr[k][1].y, r.xr[k][1].z, r.xr[k][1].w};
      if (gain) {
        float g[8];
        unpack16(r.gr[k], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sq = fmaf(xv[e], xv[e], sq);
          xv[e] *= g[e];
        }
      }
      float* up = u + (size_t)v * kSVec;
      *(float4*)up = make_float4(xv[0], xv[1], xv[2], xv[3]);
      *(float4*)(up + 4) = make_float4(xv[4], xv[5], xv[6], xv[7]);
    }
  }
  sq = wave_sum(sq);
  if (lane == 0) sqw[wid] = sq;
}

__device__ __forceinline__ float sinv(const float* sqw, int K, float eps, bool norm) {
  const float t = ((sqw[0] + sqw[1]) + sqw[2]) + sqw[3];
  return norm ? 1.0f / sqrtf(t / (float)K + eps) : 1.0f;
}

struct SShared {
  float sqw[2][4];
  int qkv_done;          // waves that have written their QKV sums
  int b_staged;          // waves that have staged their share of the second input
};

// One wave waits until an LDS counter of its workgroup reaches `target` (other waves of
// the workgroup count themselves there).  Bounded: a wait that gives up sets *err.
__device__ __forceinline__ void lds_count_wait(int* ctr, int target, int* err) {
  if ((threadIdx.x & 63) == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins == (1u << 22)) {
        __hip_atomic_fetch_or(gbl(err), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Shares of a front launch: QKV pairs split evenly over the NG projection workgroups, and
// gate/up pairs filling every workgroup up to an even split of all pairs.
__host__ __device__ inline void front_shares(int Pq, int Pg, int g, int NG, int& a0, int& a1, int& b0, int& b1) {
  const long long Pt = (long long)Pq + Pg;
  a0 = (int)((long long)g * Pq / NG);
  a1 = (int)((long long)(g + 1) * Pq / NG);
  b0 = (int)((long long)g * Pt / NG) - a0;
  b1 = (int)((long long)(g + 1) * Pt / NG) - a1;
}

// The QKV epilogue of one row pair at batch 1: that of the row-wave GEMV, with the
// rotation's cos and sin (of this pair's dimension at the current position) and the
// position given; the two outputs go to the attention of the same launch as tagged words
// (code << 32 | value bits, one 64-bit store each: a reader that sees the code sees the
// value), and a K or V row also to the cache (read by later launches).
__device__ __forceinline__ void qkv_epi_tagged(const GemvParams& p, unsigned long long* tagged, uint32_t code,
                                               int pair, float y0, float y1, float inv, float c, float sn, int pos) {
  const int n0 = 2 * pair;
  y0 *= inv;
  y1 *= inv;
  if (n0 < p.q_rows + p.kv_rows) rope_rot(y0, y1, c, sn);
  const unsigned long long hi = (unsigned long long)code << 32;
  __hip_atomic_store(gbl(tagged) + n0, hi | __float_as_uint(y0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(gbl(tagged) + n0 + 1, hi | __float_as_uint(y1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (n0 >= p.q_rows) {
    const bool isk = n0 < p.q_rows + p.kv_rows;
    const int rr = isk ? n0 - p.q_rows : n0 - p.q_rows - p.kv_rows;
    const int kvh = rr / p.head_dim, d = rr % p.head_dim;
    uint16_t* cache = (uint16_t*)(isk ? p.k_cache : p.v_cache);
    const size_t off = ((size_t)kvh * p.max_seq + pos) * p.head_dim + d;
    *gbl((uint32_t*)(cache + off)) = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
  }
}

}  // namespace

// ---------------------------------------------------------------- front launch
// prob[0] = QKV (EPI_QKV_ROPE), prob[1] = gate/up (EPI_GATEUP_SWIGLU), same K <= 8192.  The
// first n_attn workgroups score their key chunks once every QKV output of their kv group
// has arrived and write the chunk records; the back launch merges them.  In a projection
// workgroup waves 1-3 compute the QKV units, count themselves done in LDS and go on to
// gate/up; wave 0 runs the QKV epilogue, whose outputs reach the attention as tagged
// words (no store has to be waited for), then its gate/up units.  The gate/up input is
// staged while the QKV units stream.
template <int HD, int NB>
__global__ __launch_bounds__(256) void stream_front_kernel(MultiGemvParams mp) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  const int NG = (int)gridDim.x - mp.n_attn;
  const uint32_t code = (uint32_t)*gbl(mp.d_epoch) * kSeqCodeStride + (uint32_t)mp.seq_tag;
  if ((int)blockIdx.x < mp.n_attn) {
    float* stage = reinterpret_cast<float*>(lds_raw + (sizeof(AttnLds<uint16_t, HD>) + 15) / 16 * 16);
    attn_decode_block_mfma<HD, true, false, true>(mp.attn, blockIdx.x,
                                                  *reinterpret_cast<AttnLds<uint16_t, HD>*>(lds_raw), nullptr, 0,
                                                  code, mp.err, mp.tagged, stage);
    return;
  }
  __shared__ SShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = (int)blockIdx.x - mp.n_attn;
  const GemvParams& pq = mp.prob[0];
  const GemvParams& pg = mp.prob[1];
  const int K = pq.K;
  int a0, a1, b0, b1;
  front_shares((pq.N + 1) / 2, (pg.N + 1) / 2, g, NG, a0, a1, b0, b1);
  const int ub = (K + kSVec) * 4;
  const SPass A = spass(pq, a0, a1, 0, mp.part_off);
  const int poff_b = mp.part_off + ((a1 - a0) * A.nchunk * 2 * 4 + 15) / 16 * 16;
  const SPass Bp = spass(pg, b0, b1, ub, poff_b);
  const int nua = UI3::count(A.nunits, wid), nub = UI4::count(Bp.nunits, wid);
  const int npa = a1 - a0;
  if (tid == 0) {
    sh.qkv_done = 0;
    sh.b_staged = 0;
  }

  // wave 0: the position and the rotation values of its epilogue lanes first
  int pos = 0;
  float rc = 1.f, rs = 0.f;
  if (wid == 0) {
    pos = *gbl(pq.d_pos);
    const int n0 = 2 * (a0 + min(lane, max(npa - 1, 0)));
    if (lane < npa && n0 < pq.q_rows + pq.kv_rows) {
      const int d = (n0 < pq.q_rows ? n0 : n0 - pq.q_rows) % pq.head_dim;
      const int half = pq.head_dim >> 1;
      rc = gbl(pq.rope_cos)[(size_t)pos * half + (d >> 1)];
      rs = gbl(pq.rope_sin)[(size_t)pos * half + (d >> 1)];
    }
  }
  // The inputs go out before any weight load: issued behind the first weight units of
  // every workgroup they would wait in the same memory queues for most of their drain.
  SStageRegs st;
  sstage_issue(pq.x, pq.gain, K, st);
  sstage_finish(st, pq.gain, K, lds_raw, 0, sh.sqw[0]);
  sstage_issue(pg.x, pg.gain, K, st);             // the gate/up input, ahead of the first units
  SRing<NB> R;
  if (wid == 0) {
#pragma unroll
    for (int d = 0; d < NB; ++d) sload_pos<UI4, UI4>(Bp, nub, Bp, 0, false, d, 0, lane, R.w[d]);
  } else {
#pragma unroll
    for (int d = 0; d < NB; ++d) sload_pos<UI3, UI4>(A, nua, Bp, nub, true, d, wid, lane, R.w[d]);
  }
  __syncthreads();
  const float inv_a = sinv(sh.sqw[0], K, pq.eps, pq.gain != nullptr);

  if (wid != 0) {
    sstream<NB, UI3, UI4>(A, nua, Bp, nub, true, R, wid, lane, lds_raw);
    if (lane == 0) atomicAdd(&sh.qkv_done, 1);    // this wave's QKV sums are in LDS
    sstage_finish(st, pg.gain, K, lds_raw, ub, sh.sqw[1]);
    if (lane == 0) atomicAdd(&sh.b_staged, 1);
    srotate<NB>(R, nua % NB);
  } else {
    sstage_finish(st, pg.gain, K, lds_raw, ub, sh.sqw[1]);
    if (lane == 0) atomicAdd(&sh.b_staged, 1);
    // QKV epilogue and the signal to the attention workgroups
    lds_count_wait(&sh.qkv_done, 3, mp.err);
    const float* part = reinterpret_cast<const float*>(lds_raw + A.poff);
    if (lane < npa) {
      float y0 = 0.f, y1 = 0.f;
      for (int c = 0; c < A.nchunk; ++c) {
        y0 += part[(lane * A.nchunk + c) * 2];
        y1 += part[(lane * A.nchunk + c) * 2 + 1];
      }
      qkv_epi_tagged(pq, mp.tagged, code, a0 + lane, y0, y1, inv_a, rc, rs, pos);
    }
  }
  // every wave's share of the gate/up input is in LDS
  lds_count_wait(&sh.b_staged, 4, mp.err);
  const float inv_b = sinv(sh.sqw[1], K, pg.eps, pg.gain != nullptr);
  sstream<NB, UI4, UI4>(Bp, nub, Bp, 0, false, R, wid, lane, lds_raw);
  __syncthreads();
  const float* part = reinterpret_cast<const float*>(lds_raw + Bp.poff);
  float best = 0.f;
  int bidx = 0;
  for (int j = tid; j < b1 - b0; j += 256) {
    float y0 = 0.f, y1 = 0.f;
    for (int c = 0; c < Bp.nchunk; ++c) {
      y0 += part[(j * Bp.nchunk + c) * 2];
      y1 += part[(j * Bp.nchunk + c) * 2 + 1];
    }
    rw_epilogue<uint16_t>(pg, b0 + j, 0, y0, y1, inv_b, best, bidx);
  }
}

// ---------------------------------------------------------------- back launch
// Merge of the attention's chunk records (written by the front launch, B = 1) into the
// attention output rows [nq * HD] at LDS offset uoff (zero pad of 8), with the arithmetic
// of attn_merge: per head the chunk maxima, weights e^(m_s - M) and the sum of l_s w_s in
// chunk order, then o = sum_s acc_s w_s in chunk order, times 1 / sum.  In two parts: the
// record loads of the first 256 output quads (every output of up to 8 heads of 128 or 16
// of 64) are issued with the launch's input, before any weight load, and used after the
// first weight units are in flight; further quads load their records where they merge.
constexpr int kMergeMl = kMergeHeads * kMergeChunks / 256;   // (m, l) pairs per thread

struct MergeRegs {
  float m[kMergeMl], l[kMergeMl];
  float4 a[kMergeChunks];
};

template <int HD>
__device__ __forceinline__ void merge_issue(const AttnDecodeParams& at, int n_act, MergeRegs& r) {
  const int tid = threadIdx.x;
  const size_t stride = attn_rec<HD>();
  const int nrec = at.nq * n_act;
#pragma unroll
  for (int j = 0; j < kMergeMl; ++j) {
    const int i = min(tid + 256 * j, nrec - 1), h = i / n_act, q = i % n_act;
    const float* rec = at.part + ((size_t)h * at.n_split + q) * stride;
    r.m[j] = gbl(rec)[0];
    r.l[j] = gbl(rec)[1];
  }
  const int i = min(tid, at.nq * (HD / 4) - 1), h = i / (HD / 4), d4 = (i % (HD / 4)) * 4;
  const float* src = at.part + (size_t)h * at.n_split * stride + 4 + d4;
#pragma unroll
  for (int q = 0; q < kMergeChunks; ++q) r.a[q] = ldg4(src + (size_t)min(q, n_act - 1) * stride);
}

template <int HD>
__device__ __forceinline__ void merge_finish(const AttnDecodeParams& at, int n_act, MergeRegs& r, char* lds, int uoff,
                                             float* wsc /* [nq][kMergeChunks] */, float* lsc, float* linv) {
  constexpr int QG = kMergeChunks;
  const int tid = threadIdx.x;
  const size_t stride = attn_rec<HD>();
  const int n_items = at.nq * (HD / 4), nrec = at.nq * n_act;
  float* u = reinterpret_cast<float*>(lds + uoff);
  if (tid < kSVec) u[at.nq * HD + tid] = 0.f;
#pragma unroll
  for (int j = 0; j < kMergeMl; ++j) {
    const int i = tid + 256 * j;
    if (i < nrec) {
      wsc[(i / n_act) * QG + i % n_act] = r.m[j];
      lsc[(i / n_act) * QG + i % n_act] = r.l[j];
    }
  }
  __syncthreads();
  if (tid < at.nq) {
    float M = -INFINITY;
    for (int q = 0; q < n_act; ++q) M = fmaxf(M, wsc[tid * QG + q]);
    float Ls = 0.f;
    for (int q = 0; q < n_act; ++q) {
      const float w = expf(wsc[tid * QG + q] - M);
      wsc[tid * QG + q] = w;
      Ls = fmaf(lsc[tid * QG + q], w, Ls);
    }
    linv[tid] = 1.0f / Ls;
  }
  __syncthreads();
  for (int i0 = 0; i0 < n_items; i0 += 256) {
    const int i = min(i0 + tid, n_items - 1), h = i / (HD / 4), d4 = (i % (HD / 4)) * 4;
    if (i0 > 0) {
      const float* src = at.part + (size_t)h * at.n_split * stride + 4 + d4;
#pragma unroll
      for (int q = 0; q < QG; ++q) r.a[q] = ldg4(src + (size_t)min(q, n_act - 1) * stride);
    }
    if (i0 + tid < n_items) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < QG; ++q) {
        if (q < n_act) {
          const float w = wsc[h * QG + q];
          o.x = fmaf(r.a[q].x, w, o.x);
          o.y = fmaf(r.a[q].y, w, o.y);
          o.z = fmaf(r.a[q].z, w, o.z);
          o.w = fmaf(r.a[q].w, w, o.w);
        }
      }
      const float li = linv[h];
      *reinterpret_cast<float4*>(u + (size_t)h * HD + d4) = make_float4(o.x * li, o.y * li, o.z * li, o.w * li);
    }
  }
}

// prob[0] = down (no norm), prob[1] = O (no norm, EPI_ADD2: out = xres + o, out2 = out + d)
// over the same row pairs.  Every workgroup loads its input and the attention's chunk
// records (front launch) first, issues its first down units, merges the records into its
// O input while those loads are in flight, then streams its down units with its O units
// behind them in the same ring; one epilogue for both.
template <int HD, int NB>
__global__ __launch_bounds__(256) void stream_back_kernel(MultiGemvParams mp) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  __shared__ SShared sh;
  __shared__ float m_wsc[kMergeHeads * kMergeChunks], m_lsc[kMergeHeads * kMergeChunks], m_linv[kMergeHeads];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = (int)blockIdx.x, NG = (int)gridDim.x;
  const GemvParams& pd = mp.prob[0];
  const GemvParams& po = mp.prob[1];
  const int P = (pd.N + 1) / 2;
  const int h0 = (int)((long long)g * P / NG), h1 = (int)((long long)(g + 1) * P / NG);
  const int ud = (pd.K + kSVec) * 4;
  const SPass D = spass(pd, h0, h1, 0, mp.part_off);
  const int poff_o = mp.part_off + ((h1 - h0) * D.nchunk * 2 * 4 + 15) / 16 * 16;
  const SPass O = spass(po, h0, h1, (ud + 15) / 16 * 16, poff_o);
  const int nud = UI4::count(D.nunits, wid), nuo = UI4::count(O.nunits, wid);
  const int n_act = attn_active_chunks(mp.attn);

  // the input and the records before the weights (front launch)
  SStageRegs st;
  sstage_issue(pd.x, nullptr, pd.K, st);
  MergeRegs mr;
  merge_issue<HD>(mp.attn, n_act, mr);
  sstage_finish(st, nullptr, pd.K, lds_raw, D.uoff, sh.sqw[0]);
  SRing<NB> R;
#pragma unroll
  for (int d = 0; d < NB; ++d) sload_pos<UI4, UI4>(D, nud, O, nuo, true, d, wid, lane, R.w[d]);
  merge_finish<HD>(mp.attn, n_act, mr, lds_raw, O.uoff, m_wsc, m_lsc, m_linv);
  __syncthreads();
  sstream<NB, UI4, UI4>(D, nud, O, nuo, true, R, wid, lane, lds_raw);
  srotate<NB>(R, nud % NB);
  sstream<NB, UI4, UI4>(O, nuo, O, 0, false, R, wid, lane, lds_raw);
  __syncthreads();
  const float* pdp = reinterpret_cast<const float*>(lds_raw + D.poff);
  const float* pop = reinterpret_cast<const float*>(lds_raw + O.poff);
  for (int j = tid; j < h1 - h0; j += 256) {
    float d0 = 0.f, d1 = 0.f, o0 = 0.f, o1 = 0.f;
    for (int c = 0; c < D.nchunk; ++c) {
      d0 += pdp[(j * D.nchunk + c) * 2];
      d1 += pdp[(j * D.nchunk + c) * 2 + 1];
    }
    for (int c = 0; c < O.nchunk; ++c) {
      o0 += pop[(j * O.nchunk + c) * 2];
      o1 += pop[(j * O.nchunk + c) * 2 + 1];
    }
    // the row-wave epilogue at batch 1 with both inverse norms 1
    const int n0 = 2 * (h0 + j);
    const float t0 = po.xres[n0] + o0 * 1.0f;
    po.out[n0] = t0;
    po.out2[n0] = t0 + d0 * 1.0f;
    if (n0 + 1 < po.N) {
      const float t1 = po.xres[n0 + 1] + o1 * 1.0f;
      po.out[n0 + 1] = t1;
      po.out2[n0 + 1] = t1 + d1 * 1.0f;
    }
  }
}

// ------------------------------------------------------------------ host side
namespace {

// Units each wave keeps in flight.  Two and one measured the same step rate on the 70B
// shard (252.5 / 252.8 tok/s), three slower (216 with the first layout of these
// launches): every load in flight also lengthens the loaded latency of the dependent
// loads (staging, epilogues, the attention's), since a wave's loads complete in order.
constexpr int kStreamNB = 2;

template <typename F>
int stream_resident(F fn, size_t lds, hipError_t* err) {
  if (lds > 65536) {
    *err = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (*err != hipSuccess) return 0;
  }
  int per_cu = 0, dev = 0, ncu = 0;
  *err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, 256, lds);
  if (*err != hipSuccess) return 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return 0;
  *err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (*err != hipSuccess) return 0;
  return (per_cu < 2 ? per_cu : 2) * ncu;
}

// LDS of a front launch's projection workgroup: both staged inputs, then the partial sums
// of the largest QKV and gate/up shares at NG workgroups.
size_t front_lds(int K, int Pq, int Pg, int NG, bool dual, int* part_off) {
  const int nvec = K / kSVec, nchunk = (nvec + kSChunk - 1) / kSChunk;
  const size_t ub = (size_t)(K + kSVec) * 4;
  const size_t off = (dual ? 2 : 1) * ub;
  const int qa = (Pq + NG - 1) / NG;
  const int tot = (int)(((long long)Pq + Pg + NG - 1) / NG) + 1;
  *part_off = (int)((off + 15) / 16 * 16);
  return (size_t)*part_off + ((size_t)qa * nchunk * 2 * 4 + 15) / 16 * 16 + (size_t)tot * nchunk * 2 * 4;
}

}  // namespace

bool stream_front_supported(int wdtype, int K, int B, int hd) {
  return wdtype == W_BF16 && B == 1 && (hd == 64 || hd == 128) && K % kSVec == 0 && K <= 1024 * kSVec;
}

bool stream_back_supported(int wdtype, int Kd, int Ko, int B, int N, int nq, int n_split) {
  return wdtype == W_BF16 && B == 1 && Kd % kSVec == 0 && Ko % kSVec == 0 && Kd <= 1024 * kSVec &&
         Ko <= 1024 * kSVec && N >= 128 && nq <= kMergeHeads && n_split <= kMergeChunks;
}

namespace {
template <int HD, int NB>
hipError_t front_go(MultiGemvParams& mp, hipStream_t s) {
  auto fn = stream_front_kernel<HD, NB>;
  const int G = mp.attn.nq / mp.attn.nkv;
  const size_t alds = (sizeof(AttnLds<uint16_t, HD>) + 15) / 16 * 16 + (size_t)(G + 2) * HD * 4;
  // LDS sized for the largest shares the launch can have (64 projection workgroups)
  const int Pq = (mp.prob[0].N + 1) / 2, Pg = (mp.prob[1].N + 1) / 2;
  int part_off = 0;
  size_t lds = front_lds(mp.prob[0].K, Pq, Pg, 64, true, &part_off);
  if (alds > lds) lds = alds;
  static size_t cached_lds = 0;
  static int cached_res = 0;
  if (cached_lds != lds || cached_res == 0) {
    hipError_t e = hipSuccess;
    cached_res = stream_resident(fn, lds, &e);
    if (e != hipSuccess) return e;
    cached_lds = lds;
  }
  int NG = cached_res - mp.n_attn;
  if (NG > kSeqProgWords) NG = kSeqProgWords;
  // wave 0 finishes a workgroup's QKV pairs one per lane
  if (NG < 64 || (Pq + NG - 1) / NG > 64) return hipErrorInvalidValue;
  if (front_lds(mp.prob[0].K, Pq, Pg, NG, true, &part_off) > lds) return hipErrorInvalidValue;
  mp.part_off = part_off;
  launch_timed(fn, dim3(mp.n_attn + NG), dim3(256), (uint32_t)lds, s, mp);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_stream_front(const GemvParams& first, const GemvParams& second, const AttnDecodeParams& attn,
                               unsigned long long* tagged, int tag, int* err, hipStream_t s) {
  const int K = first.K;
  if (!stream_front_supported(first.wdtype, K, first.B, attn.hd) || second.K != K || second.B != 1 ||
      second.wdtype != first.wdtype || first.epi != EPI_QKV_ROPE || second.epi != EPI_GATEUP_SWIGLU ||
      first.N < 2 || second.N < 2 || !tagged || !err || !attn.d_epoch || attn.done_flag || tag < 1 ||
      tag >= (int)kSeqCodeStride || attn.B != 1 || first.q_rows != attn.nq * attn.hd ||
      first.kv_rows != attn.nkv * attn.hd || first.N != first.q_rows + 2 * first.kv_rows)
    return hipErrorInvalidValue;
  if (attn.nkv < 1 || attn.nq % attn.nkv != 0 || attn.nq / attn.nkv > kAttnMaxGroup ||
      attn.n_split > kAttnMaxSplits || attn.wdtype != first.wdtype)
    return hipErrorInvalidValue;
  MultiGemvParams mp{};
  mp.np = 2;
  mp.prob[0] = first;
  mp.prob[1] = second;
  mp.seq = 1;
  mp.tagged = tagged;
  mp.seq_tag = tag;
  mp.err = err;
  mp.d_epoch = attn.d_epoch;
  mp.attn = attn;
  mp.n_attn = attn.n_split * attn.nkv;
  return attn.hd == 128 ? front_go<128, kStreamNB>(mp, s) : front_go<64, kStreamNB>(mp, s);
}

namespace {
template <int HD, int NB>
hipError_t back_go(MultiGemvParams& mp, hipStream_t s) {
  const GemvParams& down = mp.prob[0];
  const GemvParams& o = mp.prob[1];
  auto fn = stream_back_kernel<HD, NB>;
  const int P = (down.N + 1) / 2;
  const int nchunk_d = (down.K / kSVec + kSChunk - 1) / kSChunk;
  const int nchunk_o = (o.K / kSVec + kSChunk - 1) / kSChunk;
  const size_t ud = (size_t)(down.K + kSVec) * 4, uo = (size_t)(o.K + kSVec) * 4;
  const size_t ub = (ud + 15) / 16 * 16 + uo;
  mp.part_off = (int)((ub + 15) / 16 * 16);
  // partial sums for the largest share at 64 workgroups (the least the launch runs with)
  const int per = (P + 63) / 64;
  const size_t lds = (size_t)mp.part_off + ((size_t)per * nchunk_d * 2 * 4 + 15) / 16 * 16 + (size_t)per * nchunk_o * 2 * 4;
  static size_t cached_lds = 0;
  static int cached_res = 0;
  if (cached_lds != lds || cached_res == 0) {
    hipError_t e = hipSuccess;
    cached_res = stream_resident(fn, lds, &e);
    if (e != hipSuccess) return e;
    cached_lds = lds;
  }
  int NG = cached_res;
  if (NG > P) NG = P;
  if (NG < 64) return hipErrorInvalidValue;
  launch_timed(fn, dim3(NG), dim3(256), (uint32_t)lds, s, mp);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_stream_back(const GemvParams& down, const GemvParams& o, const AttnDecodeParams& attn, int* err,
                              hipStream_t s) {
  if (!stream_back_supported(down.wdtype, down.K, o.K, down.B, down.N, attn.nq, attn.n_split) || o.B != 1 ||
      o.wdtype != down.wdtype || down.N != o.N || o.epi != EPI_ADD2 || down.gain || o.gain || !o.xres || !o.out ||
      !o.out2)
    return hipErrorInvalidValue;
  if (attn.B != 1 || attn.nkv < 1 || attn.nq % attn.nkv != 0 || (attn.hd != 64 && attn.hd != 128) ||
      attn.wdtype != down.wdtype ||
      attn.nq * attn.hd != o.K || !attn.part || !attn.d_pos)
    return hipErrorInvalidValue;
  (void)err;
  MultiGemvParams mp{};
  mp.np = 2;
  mp.prob[0] = down;
  mp.prob[1] = o;
  mp.attn = attn;
  return attn.hd == 128 ? back_go<128, kStreamNB>(mp, s) : back_go<64, kStreamNB>(mp, s);
}

}  // namespace ladder

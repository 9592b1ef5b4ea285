// Decode projections for batch 1..4, one wave per row pair, and horizontal fusion of
// independent projections (and decode attention) into one launch.
//
// A workgroup (4 waves) owns a contiguous range of row pairs of one problem.  It first
// stages its input u = x (* RMSNorm gain) for all batch rows in LDS as fp32 together
// with inv_rms = 1/sqrt(mean(x^2)+eps); every wave then streams whole row pairs: lane l
// reads the 16-byte vectors l, l+64, ... of both rows (coalesced, each weight byte read
// once), multiplies them with u from LDS in fp32, and a wave reduction gives the two
// dot products.  There is no barrier inside the row loop, and the next pair's weight
// loads are issued before the current pair's reduction and epilogue, so their latency
// overlaps.  A row's result depends only on K and the lane mapping, never on which
// workgroup computed it, so every launch shape gives bitwise identical values.
//
// One launch can carry two problems (blocks split in proportion to their bytes) and,
// in front of them, the workgroups of a split-KV decode attention: with ladder
// residuals a layer's QKV and gate/up projections read x_{2l-1} and x_{2l}, which are
// both ready before the layer starts, and the down projection does not depend on the
// attention, so each pair runs side by side in one kernel.
#include "gemv_rw.hpp"

namespace ladder {

// Shares of workgroup g of NG in a sequential launch over P0 row pairs of the first
// problem and P1 of the second.  The first NQ workgroups split the first problem evenly;
// the second problem's pairs fill every workgroup up to an even split of the total, so
// that a workgroup's shares add up to within one pair of the average.  The other
// workgroups stream the second problem from the start, which keeps HBM busy while the
// first group publishes its results and restages its input.  (With fewer pairs than
// workgroups the ranges of the second problem may overlap: some pairs are then computed
// twice, with the same values, and none is missed.)
__host__ __device__ inline int seq_first_group(int NG) { return NG > 1 ? NG / 2 : 1; }
__host__ __device__ inline void seq_shares(int P0, int P1, int g, int NG, int& a0, int& a1, int& b0, int& b1) {
  const int NQ = seq_first_group(NG);
  const long long Pt = (long long)P0 + P1;
  auto first = [&](int h) { return (int)((long long)(h < NQ ? h : NQ) * P0 / NQ); };
  a0 = first(g);
  a1 = first(g + 1);
  b0 = (int)((long long)g * Pt / NG) - a0;
  b1 = (int)((long long)(g + 1) * Pt / NG) - a1;
}

// NP: GEMV problems of the launch: 1, 2 (side by side), 3 = the paired launch (rows of
// prob[0], then after the signal the same rows of prob[1]), or 4 = the sequential launch
// (a first group of workgroups: its share of prob[0], then of prob[1]; the others: prob[1]).
// With HDA != 0 the first n_attn workgroups run decode attention (NP 4: once every share
// of prob[0] is done).
template <typename WT, int BT, int VPL, int HDA, int HPW, int NP>
__global__ __launch_bounds__(256) void gemv_rw_kernel(MultiGemvParams mp) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  if constexpr (NP == 4) {
    static_assert(sizeof(WT) == 2 && HDA != 0, "sequential launches: bf16, with attention");
    const int NG = (int)gridDim.x - mp.n_attn;
    const uint32_t code = (uint32_t)*gbl(mp.d_epoch) * kSeqCodeStride + (uint32_t)mp.seq_tag;
    if ((int)blockIdx.x < mp.n_attn) {
      // q and the newest K/V row come from this launch: the first key tile's older rows
      // are loaded, then the workgroup waits for every QKV share; the attention reads q
      // with ordinary loads (nothing in this launch read it before) and the newest row,
      // its records and its output coherently
      attn_decode_block_mfma<HDA, true>(mp.attn, blockIdx.x, *reinterpret_cast<AttnLds<uint16_t, HDA>*>(lds_raw),
                                        mp.prog, seq_first_group(NG), code, mp.err);
      return;
    }
    __shared__ RwShared sh;
    const int g = (int)blockIdx.x - mp.n_attn;
    float* u = reinterpret_cast<float*>(lds_raw);
    float* part = reinterpret_cast<float*>(lds_raw + mp.part_off);
    int a0, a1, b0, b1;
    seq_shares((mp.prob[0].N + 1) / 2, (mp.prob[1].N + 1) / 2, g, NG, a0, a1, b0, b1);
    if (g < seq_first_group(NG)) {
      if (a1 > a0) rw_pass<WT, BT, VPL, RW_OUT_EPI, true>(mp.prob[0], a0, a1, g, u, nullptr, RwWait{}, sh, part);
      prog_publish(mp.prog + g, code);             // also the barrier before u is restaged
    }
    if (b1 > b0) rw_pass<WT, BT, VPL, RW_OUT_EPI>(mp.prob[1], b0, b1, g, u, nullptr, RwWait{}, sh, part);
    return;
  }
  // paired launch with bf16 attention: the attention output and its signal are
  // coherent stores and the second pass waits for the signal without an L2 invalidate
  // (its input, the attention output, is read by nothing in this launch before the signal)
  constexpr bool kCohPair = NP == 3 && HDA != 0 && sizeof(WT) == 2;
  if constexpr (HDA != 0) {
    if ((int)blockIdx.x < mp.n_attn) {
      if constexpr (kCohPair) {
        attn_decode_block_mfma<HDA, true>(mp.attn, blockIdx.x, *reinterpret_cast<AttnLds<uint16_t, HDA>*>(lds_raw));
      } else {
        attn_decode_block<WT, HDA, HPW>(mp.attn, blockIdx.x, *reinterpret_cast<AttnLds<WT, HDA>*>(lds_raw));
      }
      return;
    }
  }
  __shared__ RwShared sh;
  const int blk = (int)blockIdx.x - mp.n_attn;
  float* u = reinterpret_cast<float*>(lds_raw);   // [B][K + pad]
  if constexpr (NP == 3) {
    const int nb = mp.blk_begin[1];
    const int P = (mp.prob[0].N + 1) / 2;
    const int pr0 = (int)((long long)blk * P / nb);
    const int pr1 = (int)((long long)(blk + 1) * P / nb);
    float* dres = reinterpret_cast<float*>(lds_raw + mp.dres_off);
    const int epoch = mp.d_epoch ? *gbl(mp.d_epoch) : 0;
    float* part = reinterpret_cast<float*>(lds_raw + mp.part_off);
    rw_pass<WT, BT, VPL, RW_OUT_LDS>(mp.prob[0], pr0, pr1, blk, u, dres, RwWait{}, sh, part);
    __syncthreads();                               // u is restaged by the second pass
    RwWait wt;
    wt.flag = mp.wait_flag;
    wt.epoch = epoch;
    wt.err = mp.err;
    uint4* wpre = mp.wpre_off ? reinterpret_cast<uint4*>(lds_raw + mp.wpre_off) : nullptr;
    // a second problem of at most 128 vectors per row (the O projection, K 1024) fills
    // every lane with half-length units: the same per-lane sums as the longer units,
    // whose upper halves would only read the zero pad
    if (VPL == 4 && !wpre && mp.prob[1].K <= 128 * Vec<WT>::N)
      rw_pass<WT, BT, 2, RW_OUT_ADD2_LDS, kCohPair>(mp.prob[1], pr0, pr1, blk, u, dres, wt, sh, part);
    else
      rw_pass<WT, BT, VPL, RW_OUT_ADD2_LDS, kCohPair>(mp.prob[1], pr0, pr1, blk, u, dres, wt, sh, part, nullptr,
                                                      wpre);
  } else {
    const int pi = (NP > 1 && blk >= mp.blk_begin[1]) ? 1 : 0;
    const int lb = blk - mp.blk_begin[pi];
    const int nb = mp.blk_begin[pi + 1] - mp.blk_begin[pi];
    const GemvParams& p = mp.prob[pi];
    const int P = (p.N + 1) / 2;
    const int pr0 = (int)((long long)lb * P / nb);
    const int pr1 = (int)((long long)(lb + 1) * P / nb);
    float* part = reinterpret_cast<float*>(lds_raw + mp.part_off);
    if (VPL == 4 && p.K <= 128 * Vec<WT>::N)      // half-length units, as in the paired launch
      rw_pass<WT, BT, 2, RW_OUT_EPI>(p, pr0, pr1, lb, u, nullptr, RwWait{}, sh, part);
    else
      rw_pass<WT, BT, VPL, RW_OUT_EPI>(p, pr0, pr1, lb, u, nullptr, RwWait{}, sh, part);
  }
}

// next[b] = index of the first maximum over the n per-block candidates.
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const float* bv, const int* bi, int n, int BT, int B,
                                                              int* next) {
  __shared__ float rv[256];
  __shared__ int ri[256];
  const int tid = threadIdx.x;
  for (int b = 0; b < B; ++b) {
    float best = -INFINITY;
    int idx = INT_MAX;
    for (int q = tid; q < n; q += 256) {
      const float v = bv[(size_t)q * BT + b];
      const int i = bi[(size_t)q * BT + b];
      if (v > best || (v == best && i < idx)) { best = v; idx = i; }
    }
    rv[tid] = best;
    ri[tid] = idx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) {
        const float v = rv[tid + o];
        const int i = ri[tid + o];
        if (v > rv[tid] || (v == rv[tid] && i < ri[tid])) { rv[tid] = v; ri[tid] = i; }
      }
      __syncthreads();
    }
    if (tid == 0) next[b] = ri[0] == INT_MAX ? 0 : ri[0];
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host side
namespace {

constexpr int kRwTargetBlocks = 1024;  // upper bound; the launch uses what fits on the device at once
constexpr int kRwBlocksPerCu = 2;
constexpr size_t kRwLdsTwoPerCu = 80 * 1024;   // LDS of a workgroup that keeps two per CU

int rw_bt(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : 4; }

// Workgroups per problem in proportion to its rows, at least 4 row pairs each.
void rw_split_blocks(MultiGemvParams& mp, int target) {
  long long rows = 0;
  for (int i = 0; i < mp.np; ++i) rows += mp.prob[i].N;
  mp.blk_begin[0] = 0;
  for (int i = 0; i < mp.np; ++i) {
    const int P = (mp.prob[i].N + 1) / 2;
    long long nb = (long long)target * mp.prob[i].N / rows;
    const int cap = (P + 3) / 4;
    if (nb > cap) nb = cap;
    if (nb < 1) nb = 1;
    mp.blk_begin[i + 1] = mp.blk_begin[i] + (int)nb;
  }
  if (mp.np == 1) mp.blk_begin[2] = mp.blk_begin[1];
}


// gemv_lds: LDS of a GEMV workgroup before its partial sums; attn_lds: of an attention
// workgroup (0 if none).  The partial sums go after gemv_lds, sized for the split.
template <typename WT, int BT, int VPL, int HDA, int HPW, int NP>
hipError_t rw_go(MultiGemvParams& mp, size_t gemv_lds, size_t attn_lds, hipStream_t s) {
  auto fn = gemv_rw_kernel<WT, BT, VPL, HDA, HPW, NP>;
  const size_t lds = gemv_lds > attn_lds ? gemv_lds : attn_lds;
  // resident workgroups of this instance at this LDS size (queried once per instance
  // and size): the GEMV workgroups of one launch are sized to fill the device once
  static size_t cached_lds = 0;
  static int cached_resident = 0;
  if (cached_lds != lds || cached_resident == 0) {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    int per_cu = 0, dev = 0, ncu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, 256, lds);
    if (e != hipSuccess) return e;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    // two long-lived workgroups per CU (8 waves) keep ~2 x 16 KB per wave in flight
    // and give every wave several pipeline units
    const int want = per_cu < kRwBlocksPerCu ? per_cu : kRwBlocksPerCu;
    cached_resident = want > 0 ? want * ncu : 256;
    cached_lds = lds;
  }
  int target = cached_resident - mp.n_attn;
  if (target < 64) target = 64;
  if (target > kRwTargetBlocks) target = kRwTargetBlocks;
  if (NP == 3) {                      // paired: the blocks split the rows of prob[0]
    mp.np = 1;
    rw_split_blocks(mp, target);
    mp.np = 2;
    mp.blk_begin[2] = mp.blk_begin[1];
  } else if (NP == 4) {               // sequential: every block has a share of both
    if (target > kSeqProgWords) target = kSeqProgWords;
    mp.blk_begin[0] = 0;
    mp.blk_begin[1] = mp.blk_begin[2] = target;
  } else {
    rw_split_blocks(mp, target);
  }
  // partial sums: the most pairs any workgroup of a problem gets, times its chunks
  const int vec = sizeof(WT) == 2 ? 8 : 4;
  size_t part = 0;
  if (NP == 4) {
    const int NG = mp.blk_begin[1];
    const int P0 = (mp.prob[0].N + 1) / 2, P1 = (mp.prob[1].N + 1) / 2;
    for (int g = 0; g < NG; ++g) {
      int a0, a1, b0, b1;
      seq_shares(P0, P1, g, NG, a0, a1, b0, b1);
      const size_t f0 = rw_part_floats(a1 - a0, mp.prob[0].K, vec, BT);
      const size_t f1 = rw_part_floats(b1 - b0, mp.prob[1].K, vec, BT);
      if (f0 > part) part = f0;
      if (f1 > part) part = f1;
    }
  }
  for (int i = 0; i < (NP == 3 ? 1 : NP == 4 ? 0 : mp.np); ++i) {
    const int nb = mp.blk_begin[i + 1] - mp.blk_begin[i];
    const int P = (mp.prob[i].N + 1) / 2;
    const int pairs = (P + nb - 1) / nb;
    size_t f = rw_part_floats(pairs, mp.prob[i].K, vec, BT);
    if (NP == 3) {
      const size_t f1 = rw_part_floats(pairs, mp.prob[1].K, vec, BT);
      if (f1 > f) f = f1;
    }
    if (f > part) part = f;
  }
  mp.part_off = (int)((gemv_lds + 15) / 16 * 16);
  size_t total = (size_t)mp.part_off + part * sizeof(float);
  // paired launch with attention: the second pass's weights, copied into LDS while its
  // workgroups wait for the attention, when that keeps two workgroups per CU
  mp.wpre_off = 0;
  if (NP == 3 && HDA != 0) {
    const int nb = mp.blk_begin[1];
    const int P = (mp.prob[0].N + 1) / 2;
    const int pairs = (P + nb - 1) / nb;
    const int nvec = mp.prob[1].K / vec;
    const int chunk = 64 * VPL;
    const int nchunk = (nvec + chunk - 1) / chunk;
    const int spu = nvec < chunk ? (nvec + 63) / 64 : VPL;
    const size_t units_max = (size_t)((pairs * nchunk + 3) / 4) * 4;   // every wave's slots
    const size_t wbytes = units_max * spu * 2 * 1024;
    const size_t off = (total + 1023) / 1024 * 1024;
    if (off + wbytes <= kRwLdsTwoPerCu) {
      mp.wpre_off = (int)off;
      total = off + wbytes;
    }
  }
  if (attn_lds > total) total = attn_lds;
  static size_t attr_lds = 65536;
  if (total > attr_lds) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)total);
    if (e != hipSuccess) return e;
    attr_lds = total;
  }
  const int grid = mp.n_attn + (NP == 3 ? mp.blk_begin[1] : mp.blk_begin[mp.np]);
  launch_timed(fn, dim3(grid), dim3(256), (uint32_t)total, s, mp);
  return hipGetLastError();
}

// Attention workgroups are only fused into launches with 4 vectors per lane per unit
// (every down projection here); the caller launches them separately otherwise.
template <typename WT, int BT, int VPL>
hipError_t rw_hda(MultiGemvParams& mp, int hda, size_t lds, size_t alds, hipStream_t s) {
  if constexpr (VPL == 4) {
    // attention rides with one problem, or with a paired launch; the fp32 path needs the
    // heads-per-wave instance, the bf16 (matrix core) path has one
    // attention rides with one problem, or (bf16) in front of a paired launch; the fp32
    // path needs the heads-per-wave instance, the bf16 (matrix core) path has one
    if constexpr (sizeof(WT) == 2) {
      if (mp.seq) {
        if (hda == 128) return rw_go<WT, BT, VPL, 128, 1, 4>(mp, lds, alds, s);
        if (hda == 64) return rw_go<WT, BT, VPL, 64, 1, 4>(mp, lds, alds, s);
        return hipErrorInvalidValue;
      }
    }
    if (mp.seq) return hipErrorInvalidValue;
    const int hpw = hda ? (sizeof(WT) == 2 ? 1 : attn_hpw(mp.attn.nq / mp.attn.nkv)) : 0;
    if (hda != 0 && mp.np != 1 && !(sizeof(WT) == 2 && mp.paired)) return hipErrorInvalidValue;
    if (hda == 128) {
      if (mp.paired) return rw_go<WT, BT, VPL, 128, 1, 3>(mp, lds, alds, s);
      if (hpw == 1) return rw_go<WT, BT, VPL, 128, 1, 1>(mp, lds, alds, s);
      if (hpw == 2) return rw_go<WT, BT, VPL, 128, 2, 1>(mp, lds, alds, s);
      return rw_go<WT, BT, VPL, 128, 4, 1>(mp, lds, alds, s);
    }
    if (hda == 64) {
      if (mp.paired) return rw_go<WT, BT, VPL, 64, 1, 3>(mp, lds, alds, s);
      if (hpw == 1) return rw_go<WT, BT, VPL, 64, 1, 1>(mp, lds, alds, s);
      if (hpw == 2) return rw_go<WT, BT, VPL, 64, 2, 1>(mp, lds, alds, s);
      return rw_go<WT, BT, VPL, 64, 4, 1>(mp, lds, alds, s);
    }
  }
  if (hda != 0 || mp.seq) return hipErrorInvalidValue;
  if (mp.paired) return sizeof(WT) == 2 ? rw_go<WT, BT, VPL, 0, 0, 3>(mp, lds, 0, s) : hipErrorInvalidValue;
  if (mp.np == 2) return rw_go<WT, BT, VPL, 0, 0, 2>(mp, lds, 0, s);
  return rw_go<WT, BT, VPL, 0, 0, 1>(mp, lds, 0, s);
}

template <typename WT>
hipError_t rw_bt_go(MultiGemvParams& mp, int bt, int hda, size_t lds, size_t alds, hipStream_t s) {
  if (bt == 1) return rw_hda<WT, 1, kRwVpl>(mp, hda, lds, alds, s);
  if (bt == 2) return rw_hda<WT, 2, kRwVpl>(mp, hda, lds, alds, s);
  return rw_hda<WT, 4, kRwVpl>(mp, hda, lds, alds, s);
}

}  // namespace

bool gemv_rw_attn_fusable(int wdtype, int K) {
  (void)wdtype;
  (void)K;
  return true;
}

namespace {
// LDS of a paired launch: u for the wider input, then prob[0]'s rows of one workgroup
// (a launch has at least 64 GEMV workgroups, or as many as give each 4 row pairs)
size_t rw_pair_lds(int wdtype, int K0, int K1, int N, int B, int* dres_off) {
  const int vec = wdtype == W_BF16 ? 8 : 4;
  const size_t ub = (size_t)B * ((K0 > K1 ? K0 : K1) + vec) * 4;
  const size_t off = (ub + 15) / 16 * 16;
  const int P = (N + 1) / 2;
  const int per = (P + 63) / 64;                   // pairs per workgroup: >= 64 workgroups,
  const size_t rows = 2 * (size_t)(per > 4 ? per : 4);   // or at most 4 pairs each
  if (dres_off) *dres_off = (int)off;
  return off + rows * 4 * sizeof(float);
}
}  // namespace

bool gemv_rw_pair_supported(int wdtype, int K_first, int K_second, int B) {
  return wdtype == W_BF16 && gemv_rw_supported(wdtype, K_first, B) && gemv_rw_supported(wdtype, K_second, B) &&
         gemv_rw_attn_fusable(wdtype, K_first);
}

hipError_t launch_gemv_paired(const GemvParams& first, const GemvParams& second, const AttnDecodeParams& attn,
                              int* err, hipStream_t s) {
  const int B = first.B, wdt = first.wdtype;
  if (!gemv_rw_pair_supported(wdt, first.K, second.K, B) || second.B != B || second.wdtype != wdt ||
      first.N != second.N || second.epi != EPI_ADD2 || !attn.done_flag || !attn.done_cnt || !attn.d_epoch || !err)
    return hipErrorInvalidValue;
  if (attn.nkv < 1 || attn.nq % attn.nkv != 0 || attn.nq / attn.nkv > kAttnMaxGroup ||
      attn.n_split > kAttnMaxSplits || (attn.hd != 64 && attn.hd != 128) || attn.wdtype != wdt || attn.B != B)
    return hipErrorInvalidValue;
  MultiGemvParams mp{};
  mp.np = 2;
  mp.prob[0] = first;
  mp.prob[1] = second;
  mp.paired = 1;
  mp.attn = attn;
  mp.n_attn = attn.n_split * attn.nkv * attn.B;
  mp.wait_flag = attn.done_flag;
  mp.d_epoch = attn.d_epoch;
  mp.err = err;
  const size_t lds = rw_pair_lds(wdt, first.K, second.K, first.N, B, &mp.dres_off);
  const size_t al = attn.hd == 128 ? sizeof(AttnLds<uint16_t, 128>) : sizeof(AttnLds<uint16_t, 64>);
  return rw_bt_go<uint16_t>(mp, rw_bt(B), attn.hd, lds, al, s);
}

hipError_t launch_gemv_paired_nowait(const GemvParams& first, const GemvParams& second, hipStream_t s) {
  const int B = first.B, wdt = first.wdtype;
  if (!gemv_rw_pair_supported(wdt, first.K, second.K, B) || second.B != B || second.wdtype != wdt ||
      first.N != second.N || second.epi != EPI_ADD2)
    return hipErrorInvalidValue;
  MultiGemvParams mp{};
  mp.np = 2;
  mp.prob[0] = first;
  mp.prob[1] = second;
  mp.paired = 1;
  const size_t lds = rw_pair_lds(wdt, first.K, second.K, first.N, B, &mp.dres_off);
  return rw_bt_go<uint16_t>(mp, rw_bt(B), 0, lds, 0, s);
}

bool gemv_rw_seq_supported(int wdtype, int K, int B, int hd) {
  return wdtype == W_BF16 && gemv_rw_supported(wdtype, K, B) && (hd == 64 || hd == 128);
}

hipError_t launch_gemv_seq(const GemvParams& first, const GemvParams& second, const AttnDecodeParams& attn,
                           uint32_t* prog, int tag, int* err, hipStream_t s) {
  const int B = first.B, wdt = first.wdtype, K = first.K;
  if (!gemv_rw_seq_supported(wdt, K, B, attn.hd) || second.K != K || second.B != B || second.wdtype != wdt ||
      first.epi != EPI_QKV_ROPE || first.N < 1 || second.N < 1 || !prog || !err || !attn.d_epoch ||
      attn.done_flag || tag < 1 || tag >= (int)kSeqCodeStride)
    return hipErrorInvalidValue;
  if (attn.nkv < 1 || attn.nq % attn.nkv != 0 || attn.nq / attn.nkv > kAttnMaxGroup ||
      attn.n_split > kAttnMaxSplits || attn.wdtype != wdt || attn.B != B || attn.q != first.out)
    return hipErrorInvalidValue;
  MultiGemvParams mp{};
  mp.np = 2;
  mp.prob[0] = first;
  mp.prob[1] = second;
  mp.seq = 1;
  mp.prog = prog;
  mp.seq_tag = tag;
  mp.err = err;
  mp.d_epoch = attn.d_epoch;
  mp.attn = attn;
  mp.n_attn = attn.n_split * attn.nkv * attn.B;
  const size_t lds = (size_t)B * (K + 8) * 4;
  const size_t al = attn.hd == 128 ? sizeof(AttnLds<uint16_t, 128>) : sizeof(AttnLds<uint16_t, 64>);
  return rw_bt_go<uint16_t>(mp, rw_bt(B), attn.hd, lds, al, s);
}

// The staged input rows (fp32, B x (K + pad)) must fit in LDS next to the partial sums:
// up to ~65 KB two workgroups share a CU, beyond that (batch 2-4 at hidden 8192, say) one
// workgroup per CU streams (the launcher sizes the grid from the occupancy it gets).
constexpr size_t kRwMaxInputLds = 150 * 1024;

bool gemv_rw_supported(int wdtype, int K, int B) {
  return B >= 1 && B <= 4 && (size_t)B * (K + (wdtype == W_BF16 ? 8 : 4)) * 4 <= kRwMaxInputLds;
}

bool gemv_rw_two_per_cu(int wdtype, int K, int B) {
  return gemv_rw_supported(wdtype, K, B) && (size_t)B * (K + (wdtype == W_BF16 ? 8 : 4)) * 4 <= 66560;
}

int gemv_rw_blocks(int wdtype, int N, int K, int B) {
  (void)wdtype;
  (void)K;
  (void)B;
  const int P = (N + 1) / 2;
  int nb = (P + 3) / 4;
  return nb < kRwTargetBlocks ? nb : kRwTargetBlocks;   // upper bound of a one-problem launch
}

hipError_t launch_gemv_multi(const GemvParams* probs, int np, const AttnDecodeParams* attn, hipStream_t s,
                             int* blocks_out) {
  if (np < 1 || np > 2) return hipErrorInvalidValue;
  const int K = probs[0].K, B = probs[0].B, wdt = probs[0].wdtype;
  for (int i = 0; i < np; ++i)
    if (probs[i].K != K || probs[i].B != B || probs[i].wdtype != wdt || probs[i].N < 1) return hipErrorInvalidValue;
  if (!gemv_rw_supported(wdt, K, B)) return hipErrorInvalidValue;
  MultiGemvParams mp{};
  mp.np = np;
  for (int i = 0; i < np; ++i) mp.prob[i] = probs[i];
  const size_t lds = (size_t)B * (K + (wdt == W_BF16 ? 8 : 4)) * 4;
  size_t al = 0;
  int hda = 0;
  if (attn) {
    if (attn->nkv < 1 || attn->nq % attn->nkv != 0 || attn->nq / attn->nkv > kAttnMaxGroup ||
        attn->n_split > kAttnMaxSplits || (attn->hd != 64 && attn->hd != 128) || attn->wdtype != wdt)
      return hipErrorInvalidValue;
    mp.attn = *attn;
    mp.n_attn = attn->n_split * attn->nkv * attn->B;
    hda = attn->hd;
    al = wdt == W_BF16 ? (hda == 128 ? sizeof(AttnLds<uint16_t, 128>) : sizeof(AttnLds<uint16_t, 64>))
                       : (hda == 128 ? sizeof(AttnLds<float, 128>) : sizeof(AttnLds<float, 64>));
  }
  const int bt = rw_bt(B);
  const hipError_t e = wdt == W_BF16 ? rw_bt_go<uint16_t>(mp, bt, hda, lds, al, s)
                                     : rw_bt_go<float>(mp, bt, hda, lds, al, s);
  if (blocks_out)
    for (int i = 0; i < np; ++i) blocks_out[i] = mp.blk_begin[i + 1] - mp.blk_begin[i];
  return e;
}

hipError_t launch_argmax_finalize(const float* best_val, const int* best_idx, int n, int BT, int B, int* next,
                                  hipStream_t s) {
  launch_timed(argmax_finalize_kernel, dim3(1), dim3(256), 0, s, best_val, best_idx, n, BT, B, next);
  return hipGetLastError();
}

int gemv_rw_bt(int B) { return rw_bt(B); }

}  // namespace ladder

// The layer stack of one decode step (ladder layers, bf16, batch 1..4) in one launch.
//
// Every workgroup is resident for the whole step (the grid is the number that fits on
// the device at once).  The first n_attn workgroups run the split-KV decode attention
// of each layer; the others (NG of them) stream the projections, each owning the same
// share of every projection's row pairs in every layer.  Per ladder layer l a
// projection workgroup runs
//
//   QKV_l     (+RoPE, K/V row)  reads x_{2l-1}   waits until every workgroup finished
//                                                 layer l-1
//   gate/up_l (+SwiGLU)         reads x_{2l}     (exists once layer l-1 is done)
//   down_l    rows kept in LDS  reads a_l        waits until every gate/up_l is done
//   O_l       x_{2l+1} = x_{2l} + o_l,           waits for the attention of layer l
//             x_{2l+2} = x_{2l+1} + d_l
//
// and the attention workgroups run attention_l once every QKV_l is done.  The ladder
// rule is what lets QKV_l and gate/up_l stream back to back, and the attention of
// layer l overlap both MLP projections.  Before each wait a workgroup already has its
// first weight unit of the next projection in flight.  A workgroup keeps the residual
// rows of its O/down share in LDS, so it never reloads what it wrote.
//
// Data that one workgroup writes for another (residual vectors, q, the SwiGLU output,
// the attention output) is stored with coherent stores, each vector at an address of
// its own for this step (x_j in slot j, q/o/a per layer), and read with ordinary
// cached loads after the producers' signal: no address is read in the kernel before
// its final value is written, so no cache can hold a stale copy.  The exceptions are
// read coherently: the newest K/V row (its cache lines are read every layer) and the
// attention's per-chunk records (reused by every layer).  A signal is a
// completed-store wait, a barrier and one store: each projection workgroup publishes
// its progress in a word of its own, and a wait for all of them polls every word (one
// shared counter would serialise hundreds of device-scope atomics per phase).  The
// attention merges, few per layer, count on a shared counter.  Every wait is bounded:
// a wait that gives up sets the error word and the step finishes (with wrong values),
// so no wave can hang.  Per-row arithmetic is that of the per-projection launches, so
// the results are bitwise those of the other schedules.
#include "gemv_rw.hpp"

namespace ladder {

namespace {

constexpr int kStepBlocksPerCu = 2;
constexpr int kStepMinGemvBlocks = 64;   // the LDS of the down rows is sized for this many
constexpr int kStepMaxGemvBlocks = kStepProgWords;

// One layer's pointers, read as plain 64-bit words through a global-address-space pointer.
__device__ __forceinline__ StepLayer load_layer(const StepLayer* p) {
  static_assert(sizeof(StepLayer) % 8 == 0, "StepLayer holds pointers only");
  constexpr int n = sizeof(StepLayer) / 8;
  uint64_t w[n];
#pragma unroll
  for (int i = 0; i < n; ++i) w[i] = gbl((const uint64_t*)p)[i];
  StepLayer s;
  __builtin_memcpy(&s, w, sizeof s);
  return s;
}

// pair range of workgroup g of NG over P row pairs
__device__ __forceinline__ void step_share(int P, int g, int NG, int& p0, int& p1) {
  p0 = (int)((long long)g * P / NG);
  p1 = (int)((long long)(g + 1) * P / NG);
}

}  // namespace

template <int BT, int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_step_kernel(StepParams sp) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  __shared__ RwShared sh;
  const int epoch = *gbl(sp.d_epoch);
  const int n_attn = sp.n_attn;
  const bool attn = (int)blockIdx.x < n_attn;
  const int NG = (int)gridDim.x - n_attn, g = (int)blockIdx.x - n_attn;
  const int qrows = sp.nq * sp.hd, kvrows = sp.nkv * sp.hd;
  float* u = reinterpret_cast<float*>(lds_raw);
  float* xrows = reinterpret_cast<float*>(lds_raw + sp.dres_off);   // [rows][BT] residual rows
  float* drows = xrows + sp.rows_lds * BT;                            // [rows][BT] down rows
  float* part = reinterpret_cast<float*>(lds_raw + sp.part_off);      // partial sums of a pass
  // progress code of phase ph (QKV, gate/up, whole layer) of layer l; the codes of this
  // step exceed every code of earlier steps
  enum { PH_QKV = 0, PH_GU = 1, PH_LAYER = 2 };
  const uint32_t base = (uint32_t)epoch * (uint32_t)(3 * sp.L);
  auto code = [&](int l, int ph) { return base + (uint32_t)(3 * l + ph + 1); };
  // x_j: x_0 (the embeddings) and x_{2L} (the result) in sp.x0, the others in slots
  auto xslot = [&](int j) { return (j == 0 || j == 2 * sp.L) ? sp.x0 : sp.xs + (size_t)(j - 1) * sp.xstride; };

  int h0 = 0, h1 = 0;                                // this workgroup's row pairs of O and down
  if (!attn) {
    step_share((sp.H + 1) / 2, g, NG, h0, h1);
    const int nr = 2 * (h1 - h0);
    for (int i = threadIdx.x; i < nr * BT; i += blockDim.x) {
      const int r = i / BT, b = i % BT, n = 2 * h0 + r;
      xrows[i] = (b < sp.B && n < sp.H) ? gbl(sp.x0)[(size_t)b * sp.H + n] : 0.f;
    }
    __syncthreads();
  }

  for (int l = 0; l < sp.L; ++l) {
    const StepLayer ly = load_layer(sp.layers + l);
    int* sy = sp.sync + 8 * l;       // [4], [5]: attention merges counter and flag
    float* q_l = sp.qs + (size_t)l * sp.qstride;
    float* o_l = sp.os + (size_t)l * sp.qstride;
    float* a_l = sp.as + (size_t)l * sp.astride;
    if (attn) {
      AttnDecodeParams at{};
      at.wdtype = W_BF16;
      at.q = q_l;
      at.k_cache = ly.k_cache;
      at.v_cache = ly.v_cache;
      at.max_seq = sp.max_seq;
      at.nq = sp.nq;
      at.nkv = sp.nkv;
      at.hd = sp.hd;
      at.B = sp.B;
      at.d_pos = sp.d_pos;
      at.n_split = sp.n_split;
      at.part = sp.part;
      at.counters = sp.attn_cnt;
      at.out = o_l;
      at.d_epoch = sp.d_epoch;
      at.done_cnt = sy + 4;
      at.done_flag = sy + 5;
      prog_wait(sp.prog, NG, code(l, PH_QKV), sp.err);
      attn_decode_block_mfma<HD, true>(at, blockIdx.x, *reinterpret_cast<AttnLds<uint16_t, HD>*>(lds_raw));
      __syncthreads();
      continue;
    }
    int p0, p1;
    // ---- QKV_l from x_{2l-1} (x_{-1} = x_0)
    GemvParams qp{};
    qp.wdtype = W_BF16;
    qp.rows = RowSrc{{ly.wq, ly.wk, ly.wv}, qrows, qrows + kvrows, 0};
    qp.N = qrows + 2 * kvrows;
    qp.K = sp.H;
    qp.B = sp.B;
    qp.x = l == 0 ? sp.x0 : xslot(2 * l - 1);
    qp.ldx = sp.H;
    qp.gain = ly.attn_norm;
    qp.eps = sp.eps;
    qp.epi = EPI_QKV_ROPE;
    qp.out = q_l;
    qp.ldo = qrows;
    qp.k_cache = ly.k_cache;
    qp.v_cache = ly.v_cache;
    qp.q_rows = qrows;
    qp.kv_rows = kvrows;
    qp.head_dim = sp.hd;
    qp.max_seq = sp.max_seq;
    qp.n_kv = sp.nkv;
    qp.rope_cos = sp.rope_cos;
    qp.rope_sin = sp.rope_sin;
    qp.d_pos = sp.d_pos;
    RwWait wt;
    wt.err = sp.err;
    if (l > 0) {
      wt.prog = sp.prog;
      wt.nprog = NG;
      wt.code = code(l - 1, PH_LAYER);
    }
    step_share((qp.N + 1) / 2, g, NG, p0, p1);
    rw_pass<uint16_t, BT, kRwVpl, RW_OUT_EPI, true>(qp, p0, p1, g, u, nullptr, wt, sh, part);
    prog_publish(sp.prog + g, code(l, PH_QKV));

    // ---- gate/up_l from x_{2l}
    GemvParams gp{};
    gp.wdtype = W_BF16;
    gp.rows = RowSrc{{ly.wg, ly.wu, nullptr}, 0, 0, 1};
    gp.N = 2 * sp.F;
    gp.K = sp.H;
    gp.B = sp.B;
    gp.x = xslot(2 * l);
    gp.ldx = sp.H;
    gp.gain = ly.mlp_norm;
    gp.eps = sp.eps;
    gp.epi = EPI_GATEUP_SWIGLU;
    gp.out = a_l;
    gp.ldo = sp.F;
    RwWait wg;
    wg.err = sp.err;
    step_share(sp.F, g, NG, p0, p1);
    rw_pass<uint16_t, BT, kRwVpl, RW_OUT_EPI, true>(gp, p0, p1, g, u, nullptr, wg, sh, part);
    prog_publish(sp.prog + g, code(l, PH_GU));

    GemvParams op{};
    op.wdtype = W_BF16;
    op.rows = RowSrc{{ly.wo, nullptr, nullptr}, sp.H, sp.H, 0};
    op.N = sp.H;
    op.K = qrows;
    op.B = sp.B;
    op.x = o_l;
    op.ldx = qrows;
    op.out = xslot(2 * l + 1);
    op.ldo = sp.H;
    RwWait wa;
    wa.flag = sy + 5;
    wa.epoch = epoch;
    wa.err = sp.err;
    GemvParams dp{};
    dp.wdtype = W_BF16;
    dp.rows = RowSrc{{ly.wd, nullptr, nullptr}, sp.H, sp.H, 0};
    dp.N = sp.H;
    dp.K = sp.F;
    dp.B = sp.B;
    dp.x = a_l;
    dp.ldx = sp.F;
    dp.out = xslot(2 * l + 2);
    dp.ldo = sp.H;
    RwWait wd;
    wd.prog = sp.prog;
    wd.nprog = NG;
    wd.code = code(l, PH_GU);
    wd.err = sp.err;
    // down_l rows into LDS; then O_l: x_{2l+1} = x_{2l} + o_l, x_{2l+2} = x_{2l+1} + d_l
    rw_pass<uint16_t, BT, kRwVpl, RW_OUT_LDS, true>(dp, h0, h1, g, u, drows, wd, sh, part);
    __syncthreads();
    op.out2 = xslot(2 * l + 2);
    rw_pass<uint16_t, BT, kRwVpl, RW_OUT_ADD2_LDSRES, true>(op, h0, h1, g, u, drows, wa, sh, part, xrows);
    prog_publish(sp.prog + g, code(l, PH_LAYER));
  }
}

namespace {

// LDS of a projection workgroup: u (the staged input), the residual rows and the down
// rows of its O/down share; at least the attention's LDS.
size_t step_lds(int H, int F, int qrows, int kvrows, int B, int hd, int* dres_off, int* rows_lds, int* part_off) {
  int kmax = H > F ? H : F;
  if (qrows > kmax) kmax = qrows;
  const size_t ub = (size_t)B * (kmax + 8) * 4;
  const size_t off = (ub + 15) / 16 * 16;
  const int P = (H + 1) / 2;
  const int per = (P + kStepMinGemvBlocks - 1) / kStepMinGemvBlocks;
  const int rows = 2 * (per > 4 ? per : 4);
  *dres_off = (int)off;
  *rows_lds = rows;
  size_t lds = off + 2 * (size_t)rows * 4 * sizeof(float);   // residual rows, then down rows
  // partial sums: the most pairs a workgroup gets in any pass (at least 64 projection
  // workgroups), times the chunks of that pass's K
  const int BT = B <= 1 ? 1 : B <= 2 ? 2 : 4;
  auto share = [](int pairs) { return (pairs + kStepMinGemvBlocks - 1) / kStepMinGemvBlocks; };
  size_t pf = rw_part_floats(share((qrows + 2 * kvrows + 1) / 2), H, 8, BT);
  const size_t f_gu = rw_part_floats(share(F), H, 8, BT);
  const size_t f_d = rw_part_floats(share(P), F, 8, BT);
  const size_t f_o = rw_part_floats(share(P), qrows, 8, BT);
  if (f_gu > pf) pf = f_gu;
  if (f_d > pf) pf = f_d;
  if (f_o > pf) pf = f_o;
  *part_off = (int)((lds + 15) / 16 * 16);
  lds = (size_t)*part_off + pf * sizeof(float);
  const size_t al = hd == 128 ? sizeof(AttnLds<uint16_t, 128>) : sizeof(AttnLds<uint16_t, 64>);
  return lds > al ? lds : al;
}

// workgroups of decode_step_kernel<BT, HD> resident at once with `lds` bytes each
template <int BT, int HD>
hipError_t step_blocks(size_t lds, int* blocks) {
  auto fn = decode_step_kernel<BT, HD>;
  static size_t cached_lds = 0;
  static int cached_blocks = 0;
  if (cached_lds != lds || cached_blocks == 0) {
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
    cached_blocks = (per_cu < kStepBlocksPerCu ? per_cu : kStepBlocksPerCu) * ncu;
    cached_lds = lds;
  }
  *blocks = cached_blocks;
  return hipSuccess;
}

// Resolve the launch: fills n_attn and dres_off, returns the grid (0 if it cannot run).
int step_plan(StepParams& sp, size_t* lds_out, hipError_t* err) {
  *err = hipSuccess;
  const int qrows = sp.nq * sp.hd;
  if (sp.nkv < 1 || sp.nq % sp.nkv != 0 || !step_supported(W_BF16, sp.H, sp.F, qrows, sp.B, sp.hd, sp.nq / sp.nkv) ||
      sp.n_split < 1 || sp.n_split > kAttnMaxSplits || sp.L < 1 || !sp.layers || !sp.sync || !sp.prog || !sp.err || !sp.xs || !sp.qs || !sp.os || !sp.as)
    return 0;
  sp.n_attn = sp.n_split * sp.nkv * sp.B;
  const size_t lds = step_lds(sp.H, sp.F, qrows, sp.nkv * sp.hd, sp.B, sp.hd, &sp.dres_off, &sp.rows_lds, &sp.part_off);
  *lds_out = lds;
  const int bt = sp.B <= 1 ? 1 : sp.B <= 2 ? 2 : 4;
  int blocks = 0;
#define STEP_BLOCKS(BT_, HD_) step_blocks<BT_, HD_>(lds, &blocks)
  if (sp.hd == 128)
    *err = bt == 1 ? STEP_BLOCKS(1, 128) : bt == 2 ? STEP_BLOCKS(2, 128) : STEP_BLOCKS(4, 128);
  else
    *err = bt == 1 ? STEP_BLOCKS(1, 64) : bt == 2 ? STEP_BLOCKS(2, 64) : STEP_BLOCKS(4, 64);
#undef STEP_BLOCKS
  if (*err != hipSuccess) return 0;
  if (blocks - sp.n_attn > kStepMaxGemvBlocks) blocks = sp.n_attn + kStepMaxGemvBlocks;
  return blocks >= sp.n_attn + kStepMinGemvBlocks ? blocks : 0;   // every workgroup resident
}

}  // namespace

bool step_supported(int wdtype, int H, int F, int qrows, int B, int hd, int G) {
  // every projection's staged input within ~65 KB of LDS (two resident workgroups per CU)
  int kmax = H > F ? H : F;
  if (qrows > kmax) kmax = qrows;
  return wdtype == W_BF16 && (hd == 64 || hd == 128) && G >= 1 && G <= kAttnMaxGroup &&
         gemv_rw_supported(wdtype, kmax, B) && (size_t)B * (kmax + 8) * 4 <= 66560;
}

bool step_fits(const StepParams& sp_in) {
  StepParams sp = sp_in;
  size_t lds = 0;
  hipError_t e;
  return step_plan(sp, &lds, &e) > 0;
}

hipError_t launch_decode_step(const StepParams& sp_in, hipStream_t s) {
  StepParams sp = sp_in;
  size_t lds = 0;
  hipError_t e;
  const int grid = step_plan(sp, &lds, &e);
  if (e != hipSuccess) return e;
  if (grid == 0) return hipErrorInvalidValue;
  const int bt = sp.B <= 1 ? 1 : sp.B <= 2 ? 2 : 4;
  const dim3 g(grid), b(256);
  const uint32_t ls = (uint32_t)lds;
#define STEP_GO(BT_, HD_) launch_timed(decode_step_kernel<BT_, HD_>, g, b, ls, s, sp)
  if (sp.hd == 128) {
    if (bt == 1) STEP_GO(1, 128);
    else if (bt == 2) STEP_GO(2, 128);
    else STEP_GO(4, 128);
  } else {
    if (bt == 1) STEP_GO(1, 64);
    else if (bt == 2) STEP_GO(2, 64);
    else STEP_GO(4, 64);
  }
#undef STEP_GO
  return hipGetLastError();
}

}  // namespace ladder

// libladder runtime: context, workspace, module schedule and the C ABI of include/ladder.h.
//
// Module loop (decode and prefill).  Modules m = 0..2L-1 alternate attention / MLP;
// module m reads x_src with src = m-1 for a ladder layer (x_{-1} = x_0) and src = m for
// a standard one, and the stream advances as x_{m+1} = x_m + out_m.  Because a ladder
// module never reads the output of the module right before it, module m+1 can start
// before x_{m+1} exists.  Three schedules realise this on one GPU:
//   SERIAL: everything on one stream in program order (the reference order);
//   SIDE:   modules on the main stream, each residual add on a side stream; module m+1
//           waits only for the add that produced its own (stale) input;
//   DUAL:   attention modules on the origin stream (A), MLP modules on a second stream
//           (B), each residual add
//           fused into the module's output projection.  A module waits for its input
//           residual, and its output projection waits for x_m, produced by the other
//           stream.  Ladder modules overlap the previous module (attention of layer l+1
//           runs beside the MLP of layer l).
// All three compute every value with the same kernels and the same arithmetic, so
// their results are bitwise identical (the race check of the test suite).
//
// Two residual buffers are in flight (x_{m-1} and x_m while x_{m+1} is formed into the
// slot of x_{m-1}); the ordering argument for each schedule is in the comments of
// run_modules().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "ladder.h"
#include "kernels.h"

using namespace ladder;

namespace {

struct StreamScratch {
  // decode
  float* q = nullptr;
  float* attn_part = nullptr;
  int* attn_cnt = nullptr;
  float* o = nullptr;
  float* a = nullptr;
  float* gpart = nullptr;
  float* gpart_sq = nullptr;
  int* gcnt = nullptr;
  // prefill (module inputs of the projections stay fp32; the GEMM splits them)
  float* u = nullptr;
  float* qkv = nullptr;
  float* qr = nullptr;
  float* ob = nullptr;
  float* gu = nullptr;
  float* ab = nullptr;
  float* gk = nullptr;   // split-K partials of the prefill GEMMs (bf16 models)
  float* apart = nullptr;  // key-chunk records of the prefill attention (bf16 models)
  int* skcnt = nullptr;    // tickets of the skinny GEMM launches (bf16 models)
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Carver {
  size_t off = 0;
  char* base = nullptr;
  template <typename T>
  T* take(size_t count) {
    const size_t bytes = align_up(count * sizeof(T) + 16, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

}  // namespace

struct ladder_ctx {
  ladder_config cfg{};
  std::vector<uint8_t> mask;
  std::vector<ladder_layer_weights> layers;
  ladder_weights w{};
  ladder_kv kv{};
  int dev = 0;
  int esz = 2;               // bytes per weight / KV element
  int wdt = W_BF16;
  int qrows = 0, kvrows = 0; // n_q_heads*head_dim, n_kv_heads*head_dim
  int n_split = 1;
  int mmax = 0;              // prefill rows per chunk
  size_t layer_kv_elems = 0;

  hipStream_t user = nullptr;   // caller's stream
  hipStream_t s0 = nullptr;     // origin stream of every call (graph capture happens here)
  hipStream_t sb = nullptr, side = nullptr;   // MLP stream of DUAL, add stream of SIDE
  std::vector<hipEvent_t> ev_x, ev_out;
  hipEvent_t ev_fork = nullptr, ev_in = nullptr, ev_done = nullptr;

  char* ws = nullptr;
  size_t ws_bytes = 0;
  size_t step_off = 0;       // offset of the per-step part in ws
  size_t step_zero_bytes = 0;   // leading bytes of the per-step part a step needs at zero
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  float* dx[2] = {nullptr, nullptr};     // decode residual ring [max_batch][H]
  float* dout[2] = {nullptr, nullptr};   // decode module outputs (SERIAL / SIDE)
  float* px[2] = {nullptr, nullptr};     // prefill residual ring [mmax][H]
  float* pout[2] = {nullptr, nullptr};
  int* ids_dev = nullptr;
  int* pos_dev = nullptr;
  int* ids_chunk = nullptr;
  float* logits = nullptr;
  int* next = nullptr;
  float* best_val = nullptr;
  int* best_idx = nullptr;
  int* arg_cnt = nullptr;
  int* epoch = nullptr;           // decode steps enqueued (bumped by the step's prologue)
  int* attn_done_cnt = nullptr;   // [L] attention merges finished in the current step
  int* attn_done_flag = nullptr;  // [L] epoch of the last step whose attention finished
  int* err_word = nullptr;        // set by a kernel whose bounded wait gave up
  StepLayer* step_layers = nullptr;  // [L] per-layer pointers of the persistent decode step
  int* step_sync = nullptr;          // [L][8] its counters and flags
  uint32_t* step_prog = nullptr;     // [kStepProgWords] its progress words
  uint32_t* seq_prog = nullptr;      // [kSeqProgWords] progress words of the sequential launches
  unsigned long long* qkv_tagged = nullptr;  // [qkv rows] tagged QKV outputs of the batch-1 streaming launch
  float* step_x = nullptr;           // x_1 .. x_{2L-1}
  float* step_q = nullptr;           // q per layer
  float* step_o = nullptr;           // attention output per layer
  float* step_a = nullptr;           // SwiGLU output per layer
  size_t step_xstride = 0, step_qstride = 0, step_astride = 0;
  bool all_ladder = false;           // every layer follows the ladder rule
  StreamScratch sc[2];

  int sched = LADDER_SCHED_FUSED;
  int use_graph = 1;
  bool gemm_step = false;            // a decode step is running through the prefill modules
  // a decode step of 33-64 sequences through the tiled GEMMs: the next attention module's
  // QKV launch also runs its layer's gate/up projection (pair_gu, ready when pair_next),
  // and the MLP module then skips it (skip_gateup)
  GemmParams pair_gu{};
  bool pair_next = false, skip_gateup = false;
  // and its O projection waits for the down projection (pair_o, when o_deferred)
  GemmParams pair_o{};
  bool o_deferred = false;
  // and its attention runs in that launch too (pair_at, when at_deferred)
  AttnDecodeParams pair_at{};
  bool at_deferred = false;
  // next-token rule: greedy, or a draw (temperature > 0) with an optional top-k cut
  float temperature = 0.f;
  int top_k = 0;
  uint64_t seed = 0;
  int trace_kind = -1;               // kernel kind timed with events during decode (-1: none)
  std::vector<hipEvent_t> trace_ev;  // start/end pairs, one pair per traced launch
  int trace_n = 0;                   // pairs recorded by the step being enqueued
  int trace_count = 0;               // pairs a decode step records
  std::map<int, hipGraphExec_t> graphs;
  int filled = 0;
  bool broken = false;
  std::string err;
};

namespace {

ladder_status fail(ladder_ctx* c, ladder_status s, const char* fmt, const char* what = "") {
  if (c) {
    char buf[512];
    snprintf(buf, sizeof buf, fmt, what);
    c->err = buf;
  }
  return s;
}

#define HIPCHK(call)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess) {                                                             \
      ctx->broken = true;                                                               \
      return fail(ctx, LADDER_ERR_HIP, "%s", (std::string(#call) + ": " + hipGetErrorString(e_)).c_str()); \
    }                                                                                   \
  } while (0)

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

ladder_status validate(const ladder_config* c, const ladder_weights* w, const ladder_kv* kv) {
  if (!c || !w || !kv || !c->ladder_mask || !w->layers) return LADDER_ERR_ARG;
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->ffn < 1 || c->vocab < 1 || c->max_batch < 1 || c->max_seq < 1 || c->max_prefill_tokens < 0)
    return LADDER_ERR_ARG;
  if (c->dtype != LADDER_F32 && c->dtype != LADDER_BF16) return LADDER_ERR_ARG;
  if (!(c->rope_theta > 0.0) || !(c->norm_eps >= 0.0f)) return LADDER_ERR_ARG;
  if (c->kv_filled < 0 || c->kv_filled > c->max_seq) return LADDER_ERR_ARG;
  if (c->rope_scale_factor != 0.0 &&
      !(c->rope_scale_factor >= 1.0 && std::isfinite(c->rope_scale_factor) && c->rope_low_freq_factor > 0.0 &&
        c->rope_high_freq_factor > c->rope_low_freq_factor && std::isfinite(c->rope_high_freq_factor) &&
        c->rope_orig_max_pos > 0))
    return LADDER_ERR_ARG;
  // fp32 models decode beyond batch 4 with the K-sliced GEMV (at most 16 rows); bf16
  // models on the matrix cores (the decode prologue takes at most 256 sequences)
  if (c->max_batch > (c->dtype == LADDER_BF16 ? 256 : 16)) return LADDER_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads != 0 || c->n_q_heads / c->n_kv_heads > 16) return LADDER_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return LADDER_ERR_SHAPE;
  const int vec = c->dtype == LADDER_BF16 ? 8 : 4;
  if (c->hidden % vec || c->ffn % vec) return LADDER_ERR_SHAPE;
  if (c->dtype == LADDER_BF16 &&
      (c->hidden % 64 || c->ffn % 64 || (c->n_q_heads * c->head_dim) % 64))
    return LADDER_ERR_SHAPE;   // K of every prefill contraction is a whole number of 64-wide MFMA steps
  for (int l = 0; l < c->n_layers; ++l)
    if (c->ladder_mask[l] > 2) return LADDER_ERR_ARG;
  if (!aligned16(w->tok_embed) || !aligned16(w->final_norm) || !aligned16(w->lm_head)) return LADDER_ERR_ARG;
  for (int l = 0; l < c->n_layers; ++l) {
    const ladder_layer_weights& L = w->layers[l];
    const void* ps[] = {L.attn_norm, L.wq, L.wk, L.wv, L.wo, L.mlp_norm, L.w_gate, L.w_up, L.w_down};
    for (const void* p : ps)
      if (!aligned16(p)) return LADDER_ERR_ARG;
  }
  if (!aligned16(kv->k) || !aligned16(kv->v)) return LADDER_ERR_ARG;
  return LADDER_OK;
}

// Rotation frequency of pair j: theta^(-2j/head_dim), then, with scaling on, Llama-3.1's
// bands by wavelength w = 2 pi / f against the original context N: short waves (w < N /
// high) keep f, long ones (w > N / low) take f / factor, and the waves between blend the
// two linearly in N / w, so f' is continuous at both band edges.
double rope_frequency(const ladder_config& c, int j) {
  const double f = std::pow(c.rope_theta, -2.0 * j / c.head_dim);
  if (c.rope_scale_factor == 0.0) return f;
  const double N = c.rope_orig_max_pos, w = 2.0 * M_PI / f;
  if (w < N / c.rope_high_freq_factor) return f;
  if (w > N / c.rope_low_freq_factor) return f / c.rope_scale_factor;
  const double s = (N / w - c.rope_low_freq_factor) / (c.rope_high_freq_factor - c.rope_low_freq_factor);
  return (1.0 - s) * f / c.rope_scale_factor + s * f;
}

// Shape of the per-step part of the workspace: buffers for batches up to B, prefill-route
// rows up to `rows`, `nsc` stream scratch sets, the GEMMs' split-K partials and the prefill
// attention's chunk records.
struct StepShape {
  int B, rows, nsc;
  bool gk, apart;
};

StepShape ws_step_shape(const ladder_ctx* c) {
  const bool bf = c->wdt == W_BF16;
  return StepShape{c->cfg.max_batch, c->mmax, 2, bf, bf};
}

// The part of the workspace that lasts across calls: RoPE table, prefill residual rings,
// step counter, error word and the persistent decode step's buffers.
void carve_fixed(ladder_ctx* c, Carver& cv) {
  const ladder_config& g = c->cfg;
  const int H = g.hidden, F = g.ffn, B = g.max_batch;
  c->rope_cos = cv.take<float>((size_t)g.max_seq * g.head_dim / 2);
  c->rope_sin = cv.take<float>((size_t)g.max_seq * g.head_dim / 2);
  for (int i = 0; i < 2; ++i) {
    c->px[i] = cv.take<float>((size_t)c->mmax * H);
    c->pout[i] = cv.take<float>((size_t)c->mmax * H);
  }
  c->ids_chunk = cv.take<int>(c->mmax);
  c->epoch = cv.take<int>(1);
  c->err_word = cv.take<int>(1);
  c->step_layers = cv.take<StepLayer>((size_t)g.n_layers);
  c->step_sync = cv.take<int>((size_t)8 * g.n_layers);
  c->step_prog = cv.take<uint32_t>(kStepProgWords);
  // vectors of the persistent decode step, each at an address of its own per step
  if (c->all_ladder && c->wdt == W_BF16) {
    const size_t sb = std::min(B, 4);
    c->step_xstride = align_up(sb * H, 64);
    c->step_qstride = align_up(sb * c->qrows, 64);
    c->step_astride = align_up(sb * F, 64);
    c->step_x = cv.take<float>((size_t)(2 * g.n_layers - 1) * c->step_xstride);
    c->step_q = cv.take<float>((size_t)g.n_layers * c->step_qstride);
    c->step_o = cv.take<float>((size_t)g.n_layers * c->step_qstride);
    c->step_a = cv.take<float>((size_t)g.n_layers * c->step_astride);
  }
}

// The part a decode step (and a prefill chunk) uses only while it runs.  The counters,
// flags and handoff words come first and end at c->step_zero_bytes from the part's start:
// the kernels need them at zero, or holding earlier codes of this context, when a step
// starts (each counter returns to zero after its last use in a step).
void carve_step(ladder_ctx* c, Carver& cv, const StepShape& sh) {
  const ladder_config& g = c->cfg;
  const int H = g.hidden, F = g.ffn, V = g.vocab, B = sh.B;
  const int qkv = c->qrows + 2 * c->kvrows;
  // GEMV split-K / argmax scratch: the largest need over every decode GEMV shape and batch
  GemvWorkspaceReq need{};
  const int shapes[5][2] = {{qkv, H}, {H, c->qrows}, {2 * F, H}, {H, F}, {V, H}};
  for (int b = 1; b <= B; ++b)
    for (auto& shp : shapes) {
      GemvWorkspaceReq r = gemv_workspace(c->wdt, shp[0], shp[1], b);
      need.part_floats = std::max(need.part_floats, r.part_floats);
      need.part_sq_floats = std::max(need.part_sq_floats, r.part_sq_floats);
      need.counters = std::max(need.counters, r.counters);
      need.best = std::max(need.best, r.best);
    }
  const size_t start = cv.off;
  c->arg_cnt = cv.take<int>(1);
  c->attn_done_cnt = cv.take<int>((size_t)g.n_layers);
  c->attn_done_flag = cv.take<int>((size_t)g.n_layers);
  c->seq_prog = cv.take<uint32_t>(kSeqProgWords);
  c->qkv_tagged = cv.take<unsigned long long>((size_t)qkv);
  for (int s = 0; s < sh.nsc; ++s) {
    c->sc[s].attn_cnt = cv.take<int>((size_t)B * g.n_kv_heads);
    c->sc[s].gcnt = cv.take<int>(need.counters);
    c->sc[s].skcnt = sh.gk ? cv.take<int>(kSkinnyMaxTiles) : nullptr;
  }
  c->step_zero_bytes = cv.off - start;
  for (int i = 0; i < 2; ++i) {
    c->dx[i] = cv.take<float>((size_t)B * H);
    c->dout[i] = cv.take<float>((size_t)B * H);
  }
  c->ids_dev = cv.take<int>(B);
  c->pos_dev = cv.take<int>(1);
  c->logits = cv.take<float>((size_t)B * V);
  c->next = cv.take<int>(B);
  const size_t nbest = std::max<size_t>(need.best, 1024 * 16);
  c->best_val = cv.take<float>(nbest);
  c->best_idx = cv.take<int>(nbest);
  for (int s = 0; s < sh.nsc; ++s) {
    StreamScratch& sc = c->sc[s];
    sc.q = cv.take<float>((size_t)B * c->qrows);
    sc.attn_part = cv.take<float>((size_t)B * g.n_q_heads * c->n_split * (g.head_dim + 4));
    sc.o = cv.take<float>((size_t)B * c->qrows);
    sc.a = cv.take<float>((size_t)B * F);
    sc.gpart = cv.take<float>(need.part_floats);
    sc.gpart_sq = cv.take<float>(need.part_sq_floats);
    sc.u = cv.take<float>((size_t)sh.rows * H);
    sc.qkv = cv.take<float>((size_t)sh.rows * qkv);
    sc.qr = cv.take<float>((size_t)sh.rows * c->qrows);
    sc.ob = cv.take<float>((size_t)sh.rows * c->qrows);
    sc.gu = cv.take<float>((size_t)sh.rows * 2 * F);
    sc.gk = sh.gk ? cv.take<float>(kGemmSplitWsFloats) : nullptr;
    sc.apart = sh.apart ? cv.take<float>(attn_prefill_part_floats(g.head_dim)) : nullptr;
    sc.ab = cv.take<float>((size_t)sh.rows * F);
  }
}

// Lay the whole workspace out (base == nullptr: only measure).
void carve(ladder_ctx* c, Carver& cv) {
  carve_fixed(c, cv);
  c->step_off = cv.off;
  carve_step(c, cv, ws_step_shape(c));
}

// Point the per-step buffers back at the context's own workspace.
void carve_ws_step(ladder_ctx* c) {
  Carver cv;
  cv.off = c->step_off;
  cv.base = c->ws;
  carve_step(c, cv, ws_step_shape(c));
}

// Event pair spanning the dispatches of the launches of kernel kind `kind` (traced
// steps are eager; the events take the dispatches' own begin/end timestamps).
ladder_status trace_mark(ladder_ctx* ctx, int kind, hipStream_t s, bool end) {
  (void)s;
  if (ctx->trace_kind != kind) return LADDER_OK;
  const size_t i = 2 * (size_t)ctx->trace_n;
  if (i + 1 >= ctx->trace_ev.size()) return LADDER_OK;
  if (!end) {
    launch_events_arm(ctx->trace_ev[i], ctx->trace_ev[i + 1]);
  } else {
    launch_events_disarm();
    ++ctx->trace_n;
  }
  return LADDER_OK;
}

#define TRACE(kind, s, end)                                   \
  do {                                                        \
    ladder_status t_ = trace_mark(ctx, (kind), (s), (end));   \
    if (t_) return t_;                                        \
  } while (0)

// Index j of the residual x_j that module m (2l attention, 2l+1 MLP of layer l) reads:
// standard layers (mask 0) read x_m; ladder layers (mask 1) x_{m-1}, with x_{-1} = x_0
// (Paper-Notes page, "method details / key design: staggered residual connection");
// parallel blocks (mask 2) feed both modules the layer input x_{2l}, i.e. the attention
// reads x_m and the MLP x_{m-1}.
inline int module_src(const ladder_ctx* c, int m) {
  const int mode = c->mask[m / 2];
  const bool back = mode == 1 || (mode == 2 && (m & 1));
  return back ? (m > 0 ? m - 1 : 0) : m;
}

void* layer_k(const ladder_ctx* c, int l) { return (char*)c->kv.k + (size_t)l * c->layer_kv_elems * c->esz; }
void* layer_v(const ladder_ctx* c, int l) { return (char*)c->kv.v + (size_t)l * c->layer_kv_elems * c->esz; }

// Stream running module m under the current schedule.
hipStream_t module_stream(const ladder_ctx* c, int m) {
  if (c->sched == LADDER_SCHED_DUAL) return (m % 2 == 0) ? c->s0 : c->sb;
  return c->s0;
}

StreamScratch& module_scratch(ladder_ctx* c, int m) {
  return c->sc[(c->sched == LADDER_SCHED_DUAL && m % 2 == 1) ? 1 : 0];
}

// ---------------------------------------------------------------- decode module
// Parameter builders of the decode kernels (shared by the module loop and the
// per-kernel timing entry point, so both launch exactly the same configuration).
GemvParams gemv_base(const ladder_ctx* ctx, int B, const StreamScratch& sc) {
  GemvParams p{};
  p.wdtype = ctx->wdt;
  p.B = B;
  p.eps = ctx->cfg.norm_eps;
  p.part = sc.gpart;
  p.part_sq = sc.gpart_sq;
  p.counters = sc.gcnt;
  return p;
}

// RMSNorm + [Wq;Wk;Wv] + RoPE + KV append of layer l
GemvParams qkv_params(const ladder_ctx* ctx, int l, int B, const float* xin, const StreamScratch& sc) {
  const ladder_config& g = ctx->cfg;
  const ladder_layer_weights& L = ctx->layers[l];
  GemvParams p = gemv_base(ctx, B, sc);
  p.rows = RowSrc{{L.wq, L.wk, L.wv}, ctx->qrows, ctx->qrows + ctx->kvrows, 0};
  p.N = ctx->qrows + 2 * ctx->kvrows;
  p.K = g.hidden;
  p.x = xin;
  p.ldx = g.hidden;
  p.gain = L.attn_norm;
  p.epi = EPI_QKV_ROPE;
  p.out = sc.q;
  p.ldo = ctx->qrows;
  p.k_cache = layer_k(ctx, l);
  p.v_cache = layer_v(ctx, l);
  p.q_rows = ctx->qrows;
  p.kv_rows = ctx->kvrows;
  p.head_dim = g.head_dim;
  p.max_seq = g.max_seq;
  p.n_kv = g.n_kv_heads;
  p.rope_cos = ctx->rope_cos;
  p.rope_sin = ctx->rope_sin;
  p.d_pos = ctx->pos_dev;
  return p;
}

// Key chunks of the matrix-core route's decode attention: at most decode_attn_fill(B) / (B *
// kv heads) workgroups' worth (and at most the context's own split), a function of the batch
// only, so that every schedule gives the same bits.  Up to 32 sequences the attention runs
// inside the skinny [QKV | gate/up] launch, its workgroups waiting there beside the gate/up
// rows: 128 measured 2766 tok/s at batch 16 on the 70B shard against 2514 with 256 and 2681
// with 64 (batch 8 within 0.3%); 256 at 17-32 sequences: 4862 / 3668 / 2762 against 4552
// / 3703 / 2716 with 128 at batch 32 / 24 / 17, the 405B shard 2007 against 1897 at batch
// 32, the 8B model at batch 24 within 0.1%.  Beyond,
// the attention shares the tiled [down | O] launch, where 256 measured 4474 / 1961 tok/s
// (70B / 405B shard, batch 64, in a launch of its own then) against 4383 / 1869.
constexpr int decode_attn_fill(int B) { return B <= 16 ? 128 : 256; }
// (Decode steps of 17-32 sequences on models narrower than 16384 took the tiled GEMMs'
// paired launches for a while: 3472 against 3077 tok/s at batch 32 on the 70B shard.  With
// the skinny launches' K cut for about 128 items per K part the skinny launches measured
// 2723 / 3712 / 4559 against 2293 / 3106 / 4020 tok/s at batch 17 / 24 / 32, the 8B model
// 4309 against 3789 at batch 24, so every batch up to 32 takes them again.)
constexpr bool kAttnInOutLaunch = true;

AttnDecodeParams attn_params(const ladder_ctx* ctx, int l, int B, const StreamScratch& sc) {
  const ladder_config& g = ctx->cfg;
  AttnDecodeParams a{};
  a.wdtype = ctx->wdt;
  a.q = sc.q;
  a.k_cache = layer_k(ctx, l);
  a.v_cache = layer_v(ctx, l);
  a.max_seq = g.max_seq;
  a.nq = g.n_q_heads;
  a.nkv = g.n_kv_heads;
  a.hd = g.head_dim;
  a.B = B;
  a.d_pos = ctx->pos_dev;
  a.n_split = ctx->n_split;
  a.part = sc.attn_part;
  a.counters = sc.attn_cnt;
  a.out = sc.o;
  a.d_epoch = ctx->epoch;   // the step counter (codes of the sequential launch's waits)
  return a;
}

// Attention of layer l that signals its completion (to the paired down + O launch).
AttnDecodeParams signalled(const ladder_ctx* ctx, AttnDecodeParams a, int l) {
  a.d_epoch = ctx->epoch;
  a.done_cnt = ctx->attn_done_cnt + l;
  a.done_flag = ctx->attn_done_flag + l;
  return a;
}

// Two launches per ladder layer (bf16, batch <= 4): [QKV | gate/up] and [attention |
// down, then (once the attention has signalled) O + both residual adds].
bool two_launch_layers(const ladder_ctx* ctx, int B) {
  const ladder_config& g = ctx->cfg;
  return gemv_rw_supported(ctx->wdt, g.hidden, B) && gemv_rw_pair_supported(ctx->wdt, g.ffn, ctx->qrows, B);
}

// The two launches of the FUSED schedule instead: [QKV, then gate/up, in every workgroup |
// attention once every QKV share is done] and [down rows, then O + both residual adds].
// Layer l's launch uses the progress tag l + 1.  Only while the first launch keeps two
// workgroups per CU: with one (batch 2-4 at hidden 8192) its attention workgroups would
// each hold a CU that no longer streams weights (at batch 4, 64 of 256), and the layout
// with the attention in the down projection's launch is faster (420 against 370 tok/s
// on the 70B shard at batch 4).
bool seq_layers(const ladder_ctx* ctx, int B) {
  const ladder_config& g = ctx->cfg;
  return two_launch_layers(ctx, B) && gemv_rw_seq_supported(ctx->wdt, g.hidden, B, g.head_dim) &&
         gemv_rw_two_per_cu(ctx->wdt, g.hidden, B) && g.n_layers < (int)kSeqCodeStride;
}

// Batch 1 with both decode launches of a layer streaming (stream.hip): the front launch
// leaves the attention as chunk records, the back launch merges them.
bool stream_layers(const ladder_ctx* ctx, int B) {
  const ladder_config& g = ctx->cfg;
  return B == 1 && seq_layers(ctx, B) && stream_front_supported(ctx->wdt, g.hidden, B, g.head_dim) &&
         stream_back_supported(ctx->wdt, g.ffn, ctx->qrows, B, g.hidden, g.n_q_heads, ctx->n_split);
}

// RMSNorm + [Wgate,Wup] (row pairs) + SwiGLU of layer l
GemvParams gateup_params(const ladder_ctx* ctx, int l, int B, const float* xin, const StreamScratch& sc) {
  const ladder_config& g = ctx->cfg;
  const ladder_layer_weights& L = ctx->layers[l];
  GemvParams p = gemv_base(ctx, B, sc);
  p.rows = RowSrc{{L.w_gate, L.w_up, nullptr}, 0, 0, 1};
  p.N = 2 * g.ffn;
  p.K = g.hidden;
  p.x = xin;
  p.ldx = g.hidden;
  p.gain = L.mlp_norm;
  p.epi = EPI_GATEUP_SWIGLU;
  p.out = sc.a;
  p.ldo = g.ffn;
  return p;
}

// Output projection (Wo for attention, Wdown for the MLP) of module m: with the residual
// add fused (out_x = x_m + out_m) or storing out_m.
GemvParams outproj_params(const ladder_ctx* ctx, int m, int B, const StreamScratch& sc, const float* xm,
                          float* out_x, float* out_store) {
  const ladder_config& g = ctx->cfg;
  const ladder_layer_weights& L = ctx->layers[m / 2];
  const bool attn = m % 2 == 0;
  GemvParams o = gemv_base(ctx, B, sc);
  o.rows = RowSrc{{attn ? L.wo : L.w_down, nullptr, nullptr}, g.hidden, g.hidden, 0};
  o.N = g.hidden;
  o.K = attn ? ctx->qrows : g.ffn;
  o.x = attn ? sc.o : sc.a;
  o.ldx = o.K;
  o.gain = nullptr;
  if (out_x) {
    o.epi = EPI_ADD;
    o.xres = xm;
    o.ldr = g.hidden;
    o.out = out_x;
  } else {
    o.epi = EPI_STORE;
    o.out = out_store;
  }
  o.ldo = g.hidden;
  return o;
}

GemvParams lmhead_params(const ladder_ctx* ctx, const float* x, int ldx, int B) {
  const ladder_config& g = ctx->cfg;
  GemvParams p = gemv_base(ctx, B, ctx->sc[0]);
  p.rows = RowSrc{{ctx->w.lm_head, nullptr, nullptr}, g.vocab, g.vocab, 0};
  p.N = g.vocab;
  p.K = g.hidden;
  p.x = x;
  p.ldx = ldx;
  p.gain = ctx->w.final_norm;
  p.epi = EPI_LOGITS;
  p.out = ctx->logits;
  p.ldo = g.vocab;
  p.best_val = ctx->best_val;
  p.best_idx = ctx->best_idx;
  p.arg_counter = ctx->arg_cnt;
  p.next_out = ctx->next;
  return p;
}

// One decode GEMV: the row-wave kernel when the batch and K allow (its per-row
// arithmetic is the same in every launch shape), else the K-sliced kernel.  Logits get
// their greedy argmax finalised by a one-workgroup kernel in the first case (the
// K-sliced kernel finalises in its last workgroup).
ladder_status run_gemv(ladder_ctx* ctx, const GemvParams& p, hipStream_t s) {
  if (gemv_rw_supported(p.wdtype, p.K, p.B)) {
    int nb = 0;
    HIPCHK(launch_gemv_multi(&p, 1, nullptr, s, &nb));
    if (p.epi == EPI_LOGITS)
      HIPCHK(launch_argmax_finalize(p.best_val, p.best_idx, nb, gemv_rw_bt(p.B), p.B, p.next_out, s));
  } else {
    HIPCHK(launch_gemv(p, s));
  }
  return LADDER_OK;
}

// Enqueue module m of one decode step.  out_x != nullptr: fused residual add
// (out_x = x_m + out_m); else out_m goes to out_store.
ladder_status decode_module(ladder_ctx* ctx, int m, int B, const float* xin, const float* xm, float* out_x,
                            float* out_store, hipStream_t s, bool wait_xm, hipEvent_t ev_xm) {
  const int l = m / 2;
  StreamScratch& sc = module_scratch(ctx, m);
  ladder_status st;
  if (m % 2 == 0) {
    TRACE(LADDER_KERNEL_QKV, s, false);
    if ((st = run_gemv(ctx, qkv_params(ctx, l, B, xin, sc), s))) return st;
    TRACE(LADDER_KERNEL_QKV, s, true);
    TRACE(LADDER_KERNEL_ATTN, s, false);
    HIPCHK(launch_attn_decode(attn_params(ctx, l, B, sc), s));
    TRACE(LADDER_KERNEL_ATTN, s, true);
  } else {
    TRACE(LADDER_KERNEL_GATEUP, s, false);
    if ((st = run_gemv(ctx, gateup_params(ctx, l, B, xin, sc), s))) return st;
    TRACE(LADDER_KERNEL_GATEUP, s, true);
  }
  if (out_x && wait_xm) HIPCHK(hipStreamWaitEvent(s, ev_xm, 0));
  const int kind = m % 2 == 0 ? LADDER_KERNEL_OPROJ : LADDER_KERNEL_DOWN;
  TRACE(kind, s, false);
  if ((st = run_gemv(ctx, outproj_params(ctx, m, B, sc, xm, out_x, out_store), s))) return st;
  TRACE(kind, s, true);
  return LADDER_OK;
}

// The two launches of a ladder layer under FUSED at row-wave batches: [QKV, then gate/up |
// attention] and [down, then O + both residual adds]; at batch 1 the streaming pair, whose
// back launch also merges the attention's chunk records.  Traced as the kernel kinds
// QKV_ATTN_GATEUP and DOWN_OPROJ.
ladder_status launch_layer_pair(ladder_ctx* ctx, int l, int B, const GemvParams* pr, const GemvParams& down,
                                const GemvParams& o, StreamScratch& sc, hipStream_t s) {
  const bool stream = stream_layers(ctx, B);
  TRACE(LADDER_KERNEL_QKV_ATTN_GATEUP, s, false);
  if (stream)
    HIPCHK(launch_stream_front(pr[0], pr[1], attn_params(ctx, l, B, sc), ctx->qkv_tagged, l + 1, ctx->err_word, s));
  else
    HIPCHK(launch_gemv_seq(pr[0], pr[1], attn_params(ctx, l, B, sc), ctx->seq_prog, l + 1, ctx->err_word, s));
  TRACE(LADDER_KERNEL_QKV_ATTN_GATEUP, s, true);
  TRACE(LADDER_KERNEL_DOWN_OPROJ, s, false);
  if (stream)
    HIPCHK(launch_stream_back(down, o, signalled(ctx, attn_params(ctx, l, B, sc), l), ctx->err_word, s));
  else
    HIPCHK(launch_gemv_paired_nowait(down, o, s));
  TRACE(LADDER_KERNEL_DOWN_OPROJ, s, true);
  return LADDER_OK;
}

// One ladder layer l (or parallel block) of a decode step on one stream, in three launches:
//   [QKV_l | gate/up_l]   the attention reads x_{2l-1} (parallel block: x_{2l}), the MLP
//                         x_{2l}: both exist;
//   [attention_l | down_l] the down projection needs only the SwiGLU output; stores d;
//   [O_l]                 x_{2l+1} = x_{2l} + o, then x_{2l+2} = x_{2l+1} + d.
// The values are those of the module-by-module order (same kernels per row, same adds).
ladder_status decode_layer_fused(ladder_ctx* ctx, int l, int B) {
  const int ma = 2 * l, mm = 2 * l + 1;
  StreamScratch& sc = ctx->sc[0];
  hipStream_t s = ctx->s0;
  float* const* X = ctx->dx;
  ladder_status st;
  GemvParams pr[2] = {qkv_params(ctx, l, B, X[module_src(ctx, ma) % 2], sc),
                      gateup_params(ctx, l, B, X[module_src(ctx, mm) % 2], sc)};
  if (ctx->sched != LADDER_SCHED_FUSED_LATE_ATTN && seq_layers(ctx, B)) {
    // [QKV_l, then gate/up_l, in half of the workgroups, gate/up_l in the others |
    // attention_l once all of QKV_l is done]: the QKV rows come first, so the attention
    // runs while gate/up streams; then [down_l rows | the same O_l rows with x_{2l+1} =
    // x_{2l} + o and x_{2l+2} = x_{2l+1} + d], which waits for nothing
    const GemvParams down = outproj_params(ctx, mm, B, sc, nullptr, nullptr, ctx->dout[0]);
    GemvParams o = outproj_params(ctx, ma, B, sc, X[ma % 2], X[(ma + 1) % 2], nullptr);
    o.epi = EPI_ADD2;
    o.add2 = nullptr;
    o.out2 = X[(ma + 2) % 2];
    return launch_layer_pair(ctx, l, B, pr, down, o, sc, s);
  }
  if (two_launch_layers(ctx, B)) {
    TRACE(LADDER_KERNEL_QKV_GATEUP, s, false);
    HIPCHK(launch_gemv_multi(pr, 2, nullptr, s, nullptr));
    TRACE(LADDER_KERNEL_QKV_GATEUP, s, true);
    // [attention | down rows, then (once the attention has signalled) the same O rows
    // with x_{2l+1} = x_{2l} + o and x_{2l+2} = x_{2l+1} + d]; the O weights are already
    // in flight while the workgroup waits
    const GemvParams down = outproj_params(ctx, mm, B, sc, nullptr, nullptr, ctx->dout[0]);
    GemvParams o = outproj_params(ctx, ma, B, sc, X[ma % 2], X[(ma + 1) % 2], nullptr);
    o.epi = EPI_ADD2;
    o.add2 = nullptr;
    o.out2 = X[(ma + 2) % 2];
    TRACE(LADDER_KERNEL_ATTN_DOWN, s, false);
    HIPCHK(launch_gemv_paired(down, o, signalled(ctx, attn_params(ctx, l, B, sc), l), ctx->err_word, s));
    TRACE(LADDER_KERNEL_ATTN_DOWN, s, true);
    return LADDER_OK;
  }
  const bool rw = gemv_rw_supported(ctx->wdt, ctx->cfg.hidden, B);
  TRACE(LADDER_KERNEL_QKV_GATEUP, s, false);
  if (rw) {
    HIPCHK(launch_gemv_multi(pr, 2, nullptr, s, nullptr));
  } else {
    if ((st = run_gemv(ctx, pr[0], s))) return st;
    if ((st = run_gemv(ctx, pr[1], s))) return st;
  }
  TRACE(LADDER_KERNEL_QKV_GATEUP, s, true);
  const GemvParams down = outproj_params(ctx, mm, B, sc, nullptr, nullptr, ctx->dout[0]);
  const AttnDecodeParams at = attn_params(ctx, l, B, sc);
  TRACE(LADDER_KERNEL_ATTN_DOWN, s, false);
  if (gemv_rw_supported(ctx->wdt, ctx->cfg.ffn, B) && gemv_rw_attn_fusable(ctx->wdt, ctx->cfg.ffn)) {
    HIPCHK(launch_gemv_multi(&down, 1, &at, s, nullptr));
  } else {
    HIPCHK(launch_attn_decode(at, s));
    if ((st = run_gemv(ctx, down, s))) return st;
  }
  TRACE(LADDER_KERNEL_ATTN_DOWN, s, true);
  GemvParams o = outproj_params(ctx, ma, B, sc, X[ma % 2], X[(ma + 1) % 2], nullptr);
  o.epi = EPI_ADD2;
  o.add2 = ctx->dout[0];
  o.out2 = X[(ma + 2) % 2];
  TRACE(LADDER_KERNEL_OPROJ_ADD2, s, false);
  if ((st = run_gemv(ctx, o, s))) return st;
  TRACE(LADDER_KERNEL_OPROJ_ADD2, s, true);
  return LADDER_OK;
}

// ---------------------------------------------------------------- prefill module
ladder_status prefill_module(ladder_ctx* ctx, int m, int B, int T, int start_pos, const float* xin,
                             const float* xm, float* out_x, float* out_store, hipStream_t s, bool wait_xm,
                             hipEvent_t ev_xm) {
  const ladder_config& g = ctx->cfg;
  const int l = m / 2, M = B * T;
  const ladder_layer_weights& L = ctx->layers[l];
  StreamScratch& sc = module_scratch(ctx, m);
  GemmParams gp{};
  gp.wdtype = ctx->wdt;
  gp.M = M;
  gp.ws = sc.gk;
  gp.ws_floats = sc.gk ? kGemmSplitWsFloats : 0;
  gp.cnt = sc.skcnt;
  const void* proj_in;
  int proj_k;
  const void* proj_w;
  // the module's RMSNorm: folded into the projection when it is a split-K launch of a
  // decode step on the matrix cores (A = the raw rows, the reduction divides by the rms),
  // else its own kernel into sc.u
  auto norm_input = [&](const void* gain) -> ladder_status {
    gp.lda = g.hidden;
    if (ctx->gemm_step && ctx->wdt == W_BF16) {
      GemmParams t = gp;
      t.A = xin;
      t.gain = gain;
      t.eps = g.norm_eps;
      if (gemm_norm_fusable(t)) {
        gp = t;
        return LADDER_OK;
      }
    }
    if (ctx->wdt == W_BF16) {
      // A as bf16 pairs, split once here instead of once per column tile of the GEMM
      GemmParams t = gp;
      t.A = sc.u;
      t.a_pairs = 1;
      if (gemm_takes_pairs(t)) {
        HIPCHK(launch_rmsnorm_pairs(xin, g.hidden, gain, g.norm_eps, M, g.hidden, sc.u, s));
        gp = t;
        return LADDER_OK;
      }
    }
    HIPCHK(launch_rmsnorm(ctx->wdt, xin, g.hidden, gain, g.norm_eps, M, g.hidden, sc.u, s));
    gp.A = sc.u;
    return LADDER_OK;
  };
  ladder_status nst;
  if (m % 2 == 0) {
    const int nqkv = ctx->qrows + 2 * ctx->kvrows;
    gp.rows = RowSrc{{L.wq, L.wk, L.wv}, ctx->qrows, ctx->qrows + ctx->kvrows, 0};
    gp.N = nqkv;
    gp.K = g.hidden;
    gp.C = sc.qkv;
    gp.ldc = nqkv;
    if ((nst = norm_input(L.attn_norm))) return nst;
    bool paired = false;
    if (ctx->pair_next && ctx->gemm_step) {
      // with the layer's gate/up projection, RoPE + KV append in the QKV reduction
      GemmParams r = gp;
      r.rope_q = sc.qr;
      r.k_cache = layer_k(ctx, l);
      r.v_cache = layer_v(ctx, l);
      r.rope_cos = ctx->rope_cos;
      r.rope_sin = ctx->rope_sin;
      r.d_pos = ctx->pos_dev;
      r.nq = g.n_q_heads;
      r.nkv = g.n_kv_heads;
      r.hd = g.head_dim;
      r.max_seq = g.max_seq;
      if (gemm_pair_ok(r, ctx->pair_gu)) {
        TRACE(LADDER_KERNEL_QKV_GATEUP, s, false);
        HIPCHK(launch_gemm_pair(r, ctx->pair_gu, s));
        TRACE(LADDER_KERNEL_QKV_GATEUP, s, true);
        ctx->skip_gateup = true;
        paired = true;
      }
    }
    ctx->pair_next = false;
    if (!paired) HIPCHK(launch_gemm(gp, s));
    if (!paired) HIPCHK(launch_rope_kv(ctx->wdt, sc.qkv, B, T, start_pos, ctx->gemm_step ? ctx->pos_dev : nullptr, g.n_q_heads, g.n_kv_heads, g.head_dim, ctx->rope_cos,
                          ctx->rope_sin, sc.qr, layer_k(ctx, l), layer_v(ctx, l), g.max_seq, s));
    if (ctx->gemm_step) {
      // a decode step (one query per sequence at *pos_dev): the split-KV decode attention
      AttnDecodeParams a = attn_params(ctx, l, B, sc);
      // key chunks: the rule of every matrix-core decode path (decode_attn_fill)
      const int fill = decode_attn_fill(B) / (B * g.n_kv_heads);
      a.n_split = std::max(1, std::min(a.n_split, fill));
      a.q = sc.qr;
      a.out = sc.ob;
      if (ctx->skip_gateup && kAttnInOutLaunch) {
        // a paired layer: the attention runs in the [O | down] launch (with its signal)
        ctx->pair_at = signalled(ctx, a, l);
        ctx->at_deferred = true;
      } else {
        HIPCHK(launch_attn_decode(a, s));
      }
    } else {
      AttnPrefillParams ap{};
      ap.wdtype = ctx->wdt;
      ap.q = sc.qr;
      ap.k_cache = layer_k(ctx, l);
      ap.v_cache = layer_v(ctx, l);
      ap.max_seq = g.max_seq;
      ap.nq = g.n_q_heads;
      ap.nkv = g.n_kv_heads;
      ap.hd = g.head_dim;
      ap.B = B;
      ap.T = T;
      ap.start_pos = start_pos;
      ap.out = sc.ob;
      ap.part = sc.apart;
      ap.part_floats = sc.apart ? attn_prefill_part_floats(g.head_dim) : 0;
      HIPCHK(launch_attn_prefill(ap, s));
    }
    proj_in = sc.ob;
    proj_k = ctx->qrows;
    proj_w = L.wo;
  } else {
    gp.rows = RowSrc{{L.w_gate, L.w_up, nullptr}, 0, 0, 1};
    gp.N = 2 * g.ffn;
    gp.K = g.hidden;
    if (ctx->wdt == W_BF16) gp.swiglu = 1;
    if ((nst = norm_input(L.mlp_norm))) return nst;
    if (ctx->wdt == W_BF16) {               // SwiGLU in the GEMM epilogue
      gp.swiglu = 1;
      gp.C = sc.ab;
      gp.ldc = g.ffn;
      // its output as bf16 pairs where the down projection takes them (prefill)
      GemmParams d{};
      d.wdtype = ctx->wdt;
      d.M = M;
      d.N = g.hidden;
      d.K = g.ffn;
      d.lda = g.ffn;
      gp.c_pairs = gemm_writes_pairs(gp) && gemm_takes_pairs(d);
      if (ctx->skip_gateup) {
        ctx->skip_gateup = false;           // run with the layer's QKV projection
      } else {
        if (T == 1) TRACE(LADDER_KERNEL_GATEUP, s, false);   // a decode step on the matrix cores
        HIPCHK(launch_gemm(gp, s));
        if (T == 1) TRACE(LADDER_KERNEL_GATEUP, s, true);
      }
    } else {
      gp.C = sc.gu;
      gp.ldc = 2 * g.ffn;
      HIPCHK(launch_gemm(gp, s));
      HIPCHK(launch_swiglu(sc.gu, M, g.ffn, sc.ab, s));
    }
    proj_in = sc.ab;
    proj_k = g.ffn;
    proj_w = L.w_down;
  }
  GemmParams op{};
  op.wdtype = ctx->wdt;
  op.ws = sc.gk;
  op.ws_floats = sc.gk ? kGemmSplitWsFloats : 0;
  op.cnt = sc.skcnt;
  op.A = proj_in;
  op.a_pairs = proj_in == sc.ab && gp.c_pairs;
  op.lda = proj_k;
  op.rows = RowSrc{{proj_w, nullptr, nullptr}, g.hidden, g.hidden, 0};
  op.M = M;
  op.N = g.hidden;
  op.K = proj_k;
  op.ldc = g.hidden;
  if (out_x) {
    if (wait_xm) HIPCHK(hipStreamWaitEvent(s, ev_xm, 0));
    op.C = out_x;
    op.res = xm;
    op.ldr = g.hidden;
  } else {
    op.C = out_store;
  }
  if (m % 2 == 0 && ctx->skip_gateup && ctx->gemm_step && out_x && !wait_xm) {
    // a paired layer's O projection waits for the down projection: one launch of both,
    // and one reduction writing x_{2l+1} = x_{2l} + o and x_{2l+2} = x_{2l+1} + d
    ctx->pair_o = op;
    ctx->o_deferred = true;
    return LADDER_OK;
  }
  if (m % 2 == 0 && ctx->at_deferred) {      // (not taken: the O projection needs it now)
    ctx->at_deferred = false;
    HIPCHK(launch_attn_decode(ctx->pair_at, s));
  }
  if (m % 2 == 1 && ctx->o_deferred) {
    ctx->o_deferred = false;
    GemmParams d = op;
    d.ws = ctx->sc[1].gk;             // the O partials take the first workspace
    d.cnt = ctx->sc[1].skcnt;
    if (ctx->at_deferred) {
      ctx->at_deferred = false;
      if (gemm_attn_chain_ok(ctx->pair_at, ctx->pair_o, d)) {
        TRACE(LADDER_KERNEL_DOWN_OPROJ, s, false);
        HIPCHK(launch_gemm_attn_chain(ctx->pair_at, ctx->pair_o, d, ctx->err_word, s));
        TRACE(LADDER_KERNEL_DOWN_OPROJ, s, true);
        return LADDER_OK;
      }
      HIPCHK(launch_attn_decode(ctx->pair_at, s));
    }
    if (gemm_chain_ok(ctx->pair_o, d)) {
      TRACE(LADDER_KERNEL_DOWN_OPROJ, s, false);
      HIPCHK(launch_gemm_chain(ctx->pair_o, d, s));
      TRACE(LADDER_KERNEL_DOWN_OPROJ, s, true);
      return LADDER_OK;
    }
    HIPCHK(launch_gemm(ctx->pair_o, s));
  }
  HIPCHK(launch_gemm(op, s));
  return LADDER_OK;
}

// Enqueue the module loop on the context's streams, starting from x_0 in X[0] and
// finishing with x_{2L} in X[(2L) % 2] and every stream joined into s0.
//
// Ordering (two residual slots: x_j lives in X[j % 2]):
//   SERIAL - program order on s0.
//   SIDE   - module m (s0) waits ev_x[src] recorded by the add that produced x_src; the
//            add m (side) waits ev_out[m], i.e. module m is complete, which also means
//            every earlier reader of X[(m+1) % 2] (module m's own input x_{m-1}, the add
//            m-1) is done before x_{m+1} overwrites it.  out_m alternates two buffers;
//            module m+2 overwrites OUT[m % 2] only after waiting for an input produced by
//            add m or later.
//   DUAL   - module m runs on stream m % 2.  Its input x_src was produced by module
//            src-1: on the same stream for a ladder module, else waited for via
//            ev_x[src].  Its output projection adds x_m, produced by module m-1 on the
//            other stream, so it waits for ev_x[m] first; that wait also orders the
//            overwrite of X[(m+1) % 2] (x_{m-1}) after module m-1's last read of it.
template <typename ModuleFn>
ladder_status run_modules(ladder_ctx* ctx, float* const X[2], float* const OUT[2], size_t add_elems,
                          ModuleFn&& module, bool fused_adds = false) {
  const int NM = 2 * ctx->cfg.n_layers;
  const int sched = ctx->sched;
  if (sched == LADDER_SCHED_DUAL) {
    HIPCHK(hipEventRecord(ctx->ev_fork, ctx->s0));
    HIPCHK(hipStreamWaitEvent(ctx->sb, ctx->ev_fork, 0));
  }
  for (int m = 0; m < NM; ++m) {
    const int src = module_src(ctx, m);
    const float* xin = X[src % 2];
    const float* xm = X[m % 2];
    float* xn = X[(m + 1) % 2];
    hipStream_t s = module_stream(ctx, m);
    ladder_status st;
    if (sched == LADDER_SCHED_SERIAL && fused_adds) {
      // module order, each output added by the producing kernel (the module has
      // consumed its input before it writes x_{m+1}, which may share its buffer)
      st = module(m, xin, xm, xn, nullptr, s, false, nullptr);
      if (st) return st;
    } else if (sched == LADDER_SCHED_SERIAL) {
      st = module(m, xin, xm, nullptr, OUT[m % 2], s, false, nullptr);
      if (st) return st;
      HIPCHK(launch_add(xm, OUT[m % 2], xn, add_elems, s));
    } else if (sched == LADDER_SCHED_SIDE) {
      if (src > 0) HIPCHK(hipStreamWaitEvent(s, ctx->ev_x[src], 0));
      st = module(m, xin, xm, nullptr, OUT[m % 2], s, false, nullptr);
      if (st) return st;
      HIPCHK(hipEventRecord(ctx->ev_out[m], s));
      HIPCHK(hipStreamWaitEvent(ctx->side, ctx->ev_out[m], 0));
      HIPCHK(launch_add(xm, OUT[m % 2], xn, add_elems, ctx->side));
      HIPCHK(hipEventRecord(ctx->ev_x[m + 1], ctx->side));
    } else {
      // producer of x_j (j >= 1) is module j-1, on stream (j-1) % 2; x_0 precedes the fork
      const bool src_other = src > 0 && ((src - 1) % 2) != (m % 2);
      if (src_other) HIPCHK(hipStreamWaitEvent(s, ctx->ev_x[src], 0));
      const bool xm_other = m > 0 && ((m - 1) % 2) != (m % 2) && !(src_other && src == m);
      st = module(m, xin, xm, xn, nullptr, s, xm_other, m > 0 ? ctx->ev_x[m] : nullptr);
      if (st) return st;
      HIPCHK(hipEventRecord(ctx->ev_x[m + 1], s));
    }
  }
  if (sched == LADDER_SCHED_SIDE) {
    HIPCHK(hipStreamWaitEvent(ctx->s0, ctx->ev_x[NM], 0));
  } else if (sched == LADDER_SCHED_DUAL) {
    HIPCHK(hipStreamWaitEvent(ctx->s0, ctx->ev_x[NM], 0));       // last MLP (stream B)
  }
  return LADDER_OK;
}

// The persistent decode step: every layer ladder, bf16, batch <= 4, all workgroups resident.
StepParams step_params(const ladder_ctx* ctx, int B);

bool step_usable(const ladder_ctx* ctx, int B) {
  const ladder_config& g = ctx->cfg;
  return ctx->all_ladder && ctx->step_x && B <= 4 &&
         step_supported(ctx->wdt, g.hidden, g.ffn, ctx->qrows, B, g.head_dim, g.n_q_heads / g.n_kv_heads) &&
         step_fits(step_params(ctx, B));
}

StepParams step_params(const ladder_ctx* ctx, int B) {
  const ladder_config& g = ctx->cfg;
  const StreamScratch& sc = ctx->sc[0];
  StepParams sp{};
  sp.layers = ctx->step_layers;
  sp.L = g.n_layers;
  sp.H = g.hidden;
  sp.F = g.ffn;
  sp.nq = g.n_q_heads;
  sp.nkv = g.n_kv_heads;
  sp.hd = g.head_dim;
  sp.B = B;
  sp.max_seq = g.max_seq;
  sp.eps = g.norm_eps;
  sp.rope_cos = ctx->rope_cos;
  sp.rope_sin = ctx->rope_sin;
  sp.d_pos = ctx->pos_dev;
  sp.d_epoch = ctx->epoch;
  sp.x0 = ctx->dx[0];
  sp.xs = ctx->step_x;
  sp.xstride = ctx->step_xstride;
  sp.qs = ctx->step_q;
  sp.os = ctx->step_o;
  sp.qstride = ctx->step_qstride;
  sp.as = ctx->step_a;
  sp.astride = ctx->step_astride;
  sp.part = sc.attn_part;
  sp.attn_cnt = sc.attn_cnt;
  sp.n_split = ctx->n_split;
  sp.sync = ctx->step_sync;
  sp.prog = ctx->step_prog;
  sp.err = ctx->err_word;
  return sp;
}

// The draw that replaces the greedy token when sampling is on: position *d_pos (decode,
// read when the kernel runs) or pos (prefill).
SampleParams sample_params(const ladder_ctx* ctx, int B, const int* d_pos, int pos) {
  SampleParams sp{};
  sp.logits = ctx->logits;
  sp.ldl = ctx->cfg.vocab;
  sp.V = ctx->cfg.vocab;
  sp.B = B;
  sp.temperature = ctx->temperature > 0.f ? ctx->temperature : 1.f;
  sp.top_k = ctx->top_k;
  sp.seed_lo = (uint32_t)(ctx->seed & 0xffffffffu);
  sp.seed_hi = (uint32_t)(ctx->seed >> 32);
  sp.d_pos = d_pos;
  sp.pos = pos;
  sp.next = ctx->next;
  return sp;
}

bool gemm_decode(const ladder_ctx* ctx, int B);

ladder_status lm_head_mc(ladder_ctx* ctx, const float* x, int ldx, int B, hipStream_t s);

// Final RMSNorm + LM head + greedy token; with sampling on, the draw then overwrites the
// token (the logits are the same either way).  Batches the row-wave GEMV cannot take (bf16)
// run the LM head on the matrix cores (lm_head_mc).
ladder_status lm_head(ladder_ctx* ctx, const float* x, int ldx, int B, hipStream_t s, const int* d_pos, int pos) {
  if (gemm_decode(ctx, B)) {
    ladder_status st = lm_head_mc(ctx, x, ldx, B, s);
    if (st) return st;
  } else {
    ladder_status st = run_gemv(ctx, lmhead_params(ctx, x, ldx, B), s);
    if (st) return st;
  }
  if (ctx->temperature > 0.f) {
    TRACE(LADDER_KERNEL_SAMPLE, s, false);
    HIPCHK(launch_sample(sample_params(ctx, B, d_pos, pos), s));
    TRACE(LADDER_KERNEL_SAMPLE, s, true);
  }
  return LADDER_OK;
}

// The LM head of the matrix-core route: the GEMM (the final RMSNorm folded into the skinny
// launch where it takes the LM head, A = the raw rows, else its own kernel) and a row argmax.
ladder_status lm_head_mc(ladder_ctx* ctx, const float* x, int ldx, int B, hipStream_t s) {
  const ladder_config& g = ctx->cfg;
  StreamScratch& sc = ctx->sc[0];
  GemmParams hp{};
  hp.wdtype = ctx->wdt;
  // the final RMSNorm folded into the skinny launch where it takes the LM head (A = the
  // raw rows), else its own kernel
  hp.A = x;
  hp.lda = ldx;
  hp.rows = RowSrc{{ctx->w.lm_head, nullptr, nullptr}, g.vocab, g.vocab, 0};
  hp.M = B;
  hp.N = g.vocab;
  hp.K = g.hidden;
  hp.C = ctx->logits;
  hp.ldc = g.vocab;
  hp.ws = sc.gk;
  hp.ws_floats = sc.gk ? kGemmSplitWsFloats : 0;
  hp.cnt = sc.skcnt;
  hp.gain = ctx->w.final_norm;
  hp.eps = g.norm_eps;
  if (!skinny_supported(hp)) {
    HIPCHK(launch_rmsnorm(ctx->wdt, x, ldx, ctx->w.final_norm, g.norm_eps, B, g.hidden, sc.u, s));
    hp.A = sc.u;
    hp.lda = g.hidden;
    hp.gain = nullptr;
  }
  HIPCHK(launch_gemm(hp, s));
  HIPCHK(launch_argmax_rows(ctx->logits, B, g.vocab, g.vocab, ctx->next, s));
  return LADDER_OK;
}

// One decode step from the embeddings the prologue left in dx[0] and pos_dev, leaving
// logits/next in the context and x_{2L} in dx[(2L) % 2].  Enqueued on s0 (possibly under
// graph capture).
bool gemm_decode(const ladder_ctx* ctx, int B);
ladder_status enqueue_decode_gemm(ladder_ctx* ctx, int B);

ladder_status enqueue_decode(ladder_ctx* ctx, int B) {
  if (gemm_decode(ctx, B)) return enqueue_decode_gemm(ctx, B);
  const ladder_config& g = ctx->cfg;
  ctx->trace_n = 0;
  ladder_status st;
  if (ctx->sched == LADDER_SCHED_PERSISTENT && step_usable(ctx, B)) {
    TRACE(LADDER_KERNEL_LAYER_STACK, ctx->s0, false);
    HIPCHK(launch_decode_step(step_params(ctx, B), ctx->s0));
    TRACE(LADDER_KERNEL_LAYER_STACK, ctx->s0, true);
  } else if (ctx->sched >= LADDER_SCHED_FUSED) {
    // ladder and parallel layers (both modules' inputs exist before the layer starts) in
    // two or three launches; standard layers module by module (fused adds)
    for (int l = 0; l < g.n_layers; ++l) {
      if (ctx->mask[l]) {
        if ((st = decode_layer_fused(ctx, l, B))) return st;
      } else {
        for (int m = 2 * l; m < 2 * l + 2; ++m) {
          st = decode_module(ctx, m, B, ctx->dx[module_src(ctx, m) % 2], ctx->dx[m % 2], ctx->dx[(m + 1) % 2],
                             nullptr, ctx->s0, false, nullptr);
          if (st) return st;
        }
      }
    }
  } else {
    auto mod = [&](int m, const float* xin, const float* xm, float* xn, float* store, hipStream_t s, bool wait,
                   hipEvent_t ev) { return decode_module(ctx, m, B, xin, xm, xn, store, s, wait, ev); };
    st = run_modules(ctx, ctx->dx, ctx->dout, (size_t)B * g.hidden, mod);
    if (st) return st;
  }
  TRACE(LADDER_KERNEL_LMHEAD, ctx->s0, false);
  if ((st = lm_head(ctx, ctx->dx[(2 * g.n_layers) % 2], g.hidden, B, ctx->s0, ctx->pos_dev, 0))) return st;
  TRACE(LADDER_KERNEL_LMHEAD, ctx->s0, true);
  ctx->trace_count = ctx->trace_n;
  return LADDER_OK;
}

// Decode steps that the row-wave projections cannot take (bf16 weights, batch > 4, or the
// staged input rows of any projection, the widest of hidden, ffn and the attention rows,
// beyond their LDS budget): one token per sequence on the matrix cores (the K-sliced GEMV
// kernels leave most of the HBM bandwidth unused at those batches), through the skinny
// projections up to 32 sequences (a ladder layer in two launches, decode_layer_skinny;
// standard layers module by module) and the tiled GEMMs beyond, with the split-KV decode
// attention, then the LM head with the final RMSNorm folded in and a row argmax.  Every
// kernel of the route takes the position from the device (the prologue's pos_dev), so it
// is replayed as a graph too.  Batches 3 and 4 also take it where the row-wave launches
// would hold one workgroup per CU (the 70B shard at batch 3: 498 against 335 tok/s; the 1B
// model at batch 3: 2290 against 2065), and batch 2 for wide models whose layers are all
// ladder or parallel blocks (70B shard: 394 against 378 tok/s; the 8B hybrid, half of its
// layers standard, stays on the row-wave launches: 459 against 429).
bool gemm_decode(const ladder_ctx* ctx, int B) {
  const int kmax = std::max(ctx->cfg.hidden, std::max(ctx->cfg.ffn, ctx->qrows));
  if (ctx->wdt != W_BF16) return false;
  bool no_standard = true;
  for (int l = 0; l < ctx->cfg.n_layers; ++l) no_standard = no_standard && ctx->mask[l] != 0;
  return !gemv_rw_supported(ctx->wdt, kmax, B) || (B >= 3 && !gemv_rw_two_per_cu(ctx->wdt, kmax, B)) ||
         (B == 2 && no_standard && ctx->cfg.hidden >= 8192);
}

// The skinny parameters of a decode step's projections on the matrix cores, as the
// module path (prefill_module with the RMSNorm folded in) builds them.
GemmParams skinny_base(const ladder_ctx* ctx, int B, const StreamScratch& sc) {
  GemmParams p{};
  p.wdtype = ctx->wdt;
  p.M = B;
  p.ws = sc.gk;
  p.ws_floats = kGemmSplitWsFloats;
  p.cnt = sc.skcnt;
  return p;
}

// A ladder layer (or parallel block) of a decode step on the matrix cores in two launches:
// [QKV with RoPE + KV append in its epilogue | split-KV attention once the QKV tiles are
// done | gate/up] (both RMSNorms folded in; by the ladder rule both inputs exist when the
// layer starts; a separate attention launch where the shapes do not allow the fused one),
// and [O + down] with both residual adds, x_{2l+1} = x_{2l} + o and x_{2l+2} = x_{2l+1} + d.
// Each projection is sliced as in its own launch and the epilogue repeats rope_kv's
// arithmetic, so the layer gives the module path's bits.  qg: the [QKV | gate/up] pair (the
// second with the workspace and tickets after the first's); od: [O + down] over the
// attention and SwiGLU outputs.
void skinny_layer_params(const ladder_ctx* ctx, int l, int B, GemmParams qg[2], GemmParams* od) {
  const ladder_config& g = ctx->cfg;
  const ladder_layer_weights& L = ctx->layers[l];
  const StreamScratch& sc = ctx->sc[0];
  float* const* X = ctx->dx;
  const int nqkv = ctx->qrows + 2 * ctx->kvrows;
  GemmParams& a = qg[0];
  GemmParams& b = qg[1];
  a = skinny_base(ctx, B, sc);
  b = a;
  *od = a;
  a.A = X[module_src(ctx, 2 * l) % 2];
  a.lda = g.hidden;
  a.gain = L.attn_norm;
  a.eps = g.norm_eps;
  a.rows = RowSrc{{L.wq, L.wk, L.wv}, ctx->qrows, ctx->qrows + ctx->kvrows, 0};
  a.N = nqkv;
  a.K = g.hidden;
  a.C = sc.qkv;
  a.ldc = nqkv;
  // RoPE + KV append in the QKV epilogue (rope_kv's arithmetic): q into sc.qr
  a.rope_q = sc.qr;
  a.k_cache = layer_k(ctx, l);
  a.v_cache = layer_v(ctx, l);
  a.rope_cos = ctx->rope_cos;
  a.rope_sin = ctx->rope_sin;
  a.d_pos = ctx->pos_dev;
  a.nq = g.n_q_heads;
  a.nkv = g.n_kv_heads;
  a.hd = g.head_dim;
  a.max_seq = g.max_seq;
  b.A = X[module_src(ctx, 2 * l + 1) % 2];
  b.lda = g.hidden;
  b.gain = L.mlp_norm;
  b.eps = g.norm_eps;
  b.rows = RowSrc{{L.w_gate, L.w_up, nullptr}, 0, 0, 1};
  b.N = 2 * g.ffn;
  b.K = g.hidden;
  b.swiglu = 1;
  b.C = sc.ab;
  b.ldc = g.ffn;
  const size_t na = align_up(skinny_ws_floats(a), 64);
  b.ws = sc.gk + std::min(na, kGemmSplitWsFloats);
  b.ws_floats = kGemmSplitWsFloats - std::min(na, kGemmSplitWsFloats);
  b.cnt = sc.skcnt + (nqkv + 127) / 128;
  GemmParams& o = *od;
  o.A = sc.ob;
  o.lda = ctx->qrows;
  o.rows = RowSrc{{L.wo, nullptr, nullptr}, g.hidden, g.hidden, 0};
  o.N = g.hidden;
  o.K = ctx->qrows;
  o.res = X[(2 * l) % 2];
  o.ldr = g.hidden;
  o.C = X[(2 * l + 1) % 2];
  o.ldc = g.hidden;
  o.A2 = sc.ab;
  o.lda2 = g.ffn;
  o.rows2 = RowSrc{{L.w_down, nullptr, nullptr}, g.hidden, g.hidden, 0};
  o.K2 = g.ffn;
  o.C2 = X[(2 * l + 2) % 2];
}

bool skinny_layer_ok(const ladder_ctx* ctx, int B) {
  const StreamScratch& sc = ctx->sc[0];
  if (ctx->wdt != W_BF16 || !sc.gk || !sc.skcnt) return false;
  GemmParams qg[2], od;
  skinny_layer_params(ctx, 0, B, qg, &od);
  const int tiles = (qg[0].N + 127) / 128 + (qg[1].N + 127) / 128;
  return tiles <= kSkinnyMaxTiles && skinny_pair_supported(qg[0], qg[1]) && skinny_supported(od);
}

ladder_status decode_layer_skinny(ladder_ctx* ctx, int l, int B, hipStream_t s) {
  const ladder_config& g = ctx->cfg;
  StreamScratch& sc = ctx->sc[0];
  GemmParams qg[2], od;
  skinny_layer_params(ctx, l, B, qg, &od);
  AttnDecodeParams at = attn_params(ctx, l, B, sc);
  at.n_split = std::max(1, std::min(at.n_split, decode_attn_fill(B) / (B * g.n_kv_heads)));
  at.q = sc.qr;
  at.out = sc.ob;
  if (skinny_pair_attn_supported(qg[0], qg[1], at)) {
    // the attention waits for the QKV tiles inside the same launch, beside the gate/up rows
    TRACE(LADDER_KERNEL_QKV_ATTN_GATEUP, s, false);
    HIPCHK(launch_skinny_pair_attn(qg[0], qg[1], at, ctx->seq_prog, l + 1, ctx->err_word, s));
    TRACE(LADDER_KERNEL_QKV_ATTN_GATEUP, s, true);
  } else {
    TRACE(LADDER_KERNEL_QKV_GATEUP, s, false);
    HIPCHK(launch_skinny_pair(qg[0], qg[1], s));
    TRACE(LADDER_KERNEL_QKV_GATEUP, s, true);
    HIPCHK(launch_attn_decode(at, s));
  }
  TRACE(LADDER_KERNEL_DOWN_OPROJ, s, false);
  HIPCHK(launch_skinny(od, s));
  TRACE(LADDER_KERNEL_DOWN_OPROJ, s, true);
  return LADDER_OK;
}

// The gate/up projection of layer l's MLP module in a decode step on the matrix cores, as
// prefill_module builds it (RMSNorm folded in), with its split-K partials in the second
// stream scratch's workspace (the QKV launch beside it uses the first's); false where the
// fold does not apply (the module then runs it alone).
bool gateup_pair_params(ladder_ctx* ctx, int l, int B, const float* xin, GemmParams* out) {
  const ladder_config& g = ctx->cfg;
  const ladder_layer_weights& L = ctx->layers[l];
  if (ctx->wdt != W_BF16 || !ctx->sc[1].gk) return false;
  GemmParams t{};
  t.wdtype = ctx->wdt;
  t.M = B;
  t.ws = ctx->sc[1].gk;
  t.ws_floats = kGemmSplitWsFloats;
  t.cnt = ctx->sc[1].skcnt;
  t.rows = RowSrc{{L.w_gate, L.w_up, nullptr}, 0, 0, 1};
  t.N = 2 * g.ffn;
  t.K = g.hidden;
  t.swiglu = 1;
  t.lda = g.hidden;
  t.A = xin;
  t.gain = L.mlp_norm;
  t.eps = g.norm_eps;
  t.C = module_scratch(ctx, 2 * l + 1).ab;
  t.ldc = g.ffn;
  if (!gemm_norm_fusable(t)) return false;
  *out = t;
  return true;
}

ladder_status enqueue_decode_gemm(ladder_ctx* ctx, int B) {
  const int pos = 0;   // unused: every kernel reads the position from pos_dev
  const ladder_config& g = ctx->cfg;
  ctx->trace_n = 0;
  const int saved = ctx->sched;
  const bool fused = saved >= LADDER_SCHED_FUSED;
  if (fused) ctx->sched = LADDER_SCHED_SERIAL;   // module order, adds in the GEMM epilogues
  auto mod = [&](int m, const float* xin, const float* xm, float* xn, float* store, hipStream_t s, bool wait,
                 hipEvent_t ev) { return prefill_module(ctx, m, B, 1, pos, xin, xm, xn, store, s, wait, ev); };
  ctx->gemm_step = true;
  ladder_status st = LADDER_OK;
  if (fused && skinny_layer_ok(ctx, B)) {
    // ladder and parallel layers in four launches each, standard layers module by module
    float* const* X = ctx->dx;
    for (int l = 0; l < g.n_layers && !st; ++l) {
      if (ctx->mask[l]) {
        st = decode_layer_skinny(ctx, l, B, ctx->s0);
      } else {
        for (int m = 2 * l; m < 2 * l + 2 && !st; ++m)
          st = mod(m, X[module_src(ctx, m) % 2], X[m % 2], X[(m + 1) % 2], nullptr, ctx->s0, false, nullptr);
      }
    }
  } else if (fused) {
    // module order (the adds in the GEMM epilogues); a ladder or parallel layer's gate/up
    // projection (its input exists when the layer starts) shares the QKV launch
    float* const* X = ctx->dx;
    for (int l = 0; l < g.n_layers && !st; ++l) {
      if (ctx->mask[l]) ctx->pair_next = gateup_pair_params(ctx, l, B, X[module_src(ctx, 2 * l + 1) % 2], &ctx->pair_gu);
      for (int m = 2 * l; m < 2 * l + 2 && !st; ++m)
        st = mod(m, X[module_src(ctx, m) % 2], X[m % 2], X[(m + 1) % 2], nullptr, ctx->s0, false, nullptr);
      ctx->pair_next = ctx->skip_gateup = false;
      if (ctx->at_deferred) {               // (not taken: the MLP module launches these)
        ctx->at_deferred = false;
        HIPCHK(launch_attn_decode(ctx->pair_at, ctx->s0));
      }
      if (ctx->o_deferred) {
        ctx->o_deferred = false;
        HIPCHK(launch_gemm(ctx->pair_o, ctx->s0));
      }
    }
  } else {
    st = run_modules(ctx, ctx->dx, ctx->dout, (size_t)B * g.hidden, mod, fused);
  }
  ctx->gemm_step = false;
  ctx->sched = saved;
  if (st) return st;
  TRACE(LADDER_KERNEL_LMHEAD, ctx->s0, false);
  if ((st = lm_head(ctx, ctx->dx[(2 * g.n_layers) % 2], g.hidden, B, ctx->s0, ctx->pos_dev, 0))) return st;
  TRACE(LADDER_KERNEL_LMHEAD, ctx->s0, true);
  ctx->trace_count = ctx->trace_n;
  return LADDER_OK;
}

ladder_status begin_call(ladder_ctx* ctx) {
  HIPCHK(hipSetDevice(ctx->dev));
  HIPCHK(hipEventRecord(ctx->ev_in, ctx->user));
  HIPCHK(hipStreamWaitEvent(ctx->s0, ctx->ev_in, 0));
  return LADDER_OK;
}

ladder_status end_call(ladder_ctx* ctx) {
  HIPCHK(hipEventRecord(ctx->ev_done, ctx->s0));
  HIPCHK(hipStreamWaitEvent(ctx->user, ctx->ev_done, 0));
  return LADDER_OK;
}

ladder_status copy_outputs(ladder_ctx* ctx, int B, const float* x_last, size_t x_pitch, float* d_logits,
                           int32_t* d_next, float* d_hidden) {
  const ladder_config& g = ctx->cfg;
  if (d_logits)
    HIPCHK(hipMemcpyAsync(d_logits, ctx->logits, (size_t)B * g.vocab * 4, hipMemcpyDeviceToDevice, ctx->s0));
  if (d_next) HIPCHK(hipMemcpyAsync(d_next, ctx->next, (size_t)B * 4, hipMemcpyDeviceToDevice, ctx->s0));
  if (d_hidden)
    HIPCHK(hipMemcpy2DAsync(d_hidden, (size_t)g.hidden * 4, x_last, x_pitch, (size_t)g.hidden * 4, B,
                            hipMemcpyDeviceToDevice, ctx->s0));
  return LADDER_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

const char* ladder_status_string(ladder_status s) {
  switch (s) {
    case LADDER_OK: return "ok";
    case LADDER_ERR_ARG: return "invalid argument";
    case LADDER_ERR_SHAPE: return "unsupported shape";
    case LADDER_ERR_CAPACITY: return "capacity exceeded (batch or sequence length)";
    case LADDER_ERR_STATE: return "KV positions read before they were written";
    case LADDER_ERR_HIP: return "HIP runtime error";
    case LADDER_ERR_OOM: return "out of device memory";
    default: return "unknown status";
  }
}

const char* ladder_last_error(const ladder_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

void ladder_free(ladder_ctx* ctx) {
  if (!ctx) return;
  (void)hipSetDevice(ctx->dev);
  if (ctx->s0) (void)hipStreamSynchronize(ctx->s0);
  for (auto& kv : ctx->graphs) (void)hipGraphExecDestroy(kv.second);
  for (hipEvent_t e : ctx->ev_x) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : ctx->ev_out) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : {ctx->ev_fork, ctx->ev_in, ctx->ev_done}) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : ctx->trace_ev) if (e) (void)hipEventDestroy(e);
  for (hipStream_t s : {ctx->sb, ctx->side}) {
    if (s) { (void)hipStreamSynchronize(s); (void)hipStreamDestroy(s); }
  }
  if (ctx->s0) (void)hipStreamDestroy(ctx->s0);
  if (ctx->ws) (void)hipFree(ctx->ws);
  delete ctx;
}

ladder_status ladder_init(const ladder_config* cfg, const ladder_weights* w, const ladder_kv* kv, void* stream,
                          ladder_ctx** out) {
  if (!out) return LADDER_ERR_ARG;
  *out = nullptr;
  ladder_status v = validate(cfg, w, kv);
  if (v != LADDER_OK) return v;
  ladder_ctx* ctx = new ladder_ctx();
  ctx->cfg = *cfg;
  ctx->mask.assign(cfg->ladder_mask, cfg->ladder_mask + cfg->n_layers);
  ctx->cfg.ladder_mask = ctx->mask.data();
  ctx->layers.assign(w->layers, w->layers + cfg->n_layers);
  ctx->w = *w;
  ctx->w.layers = ctx->layers.data();
  ctx->kv = *kv;
  ctx->wdt = cfg->dtype == LADDER_BF16 ? W_BF16 : W_F32;
  ctx->esz = cfg->dtype == LADDER_BF16 ? 2 : 4;
  ctx->qrows = cfg->n_q_heads * cfg->head_dim;
  ctx->kvrows = cfg->n_kv_heads * cfg->head_dim;
  ctx->n_split = attn_decode_splits(cfg->max_seq);
  ctx->layer_kv_elems = (size_t)cfg->max_batch * cfg->n_kv_heads * cfg->max_seq * cfg->head_dim;
  {
    long long mm = cfg->max_prefill_tokens > 0 ? cfg->max_prefill_tokens : 8192;
    const long long cap = (long long)cfg->max_batch * cfg->max_seq;
    if (mm > cap) mm = cap;
    if (mm < cfg->max_batch) mm = cfg->max_batch;
    ctx->mmax = (int)mm;
  }
  ctx->filled = cfg->kv_filled;
  ctx->user = (hipStream_t)stream;

  auto bail = [&](ladder_status s) {
    ladder_free(ctx);
    return s;
  };
  hipError_t e = hipGetDevice(&ctx->dev);
  if (e != hipSuccess) { fail(ctx, LADDER_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e)); return bail(LADDER_ERR_HIP); }
#define INITCHK(call)                                                            \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) return bail(e_ == hipErrorOutOfMemory ? LADDER_ERR_OOM : LADDER_ERR_HIP); \
  } while (0)
  // the device address of this GPU's static scratch (ladder_decode_step_static); a failed
  // lookup is kept and reported by that entry point, the context itself does not need it
  (void)static_scratch_setup(ctx->dev);
  INITCHK(hipStreamCreateWithFlags(&ctx->s0, hipStreamNonBlocking));
  INITCHK(hipStreamCreateWithFlags(&ctx->sb, hipStreamNonBlocking));
  INITCHK(hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking));
  const int NM = 2 * cfg->n_layers;
  ctx->ev_x.assign(NM + 1, nullptr);
  ctx->ev_out.assign(NM, nullptr);
  for (auto& ev : ctx->ev_x) INITCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  for (auto& ev : ctx->ev_out) INITCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  INITCHK(hipEventCreateWithFlags(&ctx->ev_fork, hipEventDisableTiming));
  INITCHK(hipEventCreateWithFlags(&ctx->ev_in, hipEventDisableTiming));
  INITCHK(hipEventCreateWithFlags(&ctx->ev_done, hipEventDisableTiming));

  ctx->all_ladder = true;
  for (int l = 0; l < cfg->n_layers; ++l) ctx->all_ladder = ctx->all_ladder && ctx->mask[l] == 1;
  Carver measure;
  carve(ctx, measure);
  ctx->ws_bytes = measure.off;
  INITCHK(hipMalloc((void**)&ctx->ws, ctx->ws_bytes));
  Carver real;
  real.base = ctx->ws;
  carve(ctx, real);
  INITCHK(hipMemsetAsync(ctx->ws, 0, ctx->ws_bytes, ctx->s0));
  {
    std::vector<StepLayer> sl(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers; ++l) {
      const ladder_layer_weights& L = ctx->layers[l];
      sl[l] = StepLayer{L.wq, L.wk, L.wv, L.wo, L.w_gate, L.w_up, L.w_down, L.attn_norm, L.mlp_norm,
                        layer_k(ctx, l), layer_v(ctx, l)};
    }
    INITCHK(hipMemcpyAsync(ctx->step_layers, sl.data(), sl.size() * sizeof(StepLayer), hipMemcpyHostToDevice,
                           ctx->s0));
    INITCHK(hipStreamSynchronize(ctx->s0));
  }

  // RoPE table: pair j at position p rotates by p * rope_frequency(j), computed in fp64
  {
    const int half = cfg->head_dim / 2;
    std::vector<float> cs((size_t)cfg->max_seq * half), sn((size_t)cfg->max_seq * half);
    for (int j = 0; j < half; ++j) {
      const double inv_freq = rope_frequency(*cfg, j);
      for (int p = 0; p < cfg->max_seq; ++p) {
        const double a = (double)p * inv_freq;
        cs[(size_t)p * half + j] = (float)std::cos(a);
        sn[(size_t)p * half + j] = (float)std::sin(a);
      }
    }
    INITCHK(hipMemcpyAsync(ctx->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, ctx->s0));
    INITCHK(hipMemcpyAsync(ctx->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, ctx->s0));
    INITCHK(hipStreamSynchronize(ctx->s0));
  }
#undef INITCHK
  *out = ctx;
  return LADDER_OK;
}

ladder_status ladder_set_schedule(ladder_ctx* ctx, int32_t schedule, int32_t use_graph) {
  if (!ctx) return LADDER_ERR_ARG;
  if (schedule < LADDER_SCHED_SERIAL || schedule > LADDER_SCHED_FUSED_LATE_ATTN) return LADDER_ERR_ARG;
  ctx->sched = schedule;
  ctx->use_graph = use_graph ? 1 : 0;
  return LADDER_OK;
}

ladder_status ladder_set_sampling(ladder_ctx* ctx, float temperature, int32_t top_k, uint64_t seed) {
  if (!ctx) return LADDER_ERR_ARG;
  if (!std::isfinite(temperature) || top_k < 0) return fail(ctx, LADDER_ERR_ARG, "bad temperature or top_k%s");
  // the decode graphs hold the draw's parameters by value
  for (auto& kv : ctx->graphs) (void)hipGraphExecDestroy(kv.second);
  ctx->graphs.clear();
  ctx->temperature = temperature > 0.f ? temperature : 0.f;
  ctx->top_k = top_k;
  ctx->seed = seed;
  return LADDER_OK;
}

ladder_status ladder_sample(const float* d_logits, int32_t B, int32_t V, int32_t ld, float temperature,
                            int32_t top_k, uint64_t seed, int32_t pos, int32_t* d_next, void* stream) {
  if (!d_logits || !d_next || B < 1 || V < 1 || ld < V || pos < 0 || !std::isfinite(temperature) ||
      !(temperature > 0.f) || top_k < 0)
    return LADDER_ERR_ARG;
  SampleParams sp{};
  sp.logits = d_logits;
  sp.ldl = ld;
  sp.V = V;
  sp.B = B;
  sp.temperature = temperature;
  sp.top_k = top_k;
  sp.seed_lo = (uint32_t)(seed & 0xffffffffu);
  sp.seed_hi = (uint32_t)(seed >> 32);
  sp.pos = pos;
  sp.next = d_next;
  if (launch_sample(sp, (hipStream_t)stream) != hipSuccess) return LADDER_ERR_HIP;
  return LADDER_OK;
}

ladder_status ladder_filled(const ladder_ctx* ctx, int32_t* out) {
  if (!ctx || !out) return LADDER_ERR_ARG;
  *out = ctx->filled;
  return LADDER_OK;
}

ladder_status ladder_workspace_bytes(const ladder_ctx* ctx, size_t* out) {
  if (!ctx || !out) return LADDER_ERR_ARG;
  *out = ctx->ws_bytes;
  return LADDER_OK;
}

ladder_status ladder_sync(ladder_ctx* ctx) {
  if (!ctx) return LADDER_ERR_ARG;
  HIPCHK(hipSetDevice(ctx->dev));
  HIPCHK(hipStreamSynchronize(ctx->s0));
  HIPCHK(hipStreamSynchronize(ctx->user));
  int err = 0;
  HIPCHK(hipMemcpy(&err, ctx->err_word, sizeof(int), hipMemcpyDeviceToHost));
  if (err) {
    ctx->broken = true;
    return fail(ctx, LADDER_ERR_HIP, "an in-kernel wait for another workgroup's signal gave up%s");
  }
  return LADDER_OK;
}

ladder_status ladder_trace_kernel(ladder_ctx* ctx, int32_t kind) {
  if (!ctx) return LADDER_ERR_ARG;
  if (ctx->broken) return LADDER_ERR_HIP;
  if (kind < -1 || kind >= LADDER_N_KERNELS) return fail(ctx, LADDER_ERR_ARG, "kernel kind out of range%s");
  if (kind >= 0 && ctx->trace_ev.empty()) {
    HIPCHK(hipSetDevice(ctx->dev));
    ctx->trace_ev.assign(2 * ((size_t)ctx->cfg.n_layers + 1), nullptr);
    for (hipEvent_t& e : ctx->trace_ev) HIPCHK(hipEventCreate(&e));
  }
  ctx->trace_kind = kind;
  ctx->trace_count = 0;
  return LADDER_OK;
}

ladder_status ladder_trace_result(ladder_ctx* ctx, float* mean_us, int32_t* count) {
  if (!ctx || !mean_us || !count) return LADDER_ERR_ARG;
  if (ctx->broken) return LADDER_ERR_HIP;
  if (ctx->trace_kind < 0 || ctx->trace_count < 1) return fail(ctx, LADDER_ERR_STATE, "no traced launches%s");
  HIPCHK(hipSetDevice(ctx->dev));
  HIPCHK(hipStreamSynchronize(ctx->s0));
  double tot = 0.0;
  for (int i = 0; i < ctx->trace_count; ++i) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, ctx->trace_ev[2 * i], ctx->trace_ev[2 * i + 1]));
    tot += ms;
  }
  *mean_us = (float)(1000.0 * tot / ctx->trace_count);
  *count = ctx->trace_count;
  return LADDER_OK;
}

ladder_status ladder_read_probe(void* stream, size_t bytes, int32_t reps, float* gbs_out) {
  if (!gbs_out || reps < 1 || bytes < (1u << 20)) return LADDER_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev))
    return LADDER_ERR_HIP;
  void* buf = nullptr;
  float* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  ladder_status st = LADDER_OK;
  float best = 0.f;
  if (hipMalloc(&buf, bytes) != hipSuccess) return LADDER_ERR_OOM;
  if (hipMalloc((void**)&sink, sizeof(float) * 8 * (size_t)ncu) != hipSuccess || hipMemsetAsync(buf, 1, bytes, s) ||
      hipEventCreate(&e0) || hipEventCreate(&e1)) {
    st = LADDER_ERR_HIP;
  } else {
    for (int per_cu : {2, 4, 8}) {
      const int grid = per_cu * ncu;
      if (launch_read_probe(buf, bytes, grid, sink, s) != hipSuccess) { st = LADDER_ERR_HIP; break; }   // warm
      bool ok = hipEventRecord(e0, s) == hipSuccess;
      for (int r = 0; r < reps && ok; ++r) ok = launch_read_probe(buf, bytes, grid, sink, s) == hipSuccess;
      ok = ok && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
      float ms = 0.f;
      if (!ok || hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f) { st = LADDER_ERR_HIP; break; }
      const float gbs = (float)((double)bytes * reps / (ms * 1e-3) / 1e9);
      if (gbs > best) best = gbs;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  (void)hipFree(buf);
  if (st == LADDER_OK) *gbs_out = best;
  return st;
}

ladder_status ladder_time_kernels(ladder_ctx* ctx, int32_t B, int32_t reps, float* us_out) {
  if (!ctx || !us_out || reps < 1) return LADDER_ERR_ARG;
  if (ctx->broken) return LADDER_ERR_HIP;
  const ladder_config& g = ctx->cfg;
  if (B < 1 || B > g.max_batch) return fail(ctx, LADDER_ERR_CAPACITY, "batch beyond capacity%s");
  if (ctx->filled < 1) return fail(ctx, LADDER_ERR_STATE, "no decode position to time at%s");
  ladder_status st = begin_call(ctx);
  if (st) return st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  HIPCHK(hipEventCreate(&e0));
  HIPCHK(hipEventCreate(&e1));
  const StreamScratch& sc = ctx->sc[0];
  hipStream_t s = ctx->s0;
  const bool rw_h = gemv_rw_supported(ctx->wdt, g.hidden, B);
  const bool rw_f = gemv_rw_supported(ctx->wdt, g.ffn, B) && gemv_rw_attn_fusable(ctx->wdt, g.ffn);
  const bool two = two_launch_layers(ctx, B);
  const bool seq = seq_layers(ctx, B);
  const bool gemv_ok = B <= 16;        // the per-kind GEMV launches take at most 16 rows
  // a batch on the matrix cores: the kinds its step launches (the skinny [QKV | gate/up]
  // and [O + down] launches of a ladder layer, the attention, the LM head, the draw)
  const bool mc = gemm_decode(ctx, B);
  const bool mc_layers = mc && skinny_layer_ok(ctx, B);
  for (int kind = 0; kind < LADDER_N_KERNELS; ++kind) {
    int launches = 0;
    HIPCHK(hipEventRecord(e0, s));   // (re-recorded after the warm-up; kept for kinds that are unavailable)
    // repetition -1 is an untimed warm-up (a kernel's first launch in a process also loads
    // its code)
    for (int r = -1; r < reps; ++r) {
      if (!gemv_ok && !mc && kind != LADDER_KERNEL_SAMPLE) break;
      if (r == 0) {
        launches = 0;
        HIPCHK(hipEventRecord(e0, s));
      }
      if (mc && kind != LADDER_KERNEL_SAMPLE) {
        if (kind == LADDER_KERNEL_LMHEAD) {
          if ((st = lm_head_mc(ctx, ctx->dx[0], g.hidden, B, s))) return st;
          ++launches;
          continue;
        }
        const bool ok = kind == LADDER_KERNEL_ATTN ||
                        (mc_layers && (kind == LADDER_KERNEL_QKV_GATEUP || kind == LADDER_KERNEL_QKV_ATTN_GATEUP ||
                                       kind == LADDER_KERNEL_DOWN_OPROJ));
        if (!ok) break;
        for (int l = 0; l < g.n_layers; ++l, ++launches) {
          if (kind == LADDER_KERNEL_ATTN) {
            AttnDecodeParams at = attn_params(ctx, l, B, sc);
            at.n_split = std::max(1, std::min(at.n_split, decode_attn_fill(B) / (B * g.n_kv_heads)));
            at.q = sc.qr;
            at.out = sc.ob;
            HIPCHK(launch_attn_decode(at, s));
            continue;
          }
          GemmParams qg[2], od;
          skinny_layer_params(ctx, l, B, qg, &od);
          if (kind == LADDER_KERNEL_QKV_ATTN_GATEUP) {
            AttnDecodeParams at = attn_params(ctx, l, B, sc);
            at.n_split = std::max(1, std::min(at.n_split, decode_attn_fill(B) / (B * g.n_kv_heads)));
            at.q = sc.qr;
            at.out = sc.ob;
            if (!skinny_pair_attn_supported(qg[0], qg[1], at)) break;
            // codes as in a decode step: a new epoch per pass over the layers, tag l + 1
            if (l == 0) HIPCHK(launch_epoch_bump(ctx->epoch, s));
            HIPCHK(launch_skinny_pair_attn(qg[0], qg[1], at, ctx->seq_prog, l + 1, ctx->err_word, s));
          } else if (kind == LADDER_KERNEL_QKV_GATEUP) {
            HIPCHK(launch_skinny_pair(qg[0], qg[1], s));
          } else {
            HIPCHK(launch_skinny(od, s));
          }
        }
        continue;
      }
      if (kind == LADDER_KERNEL_QKV_ATTN_GATEUP || kind == LADDER_KERNEL_DOWN_OPROJ) {
        if (!seq) break;
        for (int l = 0; l < g.n_layers; ++l, ++launches) {
          HIPCHK(launch_epoch_bump(ctx->epoch, s));   // a new epoch per launch, as per decode step
          const bool stream = stream_layers(ctx, B);
          if (kind == LADDER_KERNEL_QKV_ATTN_GATEUP) {
            GemvParams pr[2] = {qkv_params(ctx, l, B, ctx->dx[1], sc), gateup_params(ctx, l, B, ctx->dx[0], sc)};
            if (stream)
              HIPCHK(launch_stream_front(pr[0], pr[1], attn_params(ctx, l, B, sc), ctx->qkv_tagged, l + 1,
                                         ctx->err_word, s));
            else
              HIPCHK(launch_gemv_seq(pr[0], pr[1], attn_params(ctx, l, B, sc), ctx->seq_prog, l + 1, ctx->err_word, s));
          } else {
            const GemvParams down = outproj_params(ctx, 2 * l + 1, B, sc, nullptr, nullptr, ctx->dout[0]);
            GemvParams o = outproj_params(ctx, 2 * l, B, sc, ctx->dx[0], ctx->dx[1], nullptr);
            o.epi = EPI_ADD2;
            o.add2 = nullptr;
            o.out2 = ctx->dx[0];
            if (stream)
              HIPCHK(launch_stream_back(down, o, signalled(ctx, attn_params(ctx, l, B, sc), l), ctx->err_word, s));
            else
              HIPCHK(launch_gemv_paired_nowait(down, o, s));
          }
        }
        continue;
      }
      if (kind == LADDER_KERNEL_LAYER_STACK) {
        if (!step_usable(ctx, B)) break;
        HIPCHK(launch_epoch_bump(ctx->epoch, s));
        HIPCHK(launch_decode_step(step_params(ctx, B), s));
        ++launches;
        continue;
      }
      if (kind == LADDER_KERNEL_SAMPLE) {
        SampleParams sp = sample_params(ctx, B, ctx->pos_dev, 0);
        if (!(ctx->temperature > 0.f)) sp.top_k = 0;
        HIPCHK(launch_sample(sp, s));
        ++launches;
        continue;
      }
      if (kind == LADDER_KERNEL_LMHEAD) {
        if ((st = run_gemv(ctx, lmhead_params(ctx, ctx->dx[0], g.hidden, B), s))) return st;
        ++launches;
        continue;
      }
      for (int l = 0; l < g.n_layers; ++l, ++launches) {
        switch (kind) {
          case LADDER_KERNEL_QKV: st = run_gemv(ctx, qkv_params(ctx, l, B, ctx->dx[0], sc), s); break;
          case LADDER_KERNEL_ATTN: HIPCHK(launch_attn_decode(attn_params(ctx, l, B, sc), s)); break;
          case LADDER_KERNEL_OPROJ:
            st = run_gemv(ctx, outproj_params(ctx, 2 * l, B, sc, ctx->dx[0], ctx->dx[1], nullptr), s);
            break;
          case LADDER_KERNEL_GATEUP: st = run_gemv(ctx, gateup_params(ctx, l, B, ctx->dx[0], sc), s); break;
          case LADDER_KERNEL_DOWN:
            st = run_gemv(ctx, outproj_params(ctx, 2 * l + 1, B, sc, ctx->dx[0], ctx->dx[1], nullptr), s);
            break;
          case LADDER_KERNEL_QKV_GATEUP: {
            GemvParams pr[2] = {qkv_params(ctx, l, B, ctx->dx[1], sc), gateup_params(ctx, l, B, ctx->dx[0], sc)};
            if (rw_h) {
              HIPCHK(launch_gemv_multi(pr, 2, nullptr, s, nullptr));
            } else if (!(st = run_gemv(ctx, pr[0], s))) {
              st = run_gemv(ctx, pr[1], s);
            }
            break;
          }
          case LADDER_KERNEL_ATTN_DOWN: {
            const GemvParams down = outproj_params(ctx, 2 * l + 1, B, sc, nullptr, nullptr, ctx->dout[0]);
            const AttnDecodeParams at = attn_params(ctx, l, B, sc);
            if (two) {                         // a new epoch per launch, as per decode step
              GemvParams o = outproj_params(ctx, 2 * l, B, sc, ctx->dx[0], ctx->dx[1], nullptr);
              o.epi = EPI_ADD2;
              o.add2 = nullptr;
              o.out2 = ctx->dx[0];
              HIPCHK(launch_epoch_bump(ctx->epoch, s));
              HIPCHK(launch_gemv_paired(down, o, signalled(ctx, at, l), ctx->err_word, s));
            } else if (rw_f) {
              HIPCHK(launch_gemv_multi(&down, 1, &at, s, nullptr));
            } else {
              HIPCHK(launch_attn_decode(at, s));
              st = run_gemv(ctx, down, s);
            }
            break;
          }
          default: {
            GemvParams o = outproj_params(ctx, 2 * l, B, sc, ctx->dx[0], ctx->dx[1], nullptr);
            o.epi = EPI_ADD2;
            o.add2 = ctx->dout[0];
            o.out2 = ctx->dx[0];
            st = run_gemv(ctx, o, s);
            break;
          }
        }
        if (st) return st;
      }
    }
    HIPCHK(hipEventRecord(e1, s));
    HIPCHK(hipEventSynchronize(e1));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, e0, e1));
    us_out[kind] = launches ? 1000.f * ms / (float)launches : -1.f;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return end_call(ctx);
}

ladder_status ladder_prefill(ladder_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t T, int32_t start_pos,
                             float* d_logits, int32_t* d_next, float* d_hidden) {
  if (!ctx || !d_ids) return LADDER_ERR_ARG;
  if (ctx->broken) return LADDER_ERR_HIP;
  const ladder_config& g = ctx->cfg;
  if (B < 1 || T < 1 || start_pos < 0) return fail(ctx, LADDER_ERR_ARG, "bad B/T/start_pos%s");
  if (B > g.max_batch || (long long)start_pos + T > g.max_seq)
    return fail(ctx, LADDER_ERR_CAPACITY, "batch or positions beyond capacity%s");
  if (start_pos > ctx->filled) return fail(ctx, LADDER_ERR_STATE, "prefill starts after unfilled positions%s");
  ladder_status st = begin_call(ctx);
  if (st) return st;
  const int tc_max = std::max(1, ctx->mmax / B);
  const int NM = 2 * g.n_layers;
  for (int t0 = 0; t0 < T; t0 += tc_max) {
    const int Tc = std::min(tc_max, T - t0);
    const int M = B * Tc;
    HIPCHK(hipMemcpy2DAsync(ctx->ids_chunk, (size_t)Tc * 4, d_ids + t0, (size_t)T * 4, (size_t)Tc * 4, B,
                            hipMemcpyDeviceToDevice, ctx->s0));
    HIPCHK(launch_embed(ctx->wdt, ctx->w.tok_embed, g.vocab, g.hidden, ctx->ids_chunk, M, ctx->px[0], ctx->s0));
    const int sp = start_pos + t0;
    auto mod = [&](int m, const float* xin, const float* xm, float* xn, float* store, hipStream_t s, bool wait,
                   hipEvent_t ev) { return prefill_module(ctx, m, B, Tc, sp, xin, xm, xn, store, s, wait, ev); };
    const int saved = ctx->sched;
    const bool fused = saved >= LADDER_SCHED_FUSED;
    // prefill under the fused schedules: attention and MLP modules on two streams, each
    // module's residual adds in its GEMMs (the DUAL schedule; one stream in module order
    // took 49.3 against 45.1 ms for the 70B shard's 1024-token prompt, with the same bits:
    // the streams only overlap launches that fill the device partly, such as the QKV GEMM's
    // 320 workgroups and the attention)
    if (fused) ctx->sched = LADDER_SCHED_DUAL;
    st = run_modules(ctx, ctx->px, ctx->pout, (size_t)M * g.hidden, mod, fused);
    ctx->sched = saved;
    if (st) return st;
    if (t0 + Tc == T) {
      const float* xl = ctx->px[NM % 2] + (size_t)(Tc - 1) * g.hidden;
      st = lm_head(ctx, xl, Tc * g.hidden, B, ctx->s0, nullptr, start_pos + T - 1);
      if (st) return st;
      st = copy_outputs(ctx, B, xl, (size_t)Tc * g.hidden * 4, d_logits, d_next, d_hidden);
      if (st) return st;
    }
  }
  ctx->filled = std::max(ctx->filled, start_pos + T);
  return end_call(ctx);
}

ladder_status ladder_decode_step(ladder_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t pos, float* d_logits,
                                 int32_t* d_next, float* d_hidden) {
  if (!ctx || !d_ids) return LADDER_ERR_ARG;
  if (ctx->broken) return LADDER_ERR_HIP;
  const ladder_config& g = ctx->cfg;
  if (B < 1 || pos < 0) return fail(ctx, LADDER_ERR_ARG, "bad B/pos%s");
  if (B > g.max_batch || pos >= g.max_seq) return fail(ctx, LADDER_ERR_CAPACITY, "batch or position beyond capacity%s");
  if (pos > ctx->filled) return fail(ctx, LADDER_ERR_STATE, "decode position after unfilled positions%s");
  ladder_status st = begin_call(ctx);
  if (st) return st;
  HIPCHK(launch_decode_prologue(d_ids, ctx->ids_dev, B, ctx->pos_dev, pos, ctx->epoch, ctx->wdt, ctx->w.tok_embed,
                                g.vocab, g.hidden, ctx->dx[0], ctx->s0));
  // occupancy queries of the persistent launch happen here, not under graph capture
  if (ctx->sched == LADDER_SCHED_PERSISTENT) (void)step_usable(ctx, B);
  // traced steps run eagerly: event records captured into a graph carry no timestamps
  if (ctx->use_graph && ctx->trace_kind < 0) {
    const int key = (B * 8 + ctx->sched) * 2 + (ctx->temperature > 0.f ? 1 : 0);
    auto it = ctx->graphs.find(key);
    if (it == ctx->graphs.end()) {
      hipGraph_t graph = nullptr;
      HIPCHK(hipStreamBeginCapture(ctx->s0, hipStreamCaptureModeRelaxed));
      st = enqueue_decode(ctx, B);
      hipError_t ce = hipStreamEndCapture(ctx->s0, &graph);
      if (st) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
      }
      HIPCHK(ce);
      hipGraphExec_t exec = nullptr;
      hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      HIPCHK(ie);
      it = ctx->graphs.emplace(key, exec).first;
    }
    HIPCHK(hipGraphLaunch(it->second, ctx->s0));
  } else {
    st = enqueue_decode(ctx, B);
    if (st) return st;
  }
  st = copy_outputs(ctx, B, ctx->dx[(2 * g.n_layers) % 2], (size_t)g.hidden * 4, d_logits, d_next, d_hidden);
  if (st) return st;
  ctx->filled = std::max(ctx->filled, pos + 1);
  return end_call(ctx);
}

ladder_status ladder_decode_step_static(ladder_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t pos,
                                        float* d_logits, int32_t* d_next, float* d_hidden) {
  if (!ctx || !d_ids) return LADDER_ERR_ARG;
  if (ctx->broken) return LADDER_ERR_HIP;
  const ladder_config& g = ctx->cfg;
  if (B < 1 || pos < 0) return fail(ctx, LADDER_ERR_ARG, "bad B/pos%s");
  if (B > g.max_batch || pos >= g.max_seq) return fail(ctx, LADDER_ERR_CAPACITY, "batch or position beyond capacity%s");
  if (pos > ctx->filled) return fail(ctx, LADDER_ERR_STATE, "decode position after unfilled positions%s");
  void* base = nullptr;
  const hipError_t se = static_scratch(ctx->dev, &base);
  if (se != hipSuccess || !base)
    return fail(ctx, LADDER_ERR_HIP, "the static scratch has no device address: %s", hipGetErrorString(se));
  // every schedule gives the same bits; FUSED runs on the context's stream alone with one
  // set of stream scratch
  const StepShape sh{B, B, 1, gemm_decode(ctx, B), false};
  // the per-step pointers go back to the workspace however this call ends
  struct Restore {
    ladder_ctx* c;
    int sched;
    ~Restore() {
      c->sched = sched;
      carve_ws_step(c);
    }
  } restore{ctx, ctx->sched};
  Carver measure;
  carve_step(ctx, measure, sh);
  if (measure.off > kStaticScratchBytes) {
    char what[160];
    snprintf(what, sizeof what, "%zu bytes at batch %d, above the %zu bytes it holds", measure.off, (int)B,
             kStaticScratchBytes);
    return fail(ctx, LADDER_ERR_CAPACITY, "the static scratch is too small for this step: %s", what);
  }
  Carver cv;
  cv.base = (char*)base;
  carve_step(ctx, cv, sh);
  ctx->sched = LADDER_SCHED_FUSED;
  ladder_status st = begin_call(ctx);
  if (st) return st;
  HIPCHK(launch_zero_bytes(base, ctx->step_zero_bytes, ctx->s0));
  HIPCHK(launch_decode_prologue(d_ids, ctx->ids_dev, B, ctx->pos_dev, pos, ctx->epoch, ctx->wdt, ctx->w.tok_embed,
                                g.vocab, g.hidden, ctx->dx[0], ctx->s0));
  if ((st = enqueue_decode(ctx, B))) return st;
  st = copy_outputs(ctx, B, ctx->dx[(2 * g.n_layers) % 2], (size_t)g.hidden * 4, d_logits, d_next, d_hidden);
  if (st) return st;
  ctx->filled = std::max(ctx->filled, pos + 1);
  return end_call(ctx);
}

}  // extern "C"

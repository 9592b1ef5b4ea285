// Host-side launchers of the gfx950 kernels (internal to libladder; not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ladder {

enum WDtype { W_F32 = 0, W_BF16 = 1 };

// Rows of a (virtual) weight matrix [N][K] gathered from up to three stored
// matrices, each row-major [rows][K]:
//   interleave == 0: rows [0,n0) from m[0], [n0,n1) from m[1], [n1,N) from m[2];
//   interleave == 1: row r is row r/2 of m[r & 1] (gate/up pairs side by side).
struct RowSrc {
  const void* m[3];
  int n0, n1;
  int interleave;
};

// ---------------------------------------------------------------- decode GEMV
enum GemvEpi {
  EPI_STORE = 0,        // out[b][n] = y
  EPI_ADD = 1,          // out[b][n] = xres[b][n] + y   (ladder residual add, fused)
  EPI_QKV_ROPE = 2,     // q -> out (fp32, rotated); k (rotated), v -> KV cache at pos
  EPI_GATEUP_SWIGLU = 3,// out[b][n] = silu(y[2n]) * y[2n+1]
  EPI_LOGITS = 4,       // out[b][n] = y; greedy argmax -> next_out[b]
  EPI_ADD2 = 5,         // out[b][n] = xres[b][n] + y; out2[b][n] = out[b][n] + add2[b][n]
};

struct GemvParams {
  int wdtype;
  RowSrc rows;
  int N, K, B;
  const float* x; int ldx;        // input rows [B][ldx] (fp32)
  const void* gain; float eps;    // RMSNorm gain of the input (nullptr: no norm)
  int epi;
  float* out; int ldo;
  const float* xres; int ldr;     // EPI_ADD, EPI_ADD2
  const float* add2; float* out2; // EPI_ADD2 (same leading dimension as out)
  // EPI_QKV_ROPE
  void* k_cache; void* v_cache;   // this layer: [max_batch][n_kv][max_seq][head_dim]
  int q_rows, kv_rows, head_dim, max_seq, n_kv;
  const float* rope_cos; const float* rope_sin;   // [max_seq][head_dim/2]
  const int* d_pos;
  // EPI_LOGITS
  float* best_val; int* best_idx; int* arg_counter; int* next_out;
  // split-K workspace (used when B is large enough that K is split)
  float* part; float* part_sq; int* counters;
};

struct GemvWorkspaceReq { size_t part_floats, part_sq_floats, counters, best; };
// Workspace a decode GEMV of this shape needs at batch B (upper bounds).
GemvWorkspaceReq gemv_workspace(int wdtype, int N, int K, int B);
hipError_t launch_gemv(const GemvParams& p, hipStream_t s);

// ----------------------------------------------------------- decode attention
struct AttnDecodeParams {
  int wdtype;                          // KV cache element type
  const float* q;                      // [B][nq*hd], rotated
  const void* k_cache; const void* v_cache;  // this layer's base
  int max_seq, nq, nkv, hd, B;
  const int* d_pos;                    // keys 0..pos
  int n_split;
  float* part;                         // [B][nq][n_split][hd+4]: max, sum, -, -, acc[hd]
  int* counters;                       // [B][nkv]
  float* out;                          // [B][nq*hd]
  // completion signal (nullable): after the last of the B*nkv merges, done_flag = *d_epoch
  const int* d_epoch;
  int* done_cnt;                       // merges finished (reset to 0 by the last)
  int* done_flag;
};
int attn_decode_splits(int max_seq);
hipError_t launch_attn_decode(const AttnDecodeParams& p, hipStream_t s);

// ------------------------------------------- row-wave GEMV (batch <= 4), fused launches
// Up to two GEMV problems with the same K and batch, optionally preceded by the
// workgroups of a split-KV decode attention, in one launch.
struct MultiGemvParams {
  GemvParams prob[2];
  int np;
  int blk_begin[3];       // problem p owns blocks [blk_begin[p], blk_begin[p+1]) after the attention ones
  int n_attn;             // leading workgroups running decode attention (0 = none)
  AttnDecodeParams attn;
  // paired launch: every GEMV workgroup computes rows R of prob[0] (kept in LDS), then,
  // once *wait_flag == *d_epoch, the same rows R of prob[1], whose EPI_ADD2 epilogue
  // adds prob[0]'s row in place of add2
  int paired;
  int dres_off;           // LDS byte offset of prob[0]'s rows [rows per block][BT]
  const int* wait_flag;
  const int* d_epoch;
  int* err;               // set to 1 if a wait ever gives up (never expected)
  int part_off;           // LDS byte offset of the partial sums (set by the launcher)
  int wpre_off;           // LDS byte offset of prob[1]'s weights copied during the wait (0: none)
  // sequential launch: every GEMV workgroup computes its share of prob[0] (coherent
  // stores), publishes code(*d_epoch, seq_tag) in prog[its index], then its share of
  // prob[1]; the attention workgroups start once every word has reached that code
  int seq;
  uint32_t* prog;
  int seq_tag;            // 1 <= seq_tag < kSeqCodeStride
  // batch-1 streaming front launch: the QKV outputs as (code << 32 | value bits) words,
  // one per QKV row, polled by the attention workgroups of the same launch
  unsigned long long* tagged;
};
// Progress code of a sequential launch: epoch * kSeqCodeStride + tag, so that the codes
// of a decode step exceed those of every earlier step.
constexpr uint32_t kSeqCodeStride = 1024;
constexpr int kSeqProgWords = 1024;     // progress words of a sequential launch (>= its GEMV workgroups)
bool gemv_rw_supported(int wdtype, int K, int B);
bool gemv_rw_two_per_cu(int wdtype, int K, int B);   // ... with two workgroups per CU
bool gemv_rw_attn_fusable(int wdtype, int K);   // a launch of this K can carry attention workgroups
int gemv_rw_blocks(int wdtype, int N, int K, int B);   // workgroups of a one-problem launch
int gemv_rw_bt(int B);
// blocks_out (nullable): workgroups given to each problem
hipError_t launch_gemv_multi(const GemvParams* probs, int np, const AttnDecodeParams* attn, hipStream_t s,
                             int* blocks_out);
// Paired launch [attention | first: rows, then (once the attention has signalled) second:
// the same rows with EPI_ADD2 taking first's result as add2].  first.N == second.N; the
// attention's completion signal (done_cnt/done_flag, epoch *d_epoch) is what the second
// pass waits for.  err: device word set on a failed wait.
bool gemv_rw_pair_supported(int wdtype, int K_first, int K_second, int B);
hipError_t launch_gemv_paired(const GemvParams& first, const GemvParams& second, const AttnDecodeParams& attn,
                              int* err, hipStream_t s);
// Paired launch without attention: rows R of first (kept in LDS), then the same rows R of
// second with EPI_ADD2 taking first's result as add2; nothing waits.
hipError_t launch_gemv_paired_nowait(const GemvParams& first, const GemvParams& second, hipStream_t s);
// Sequential launch [first, then second, in every GEMV workgroup | attention once every
// workgroup has finished first]: first must be the QKV projection (EPI_QKV_ROPE) that
// produces the attention's q and newest K/V row; the attention must not signal
// (done_flag null).  prog: kSeqProgWords words, zero or holding codes of earlier launches
// of this context; tag: distinguishes the launches of one decode step (1 <= tag <
// kSeqCodeStride, increasing within the step); the code waited for is
// *attn.d_epoch * kSeqCodeStride + tag.  err: set if the wait gives up.
bool gemv_rw_seq_supported(int wdtype, int K, int B, int hd);
hipError_t launch_gemv_seq(const GemvParams& first, const GemvParams& second, const AttnDecodeParams& attn,
                           uint32_t* prog, int tag, int* err, hipStream_t s);
// Batch-1 streaming launches of one ladder layer (stream.hip), always used as a pair:
//   front: [QKV then gate/up in every workgroup | attention chunk records once every QKV
//          output of the kv group is there]; the QKV outputs reach the attention as tagged
//          words (no progress words);
//   back:  [attention merge of those records (attn.done_cnt/done_flag signal, epoch
//          *attn.d_epoch) | down, then (after the signal) O + both residual adds]; same
//          projections as launch_gemv_paired_nowait.
// Each workgroup streams its weight units with the next pass's units in flight across
// the pass boundary; the results equal the row-wave launches' bit for bit.
bool stream_front_supported(int wdtype, int K, int B, int hd);
bool stream_back_supported(int wdtype, int Kd, int Ko, int B, int N, int nq, int n_split);
// tagged: one 64-bit word per QKV row (zero or holding codes of earlier launches of this
// context); tag as for launch_gemv_seq.
hipError_t launch_stream_front(const GemvParams& first, const GemvParams& second, const AttnDecodeParams& attn,
                               unsigned long long* tagged, int tag, int* err, hipStream_t s);
hipError_t launch_stream_back(const GemvParams& down, const GemvParams& o, const AttnDecodeParams& attn, int* err,
                              hipStream_t s);
// next[b] = first maximum of n per-workgroup candidates (best_val/best_idx [n][BT])
hipError_t launch_argmax_finalize(const float* best_val, const int* best_idx, int n, int BT, int B, int* next,
                                  hipStream_t s);

// --------------------------------------------------- persistent decode step
constexpr int kStepProgWords = 1024;
// One launch for the whole layer stack of a decode step (all layers ladder, bf16 weights
// and cache, batch <= 4).
struct StepLayer {
  const void* wq; const void* wk; const void* wv; const void* wo;
  const void* wg; const void* wu; const void* wd;
  const void* attn_norm; const void* mlp_norm;
  void* k_cache; void* v_cache;        // this layer's [max_batch][n_kv][max_seq][hd]
};
struct StepParams {
  const StepLayer* layers;             // device array [L]
  int L, H, F, nq, nkv, hd, B, max_seq;
  float eps;
  const float* rope_cos; const float* rope_sin;
  const int* d_pos; const int* d_epoch;
  float* x0;                           // [B][H]: x_0 on entry, x_{2L} on exit
  float* xs; size_t xstride;           // x_j (1 <= j < 2L) at xs + (j-1)*xstride, [B][H] each
  float* qs; float* os; size_t qstride;  // q and the attention output of layer l at +l*qstride ([B][nq*hd])
  float* as; size_t astride;           // SwiGLU output of layer l at as + l*astride ([B][F])
  float* part; int* attn_cnt; int n_split;   // attention records [B][nq][n_split][hd+4], tickets [B][nkv]
  int* sync;                           // [L][8] counters and flags (zero before the first step)
  uint32_t* prog;                      // [kStepProgWords] progress word per projection workgroup
  int* err;                            // set if a wait gives up
  int n_attn;                          // set by the launcher
  int dres_off;                        // set by the launcher
  int rows_lds;                        // set by the launcher
  int part_off;                        // set by the launcher
};
bool step_supported(int wdtype, int H, int F, int qrows, int B, int hd, int G);
// true when every workgroup of the launch can be resident (queries the occupancy once)
bool step_fits(const StepParams& sp);
hipError_t launch_decode_step(const StepParams& sp, hipStream_t s);

// ------------------------------------------------------------ sampling
// next[b] = a draw from softmax(logits[b] / temperature) over the top_k largest logits
// (all when top_k is 0 or >= V; ties at the cut are kept), by the Gumbel-max rule with
// Philox4x32-10 uniforms of counter (i / 4, b, pos, 0) and key (seed_lo, seed_hi).
// pos = *d_pos when d_pos is set (read when the kernel runs), else pos.
struct SampleParams {
  const float* logits; int ldl;        // [B][ldl], V used
  int V, B;
  float temperature;                   // > 0, finite
  int top_k;                           // >= 0
  uint32_t seed_lo, seed_hi;
  const int* d_pos; int pos;
  int* next;                           // [B]
};
hipError_t launch_sample(const SampleParams& p, hipStream_t s);

// ---------------------------------------------------------- prefill attention
struct AttnPrefillParams {
  int wdtype;
  const float* q;                      // [B*T][nq*hd] rotated, fp32
  const void* k_cache; const void* v_cache;
  int max_seq, nq, nkv, hd, B, T, start_pos;
  float* out;                          // [B*T][nq*hd]
  // key split (bf16, nullable): when the query tiles give the device few workgroups, each
  // tile's keys are cut into at most kAttnPrefillMaxChunks chunks whose records
  // [B][nq][T][chunks][hd+4] a merge kernel combines; part_floats >= attn_prefill_part_floats(hd)
  float* part; size_t part_floats;
  int kchunk, nchunk;                  // set by the launcher
};
constexpr int kAttnPrefillMaxChunks = 4;
constexpr size_t attn_prefill_part_floats(int hd) {
  return (size_t)256 * 128 * kAttnPrefillMaxChunks * (hd + 4);   // B*T*nq < 256 query tiles of 128
}
hipError_t launch_attn_prefill(const AttnPrefillParams& p, hipStream_t s);

// ----------------------------------------------------------------- GEMM (prefill)
// C[M][N] (fp32, ldc) = (res ? res[M][N] : 0) + A[M][K] . B^T, B rows from RowSrc; with
// swiglu (bf16 models, N even, rows interleaved gate/up): C[M][N/2] = silu(c[2n]) * c[2n+1].
struct GemmParams {
  int wdtype;                          // W_BF16: MFMA on bf16 pairs of A and the bf16 weights; W_F32: VALU
  // A: fp32 [M][lda] (lda a multiple of 4 for bf16 models); or, with a_pairs (bf16
  // models, where gemm_takes_pairs() holds), A already split into bf16 pairs hi = bf16(a),
  // lo = bf16(a - hi): row m holds lda / 4 groups of 16 bytes, the 4 hi then the 4 lo
  // values of 4 consecutive columns (the bytes of an fp32 row)
  const void* A; int lda;
  int a_pairs;
  RowSrc rows;
  int M, N, K;
  float* C; int ldc;
  const float* res; int ldr;
  int swiglu;
  // c_pairs (SwiGLU launches where gemm_writes_pairs() holds): C is written as bf16 pairs
  // in a_pairs' layout, ready to be the A of the next projection ([M][ldc / 4] groups)
  int c_pairs;
  // split-K partials (nullable: no split); kGemmSplitWsFloats floats cover any split the
  // launcher chooses
  float* ws; size_t ws_floats;
  // gain (nullable, bf16 [K]): RMSNorm fused into a split-K launch, A being the raw rows:
  // the workgroups multiply A by the gain on its way into LDS, those of the first column
  // tile also store each slice's per-row sum of squares after the partials in ws, and the
  // reduction scales each row's sums by 1 / sqrt(mean square + eps).  Only valid where
  // gemm_norm_fusable() holds for p with the gain set (the launch is refused otherwise).
  const void* gain; float eps;
  // tickets of the skinny launch (M <= 32): kSkinnyMaxTiles ints, zero between launches
  // (each launch returns them to zero); nullable: no skinny launch
  int* cnt;
  // second K part (skinny launches only; A2 nullable): C = res + A . W^T and
  // C2 = C + A2 . W2^T, with W2 rows from rows2 (the same N rows), K2 columns, fp32 A2 [M][lda2]
  const void* A2; int lda2;
  RowSrc rows2;
  int K2;
  float* C2;
  // RoPE + KV append in the epilogue of a decode step's QKV projection (skinny launches
  // only; rope_q nullable: none).  Row m is sequence m at position *d_pos; output columns
  // [0, nq*hd) are q, then nkv*hd of k, then nkv*hd of v.  q is rotated into rope_q
  // [M][nq*hd], k rotated and v as they are go to the bf16 caches [M][nkv][max_seq][hd] at
  // that position (rope_kv's arithmetic and rounding); C is not written.
  float* rope_q; void* k_cache; void* v_cache;
  const float* rope_cos; const float* rope_sin; const int* d_pos;
  int nq, nkv, hd, max_seq;
};
constexpr size_t kGemmSplitWsFloats = (size_t)512 * 128 * 128;
constexpr int kSkinnyMaxTiles = 2048;
// C = (R) + A . W^T: for bf16 weights and M <= 64 rows a skinny launch (weights streamed
// into the matrix cores, K slices reduced in the same launch) where skinny_supported(p),
// else the tiled GEMM with a separate split-K reduction.
hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
bool skinny_supported(const GemmParams& p);
hipError_t launch_skinny(const GemmParams& p, hipStream_t s);
// Two skinny problems in one launch (same M, both with or both without the RMSNorm fold,
// workspaces and tickets of their own); each gives the bits of its own launch_skinny.
bool skinny_pair_supported(const GemmParams& a, const GemmParams& b);
hipError_t launch_skinny_pair(const GemmParams& a, const GemmParams& b, hipStream_t s);
// The pair [QKV | gate/up] of a decode step with its split-KV attention in the same launch:
// a (the QKV projection) carries the RoPE + KV epilogue (rope_q set) and the RMSNorm fold;
// the attention's q, caches, position and shape are a's; its workgroups wait (bounded; a
// wait that gives up sets *err) until every QKV tile has published *at.d_epoch *
// kSeqCodeStride + tag in prog[tile] (prog: one word per QKV tile, holding codes of earlier
// launches only), then write their records and merge them (tickets at.counters, output
// at.out); the attention gives the bits of launch_attn_decode with the same n_split.
bool skinny_pair_attn_supported(const GemmParams& a, const GemmParams& b, const AttnDecodeParams& at);
hipError_t launch_skinny_pair_attn(const GemmParams& a, const GemmParams& b, const AttnDecodeParams& at,
                                   uint32_t* prog, int tag, int* err, hipStream_t s);
// Workspace floats the skinny launch of p takes (partials and sums of squares).
size_t skinny_ws_floats(const GemmParams& p);
// K slices launch_gemm uses for p (1: no split).
int gemm_splits(const GemmParams& p);
// Whether a launch can take A as bf16 pairs (GemmParams::a_pairs): bf16 weights,
// more than 64 rows (the 128-row tiles), no folded RMSNorm.
bool gemm_takes_pairs(const GemmParams& p);
// Two projections of 33-64 rows that each take a split-K tiled launch (gemm_splits() > 1,
// their own workspaces), with or without the folded RMSNorm in both: one launch of both
// problems' workgroups, then each problem's reduction; the same bits as launch_gemm of
// each.
bool gemm_pair_ok(const GemmParams& a, const GemmParams& b);
hipError_t launch_gemm_pair(const GemmParams& a, const GemmParams& b, hipStream_t s);
// A pair whose second problem adds onto the first's output (a: C = res + A.W^T, b: C =
// a.C + A.W^T, the same N, no gain or SwiGLU): one launch of both, then one reduction
// writing both outputs; the same bits as launch_gemm of a, then of b.
bool gemm_chain_ok(const GemmParams& a, const GemmParams& b);
hipError_t launch_gemm_chain(const GemmParams& a, const GemmParams& b, hipStream_t s);
// The same chained pair with the decode attention whose output is a's A in the same launch
// (bf16; the attention with its completion signal: done_cnt, done_flag, d_epoch): the
// attention and b's workgroups run side by side, a's wait for the signal (bounded; a wait
// that gives up sets *err).  The same bits as launch_attn_decode, then launch_gemm_chain.
bool gemm_attn_chain_ok(const AttnDecodeParams& at, const GemmParams& a, const GemmParams& b);
hipError_t launch_gemm_attn_chain(const AttnDecodeParams& at, const GemmParams& a, const GemmParams& b, int* err,
                                  hipStream_t s);
// Whether a SwiGLU launch can write its output as bf16 pairs (GemmParams::c_pairs): the
// tiled kernel without split K, more than 64 rows.
bool gemm_writes_pairs(const GemmParams& p);
bool gemm_norm_fusable(const GemmParams& p);

// ------------------------------------------------------------ launch timing
// Arm: the decode-path kernels launched until disarm record `start` (first dispatch
// begins) and `stop` (each dispatch ends) through hipExtLaunchKernelGGL.
void launch_events_arm(hipEvent_t start, hipEvent_t stop);
void launch_events_disarm();

// ------------------------------------------------------------------ elementwise
hipError_t launch_embed(int wdtype, const void* table, int V, int H, const int* ids, int M, float* x, hipStream_t s);
// out[m][:] = RMSNorm(x[m*ldx + :]) * gain (fp32)
hipError_t launch_rmsnorm(int wdtype, const float* x, int ldx, const void* gain, float eps, int M, int H,
                          float* out, hipStream_t s);
// The same RMSNorm with bf16 gains, its output split into bf16 pairs for a GEMM's a_pairs
// input ([M][H / 4] groups of 4 hi then 4 lo values, the bytes of an fp32 [M][H] output);
// each value is the fp32 RMSNorm output split as the GEMM would split it.  H and ldx
// multiples of 4.
hipError_t launch_rmsnorm_pairs(const float* x, int ldx, const void* gain, float eps, int M, int H, void* out,
                                hipStream_t s);
// qkv [B*T][q_rows + 2 kv_rows] -> q (rotated, fp32) and KV cache rows p0..p0+T-1, with
// p0 = *d_pos when d_pos is set (read when the kernel runs), else start_pos
hipError_t launch_rope_kv(int wdtype, const float* qkv, int B, int T, int start_pos, const int* d_pos, int nq, int nkv, int hd,
                          const float* rope_cos, const float* rope_sin, float* q_out,
                          void* k_cache, void* v_cache, int max_seq, hipStream_t s);
// gu [M][2F] interleaved (gate, up) -> a [M][F] (fp32)
hipError_t launch_swiglu(const float* gu, int M, int F, float* a, hipStream_t s);
hipError_t launch_add(const float* x, const float* y, float* out, size_t n, hipStream_t s);
// next[b] = index of the first maximum of x[b][0..V) (row pitch ld)
hipError_t launch_argmax_rows(const float* x, int B, int V, int ld, int* next, hipStream_t s);
hipError_t launch_epoch_bump(int* d_epoch, hipStream_t s);   // ++*d_epoch
// plain streaming read of bytes of buf by grid workgroups (sink: >= grid floats, never
// read in practice)
hipError_t launch_read_probe(const void* buf, size_t bytes, int grid, float* sink, hipStream_t s);
// ids_dst = ids_src, *d_pos = pos, ++*d_epoch (the step counter of in-kernel signals;
// nullable), and x[b][:] = table[ids_src[b]][:] in fp32 for b < B (B <= 256)
hipError_t launch_decode_prologue(const int* ids_src, int* ids_dst, int B, int* d_pos, int pos, int* d_epoch,
                                  int wdtype, const void* table, int V, int H, float* x, hipStream_t s);

// ------------------------------------------------------------------ static scratch
// Device bytes of the library's static scratch array (one copy per GPU, held until the
// process ends).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
// Look up the device address of device dev's copy (dev must be current); once per
// device, later calls return the first result.
hipError_t static_scratch_setup(int dev);
// The address static_scratch_setup found (hipErrorNotInitialized before it ran).
hipError_t static_scratch(int dev, void** ptr);
// Zero bytes (a multiple of 16) at p (16-byte aligned) with a kernel.
hipError_t launch_zero_bytes(void* p, size_t bytes, hipStream_t s);

}  // namespace ladder

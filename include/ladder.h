/*
 * ladder.h -- C ABI of libladder: the per-token forward step of a Ladder Residual
 * Transformer (attention and SwiGLU-MLP modules, Llama-3.1 shaped) on one AMD
 * Instinct MI355X (gfx950).
 *
 * The method (arXiv 2501.06589; Paper-Notes page "Ladder Residual:
 * Parallelism-Aware Architecture for Accelerating Large Model Inference",
 * sections "core idea" and "method details / key design"): every attention and
 * every MLP is one module h; the standard residual update x_{i+1} = h_{i+1}(x_i) + x_i
 * becomes x_{i+1} = h_{i+1}(x_{i-1}) + x_i, so a module reads the residual stream
 * from one step earlier while the stream itself still accumulates every module's
 * output (section "overall framework").  A module therefore never waits for the
 * previous module's result; the pages use this to overlap the tensor-parallel
 * all-reduce with compute (section "asynchronous AllReduce implementation").
 * Layers can be mixed: standard lower layers, ladder upper layers (section
 * "hybrid Ladder adaptation"), and parallel blocks (the "Parallel" baseline of the
 * results tables, which the pages do not define; taken here as the block whose
 * attention and MLP both read the layer input, x_{2l+2} = x_{2l} + A(x_{2l}) + M(x_{2l})).
 *
 * This library runs one tensor-parallel rank's shard of such a model with the
 * cross-GPU all-reduce replaced by identity.  Module numbering: m = 0..2L-1,
 * m = 2l is layer l's attention, m = 2l+1 its MLP; x_0 is the token embedding,
 * x_{m+1} = x_m + out_m; a ladder module reads x_{m-1} (x_{-1} taken as x_0), a
 * standard module reads x_m, and a parallel block's attention reads x_m and its MLP
 * x_{m-1}.  The final hidden state is x_{2L}; logits are
 * RMSNorm(x_{2L}) . W_lm^T and the next token is their argmax (lowest index on
 * exact ties).
 *
 * Conventions for every entry point
 *   - Pointers named d_* and every pointer inside ladder_weights / ladder_kv are
 *     device pointers on the GPU that was current at ladder_init; others are host.
 *   - Matrices are row-major [out][in] (the nn.Linear layout), 16-byte aligned.
 *   - bf16 tensors hold raw bfloat16 bit patterns (uint16).
 *   - The caller owns weights, KV cache, ids and outputs and keeps them alive and
 *     unmodified until ladder_free; the context owns its workspace, streams,
 *     events and graphs.
 *   - Work is enqueued asynchronously on the stream given to ladder_init; the
 *     context's internal streams are joined back into it before each call returns.
 *   - Argument errors are reported synchronously and leave the context usable;
 *     LADDER_ERR_HIP is sticky (the context must then be freed).
 *   - A context is not thread-safe.
 */
#ifndef LADDER_H
#define LADDER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ladder_status;
#define LADDER_OK 0
#define LADDER_ERR_ARG (-1)      /* null pointer, unknown enum, non-positive size */
#define LADDER_ERR_SHAPE (-2)    /* dimensions this build does not support */
#define LADDER_ERR_CAPACITY (-3) /* B > max_batch, or positions beyond max_seq */
#define LADDER_ERR_STATE (-4)    /* reads KV positions that were never written */
#define LADDER_ERR_HIP (-5)      /* a HIP runtime call failed (sticky) */
#define LADDER_ERR_OOM (-6)      /* workspace allocation failed */

#define LADDER_F32 0             /* weights and KV cache fp32 */
#define LADDER_BF16 1            /* weights and KV cache bf16; residual and accumulation fp32 */

/* Execution schedule of the module loop.  All give bitwise identical results. */
#define LADDER_SCHED_SERIAL 0    /* one stream, modules and residual adds in program order */
#define LADDER_SCHED_SIDE 1      /* residual adds on a side stream: module m+1 starts on its
                                    stale input while x_{m+1} = x_m + out_m completes */
#define LADDER_SCHED_DUAL 2      /* attention and MLP modules on two streams, residual add
                                    fused into each module's output projection; a ladder
                                    module overlaps the previous module */
#define LADDER_SCHED_FUSED 3     /* one stream; a ladder layer's (or parallel block's)
                                    attention and MLP run side by side (their inputs
                                    x_{2l-1} and x_{2l} both exist when the layer starts; a
                                    parallel block reads x_{2l} twice).  bf16, row-wave
                                    batches: two launches per layer, [QKV (half of the
                                    workgroups first), then gate/up | the attention once
                                    every QKV share is done] and [down rows, then the O rows
                                    + both residual adds] while the first launch keeps two
                                    workgroups per CU, else as FUSED_LATE_ATTN; fp32:
                                    [QKV | gate/up], [attention | down], [O + both adds]
                                    (default); prefill as DUAL */
#define LADDER_SCHED_PERSISTENT 4 /* decode: the whole layer stack in one launch of resident
                                    workgroups that signal each other (every layer ladder,
                                    bf16, a batch the row-wave GEMV takes, see
                                    ladder_decode_step; otherwise as FUSED); prefill as FUSED */
#define LADDER_SCHED_FUSED_LATE_ATTN 5 /* as FUSED, but with bf16 and a row-wave batch the attention
                                    shares the down projection's launch and the O rows wait
                                    for it there: [QKV | gate/up], [attention | down, then O +
                                    both adds]; prefill as FUSED */

typedef struct ladder_config {
  int32_t n_layers;
  int32_t hidden;          /* H */
  int32_t n_q_heads;       /* per-rank query heads */
  int32_t n_kv_heads;      /* per-rank key/value heads; n_q_heads % n_kv_heads == 0 */
  int32_t head_dim;        /* 64 or 128 */
  int32_t ffn;             /* per-rank SwiGLU width F */
  int32_t vocab;           /* per-rank vocabulary rows of embedding and LM head */
  double rope_theta;       /* pair j of a head rotates by p * theta^(-2j/head_dim) */
  float norm_eps;          /* RMSNorm epsilon (1e-5) */
  int32_t dtype;           /* LADDER_F32 or LADDER_BF16 */
  int32_t max_batch;       /* 1..256 with bf16 weights, 1..16 with fp32 */
  int32_t max_seq;         /* KV capacity per sequence */
  int32_t max_prefill_tokens; /* rows per prefill chunk (B * tokens); 0 = 8192 */
  int32_t kv_filled;       /* KV positions already valid at init (resume on an existing cache) */
  const uint8_t* ladder_mask; /* host, n_layers bytes, copied: 0 = standard layer (each module
                                 reads the residual right before it), 1 = ladder layer (each
                                 module reads the residual one module earlier), 2 = parallel
                                 block (attention and MLP both read the layer input); other
                                 values: LADDER_ERR_ARG */
  /* Rotary frequency scaling of Llama-3.1 checkpoints (the inference code's
   * `apply_rope_scaling`, named on the codewithpapers record of the method's pages, which
   * give no constants; the rule is Llama-3.1's published one, constants 8 / 1 / 4 / 8192).
   * rope_scale_factor 0: off (pair j turns by p * theta^(-2j/head_dim)).  Otherwise, with
   * f = theta^(-2j/head_dim), its wavelength w = 2 pi / f and N = rope_orig_max_pos, pair j
   * turns by p * f' where f' = f for w < N / rope_high_freq_factor, f' = f /
   * rope_scale_factor for w > N / rope_low_freq_factor, and in between f' = (1 - s) f /
   * rope_scale_factor + s f with s = (N / w - rope_low_freq_factor) /
   * (rope_high_freq_factor - rope_low_freq_factor).  Computed in fp64 at init.
   * LADDER_ERR_ARG unless factor >= 1, 0 < low < high (finite) and N > 0. */
  double rope_scale_factor;
  double rope_low_freq_factor;
  double rope_high_freq_factor;
  int32_t rope_orig_max_pos;
} ladder_config;

typedef struct ladder_layer_weights {
  const void* attn_norm;   /* [H] */
  const void* wq;          /* [n_q_heads*head_dim][H] */
  const void* wk;          /* [n_kv_heads*head_dim][H] */
  const void* wv;          /* [n_kv_heads*head_dim][H] */
  const void* wo;          /* [H][n_q_heads*head_dim] */
  const void* mlp_norm;    /* [H] */
  const void* w_gate;      /* [F][H] */
  const void* w_up;        /* [F][H] */
  const void* w_down;      /* [H][F] */
} ladder_layer_weights;

typedef struct ladder_weights {
  const void* tok_embed;   /* [vocab][H] */
  const void* final_norm;  /* [H] */
  const void* lm_head;     /* [vocab][H] */
  const ladder_layer_weights* layers; /* host array of n_layers entries; copied at init */
} ladder_weights;

typedef struct ladder_kv {
  void* k;                 /* [n_layers][max_batch][n_kv_heads][max_seq][head_dim], dtype */
  void* v;                 /* same layout */
} ladder_kv;

typedef struct ladder_ctx ladder_ctx;

/* Validate the configuration, copy the weight/KV pointers and the mask, allocate
 * the workspace and build the RoPE table (fp64 on the host, stored fp32).
 * stream: a hipStream_t of the current device (NULL = the null stream).
 * On success *out receives the context; on error *out is NULL. */
ladder_status ladder_init(const ladder_config* cfg, const ladder_weights* w, const ladder_kv* kv,
                          void* stream, ladder_ctx** out);

/* Prompt processing: d_ids [B][T] int32 at positions start_pos..start_pos+T-1 for
 * sequences (cache slots) 0..B-1.  Writes K/V rows of those positions.  Requires
 * start_pos <= positions already filled and start_pos + T <= max_seq.
 * Outputs (each nullable) are for the last position: d_logits [B][vocab] fp32,
 * d_next [B] int32 (greedy), d_hidden [B][H] fp32 (x_{2L}). */
ladder_status ladder_prefill(ladder_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t T, int32_t start_pos,
                             float* d_logits, int32_t* d_next, float* d_hidden);

/* One decode step: d_ids [B] int32 at position pos (pos <= positions filled,
 * pos < max_seq).  Same outputs as ladder_prefill.  d_ids may alias d_next of the
 * previous step, so a generation loop needs no host synchronisation.  Replays a
 * captured HIP graph per (B, schedule, next-token rule) when graphs are enabled.
 * Batches whose staged projection inputs fit the row-wave GEMV (B <= 4 and
 * B * (K + 8) * 4 bytes <= 150 KB for K the widest of hidden, ffn and
 * n_q_heads * head_dim; at B = 3 and 4 only up to 65 KB, two workgroups per CU; not B = 2
 * for models of hidden >= 8192 whose layers are all ladder or parallel blocks) run the
 * schedule's GEMV launches; other bf16 batches run one token per sequence on the matrix
 * cores (with the split-KV decode attention), under every schedule: up to 32 sequences
 * through skinny weight-streaming launches (a ladder layer in two launches under the
 * FUSED schedules, [QKV + RoPE/KV | attention | gate/up] and [O + down], module by module
 * otherwise, with the same bits), beyond that through tiled GEMMs (under the FUSED
 * schedules a ladder or parallel layer in four launches: [QKV | gate/up], their split-K
 * reduction with RoPE + KV and SwiGLU, [attention | down | O once the attention has
 * signalled], their reduction with both residual adds). */
ladder_status ladder_decode_step(ladder_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t pos,
                                 float* d_logits, int32_t* d_next, float* d_hidden);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ladder_decode_step with the same
 * arguments, checks and outputs (bitwise the same values), enqueued eagerly on the
 * context's stream with the FUSED schedule whatever schedule is selected, whose per-step
 * buffers (residual ring, GEMV split-K partials and counters, attention chunk records,
 * handoff words, logits and argmax partials) live in the library's static scratch: one
 * 64 MiB device array per GPU (LADDER_STATIC_SCRATCH_BYTES), held from the library's
 * load until the process ends, its address looked up by ladder_init.  The call allocates
 * nothing (no hipMalloc or hipFree, no graph, no event) and clears the scratch's counters
 * and flags itself with a kernel.  Every call on one GPU shares that GPU's array, and it
 * keeps the last call's contents: calls that overlap on one GPU (other streams, other
 * contexts) race and give wrong results; calls ordered on one stream are safe.
 * LADDER_ERR_CAPACITY (with the bytes needed in ladder_last_error) when the step at batch
 * B needs more than the array holds; LADDER_ERR_HIP if the address lookup failed. */
#define LADDER_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
ladder_status ladder_decode_step_static(ladder_ctx* ctx, const int32_t* d_ids, int32_t B, int32_t pos,
                                        float* d_logits, int32_t* d_next, float* d_hidden);

/* Select the schedule (LADDER_SCHED_*) and whether decode steps use HIP graphs. */
ladder_status ladder_set_schedule(ladder_ctx* ctx, int32_t schedule, int32_t use_graph);

/* Next-token rule of prefill and decode steps (the inference code's `logits_to_probs`,
 * `multinomial_sample_one_no_sync` and `sample`, named on the codewithpapers record of the
 * method's pages).  temperature <= 0: greedy argmax (the default; top_k and seed ignored).
 * temperature > 0: d_next[b] is drawn from softmax(logits[b] / temperature) over the
 * top_k largest logits (every logit >= the k-th largest; top_k 0 or >= vocab keeps all)
 * by the Gumbel-max rule, argmax_i logits_i / temperature - log(-log U_i), with U_i from
 * Philox4x32-10 (Salmon et al., SC 2011): counter (i / 4, b, pos, 0), key (seed low 32
 * bits, seed high 32 bits), word i % 4, U = (2 (word >> 9) + 1) / 2^24.  pos is the
 * position whose logits are drawn from (the decode step's pos; start_pos + T - 1 in a
 * prefill), so a draw depends only on (seed, pos, b, i).  The logits output is unchanged.
 * LADDER_ERR_ARG: temperature not finite, or top_k < 0.  Drops the cached decode graphs. */
ladder_status ladder_set_sampling(ladder_ctx* ctx, float temperature, int32_t top_k, uint64_t seed);

/* The same draw on caller logits, outside any context: d_next[b] (device, B int32) from
 * d_logits (device, fp32 [B][ld], the first V of each row used) at position pos, with
 * temperature > 0 (finite), top_k >= 0 and seed as in ladder_set_sampling.  Enqueued on
 * `stream` (a hipStream_t, NULL = the null stream); nothing is allocated.  LADDER_ERR_ARG
 * on null pointers, B < 1, V < 1, ld < V, pos < 0 or a bad temperature / top_k;
 * LADDER_ERR_HIP if the launch fails. */
ladder_status ladder_sample(const float* d_logits, int32_t B, int32_t V, int32_t ld, float temperature,
                            int32_t top_k, uint64_t seed, int32_t pos, int32_t* d_next, void* stream);

/* Number of KV positions the context regards as filled. */
ladder_status ladder_filled(const ladder_ctx* ctx, int32_t* out);

/* Device bytes the context allocated for its workspace. */
ladder_status ladder_workspace_bytes(const ladder_ctx* ctx, size_t* out);

/* Wait for all work of the context (its stream and internal streams).  Also reports
 * LADDER_ERR_HIP (sticky) if a decode kernel's bounded wait for another workgroup's
 * signal ever gave up, which does not happen in a correct run. */
ladder_status ladder_sync(ladder_ctx* ctx);

/* Decode kernel kinds, for ladder_time_kernels and ladder_trace_kernel. */
#define LADDER_KERNEL_QKV 0      /* RMSNorm + [Wq;Wk;Wv] GEMV + RoPE + KV append */
#define LADDER_KERNEL_ATTN 1     /* split-KV GQA decode attention (+ chunk merge) */
#define LADDER_KERNEL_OPROJ 2    /* Wo GEMV + fused residual add */
#define LADDER_KERNEL_GATEUP 3   /* RMSNorm + [Wgate,Wup] GEMV + SwiGLU */
#define LADDER_KERNEL_DOWN 4     /* Wdown GEMV + fused residual add */
#define LADDER_KERNEL_LMHEAD 5   /* final RMSNorm + LM head GEMV + greedy argmax */
#define LADDER_KERNEL_QKV_GATEUP 6  /* fused ladder launch: QKV (+RoPE/KV) | gate/up (+SwiGLU); at
                                       33-64 sequences on the matrix cores the tiled split-K launch
                                       of both projections with their reductions (traced, not
                                       replayed by ladder_time_kernels) */
#define LADDER_KERNEL_ATTN_DOWN 7   /* fused ladder launch: decode attention | down projection; with
                                       bf16 weights and a row-wave batch followed, in the same launch, by
                                       the O projection + both residual adds */
#define LADDER_KERNEL_OPROJ_ADD2 8  /* fused ladder launch: O projection + both residual adds (three-
                                       launch layers only) */
#define LADDER_KERNEL_LAYER_STACK 9  /* persistent launch of a decode step's whole layer stack
                                        (LADDER_SCHED_PERSISTENT); ladder_time_kernels stores
                                        -1 where that launch is not available */
#define LADDER_KERNEL_QKV_ATTN_GATEUP 10 /* fused ladder launch (FUSED, bf16): QKV (+RoPE/KV),
                                        gate/up (+SwiGLU) and the split-KV attention once the
                                        QKV outputs are done: at batch 1 the streaming front
                                        launch, at row-wave batches with two workgroups per CU
                                        the sequential launch, at batches 3-32 on the matrix
                                        cores the skinny [QKV | attention | gate/up] launch; -1
                                        from ladder_time_kernels where not available */
#define LADDER_KERNEL_DOWN_OPROJ 11  /* fused ladder launch (the same layers): down rows, then
                                        the O rows + both residual adds (at 33-64 sequences on
                                        the matrix cores the tiled [attention | down | O] launch
                                        and its reduction, traced only); -1 where not
                                        available */
#define LADDER_KERNEL_SAMPLE 12   /* stochastic draw from the logits (ladder_set_sampling); timed
                                        with the context's sampling settings, or temperature 1
                                        and no top-k cut when sampling is off */
#define LADDER_N_KERNELS 13

/* Profiling aid.  For each kernel kind, enqueue it on the context's stream exactly as
 * a decode step at batch B launches it (once per layer; the LM head once), once untimed
 * and then reps times (the GEMV kinds at B <= 16 only; -1 beyond; at a batch that runs on
 * the matrix cores only the kinds such a step launches: QKV_ATTN_GATEUP as its
 * [QKV | attention | gate/up] launch (batches up to 32), QKV_GATEUP as the same launch
 * without the attention, DOWN_OPROJ as its [O + down] launch, ATTN as the attention launched
 * alone, LMHEAD and SAMPLE, -1 for the others),
 * (the fused kinds use each layer as if it were a ladder layer),
 * between two HIP events, and store the mean duration of one launch in microseconds
 * in us_out[kind] (host array of LADDER_N_KERNELS floats).  Works on the context's
 * current buffers and the position of the last decode step, whose KV row it
 * overwrites; requires at least one filled position.  Blocks until done. */
ladder_status ladder_time_kernels(ladder_ctx* ctx, int32_t B, int32_t reps, float* us_out);

/* Measurement aid: the HBM streaming-read ceiling of the current device.  Reads a
 * bytes-sized device buffer (allocated and freed here; >= 1 MiB) with plain 16-byte
 * loads, reps times for each of 2, 4 and 8 workgroups per CU, on `stream` (a
 * hipStream_t, NULL = the null stream), and stores the best rate in GB/s (1e9 B/s) in
 * *gbs_out.  Blocks until done.  LADDER_ERR_OOM if the buffer cannot be allocated. */
ladder_status ladder_read_probe(void* stream, size_t bytes, int32_t reps, float* gbs_out);

/* Measurement aid.  kind in [0, LADDER_N_KERNELS): from the next decode step on, every
 * launch of that kernel kind gets a pair of HIP events on the stream it runs on, taken
 * from the dispatch's own begin and end timestamps (hipExtLaunchKernelGGL; for a kind
 * made of two kernels, the first one's begin and the last one's end).  While a kind is
 * traced, decode steps are launched eagerly: the same kernels with the same arguments,
 * without a HIP graph.  kind = -1 turns it off.  Creates 2 (n_layers + 1) events on
 * first use.  LADDER_ERR_ARG for another kind. */
ladder_status ladder_trace_kernel(ladder_ctx* ctx, int32_t kind);

/* Mean duration in microseconds (*mean_us) and number (*count) of the traced launches
 * of the most recently enqueued decode step; waits for the context's stream.
 * LADDER_ERR_STATE if tracing is off or no decode step ran since it was turned on. */
ladder_status ladder_trace_result(ladder_ctx* ctx, float* mean_us, int32_t* count);

/* Release the context (NULL is a no-op).  Does not free caller buffers. */
void ladder_free(ladder_ctx* ctx);

/* Static description of a status code. */
const char* ladder_status_string(ladder_status s);

/* Text of the last error recorded by the context (empty if none). */
const char* ladder_last_error(const ladder_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* LADDER_H */

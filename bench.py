#!/usr/bin/env python3
"""Throughput of the Ladder Residual Transformer forward step on one MI355X.

Default workload: one tensor-parallel rank's shard of a 70B-shape model (TP=8: 80 ladder
layers, hidden 8192, 8 query heads + 1 kv head of 128, ffn 3584, vocab 16032, bf16),
batch 1, 1024-token prompt, decode steps at positions 1024.. .  One "step" is one
decode step: every module of every layer (RMSNorm, QKV + RoPE + KV append, GQA
attention, O projection, SwiGLU MLP, ladder residual adds), then the LM head and the
greedy argmax.  Weights are random N(0, 0.02) from a fixed seed and the prompt is
uniform random ids (synthetic data of the workload's shape).

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tok/s + % HBM roofline, 70B-shape TP8 one-rank shard, batch 1"
HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15      # FLOP/s, dense bf16
CSRC = "ladder_residual_transformer_amd/csrc/"
# the kernel each schedule's roofline reports: (trace kind, description, traffic file, sources)
DOMINANT = {
    "fused": ("qkv_attn_gateup", "front launch of a ladder layer [RMSNorm+QKV+RoPE+KV, then RMSNorm+gate/up+"
              "SwiGLU, in every workgroup | split-KV GQA attention chunks once their kv group's QKV outputs "
              "arrive]; at batch 1 the streaming launch (stream.hip), at batches 3-32 the skinny "
              "[QKV | attention | gate/up] launch (skinny.hip), else the row-wave one",
              "traffic_qkv_attn_gateup_70b_b1.json",
              ("stream.hip", "gemv_rw.hip", "gemv_rw.hpp", "skinny.hip", "attn_decode.hpp", "common.hpp")),
    # FUSED without the bf16 two-launch layers, and the schedule with the attention in the
    # down projection's launch: the [QKV | gate/up] launch
    "fused3": ("qkv_gateup", "fused ladder launch [RMSNorm+QKV | RMSNorm+gate/up+SwiGLU]: the row-wave launch "
               "(RoPE+KV in its epilogue) or, at batches on the matrix cores without the attention in the "
               "launch, the skinny weight-streaming launch (skinny.hip), or at 33-64 sequences the tiled "
               "split-K launch of both projections with their two reductions (gemm.hip)",
               "traffic_qkv_gateup_70b_b1.json",
               ("gemv_rw.hip", "gemv_rw.hpp", "attn_decode.hpp", "common.hpp")),
    "persistent": ("layer_stack", "persistent decode launch of the whole layer stack (every projection, "
                   "attention and residual add of every layer)", "traffic_layer_stack_70b_b1.json",
                   ("decode_step.hip", "gemv_rw.hpp", "attn_decode.hpp", "common.hpp")),
    # module-by-module schedules and all-standard stacks: the MLP's gate/up launch
    "module": ("gateup", "RMSNorm+gate/up+SwiGLU launch of each MLP module", None, ()),
}
LAYER_KINDS = {"standard": 0, "ladder": 1, "parallel": 2}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha(sources) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, CSRC + rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(cfg, B, pos):
    """Algorithmic HBM bytes of one decode step at position pos: every layer weight, the
    final norm and the LM head once, one embedding row per sequence, the KV rows 0..pos
    read and row pos written."""
    esz = 2 if cfg.dtype == "bf16" else 4
    kv_row = B * cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * esz
    return cfg.decode_weight_bytes(B) + kv_row * (pos + 1) + kv_row


def prefill_flops(cfg, B, T):
    H, F, hd = cfg.hidden, cfg.ffn, cfg.head_dim
    q, kv = cfg.n_q_heads * hd, cfg.n_kv_heads * hd
    proj = 2 * cfg.n_layers * (H * (q + 2 * kv) + q * H + 3 * H * F) * B * T
    attn = cfg.n_layers * B * cfg.n_q_heads * 4 * hd * (T * (T + 1) // 2)
    head = 2 * cfg.vocab * H * B
    return proj + attn + head


def qkv_gateup_bytes(cfg, B):
    """Algorithmic bytes of one fused [QKV | gate/up] launch: both weight blocks and norm
    gains once, the two input residual rows, q and the SwiGLU output written, one K and
    one V row appended per kv head (the skinny launch writes the K and V rows in fp32 for
    the RoPE kernel instead; the weights are 99.9% of either count)."""
    esz = 2 if cfg.dtype == "bf16" else 4
    H, F, hd = cfg.hidden, cfg.ffn, cfg.head_dim
    q, kv = cfg.n_q_heads * hd, cfg.n_kv_heads * hd
    weights = (H * (q + 2 * kv) + 2 * F * H + 2 * H) * esz
    return weights + 2 * B * H * 4 + B * q * 4 + B * F * 4 + 2 * B * kv * esz


def qkv_attn_gateup_bytes(cfg, B, pos):
    """Algorithmic bytes of one front launch [QKV, then gate/up | attention] at position
    pos: those of [QKV | gate/up], plus the attention's reads of q and of the KV rows
    0..pos (the newest one just written) and its output written (at batch 1 the launch
    leaves per-chunk records that the back launch merges into that output; the count is
    the method's, B * nq * hd * 4 bytes, 0.003% of the launch)."""
    esz = 2 if cfg.dtype == "bf16" else 4
    q, kv = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    return qkv_gateup_bytes(cfg, B) + 2 * B * q * 4 + 2 * B * kv * esz * (pos + 1)


def gateup_bytes(cfg, B):
    """Algorithmic bytes of one gate/up launch: both weight blocks and the norm gain once,
    the input residual row read and the SwiGLU output written."""
    esz = 2 if cfg.dtype == "bf16" else 4
    H, F = cfg.hidden, cfg.ffn
    return (2 * F * H + H) * esz + B * H * 4 + B * F * 4


def layer_stack_bytes(cfg, B, pos):
    """Algorithmic bytes of the whole layer stack of one decode step at position pos:
    every layer's weights and norm gains once, its KV rows 0..pos read and row pos
    written, and per layer the two residual rows read and written, q, the attention
    output and the SwiGLU output written once and read once."""
    esz = 2 if cfg.dtype == "bf16" else 4
    H, F, hd = cfg.hidden, cfg.ffn, cfg.head_dim
    q, kv = cfg.n_q_heads * hd, cfg.n_kv_heads * hd
    weights = (H * (q + 2 * kv) + q * H + 3 * F * H + 2 * H) * esz
    kv_rows = 2 * B * kv * esz * (pos + 2)
    acts = 4 * B * H * 4 + 2 * B * q * 4 * 2 + 2 * B * F * 4
    return cfg.n_layers * (weights + kv_rows + acts)


def cpu_baseline(cfg, w, prompt, sample_layers, steps):
    """The oracle (numpy float32) on a bounded sample: `sample_layers` real-width layers
    plus the LM head; decode time per token extrapolated to the full depth."""
    import numpy as np
    import synth
    from oracle import LadderOracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sub = synth.scaled_config(cfg, sample_layers)
    ws = synth.ModelWeights(w.dtype, w.tok_embed, w.final_norm, w.lm_head, w.layers[:sample_layers])
    o = LadderOracle(sub, ws, dtype=np.float32, cache_weights=True)
    cache = o.new_cache()
    B, T = prompt.shape
    t0 = time.perf_counter()
    r = o.forward(prompt, cache, 0, logits="last")
    t_prefill = time.perf_counter() - t0
    tok = np.argmax(r.logits[:, -1], axis=-1)
    o.forward(tok[:, None], cache, T, logits="last")          # warm (weights cached)
    t0 = time.perf_counter()
    for k in range(steps):
        r = o.forward(tok[:, None], cache, T + 1 + k, logits=None)
    t_layers = (time.perf_counter() - t0) / steps
    hd = o.head()
    t0 = time.perf_counter()
    for _ in range(steps):
        from oracle import rms_norm
        np.matmul(rms_norm(r.hidden[:, -1], hd["final_norm"], cfg.norm_eps), hd["lm_head"].T)
    t_head = (time.perf_counter() - t0) / steps
    per_token = t_layers * cfg.n_layers / sample_layers + t_head
    return {"value": B / per_token, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": sample_layers < cfg.n_layers, "layers_timed": sample_layers,
            "layers_total": cfg.n_layers,
            "sample": (f"numpy float32 oracle, {sample_layers} of {cfg.n_layers} layers at full width plus the LM "
                       f"head, {steps} decode steps at KV length {T + 1}, per-token time scaled by "
                       f"{cfg.n_layers}/{sample_layers} for the layer stack; prefill of the {T}-token prompt "
                       f"over the sample took {t_prefill:.1f} s"),
            "prefill_tok_s_extrapolated": B * T / (t_prefill * cfg.n_layers / sample_layers)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="70b_tp8_shard")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--schedule", choices=("serial", "side", "dual", "fused", "persistent", "fused_late_attn"),
                    default="fused")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--layers", choices=("workload",) + tuple(LAYER_KINDS), default="workload",
                    help="layer kind of every layer: the workload's own mask (default; the 70B shard is "
                         "all ladder), or all standard, all ladder, or all parallel blocks")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: next tokens drawn from softmax(logits / T) (Gumbel-max, seeded) instead of greedy")
    ap.add_argument("--top-k", type=int, default=0, help="with --temperature: keep only the k largest logits")
    ap.add_argument("--prefill-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-layers", type=int, default=16)
    ap.add_argument("--cpu-steps", type=int, default=6)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device-to-device copy of MB megabytes 5 times (the reference "
                         "for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs one GPU's share of the model (one tensor-parallel rank's shard); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe * 1000 * 1000 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 5}))
        return

    import synth
    from ladder_residual_transformer_amd import DeviceWeights, LadderModel, load

    load()
    wl = synth.WORKLOADS[args.workload]
    cfg = wl.model
    if args.layers != "workload":
        mask = (LAYER_KINDS[args.layers],) * cfg.n_layers
        if mask != tuple(cfg.ladder_mask):
            cfg = cfg.with_mask(mask, name=f"{cfg.name} ({args.layers} layers)")
    B, P = args.batch, wl.prompt_len
    if args.steps < 1 or args.warmup < 0 or max(args.steps, args.warmup) > wl.decode_len:
        sys.exit(f"steps and warmup must be within the {wl.decode_len} decode positions")
    torch.cuda.set_device(0)
    t = time.time()
    w = synth.gen_weights(cfg, seed=0)
    log(f"[bench] generated {cfg.weight_bytes() / 1e9:.2f} GB of {cfg.name} weights in {time.time() - t:.1f} s")
    t = time.time()
    dw = DeviceWeights(w)
    model = LadderModel(cfg, dw, B, wl.max_seq)
    sched = {"serial": 0, "side": 1, "dual": 2, "fused": 3, "persistent": 4, "fused_late_attn": 5}[args.schedule]
    model.set_schedule(sched, not args.no_graph)
    if args.temperature > 0:
        model.set_sampling(args.temperature, args.top_k, seed=0)
    torch.cuda.synchronize()
    log(f"[bench] uploaded weights and built the context in {time.time() - t:.1f} s "
        f"(workspace {model.workspace_bytes() / 1e6:.0f} MB)")
    prompt = synth.gen_ids(B, P, cfg.vocab, seed=1)
    ids = torch.from_numpy(prompt).cuda()

    # ---- prefill
    _, first, _ = model.prefill(ids, logits=False, hidden=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.prefill_reps):
        _, first, _ = model.prefill(ids, logits=False, hidden=False)
    torch.cuda.synchronize()
    prefill_s = (time.perf_counter() - t0) / args.prefill_reps
    pflops = prefill_flops(cfg, B, P)
    log(f"[bench] prefill {B}x{P}: {prefill_s * 1e3:.1f} ms, {B * P / prefill_s:.0f} tok/s, "
        f"{pflops / prefill_s / 1e12:.1f} TFLOP/s")

    # ---- decode: W untimed steps, then exactly K timed steps (positions P..)
    bufs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(2)]
    bufs[0].copy_(first)
    cur = bufs[0]
    for k in range(args.warmup):
        model.decode_step(cur, P + k, out=(None, bufs[(k + 1) % 2], None))
        cur = bufs[(k + 1) % 2]
    torch.cuda.synchronize()
    bufs[0].copy_(first)
    cur = bufs[0]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for k in range(args.steps):
        model.decode_step(cur, P + k, out=(None, bufs[(k + 1) % 2], None))
        cur = bufs[(k + 1) % 2]
    e1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    model.sync()
    gpu_ms = e0.elapsed_time(e1)
    toks = cur.cpu().numpy()
    assert np.all((toks >= 0) & (toks < cfg.vocab)), "decode produced an out-of-range token id"
    tok_s = B * args.steps / dt
    total_bytes = sum(decode_bytes(cfg, B, P + k) for k in range(args.steps))
    hbm_frac = total_bytes / dt / HBM_PEAK
    log(f"[bench] decode {args.steps} steps: {dt * 1e3 / args.steps:.3f} ms/step (events {gpu_ms / args.steps:.3f}), "
        f"{tok_s:.1f} tok/s, {total_bytes / args.steps / 1e9:.2f} GB/step, {100 * hbm_frac:.1f}% of HBM peak")

    # ---- the dominant kernel, measured live: the same K decode steps again, each launch
    # of that kernel with a pair of HIP events on the stream it runs on, taken from its
    # dispatch's own begin/end timestamps (traced steps are launched eagerly).  Fused
    # schedule: the [QKV, then gate/up | attention] launch of every layer (~80% of the
    # step's bytes; [QKV | gate/up] where the attention has a launch of its own, and under the
    # schedule with the attention in the down projection's launch); persistent schedule:
    # the one launch of the whole layer stack.  Which of them a step launches depends on
    # the shape (the two-launch layers need the staged input rows to fit in LDS), so the
    # candidates are probed in order with one traced step.
    from ladder_residual_transformer_amd import LadderError
    cands = {"persistent": ("persistent", "fused", "fused3", "module"), "fused": ("fused", "fused3", "module"),
             "fused_late_attn": ("fused3", "module")}.get(args.schedule, ("module",))
    dom = None
    for c in cands:
        model.trace_kernel(DOMINANT[c][0])
        bufs[0].copy_(first)
        model.decode_step(bufs[0], P, out=(None, bufs[1], None))
        try:
            if model.trace_result()[1] > 0:
                dom = c
                break
        except LadderError:
            pass
    if dom is None:
        sys.exit("bench.py: no launch of a dominant kernel kind in a traced step")
    kind, kdesc, tfile, ksrc = DOMINANT[dom]
    model.trace_kernel(kind)
    bufs[0].copy_(first)
    model.decode_step(bufs[0], P, out=(None, bufs[1], None))
    torch.cuda.synchronize()
    cur = bufs[0]
    tot_us, n_launch, tot_bytes = 0.0, 0, 0
    t0 = time.perf_counter()
    for k in range(args.steps):
        model.decode_step(cur, P + k, out=(None, bufs[(k + 1) % 2], None))
        cur = bufs[(k + 1) % 2]
        us, n = model.trace_result()                # waits for the step
        tot_us += us * n
        n_launch += n
        tot_bytes += n * {"layer_stack": lambda: layer_stack_bytes(cfg, B, P + k),
                          "qkv_gateup": lambda: qkv_gateup_bytes(cfg, B),
                          "qkv_attn_gateup": lambda: qkv_attn_gateup_bytes(cfg, B, P + k),
                          "gateup": lambda: gateup_bytes(cfg, B)}[kind]()
    torch.cuda.synchronize()
    dt_traced = time.perf_counter() - t0
    if n_launch == 0:
        sys.exit(f"bench.py: no {kind} launch in the traced steps")
    us_launch = tot_us / n_launch
    bytes_launch = tot_bytes / n_launch
    model.trace_kernel(None)
    achieved = bytes_launch / (us_launch * 1e-6) / 1e9
    log(f"[bench] traced decode: {dt_traced * 1e3 / args.steps:.3f} ms/step (read out per step); {kind} "
        f"launch {us_launch:.2f} us mean over {n_launch} launches, {achieved:.0f} GB/s")
    traffic = None
    tpath = os.path.join(ROOT, "profiles", tfile) if tfile else None
    if tpath and os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("kernel_sha") == kernel_sha(ksrc) and tr.get("batch") == B and tr.get("workload") == cfg.name:
            traffic = tr.get("bytes_per_launch")

    # every kernel kind replayed in isolation (diagnostic)
    ku = model.time_kernels(B, reps=3)
    log(f"[bench] kernel us/launch in isolation: " + ", ".join(f"{k} {v:.2f}" for k, v in ku.items()))

    # the part's measured streaming-read ceiling (a plain read kernel over 4 GiB)
    from ladder_residual_transformer_amd import abi
    ceiling = abi.ladder_read_probe(torch.cuda.current_stream().cuda_stream, 4 << 30, 5)
    log(f"[bench] streaming-read ceiling {ceiling:.0f} GB/s ({100 * ceiling * 1e9 / HBM_PEAK:.1f}% of the 8 TB/s peak)")

    cpu = None
    if not args.no_cpu_baseline:
        t = time.time()
        cpu = cpu_baseline(cfg, w, prompt, min(args.cpu_sample_layers, cfg.n_layers), args.cpu_steps)
        log(f"[bench] cpu baseline {cpu['value']:.4f} tok/s on {cpu['cores']} threads ({time.time() - t:.1f} s)")

    out = {
        "metric": METRIC, "value": round(tok_s, 3), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dt * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}, batch {B}, prompt {P}, decode positions {P}..{P + args.steps - 1}",
                   "batch": B, "prompt_len": P, "layers": cfg.n_layers, "hidden": cfg.hidden,
                   "schedule": args.schedule, "hip_graph": not args.no_graph,
                   "next_token": ({"rule": "sample", "temperature": args.temperature, "top_k": args.top_k, "seed": 0}
                                  if args.temperature > 0 else {"rule": "greedy"}),
                   "layer_kinds": {k: sum(1 for v in cfg.ladder_mask if v == c) for k, c in LAYER_KINDS.items()}},
        "decode_hbm_frac": round(hbm_frac, 4),
        "decode_bytes_per_step": total_bytes // args.steps,
        "prefill_tok_s": round(B * P / prefill_s, 1),
        "prefill_mfma_frac": round(pflops / prefill_s / MFMA_BF16_PEAK, 4),
        "roofline": {"bound": "hbm", "kernel": kdesc,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": traffic,
                     "bytes_per_launch": int(bytes_launch), "us_per_launch": round(us_launch, 3),
                     "launches_timed": n_launch, "traced_ms_per_step": round(dt_traced * 1e3 / args.steps, 4),
                     "read_ceiling_gbs": round(ceiling, 1),
                     "frac_of_read_ceiling": round(achieved / ceiling, 4)},
        "kernels_us_isolated": {k: round(v, 3) for k, v in ku.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.free()


if __name__ == "__main__":
    main()

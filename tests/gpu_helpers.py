"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import synth
from oracle import LadderOracle, greedy_generate

TOL = {"f32": 1e-5, "bf16": 1e-2}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| (the parity metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def step_rel_err(got, ref) -> float:
    """The parity metric per step, worst step: arrays [B, steps, X], one step = all B rows."""
    return max(rel_err(got[:, k], ref[:, k]) for k in range(ref.shape[1]))


def small_config(name, base: synth.ModelConfig, **changes) -> synth.ModelConfig:
    return dataclasses.replace(base, name=name, **changes)


def make_model(cfg, weights, max_batch, max_seq, **kw):
    from ladder_residual_transformer_amd import DeviceWeights, LadderModel
    dw = DeviceWeights(weights)
    return LadderModel(cfg, dw, max_batch, max_seq, **kw)


def gpu_teacher_forced(model, prompt: np.ndarray, cont: np.ndarray):
    """Prefill ``prompt`` then decode ``cont`` [B, n] one token per step (ids given).

    Returns logits [B, n+1, V], hidden [B, n+1, H] and argmax tokens [B, n+1]:
    index 0 from the prefill (last prompt position), index k from decode step k.
    """
    B, T = prompt.shape
    ids = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    lg, nx, hd = model.prefill(ids)
    logits, hidden, nxt = [lg], [hd], [nx]
    for k in range(cont.shape[1]):
        step = torch.from_numpy(np.ascontiguousarray(cont[:, k], dtype=np.int32)).cuda()
        lg, nx, hd = model.decode_step(step, T + k)
        logits.append(lg)
        hidden.append(hd)
        nxt.append(nx)
    torch.cuda.synchronize()
    model.sync()                  # also reports a failed in-kernel wait
    return (torch.stack(logits, 1).cpu().numpy(), torch.stack(hidden, 1).cpu().numpy(),
            torch.stack(nxt, 1).cpu().numpy())


def gpu_free_running(model, prompt: np.ndarray, n_decode: int):
    """Greedy generation feeding each step's own device-side argmax back (no host sync)."""
    B, T = prompt.shape
    ids = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    lg, nx, hd = model.prefill(ids)
    toks = [nx]
    for k in range(n_decode):
        lg, nx, hd = model.decode_step(toks[-1], T + k, logits=False, hidden=False)
        toks.append(nx)
    torch.cuda.synchronize()
    model.sync()
    return torch.stack(toks, 1).cpu().numpy()


def check_against_oracle(cfg, gl, gh, gt, ref: dict, tol: float, label: str):
    """Compare GPU logits/hidden/argmax with the oracle's greedy record (same tokens fed).

    Argmax must agree at every step whose oracle top-1/top-2 margin exceeds twice the
    measured logit error; closer steps are reported as near-ties.
    """
    n = ref["logits"].shape[1]
    worst_l = worst_h = 0.0
    near = 0
    for k in range(n):
        el = rel_err(gl[:, k], ref["logits"][:, k])
        eh = rel_err(gh[:, k], ref["hidden"][:, k])
        worst_l, worst_h = max(worst_l, el), max(worst_h, eh)
        abs_err = np.max(np.abs(gl[:, k] - ref["logits"][:, k]))
        for b in range(gt.shape[0]):
            if gt[b, k] != ref["tokens"][b, k]:
                assert ref["margins"][b, k] <= 2 * abs_err, (
                    f"{label}: step {k} row {b}: token {gt[b, k]} != {ref['tokens'][b, k]} "
                    f"with margin {ref['margins'][b, k]:.3g} > 2*err {abs_err:.3g}")
                near += 1
    log(f"{label}: max rel err logits {worst_l:.3g} hidden {worst_h:.3g} near-ties {near}")
    assert worst_l <= tol, f"{label}: logits rel err {worst_l}"
    assert worst_h <= tol, f"{label}: hidden rel err {worst_h}"
    return worst_l, worst_h


def oracle_record(cfg, weights, prompt, n_decode, dtype=np.float64, cache_weights=True):
    o = LadderOracle(cfg, weights, dtype=dtype, cache_weights=cache_weights)
    return greedy_generate(o, prompt, n_decode)

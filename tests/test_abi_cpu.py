"""The C ABI library without a GPU: it loads, exports every declared entry point, and
rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest
import torch

import ladder_residual_transformer_amd as L
from ladder_residual_transformer_amd import abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ladder.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ladder_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = L.load()
    names = declared_functions()
    assert {"ladder_init", "ladder_prefill", "ladder_decode_step", "ladder_free"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(abi.EXPORTED)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("LADDER_OK", "LADDER_ERR_ARG", "LADDER_ERR_SHAPE", "LADDER_ERR_CAPACITY", "LADDER_ERR_STATE",
                 "LADDER_ERR_HIP", "LADDER_ERR_OOM", "LADDER_F32", "LADDER_BF16", "LADDER_SCHED_SERIAL",
                 "LADDER_SCHED_SIDE", "LADDER_SCHED_DUAL", "LADDER_SCHED_FUSED",
                 "LADDER_SCHED_PERSISTENT", "LADDER_SCHED_FUSED_LATE_ATTN", "LADDER_KERNEL_LAYER_STACK",
                 "LADDER_KERNEL_QKV_ATTN_GATEUP", "LADDER_KERNEL_DOWN_OPROJ", "LADDER_KERNEL_SAMPLE",
                 "LADDER_N_KERNELS"):
        m = re.search(r"#define\s+%s\s+\(?(-?\d+)\)?" % name, text)
        assert m, name
        assert int(m.group(1)) == getattr(abi, name), name


def test_struct_layout():
    """The ctypes structs lay out like the C header, as gcc compiles it."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    fields = [f[0] for f in abi.ladder_config._fields_]
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"ladder.h\"\nint main(void) {\n"
    src += '  printf("%zu\\n", sizeof(ladder_config));\n'
    src += "".join('  printf("%%zu\\n", offsetof(ladder_config, %s));\n' % f for f in fields)
    src += '  printf("%zu %zu\\n", sizeof(ladder_layer_weights), sizeof(ladder_weights));\n  return 0;\n}\n'
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        with open(c, "w") as fh:
            fh.write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    assert int(out[0]) == ctypes.sizeof(abi.ladder_config)
    for f, off in zip(fields, out[1:1 + len(fields)]):
        assert int(off) == getattr(abi.ladder_config, f).offset, f
    assert int(out[-2]) == ctypes.sizeof(abi.ladder_layer_weights) == 9 * 8
    assert int(out[-1]) == ctypes.sizeof(abi.ladder_weights) == 32


FAKE = 0x100000


def make_args(n_layers=2, hidden=256, nq=4, nkv=2, hd=64, ffn=688, vocab=1024, dtype=0, max_batch=1, max_seq=32,
              mask=None, ptr=FAKE, rope=(0.0, 0.0, 0.0, 0)):
    m = (ctypes.c_uint8 * n_layers)(*(mask or [1] * n_layers))
    cfg = abi.ladder_config(n_layers, hidden, nq, nkv, hd, ffn, vocab, 1e4, 1e-5, dtype, max_batch, max_seq, 0, 0,
                            ctypes.cast(m, ctypes.POINTER(ctypes.c_uint8)), *rope)
    layers = (abi.ladder_layer_weights * n_layers)()
    for i in range(n_layers):
        for f, _ in abi.ladder_layer_weights._fields_:
            setattr(layers[i], f, ptr)
    w = abi.ladder_weights(ptr, ptr, ptr, layers)
    kv = abi.ladder_kv(ptr, ptr)
    return cfg, w, kv, (m, layers)


def init_status(cfg, w, kv):
    out = ctypes.c_void_p(123)
    st = L.load().ladder_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("change, status", [
    (dict(hd=96), abi.LADDER_ERR_SHAPE),
    (dict(max_batch=17), abi.LADDER_ERR_SHAPE),         # fp32: the K-sliced GEMV takes at most 16 rows
    (dict(dtype=1, ffn=704, max_batch=257), abi.LADDER_ERR_SHAPE),   # bf16: at most 256 sequences
    (dict(nq=6, nkv=4), abi.LADDER_ERR_SHAPE),
    (dict(nq=34, nkv=2), abi.LADDER_ERR_SHAPE),        # more than 16 query heads per kv head
    (dict(hidden=258), abi.LADDER_ERR_SHAPE),          # not a whole number of 16-byte vectors
    (dict(dtype=1, ffn=688), abi.LADDER_ERR_SHAPE),    # bf16 prefill needs K % 64 == 0
    (dict(dtype=2), abi.LADDER_ERR_ARG),
    (dict(n_layers=0), abi.LADDER_ERR_ARG),
    (dict(max_seq=0), abi.LADDER_ERR_ARG),
    (dict(mask=[1, 3]), abi.LADDER_ERR_ARG),           # 0 standard, 1 ladder, 2 parallel only
    (dict(ptr=FAKE + 2), abi.LADDER_ERR_ARG),          # misaligned weight pointer
    (dict(rope=(0.5, 1.0, 4.0, 8192)), abi.LADDER_ERR_ARG),   # RoPE scaling factor below 1
    (dict(rope=(8.0, 4.0, 1.0, 8192)), abi.LADDER_ERR_ARG),   # low_freq_factor >= high_freq_factor
    (dict(rope=(8.0, 0.0, 4.0, 8192)), abi.LADDER_ERR_ARG),   # low_freq_factor not positive
    (dict(rope=(8.0, 1.0, 4.0, 0)), abi.LADDER_ERR_ARG),      # no original context length
    (dict(rope=(float("nan"), 1.0, 4.0, 8192)), abi.LADDER_ERR_ARG),
])
def test_init_rejects_bad_arguments(change, status):
    cfg, w, kv, keep = make_args(**change)
    st, out = init_status(cfg, w, kv)
    assert st == status
    assert out is None


def test_init_null_pointers():
    cfg, w, kv, keep = make_args()
    out = ctypes.c_void_p()
    lib = L.load()
    assert lib.ladder_init(None, ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(out)) == abi.LADDER_ERR_ARG
    assert lib.ladder_init(ctypes.byref(cfg), None, ctypes.byref(kv), None, ctypes.byref(out)) == abi.LADDER_ERR_ARG
    assert lib.ladder_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), None, None) == abi.LADDER_ERR_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
@pytest.mark.parametrize("mask, rope", [(None, (0.0, 0.0, 0.0, 0)), ([2, 0], (0.0, 0.0, 0.0, 0)),
                                        ([0, 2, 1], (0.0, 0.0, 0.0, 0)), (None, (8.0, 1.0, 4.0, 8192)),
                                        (None, (1.0, 1.0, 4.0, 8192))])
def test_valid_config_without_device_reports_hip_error(mask, rope):
    cfg, w, kv, keep = make_args(n_layers=len(mask) if mask else 2, mask=mask, rope=rope)
    st, out = init_status(cfg, w, kv)
    assert st == abi.LADDER_ERR_HIP and out is None


def test_null_context_calls():
    lib = L.load()
    assert lib.ladder_prefill(None, None, 1, 1, 0, None, None, None) == abi.LADDER_ERR_ARG
    assert lib.ladder_decode_step(None, None, 1, 0, None, None, None) == abi.LADDER_ERR_ARG
    assert lib.ladder_decode_step_static(None, None, 1, 0, None, None, None) == abi.LADDER_ERR_ARG
    assert lib.ladder_set_schedule(None, 0, 0) == abi.LADDER_ERR_ARG
    assert lib.ladder_set_sampling(None, 1.0, 0, 0) == abi.LADDER_ERR_ARG
    # argument errors of the context-free draw are found before anything is launched
    fake = ctypes.c_void_p(FAKE)
    assert lib.ladder_sample(None, 1, 8, 8, 1.0, 0, 0, 0, fake, None) == abi.LADDER_ERR_ARG      # no logits
    assert lib.ladder_sample(fake, 1, 8, 8, 1.0, 0, 0, 0, None, None) == abi.LADDER_ERR_ARG      # no output
    assert lib.ladder_sample(fake, 0, 8, 8, 1.0, 0, 0, 0, fake, None) == abi.LADDER_ERR_ARG      # B < 1
    assert lib.ladder_sample(fake, 1, 8, 7, 1.0, 0, 0, 0, fake, None) == abi.LADDER_ERR_ARG      # ld < V
    assert lib.ladder_sample(fake, 1, 8, 8, 0.0, 0, 0, 0, fake, None) == abi.LADDER_ERR_ARG      # T = 0
    assert lib.ladder_sample(fake, 1, 8, 8, float("inf"), 0, 0, 0, fake, None) == abi.LADDER_ERR_ARG
    assert lib.ladder_sample(fake, 1, 8, 8, 1.0, -1, 0, 0, fake, None) == abi.LADDER_ERR_ARG     # top_k < 0
    assert lib.ladder_sample(fake, 1, 8, 8, 1.0, 0, 0, -1, fake, None) == abi.LADDER_ERR_ARG     # pos < 0
    assert lib.ladder_sync(None) == abi.LADDER_ERR_ARG
    assert lib.ladder_trace_kernel(None, 0) == abi.LADDER_ERR_ARG
    assert lib.ladder_trace_result(None, None, None) == abi.LADDER_ERR_ARG
    g = ctypes.c_float()
    assert lib.ladder_read_probe(None, 1 << 20, 1, None) == abi.LADDER_ERR_ARG      # no output
    assert lib.ladder_read_probe(None, 1 << 20, 0, ctypes.byref(g)) == abi.LADDER_ERR_ARG   # no repetition
    assert lib.ladder_read_probe(None, 4096, 1, ctypes.byref(g)) == abi.LADDER_ERR_ARG     # below 1 MiB
    lib.ladder_free(None)                                  # no-op
    assert lib.ladder_last_error(None) == b""


def test_status_strings():
    assert L.status_string(0) == "ok"
    assert "capacity" in L.status_string(abi.LADDER_ERR_CAPACITY)
    assert L.status_string(99) == "unknown status"

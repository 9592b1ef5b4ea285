"""Oracle: a plain, slow CPU reference of the Ladder Residual Transformer forward step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
GPU library; the only thing both sides consume in common is the seeded inputs
of ``synth``, which this package does not import.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (a library routine, a closed form, an invariant or a brute
force expansion); the pin is named in each docstring.
"""
from .ladder import (  # noqa: F401
    LadderOracle,
    ForwardResult,
    upcast,
    round_to_storage,
    rms_norm,
    rope_angles,
    rope_inv_freq,
    llama3_scale_inv_freq,
    apply_rope,
    gqa_attention,
    silu,
    swiglu_mlp,
    module_input_index,
    greedy_generate,
    teacher_forced,
)
from .sampling import (  # noqa: F401
    philox4x32,
    sampling_uniforms,
    topk_keep,
    sampling_probs,
    sample_scores,
    sample_token,
    sample_rows,
)

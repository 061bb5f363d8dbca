"""CPU oracle of the W4A4 quantized linear: zigzag permutation, composite SVD.Hadamard block
rotation, symmetric int4 RTN / per-step / per-token quantization, integer GEMM and dequantization;
the same steps on the int8 grid for the W8A8 linears (``bits=8``); group-wise (per rotation block)
per-step activation scales with their block-wise GEMM (``*_grouped``, linear mode "per_block");
the GPTQ weight solver (``gptq_*``).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package. It shares no code with the GPU library and never imports
it; the GPU library never imports this package.

Parity unpinned: none of the functions here. Each is pinned by the CPU tests (closed forms,
library routines, brute force and invariants); see the test module docstrings.
"""
from .reference import (  # noqa: F401
    build,
    colnorm2,
    zigzag_perm,
    block_svd,
    hadamard,
    rotation,
    rotate_rows,
    pack_weights,
    weight_rtn,
    pack_int4,
    unpack_int4,
    pack_codes,
    BITS_QMAX,
    quantize_act,
    rotate_quant_act,
    int_gemm,
    int_gemm_sampled,
    dequant,
    gemm,
    calibrate_table,
    quantize_act_grouped,
    int_gemm_grouped,
    dequant_grouped,
    gemm_grouped,
    calibrate_table_grouped,
    GPTQ_DAMP,
    gptq_hessian,
    gptq_factor,
    gptq_pack,
    linear,
    stack_prepare,
    stack_run,
    stack_calibrate,
    STACK_LINEARS,
    e3m2_value,
    e3m2_encode,
    f6_bytes,
    f6_operand,
    f6_codes,
)

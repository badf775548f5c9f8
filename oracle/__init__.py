"""CPU oracle for the OCP MX v1.0 MXFP4 quantizer and block-scaled GEMMs.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables
or helpers with the HIP library; both sides are written independently from the
pages they cite.

Sources (cited by page title and section):
  * "MXFP4", AI Wiki (aiwiki.ai/wiki/mxfp4): §Format specification (parameter
    table, E2M1 value table), §Conversion rules, §Clipping in the reference
    algorithm, §Training with MXFP4, §Use in models / gpt-oss.
  * "Training an MoE LLM in MXFP4: How We Closed the Gap to BF16", The
    Singularity Report: hybrid 1D/2D blocks, randomized Hadamard transform,
    stochastic rounding.
  * Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
    easy as 1, 2, 3", SC'11 (the counter-based generator named for the
    stochastic-rounding bits; not on the pages).

Everything is plain NumPy: float32 where the method is defined in float32
(the canonical quantizer steps), float64 for the GEMM reference.  Every
function is pinned in ``tests/test_oracle_*.py`` against facts the pages or the
mathematics fix.  Readings of points the pages leave open are listed in the
module docstrings where they are taken.
"""

from .formats import (
    E2M1_GRID,
    e2m1_decode,
    e8m0_decode,
    bf16_bits_to_f32,
)
from .philox import philox4x32_10, sr_bits8, sr_bits16
from .rht import rht_forward_f32, rht_inverse_f32, hadamard32_f64
from .quantize import (
    quantize,
    clip_count,
    quantize_gather,
    quantize_scatter,
    transpose_2d,
    round_up_exponent,
    dequantize,
    shared_exponent,
    round_e2m1,
    pack_nibbles,
    unpack_nibbles,
)
from .gemm import gemm_ref, grouped_gemm_ref, block_dot_exact
from . import elements

__all__ = [
    "E2M1_GRID",
    "e2m1_decode",
    "e8m0_decode",
    "bf16_bits_to_f32",
    "philox4x32_10",
    "sr_bits16",
    "sr_bits8",
    "rht_forward_f32",
    "rht_inverse_f32",
    "hadamard32_f64",
    "quantize",
    "clip_count",
    "quantize_gather",
    "quantize_scatter",
    "transpose_2d",
    "round_up_exponent",
    "dequantize",
    "shared_exponent",
    "round_e2m1",
    "pack_nibbles",
    "unpack_nibbles",
    "gemm_ref",
    "grouped_gemm_ref",
    "block_dot_exact",
]

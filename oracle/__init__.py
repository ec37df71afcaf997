"""CPU oracle for the NVFP4 linear-projection hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call, link or execute this package; only the tests,
the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code
with the HIP library.

It is a plain, slow, obviously-correct statement of what the hot path
computes, in float64 (exact wherever the values are dyadic), written from the
method described in the Full-Stack FP4 pages.

Citation key used in this package:

[FS4 §n]   "Full-Stack FP4: Stable LLM Pretraining with Quantized Projections,
           Optimizers, and Attention" (arXiv 2607.04422), technical summary on
           gist.science, Spanish and French editions, section n:
           §1 problem, §2.1 LoRA-SVD projections, §2.3 NVFP4 Root optimizer,
           §3 contributions, §4 results, §5 limitations.

The pages name NVFP4 but never define it.  The format used here is the
two-level block format: E2M1 element codes {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a
sign bit, one E4M3 (FN) decode scale per 16 consecutive elements along the
contraction dimension, one FP32 decode scale per tensor, two codes per byte,
round-to-nearest-even.  Each function below states which reading of a silent
point it takes.

Modules
-------
formats         E2M1 / E4M3 tables and round-to-nearest-even encoders
quantize        two-level block quantizer, row- and column-wise, dequantizer
exact           the same quantizer in exact rational arithmetic (brute force)
linear          block-scaled NT GEMM, LoRA-SVD linear forward and backward
newton_schulz   NVFP4 Newton-Schulz iteration (and the unquantized fp64 one)
lora            Cholesky-QR, the subspace-constrained low-rank gradients and
                the randomized-SVD realignment
adamw           the Q-AdamW optimizer-state codecs (second and first moment)
attention       NVFP4 mixed-precision attention (Q-Attn), forward and backward
"""
from .formats import (E2M1_GRID, e2m1_decode, e2m1_rne_index, e4m3_decode, e4m3_rne_satfinite,
                      tensor_scale_from_amax)
from .quantize import NVFP4, quantize, quantize_rows, dequantize, block_values
from .linear import gemm_nt, gemm_nt_abs, linear_fwd, linear_bwd, rel_err
from .newton_schulz import ns_normalize, ns_step, newton_schulz, newton_schulz_fp64, abs_quantile, clip_abs
from .lora import cholesky_qr, subspace_project, lora_realign, bf16_rne
from .adamw import vstate_encode, vstate_decode, mstate_encode, mstate_decode
from .attention import attention_fwd, attention_bwd

__all__ = [
    "E2M1_GRID", "e2m1_decode", "e2m1_rne_index", "e4m3_decode", "e4m3_rne_satfinite",
    "tensor_scale_from_amax", "NVFP4", "quantize", "quantize_rows", "dequantize", "block_values",
    "gemm_nt", "gemm_nt_abs", "linear_fwd", "linear_bwd", "rel_err",
    "ns_normalize", "ns_step", "newton_schulz", "newton_schulz_fp64",
]

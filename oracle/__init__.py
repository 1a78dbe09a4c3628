"""CPU oracle for the weight-only quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library in ``gemm_decode_amd/`` and imports nothing from it.

What it computes (plain, slow, obviously correct; NumPy only):

* ``quant``  -- the quantisers and the canonical packed layouts (W8 per output
  channel and with groups of 32, 64 or 128; W4 asymmetric with groups of 32, 64 or
  128 and per output channel), step by step.
* ``linear`` -- dequantise to fp32 (exact) and y = x . dequant(W)^T in fp64,
  chunked along N; sampled-column variants for full-size checks; the
  comparison statistics with the per-element tolerance; the full-K activation
  permutation (x gathered along K before the product); the layer with a residual
  added to its output.
* ``topk``   -- the k best bf16 logits of a row and the token drawn from them
  with a temperature and a caller-supplied uniform draw (the LM head + top-k
  step of the tileInfer README's feature list; reading in its docstring).
* ``moe``    -- the grouped (mixture-of-experts) layer, each expert applied to its
  own rows, and the SiLU-gated product of a fused gate/up projection (reading in
  its docstring).

Passages followed:

* tileInfer README, feature table ("INT8 Weight-Only Quantization") and the
  "Key Optimizations" list: int8 weights with one scale per output channel, bf16
  activations; decode multiplies the dequantised weights in registers, prefill
  dequantises to bf16 on the fly before a GEMM.
* "Marlin register and launch scheduling benchmark", "Validation and limits":
  INT4 and INT8 weights with bf16 activations, per-channel scales and groups of
  32, 64 and 128.
* "Heuristic: Mit han lab Llm awq Kernel Selection Thresholds", code excerpt
  from awq/quantize/qmodule.py: the token count is numel(x) / x.shape[-1].

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
hand-derived worked examples (``tests/golden/``), closed-form error bounds,
brute force on tiny inputs and reductions to NumPy library routines.
"""
from .quant import (  # noqa: F401
    FORMATS, GROUP, GROUPED, SMALL_GROUPS, W4PC, bf16_bits_to_f32, bf16_rne_bits, dequant, pack,
    packed_sizes, quantize_w4, quantize_w4g128, quantize_w8, unpack_w4g, unpack_w4g128, unpack_w4pc,
)
from .linear import (  # noqa: F401
    compare, gather_activations, ref_linear, ref_linear_columns, ref_linear_perm, ref_linear_residual, token_count,
    use_gemv,
)
from .topk import ref_topk_sample, sample_row, topk_row  # noqa: F401
from .moe import (  # noqa: F401
    check_offsets, ref_linear_silu_mul, ref_moe_linear, ref_moe_silu_mul, silu, silu_mul,
)

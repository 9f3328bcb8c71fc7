"""CPU oracle for block-scaled FP8 quantization and GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
tables with the HIP library; the one module both sides draw from is the seeded
input generator in ``inputs/``, which holds none of the method's arithmetic.

It is a plain, slow, obviously-correct statement of what the method computes:

* ``e4m3``            -- the E4M3FN code table (decode) and round-to-nearest-even
                         encode with saturation at 448.
* ``act_quant``       -- dynamic 1x128 activation quantization.
* ``weight_dequant``  -- 128x128 block-scaled weight dequantization.
* ``weight_quant``    -- 128x128 block weight quantization (its inverse).
* ``fp8_gemm``        -- the block-scaled FP8 GEMM, each 128-wide K slice's
                         partial sum scaled and accumulated, in float64, plus the
                         per-element error bound GPU results are held to.

Every reading taken where the pages leave a step open is stated in the
docstring of the function that takes it.  Parity status: every function here is
pinned by ``tests/test_oracle_*.py`` except the two page claims that carry no
numbers (the <0.25% training-loss figure and the FP32 promotion interval on
H800 hardware): those are "parity unpinned" and nothing here computes them.
"""

from . import e4m3  # noqa: F401
from .act_quant import act_quant  # noqa: F401
from .weight_dequant import weight_dequant, f32_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
from .weight_quant import weight_quant  # noqa: F401
from .fp8_gemm import fp8_gemm, dequantized_operands, gemm_tolerance, gemm_check  # noqa: F401

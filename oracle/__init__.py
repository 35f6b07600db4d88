"""CPU oracle of the BF16 encoder forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite (``tests/``), the smoke check
(``__graft_entry__.smoke``) and the CPU-baseline leg of ``bench.py`` may
import, call, link or run anything in this package.  The HIP library never
does, and this package imports nothing from the HIP side: the two share no
code, only the seeded inputs of ``transformer_encoder_bf16_amd/inputs.py``.

It is plain numpy in float32 with BF16 rounding wherever a tensor is stored
(the tensor boundaries of the pass), plus a small C helper for the
counter-based weight generator.  Matrix products use numpy's matmul as a
library step; nothing is fused, blocked or reordered beyond that.

Pins (tests/test_oracle_*.py): a float64 brute force written separately in
tests/brute, published SplitMix64 outputs, torch's float32->bfloat16
conversion, closed forms of GELU and the normal CDF, and invariants of RoPE,
LayerNorm and attention.  The agreement with the upstream Laya runtime on a
trained checkpoint is "parity unpinned": neither is available.
"""
from .model import Oracle, attention, layer_kinds, layer_norm, linear, pack  # noqa: F401
from .numerics import bf16_bits_to_f32, bf16_round, f32_to_bf16_bits, gelu, nrms  # noqa: F401
from .rope import f64_to_bf16, rope_apply, rope_tables  # noqa: F401
from .weights import Weights, build, fnv1a64, tensor_bits, tensor_shapes  # noqa: F401

"""CPU oracle of the MXFP4 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64
restatement of what the layer computes.  Only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it; the library and its Python binding never do, and it imports nothing
from them.

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  mx.e2m1_value      OCP E2M1 value table (tests/golden), sign symmetry
  mx.e4m3_value      torch.float8_e4m3fn decode, exhaustive
  mx.e8m0_value      torch.float8_e8m0fnu decode and fp32 exponent field, exhaustive
  mx.unpack_fp4 / dequant_mxfp4 / dequant_mxfp8   brute-force per-element loops,
                     power-of-two scale law
  moe.route          numpy stable argsort; fp64 brute-force sort; softmax identities
  moe.permute        numpy stable argsort + bincount; inverse-permutation property
  moe.silu / gate_up silu(z) - silu(-z) = z; gate/up separation by zeroed rows
  moe.expert_mlp     pure-Python triple loops
  moe.combine        one-hot weights, k = 1 copy
  moe.moe_layer      dense one-expert equivalence, token-order permutation invariance,
                     pure-Python brute force of the whole layer on tiny inputs
  moe.moe_tokens     equals moe_layer rows
  moe.rms_rescale / to_bf16_bits   unit RMS; torch bf16 rounding
"""
from . import mx, moe  # noqa: F401

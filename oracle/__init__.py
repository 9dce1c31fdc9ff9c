"""CPU reference decoder.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package.  It shares no code with the HIP library or its binding.

Parity pins (all CPU tests): every function here is pinned by at least one
closed form, invariant, special case or brute-force check; none is "parity
unpinned".
"""
from .decoder import (f64, f16_round, rmsnorm, rope, rope_angles, silu, softmax,
                      attend, greedy, top2_margin, Weights, OracleDecoder,
                      prefill_matrix, greedy_decode)
from .moe import (e4m3_value, e4m3_decode, dequant, e2m1_value, e8m0_value, mx_dequant, route, MoEWeights, expert_ffn, moe_ffn,
                  OracleMoEDecoder, prefill_matrix_moe, greedy_decode_moe)

__all__ = ["f64", "f16_round", "rmsnorm", "rope", "rope_angles", "silu", "softmax",
           "attend", "greedy", "top2_margin", "Weights", "OracleDecoder",
           "prefill_matrix", "greedy_decode",
           "e4m3_value", "e4m3_decode", "dequant", "e2m1_value", "e8m0_value", "mx_dequant", "route", "MoEWeights", "expert_ffn", "moe_ffn",
           "OracleMoEDecoder", "prefill_matrix_moe", "greedy_decode_moe"]

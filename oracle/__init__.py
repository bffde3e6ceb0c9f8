"""CPU oracle for block-causal chunk attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU baseline
import this package. The GPU library never does, and this package imports
nothing from it.
"""
from .oracle import (OracleLib, attend, attend_masked, lse_merge, e4m3_decode, e4m3_encode,
                     quant_e4m3, block_scales, quant_int8, rope, attend_sequence, threads, set_threads, build, compile_oracle, default,
                     LIB_PATH, SRC_PATH)

__all__ = ["OracleLib", "attend", "attend_masked", "lse_merge", "e4m3_decode", "e4m3_encode",
           "quant_e4m3", "block_scales", "quant_int8", "rope", "attend_sequence", "threads", "set_threads", "build", "compile_oracle", "default",
           "LIB_PATH", "SRC_PATH"]

"""CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never does; it shares no code with
it.  Contents:

  kda_oracle.c / recurrent.py   token-by-token fp64 recurrence (the definition),
                                and its fp32 twin (a diagnostic of the fp32 floor)
  chunked.py                    fp64 chunked re-derivation of the same result
  gate.py                       the Kimi gate activation (fp64)
  conv.py                       short causal conv with carried taps (fp64)
  heads.py                      q/k L2 normalisation, grouped key heads (fp64)
"""
from .recurrent import (OracleLib, decode, lib_path, num_threads, prefill,  # noqa: F401
                        prefill_f32, set_num_threads)
from .chunked import chunked_prefill, unit_lower_inverse  # noqa: F401
from .gate import kimi_gate, softplus  # noqa: F401
from .conv import causal_conv1d, silu  # noqa: F401
from .heads import L2NORM_EPS, expand_key_heads, l2norm  # noqa: F401

"""FP64 CPU oracle (test infrastructure only; see ``oracle.attention``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do, and this package never imports them.
"""
from .attention import (default_scale, attention, attention_head, int8_scores,
                        attention_int8, attention_int8_head, quantize_int8, quantize_int8_tiles,
                        deviation, attention_probabilities, attention_delta,
                        attention_backward_head, run_heads)
from .distance import wasserstein, wasserstein1_cdf
from .fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, quantize_fp8, fp8_scores,
                  attention_fp8_head, attention_fp8)

__all__ = ["default_scale", "attention", "attention_head", "int8_scores",
           "attention_int8", "attention_int8_head", "quantize_int8", "quantize_int8_tiles",
           "deviation", "attention_probabilities", "attention_delta",
           "attention_backward_head", "run_heads",
           "wasserstein", "wasserstein1_cdf", "E4M3_MAX", "e4m3_decode", "e4m3_encode",
           "quantize_fp8", "fp8_scores", "attention_fp8_head", "attention_fp8"]

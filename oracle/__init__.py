"""fp64 CPU oracles (attention forward, backward and FP8 forward; QKV prologue): test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. It shares no code with the HIP library.
"""
from .attention import attention_fp64, bf16_bits_to_f64, f32_to_f64, segments  # noqa: F401
from .prologue import norm_rope_rows_fp64, qkv_prologue_fp64  # noqa: F401,E402
from .attention_bwd import attention_bwd_fp64  # noqa: F401,E402
from .attention_fp8 import attention_fp8_fp64, e4m3_bits_to_f64  # noqa: F401,E402

"""CPU oracle of the StateKV frame step (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library or its binding.
"""
from .statekv_oracle import (  # noqa: F401
    CompressedState, DecodeResult, LayerConfig, OracleStream, StepResult, decode_step, frame_step,
    round_f64_to_bf16, round_storage, rope_cos_sin, rope_inv_freq, rope_rotate,
    select_recent, select_top_b, yarn_inv_freq, yarn_logit_scale,
)

"""RAT+ recurrence-augmented dilated attention on AMD Instinct MI355X (gfx950).

The hot path lives in the HIP library ``librat.so`` (C ABI in
``include/rat.h``); ``ops`` is its thin torch binding and ``inputs`` the
seeded synthetic workloads.  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from .ops import (RESTART, SLIDING, RatError, attn_prefill_workspace_bytes, build_decode_caches,  # noqa: F401
                  chunk_attn_prefill,
                  decode_step, decode_step_sliding, decode_workspace_bytes, dilated_attn_decode, dilated_attn_decode_static, dilated_attn_prefill, history_rows,
                  layer_backward, layer_prefill, load_library, prefill_two_calls, scan_prefill, scan_workspace_bytes,
                  sliding_state_from_prefill)

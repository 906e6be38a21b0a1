"""CPU oracle of the TokenGate gated-prefill path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library.
"""
from .tokengate_oracle import *  # noqa: F401,F403
from .tokengate_oracle import (FORCED_GT_BUDGET, BUDGET_GT_LEN, NAN_SCORE,  # noqa: F401
                               gelu, sigmoid, gate_score, select_one, topk_select,
                               compact, rmsnorm, rope, gated_attention, decode_attention, silu,
                               gated_attention_backward, gelu_grad, gate_score_backward,
                               compact_backward, gdn_mixer,
                               qkv_rope, o_proj, swiglu_act, down_proj,
                               upper_layer, gated_prefill)

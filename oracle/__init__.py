"""CPU oracle (test infrastructure only; never on the product path)."""
from .attention_bwd_ref import attention_bwd_ref, blocked_attention_bwd_ref  # noqa: F401
from .attention_ref import (MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE,  # noqa: F401
                            attention_general_ref, attention_ref, attention_varlen_ref,
                            brute_ref,
                            online_attention_ref, online_softmax_stats, partition,
                            probabilities_ref, visible_general)

"""CPU float64 oracle of the BPT layer forward: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it; the
HIP library never imports, links or calls anything here.
"""
from .bpt_oracle import (WEIGHT_KEYS, attention_backward_dq_rows,  # noqa: F401
                         attention_backward_kv_rows,
                         attention_backward_sequence, attention_lse_sequence, attention_sequence,
                         blockwise_layer_forward, gelu_tanh, layer_forward, layer_forward_rows,
                         merge_summaries, softmax_summary, layer_backward,
                         layer_norm_backward, gelu_tanh_derivative,
                         layer_lse, layer_lse_rows, layer_norm,
                         max_abs_err, online_softmax_tiles, rel_fro_err, softmax_rows,
                         stack_forward, stack_forward_rows, visible)

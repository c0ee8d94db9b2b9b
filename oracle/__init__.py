"""CPU oracle (test infrastructure only; see chipmunk_oracle's header)."""
from .chipmunk_oracle import (ROW_BLOCK, attn_dense, attn_rest, attn_sparse, bf16_bits, bf16_round,  # noqa: F401
                              from_bf16_bits, gelu_tanh, identify_topk, mlp_dense, mlp_sparse,
                              rel_frobenius)

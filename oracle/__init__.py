"""CPU oracle (test infrastructure only; see chipmunk_oracle's header)."""
from .chipmunk_oracle import (ROW_BLOCK, attn_dense, attn_reident, attn_rest, attn_sparse,  # noqa: F401
                              bf16_bits, bf16_round, from_bf16_bits, gelu_tanh, identify_topk,
                              mlp_dense, mlp_sparse, rel_frobenius)

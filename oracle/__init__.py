"""CPU oracle (test infrastructure only; see chipmunk_oracle's header)."""
from .chipmunk_oracle import (CACHED, DENSE, ROW_BLOCK, SPARSE, attn_dense, attn_schedule, mlp_schedule, attn_reident, attn_rest, attn_sparse,  # noqa: F401
                              bf16_bits, bf16_round, dequantize_fp8_rows, fp8_blocks, fp8_cols,
                              fp8_e4m3_decode, fp8_e4m3_encode, fp8_row_exponent, fp8_rows, from_bf16_bits,
                              gelu_tanh, identify_topk, mlp_dense, mlp_sparse, quantize_fp8_blocks,
                              quantize_fp8_rows, rel_frobenius)

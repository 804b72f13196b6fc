"""MI355X-native C3 hot path: concurrent bf16 GEMM + collective-shaped copy (CU or SDMA)."""

"""Load-balanced split-KV decode attention with a fused RoPE/QK-Norm prologue, for MI355X."""

"""Float64 CPU oracle for S2-Attn (test infrastructure only; see s2attn_oracle)."""

"""Shifted Sparse Attention (S2-Attn) on AMD MI355X: HIP kernels behind a C ABI.

The compute lives in libs2attn.so (built from csrc/ by ``build.py``); this
package only marshals torch tensors into the C ABI declared in include/s2attn.h.
"""

from .binding import (RoPE, S2Attn, S2AttnError, S2AttnRoPE, rope, s2attn, s2attn_bwd,  # noqa: F401
                      s2attn_bwd_dkdv, s2attn_bwd_dq, s2attn_bwd_noalloc, s2attn_bwd_prep, s2attn_bwd_prep_dq,
                      s2attn_bwd_rope, s2attn_bwd_workspace_bytes, s2attn_fwd, s2attn_fwd_rope, s2attn_rope,
                      s2attn_status_str, s2attn_with_rope)

"""gfx950-native Infini-attention forward pass.

The compute runs in ``libinfini_attn.so`` (hand-written HIP for MI355X); this
package only binds its C ABI (see ``include/infini_attn.h``).
"""

from ._lib import (  # noqa: F401
    BF16, DELTA, F32, LINEAR, InfiniAttnDesc, InfiniAttnError, backward, block_forward, decode, forward,
    handle_for, infini_attn_backward, infini_attn_block_forward, infini_attn_block_forward_qkv,
    infini_attn_decode_noalloc,
    infini_attn_check, infini_attn_create, infini_attn_decode, infini_attn_destroy,
    infini_attn_forward, infini_attn_get_timing, infini_attn_set_timing, infini_attn_update,
    infini_attn_workspace_size, load, make_desc, release_handles, strerror, update,
)

"""MI355X-native (gfx950) kernels for one Ulysses rank's share of Multi-head Latent Attention.

The computation lives in libmla.so (hand-written HIP, C ABI in include/mla.h);
this package only builds it and marshals arguments to it.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MLA_BF16, MLA_EINVAL, MLA_ELAUNCH, MLA_EUNSUPPORTED, MLA_F32, MLA_OK, MlaError,
    load_library, mla_attention_fwd, mla_attention_fwd_noalloc, mla_attention_workspace_size, mla_head_shard_sizes,
    mla_latent_decode_fwd, mla_latent_decode_workspace_size, mla_latent_up_proj, mla_latent_up_proj_linear,
    mla_pack_heads,
    mla_unpack_heads, mla_pack_expanded, mla_causal_partition, mla_kv_exchange_ranges, mla_apply_rope,
    mla_project_pack, mla_attention_bwd, mla_attention_bwd_workspace_size,
    mla_latent_up_proj_bwd, mla_latent_up_proj_bwd_workspace_size, mla_peak_mfma_bf16, PEAK_EXPORTS,
)

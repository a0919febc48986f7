"""MLA over a paged, compressed latent KV cache on MI355X (gfx950).

The computation lives in libmla_latent_kv.so (HIP kernels behind the C ABI of
include/mla.h); this package is its Python binding plus a paged-pool helper.
Importing fails if the library has not been built.
"""
from ._lib import MLAError, LIB_PATH  # noqa: F401  (raises ImportError if not built)
from .api import (  # noqa: F401
    MLAConfig, mla_abi_version, mla_validate_config, mla_cache_row_elems,
    mla_cache_bytes_per_token, mla_rope_table, mla_decode_workspace_size, mla_decode,
    mla_decode_noalloc,
    mla_absorb_query, mla_latent_attention, mla_attention_partials, mla_combine_output,
    mla_output_projection,
    mla_cache_append_workspace_size, mla_cache_append, mla_prefill_workspace_size, mla_prefill_attention_form, mla_prefill,
    mla_output_gate_workspace_size, mla_output_gate_projection,
    mla_probe_sink, mla_probe_hbm_read, mla_probe_mfma, mla_probe_lds_read,
)
from .pool import LatentKVPool  # noqa: F401

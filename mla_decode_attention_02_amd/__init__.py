"""Paged MLA decode attention for AMD Instinct MI355X (gfx950), plus paged
multi-head / grouped-query decode over separate K and V caches.

The compute runs in the HIP library ``libmla_decode.so`` (C ABI, declared in
``include/mla_decode.h`` and ``include/mha_decode.h``); this package only marshals torch tensors into that
ABI.  Importing the package does not load the library; the first call does,
and raises if the library has not been built.
"""

__all__ = ["get_metadata", "get_metadata_shape", "workspace_size", "mla_decode",
           "mla_decode_splitkv", "mla_decode_combine", "mla_decode_fused", "mla_merge_partials",
           "mha_get_metadata", "mha_get_metadata_shape", "mha_workspace_size", "mha_decode",
           "mha_decode_splitkv", "mha_decode_combine", "mla_decode_noalloc", "check_paged_inputs", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)

"""MI355X (gfx950) implementation of E2Former-V2's on-the-fly equivariant
attention layer (arXiv 2601.16622): a HIP library with a C ABI (include/e2a.h)
and this thin Python binding.

The binding (and with it the built library) loads on first use of one of the
names below, so that the build step can run before the library exists."""

_EXPORTS = (
    "E2AError",
    "e2a_attention_bwd",
    "e2a_attention_bwd_workspace_bytes",
    "e2a_attention_bwd_weights",
    "e2a_attention_bwd_weights_workspace_bytes",
    "e2a_attention_fwd",
    "e2a_attention_fwd_noalloc",
    "e2a_attention_workspace_bytes",
    "e2a_block_fwd",
    "e2a_block_workspace_bytes",
    "e2a_build_neighbors",
    "e2a_conv_fwd",
    "e2a_destination_order",
    "e2a_destination_order_workspace_bytes",
    "e2a_neighbors_workspace_bytes",
    "e2a_pack_so2_weights",
    "e2a_so2_packed_bytes",
    "e2a_so2_param_count",
    "e2a_version",
    "library_path",
)


def __getattr__(name):
    if name in _EXPORTS:
        from . import e2a
        return getattr(e2a, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def __dir__():
    return sorted(list(globals()) + list(_EXPORTS))

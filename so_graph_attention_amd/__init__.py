"""MI355X (gfx950) implementation of E2Former-V2's on-the-fly equivariant
attention layer (arXiv 2601.16622): a HIP library with a C ABI (include/e2a.h)
and this thin Python binding."""
from .e2a import (  # noqa: F401
    E2AError,
    e2a_attention_fwd,
    e2a_attention_workspace_bytes,
    e2a_build_neighbors,
    e2a_neighbors_workspace_bytes,
    e2a_so2_param_count,
    e2a_version,
    library_path,
)

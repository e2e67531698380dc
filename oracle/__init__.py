"""fp64 CPU oracle for the on-the-fly equivariant attention layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import anything from this package.  The HIP library never
calls it, and it shares no code, table or constant with the HIP sources.
"""
from .e2a_oracle import (  # noqa: F401
    NORM_EPS,
    attention,
    attention_backward,
    attention_online,
    attention_position_backward,
    attention_weight_backward,
    block,
    convolution,
    degree_linear,
    degree_rms_norm,
    edge_messages,
    edge_messages_vjp,
    edge_messages_weight_vjp,
    edge_rotation,
    edge_unit,
    gated_ffn,
    min_image,
    neighbor_list,
    neighbor_list_bruteforce,
    qk_projection,
    radial_basis,
    real_sph_harm,
    segment_softmax,
    so2_blocks,
    wigner_d,
)

"""MI355X-native Ulysses H3 hot path: seq2head / packed attention / head2seq / AdaLN,
the backward of the relayouts and of the attention, the gated AdaLN chain, and
the ragged reduce-scatter and row gather of the token-sharded blocks.

The compute lives in ``libh3.so`` (hand-written HIP for gfx950, C ABI declared
in ``include/h3.h``); this package is its thin ctypes binding.  Importing it
fails if the library has not been built.
"""
from .h3 import (  # noqa: F401
    EXPORTS, H3_ADALN_GATE_MODULATE, H3_ADALN_GATE_RESIDUAL, H3_ADALN_MODULATE, HEAD_DIM, H3Error, Layout,
    PlanInfo, adaln_gate_modulate, adaln_segment, clip_segments, gather_rows, head2seq, head2seq_backward,
    head_split, library, NOALLOC_SCRATCH_BYTES, packed_attn, packed_attn_backward, packed_attn_backward_noalloc,
    packed_attn_backward_workspace, partition, reduce_scatter, seq2head, seq2head_backward, version,
)

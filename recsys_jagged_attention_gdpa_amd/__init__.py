"""MI355X-native jagged attention: GDPA (activation, no row normalisation) and
JFA (online softmax) over variable-length, unpadded batches, forward and
backward, as hand-written gfx950 HIP kernels behind a C ABI
(include/jagged_attn.h, libjagged_attn.so).

The shared library is loaded on first use; nothing here computes attention
itself.
"""
from . import _lib  # noqa: F401
from ._lib import (JaError, JaProblem, ja_workspace_size, jagged_attn_bwd,  # noqa: F401
                   jagged_attn_fwd, jagged_attn_fwd_mx, jagged_gdpa_bwd, jagged_gdpa_fwd,
                   jagged_gdpa_fwd_mx, jagged_rope, make_problem)
from .ops import (attn_backward, attn_forward, gdpa, gdpa_backward, gdpa_forward,  # noqa: F401
                  jagged_attention, mx_forward, rope)

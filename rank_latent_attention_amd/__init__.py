"""FLARE / FLARE++ low-rank attention routing on MI355X (gfx950): forward and backward.

The compute path is the HIP library built from csrc/flare.hip and
csrc/backward.h (C ABI in include/flare.h); ``rank_latent_attention_amd.flare``
is its Python binding.
"""
from .flare import (FlareError, flare_backward, flare_decode, flare_encode, flare_encode_backward,  # noqa: F401
                    flare_forward, flare_forward_noalloc, flare_forward_proj, flare_pp_backward, flare_pp_backward_norm,
                    flare_pp_forward, flare_pp_forward_norm, flare_pp_forward_proj, load, workspace, workspace_size)

"""FLARE / FLARE++ low-rank attention routing forward on MI355X (gfx950).

The compute path is the HIP library built from csrc/flare.hip (C ABI in
include/flare.h); ``rank_latent_attention_amd.flare`` is its Python binding.
"""
from .flare import (FlareError, flare_backward, flare_decode, flare_encode, flare_encode_backward,  # noqa: F401
                    flare_forward, flare_pp_backward, flare_pp_forward, flare_pp_forward_norm, load, workspace,
                    workspace_size)

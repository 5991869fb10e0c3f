"""Batch-invariant LM head for AMD Instinct MI355X (gfx950).

The HIP library ``liblmhead.so`` (C-ABI: ``include/lmhead.h``) does all the
work; ``invariant_lm_head_amd.lmhead`` marshals torch tensors into it.
"""
from . import _build, lmhead  # noqa: F401

__all__ = ["lmhead", "build"]


def build(verbose: bool = False):
    """Compile the HIP library for gfx950 (always recompiles)."""
    return _build.build(verbose=verbose)

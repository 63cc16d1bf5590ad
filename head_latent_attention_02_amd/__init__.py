"""MLA forward hot path on MI355X (gfx950): explicit (LAGA-local) training
forward and absorbed split-KV decode, behind the C-ABI library ``libmla.so``.

The binding (``head_latent_attention_02_amd.mla``) loads the library lazily on
first use and raises if it is missing; nothing here falls back to CPU code.
"""
__all__ = ["inputs"]

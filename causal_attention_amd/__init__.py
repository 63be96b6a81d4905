"""Fused causal attention for MI355X (gfx950).

``causal_attention_amd.attn`` is the Python binding of the C-ABI library
``libattn.so`` (built from ``csrc/``); ``causal_attention_amd.debug`` binds the
per-tile softmax trace of its debug build ``libattn_debug.so``;
``causal_attention_amd.inputs`` holds the seeded synthetic input generators.
Importing the package loads nothing: a library is opened on first use of its
binding.
"""

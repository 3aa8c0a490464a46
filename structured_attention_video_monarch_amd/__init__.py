"""MonarchAttention forward for MI355X (gfx950): Python binding.

The binding loads ``libmonarch_attn.so`` lazily, on first use, so that
``structured_attention_video_monarch_amd.inputs`` can be imported without it.
"""

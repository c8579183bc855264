"""MI355X (gfx950) speculative-verification attention.

The compute lives in the HIP library ``libverify_attn.so`` (C ABI declared in
``include/verify_attn.h``); ``long_context_verify_tree_amd.ops`` is the thin
Python binding over it and ``synth`` draws seeded synthetic inputs.  Nothing
is imported eagerly, so importing the package never touches the GPU.
"""

__all__ = ["ops", "synth"]

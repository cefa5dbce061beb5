"""MI355X-native routed mixture-of-experts FFN layer.

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP for
gfx950, declared in ``include/moe.h``); ``binding`` marshals arguments to it
and nothing else.  ``synth`` draws the seeded synthetic inputs.
"""
__all__ = ["binding", "synth"]

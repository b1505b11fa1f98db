"""MI355X (gfx950) routed-expert FFN layer: Python binding of libmoe.so.

The binding is loaded on first use so that ``routed_expert_ffn_route_amd.synth``
(the seeded input generators) imports without a GPU library present.
"""


def __getattr__(name):
    if name in ("moe", "binding"):
        from . import binding
        return binding
    raise AttributeError(name)

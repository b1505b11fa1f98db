"""MI355X (gfx950) routed-expert FFN layer.

* ``binding`` -- ctypes binding of libmoe.so (include/moe.h): moe_route, moe_forward, ...
* ``synth``   -- seeded synthetic layers and inputs.
* ``build``   -- compiles libmoe.so with hipcc.

Submodules are imported explicitly (``from routed_expert_ffn_route_amd import binding``);
importing the package itself loads no GPU library.
"""

"""Grouped routed-expert MoE decode for one MI355X (gfx950): a C-ABI HIP library and its binding.

``moe_routed_expert_route_amd.binding`` loads ``libmoe_route.so`` (built from ``csrc/``) and
exposes its entry points under the same names; ``synth`` draws the seeded synthetic inputs.
Importing this package loads nothing; the binding raises if the library is missing.
"""

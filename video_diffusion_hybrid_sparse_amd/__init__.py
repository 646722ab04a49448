"""MI355X-native (gfx950) VDN-H3 hybrid attention layer.

The layer runs in a C-ABI HIP library (``libvdn_hybrid_attn.so``, built in-tree); the
binding module marshals torch tensors into it.  ``shapes`` and ``synth`` hold workload
sizes and seeded synthetic inputs.
"""

"""KVarN tile quantizer + paged decode attention for MI355X (gfx950).

The HIP library and its ctypes binding live in `kvarn`; importing this package does not
load the library, so the seeded workload generators in `synth` stay importable anywhere.
"""

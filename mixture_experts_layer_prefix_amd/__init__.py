"""MI355X-native MoE layer forward: HIP kernels for gfx950 behind a C ABI.

The compute path lives in ``csrc/`` (built into ``libmoe.so``); ``moe`` is a
thin ctypes binding with the same entry-point names.  ``configs`` and
``inputs`` hold the workload shapes and the seeded input generators.
"""

"""Speculative-decoding verification sampler for MI355X (gfx950).

The device path is the HIP library ``libspecverify.so`` built from
``csrc/``; ``binding`` marshals arguments to its C ABI.  ``workloads``
draws seeded synthetic batches.
"""

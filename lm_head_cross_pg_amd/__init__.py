"""MI355X (gfx950) fused tied LM head + logit softcap cross-entropy -> bits-per-byte.

The compute lives in the HIP library ``libpg_lmhead.so`` (C ABI, see include/pg_lmhead.h); the
``abi`` module is a thin ctypes binding with the same entry-point names. ``synth`` draws seeded
synthetic inputs. Importing this package does not load the library; ``abi`` does, and fails loudly
when it has not been built.
"""
__all__ = ["abi", "synth"]

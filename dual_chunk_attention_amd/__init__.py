"""MI355X-native Dual Chunk Attention (DCA).

The compute lives in the HIP library ``libdca.so`` (C ABI declared in include/dca.h); the Python
binding in :mod:`dual_chunk_attention_amd.dca` only marshals arguments to it.  Importing this
package loads nothing; the library is loaded on first use and a missing library raises.
"""
__all__ = ["dca", "synth"]

"""Paged KV decode attention for MI355X (gfx950).

Exact single-token decode attention over a paged key/value history, computed
as split-KV tiles that each return a normalised output and a log-sum-exp,
combined by an FP32 log-sum-exp merge.  The compute runs in hand-written HIP
kernels behind a C ABI (``include/pkv.h``, built into ``libpkv.so`` next to
this file); ``paged_kv_cache_10_amd.pkv`` is the thin Python binding.

Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""

__all__ = ["pkv", "inputs"]

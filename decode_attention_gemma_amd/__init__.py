"""g4attn: Gemma-4-style decode/prefill attention over a device-resident KV cache
for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libg4attn.so`` (hand-written HIP
kernels); ``decode_attention_gemma_amd.g4attn`` is its thin ctypes binding.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""

__all__ = ["workloads", "g4attn"]

"""Batched attention over a paged KV cache on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libpaged_attn.so`` (hand-written HIP
kernels); ``paged_kv_attention_prefill_amd.binding`` marshals torch tensors
into it.  Importing this package does not load the library; the binding loads
it on first use and raises if it is missing.
"""
__all__ = ["workloads", "binding"]

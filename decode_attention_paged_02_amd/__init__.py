"""pda -- paged decode attention for MI355X (gfx950).

Single-token decode attention over a paged KV cache: GQA/MQA/MHA head
grouping, split-KV (Flash-Decoding) with an LSE-weighted combine, and the MLA
latent variant.  Every step runs in hand-written HIP kernels behind the C ABI
declared in ``include/pda.h`` (library ``libpda.so``); ``pda`` is a thin
ctypes binding over it.  ``workloads`` holds the seeded input generators and
``accounting`` the byte/FLOP counters used by the benchmark.

Importing the package does not load the HIP library; the first call through
``decode_attention_paged_02_amd.pda`` does, and fails loudly if it is missing.
"""

__all__ = ["pda", "workloads", "accounting"]

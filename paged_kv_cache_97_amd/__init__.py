"""pagedkv: PagedAttention hot path for AMD Instinct MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (hand-written HIP kernels behind a C
ABI, see ``include/pagedkv.h``).  ``ops`` marshals torch tensors into those
calls; ``blocks`` is the host-side block allocator; ``workloads`` builds the
seeded synthetic inputs.
"""
__all__ = ["blocks", "workloads", "ops"]

"""Block-scaled FP8 attention with the Delta-Matching row correction, for MI355X (gfx950).

The compute lives in libdm.so (HIP kernels behind the C ABI of include/dm_attn.h);
``fp8_attention_amd.api`` is its Python binding and ``fp8_attention_amd.workloads``
draws the seeded synthetic inputs.  Importing the package does not load the
library; the first call into ``api`` does, and fails loudly if it is not built.
"""

"""EAGLE target-verify attention (topk = 1) for MI355X (gfx950).

The compute path is ``libverify_attn.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/verify_attn.h``); ``binding`` marshals torch
tensors into it.  ``workloads`` draws seeded synthetic inputs.  Importing the
package loads nothing; the library is loaded on first use and its absence is
an error, never a fallback.
"""

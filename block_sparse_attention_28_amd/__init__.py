"""MI355X (gfx950) gated block-sparse attention: SeerAttention-R decode and
SeerAttention block-sparse prefill, as hand-written HIP kernels behind the C
ABI of include/seer.h.

Submodules: ``seer`` (ctypes binding of the C ABI), ``pipeline`` (buffers and
call order of one decode step), ``workloads`` and ``inputs`` (seeded
synthetic inputs), ``build`` (hipcc build of libseer.so).
"""
__all__ = ["seer", "pipeline", "workloads", "inputs", "build"]

"""Block-diffusion VLM denoise step on AMD MI355X (gfx950).

The computation lives in libbd.so (HIP kernels behind the C ABI of
include/bd.h); ``vlm_decoding_amd.bd`` is its ctypes binding and
``vlm_decoding_amd.step`` allocates device buffers for a whole step.
"""

"""MI355X (gfx950) library for cached block-wise masked-diffusion LLM decoding.

``libdllm.so`` (HIP kernels + C ABI, see include/dllm.h) is built in-tree by
``diffusion_block_denoise_amd.build``; ``diffusion_block_denoise_amd.dllm`` is its ctypes
binding.
"""

__all__ = ["dllm", "build"]

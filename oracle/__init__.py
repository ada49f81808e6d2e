"""Oracle: a plain, slow, fp64 CPU implementation of cached block-wise masked-diffusion decoding.

TEST INFRASTRUCTURE ONLY.  It exists to check the GPU library.  Only the test
suite, the smoke check of the entry module and the CPU-baseline leg of the
benchmark may import or run it; the product path never does, and this package
imports nothing from the product package.

Contents
--------
``oracle.model``   the bidirectional transformer forward over a row set with a
                   KV cache, and the lm_head softmax statistics.
``oracle.decode``  the commit rule, the per-block step schedule and the block
                   loop with its cache policy (no cache, prefix cache, dual cache).

Every function is fp64 over weights that were already rounded to their
storage type (bf16 or fp32); no intermediate result is rounded.
"""

from . import decode, model

__all__ = ["model", "decode"]

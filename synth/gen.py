"""Counter-based seeded generator for synthetic weights, prompts and token states.

It holds none of the decoding method's arithmetic: it only produces inputs.
The same values come out of the NumPy backend (host) and the torch backend
(host or device), bit for bit, so the oracle and the GPU path see identical
data without either importing the other.

Definition
----------
``fmix32`` is the 32-bit finaliser of Austin Appleby's MurmurHash3 (public
domain).  For a stream ``(seed, tensor_id)`` the host derives two 32-bit keys

    k1 = fmix32((seed * 0x9E3779B9 + (tensor_id + 1) * 0x7F4A7C15) mod 2^32)
    k2 = fmix32(k1 ^ 0x5BD1E995)

and element ``i`` (row-major flat index, ``i < 2^32``) gets the 32-bit word

    u(i) = fmix32(fmix32(i ^ k1) ^ k2).

Normal values: ``TABLE[u >> 16]``, where ``TABLE[j]`` is ``std * Phi^{-1}((j + 0.5) / 65536)``
computed in fp64 (SciPy ``ndtri``), rounded to fp32 and then, for bf16
tensors, to bf16 with round-to-nearest-even.  Token ids uniform in ``[0, n)``:
``(u * n) >> 32``.

All 32-bit products are formed as two 16-bit halves so that the torch backend
stays inside int64 without overflow.
"""

from __future__ import annotations

import numpy as np

M32 = 0xFFFFFFFF
_C1, _C2 = 0x85EBCA6B, 0xC2B2AE35

__all__ = ["stream_keys", "normal_table", "words_np", "words_torch", "normal_np", "normal_torch",
           "tokens_np", "tokens_torch", "bf16_bits_to_f32", "f32_to_bf16_bits"]


def _fmix32_int(h: int) -> int:
    h &= M32
    h ^= h >> 16
    h = (h * _C1) & M32
    h ^= h >> 13
    h = (h * _C2) & M32
    h ^= h >> 16
    return h


def stream_keys(seed: int, tensor_id: int) -> tuple[int, int]:
    k1 = _fmix32_int((seed * 0x9E3779B9 + (tensor_id + 1) * 0x7F4A7C15) & M32)
    k2 = _fmix32_int(k1 ^ 0x5BD1E995)
    return k1, k2


# ----------------------------------------------------------------------------- bf16 helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_TABLE_CACHE: dict = {}


def normal_table(std: float, dtype: str) -> np.ndarray:
    """65536 normal quantiles scaled by ``std``, as fp32 values exactly representable in ``dtype``."""
    key = (float(std), dtype)
    if key not in _TABLE_CACHE:
        from scipy.special import ndtri
        j = np.arange(65536, dtype=np.float64)
        t = (std * ndtri((j + 0.5) / 65536.0)).astype(np.float32)
        if dtype == "bf16":
            t = bf16_bits_to_f32(f32_to_bf16_bits(t))
        elif dtype != "f32":
            raise ValueError(dtype)
        _TABLE_CACHE[key] = t
    return _TABLE_CACHE[key]


# ----------------------------------------------------------------------------- numpy backend
def _fmix32_np(h: np.ndarray) -> np.ndarray:
    h = h ^ (h >> np.uint64(16))
    h = (h * np.uint64(_C1)) & np.uint64(M32)
    h = h ^ (h >> np.uint64(13))
    h = (h * np.uint64(_C2)) & np.uint64(M32)
    h = h ^ (h >> np.uint64(16))
    return h


def words_np(start: int, count: int, seed: int, tensor_id: int) -> np.ndarray:
    """u(i) for i in [start, start+count) as uint64 holding 32-bit values."""
    if start < 0 or start + count > 2 ** 32:
        raise ValueError("element index out of the 32-bit counter range")
    k1, k2 = stream_keys(seed, tensor_id)
    i = np.arange(start, start + count, dtype=np.uint64)
    return _fmix32_np(_fmix32_np(i ^ np.uint64(k1)) ^ np.uint64(k2))


def normal_np(shape, seed: int, tensor_id: int, std: float, dtype: str,
              chunk: int = 1 << 24) -> np.ndarray:
    """Normal tensor as fp32 values (bf16-representable when ``dtype == 'bf16'``)."""
    n = int(np.prod(shape))
    table = normal_table(std, dtype)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        out[s:s + c] = table[(words_np(s, c, seed, tensor_id) >> np.uint64(16)).astype(np.int64)]
    return out.reshape(shape)


def tokens_np(shape, seed: int, tensor_id: int, n: int) -> np.ndarray:
    """Token ids uniform in [0, n) as int32."""
    cnt = int(np.prod(shape))
    u = words_np(0, cnt, seed, tensor_id)
    return ((u * np.uint64(n)) >> np.uint64(32)).astype(np.int32).reshape(shape)


# ----------------------------------------------------------------------------- torch backend
def _mul32_t(h, c: int):
    # (h * c) mod 2^32 for h < 2^32, without leaving int64.
    hi, lo = c >> 16, c & 0xFFFF
    return ((((h * hi) & 0xFFFF) << 16) + h * lo) & M32


def _fmix32_t(h):
    h = h ^ (h >> 16)
    h = _mul32_t(h, _C1)
    h = h ^ (h >> 13)
    h = _mul32_t(h, _C2)
    h = h ^ (h >> 16)
    return h


def words_torch(start: int, count: int, seed: int, tensor_id: int, device="cpu"):
    import torch
    if start < 0 or start + count > 2 ** 32:
        raise ValueError("element index out of the 32-bit counter range")
    k1, k2 = stream_keys(seed, tensor_id)
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    return _fmix32_t(_fmix32_t(i ^ k1) ^ k2)


def normal_torch(shape, seed: int, tensor_id: int, std: float, dtype: str, device="cpu",
                 chunk: int = 1 << 26, out=None):
    """Same values as :func:`normal_np`, as a torch tensor of ``dtype`` on ``device``."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    n = 1
    for s in shape:
        n *= int(s)
    table = torch.from_numpy(normal_table(std, dtype)).to(device=device, dtype=tdt)
    if out is None:
        out = torch.empty(n, dtype=tdt, device=device)
    flat = out.view(-1)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        flat[s:s + c] = table[words_torch(s, c, seed, tensor_id, device) >> 16]
    return out.view(*shape)


def tokens_torch(shape, seed: int, tensor_id: int, n: int, device="cpu"):
    import torch
    cnt = 1
    for s in shape:
        cnt *= int(s)
    u = words_torch(0, cnt, seed, tensor_id, device)
    # u < 2^32 and n < 2^31, so split the product to stay within int64.
    hi = (u >> 16) * n
    lo = (u & 0xFFFF) * n
    r = (hi + (lo >> 16)) >> 16
    return r.to(torch.int32).view(*shape)

"""ctypes binding of libdllm.so: the C ABI of include/dllm.h under the same names.

Argument marshalling only: every step of the decode runs in the HIP library.  PyTorch is used
for device memory (weights, workspace, debug buffers) and the stream handle.  Loading fails
loudly when the library has not been built; there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdllm.so")

DLLM_OK, DLLM_EINVAL, DLLM_ENOSPACE, DLLM_ESTATE, DLLM_EHIP, DLLM_EINTERNAL = 0, -1, -2, -3, -4, -5
DLLM_F32, DLLM_BF16 = 0, 1
DLLM_NO_CACHE, DLLM_PREFIX_CACHE, DLLM_DUAL_CACHE = 0, 1, 2
LAYER_TENSORS = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"]
ERR_NAMES = {DLLM_EINVAL: "EINVAL", DLLM_ENOSPACE: "ENOSPACE", DLLM_ESTATE: "ESTATE",
             DLLM_EHIP: "EHIP", DLLM_EINTERNAL: "EINTERNAL"}


class dllm_cfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("mask_id", C.c_int32),
                ("rms_eps", C.c_float), ("rope_base", C.c_float), ("logit_scale", C.c_float),
                ("dtype", C.c_int32),
                ("batch", C.c_int32), ("prompt_len", C.c_int32), ("gen_length", C.c_int32),
                ("block_size", C.c_int32), ("steps", C.c_int32), ("threshold", C.c_float),
                ("use_cache", C.c_int32), ("refresh_every_step", C.c_int32),
                ("suffix_window", C.c_int32), ("attention", C.c_int32),
                ("exit_steps", C.c_int32), ("exit_floor", C.c_float),
                ("first_threshold", C.c_float),
                ("stream", C.c_void_p)]


class dllm_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layer", C.POINTER(C.c_void_p))]


class dllm_stats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("full_forwards", C.c_int64),
                ("cached_forwards", C.c_int64), ("committed", C.c_int64),
                ("commits_hist", C.c_int64 * 9), ("ms_refresh", C.c_double),
                ("ms_step", C.c_double), ("nan_count", C.c_int64),
                ("early_exits", C.c_int64)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["commits_hist"] = list(self.commits_hist)
        return d


DLLM_KC_GEMM_SKINNY, DLLM_KC_GEMM_TILED, DLLM_KC_ATTENTION, DLLM_KC_COUNT = 0, 1, 2, 3
KC_NAMES = ["gemm_skinny", "gemm_tiled", "attention"]


class dllm_kernel_prof(C.Structure):
    _fields_ = [("launches", C.c_int64), ("ms", C.c_double), ("bytes", C.c_double),
                ("flops", C.c_double)]


class DllmError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


_P = C.c_void_p
_I32P = C.POINTER(C.c_int32)
_SIGS = {
    "dllm_validate_cfg": (C.c_int, [C.POINTER(dllm_cfg)]),
    "dllm_workspace_bytes": (C.c_int, [C.POINTER(dllm_cfg), C.POINTER(C.c_size_t)]),
    "dllm_create": (C.c_int, [C.POINTER(dllm_weights), C.POINTER(dllm_cfg), _P, C.c_size_t,
                              C.POINTER(_P)]),
    "dllm_create_static_scratch": (C.c_int, [C.POINTER(dllm_weights), C.POINTER(dllm_cfg), _P,
                                             C.POINTER(C.c_size_t), C.POINTER(_P)]),
    "dllm_prefill": (C.c_int, [_P, _I32P]),
    "dllm_block_begin": (C.c_int, [_P, C.c_int32]),
    "dllm_denoise_step": (C.c_int, [_P, _I32P, _I32P]),
    "dllm_generate": (C.c_int, [_P, _I32P, _I32P, C.POINTER(dllm_stats)]),
    "dllm_get_tokens": (C.c_int, [_P, _I32P]),
    "dllm_set_tokens": (C.c_int, [_P, _I32P]),
    "dllm_get_step_info": (C.c_int, [_P, _I32P, C.POINTER(C.c_float), C.POINTER(C.c_float),
                                     C.POINTER(C.c_uint8)]),
    "dllm_debug_block_logits": (C.c_int, [_P, _P]),
    "dllm_get_stats": (C.c_int, [_P, C.POINTER(dllm_stats)]),
    "dllm_get_position": (C.c_int, [_P, _I32P, _I32P]),
    "dllm_set_profiling": (C.c_int, [_P, C.c_int]),
    "dllm_get_profile": (C.c_int, [_P, C.POINTER(dllm_kernel_prof)]),
    "dllm_last_error": (C.c_char_p, [_P]),
    "dllm_destroy": (None, [_P]),
}
EXPORTS = list(_SIGS)

_LIB = None


def load(path: str | None = None):
    """Load libdllm.so once.  Raises if it is missing (build it with build.py first)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build the HIP library first "
                           "(python -m diffusion_block_denoise_amd.build)")
    # torch first: its HIP runtime (torch/lib/libamdhip64.so, soname libamdhip64.so.7) is then the
    # one the library's libamdhip64.so.7 dependency binds to.  Loaded the other way round, ROCm's
    # copy comes in first and torch, which asks for the unversioned name, loads its own: two HIP
    # runtimes in one process, and the second to touch the GPU finds no device.
    import torch  # noqa: F401
    lib = C.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _LIB = lib
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


def make_cfg(cfg: dict, stream=None, refresh_every_step: bool = False) -> dllm_cfg:
    """dllm_cfg from a workload dict (synth.configs fields)."""
    c = dllm_cfg()
    for k in ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
              "mask_id", "batch", "prompt_len", "gen_length", "block_size", "steps", "use_cache"):
        setattr(c, k, int(cfg[k]))
    c.rms_eps = float(cfg["rms_eps"])
    c.rope_base = float(cfg["rope_base"])
    c.logit_scale = float(cfg["logit_scale"])
    c.threshold = float(cfg["threshold"])
    c.dtype = DLLM_BF16 if cfg["dtype"] == "bf16" else DLLM_F32
    c.refresh_every_step = 1 if refresh_every_step else 0
    c.suffix_window = int(cfg.get("suffix_window", -1))
    c.attention = {"full": 0, "block_causal": 1}[cfg.get("attention", "full")]
    c.exit_steps = int(cfg.get("exit_steps", 0))
    c.exit_floor = float(cfg.get("exit_floor", 0.9))
    c.first_threshold = float(cfg.get("first_threshold", -1.0))
    c.stream = stream
    return c


def dllm_validate_cfg(cfg: dllm_cfg) -> int:
    return load().dllm_validate_cfg(C.byref(cfg))


def dllm_workspace_bytes(cfg: dllm_cfg) -> int:
    n = C.c_size_t(0)
    rc = load().dllm_workspace_bytes(C.byref(cfg), C.byref(n))
    if rc:
        raise DllmError("dllm_workspace_bytes", rc, "invalid configuration")
    return n.value


def static_scratch_workspace_bytes(cfg: dllm_cfg) -> int:
    """Workspace bytes of a static-scratch handle (dllm_create_static_scratch's size query)."""
    lib = load()
    n = C.c_size_t(0)
    rc = lib.dllm_create_static_scratch(None, C.byref(cfg), None, C.byref(n), None)
    if rc:
        raise DllmError("dllm_create_static_scratch", rc, lib.dllm_last_error(None).decode())
    return n.value


class Handle:
    """A dllm_t with the torch tensors it points at (weights, workspace) kept alive.

    Methods mirror the C functions (``dllm_`` prefix dropped) and only marshal arguments.
    ``static_scratch``: create it with dllm_create_static_scratch (scratch in the library's
    static device array, a smaller workspace).
    """

    def __init__(self, cfg: dict, weights: dict, stream=None, refresh_every_step=False,
                 workspace=None, static_scratch=False):
        import torch
        self.lib = load()
        self.cfg = cfg
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        self.stream = stream
        self.c = make_cfg(cfg, stream, refresh_every_step)
        rc = self.lib.dllm_validate_cfg(C.byref(self.c))
        if rc:
            raise DllmError("dllm_validate_cfg", rc, "invalid configuration")
        self.ws_bytes = (static_scratch_workspace_bytes(self.c) if static_scratch
                         else dllm_workspace_bytes(self.c))
        if workspace is None:
            workspace = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device="cuda")
        self.workspace = workspace
        base = workspace.data_ptr()
        aligned = (base + 255) // 256 * 256
        self.weights = weights
        nl = cfg["n_layers"]
        self._layer = (C.c_void_p * (9 * nl))()
        for l in range(nl):
            for j, n in enumerate(LAYER_TENSORS):
                t = weights[f"layers.{l}.{n}"]
                assert t.is_cuda and t.is_contiguous()
                self._layer[9 * l + j] = t.data_ptr()
        self.w = dllm_weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                              weights["lm_head"].data_ptr(),
                              C.cast(self._layer, C.POINTER(C.c_void_p)))
        h = C.c_void_p()
        avail = workspace.numel() - (aligned - base)
        if static_scratch:
            n = C.c_size_t(avail)
            rc = self.lib.dllm_create_static_scratch(C.byref(self.w), C.byref(self.c),
                                                     C.c_void_p(aligned), C.byref(n), C.byref(h))
            fn = "dllm_create_static_scratch"
        else:
            rc = self.lib.dllm_create(C.byref(self.w), C.byref(self.c), C.c_void_p(aligned),
                                      C.c_size_t(avail), C.byref(h))
            fn = "dllm_create"
        if rc:
            raise DllmError(fn, rc, self.lib.dllm_last_error(None).decode())
        self.h = h
        self.B = cfg["batch"]
        self.L = cfg["prompt_len"] + cfg["gen_length"]
        self.Bs = cfg["block_size"]

    def _check(self, fn, rc):
        if rc:
            raise DllmError(fn, rc, self.lib.dllm_last_error(self.h).decode())

    def prefill(self, prompt) -> None:
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        self._check("dllm_prefill", self.lib.dllm_prefill(self.h, _ptr(p, C.c_int32)))

    def block_begin(self, block: int) -> None:
        self._check("dllm_block_begin", self.lib.dllm_block_begin(self.h, int(block)))

    def denoise_step(self):
        n = np.zeros(self.B, dtype=np.int32)
        done = C.c_int32(0)
        self._check("dllm_denoise_step",
                    self.lib.dllm_denoise_step(self.h, _ptr(n, C.c_int32), C.byref(done)))
        return n, bool(done.value)

    def generate(self, prompt):
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        out = np.zeros((self.B, self.L), dtype=np.int32)
        st = dllm_stats()
        self._check("dllm_generate", self.lib.dllm_generate(self.h, _ptr(p, C.c_int32),
                                                            _ptr(out, C.c_int32), C.byref(st)))
        return out, st.as_dict()

    def get_tokens(self):
        x = np.zeros((self.B, self.L), dtype=np.int32)
        self._check("dllm_get_tokens", self.lib.dllm_get_tokens(self.h, _ptr(x, C.c_int32)))
        return x

    def set_tokens(self, x) -> None:
        x = np.ascontiguousarray(x, dtype=np.int32)
        assert x.shape == (self.B, self.L)
        self._check("dllm_set_tokens", self.lib.dllm_set_tokens(self.h, _ptr(x, C.c_int32)))

    def get_step_info(self):
        shp = (self.B, self.Bs)
        tok = np.zeros(shp, np.int32)
        conf = np.zeros(shp, np.float32)
        p2 = np.zeros(shp, np.float32)
        com = np.zeros(shp, np.uint8)
        self._check("dllm_get_step_info",
                    self.lib.dllm_get_step_info(self.h, _ptr(tok, C.c_int32), _ptr(conf, C.c_float),
                                                _ptr(p2, C.c_float), _ptr(com, C.c_uint8)))
        return dict(tok=tok, conf=conf, p2=p2, committed=com.astype(bool))

    def debug_block_logits(self):
        import torch
        out = torch.empty((self.B, self.Bs, self.cfg["vocab"]), dtype=torch.float32,
                          device="cuda")
        self._check("dllm_debug_block_logits",
                    self.lib.dllm_debug_block_logits(self.h, C.c_void_p(out.data_ptr())))
        return out

    def get_stats(self) -> dict:
        st = dllm_stats()
        self._check("dllm_get_stats", self.lib.dllm_get_stats(self.h, C.byref(st)))
        return st.as_dict()

    def get_position(self):
        b, j = C.c_int32(0), C.c_int32(0)
        self._check("dllm_get_position", self.lib.dllm_get_position(self.h, C.byref(b), C.byref(j)))
        return b.value, j.value

    def set_profiling(self, class_mask: int) -> None:
        self._check("dllm_set_profiling", self.lib.dllm_set_profiling(self.h, int(class_mask)))

    def get_profile(self) -> dict:
        arr = (dllm_kernel_prof * DLLM_KC_COUNT)()
        self._check("dllm_get_profile", self.lib.dllm_get_profile(self.h, arr))
        return {KC_NAMES[i]: dict(launches=arr[i].launches, ms=arr[i].ms, bytes=arr[i].bytes,
                                  flops=arr[i].flops) for i in range(DLLM_KC_COUNT)}

    def destroy(self) -> None:
        if getattr(self, "h", None):
            self.lib.dllm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

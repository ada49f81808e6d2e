"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Every source of the library is compiled with the sanitizers on its host side only (device code is
built as usual and never runs here), and linked with tests/abi_host_check.c, which drives the
host-only paths of the C ABI: configuration checks, workspace sizing for every workload (the
split-K planners and their CU schedule model), dllm_create's argument errors and calls on a NULL
handle.  Any sanitizer report fails the run.
"""

import os
import shutil
import subprocess
import sys

import pytest

import synth
from diffusion_block_denoise_amd import build as lib_build
from diffusion_block_denoise_amd import dllm

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# (field, value) changes that make tiny_f32 invalid (the same cases as test_abi's)
BAD = [("dtype", 7), ("n_layers", 0), ("n_heads", 6), ("head_dim", 48), ("mask_id", 512),
       ("vocab", 1), ("gen_length", 60), ("block_size", 0), ("block_size", 512), ("steps", 6),
       ("use_cache", 3), ("batch", 0), ("prompt_len", -1), ("rms_eps", -1.0),
       ("rope_base", 0.0), ("attention", 2)]


def _cfg_init(c) -> str:
    vals = []
    for name, _ in dllm.dllm_cfg._fields_:
        v = getattr(c, name)
        if name == "stream":
            vals.append("0")
        elif isinstance(v, float):
            vals.append(repr(float(v)) + "f")
        else:
            vals.append(str(int(v)))
    return "{" + ", ".join(vals) + "}"


def _cfgs_header() -> str:
    good = [dllm.make_cfg(synth.configs.get(n)) for n in synth.configs.ORDER]
    good.append(dllm.make_cfg(synth.configs.get("llada8b", suffix_window=32)))
    good.append(dllm.make_cfg(synth.configs.get("llada8b_long", attention="block_causal")))
    bad = []
    for field, value in BAD:
        c = dllm.make_cfg(synth.configs.get("tiny_f32"))
        setattr(c, field, value)
        bad.append(c)
    return ("static dllm_cfg GOOD_CFGS[] = {\n  " + ",\n  ".join(_cfg_init(c) for c in good)
            + "\n};\n#define N_GOOD " + str(len(good)) + "\n"
            + "static dllm_cfg BAD_CFGS[] = {\n  " + ",\n  ".join(_cfg_init(c) for c in bad)
            + "\n};\n#define N_BAD " + str(len(bad)) + "\n")


def test_host_paths_under_sanitizers(tmp_path):
    try:
        cc = lib_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not os.path.exists(CLANGXX):
        pytest.skip("ROCm clang++ not available")
    (tmp_path / "cfgs.h").write_text(_cfgs_header())
    # sanitizers on the host side of every source; the device code is built as usual
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = [f for f in lib_build.HIP_FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    procs, objs = [], []
    for src in lib_build.SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([cc, *flags, *san, "-c", os.path.join(lib_build.CSRC, src),
                                       "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for pr in procs:
        out, _ = pr.communicate()
        assert pr.returncode == 0, out
    exe = str(tmp_path / "abi_host_check")
    link = [CLANGXX, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-I", os.path.join(ROOT, "include"), "-I", str(tmp_path),
            "-x", "c", os.path.join(HERE, "abi_host_check.c"), "-x", "none", *objs,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       env=env, timeout=300)
    print(r.stdout, file=sys.stderr)
    assert r.returncode == 0, r.stdout
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout
    assert "abi host checks ok" in r.stdout

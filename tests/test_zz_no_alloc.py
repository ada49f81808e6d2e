"""dllm_create_static_scratch, the allocation-free variant of dllm_create, through the C ABI.

Its handles keep their partial results (split-K tiles, attention key-chunk partials, lm_head
tile partials) in the library's static device array instead of the workspace.  The kernels are
the same, so every output must equal that of a dllm_create handle bit for bit: the token state
of a whole decode, and per step the argmax tokens, confidences, runner-up probabilities, commits
and logits.  Two handles are made in a row, the second for a smaller input, and then the first
is used again (the array keeps the last call's contents; nothing in it may need to start at zero).
"""

import gc

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


def _cfg(**kw):
    base = dict(n_layers=2, d_model=256, n_heads=8, n_kv_heads=2, head_dim=32, ffn_dim=512,
                vocab=1000, mask_id=999, batch=4, prompt_len=40, gen_length=64, block_size=16,
                use_cache=2, random_gains=True, threshold=0.7)
    base.update(kw)
    return synth.configs.get("small_bf16", **base)


def _compare(cfg, ha, hs):
    prompt = synth.prompt_np(cfg)
    xa, sa = ha.generate(prompt)
    xs, ss = hs.generate(prompt)
    assert np.array_equal(xa, xs)
    assert sa["steps"] == ss["steps"] and sa["committed"] == ss["committed"]
    nb = cfg["gen_length"] // cfg["block_size"]
    for b in sorted({0, nb - 1}):
        x0 = synth.block_state_np(cfg, b)
        for h in (ha, hs):
            h.set_tokens(x0)
            h.block_begin(b)
        done = False
        n = 0
        while not done and n < cfg["block_size"]:
            _, done_a = ha.denoise_step()
            _, done = hs.denoise_step()
            assert done_a == done
            ia, i_s = ha.get_step_info(), hs.get_step_info()
            for k in ("tok", "conf", "p2", "committed"):
                assert np.array_equal(ia[k], i_s[k]), (b, n, k)
            la = ha.debug_block_logits().cpu().numpy()
            ls = hs.debug_block_logits().cpu().numpy()
            assert np.array_equal(la, ls), (b, n)
            assert np.array_equal(ha.get_tokens(), hs.get_tokens())
            n += 1


def test_static_scratch_matches_workspace_scratch():
    from diffusion_block_denoise_amd import dllm
    big = _cfg()
    small = _cfg(batch=1, prompt_len=24, gen_length=32, d_model=128, n_heads=4, n_kv_heads=4,
                 ffn_dim=256, vocab=512, mask_id=511)
    c_big, c_small = dllm.make_cfg(big), dllm.make_cfg(small)
    assert dllm.static_scratch_workspace_bytes(c_big) < dllm.dllm_workspace_bytes(c_big)
    _log("case static scratch: first handle (batch 4)")
    Wb = synth.weights_torch(big, device="cuda")
    ha, hs = dllm.Handle(big, Wb), dllm.Handle(big, Wb, static_scratch=True)
    _compare(big, ha, hs)
    _log("case static scratch: second handle, smaller input (batch 1)")
    Ws = synth.weights_torch(small, device="cuda")
    ha2, hs2 = dllm.Handle(small, Ws), dllm.Handle(small, Ws, static_scratch=True)
    _compare(small, ha2, hs2)
    _log("case static scratch: the first handle again")
    _compare(big, ha, hs)
    for h in (ha, hs, ha2, hs2):
        h.destroy()


def test_static_scratch_llada8b_block():
    """The LLaDA-8B shape (83 MB of scratch): one block, refresh and every step, bit-exact."""
    import torch
    from diffusion_block_denoise_amd import dllm
    cfg = synth.configs.get("llada8b")
    _log("case static scratch: llada8b")
    W = synth.weights_torch(cfg, device="cuda")
    ha, hs = dllm.Handle(cfg, W), dllm.Handle(cfg, W, static_scratch=True)
    b = 3
    x0 = synth.block_state_np(cfg, b)
    for h in (ha, hs):
        h.set_tokens(x0)
        h.block_begin(b)
    done = False
    while not done:
        _, da = ha.denoise_step()
        _, done = hs.denoise_step()
        assert da == done
        ia, i_s = ha.get_step_info(), hs.get_step_info()
        for k in ("tok", "conf", "p2", "committed"):
            assert np.array_equal(ia[k], i_s[k]), k
    assert np.array_equal(ha.get_tokens(), hs.get_tokens())
    ha.destroy()
    hs.destroy()
    del ha, hs, W
    gc.collect()
    torch.cuda.empty_cache()


def test_static_scratch_rejects_oversized_and_null():
    import ctypes as C
    from diffusion_block_denoise_amd import dllm
    lib = dllm.load()
    cfg = dllm.make_cfg(_cfg(vocab=1 << 22, mask_id=(1 << 22) - 1, batch=64, block_size=64))
    n = C.c_size_t(0)
    rc = lib.dllm_create_static_scratch(None, C.byref(cfg), None, C.byref(n), None)
    assert rc == dllm.DLLM_ENOSPACE
    assert b"static scratch" in lib.dllm_last_error(None)
    ok = dllm.make_cfg(_cfg())
    assert lib.dllm_create_static_scratch(None, C.byref(ok), None, None, None) == dllm.DLLM_EINVAL

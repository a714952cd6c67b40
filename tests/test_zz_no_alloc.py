"""The allocation-free decode entry point against the existing one, through
the C ABI.

gqa_attention_decode_splitkv_noalloc keeps its split-KV partial states in
the library's own scratch buffer; it must give exactly the output of
gqa_attention_decode_splitkv with a caller workspace (the same kernels),
on two calls in a row, the second with a smaller input (so the buffer holds
the first call's states when the second starts), and refuse a call whose
states would not fit the buffer before launching anything.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import to_f64

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, q, k, v, out, kv_len, sink, scale, tile):
    from gqa_attention_forward_amd import _lib
    st = lib.gqa_attention_decode_splitkv_noalloc(
        q.data_ptr(), _lib.strides3(q.stride()[:3]), k.data_ptr(), _lib.strides3(k.stride()[:3]),
        v.data_ptr(), _lib.strides3(v.stride()[:3]), out.data_ptr(),
        _lib.strides3(out.stride()[:3]), q.shape[0], q.shape[1], k.shape[1], k.shape[2],
        q.shape[3], None if kv_len is None else kv_len.data_ptr(), scale,
        None if sink is None else sink.data_ptr(), tile,
        torch.cuda.current_stream().cuda_stream)
    return st


def _call_workspace(lib, q, k, v, out, kv_len, sink, scale, tile):
    from gqa_attention_forward_amd import _lib
    B, Hq, _, d = q.shape
    nb = ctypes.c_size_t()
    _lib.check(lib.gqa_attention_workspace_size(B, Hq, 1, k.shape[2], d, tile, ctypes.byref(nb)))
    ws = torch.empty(nb.value, dtype=torch.uint8, device=q.device)
    st = lib.gqa_attention_decode_splitkv(
        q.data_ptr(), _lib.strides3(q.stride()[:3]), k.data_ptr(), _lib.strides3(k.stride()[:3]),
        v.data_ptr(), _lib.strides3(v.stride()[:3]), out.data_ptr(),
        _lib.strides3(out.stride()[:3]), B, Hq, k.shape[1], k.shape[2], d,
        None if kv_len is None else kv_len.data_ptr(), scale,
        None if sink is None else sink.data_ptr(), tile, ws.data_ptr(), nb.value,
        torch.cuda.current_stream().cuda_stream)
    return st


def test_noalloc_decode_matches_workspace_decode():
    from gqa_attention_forward_amd import _lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    lib = _lib.load()
    # the decode workload (16 x 32 heads x 8192 keys, splits of 1024: 2.1 MB
    # of partial states), then a smaller one with ragged lengths, a sink and
    # splits of 256 (1.2 MB), then d = 64
    cases = [(16, 32, 8, 8192, 128, 1024, False), (4, 16, 4, 3000, 128, 256, True),
             (3, 8, 2, 5000, 64, 512, True)]
    for B, Hq, Hkv, Skv, d, tile, ragged in cases:
        print(f"[case] noalloc decode B={B} Hq={Hq} Hkv={Hkv} Skv={Skv} d={d} tile={tile}",
              flush=True)
        inp = workloads.make_dense(B, Hq, Hkv, 1, Skv, d, seed=B * 100 + d,
                                   kv_len="random" if ragged else None, sink=ragged,
                                   nan_pad=ragged)
        g = {k_: (v_.to(dev) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in inp.items()}
        a = torch.full_like(g["q"], float("nan"))
        b = torch.full_like(g["q"], float("nan"))
        _lib.check(_call_noalloc(lib, g["q"], g["k"], g["v"], a, g["kv_len"], g["sink"],
                                 inp["scale"], tile))
        _lib.check(_call_workspace(lib, g["q"], g["k"], g["v"], b, g["kv_len"], g["sink"],
                                   inp["scale"], tile))
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        # and the oracle, to the parity bar
        kvl = None if inp["kv_len"] is None else inp["kv_len"].numpy()
        want = oracle.attention_fp64(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                     scale=inp["scale"], kv_len=kvl,
                                     sink=None if inp["sink"] is None else to_f64(inp["sink"]))
        err = np.abs(a.float().cpu().numpy() - want)
        print(f"  max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
        assert err.max() <= 1e-2 and err.mean() <= 1e-3


def test_noalloc_refuses_states_beyond_the_scratch():
    from gqa_attention_forward_amd import _lib
    dev = torch.device("cuda:0")
    lib = _lib.load()
    # 64 x 32 rows x 8 splits x 130 floats = 8,519,680 bytes > 8 MiB
    q = torch.zeros(64, 32, 1, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(64, 8, 8192, 128, dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 7.0)
    st = _call_noalloc(lib, q, k, k, out, None, None, 0.088, 1024)
    assert st == _lib.GQA_ERR_WORKSPACE, lib.gqa_last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing ran
    # the same rows in splits of 2048 fit (4,259,840 bytes)
    _lib.check(_call_noalloc(lib, q, k, k, out, None, None, 0.088, 2048))
    torch.cuda.synchronize()
    assert bool((out == 0).all())

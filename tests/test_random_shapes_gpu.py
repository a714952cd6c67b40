"""GPU parity over randomly drawn shapes: every entry point, head dim, group
size, causal flag and split size in combinations the named cases do not list.

Each case is drawn from a fixed-seed generator and checked in full against the
fp64 oracle, to the bound in bf16_bound.py (the usual bar, and one bf16
spacing where |O| >= 2).
"""

import random

import numpy as np
import pytest
import torch

import oracle
import workloads
from bf16_bound import bf16_spacing, check
from workloads import to_f64


def gqa():
    import gqa_attention_forward_amd as m
    return m


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(inp):
    d = dev()
    return {k: (v.to(d) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _dense_case(r, seed):
    d = r.choice([32, 64, 128, 256])
    G = r.choice([1, 2, 3, 4, 5, 8, 16, 32])
    Hkv = r.choice([1, 2, 3])
    B = r.randint(1, 3)
    Sq = r.choice([1, 1, 2, 7, 16, 33, 100])
    Skv = r.randint(1, 700)
    tile = r.choice([0, 0, 64, 128, 320, 1024])
    use_sink = r.random() < 0.5
    decode = Sq == 1 and tile > 0 and r.random() < 0.5
    fused = decode and G <= 32 and r.random() < 0.5
    causal = (not decode) and r.random() < 0.5
    what = (f"dense d={d} G={G} Hkv={Hkv} B={B} Sq={Sq} Skv={Skv} causal={causal} tile={tile} "
            f"sink={use_sink} decode={decode} fused={fused} seed={seed}")
    print(f"[case] {what}", flush=True)
    inp = workloads.make_dense(B, G * Hkv, Hkv, Sq, Skv, d, seed=seed, kv_len="random",
                               sink=use_sink, nan_pad=True)
    g = to_dev(inp)
    kw = dict(kv_len=g["kv_len"], scale=inp["scale"], sink=g["sink"])
    if decode:
        out = gqa().decode_splitkv(g["q"], g["k"], g["v"], tile_s_kv=tile, fused=fused, **kw)
    else:
        out = gqa().prefill(g["q"], g["k"], g["v"], causal=causal, tile_s_kv=tile, **kw)
    torch.cuda.synchronize()
    want = oracle.attention_fp64(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                 scale=inp["scale"], kv_len=inp["kv_len"].numpy(),
                                 sink=None if inp["sink"] is None else to_f64(inp["sink"]),
                                 causal=causal)
    check(out.float().cpu().numpy(), want, what)


def _paged_case(r, seed):
    d = r.choice([32, 64, 128, 256])
    G = r.choice([1, 2, 3, 4, 5, 8, 16, 32])
    Hkv = r.choice([1, 2, 3])
    B = r.randint(1, 4)
    causal = r.random() < 0.5
    tile = r.choice([0, 0, 64, 128, 320, 1024])
    append = r.random() < 0.4
    top = max(1, 32 // G) if append else r.choice([1, 4, 40])
    q_lens = [r.randint(0 if r.random() < 0.1 else 1, top) for _ in range(B)]
    if sum(q_lens) == 0:
        q_lens[0] = 1
    kv_lens = [max(q, r.randint(0, 900)) for q in q_lens]
    what = (f"paged d={d} G={G} Hkv={Hkv} q_lens={q_lens} kv_lens={kv_lens} causal={causal} "
            f"tile={tile} append={append} seed={seed}")
    print(f"[case] {what}", flush=True)
    w = workloads.make_paged(B=B, Hq=G * Hkv, Hkv=Hkv, d=d, q_lens=q_lens, kv_lens=kv_lens,
                             seed=seed)
    g = to_dev(w)
    kw = dict(max_q_len=w["max_q_len"], scale=w["scale"], sink=g["sink"], causal=causal,
              tile_s_kv=tile)
    if append:
        kn, vn, kh, vh = workloads.take_new_kv(w)
        kc, vc = kh.to(dev()), vh.to(dev())
        out = gqa().paged_append(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"],
                                 g["kv_len"], kn.to(dev()), vn.to(dev()), **kw)
    else:
        out = gqa().paged(g["q"], g["cu_seqlens_q"], g["k_cache"], g["v_cache"],
                          g["page_table"], g["kv_len"], **kw)
    torch.cuda.synchronize()
    want = oracle.paged_attention_fp64(to_f64(w["q"]), w["cu_seqlens_q"].numpy(),
                                       to_f64(w["k_cache"]), to_f64(w["v_cache"]),
                                       w["page_table"].numpy(), w["kv_len"].numpy(),
                                       scale=w["scale"], page_size=64, sink=to_f64(w["sink"]),
                                       causal=causal)
    check(out.float().cpu().numpy(), want, what)
    if append:
        assert torch.equal(kc.cpu().view(torch.int16), w["k_cache"].view(torch.int16))
        assert torch.equal(vc.cpu().view(torch.int16), w["v_cache"].view(torch.int16))


def test_bound_is_one_spacing_only_above_two():
    assert bf16_spacing(1.99) == 2.0 ** -7 and bf16_spacing(2.0) == 2.0 ** -6
    assert bf16_spacing(-3.5) == 2.0 ** -6 and bf16_spacing(0.0) == 0.0


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [1234, 777, 4242])
def test_random_shapes(seed):
    r = random.Random(seed)
    for i in range(120):
        case_seed = seed * 1000 + i
        if r.random() < 0.6:
            _dense_case(r, case_seed)
        else:
            _paged_case(r, case_seed)

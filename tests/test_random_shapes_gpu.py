"""GPU parity over randomly drawn shapes: every entry point, head dim, group
size, causal flag and split size in combinations the named cases do not list.

Each case is drawn from a fixed-seed generator and checked in full against the
fp64 oracle, to the bound in bf16_bound.py: the usual bar, where an element
above 1e-2 must stay within the rounding bound derived there from the oracle's
weights (each such element is printed and counted).
"""

import random

import numpy as np
import pytest
import torch

import oracle
import workloads
import bf16_bound
from bf16_bound import check
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
    d = r.choice([32, 64, 128, 256, 512])
    G = r.choice([1, 2, 3, 4, 5, 8, 16, 32])
    Hkv = r.choice([1, 2, 3])
    B = r.randint(1, 3)
    Sq = r.choice([1, 1, 2, 7, 16, 33, 100])
    Skv = r.randint(1, 700)
    tile = r.choice([0, 0, 64, 128, 320, 1024])
    use_sink = r.random() < 0.5
    decode = Sq == 1 and tile > 0 and r.random() < 0.5
    fused = decode and G <= 32 and d <= 256 and r.random() < 0.5
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
    q64, k64, v64 = to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"])
    snk = None if inp["sink"] is None else to_f64(inp["sink"])
    kvl = inp["kv_len"].numpy()
    want = oracle.attention_fp64(q64, k64, v64, scale=inp["scale"], kv_len=kvl, sink=snk,
                                 causal=causal)
    spread = lambda idx: bf16_bound.spread_dense(q64, k64, v64, scale=inp["scale"],  # noqa: E731
                                                 kv_len=kvl, sink=snk, causal=causal,
                                                 want=want, idx=idx)
    check(out.float().cpu().numpy(), want, what, spread)


def _paged_case(r, seed):
    d = r.choice([32, 64, 128, 256, 512])
    G = r.choice([1, 2, 3, 4, 5, 8, 16, 32])
    Hkv = r.choice([1, 2, 3])
    B = r.randint(1, 4)
    causal = r.random() < 0.5
    tile = r.choice([0, 0, 64, 128, 320, 1024])
    append = d <= 256 and r.random() < 0.4
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
    # (with append, w's pools already hold the new rows: the attention's keys)
    spread = lambda idx: bf16_bound.spread_paged(w, causal=causal, want=want, idx=idx)  # noqa: E731
    check(out.float().cpu().numpy(), want, what, spread)
    if append:
        assert torch.equal(kc.cpu().view(torch.int16), w["k_cache"].view(torch.int16))
        assert torch.equal(vc.cpu().view(torch.int16), w["v_cache"].view(torch.int16))


def test_spacing():
    sp = bf16_bound.bf16_spacing
    assert sp(1.99) == 2.0 ** -7 and sp(2.0) == 2.0 ** -6
    assert sp(-3.5) == 2.0 ** -6 and sp(0.0) == 0.0 and sp(0.75) == 2.0 ** -8


def test_rounding_bound_covers_simulated_rounding():
    """CPU check of the derivation: rows of 1-6 keys with values spread far
    from O, weights rounded to bf16 (RNE, through torch), normalised by the
    sum of the rounded weights, O rounded to bf16.  Every error stays within
    rounding_bound, some exceed 1e-2 (so the exception is needed), and the
    bound is not loose by more than a small factor on the worst rows."""
    rng = np.random.default_rng(0)
    worst, above = 0.0, 0
    for _ in range(4000):
        n = int(rng.integers(1, 7))
        s = rng.normal(0.0, 2.0, n)
        v = rng.normal(0.0, 3.0, n)
        sink = rng.normal() if rng.random() < 0.5 else -np.inf
        m = max(s.max(), sink)
        off = rng.uniform(0, 8)  # the kernels' reference may lag the max by up to 8 (log2)
        p = np.exp2((s - m) * 1.4426950408889634 + off)
        ps = np.exp2((sink - m) * 1.4426950408889634 + off) if sink > -np.inf else 0.0
        w = p / (p.sum() + ps)
        o = float(np.sum(w * v))
        pr = torch.tensor(p, dtype=torch.float32).to(torch.bfloat16).double().numpy()
        ot = np.sum(pr * v) / (pr.sum() + ps)
        ob = float(torch.tensor(ot, dtype=torch.float32).to(torch.bfloat16).double())
        err = abs(ob - o)
        bound = float(bf16_bound.rounding_bound(o, np.sum(w * np.abs(v - o))))
        assert err <= bound, (err, bound, n)
        above += err > bf16_bound.MAX_ABS
        worst = max(worst, err / bound)
    assert above > 0 and worst > 0.4


def test_spread_helpers():
    """sum_j w_j |v_j - O| from the helpers equals the sum written out from
    the softmax of the scores (two keys plus a sink), and the paged helper
    agrees with the dense one on the same sequence."""
    from scipy.special import softmax
    w = workloads.make_paged(B=2, Hq=4, Hkv=2, d=8, q_lens=[2, 3], kv_lens=[2, 70], seed=3)
    q, sink = to_f64(w["q"]), to_f64(w["sink"])
    ks = oracle.gather_paged_fp64(to_f64(w["k_cache"]), w["page_table"].numpy(),
                                  w["kv_len"].numpy(), 64)
    vs = oracle.gather_paged_fp64(to_f64(w["v_cache"]), w["page_table"].numpy(),
                                  w["kv_len"].numpy(), 64)
    want = oracle.paged_attention_fp64(q, w["cu_seqlens_q"].numpy(), to_f64(w["k_cache"]),
                                       to_f64(w["v_cache"]), w["page_table"].numpy(),
                                       w["kv_len"].numpy(), scale=w["scale"], page_size=64,
                                       sink=sink, causal=True)
    # sequence 0: 2 queries over 2 keys (bottom-right causal: row 0 sees key 0)
    t, h, e = 1, 3, 5
    s_ = w["scale"] * ks[0][h // 2] @ q[t, h]
    p_ = softmax(np.append(s_, sink[h]))
    direct = float(np.sum(p_[:2] * np.abs(vs[0][h // 2][:, e] - want[t, h, e])))
    got = bf16_bound.spread_paged(w, causal=True, want=want, idx=(np.array([t]), np.array([h]),
                                                                   np.array([e])))
    assert abs(got[0] - direct) <= 1e-12
    # sequence 1 through the dense helper: its rows as a [1, Hq, 3, d] problem
    qd = q[2:5].transpose(1, 0, 2)[None]
    kd = np.stack(ks[1])[None]
    vd = np.stack(vs[1])[None]
    wd = oracle.attention_fp64(qd, kd, vd, scale=w["scale"], sink=sink, causal=True)
    idx_d = (np.array([0, 0]), np.array([0, 3]), np.array([2, 1]), np.array([7, 0]))
    dense = bf16_bound.spread_dense(qd, kd, vd, scale=w["scale"], kv_len=[70], sink=sink,
                                    causal=True, want=wd, idx=idx_d)
    paged = bf16_bound.spread_paged(w, causal=True, want=want,
                                    idx=(np.array([4, 3]), np.array([0, 3]), np.array([7, 0])))
    np.testing.assert_allclose(dense, paged, rtol=1e-12)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [1234, 777, 4242, 11, 22, 33])
def test_random_shapes(seed):
    r = random.Random(seed)
    for i in range(120):
        case_seed = seed * 1000 + i
        if r.random() < 0.6:
            _dense_case(r, case_seed)
        else:
            _paged_case(r, case_seed)

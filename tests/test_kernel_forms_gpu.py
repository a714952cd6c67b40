"""GPU parity for launch shapes that the named workloads do not reach.

The host picks a kernel form from the rows per (b, kv head), the head dim,
the split count and the grid size (stream kernel with 2 or 4 waves, one or
two 16-column blocks; shared-tile prefill kernel with 2, 4 or 8 waves, one
or two key groups; with or without non-temporal loads).  Small test shapes
land in the small-grid forms, so these families build grids of 256 to 511
(b, kv head) pairs, where the 2-wave stream forms and the one-group 8-wave
forms are chosen, and check each against the fp64 oracle in full, to the
bound in bf16_bound.py (random kv lengths give rows that see few keys; an
element above 1e-2 must stay within the rounding bound derived there, and is
printed and counted).

Family A: short groups (4 or 32 rows; two q-tiles at d = 256) over
B x Hkv = 256, one pass and one split of 64 keys, dense and paged.
Family B: 128-, 256- and 512-row groups over B x Hkv = 288, at d = 64 and
128, one pass and splits of 64 keys, dense and paged, causal.
Head-major pools: a paged cache stored [n_pages, Hkv, 64, d] and passed by
strides gives the token-major pool's result bit for bit (at d = 128 and up
to 16 rows the two pools take the stream kernel's two K load forms: whole
rows staged through LDS, and straight into the MFMA operand).
With the named workloads and the other GPU tests, these launch every kernel
form the library builds (a kernel trace of the GPU suite lists them).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bf16_bound
from bf16_bound import check
from workloads import to_f64

pytestmark = pytest.mark.gpu


def gqa():
    import gqa_attention_forward_amd as m
    return m


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(inp):
    d = dev()
    return {k: (v.to(d) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_case(layout, B, Hkv, G, Sq, Skv, d, tile, causal, seed):
    what = f"{layout} B={B} Hkv={Hkv} G={G} Sq={Sq} Skv={Skv} d={d} tile={tile} causal={causal}"
    print(f"[case] {what}", flush=True)
    m = gqa()
    if layout == "dense":
        inp = workloads.make_dense(B, Hkv * G, Hkv, Sq, Skv, d, seed=seed, kv_len="random",
                                   sink=True, nan_pad=True)
        g = to_dev(inp)
        out = m.prefill(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=inp["scale"],
                        sink=g["sink"], causal=causal, tile_s_kv=tile)
        torch.cuda.synchronize()
        q64, k64, v64 = to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"])
        kvl, snk = inp["kv_len"].numpy(), to_f64(inp["sink"])
        want = oracle.attention_fp64(q64, k64, v64, scale=inp["scale"], kv_len=kvl, sink=snk,
                                     causal=causal)
        spread = lambda idx: bf16_bound.spread_dense(  # noqa: E731
            q64, k64, v64, scale=inp["scale"], kv_len=kvl, sink=snk, causal=causal, want=want,
            idx=idx)
    else:
        r = np.random.default_rng(seed)
        q_lens = [int(x) for x in r.integers(1, Sq + 1, B)]
        q_lens[0] = Sq
        kv_lens = [max(q, int(x)) for q, x in zip(q_lens, r.integers(1, Skv + 1, B))]
        w = workloads.make_paged(B=B, Hq=Hkv * G, Hkv=Hkv, d=d, q_lens=q_lens, kv_lens=kv_lens,
                                 seed=seed)
        g = to_dev(w)
        out = m.paged(g["q"], g["cu_seqlens_q"], g["k_cache"], g["v_cache"], g["page_table"],
                      g["kv_len"], max_q_len=w["max_q_len"], scale=w["scale"], sink=g["sink"],
                      causal=causal, tile_s_kv=tile)
        torch.cuda.synchronize()
        want = oracle.paged_attention_fp64(to_f64(w["q"]), w["cu_seqlens_q"].numpy(),
                                           to_f64(w["k_cache"]), to_f64(w["v_cache"]),
                                           w["page_table"].numpy(), w["kv_len"].numpy(),
                                           scale=w["scale"], page_size=64,
                                           sink=to_f64(w["sink"]), causal=causal)
        spread = lambda idx: bf16_bound.spread_paged(w, causal=causal, want=want, idx=idx)  # noqa: E731
    check(out.float().cpu().numpy(), want, what, spread)


# Family A: 64 x 4 = 256 (b, kv head) pairs, G = 4; one split of 64 keys
# (Skv <= 64) or one pass over 200 keys
@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("Sq", [1, 8])
@pytest.mark.parametrize("layout", ["dense", "paged"])
@pytest.mark.parametrize("tile", [0, 64])
def test_short_groups_wide_grid(d, Sq, layout, tile):
    Skv = 64 if tile else 200
    run_case(layout, 64, 4, 4, Sq, Skv, d, tile, Sq > 1, seed=200 + d + Sq + tile)


# Family B: 72 x 4 = 288 (b, kv head) pairs, G = 4; groups of 128, 256 and
# 512 rows over 100 keys (two tiles, the last one ragged)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq", [32, 64, 128])
@pytest.mark.parametrize("layout", ["dense", "paged"])
@pytest.mark.parametrize("tile", [0, 64])
def test_large_groups_wide_grid(d, Sq, layout, tile):
    run_case(layout, 72, 4, 4, Sq, 100, d, tile, True, seed=300 + d + Sq + tile)


# The remaining single-q-tile forms: paged one pass with 64-row groups at
# d = 128 and 256, and at d = 32 a split and one pass with 64- and 128-row
# groups (the 2- and 4-wave forms)
@pytest.mark.parametrize("d,Sq,tile,seed", [(128, 16, 0, 528), (256, 16, 0, 656), (32, 16, 64, 432),
                                            (32, 16, 0, 433), (32, 32, 0, 434)])
def test_paged_64_row_groups(d, Sq, tile, seed):
    run_case("paged", 6, 2, 4, Sq, 300, d, tile, True, seed=seed)


# Paged splits on the 2-wave stream kernel: 32 x 4 pairs x 2 splits of 64
# keys (the pools pad sequences to 128 keys) = 256 workgroups, below the 512
# at which short groups move to the shared-tile kernel
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("Sq", [1, 8])
def test_paged_split_stream_wide_grid(d, Sq):
    run_case("paged", 32, 4, 4, Sq, 128, d, 64, Sq > 1, seed=500 + d + Sq)


# Paged pools with one kv head (row stride d, so the stream kernel loads K
# in MFMA operand shape) over 256 sequences: the 2-wave stream forms, one
# pass and splits of 64 keys (token-major pools with several kv heads take
# the whole-row K forms instead)
@pytest.mark.parametrize("tile", [0, 64])
def test_paged_one_head_wide_grid(tile):
    run_case("paged", 256, 1, 4, 1, 128, 128, tile, False, seed=700 + tile)


# The pool stored head-major ([n_pages, Hkv, 64, d]) and passed through the
# stride arguments as the same logical [n_pages, 64, Hkv, d] view: the
# result must match the oracle and, bit for bit, the token-major pool's.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq", [1, 8])
@pytest.mark.parametrize("tile", [0, 64])
def test_paged_head_major_pool(d, Sq, tile):
    B, Hkv, G = 6, 2, 4
    print(f"[case] head-major pool d={d} Sq={Sq} tile={tile}", flush=True)
    m = gqa()
    r = np.random.default_rng(600 + d + Sq + tile)
    q_lens = [int(x) for x in r.integers(1, Sq + 1, B)]
    kv_lens = [max(q, int(x)) for q, x in zip(q_lens, r.integers(1, 300, B))]
    w = workloads.make_paged(B=B, Hq=Hkv * G, Hkv=Hkv, d=d, q_lens=q_lens, kv_lens=kv_lens,
                             seed=600 + d)
    g = to_dev(w)
    kh = g["k_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vh = g["v_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert kh.stride(1) == d and kh.stride(2) == 64 * d
    outs = []
    for kc, vc in ((g["k_cache"], g["v_cache"]), (kh, vh)):
        outs.append(m.paged(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"], g["kv_len"],
                            max_q_len=w["max_q_len"], scale=w["scale"], sink=g["sink"],
                            causal=Sq > 1, tile_s_kv=tile))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    want = oracle.paged_attention_fp64(to_f64(w["q"]), w["cu_seqlens_q"].numpy(),
                                       to_f64(w["k_cache"]), to_f64(w["v_cache"]),
                                       w["page_table"].numpy(), w["kv_len"].numpy(),
                                       scale=w["scale"], page_size=64, sink=to_f64(w["sink"]),
                                       causal=Sq > 1)
    check(outs[1].float().cpu().numpy(), want, f"head-major pool d={d} Sq={Sq} tile={tile}",
          lambda idx: bf16_bound.spread_paged(w, causal=Sq > 1, want=want, idx=idx))

"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance (over valid output positions, every d): max-abs 1e-2 and mean-abs
1e-3 against the oracle on the same bf16 inputs.  Where the result is fixed
exactly (one visible key, an all-masked row), the test is bit-exact.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import to_f64

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def gqa():
    import gqa_attention_forward_amd as m
    return m


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def note(msg):
    print(f"[case] {msg}", flush=True)


def assert_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    print(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} max|O|={np.abs(want).max(initial=0):.3f}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max {mx} mean {mean}"


def to_dev(inp):
    d = dev()
    return {k: (v.to(d) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def run_dense(inp, *, causal=False, tile=0, use_sink=True, decode=False):
    g = to_dev(inp)
    kw = dict(kv_len=g["kv_len"], scale=inp["scale"], sink=g["sink"] if use_sink else None)
    if decode:
        out = gqa().decode_splitkv(g["q"], g["k"], g["v"], tile_s_kv=tile, **kw)
    else:
        out = gqa().prefill(g["q"], g["k"], g["v"], causal=causal, tile_s_kv=tile, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_dense(inp, *, causal=False, use_sink=True):
    kvl = None if inp["kv_len"] is None else inp["kv_len"].numpy()
    snk = to_f64(inp["sink"]) if use_sink else None
    return oracle.attention_fp64(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                 scale=inp["scale"], kv_len=kvl, sink=snk, causal=causal)


# ---------------------------------------------------------------- named workloads

def test_tiny_prefill_full():
    c = workloads.CASES["tiny_prefill"]
    note(f"tiny_prefill {c}")
    inp = workloads.make_case(c)
    assert_close(run_dense(inp), oracle_dense(inp), "tiny_prefill")


def _sampled_rows(inp, out, rows, causal):
    q, k, v = inp["q"], inp["k"].float().numpy(), inp["v"].float().numpy()
    b, h, i = rows
    want = oracle.attention_rows_fp64(q.float().numpy(), k, v, b, h, i, scale=inp["scale"],
                                      kv_len=inp["kv_len"].numpy(), causal=causal)
    return out[b, h, i], want


def _rows(c, n, seed):
    r = np.random.default_rng(seed)
    b = r.integers(0, c.B, n)
    h = r.integers(0, c.Hq, n)
    i = r.integers(0, c.Sq, n)
    i[:4] = [0, c.Sq - 1, c.Sq // 2, max(0, c.Sq - 2)]  # include the edges
    return b, h, i


# The decode and short-q workloads at full size, in the launch configuration
# the benchmark times (decode: splits of 1024; short-q: splits of 2048, and
# one pass), compared with the oracle at every output element.
@pytest.mark.parametrize("name,tile", [("decode_splitkv", 1024), ("decode_splitkv_d256", 1024),
                                       ("decode_splitkv_d512", 1024),
                                       ("shortq_longkv", 2048), ("shortq_longkv", 4096),
                                       ("shortq_longkv", 0)])
def test_full_size_in_full(name, tile):
    c = workloads.CASES.get(name) or workloads.HEAD_DIM_CASES[name]
    note(f"{name} full size, every element, tile={tile} {c}")
    inp = workloads.make_case(c)
    out = run_dense(inp, tile=tile, use_sink=False, decode=c.decode)
    assert_close(out, oracle_dense(inp, use_sink=False), f"{name} tile={tile} (all {out.size} elements)")


def causal_block_rows(c, seed):
    """Rows of a causal workload that reach every workgroup of every kernel
    form: for each (b, kv head) and each block of 32 query positions (a
    workgroup covers 32 or 64 positions at G = 4), the block's first row
    (first position, first head of the group), its last row (last position,
    last head) and one drawn row in between; these are the first and last
    rows of the block's diagonal key tiles."""
    r = np.random.default_rng(seed)
    G = c.G
    bb, hh, ii = [], [], []
    for b in range(c.B):
        for g in range(c.Hkv):
            for p0 in range(0, c.Sq, 32):
                p1 = min(c.Sq, p0 + 32) - 1
                for p, h in ((p0, g * G), (p1, g * G + G - 1),
                             (int(r.integers(p0, p1 + 1)), g * G + int(r.integers(0, G)))):
                    bb.append(b)
                    hh.append(h)
                    ii.append(p)
    return np.array(bb), np.array(hh), np.array(ii)


@pytest.mark.parametrize("name", ["causal_prefill", "causal_prefill_d32", "causal_prefill_d256",
                                  "causal_prefill_d512"])
def test_causal_full_size_every_workgroup(name):
    c = workloads.CASES.get(name) or workloads.HEAD_DIM_CASES[name]
    note(f"{name} full size {c}")
    inp = workloads.make_case(c)
    out = run_dense(inp, causal=True, use_sink=False)
    assert out.shape == (c.B, c.Hq, c.Sq, c.d)
    assert np.all(np.isfinite(out))
    b, h, i = causal_block_rows(c, 7)
    want = oracle.attention_rows_fp64(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]), b, h,
                                      i, scale=inp["scale"], kv_len=inp["kv_len"].numpy(),
                                      causal=True)
    assert_close(out[b, h, i], want, f"{name} ({b.size} rows, every 32-position block)")


@pytest.mark.parametrize("layout", ["prefill", "decode"])
def test_mqa_zero_kv_head_stride(layout):
    """MQA through a zero K/V head stride (nvfp4-megamoe-kernel commit log,
    the batched multi-head decode commit): K/V of one head seen as Hkv heads
    by expand(), so every query head reads the same rows.  The result must be
    the oracle's MQA (Hkv = 1) result."""
    B, Hq, d = 2, 8, 128
    Sq, Skv, tile = (40, 700, 0) if layout == "prefill" else (1, 3000, 1024)
    note(f"MQA zero head stride {layout} B={B} Hq={Hq} Sq={Sq} Skv={Skv}")
    inp = workloads.make_dense(B, Hq, 1, Sq, Skv, d, seed=17, kv_len="random", sink=True,
                               nan_pad=True)
    g = to_dev(inp)
    want = oracle_dense(inp, causal=layout == "prefill")
    for hkv in (Hq, 2):
        k = g["k"].expand(B, hkv, Skv, d)
        v = g["v"].expand(B, hkv, Skv, d)
        assert k.stride(1) == 0
        kw = dict(kv_len=g["kv_len"], scale=inp["scale"], sink=g["sink"])
        if layout == "prefill":
            out = gqa().prefill(g["q"], k, v, causal=True, **kw)
        else:
            out = gqa().decode_splitkv(g["q"], k, v, tile_s_kv=tile, **kw)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy(), want, f"MQA {layout} via {hkv} aliased kv heads")


def test_wide_key_row_stride():
    """K/V rows 2^25 - 8 elements apart (the largest key-row stride the
    library accepts): the 64-key prefill tiles and the 32-key stream tiles
    address up to 63 rows past a tile's first row in 32-bit byte offsets.
    About 6.7 GB per tensor on the device."""
    stride = (1 << 25) - 8
    B, Hq, Skv, d = 1, 4, 100, 128
    note(f"key-row stride {stride} elements, Skv={Skv}")
    D = dev()
    for Sq in (64, 1):
        inp = workloads.make_dense(B, Hq, 1, Sq, Skv, d, seed=19)
        ks = torch.empty((Skv - 1) * stride + d, dtype=torch.bfloat16, device=D)
        vs = torch.empty_like(ks)
        k = ks.as_strided((B, 1, Skv, d), (0, 0, stride, 1))
        v = vs.as_strided((B, 1, Skv, d), (0, 0, stride, 1))
        k.copy_(inp["k"].to(D))
        v.copy_(inp["v"].to(D))
        want = oracle_dense(inp, use_sink=False)
        for tile in (0, 64):
            out = gqa().prefill(inp["q"].to(D), k, v, scale=inp["scale"], tile_s_kv=tile)
            torch.cuda.synchronize()
            assert_close(out.float().cpu().numpy(), want, f"wide stride Sq={Sq} tile={tile}")
        del ks, vs, k, v
        torch.cuda.empty_cache()


def _paged_oracle(w, causal=False):
    return oracle.paged_attention_fp64(to_f64(w["q"]), w["cu_seqlens_q"].numpy(),
                                       to_f64(w["k_cache"]), to_f64(w["v_cache"]),
                                       w["page_table"].numpy(), w["kv_len"].numpy(),
                                       scale=w["scale"], page_size=64,
                                       sink=None if w["sink"] is None else to_f64(w["sink"]),
                                       causal=causal)


def _paged_run(w, causal=False, tile=0):
    g = to_dev(w)
    out = gqa().paged(g["q"], g["cu_seqlens_q"], g["k_cache"], g["v_cache"], g["page_table"],
                      g["kv_len"], max_q_len=w["max_q_len"], scale=w["scale"], sink=g["sink"],
                      causal=causal, tile_s_kv=tile)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("tile", [0, 1024, 512, 64])
def test_ragged_paged_full(tile):
    note(f"ragged paged workload (B=8, Hq=32, Hkv=1, NaN padding, sink), tile={tile}")
    w = workloads.make_paged()
    assert_close(_paged_run(w, tile=tile), _paged_oracle(w), f"paged tile={tile}")


@pytest.mark.parametrize("tile", [0, 256])
def test_paged_causal_chunked_prefill(tile):
    """Chunked prefill over a cached prefix: q_len <= kv_len, bottom-right causal."""
    note(f"paged causal chunked prefill tile={tile}")
    w = workloads.make_paged(B=5, Hq=16, Hkv=4, d=128, q_lens=[7, 64, 1, 33, 100],
                             kv_lens=[300, 64, 1000, 40, 777], seed=21)
    assert_close(_paged_run(w, causal=True, tile=tile), _paged_oracle(w, causal=True),
                 f"paged causal tile={tile}")


@pytest.mark.parametrize("tile", [0, 1024])
def test_paged_causal_chunked_full(tile):
    """The timed chunked-prefill workload (8 chunks of 512 over prefixes up to
    3584, Hq=32, Hkv=1, sink): sampled rows against the oracle row by row."""
    note(f"paged causal chunked prefill, full size, tile={tile}")
    w = workloads.make_paged_chunked()
    out = _paged_run(w, causal=True, tile=tile)
    r = np.random.default_rng(5 + tile)
    cu = w["cu_seqlens_q"].numpy()
    t = r.integers(0, w["total_q"], 96)
    t[:2 * w["B"]] = np.concatenate([cu[:-1], cu[1:] - 1])  # first and last row of every chunk
    h = r.integers(0, w["Hq"], t.size)
    want = oracle.paged_attention_rows_fp64(w["q"].float().numpy(), cu, w["k_cache"].float().numpy(),
                                            w["v_cache"].float().numpy(), w["page_table"].numpy(),
                                            w["kv_len"].numpy(), t, h, scale=w["scale"],
                                            page_size=64, sink=to_f64(w["sink"]), causal=True)
    assert_close(out[t, h], want, f"paged causal chunked full tile={tile}")


# paged append (the query tokens' K/V handed in beside the cache and written
# into it by the same launch): B, Hq, Hkv, d, q_lens, kv_lens
APPEND_CASES = [
    (6, 32, 8, 128, [1] * 6, [1, 63, 64, 65, 1000, 4096]),   # decode, G = 4
    (4, 32, 1, 128, [1] * 4, [5, 700, 2049, 3000]),          # G = 32: two 16-column blocks
    (4, 16, 4, 64, [1, 2, 5, 8], [8, 64, 200, 1030]),        # short query blocks
    (3, 8, 4, 256, [1, 4, 16], [16, 300, 2000]),             # d = 256, 32 rows: two q-tiles
    (3, 8, 8, 32, [1, 7, 20], [20, 90, 700]),                # d = 32, G = 1
    (4, 16, 4, 128, [1, 2, 3, 4], [8, 64, 200, 1030]),       # token-major pool, up to 16 rows:
                                                             # the stream kernel's whole-row K form
]


@pytest.mark.parametrize("case", range(len(APPEND_CASES)))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [0, 64, 1024])
def test_paged_append(case, causal, tile):
    B, Hq, Hkv, d, q_lens, kv_lens = APPEND_CASES[case]
    note(f"paged append case={APPEND_CASES[case]} causal={causal} tile={tile}")
    w = workloads.make_paged(B=B, Hq=Hq, Hkv=Hkv, d=d, q_lens=q_lens, kv_lens=kv_lens,
                             seed=40 + case)
    kn, vn, kh, vh = workloads.take_new_kv(w)
    g = to_dev(w)
    kc, vc = kh.to(dev()), vh.to(dev())
    out = gqa().paged_append(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"], g["kv_len"],
                             kn.to(dev()), vn.to(dev()), max_q_len=w["max_q_len"],
                             scale=w["scale"], sink=g["sink"], causal=causal, tile_s_kv=tile)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), _paged_oracle(w, causal=causal),
                 f"append case={case} c={causal} t={tile}")
    # the holes are filled with exactly the new rows; nothing else changed
    assert torch.equal(kc.cpu().view(torch.int16), w["k_cache"].view(torch.int16))
    assert torch.equal(vc.cpu().view(torch.int16), w["v_cache"].view(torch.int16))


@pytest.mark.parametrize("layout", ["token-major", "head-major"])
def test_paged_decode_full_size(layout):
    """The timed paged decode workload (16 sequences of 8192 keys, Hq 32,
    Hkv 8, splits of 1024), every output row against the oracle.  The
    head-major pool ([n_pages, Hkv, 64, d] passed as the same logical view by
    strides) takes the stream kernel with K in MFMA operand form, the
    token-major one the stream kernel with K loaded as whole rows."""
    note(f"paged decode, full size, {layout} pool, tile=1024")
    w = workloads.make_paged_decode()
    g = to_dev(w)
    kc, vc = g["k_cache"], g["v_cache"]
    if layout == "head-major":
        kc = kc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vc = vc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        assert kc.stride(1) == w["d"]
    out = gqa().paged(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"], g["kv_len"],
                      max_q_len=1, scale=w["scale"], tile_s_kv=1024)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    t = np.repeat(np.arange(w["B"]), w["Hq"])
    h = np.tile(np.arange(w["Hq"]), w["B"])
    want = oracle.paged_attention_rows_fp64(w["q"].float().numpy(), w["cu_seqlens_q"].numpy(),
                                            w["k_cache"].float().numpy(),
                                            w["v_cache"].float().numpy(), w["page_table"].numpy(),
                                            w["kv_len"].numpy(), t, h, scale=w["scale"],
                                            page_size=64)
    assert_close(out[t, h], want, f"paged decode full size, {layout} pool (all {t.size} rows)")


def test_paged_append_decode_full_size():
    """The timed append workload (16 sequences of 8192 keys, Hq 32, Hkv 8,
    splits of 1024): sampled rows against the oracle over the full cache,
    and the cache rows restored bit for bit."""
    note("paged append decode, full size, tile=1024")
    w = workloads.make_paged_decode()
    kn, vn, kh, vh = workloads.take_new_kv(w)
    g = to_dev(w)
    kc, vc = kh.to(dev()), vh.to(dev())
    out = gqa().paged_append(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"], g["kv_len"],
                             kn.to(dev()), vn.to(dev()), max_q_len=1, scale=w["scale"],
                             tile_s_kv=1024)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    t = np.repeat(np.arange(w["B"]), 4)
    h = np.random.default_rng(3).integers(0, w["Hq"], t.size)
    want = oracle.paged_attention_rows_fp64(w["q"].float().numpy(), w["cu_seqlens_q"].numpy(),
                                            w["k_cache"].float().numpy(),
                                            w["v_cache"].float().numpy(), w["page_table"].numpy(),
                                            w["kv_len"].numpy(), t, h, scale=w["scale"],
                                            page_size=64)
    assert_close(out[t, h], want, "paged append decode full size")
    assert torch.equal(kc.cpu().view(torch.int16), w["k_cache"].view(torch.int16))
    assert torch.equal(vc.cpu().view(torch.int16), w["v_cache"].view(torch.int16))
    # the plain paged decode over the (now complete) cache, as the bench times it
    plain = gqa().paged(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"], g["kv_len"],
                        max_q_len=1, scale=w["scale"], tile_s_kv=1024)
    torch.cuda.synchronize()
    assert_close(plain.float().cpu().numpy()[t, h], want, "paged decode full size")


@pytest.mark.parametrize("tile", [0, 256])
def test_paged_head_major_pages(tile):
    """Pools stored head-major ([page][kv head][row][d]) and passed by strides
    give the same result as the oracle over the logical [page][row][h][d] view."""
    note(f"paged head-major pages tile={tile}")
    w = workloads.make_paged(B=4, Hq=16, Hkv=4, d=128, q_lens=[1, 9, 3, 30],
                             kv_lens=[500, 64, 1300, 90], seed=35)
    g = to_dev(w)
    kc = g["k_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vc = g["v_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert kc.stride(1) == 128 and kc.stride(2) == 64 * 128
    out = gqa().paged(g["q"], g["cu_seqlens_q"], kc, vc, g["page_table"], g["kv_len"],
                      max_q_len=w["max_q_len"], scale=w["scale"], sink=g["sink"], tile_s_kv=tile)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), _paged_oracle(w), f"head-major pages tile={tile}")


@pytest.mark.parametrize("G", [4, 32])
@pytest.mark.parametrize("tile", [0, 1024])
def test_paged_decode_shape(G, tile):
    """One query token per sequence (the stream kernel's paged path)."""
    note(f"paged decode G={G} tile={tile}")
    w = workloads.make_paged(B=6, Hq=32, Hkv=32 // G, d=128, q_lens=[1] * 6,
                             kv_lens=[1, 63, 64, 65, 2000, 4096], seed=22 + G)
    assert_close(_paged_run(w, tile=tile), _paged_oracle(w), f"paged decode G={G} tile={tile}")


def test_paged_d64():
    note("paged d=64 ragged")
    w = workloads.make_paged(B=3, Hq=8, Hkv=2, d=64, q_lens=[5, 40, 17], kv_lens=[100, 3, 640],
                             seed=23)
    assert_close(_paged_run(w, tile=0), _paged_oracle(w), "paged d64")
    assert_close(_paged_run(w, tile=128), _paged_oracle(w), "paged d64 split")


# ---------------------------------------------------------------- small sweeps

SWEEP = [
    # B, Hq, Hkv, Sq, Skv, d
    (2, 8, 2, 37, 301, 128),
    (2, 8, 2, 37, 301, 64),
    (1, 32, 4, 16, 700, 128),
    (3, 4, 4, 5, 129, 128),
    (2, 12, 3, 70, 70, 64),
    # 33..64 and 65..128 query rows per (b, kv head): the 2- and 4-wave
    # shared-tile forms, both head dims
    (2, 8, 2, 12, 333, 128),
    (2, 8, 2, 12, 333, 64),
    (1, 16, 2, 12, 400, 128),
    (1, 16, 2, 12, 400, 64),
]


@pytest.mark.parametrize("shape", SWEEP)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [0, 64, 192])
def test_sweep(shape, causal, tile):
    B, Hq, Hkv, Sq, Skv, d = shape
    note(f"sweep {shape} causal={causal} tile={tile}")
    inp = workloads.make_dense(B, Hq, Hkv, Sq, Skv, d, seed=hash((shape, causal)) % 10000,
                               kv_len="random", sink=True, nan_pad=True)
    got = run_dense(inp, causal=causal, tile=tile)
    want = oracle_dense(inp, causal=causal)
    assert_close(got, want, f"{shape} c={causal} t={tile}")


# head dims 32, 256 and 512 (AstrAI commit log: scalar prefill at d = 32,
# scalar decode at d = 256; nvfp4-megamoe-kernel commit log: head dims up to
# 512), through every kernel form: one 16-column block (rows <= 16), two
# (rows <= 32; two q-tiles at d = 256), the shared-tile prefill kernel at 2
# and 4 waves (d = 32) or 4 waves (d = 256), and at d = 512 the split-head-dim
# kernel (up to 32 rows per (b, kv head)) and the whole-head kernel (more
# rows: 128 per workgroup, 37 x 4 = 148 rows in the last shape)
SWEEP_HD = [
    # B, Hq, Hkv, Sq, Skv
    (2, 8, 2, 1, 500),
    (2, 8, 2, 6, 333),
    (2, 8, 2, 12, 333),
    (1, 16, 2, 12, 400),
    (2, 8, 2, 37, 301),
]


@pytest.mark.parametrize("d", [32, 256, 512])
@pytest.mark.parametrize("shape", SWEEP_HD)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [0, 64, 192])
def test_sweep_head_dims(d, shape, causal, tile):
    B, Hq, Hkv, Sq, Skv = shape
    note(f"head dim sweep d={d} {shape} causal={causal} tile={tile}")
    inp = workloads.make_dense(B, Hq, Hkv, Sq, Skv, d, seed=hash((shape, causal, d)) % 10000,
                               kv_len="random", sink=True, nan_pad=True)
    got = run_dense(inp, causal=causal, tile=tile)
    want = oracle_dense(inp, causal=causal)
    assert_close(got, want, f"d={d} {shape} c={causal} t={tile}")


@pytest.mark.parametrize("d", [32, 256, 512])
@pytest.mark.parametrize("tile", [1024, 64])
def test_decode_head_dims(d, tile):
    note(f"decode d={d} tile={tile}")
    inp = workloads.make_dense(4, 32, 8, 1, 3000, d, seed=77 + d, kv_len="random", sink=True,
                               nan_pad=True)
    got = run_dense(inp, tile=tile, decode=True)
    assert_close(got, oracle_dense(inp), f"decode d={d} tile={tile}")


# in-kernel split merge (one launch): B, Hq, Hkv, Skv, d
FUSED_CASES = [
    (4, 32, 8, 3000, 128),   # G = 4, one 16-column block
    (3, 32, 1, 2500, 128),   # G = 32, two blocks
    (2, 16, 4, 5000, 64),
    (2, 8, 4, 1800, 256),    # d = 256 (one block per q-tile)
    (2, 8, 8, 900, 32),      # G = 1
]


@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
@pytest.mark.parametrize("tile", [1024, 64])
def test_decode_fused(case, tile):
    B, Hq, Hkv, Skv, d = FUSED_CASES[case]
    note(f"fused decode {FUSED_CASES[case]} tile={tile}")
    inp = workloads.make_dense(B, Hq, Hkv, 1, Skv, d, seed=60 + case, kv_len="random", sink=True,
                               nan_pad=True)
    g = to_dev(inp)
    tickets = torch.zeros(B * Hq, dtype=torch.int32, device=dev())
    kw = dict(kv_len=g["kv_len"], scale=inp["scale"], sink=g["sink"], tile_s_kv=tile)
    outs = []
    for _ in range(3):  # the tickets must come back to zero after every call
        outs.append(gqa().decode_splitkv(g["q"], g["k"], g["v"], fused=True, tickets=tickets,
                                         **kw))
        torch.cuda.synchronize()
        assert int(tickets.abs().sum()) == 0
    got = outs[0].float().cpu().numpy()
    assert_close(got, oracle_dense(inp), f"fused decode case={case} tile={tile}")
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    two = gqa().decode_splitkv(g["q"], g["k"], g["v"], **kw).float().cpu().numpy()
    assert np.abs(got - two).max() <= 2 * 2.0 ** -8 * np.abs(two).max() + 1e-6


def test_decode_fused_full_size():
    c = workloads.CASES["decode_splitkv"]
    note(f"fused decode full size {c}")
    inp = workloads.make_case(c)
    g = to_dev(inp)
    tickets = torch.zeros(c.B * c.Hq, dtype=torch.int32, device=dev())
    out = gqa().decode_splitkv(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=inp["scale"],
                               tile_s_kv=c.tile_s_kv, fused=True, tickets=tickets)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    assert np.all(np.isfinite(out)) and int(tickets.abs().sum()) == 0
    assert_close(out, oracle_dense(inp, use_sink=False), "fused decode full size, every element")


@pytest.mark.parametrize("d", [32, 256, 512])
@pytest.mark.parametrize("causal", [False, True])
def test_paged_head_dims(d, causal):
    note(f"paged d={d} causal={causal}")
    w = workloads.make_paged(B=4, Hq=16, Hkv=4, d=d, q_lens=[1, 40, 7, 90],
                             kv_lens=[300, 64, 1000, 777], seed=31 + d)
    want = _paged_oracle(w, causal=causal)
    assert_close(_paged_run(w, causal=causal, tile=0), want, f"paged d={d} c={causal}")
    assert_close(_paged_run(w, causal=causal, tile=128), want, f"paged d={d} c={causal} split")


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 32, 64])
def test_group_sizes(G):
    """The pages' SDPA-checked group sizes (AstrAI commit log, HB packing commit),
    and G = 64, whose single-token rows already take the shared-tile kernel."""
    Hkv = 2 if G <= 8 else 1
    note(f"group size G={G}")
    for Sq in (1, 9, 64):
        inp = workloads.make_dense(2, Hkv * G, Hkv, Sq, 200, 128, seed=50 + G + Sq,
                                   kv_len="random", sink=G % 2 == 0, nan_pad=True)
        want = oracle_dense(inp, causal=Sq > 1)
        for tile in (0, 64):
            got = run_dense(inp, causal=Sq > 1, tile=tile)
            assert_close(got, want, f"G={G} Sq={Sq} tile={tile}")


# The 8-wave prefill form splits a workgroup's keys between two wave groups
# when its grid fits the 256 CUs in one round (at most 256 workgroups of 256
# rows) and either the doubled grid still does or a workgroup may walk 32 or
# more 64-key tiles; else it keeps one group.  These shapes sit on both sides
# of the boundary (B, Hq, Hkv, S, d; workgroups = B Hkv ceil(S G / 256)),
# with ragged last q-tiles, causal and not, one pass and split.
KEY_GROUP_CASES = [
    (1, 8, 2, 8192, 128),   # 256 workgroups: two key groups
    (1, 8, 2, 8300, 128),   # 260: one group, ragged
    (2, 16, 4, 2040, 64),   # 256: two key groups, ragged
    (2, 16, 4, 2304, 64),   # 288: one group
]


@pytest.mark.parametrize("case", range(len(KEY_GROUP_CASES)))
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("tile", [0, 2048])
def test_prefill_key_group_boundary(case, causal, tile):
    B, Hq, Hkv, S, d = KEY_GROUP_CASES[case]
    note(f"key-group boundary B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} causal={causal} tile={tile}")
    inp = workloads.make_dense(B, Hq, Hkv, S, S, d, seed=70 + case, kv_len=[S - 5 * b for b in range(B)])
    out = run_dense(inp, causal=causal, tile=tile, use_sink=False)
    r = np.random.default_rng(case)
    bi, hi, ii = r.integers(0, B, 96), r.integers(0, Hq, 96), r.integers(0, S, 96)
    ii[:4] = [0, S - 1, S - 2, S // 2]
    want = oracle.attention_rows_fp64(inp["q"].float().numpy(), inp["k"].float().numpy(),
                                      inp["v"].float().numpy(), bi, hi, ii, scale=inp["scale"],
                                      kv_len=inp["kv_len"].numpy(), causal=causal)
    assert_close(out[bi, hi, ii], want, f"key groups case={case} causal={causal} tile={tile}")


# Short query groups go to the shared-tile prefill form when the grid (B x
# Hkv x splits) fills the 256 CUs at least twice: every group of up to 64
# rows at d <= 64, and 17-32 rows at d = 128 and 256.  These shapes reach
# that grid (B, Hq, Hkv, Sq, Skv, d, split size); the last one stays below it.
SHORT_GROUP_CASES = [
    (16, 32, 8, 1, 2048, 64, 256),    # d = 64 decode, 1024 workgroups
    (8, 32, 8, 8, 2048, 32, 256),     # d = 32, 32-row groups
    (8, 32, 8, 8, 2048, 128, 256),    # d = 128, 32-row groups
    (8, 64, 8, 3, 1024, 256, 128),    # d = 256, 24-row groups
    (2, 32, 8, 1, 2048, 64, 256),     # d = 64 decode, 128 workgroups: stream kernel
]


@pytest.mark.parametrize("case", range(len(SHORT_GROUP_CASES)))
def test_short_groups_large_grid(case):
    B, Hq, Hkv, Sq, Skv, d, tile = SHORT_GROUP_CASES[case]
    note(f"short groups B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} d={d} tile={tile}")
    inp = workloads.make_dense(B, Hq, Hkv, Sq, Skv, d, seed=90 + case, kv_len="random", sink=True,
                               nan_pad=True)
    for causal in ([False, True] if Sq > 1 else [False]):
        want = oracle_dense(inp, causal=causal)
        assert_close(run_dense(inp, causal=causal, tile=tile), want,
                     f"short groups case={case} causal={causal}")
        if Sq == 1:
            assert_close(run_dense(inp, tile=tile, decode=True), want, f"decode case={case}")


def test_paged_decode_large_grid_d64():
    """Paged decode at d = 64 over 64 sequences (4096 workgroups of splits):
    the shared-tile form, page-table addressing, ragged kv_len, sink."""
    note("paged decode d=64, 64 sequences, splits of 256")
    rng = np.random.default_rng(11)
    kv = [int(x) for x in rng.integers(1, 2048, 64)]
    w = workloads.make_paged(B=64, Hq=32, Hkv=8, d=64, q_lens=[1] * 64, kv_lens=kv, seed=12)
    assert_close(_paged_run(w, tile=256), _paged_oracle(w), "paged decode d=64 large grid")


@pytest.mark.parametrize("Sq,G,causal", [(8, 8, True), (48, 4, True), (24, 8, False), (6, 8, False)])
def test_split_workspace_full_of_nan(Sq, G, causal):
    """The library's split paths leave an empty state's O~ unwritten and their
    merge must never read it: with the workspace filled with NaN bytes first,
    the result still matches the oracle.  Groups of 48-192 rows with per-batch
    lengths (the sparse merge above 64 rows, the dense one below), dense and
    paged."""
    note(f"NaN-filled workspace Sq={Sq} G={G} causal={causal}")
    B, Hkv, Skv, d, tile = 3, 2, 700, 64, 128
    inp = workloads.make_dense(B, Hkv * G, Hkv, Sq, Skv, d, seed=120 + Sq, kv_len="random",
                               sink=True, nan_pad=True)
    g = to_dev(inp)
    m = gqa()
    ws = torch.full((m.workspace_size(B, Hkv * G, Sq, Skv, d, tile),), 255, dtype=torch.uint8,
                    device=dev())
    out = m.prefill(g["q"], g["k"], g["v"], kv_len=g["kv_len"], scale=inp["scale"],
                    sink=g["sink"], causal=causal, tile_s_kv=tile, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), oracle_dense(inp, causal=causal), "dense, NaN workspace")
    q_lens = [max(1, Sq - 3 * b) for b in range(B)]
    w = workloads.make_paged(B=B, Hq=Hkv * G, Hkv=Hkv, d=d, q_lens=q_lens,
                             kv_lens=[max(q, 100 + 250 * b) for b, q in enumerate(q_lens)],
                             seed=130 + Sq)
    gw = to_dev(w)
    wsp = torch.full((m.workspace_size(1, Hkv * G, w["total_q"], w["page_table"].shape[1] * 64, d,
                                       tile),), 255, dtype=torch.uint8, device=dev())
    outp = m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"], gw["v_cache"], gw["page_table"],
                   gw["kv_len"], max_q_len=w["max_q_len"], scale=w["scale"], sink=gw["sink"],
                   causal=causal, tile_s_kv=tile, workspace=wsp)
    torch.cuda.synchronize()
    assert_close(outp.float().cpu().numpy(), _paged_oracle(w, causal=causal), "paged, NaN workspace")


@pytest.mark.parametrize("Skv", [1, 63, 1024, 3000])
def test_decode_sweep(Skv):
    note(f"decode Skv={Skv}")
    inp = workloads.make_dense(4, 32, 8, 1, Skv, 128, seed=Skv, kv_len="random", sink=True,
                               nan_pad=True)
    got = run_dense(inp, tile=1024, decode=True)
    assert_close(got, oracle_dense(inp), f"decode Skv={Skv}")


# ---------------------------------------------------------------- invariants and edges

# every head dim, at query lengths that reach each kernel form (4 rows per
# kv head: stream kernel / split-head-dim d = 512 kernel; 64 rows: shared-tile
# prefill kernel / whole-head d = 512 kernel)
@pytest.mark.parametrize("d", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("Sq", [1, 16])
def test_kvlen_one_is_exact_v0(d, Sq):
    """One valid key among 128 padded (NaN) rows: O is that V row, bit for bit."""
    note(f"kv_len = 1, Skv = 128 NaN padded, d={d} Sq={Sq}")
    inp = workloads.make_dense(2, 8, 2, Sq, 128, d, seed=3, kv_len=[1, 1], nan_pad=True)
    for tile in (0, 64):
        out = run_dense(inp, tile=tile, use_sink=False)
        v0 = inp["v"][:, :, :1].float().numpy()
        want = np.repeat(v0, 4, axis=1)
        np.testing.assert_array_equal(out, np.broadcast_to(want, out.shape))


@pytest.mark.parametrize("d,Sq", [(64, 6), (128, 6), (128, 40), (256, 40), (512, 6), (512, 40)])
def test_empty_rows_are_zero_and_sink_neg_inf_is_no_sink(d, Sq):
    note(f"kv_len = 0 rows, causal rows with no key, sink = -inf, d={d} Sq={Sq}")
    inp = workloads.make_dense(2, 4, 1, Sq, 64, d, seed=4, kv_len=[0, 3], nan_pad=True)
    out = run_dense(inp, use_sink=False)
    assert np.all(out[0] == 0)
    outc = run_dense(inp, causal=True, use_sink=False)
    assert np.all(outc[1, :, :3] == 0)          # rows 0..2 see no key (bottom-right)
    assert_close(outc, oracle_dense(inp, causal=True, use_sink=False), "causal empty rows")
    inp2 = dict(inp, sink=torch.full((4,), -math.inf), kv_len=torch.tensor([64, 5], dtype=torch.int32))
    inp2["k"] = inp["k"].nan_to_num()
    inp2["v"] = inp["v"].nan_to_num()
    a = run_dense(inp2, use_sink=True)
    b = run_dense(inp2, use_sink=False)
    np.testing.assert_array_equal(a, b)


def test_decode_equals_last_prefill_row():
    note("decode vs last row of causal prefill")
    inp = workloads.make_dense(2, 16, 4, 40, 300, 128, seed=5, kv_len=[300, 211], sink=True,
                               nan_pad=True)
    pre = run_dense(inp, causal=True)
    dec_inp = dict(inp, q=inp["q"][:, :, -1:].contiguous())
    dec = run_dense(dec_inp, tile=128, decode=True)
    assert np.abs(pre[:, :, -1] - dec[:, :, 0]).max() <= 4e-3


def test_strided_views():
    """(B, S, H, d) storage seen as [B, H, S, d]: distinct s and h strides."""
    note("strided q/k/v/o views")
    B, Hq, Hkv, S, d = 2, 8, 2, 33, 128
    base = workloads.make_dense(B, Hq, Hkv, S, S, d, seed=6, sink=True)
    D = dev()
    q = base["q"].transpose(1, 2).contiguous().to(D).transpose(1, 2)
    k = base["k"].transpose(1, 2).contiguous().to(D).transpose(1, 2)
    v = base["v"].transpose(1, 2).contiguous().to(D).transpose(1, 2)
    out = torch.empty(B, S, Hq, d, dtype=torch.bfloat16, device=D).transpose(1, 2)
    gqa().prefill(q, k, v, scale=base["scale"], sink=base["sink"].to(D), causal=True, out=out)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), oracle_dense(base, causal=True), "strided")


def test_partial_states_match_oracle():
    note("split-KV partial states vs oracle partials")
    inp = workloads.make_dense(2, 8, 2, 3, 300, 128, seed=8, kv_len=[300, 100])
    g = to_dev(inp)
    ml, ot, ws = gqa().splitkv_partial(g["q"], g["k"], g["v"], tile_s_kv=128, kv_len=g["kv_len"],
                                       scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    m, l, o = oracle.splitkv_partials_fp64(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                           scale=inp["scale"], tile=128,
                                           kv_len=inp["kv_len"].numpy(), causal=True)
    ns = m.shape[-1]
    ml = ml.cpu().numpy().reshape(2, 8, 3, ns, 2)
    ot = ot.cpu().numpy().reshape(2, 8, 3, ns, 128)
    live = m > -np.inf
    assert np.array_equal(ml[..., 0] > -np.inf, live)
    assert np.all(ml[..., 1][~live] == 0) and np.all(ot[~live] == 0)
    # compare normalised partials (each one's softmax over its own split)
    np.testing.assert_allclose(ml[..., 0][live], m[live], rtol=1e-5, atol=1e-5)
    rel = ot[live] / ml[..., 1][live][:, None] - o[live] / l[live][:, None]
    assert np.abs(rel).max() <= MAX_ABS
    out = gqa().splitkv_merge(ws, B=2, Hq=8, Sq=3, d=128, n_split=ns)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().numpy(), oracle_dense(inp, causal=True, use_sink=False), "merge")


def test_repeat_runs_bit_identical():
    note("repeated launches are bit-identical")
    inp = workloads.make_dense(2, 32, 8, 64, 1000, 128, seed=9, kv_len="random", sink=True,
                               nan_pad=True)
    g = to_dev(inp)
    ref = gqa().prefill(g["q"], g["k"], g["v"], kv_len=g["kv_len"], sink=g["sink"], causal=True)
    for _ in range(20):
        again = gqa().prefill(g["q"], g["k"], g["v"], kv_len=g["kv_len"], sink=g["sink"],
                              causal=True)
        assert torch.equal(ref.view(torch.int16), again.view(torch.int16))


def test_empty_batch_is_noop():
    note("B = 0")
    D = dev()
    q = torch.empty(0, 4, 3, 64, dtype=torch.bfloat16, device=D)
    k = torch.empty(0, 1, 5, 64, dtype=torch.bfloat16, device=D)
    out = gqa().prefill(q, k, k)
    assert out.shape == q.shape


# ---------------------------------------------------------------- graph capture

def _graph_cases():
    """(name, fn(out) -> None, out) for every entry point, inputs on the GPU."""
    m = gqa()
    cases = []
    inp = workloads.make_dense(2, 32, 8, 1, 3000, 128, seed=91, kv_len="random", sink=True)
    g = to_dev(inp)
    kw = dict(kv_len=g["kv_len"], scale=inp["scale"], sink=g["sink"])
    ws = torch.empty(m.workspace_size(2, 32, 1, 3000, 128, 1024), dtype=torch.uint8, device=dev())
    tk = torch.zeros(64, dtype=torch.int32, device=dev())
    cases.append(("decode split", lambda o: m.decode_splitkv(g["q"], g["k"], g["v"], tile_s_kv=1024,
                                                            out=o, workspace=ws, **kw), g["q"]))
    cases.append(("decode fused", lambda o: m.decode_splitkv(g["q"], g["k"], g["v"], tile_s_kv=1024,
                                                            out=o, workspace=ws, fused=True,
                                                            tickets=tk, **kw), g["q"]))
    inp2 = workloads.make_dense(1, 16, 4, 100, 700, 64, seed=92, kv_len="random", sink=True)
    g2 = to_dev(inp2)
    kw2 = dict(kv_len=g2["kv_len"], scale=inp2["scale"], sink=g2["sink"], causal=True)
    ws2 = torch.empty(m.workspace_size(1, 16, 100, 700, 64, 256), dtype=torch.uint8, device=dev())
    cases.append(("prefill one pass", lambda o: m.prefill(g2["q"], g2["k"], g2["v"], out=o, **kw2),
                  g2["q"]))
    cases.append(("prefill split", lambda o: m.prefill(g2["q"], g2["k"], g2["v"], tile_s_kv=256,
                                                      out=o, workspace=ws2, **kw2), g2["q"]))
    w = workloads.make_paged(B=3, Hq=16, Hkv=4, d=128, q_lens=[1, 5, 2], kv_lens=[300, 90, 1000],
                             seed=93)
    kn, vn, kh, vh = workloads.take_new_kv(w)
    gw = to_dev(w)
    kc, vc, kn, vn = kh.to(dev()), vh.to(dev()), kn.to(dev()), vn.to(dev())
    pk = dict(max_q_len=w["max_q_len"], scale=w["scale"], sink=gw["sink"])
    cases.append(("paged", lambda o: m.paged(gw["q"], gw["cu_seqlens_q"], gw["k_cache"],
                                             gw["v_cache"], gw["page_table"], gw["kv_len"], out=o,
                                             **pk), gw["q"]))
    cases.append(("paged append", lambda o: m.paged_append(gw["q"], gw["cu_seqlens_q"], kc, vc,
                                                           gw["page_table"], gw["kv_len"], kn, vn,
                                                           out=o, **pk), gw["q"]))
    return cases


def test_graph_replay_matches_eager():
    """Each entry point captured in a HIP graph replays bit-identically to its
    eager call, three times, with eager launches and a synchronisation between
    the replays (and the output cleared before each)."""
    note("graph capture of every entry point")
    for name, fn, like in _graph_cases():
        eager = torch.empty_like(like)
        fn(eager)
        torch.cuda.synchronize()
        out = torch.empty_like(like)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(out)  # first use on this stream outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            fn(out)
        for r in range(3):
            out.zero_()
            graph.replay()
            other = torch.empty_like(like)
            fn(other)  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"{name} replay {r}"
            assert torch.equal(other.view(torch.int16), eager.view(torch.int16)), name


# ---------------------------------------------------------------- long contexts

def test_long_context_128k():
    """131072 keys: split-KV decode (128 splits, runs of splits), the in-kernel
    merge, a one-pass 16-query prefill over the same keys, and a paged decode
    over ~1600 pages; sampled rows against the oracle."""
    note("long context: 131072 keys")
    inp = workloads.make_dense(2, 16, 2, 1, 131072, 128, seed=77, kv_len=[131072, 100003],
                               sink=True, nan_pad=True)
    g = to_dev(inp)
    kw = dict(kv_len=g["kv_len"], scale=inp["scale"], sink=g["sink"])
    m = gqa()
    rows = (np.repeat([0, 1], 8), np.tile(np.arange(0, 16, 2), 2), np.zeros(16, dtype=int))
    k32, v32 = inp["k"].float().numpy(), inp["v"].float().numpy()
    want = oracle.attention_rows_fp64(inp["q"].float().numpy(), k32, v32, *rows, scale=inp["scale"],
                                      kv_len=inp["kv_len"].numpy(), sink=to_f64(inp["sink"]))
    for label, out in (("split", m.decode_splitkv(g["q"], g["k"], g["v"], tile_s_kv=1024, **kw)),
                       ("fused", m.decode_splitkv(g["q"], g["k"], g["v"], tile_s_kv=1024,
                                                  fused=True, **kw))):
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy()[rows], want, f"128k decode {label}")
    # 16 queries at the end of the same keys (bottom-right causal), one pass
    q16 = workloads.make_dense(2, 16, 2, 16, 8, 128, seed=78)["q"]
    out = m.prefill(q16.to(dev()), g["k"], g["v"], causal=True, **kw)
    torch.cuda.synchronize()
    r16 = (np.repeat([0, 1], 8), np.tile(np.arange(0, 16, 2), 2), np.tile([0, 15, 7, 3], 4))
    want16 = oracle.attention_rows_fp64(q16.float().numpy(), k32, v32, *r16, scale=inp["scale"],
                                        kv_len=inp["kv_len"].numpy(), sink=to_f64(inp["sink"]),
                                        causal=True)
    assert_close(out.float().cpu().numpy()[r16], want16, "128k prefill")
    # paged decode over the same lengths
    w = workloads.make_paged(B=2, Hq=16, Hkv=2, d=128, q_lens=[1, 1], kv_lens=[100000, 3000],
                             seed=79)
    outp = _paged_run(w, tile=1024)
    t = np.repeat([0, 1], 8)
    h = np.tile(np.arange(0, 16, 2), 2)
    wp = oracle.paged_attention_rows_fp64(w["q"].float().numpy(), w["cu_seqlens_q"].numpy(),
                                          w["k_cache"].float().numpy(),
                                          w["v_cache"].float().numpy(), w["page_table"].numpy(),
                                          w["kv_len"].numpy(), t, h, scale=w["scale"],
                                          page_size=64, sink=to_f64(w["sink"]))
    assert_close(outp[t, h], wp, "100k paged decode")

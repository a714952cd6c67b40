"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties the oracle to a closed form, an invariant the pages state,
brute force on tiny inputs, the numbers the pages print (tests/golden), or
torch's SDPA in float64 as an independent library routine.  The set is
chosen so that a plausible slip in the oracle (a dropped sink term, the sink
multiplied by scale, a wrong head map, top-left instead of bottom-right
causal alignment, a wrong sign, a transposed operand, a bad merge weight)
fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_claims.json")
RNG = np.random.default_rng(12345)


def rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, scale, kv_len, sink, causal):
    """Pure-Python loops, no numpy arithmetic: the definition term by term."""
    B, Hq, Sq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        n = int(kv_len[b])
        for h in range(Hq):
            g = h // G
            for i in range(Sq):
                hi = n if not causal else min(max(n - Sq + i + 1, 0), n)
                s = []
                for j in range(hi):
                    acc = 0.0
                    for t in range(d):
                        acc += float(q[b, h, i, t]) * float(k[b, g, j, t])
                    s.append(scale * acc)
                sk = -math.inf if sink is None else float(sink[h])
                m = max(s + [sk])
                if m == -math.inf:
                    continue
                w = [math.exp(x - m) for x in s]
                z = sum(w) + (math.exp(sk - m) if sk != -math.inf else 0.0)
                for t in range(d):
                    acc = 0.0
                    for j in range(hi):
                        acc += w[j] * float(v[b, g, j, t])
                    out[b, h, i, t] = acc / z
    return out


@pytest.mark.parametrize("trial", range(12))
def test_brute_force_tiny(trial):
    r = np.random.default_rng(100 + trial)
    B = int(r.integers(1, 3))
    Hkv = int(r.integers(1, 3))
    G = int(r.choice([1, 2, 3, 4]))
    Hq = Hkv * G
    Sq = int(r.integers(1, 5))
    Skv = int(r.integers(1, 10))
    d = int(r.integers(1, 9))
    q, k, v = (r.standard_normal(s) for s in [(B, Hq, Sq, d), (B, Hkv, Skv, d), (B, Hkv, Skv, d)])
    kv_len = r.integers(0, Skv + 1, size=B)
    sink = r.standard_normal(Hq) if trial % 2 else None
    causal = bool(trial % 3 == 0)
    scale = float(r.uniform(0.1, 1.0))
    want = brute_force(q, k, v, scale, kv_len, sink, causal)
    got = oracle.attention_fp64(q, k, v, scale=scale, kv_len=kv_len, sink=sink, causal=causal)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- SDPA (library routine)

def sdpa_fp64(q, k, v, scale, mask=None, is_causal=False):
    f = torch.nn.functional.scaled_dot_product_attention
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))  # noqa: E731
    return f(t(q), t(k), t(v), attn_mask=None if mask is None else t(mask),
             is_causal=is_causal, scale=scale, enable_gqa=True).numpy()


@pytest.mark.parametrize("G", json.load(open(GOLDEN))["group_sizes"]["G"])
def test_sdpa_plain_and_square_causal(G):
    Hkv = 2 if G < 32 else 1
    Hq = Hkv * G
    B, S, d = 2, 24, 16
    q, k, v = rand(B, Hq, S, d), rand(B, Hkv, S, d), rand(B, Hkv, S, d)
    for causal in (False, True):
        want = sdpa_fp64(q, k, v, 0.3, is_causal=causal)
        got = oracle.attention_fp64(q, k, v, scale=0.3, causal=causal)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_sdpa_kvlen_and_bottom_right_causal(G):
    """kv_len and bottom-right alignment through an explicit boolean mask."""
    Hkv, B, Sq, Skv, d = 2, 3, 5, 19, 8
    Hq = Hkv * G
    q, k, v = rand(B, Hq, Sq, d), rand(B, Hkv, Skv, d), rand(B, Hkv, Skv, d)
    kv_len = np.array([19, 11, 6])
    for causal in (False, True):
        mask = np.zeros((B, 1, Sq, Skv), dtype=bool)
        for b in range(B):
            for i in range(Sq):
                hi = kv_len[b] if not causal else kv_len[b] - Sq + i + 1
                mask[b, 0, i, :hi] = True
        want = sdpa_fp64(q, k, v, 0.25, mask=mask)
        got = oracle.attention_fp64(q, k, v, scale=0.25, kv_len=kv_len, causal=causal)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_top_left_alignment_differs():
    """Guards the alignment pin: SDPA's is_causal (top-left) differs at Sq != Skv."""
    q, k, v = rand(1, 2, 4, 8), rand(1, 2, 12, 8), rand(1, 2, 12, 8)
    top_left = sdpa_fp64(q, k, v, 0.3, is_causal=True)
    ours = oracle.attention_fp64(q, k, v, scale=0.3, causal=True)
    assert np.abs(top_left - ours).max() > 1e-3


@pytest.mark.parametrize("G", [1, 4, 32])
def test_sdpa_sink_as_extra_zero_value_column(G):
    """The sink is an extra scaled-domain logit with no value row.

    SDPA sees one more key with a zero K row (score 0) and a zero V row, and
    an additive float mask that puts sink[h] on that column -- so its logit
    is sink[h] exactly, not scale*sink[h]  (nvfp4-megamoe-kernel commit log,
    the sink-bias commit).
    """
    Hkv = 1 if G == 32 else 2
    Hq = Hkv * G
    B, Sq, Skv, d = 2, 6, 13, 8
    q, k, v = rand(B, Hq, Sq, d), rand(B, Hkv, Skv, d), rand(B, Hkv, Skv, d)
    sink = 2.0 * rand(Hq)
    kv_len = np.array([13, 7])
    k2 = np.concatenate([k, np.zeros((B, Hkv, 1, d))], axis=2)
    v2 = np.concatenate([v, np.zeros((B, Hkv, 1, d))], axis=2)
    mask = np.full((B, Hq, Sq, Skv + 1), -np.inf)
    for b in range(B):
        mask[b, :, :, :kv_len[b]] = 0.0
    mask[:, :, :, Skv] = sink[None, :, None]
    want = sdpa_fp64(q, k2, v2, 0.4, mask=mask)
    got = oracle.attention_fp64(q, k, v, scale=0.4, kv_len=kv_len, sink=sink)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # the wrong reading (sink multiplied by scale) is far off
    wrong = oracle.attention_fp64(q, k, v, scale=0.4, kv_len=kv_len, sink=0.4 * sink)
    assert np.abs(wrong - want).max() > 1e-3


# ---------------------------------------------------------------- invariants

def test_weights_sum_to_one():
    B, Hkv, G, Sq, Skv, d = 2, 2, 4, 7, 21, 16
    q, k = rand(B, Hkv * G, Sq, d), rand(B, Hkv, Skv, d)
    sink = rand(Hkv * G)
    for causal in (False, True):
        for snk in (None, sink):
            w, ws = oracle.softmax_weights_fp64(q, k, scale=0.3, kv_len=[21, 9], sink=snk,
                                                causal=causal)
            tot = w.sum(-1) + ws
            np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-15)
            assert np.all(w[1, :, :, 9:] == 0.0)


def _scores_with_sink(q, k, scale, kv_len, sink, causal):
    """Scores of every row with the sink appended as one more column, invisible
    keys at -inf, written with einsum (not the oracle's matmul).  Returns
    [B, Hq, Sq, Skv + 1] and the number of visible keys per row."""
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kx = np.stack([k[:, h // G] for h in range(Hq)], axis=1)      # [B, Hq, Skv, d]
    s = scale * np.einsum("bhid,bhjd->bhij", q, kx)
    hi = np.empty((B, Sq), dtype=np.int64)
    for b in range(B):
        for i in range(Sq):
            hi[b, i] = kv_len[b] if not causal else min(max(kv_len[b] - Sq + i + 1, 0), kv_len[b])
    vis = np.arange(Skv)[None, None, None, :] < hi[:, None, :, None]
    s = np.where(vis, s, -np.inf)
    sk = np.broadcast_to((np.full(Hq, -np.inf) if sink is None else sink)[None, :, None, None],
                         (B, Hq, Sq, 1))
    return np.concatenate([s, sk], axis=-1), hi


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_sink", [False, True])
def test_definition_weights_are_a_softmax_summing_to_one(causal, with_sink):
    """The weights inside attention_fp64 itself (the function every GPU
    comparison uses): with V the identity (one key per d column), O[.., j] is
    the weight of key j.  They must equal scipy's softmax over the row's
    scores with the sink appended as one more column (the sink column has no
    value row, so its weight is 1 - sum_j O[.., j]), be zero past the row's
    visible keys, and -- with V all ones -- every row must sum to 1 minus the
    sink weight (to 1 exactly up to rounding without a sink).  Groups of 4
    over 3 kv heads, so a wrong head map changes the weights."""
    from scipy.special import softmax
    B, Hkv, G, Sq, d = 2, 3, 4, 6, 24
    Skv = d                                    # V = identity: key j carries e_j
    Hq = Hkv * G
    q, k = rand(B, Hq, Sq, d), rand(B, Hkv, Skv, d)
    sink = rand(Hq) if with_sink else None
    kv_len = [24, 10]
    eye = np.broadcast_to(np.eye(Skv), (B, Hkv, Skv, d)).copy()
    w = oracle.attention_fp64(q, k, eye, scale=0.35, kv_len=kv_len, sink=sink, causal=causal)
    s_ext, hi = _scores_with_sink(q, k, 0.35, kv_len, sink, causal)
    live = np.isfinite(s_ext).any(-1)
    want = np.zeros_like(s_ext)
    want[live] = softmax(s_ext[live], axis=-1)
    np.testing.assert_allclose(w, want[..., :Skv], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(w.sum(-1)[live] + want[..., Skv][live], 1.0, rtol=0, atol=1e-14)
    for b in range(B):
        for i in range(Sq):
            assert np.all(w[b, :, i, hi[b, i]:] == 0.0)
    ones = oracle.attention_fp64(q, k, np.ones((B, Hkv, Skv, d)), scale=0.35, kv_len=kv_len,
                                 sink=sink, causal=causal)
    tot = np.where(live[..., None], 1.0 - want[..., Skv][..., None], 0.0)
    np.testing.assert_allclose(ones, np.broadcast_to(tot, ones.shape), rtol=0, atol=1e-14)
    if not with_sink:
        assert np.all(np.abs(ones[live] - 1.0) <= 1e-15)


def test_softmax_weights_head_map_matches_the_definition():
    """softmax_weights_fp64 (used to size the rounding bound of the GPU tests)
    gives the same weights as attention_fp64 with V = identity at G = 4 over 3
    kv heads, and a head map of h % Hkv instead of h // G would not."""
    B, Hkv, G, Sq, d = 2, 3, 4, 5, 16
    Skv, Hq = d, Hkv * G
    q, k = rand(B, Hq, Sq, d), rand(B, Hkv, Skv, d)
    sink = rand(Hq)
    eye = np.broadcast_to(np.eye(Skv), (B, Hkv, Skv, d)).copy()
    for causal in (False, True):
        w_def = oracle.attention_fp64(q, k, eye, scale=0.3, kv_len=[16, 7], sink=sink,
                                      causal=causal)
        w, ws = oracle.softmax_weights_fp64(q, k, scale=0.3, kv_len=[16, 7], sink=sink,
                                            causal=causal)
        np.testing.assert_allclose(w, w_def, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(ws, 1.0 - w_def.sum(-1), rtol=0, atol=1e-14)
        # the slip this guards against: query head h reading kv head h % Hkv
        k_slip = np.stack([k[:, (h % Hkv)] for h in range(Hq)], axis=1)
        w_slip = oracle.attention_fp64(q, k_slip, np.broadcast_to(np.eye(Skv), (B, Hq, Skv, d)).copy(),
                                       scale=0.3, kv_len=[16, 7], sink=sink, causal=causal)
        assert np.abs(w_slip - w).max() > 1e-2


def test_gqa_equals_repeated_mha():
    B, Hkv, G, Sq, Skv, d = 2, 3, 4, 5, 17, 8
    q, k, v = rand(B, Hkv * G, Sq, d), rand(B, Hkv, Skv, d), rand(B, Hkv, Skv, d)
    sink = rand(Hkv * G)
    a = oracle.attention_fp64(q, k, v, scale=0.3, sink=sink, kv_len=[17, 4], causal=True)
    b = oracle.attention_fp64(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), scale=0.3,
                              sink=sink, kv_len=[17, 4], causal=True)
    np.testing.assert_array_equal(a, b)


def test_g1_equals_per_head_mha():
    B, H, Sq, Skv, d = 2, 3, 4, 9, 8
    q, k, v = rand(B, H, Sq, d), rand(B, H, Skv, d), rand(B, H, Skv, d)
    full = oracle.attention_fp64(q, k, v, scale=0.5)
    for h in range(H):
        one = oracle.attention_fp64(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], scale=0.5)
        np.testing.assert_array_equal(full[:, h:h + 1], one)


def test_padding_excluded_and_golden_dilution():
    g = json.load(open(GOLDEN))["padded_dilution"]
    N, n = g["N_padded"], g["kv_len"]
    d = 16
    q, k, v = rand(1, 4, 3, d), rand(1, 1, N, d), rand(1, 1, N, d)
    k[:, :, n:] = np.nan
    v[:, :, n:] = np.nan
    o = oracle.attention_fp64(q, k, v, scale=0.25, kv_len=[n])
    # one valid key: weight exactly 1, so O is that V row exactly
    np.testing.assert_array_equal(o, np.broadcast_to(v[:, :, :1], o.shape))
    w, _ = oracle.softmax_weights_fp64(q, k, scale=0.25, kv_len=[n])
    assert np.all(w[..., 0] == g["weight_correct"]) and np.all(w[..., 1:] == 0.0)
    # counting the padding (kv_len = N) on equal scores gives the page's 1/N
    w_bad, _ = oracle.softmax_weights_fp64(np.zeros((1, 4, 3, d)), np.nan_to_num(k), scale=0.25,
                                           kv_len=[N])
    np.testing.assert_allclose(w_bad[..., :N], g["weight_if_padding_counted"], rtol=1e-15)


def test_nan_padding_equals_truncation():
    B, Hkv, G, Sq, Skv, d = 3, 2, 2, 4, 40, 8
    q, k, v = rand(B, Hkv * G, Sq, d), rand(B, Hkv, Skv, d), rand(B, Hkv, Skv, d)
    kv_len = np.array([40, 17, 1])
    kp, vp = k.copy(), v.copy()
    for b in range(B):
        kp[b, :, kv_len[b]:] = np.nan
        vp[b, :, kv_len[b]:] = np.nan
    for causal in (False, True):
        a = oracle.attention_fp64(q, kp, vp, scale=0.3, kv_len=kv_len, causal=causal)
        for b in range(B):
            n = kv_len[b]
            t = oracle.attention_fp64(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                                      scale=0.3, causal=causal)
            np.testing.assert_array_equal(a[b:b + 1], t)


def test_sink_neg_inf_equals_no_sink():
    q, k, v = rand(2, 4, 3, 8), rand(2, 2, 10, 8), rand(2, 2, 10, 8)
    a = oracle.attention_fp64(q, k, v, scale=0.3, kv_len=[10, 3])
    b = oracle.attention_fp64(q, k, v, scale=0.3, kv_len=[10, 3], sink=np.full(4, -np.inf))
    np.testing.assert_array_equal(a, b)


def test_normalise_once_golden():
    g = json.load(open(GOLDEN))["normalise_once"]
    N, d = g["N"], 8
    q, k, v = np.zeros((1, 2, 1, d)), rand(1, 1, N, d), rand(1, 1, N, d)
    o = oracle.attention_fp64(q, k, v, scale=0.3)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0].mean(0), rtol=1e-13, atol=1e-15)
    m, l, _ = oracle.splitkv_partials_fp64(q, k, v, scale=0.3, tile=N)
    assert l[0, 0, 0, 0] == g["unnormalised_row_sum_uniform"] and m[0, 0, 0, 0] == 0.0
    # dividing a second time would be off by exactly the page's factor
    np.testing.assert_allclose(o[0, 0, 0] / l[0, 0, 0, 0] * g["bug_factor"], o[0, 0, 0])


# ---------------------------------------------------------------- closed forms

def test_zero_q_with_sink_closed_form():
    n, d = 9, 8
    q, k, v = np.zeros((1, 2, 1, d)), rand(1, 1, n, d), rand(1, 1, n, d)
    sigma = np.array([0.7, -1.3])
    o = oracle.attention_fp64(q, k, v, scale=0.5, sink=sigma)
    for h in range(2):
        np.testing.assert_allclose(o[0, h, 0], v[0, 0].sum(0) / (n + math.exp(sigma[h])),
                                   rtol=1e-13)


def test_one_key_with_sink_closed_form():
    d = 8
    q, k, v = rand(1, 1, 1, d), rand(1, 1, 1, d), rand(1, 1, 1, d)
    s0 = 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])
    sigma = 0.9
    o = oracle.attention_fp64(q, k, v, scale=0.5, sink=[sigma])
    want = v[0, 0, 0] * math.exp(s0) / (math.exp(s0) + math.exp(sigma))
    np.testing.assert_allclose(o[0, 0, 0], want, rtol=1e-13)


def test_identical_keys_give_mean_of_v():
    q = rand(1, 3, 4, 8)
    k = np.repeat(rand(1, 1, 1, 8), 11, axis=2)
    v = rand(1, 1, 11, 8)
    o = oracle.attention_fp64(q, k, v, scale=0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v[0, 0].mean(0), o.shape), rtol=1e-12,
                               atol=1e-14)


def test_logistic_mix_d1_n2():
    q = np.array([[[[1.5]]]])
    k = np.array([[[[2.0], [-1.0]]]])
    v = np.array([[[[3.0], [-5.0]]]])
    o = oracle.attention_fp64(q, k, v, scale=0.5)
    s0, s1 = 0.5 * 1.5 * 2.0, 0.5 * 1.5 * -1.0
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(o[0, 0, 0, 0], p0 * 3.0 + (1 - p0) * -5.0, rtol=1e-14)


def test_dominant_logit_selects_row():
    d, n = 4, 7
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, d))
    k[0, 0, 3, 0] = 40.0
    v = rand(1, 1, n, d)
    o = oracle.attention_fp64(q, k, v, scale=1.0)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 3], rtol=0, atol=1e-15 * 50)


def test_causal_row0_and_decode_is_last_prefill_row():
    B, Hkv, G, S, d = 2, 2, 4, 33, 16
    q, k, v = rand(B, Hkv * G, S, d), rand(B, Hkv, S, d), rand(B, Hkv, S, d)
    o = oracle.attention_fp64(q, k, v, scale=0.25, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], np.repeat(v[:, :, 0], G, axis=1))
    dec = oracle.attention_fp64(q[:, :, -1:], k, v, scale=0.25, causal=True)
    np.testing.assert_allclose(dec[:, :, 0], o[:, :, -1], rtol=1e-13, atol=1e-15)
    dec_nc = oracle.attention_fp64(q[:, :, -1:], k, v, scale=0.25, causal=False)
    np.testing.assert_array_equal(dec, dec_nc)


def test_no_visible_key_no_sink_is_zero():
    q, k, v = rand(2, 2, 3, 4), rand(2, 1, 5, 4), rand(2, 1, 5, 4)
    o = oracle.attention_fp64(q, k, v, scale=0.5, kv_len=[0, 5])
    assert np.all(o[0] == 0.0) and not np.any(np.isnan(o))
    # causal with Sq > kv_len: leading rows see nothing
    o2 = oracle.attention_fp64(rand(1, 1, 6, 4), k[:1], v[:1], scale=0.5, kv_len=[2], causal=True)
    assert np.all(o2[0, 0, :4] == 0.0) and np.all(o2[0, 0, 4:] != 0.0)


# ---------------------------------------------------------------- split-KV merge

@pytest.mark.parametrize("tile", [1, 3, 8, 64, 1024])
def test_split_merge_equals_single_pass(tile):
    B, Hkv, G, Sq, Skv, d = 2, 2, 2, 3, 50, 8
    q, k, v = rand(B, Hkv * G, Sq, d), rand(B, Hkv, Skv, d), rand(B, Hkv, Skv, d)
    sink = rand(Hkv * G)
    kv_len = np.array([50, 13])
    for causal in (False, True):
        for snk in (None, sink):
            one = oracle.attention_fp64(q, k, v, scale=0.3, kv_len=kv_len, sink=snk, causal=causal)
            m, l, o = oracle.splitkv_partials_fp64(q, k, v, scale=0.3, tile=tile, kv_len=kv_len,
                                                   causal=causal)
            assert m.shape[-1] == -(-Skv // tile)
            got = oracle.merge_partials_fp64(m, l, o, sink=snk)
            np.testing.assert_allclose(got, one, rtol=1e-12, atol=1e-14)


def test_merge_any_order_or_tree():
    """Associativity of the (m, l, O~) merge (kernbench2 2-D mesh mlo commit)."""
    B, H, Sq, Skv, d = 1, 2, 2, 37, 4
    q, k, v = rand(B, H, Sq, d), rand(B, H, Skv, d), rand(B, H, Skv, d)
    m, l, o = oracle.splitkv_partials_fp64(q, k, v, scale=0.5, tile=4)
    ns = m.shape[-1]
    ref = oracle.merge_partials_fp64(m, l, o)
    parts = [(m[..., s], l[..., s], o[..., s, :]) for s in range(ns)]
    fin = lambda st: st[2] / st[1][..., None]  # noqa: E731
    for trial in range(5):
        order = np.random.default_rng(trial).permutation(ns)
        acc = parts[order[0]]
        for s in order[1:]:
            acc = oracle.merge_pair_fp64(acc, parts[s])
        np.testing.assert_allclose(fin(acc), ref, rtol=1e-12)
    # balanced tree
    level = parts
    while len(level) > 1:
        level = [oracle.merge_pair_fp64(level[i], level[i + 1]) if i + 1 < len(level) else level[i]
                 for i in range(0, len(level), 2)]
    np.testing.assert_allclose(fin(level[0]), ref, rtol=1e-12)


def test_empty_split_and_single_tile():
    q, k, v = rand(1, 1, 1, 4), rand(1, 1, 10, 4), rand(1, 1, 10, 4)
    m, l, o = oracle.splitkv_partials_fp64(q, k, v, scale=0.5, tile=4, kv_len=[5])
    assert m[0, 0, 0, 2] == -np.inf and l[0, 0, 0, 2] == 0 and np.all(o[0, 0, 0, 2] == 0)
    ident = (np.array(-np.inf), np.array(0.0), np.zeros(4))
    st = (m[0, 0, 0, 0], l[0, 0, 0, 0], o[0, 0, 0, 0])
    out = oracle.merge_pair_fp64(st, ident)
    assert out[0] == st[0] and out[1] == st[1] and np.array_equal(out[2], st[2])
    # one tile covering everything == one pass (loop body empty)
    m1, l1, o1 = oracle.splitkv_partials_fp64(q, k, v, scale=0.5, tile=1024)
    one = oracle.attention_fp64(q, k, v, scale=0.5)
    np.testing.assert_allclose(o1[..., 0, :] / l1[..., 0, None], one, rtol=1e-14)


# ---------------------------------------------------------------- paged, rows subsets

def test_paged_equals_contiguous():
    w = workloads.make_paged(B=4, Hq=8, Hkv=2, d=16, max_q=5, max_kv=300, seed=7, extra_pages=5)
    f = workloads.to_f64
    out = oracle.paged_attention_fp64(f(w["q"]), w["cu_seqlens_q"].numpy(), f(w["k_cache"]),
                                      f(w["v_cache"]), w["page_table"].numpy(), w["kv_len"].numpy(),
                                      scale=w["scale"], page_size=64, sink=f(w["sink"]))
    assert not np.any(np.isnan(out))
    cu = w["cu_seqlens_q"].numpy()
    pt = w["page_table"].numpy()
    for b in range(4):
        n = int(w["kv_len"][b])
        rows = np.arange(n)
        kb = f(w["k_cache"])[pt[b, rows // 64], rows % 64].transpose(1, 0, 2)[None]
        vb = f(w["v_cache"])[pt[b, rows // 64], rows % 64].transpose(1, 0, 2)[None]
        qb = f(w["q"])[cu[b]:cu[b + 1]].transpose(1, 0, 2)[None]
        dense = oracle.attention_fp64(qb, kb, vb, scale=w["scale"], sink=f(w["sink"]))
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], dense[0].transpose(1, 0, 2),
                                   rtol=1e-14, atol=1e-15)


def test_paged_permuted_table_is_invariant():
    w = workloads.make_paged(B=3, Hq=4, Hkv=1, d=8, max_q=4, max_kv=200, seed=3, extra_pages=2)
    f = workloads.to_f64
    kc, vc, pt = f(w["k_cache"]), f(w["v_cache"]), w["page_table"].numpy()
    perm = np.random.default_rng(0).permutation(kc.shape[0])
    inv = np.argsort(perm)
    pt2 = np.where(pt >= 0, inv[np.maximum(pt, 0)], -1)
    args = dict(scale=w["scale"], page_size=64, sink=f(w["sink"]))
    a = oracle.paged_attention_fp64(f(w["q"]), w["cu_seqlens_q"], kc, vc, pt, w["kv_len"], **args)
    b = oracle.paged_attention_fp64(f(w["q"]), w["cu_seqlens_q"], kc[perm], vc[perm], pt2,
                                    w["kv_len"], **args)
    np.testing.assert_array_equal(a, b)


def test_row_subsets_match_full():
    q, k, v = rand(2, 4, 6, 8), rand(2, 2, 12, 8), rand(2, 2, 12, 8)
    sink = rand(4)
    full = oracle.attention_fp64(q, k, v, scale=0.3, kv_len=[12, 5], sink=sink, causal=True)
    bi, hi, ii = [0, 1, 1, 0, 1, 1, 0], [3, 0, 2, 1, 0, 0, 3], [5, 0, 4, 2, 3, 1, 0]
    for chunk in (512, 1):  # rows of one (b, h) together, and one at a time
        rows = oracle.attention_rows_fp64(q, k, v, bi, hi, ii, scale=0.3, kv_len=[12, 5],
                                          sink=sink, causal=True, row_chunk=chunk)
        np.testing.assert_allclose(rows, full[bi, hi, ii], rtol=1e-13, atol=1e-15)
    w = workloads.make_paged(B=3, Hq=4, Hkv=1, d=8, max_q=6, max_kv=150, seed=5, extra_pages=1)
    f = workloads.to_f64
    args = dict(scale=w["scale"], page_size=64, sink=f(w["sink"]))
    pf = oracle.paged_attention_fp64(f(w["q"]), w["cu_seqlens_q"], f(w["k_cache"]),
                                     f(w["v_cache"]), w["page_table"], w["kv_len"], **args)
    t_idx = [0, w["total_q"] - 1, w["total_q"] // 2]
    h_idx = [1, 3, 0]
    pr = oracle.paged_attention_rows_fp64(f(w["q"]), w["cu_seqlens_q"], f(w["k_cache"]),
                                          f(w["v_cache"]), w["page_table"], w["kv_len"], t_idx,
                                          h_idx, **args)
    np.testing.assert_allclose(pr, pf[t_idx, h_idx], rtol=1e-13, atol=1e-15)


def test_paged_append_equals_attention_over_the_full_cache():
    """The append form stores each token's K/V at key row kv_len - q_len + i:
    with those rows cut out of a pool (NaN in their place) and handed in as
    k_new / v_new, it must give back the original pool and exactly the
    attention over it (any wrong row or token index leaves a NaN hole or
    moves a key)."""
    f = workloads.to_f64
    for causal in (False, True):
        w = workloads.make_paged(B=4, Hq=8, Hkv=2, d=16, q_lens=[1, 3, 1, 5],
                                 kv_lens=[1, 70, 128, 129], seed=9)
        kn, vn, kh, vh = workloads.take_new_kv(w)
        assert torch.isnan(kh.float()).any()
        args = dict(scale=w["scale"], page_size=64, sink=f(w["sink"]), causal=causal)
        want = oracle.paged_attention_fp64(f(w["q"]), w["cu_seqlens_q"], f(w["k_cache"]),
                                           f(w["v_cache"]), w["page_table"], w["kv_len"], **args)
        got, kc, vc = oracle.paged_append_fp64(f(w["q"]), w["cu_seqlens_q"], f(kh), f(vh),
                                               w["page_table"], w["kv_len"], f(kn), f(vn), **args)
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(kc, f(w["k_cache"]))
        np.testing.assert_array_equal(vc, f(w["v_cache"]))


def test_paged_append_drops_tokens_before_row_zero():
    """kv_len 2 with 3 query tokens: token 0 would be key row -1 and is dropped;
    tokens 1 and 2 become key rows 0 and 1 (checked against the plain
    definition over those two keys)."""
    rng = np.random.default_rng(4)
    q, kn, vn = rng.standard_normal((3, 2, 8)), rng.standard_normal((3, 1, 8)), \
        rng.standard_normal((3, 1, 8))
    kc = np.full((2, 64, 1, 8), np.nan)
    vc = np.full((2, 64, 1, 8), np.nan)
    out, kc2, _ = oracle.paged_append_fp64(q, [0, 3], kc, vc, [[1, 0]], [2], kn, vn, scale=0.5,
                                           page_size=64)
    np.testing.assert_array_equal(kc2[1, :2, 0], kn[1:, 0])
    assert np.isnan(kc2[1, 2:]).all() and np.isnan(kc2[0]).all()
    want = oracle.attention_fp64(q.transpose(1, 0, 2)[None], kn[1:].transpose(1, 0, 2)[None],
                                 vn[1:].transpose(1, 0, 2)[None], scale=0.5)
    np.testing.assert_array_equal(out, want[0].transpose(1, 0, 2))


# ---------------------------------------------------------------- workloads

def test_workloads_deterministic_and_structured():
    a = workloads.make_dense(2, 4, 1, 3, 9, 8, seed=11, kv_len="random", sink=True, nan_pad=True)
    b = workloads.make_dense(2, 4, 1, 3, 9, 8, seed=11, kv_len="random", sink=True, nan_pad=True)
    for key in ("q", "k", "v", "kv_len", "sink"):
        assert torch.equal(a[key].view(torch.int16) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.int16) if b[key].dtype == torch.bfloat16 else b[key])
    w = workloads.make_paged()
    pt = w["page_table"].numpy()
    used = pt[pt >= 0]
    assert len(np.unique(used)) == len(used)                     # no page shared
    assert w["k_cache"].shape[0] == len(used) + 16
    unused = np.setdiff1d(np.arange(w["k_cache"].shape[0]), used)
    assert torch.isnan(w["k_cache"][unused].float()).all()
    for b in range(8):
        n = int(w["kv_len"][b])
        padded = 128 * -(-n // 128)
        assert (pt[b] >= 0).sum() == padded // 64
        last = pt[b, (padded - 1) // 64]
        tail = w["k_cache"][last, (n % 64 or 64):].float()
        assert torch.isnan(tail).all()
    assert 1 <= int(w["q_len"].min()) and int(w["q_len"].max()) <= 64
    assert int(w["kv_len"].max()) <= 4096

"""Plain float64 definition of grouped-query attention forward.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  No online softmax,
no tiling, no fusion: each query row's softmax is taken over all of its
visible keys at once, exactly as the definition reads.  numpy matmul is the
only library primitive used.

What is computed (all arithmetic in float64; inputs are whatever values the
caller passes, normally the exact bf16 values promoted):

    for every batch b, query head h, query row i < q_len[b]:
        g   = h // (Hq // Hkv)                  query head h reads kv head g
        n   = kv_len[b]                          true length, not padded length
        hi  = n                 (non-causal)
            = clip(n - q_len[b] + i + 1, 0, n)   (causal, bottom-right aligned)
        s_j = scale * <q[b,h,i], k[b,g,j]>       for j < hi
        m   = max({s_j} U {sink[h]})             no sink == -inf
        if m == -inf: O = 0                      no visible key and no sink
        w_j = exp(s_j - m);  Z = sum_j w_j + exp(sink[h] - m)
        O[b,h,i] = sum_j w_j v[b,g,j] / Z

Sources:
* head grouping (h -> h // G) and one kv head serving G consecutive query
  heads: AstrAI commit log, the commit packing HB = min(G, warps) query heads
  per block; nvfp4-megamoe-kernel commit log, the multi-head decode commit
  (MQA through a zero K head stride).
* the true kv_len distinct from the padded length, padded columns kept out
  of the max and the sum: nvfp4-megamoe-kernel commit log, the commit that
  passes N_orig as s_k (the 1/128 dilution bug).
* the sink as an extra logit already in the scaled domain (compared with
  max(scale*QK) directly, never multiplied by scale): nvfp4-megamoe-kernel
  commit log, the sink-bias commit.  The sink has no value row, so it enters
  only the max and the denominator.
* divide by the row sum exactly once: nvfp4-megamoe-kernel commit log, the
  normalise-once commit.
* split partials (m, l, O~) with O~ un-normalised, and their merge:
  nvfp4-megamoe-kernel commit log, the multi-tile FA2 commit (P left
  un-normalised, final O = acc / running sum); kernbench2 benches commit
  log, the tile-granular ring-KV commit (persistent (m, l, O) state, tiles
  of TILE_S_KV) and the 2-D mesh all-reduce-mlo commit (the merge is
  associative, so any order or tree gives the same result).

Readings where the pages are silent (listed again in the design notes):
* causal alignment when q_len != kv_len is bottom-right (query i sees keys
  j <= kv_len - q_len + i); at q_len == kv_len this is "query i sees 0..i".
* a row with no visible key and no sink returns 0, never NaN.
"""

from __future__ import annotations

import numpy as np

_NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _visible(n: int, q_len: int, i: np.ndarray, causal: bool) -> np.ndarray:
    """Number of keys each query row i sees (keys 0 .. hi-1)."""
    i = np.asarray(i, dtype=np.int64)
    if not causal:
        return np.full(i.shape, n, dtype=np.int64)
    return np.clip(n - q_len + i + 1, 0, n)


def _attend_rows(qr: np.ndarray, K: np.ndarray, V: np.ndarray, hi: np.ndarray,
                 scale: float, sink_h: float | None) -> np.ndarray:
    """Softmax attention for a block of query rows that share one (K, V).

    qr [r, d]; K, V [n, d]; hi [r] visible-key counts; returns [r, d].
    """
    r, d = qr.shape
    n = K.shape[0]
    out = np.zeros((r, d), dtype=np.float64)
    if r == 0:
        return out
    sink = _NEG_INF if sink_h is None else float(sink_h)
    if n == 0:
        # only the sink column could be visible; it carries no value row
        return out
    s = scale * (qr @ K.T)                                    # [r, n]
    vis = np.arange(n)[None, :] < hi[:, None]                 # [r, n]
    s_masked = np.where(vis, s, _NEG_INF)
    m = np.maximum(s_masked.max(axis=1), sink)                # [r]
    live = m > _NEG_INF
    if not np.any(live):
        return out
    ml = m[live]
    w = np.where(vis[live], np.exp(s_masked[live] - ml[:, None]), 0.0)
    z = w.sum(axis=1) + (np.exp(sink - ml) if sink > _NEG_INF else 0.0)
    out[live] = (w @ V) / z[:, None]
    return out


def attention_fp64(q, k, v, *, scale: float, kv_len=None, sink=None,
                   causal: bool = False, row_chunk: int = 1024) -> np.ndarray:
    """Dense-layout GQA forward.

    q [B, Hq, Sq, d]; k, v [B, Hkv, Skv, d]; kv_len int [B] or None (= Skv);
    sink [Hq] (scaled-domain logits) or None; returns float64 [B, Hq, Sq, d].
    Every query row of the dense layout is a real row (q_len = Sq).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Skv, dk = k.shape
    assert Bk == B and dk == d and v.shape == k.shape and Hq % Hkv == 0
    G = Hq // Hkv
    kvl = np.full(B, Skv, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    snk = None if sink is None else _f64(sink)
    out = np.zeros((B, Hq, Sq, d), dtype=np.float64)
    for b in range(B):
        n = int(min(max(kvl[b], 0), Skv))
        for h in range(Hq):
            g = h // G
            K = k[b, g, :n]
            V = v[b, g, :n]
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                hi = _visible(n, Sq, rows, causal)
                kmax = int(hi.max()) if hi.size else 0
                out[b, h, rows] = _attend_rows(q[b, h, rows], K[:kmax], V[:kmax], hi,
                                               scale, None if snk is None else snk[h])
    return out


def attention_rows_fp64(q, k, v, b_idx, h_idx, i_idx, *, scale: float, kv_len=None,
                        sink=None, causal: bool = False, row_chunk: int = 512) -> np.ndarray:
    """The same definition evaluated only at selected rows (b, h, i).

    Used to check full-size runs on selected outputs; returns [len(b_idx), d].
    The rows asked for one (b, h) are evaluated together (each still over
    its own visible keys), in groups of at most `row_chunk`.
    """
    q = np.asarray(q)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kvl = np.full(B, Skv, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    b_idx, h_idx, i_idx = (np.asarray(x, dtype=np.int64) for x in (b_idx, h_idx, i_idx))
    out = np.zeros((len(b_idx), d), dtype=np.float64)
    for b, h in sorted(set(zip(b_idx.tolist(), h_idx.tolist()))):
        sel = np.nonzero((b_idx == b) & (h_idx == h))[0]
        n = int(min(max(kvl[b], 0), Skv))
        for c0 in range(0, sel.size, row_chunk):
            part = sel[c0:c0 + row_chunk]
            hi = _visible(n, Sq, i_idx[part], causal)
            kmax = int(hi.max())
            K = _f64(k[b, h // G, :kmax])
            V = _f64(v[b, h // G, :kmax])
            out[part] = _attend_rows(_f64(q[b, h, i_idx[part]]), K, V, hi, scale,
                                     None if sink is None else float(np.asarray(sink)[h]))
    return out


def softmax_weights_fp64(q, k, *, scale: float, kv_len=None, sink=None,
                         causal: bool = False):
    """Normalised softmax weights of every row, keys and sink column apart.

    Returns (w [B, Hq, Sq, Skv], w_sink [B, Hq, Sq]); invisible keys get 0.
    A row with nothing visible has all-zero weights.
    """
    q, k = _f64(q), _f64(k)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kvl = np.full(B, Skv, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    w = np.zeros((B, Hq, Sq, Skv))
    ws = np.zeros((B, Hq, Sq))
    for b in range(B):
        n = int(min(max(kvl[b], 0), Skv))
        hi = _visible(n, Sq, np.arange(Sq), causal)
        for h in range(Hq):
            snk = _NEG_INF if sink is None else float(np.asarray(sink)[h])
            s = scale * (q[b, h] @ k[b, h // G].T)               # [Sq, Skv]
            vis = np.arange(Skv)[None, :] < hi[:, None]
            s = np.where(vis, s, _NEG_INF)
            m = np.maximum(s.max(axis=1), snk)
            for i in range(Sq):
                if m[i] == _NEG_INF:
                    continue
                e = np.where(vis[i], np.exp(s[i] - m[i]), 0.0)
                es = np.exp(snk - m[i]) if snk > _NEG_INF else 0.0
                z = e.sum() + es
                w[b, h, i] = e / z
                ws[b, h, i] = es / z
    return w, ws


def splitkv_partials_fp64(q, k, v, *, scale: float, tile: int, kv_len=None,
                          causal: bool = False):
    """Per-split partial states of the split-KV form.

    Split s covers keys [s*tile, (s+1)*tile) intersected with the row's
    visible range.  Each partial is (m_s, l_s, O~_s) with
        m_s  = max_j s_j,   l_s = sum_j exp(s_j - m_s),
        O~_s = sum_j exp(s_j - m_s) v_j   (un-normalised),
    and an empty split is (-inf, 0, 0).  The sink is not part of any split;
    it enters once, at the merge.  n_split = ceil(Skv / tile).
    Returns m, l [B, Hq, Sq, n_split] and o [B, Hq, Sq, n_split, d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    ns = max(1, -(-Skv // tile))
    kvl = np.full(B, Skv, dtype=np.int64) if kv_len is None else np.asarray(kv_len, dtype=np.int64)
    m = np.full((B, Hq, Sq, ns), _NEG_INF)
    l = np.zeros((B, Hq, Sq, ns))
    o = np.zeros((B, Hq, Sq, ns, d))
    for b in range(B):
        n = int(min(max(kvl[b], 0), Skv))
        hi = _visible(n, Sq, np.arange(Sq), causal)
        for h in range(Hq):
            g = h // G
            s_all = scale * (q[b, h] @ k[b, g].T)                # [Sq, Skv]
            for sp in range(ns):
                lo_j, hi_j = sp * tile, min((sp + 1) * tile, Skv)
                cols = np.arange(lo_j, hi_j)
                for i in range(Sq):
                    c = cols[cols < hi[i]]
                    if c.size == 0:
                        continue
                    s = s_all[i, c]
                    ms = s.max()
                    e = np.exp(s - ms)
                    m[b, h, i, sp] = ms
                    l[b, h, i, sp] = e.sum()
                    o[b, h, i, sp] = e @ v[b, g, c]
    return m, l, o


def merge_partials_fp64(m, l, o, *, sink=None, head_axis: int = 1):
    """Merge split partials into the normalised output (one normalisation).

    m, l [..., n_split]; o [..., n_split, d]; sink [Hq] broadcast along
    `head_axis` of m's leading dims, or None.
        M = max(sink, max_s m_s)
        L = exp(sink - M) + sum_s l_s exp(m_s - M)
        O = sum_s O~_s exp(m_s - M) / L
    Empty splits (m_s = -inf) weigh 0; with M = -inf the row is 0.
    """
    m, l, o = _f64(m), _f64(l), _f64(o)
    lead = m.shape[:-1]
    if sink is None:
        snk = np.full(lead, _NEG_INF)
    else:
        shape = [1] * len(lead)
        shape[head_axis] = -1
        snk = np.broadcast_to(_f64(sink).reshape(shape), lead)
    M = np.maximum(m.max(axis=-1), snk)
    live = M > _NEG_INF
    Msafe = np.where(live, M, 0.0)
    ws = np.where(m > _NEG_INF, np.exp(m - Msafe[..., None]), 0.0)
    wsink = np.where(snk > _NEG_INF, np.exp(snk - Msafe), 0.0)
    L = wsink + (l * ws).sum(axis=-1)
    num = (o * ws[..., None]).sum(axis=-2)
    out = np.zeros(num.shape)
    out[live] = num[live] / L[live][..., None]
    return out


def merge_pair_fp64(a, b):
    """Associative combine of two un-normalised states (m, l, O~).

    m = max(m1, m2); l = l1 e^(m1-m) + l2 e^(m2-m); O~ likewise.  A state with
    m = -inf is the identity.  Arrays broadcast elementwise (o has a trailing d).
    """
    m1, l1, o1 = (_f64(x) for x in a)
    m2, l2, o2 = (_f64(x) for x in b)
    m = np.maximum(m1, m2)
    ms = np.where(m > _NEG_INF, m, 0.0)
    w1 = np.where(m1 > _NEG_INF, np.exp(m1 - ms), 0.0)
    w2 = np.where(m2 > _NEG_INF, np.exp(m2 - ms), 0.0)
    return m, l1 * w1 + l2 * w2, o1 * w1[..., None] + o2 * w2[..., None]


def gather_paged_fp64(cache, page_table, kv_len, page_size: int):
    """Contiguous copy of each sequence's first kv_len[b] rows from a paged pool.

    cache [n_pages, page_size, Hkv, d]; page_table int [B, max_pages]; row j
    of sequence b sits in page page_table[b, j // page_size], in-page row
    j % page_size (AstrAI commit log, the paged KV / KVSource commits; int32
    page tables).  Integer indexing only.  Returns a list of [Hkv, n_b, d].
    """
    cache = np.asarray(cache)
    pt = np.asarray(page_table, dtype=np.int64)
    seqs = []
    for b in range(pt.shape[0]):
        n = int(kv_len[b])
        j = np.arange(n)
        pages = pt[b, j // page_size]
        rows = cache[pages, j % page_size]                         # [n, Hkv, d]
        seqs.append(_f64(rows).transpose(1, 0, 2))
    return seqs


def paged_attention_fp64(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, *,
                         scale: float, page_size: int, sink=None,
                         causal: bool = False) -> np.ndarray:
    """Ragged-Q, paged-KV form of the same definition.

    q [total_q, Hq, d] packed by cu_seqlens_q [B+1]; returns [total_q, Hq, d].
    Sequence b's K/V are gathered from the pool first, then attended exactly
    as in `attention_fp64` with q_len = cu[b+1] - cu[b], kv_len = kv_len[b].
    """
    q = _f64(q)
    total_q, Hq, d = q.shape
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    Ks = gather_paged_fp64(k_cache, page_table, kv_len, page_size)
    Vs = gather_paged_fp64(v_cache, page_table, kv_len, page_size)
    Hkv = Ks[0].shape[0] if Ks else 1
    G = Hq // Hkv
    out = np.zeros((total_q, Hq, d))
    for b in range(len(cu) - 1):
        qlen = int(cu[b + 1] - cu[b])
        n = int(kv_len[b])
        rows = np.arange(qlen)
        hi = _visible(n, qlen, rows, causal)
        for h in range(Hq):
            g = h // G
            out[cu[b] + rows, h] = _attend_rows(q[cu[b] + rows, h], Ks[b][g], Vs[b][g], hi,
                                                scale, None if sink is None else float(np.asarray(sink)[h]))
    return out


def paged_append_fp64(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, k_new, v_new, *,
                      scale: float, page_size: int, sink=None, causal: bool = False):
    """Append form of `paged_attention_fp64`: the query tokens bring their own K/V.

    AstrAI commit log, the paged decode fix (the decode kernel reads the
    newest tokens' K/V through separate new-K / new-V pointers rather than
    from the cache).  Token i of sequence b (packed row cu[b] + i) holds key
    row j = kv_len[b] - q_len_b + i of that sequence; a token with j < 0 is
    dropped.  The rows are stored into copies of the pools first (page
    page_table[b, j // page_size], in-page row j % page_size), then the
    attention is exactly `paged_attention_fp64` over those copies.
    Returns (out [total_q, Hq, d], k_cache', v_cache').
    """
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    kn, vn = _f64(k_new), _f64(v_new)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    pt = np.asarray(page_table, dtype=np.int64)
    for b in range(len(cu) - 1):
        qlen = int(cu[b + 1] - cu[b])
        n = int(kv_len[b])
        for i in range(qlen):
            j = n - qlen + i
            if j < 0:
                continue
            page = pt[b, j // page_size]
            kc[page, j % page_size] = kn[cu[b] + i]
            vc[page, j % page_size] = vn[cu[b] + i]
    out = paged_attention_fp64(q, cu, kc, vc, page_table, kv_len, scale=scale,
                               page_size=page_size, sink=sink, causal=causal)
    return out, kc, vc


def paged_attention_rows_fp64(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, t_idx,
                              h_idx, *, scale: float, page_size: int, sink=None,
                              causal: bool = False) -> np.ndarray:
    """`paged_attention_fp64` evaluated only at packed rows (t, h)."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    pt = np.asarray(page_table, dtype=np.int64)
    Hq = q.shape[1]
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((len(t_idx), q.shape[2]))
    for r, (t, h) in enumerate(zip(t_idx, h_idx)):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        qlen = int(cu[b + 1] - cu[b])
        i = int(t - cu[b])
        n = int(kv_len[b])
        hi = _visible(n, qlen, np.array([i]), causal)
        j = np.arange(int(hi[0]))
        pages = pt[b, j // page_size]
        K = _f64(k_cache[pages, j % page_size, h // G])
        V = _f64(v_cache[pages, j % page_size, h // G])
        out[r] = _attend_rows(_f64(q[t, h])[None, :], K, V, hi, scale,
                              None if sink is None else float(np.asarray(sink)[h]))[0]
    return out

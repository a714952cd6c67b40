"""Seeded synthetic inputs for the GQA forward pass.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  Both sides of every parity check (the HIP library and the fp64
oracle) are fed from here, and so is the benchmark.

Recipe (the same on every machine, CPU generator):
* ``torch.Generator('cpu').manual_seed(seed)``; draws happen in a fixed order.
* Q, K, V: float32 N(0, 1) draws rounded to bf16 (round-to-nearest-even).
* dense layout: Q/O [B, Hq, Sq, d], K/V [B, Hkv, Skv, d], d contiguous.
* paged layout: Q/O packed [total_q, Hq, d] with cu_seqlens_q [B+1]; K/V in a
  page pool [n_pages, 64, Hkv, d]; page_table int32 [B, max_pages] built from
  a seeded random permutation of the pool, unused entries -1; rows at or past
  kv_len[b] and pages no sequence references are NaN, so a kernel that lets a
  padded column into the max, the sum or P.V fails loudly.
* scale is the float32 value of 1/sqrt(d).

The five named workloads follow the shapes of the pages' GQA cases (the
short-q/long-kv G=8 B=16 q=16 kv=16k prefill of the AstrAI commit log, the
decode and S_q=16 prefill panels of the kernbench2 bench commits, the
head-dim x T x s_k grid of the nvfp4-megamoe-kernel commits).  None of them
is a public benchmark or dataset.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


def f32_scale(d: int) -> float:
    """float32 value of 1/sqrt(d), as a Python float."""
    return float(np.float32(1.0 / math.sqrt(d)))


def _randn_bf16(g: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


@dataclass
class DenseCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    causal: bool = False
    tile_s_kv: int = 0          # 0 = one pass; >0 = split-KV tiles of this many keys
    decode: bool = False        # Sq == 1 through the decode entry point
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The named workloads; seed 1000 + k for workload k.
CASES = {
    "tiny_prefill": DenseCase("tiny_prefill", 1, 4, 1, 16, 128, 64, seed=1001),
    "decode_splitkv": DenseCase("decode_splitkv", 16, 32, 8, 1, 8192, 128,
                                tile_s_kv=1024, decode=True, seed=1002),
    "shortq_longkv": DenseCase("shortq_longkv", 16, 32, 4, 16, 16384, 128, seed=1003),
    "causal_prefill": DenseCase("causal_prefill", 2, 32, 8, 8192, 8192, 128,
                                causal=True, seed=1004),
}

PAGED_SEED = 1005
CHUNKED_SEED = 1006

# The same decode and causal prefill shapes at the other head dims the pages'
# kernels cover (decode at d = 256, prefill at d = 32, and d = 512); measured
# beside the named workloads.
HEAD_DIM_CASES = {
    "decode_splitkv_d256": DenseCase("decode_splitkv_d256", 16, 32, 8, 1, 8192, 256,
                                     tile_s_kv=1024, decode=True, seed=1008),
    "causal_prefill_d32": DenseCase("causal_prefill_d32", 2, 32, 8, 8192, 8192, 32,
                                    causal=True, seed=1009),
    "causal_prefill_d256": DenseCase("causal_prefill_d256", 2, 32, 8, 8192, 8192, 256,
                                     causal=True, seed=1010),
    # d = 512 (the nvfp4-megamoe-kernel sweep's widest head)
    "decode_splitkv_d512": DenseCase("decode_splitkv_d512", 16, 32, 8, 1, 8192, 512,
                                     tile_s_kv=1024, decode=True, seed=1012),
    "causal_prefill_d512": DenseCase("causal_prefill_d512", 2, 32, 8, 8192, 8192, 512,
                                     causal=True, seed=1013),
}


def make_dense(B, Hq, Hkv, Sq, Skv, d, seed, *, kv_len=None, sink=False,
               nan_pad=False):
    """Dense-layout inputs.

    Draw order: Q, K, V, then (if asked) kv_len ~ U[1, Skv] and sink ~ N(0,1).
    `kv_len` may also be given explicitly (list/array of B ints).  With
    `nan_pad`, K/V rows at or past kv_len[b] are set to NaN.
    Returns a dict of CPU tensors: q, k, v (bf16), kv_len (int32 [B] or None),
    sink (float32 [Hq] or None), scale (float).
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = _randn_bf16(g, (B, Hq, Sq, d))
    k = _randn_bf16(g, (B, Hkv, Skv, d))
    v = _randn_bf16(g, (B, Hkv, Skv, d))
    kvl = None
    if isinstance(kv_len, str) and kv_len == "random":
        kvl = torch.randint(1, Skv + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    elif kv_len is not None:
        kvl = torch.as_tensor(np.asarray(kv_len), dtype=torch.int32)
    snk = torch.randn(Hq, generator=g, dtype=torch.float32) if sink else None
    if nan_pad and kvl is not None:
        for b in range(B):
            n = int(kvl[b])
            k[b, :, n:] = float("nan")
            v[b, :, n:] = float("nan")
    return {"q": q, "k": k, "v": v, "kv_len": kvl, "sink": snk, "scale": f32_scale(d)}


def make_case(case: DenseCase):
    """Inputs of a named dense workload (kv_len = Skv for every sequence)."""
    out = make_dense(case.B, case.Hq, case.Hkv, case.Sq, case.Skv, case.d, case.seed)
    out["kv_len"] = torch.full((case.B,), case.Skv, dtype=torch.int32)
    return out


def make_paged(B=8, Hq=32, Hkv=1, d=128, *, max_q=64, max_kv=4096, page_size=64,
               pad_to=128, extra_pages=16, seed=PAGED_SEED, q_lens=None, kv_lens=None,
               sink=True):
    """Ragged-Q, paged-KV inputs (the ragged paged workload by default).

    Draw order: q_len ~ U[1, max_q] and kv_len ~ U[1, max_kv] per sequence
    (unless given), then Q, K, V (logical [padded_b, Hkv, d] per sequence,
    padded_b = pad_to * ceil(kv_len_b / pad_to)), then the permutation of the
    page pool, then sink ~ N(0, 1) per query head.
    The pool holds every used page plus `extra_pages` unreferenced ones.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    if q_lens is None:
        q_lens = torch.randint(1, max_q + 1, (B,), generator=g, dtype=torch.int64)
    else:
        q_lens = torch.as_tensor(np.asarray(q_lens), dtype=torch.int64)
    if kv_lens is None:
        kv_lens = torch.randint(1, max_kv + 1, (B,), generator=g, dtype=torch.int64)
    else:
        kv_lens = torch.as_tensor(np.asarray(kv_lens), dtype=torch.int64)
    padded = [pad_to * max(1, -(-int(n) // pad_to)) for n in kv_lens]
    total_q = int(q_lens.sum())
    q = _randn_bf16(g, (total_q, Hq, d))
    ks = [_randn_bf16(g, (p, Hkv, d)) for p in padded]
    vs = [_randn_bf16(g, (p, Hkv, d)) for p in padded]
    n_used = sum(p // page_size for p in padded)
    n_pool = n_used + extra_pages
    perm = torch.randperm(n_pool, generator=g)
    snk = torch.randn(Hq, generator=g, dtype=torch.float32) if sink else None

    max_pages = max(p // page_size for p in padded)
    page_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    k_cache = torch.full((n_pool, page_size, Hkv, d), float("nan"), dtype=torch.bfloat16)
    v_cache = torch.full((n_pool, page_size, Hkv, d), float("nan"), dtype=torch.bfloat16)
    off = 0
    for b in range(B):
        kb, vb = ks[b].clone(), vs[b].clone()
        n = int(kv_lens[b])
        kb[n:] = float("nan")
        vb[n:] = float("nan")
        for p in range(padded[b] // page_size):
            pid = int(perm[off + p])
            page_table[b, p] = pid
            k_cache[pid] = kb[p * page_size:(p + 1) * page_size]
            v_cache[pid] = vb[p * page_size:(p + 1) * page_size]
        off += padded[b] // page_size
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(q_lens, 0).to(torch.int32)
    return {
        "q": q, "k_cache": k_cache, "v_cache": v_cache, "page_table": page_table,
        "cu_seqlens_q": cu, "kv_len": kv_lens.to(torch.int32), "q_len": q_lens.to(torch.int32),
        "sink": snk, "scale": f32_scale(d), "page_size": page_size,
        "max_q_len": int(q_lens.max()), "total_q": total_q, "B": B, "Hq": Hq, "Hkv": Hkv,
        "d": d,
    }


def make_paged_chunked(B=8, Hq=32, Hkv=1, d=128, *, chunk=512, max_prefix=3584,
                       seed=CHUNKED_SEED):
    """Causal chunked prefill over a cached prefix, same heads as the paged workload.

    Each sequence appends a chunk of `chunk` query tokens to a cached prefix of
    prefix_b ~ U[0, max_prefix] tokens, so kv_len_b = prefix_b + chunk and the
    chunk's row i sees keys 0 .. prefix_b + i (bottom-right aligned causal).
    Draw order: the prefixes from `seed`, then everything else as in
    `make_paged` from `seed + 1`.
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    prefix = torch.randint(0, max_prefix + 1, (B,), generator=g, dtype=torch.int64)
    return make_paged(B, Hq, Hkv, d, max_q=chunk, max_kv=max_prefix + chunk, seed=seed + 1,
                      q_lens=[chunk] * B, kv_lens=(prefix + chunk).tolist())


def make_paged_decode(B=16, Hq=32, Hkv=8, d=128, kv=8192, seed=1011):
    """The split-KV decode shape over a paged pool: one query token per
    sequence, every sequence kv keys long (the token's own key included)."""
    return make_paged(B, Hq, Hkv, d, q_lens=[1] * B, kv_lens=[kv] * B, seed=seed, sink=False)


def take_new_kv(w):
    """Append-form inputs from a paged workload: the K/V rows of every query
    token (token i of sequence b is key row kv_len[b] - q_len_b + i) are
    copied out of the pools into packed [total_q, Hkv, d] tensors, and those
    cache rows are set to NaN.  Requires kv_len[b] >= q_len_b.
    Returns (k_new, v_new, k_cache_with_holes, v_cache_with_holes)."""
    cu = w["cu_seqlens_q"].numpy().astype(np.int64)
    pt = w["page_table"].numpy().astype(np.int64)
    kv_len = w["kv_len"].numpy().astype(np.int64)
    ps = w["page_size"]
    kc, vc = w["k_cache"].clone(), w["v_cache"].clone()
    k_new = torch.empty((w["total_q"],) + tuple(kc.shape[2:]), dtype=kc.dtype)
    v_new = torch.empty_like(k_new)
    for b in range(len(cu) - 1):
        qlen = int(cu[b + 1] - cu[b])
        assert kv_len[b] >= qlen, "each sequence's keys must include its query tokens"
        for i in range(qlen):
            j = int(kv_len[b]) - qlen + i
            page, row = int(pt[b, j // ps]), j % ps
            k_new[cu[b] + i] = kc[page, row]
            v_new[cu[b] + i] = vc[page, row]
            kc[page, row] = float("nan")
            vc[page, row] = float("nan")
    return k_new, v_new, kc, vc


def to_f64(t) -> np.ndarray:
    """Exact float64 copy of a CPU tensor (bf16 and f32 promote exactly)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()

"""The Python binding's argument checks (CPU only, nothing is launched).

The library takes B, Hkv, Skv and d from q and k alone, so the binding must
reject a v, out, kv_len, sink or page table that disagrees with them before
the call: otherwise the kernels would read or write past a buffer.  Shape
checks run before the device checks, so CPU tensors exercise them here; a
consistent set of CPU tensors is refused as not on the GPU (there is no CPU
path).
"""

import pytest
import torch

import gqa_attention_forward_amd as m

BF = torch.bfloat16


def dense(B=2, Hq=8, Hkv=2, Sq=3, Skv=40, d=64):
    q = torch.zeros(B, Hq, Sq, d, dtype=BF)
    k = torch.zeros(B, Hkv, Skv, d, dtype=BF)
    return q, k, k.clone()


def test_dense_v_with_fewer_keys_is_rejected():
    q, k, _ = dense()
    v = torch.zeros(2, 2, 39, 64, dtype=BF)
    with pytest.raises(ValueError, match="v has shape"):
        m.prefill(q, k, v)
    with pytest.raises(ValueError, match="v has shape"):
        m.splitkv_partial(q, k, v, tile_s_kv=64)


def test_dense_k_with_another_head_dim_or_batch_is_rejected():
    q, _, _ = dense()
    for k in (torch.zeros(2, 2, 40, 32, dtype=BF), torch.zeros(1, 2, 40, 64, dtype=BF)):
        with pytest.raises(ValueError, match="does not match q"):
            m.prefill(q, k, k)


def test_dense_out_kv_len_and_sink_must_match():
    q, k, v = dense()
    with pytest.raises(ValueError, match="out has shape"):
        m.prefill(q, k, v, out=torch.zeros(2, 8, 2, 64, dtype=BF))
    with pytest.raises(ValueError, match="kv_len must be a contiguous \\[2\\]"):
        m.prefill(q, k, v, kv_len=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="sink must be a contiguous \\[8\\]"):
        m.prefill(q, k, v, sink=torch.zeros(2, dtype=torch.float32))
    with pytest.raises(ValueError, match="sink must be a contiguous"):
        m.prefill(q, k, v, sink=torch.zeros(16, dtype=torch.float32)[::2])


def test_decode_checks_shapes_first():
    q, k, v = dense(Sq=1)
    with pytest.raises(ValueError, match="out has shape"):
        m.decode_splitkv(q, k, v, out=torch.zeros(2, 8, 1, 32, dtype=BF))
    with pytest.raises(ValueError, match="v has shape"):
        m.decode_splitkv(q, k, v[:, :, :10], fused=True)


def test_merge_out_must_match_sizes():
    ws = torch.zeros(4096, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out has shape"):
        m.splitkv_merge(ws, B=2, Hq=8, Sq=3, d=64, n_split=2,
                        out=torch.zeros(2, 8, 3, 32, dtype=BF))
    with pytest.raises(ValueError, match="sink must be"):
        m.splitkv_merge(ws, B=2, Hq=8, Sq=3, d=64, n_split=2, sink=torch.zeros(3))


def paged_inputs(B=3, Hq=8, Hkv=2, d=64, total_q=5, pages=4):
    q = torch.zeros(total_q, Hq, d, dtype=BF)
    kc = torch.zeros(16, 64, Hkv, d, dtype=BF)
    cu = torch.tensor([0, 1, 3, 5], dtype=torch.int32)[: B + 1]
    pt = torch.zeros(B, pages, dtype=torch.int32)
    kvl = torch.full((B,), 100, dtype=torch.int32)
    return q, cu, kc, kc.clone(), pt, kvl


def test_paged_shapes_must_agree():
    q, cu, kc, vc, pt, kvl = paged_inputs()
    with pytest.raises(ValueError, match="page_table has shape"):
        m.paged(q, cu, kc, vc, pt[:2], kvl, max_q_len=2)
    with pytest.raises(ValueError, match="kv_len must be a contiguous \\[3\\]"):
        m.paged(q, cu, kc, vc, pt, kvl[:2], max_q_len=2)
    with pytest.raises(ValueError, match="do not match page_size"):
        m.paged(q, cu, kc[:, :32], vc[:, :32], pt, kvl, max_q_len=2)
    with pytest.raises(ValueError, match="do not match page_size"):
        m.paged(q[..., :32], cu, kc, vc, pt, kvl, max_q_len=2)
    with pytest.raises(ValueError, match="share shape"):
        m.paged(q, cu, kc, vc[:8], pt, kvl, max_q_len=2)
    with pytest.raises(ValueError, match="out has shape"):
        m.paged(q, cu, kc, vc, pt, kvl, max_q_len=2, out=torch.zeros(4, 8, 64, dtype=BF))


def test_consistent_cpu_tensors_are_refused_not_computed():
    q, k, v = dense()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        m.prefill(q, k, v, kv_len=torch.zeros(2, dtype=torch.int32),
                  sink=torch.zeros(8, dtype=torch.float32))
    q, cu, kc, vc, pt, kvl = paged_inputs()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        m.paged(q, cu, kc, vc, pt, kvl, max_q_len=2)

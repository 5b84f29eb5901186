"""The seeded synthetic workloads (no GPU): each named configuration has the
shapes, length mix and page structure of its recipe, the same on every build
(the byte and flop counts behind the reported rates depend on them), and its
page tables address disjoint pages except where a prefix is shared on
purpose ("FlashInfer内核库深度解析", PageAttention: pages from a pool through
a per-request table; "FlashAttention-3 内核在最新大模型推理中的集成实践",
section 二: packed sequences addressed by cu_seqlens)."""
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402


def test_single_sequence_fp32_decode():
    c = workloads.make_config(1)
    assert c.q.shape == (1, 4, 64) and c.q.dtype == torch.float32
    assert c.kv_lens.tolist() == [256] and c.page_size == 16 and c.Hkv == 4
    assert c.page_table.tolist() == [list(range(16))]       # contiguous KV as identity-mapped pages
    assert c.scale == 1.0 / 8.0
    assert c.kv_bytes() == 2 * 256 * 4 * 64 * 4


def test_paged_decode_batch():
    c = workloads.make_config(2)
    assert (c.B, c.Hq, c.Hkv, c.D, c.page_size, c.num_pages) == (64, 32, 8, 128, 16, 300000)
    lens = c.kv_lens.tolist()
    assert all(512 <= L <= 4096 for L in lens)
    assert sum(lens) == 140653                                  # seed 2
    assert c.kv_bytes() == 4096 * 140653
    used = []
    for b, L in enumerate(lens):
        n = (L + 15) // 16
        ids = c.page_table[b, :n].tolist()
        assert all(0 <= i < c.num_pages for i in ids)
        used += ids
    assert len(set(used)) == len(used)                          # no page shared between requests
    again = workloads.make_config(2)
    assert torch.equal(again.kv_lens, c.kv_lens) and torch.equal(again.page_table, c.page_table)


def test_ragged_prefill():
    c = workloads.make_config(3)
    assert (c.B, c.Hq, c.Hkv, c.D, c.causal) == (8, 64, 8, 128, True)
    lens = c.lens_q
    assert all(1024 <= L <= 4096 for L in lens)
    assert torch.equal(c.cu_seqlens_q, c.cu_seqlens_k) and c.lens_k == lens
    assert c.cu_seqlens_q[0].item() == 0 and c.cu_seqlens_q[-1].item() == c.q.shape[0] == sum(lens)
    assert c.flops() == 4 * 128 * 64 * sum(L * (L + 1) // 2 for L in lens)


def test_chunked_paged_prefill_with_shared_prefix():
    c = workloads.make_config(5)
    assert (c.B, c.Hq, c.Hkv, c.D, c.page_size) == (16, 16, 16, 256, 16)
    assert c.cu_seqlens_q.tolist() == list(range(0, 8192 + 1, 512))
    assert c.kv_lens.tolist() == [8704] * 16
    assert c.pool_k.shape == (4864, 16, 16, 256)
    t = c.page_table
    assert t.shape[1] >= 8704 // 16
    prefix = t[:, :256]
    assert (prefix == prefix[0]).all()                          # 4096 shared tokens, one copy
    own = t[:, 256:544].reshape(-1).tolist()
    assert len(set(own)) == len(own) == 16 * 288                # own pages disjoint
    assert not set(own) & set(prefix[0].tolist())
    assert all(0 <= i < 4864 for i in own + prefix[0].tolist())


def test_long_prefill_recipe():
    """The 32K prefill and its sweep prefixes (built on the GPU machine only: 640
    MB of inputs): the recipe's counts."""
    assert workloads.CONFIG_NAMES[4] == "prefill_causal_bf16_b1_l32768_hq64_hkv8_d128"
    for L in (1024, 4096, 16384, 32768):
        assert workloads.prefill_flops([L], [L], 64, 128, True) == 4 * 128 * 64 * L * (L + 1) // 2

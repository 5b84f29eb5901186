"""GPU parity of attn_decode_paged_fp8 (decode over an E4M3 cache) against the oracle.

The oracle takes the same E4M3 bytes and scales (oracle.ref_decode_paged_fp8),
so the comparison measures the kernel, not the quantisation: the tolerance is
that of the 16-bit decode path.
"""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _run(case, gpu, fp8, split_pages=0, table=None, lens=None, max_kv_len=None, q=None, window=-1,
         layout="NHD"):
    import attention_qk_online_amd as A
    kb, vb, ks, vs = fp8
    if layout == "HND":
        kb, vb = kb.transpose(1, 2).contiguous(), vb.transpose(1, 2).contiguous()
    t = (case.page_table if table is None else table).to(gpu)
    kl = (case.kv_lens if lens is None else lens).to(gpu)
    out, lse = A.decode_paged_fp8((case.q if q is None else q).to(gpu), kb.to(gpu), vb.to(gpu), t,
                                  kl, ks, vs, scale=case.scale,
                                  max_kv_len=case.max_kv_len if max_kv_len is None else max_kv_len,
                                  split_pages=split_pages, kv_layout=layout, window_left=window)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, fp8, q=None, requests=None, window=-1):
    kb, vb, ks, vs = fp8
    return oracle.ref_decode_paged_fp8(case.q if q is None else q, kb, vb, ks, vs, case.page_table,
                                       case.kv_lens, case.scale, requests=requests,
                                       window_left=window)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 8), (256, 16, 2)])
@pytest.mark.parametrize("split_pages", [0, 2])
def test_fp8_window(gpu, D, Hq, Hkv, split_pages):
    """Sliding window on the E4M3 cache: windows inside a page, on page edges
    and wider than the keys, against the oracle's windowed fp8 decode."""
    lens = [1, 15, 16, 17, 300, 64, 1000, 0, 33]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=torch.bfloat16, seed=520 + D + Hq, extra_pages=4)
    fp8 = case.fp8_pools()
    for window in (0, 5, 15, 16, 17, 100, 1000):
        out, lse = _run(case, gpu, fp8, split_pages, window=window)
        ro, rl = _oracle(case, fp8, window=window)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"fp8 D{D} window {window} split{split_pages}")


def test_fp8_window_hnd_and_wide(gpu):
    """HND equals NHD bit for bit with a window; a window covering every key
    equals the plain E4M3 call bit for bit."""
    case = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[33, 400, 16, 1, 250],
                                 dtype=torch.bfloat16, seed=530, extra_pages=3)
    fp8 = case.fp8_pools()
    o1, l1 = _run(case, gpu, fp8, 2, window=37)
    o2, l2 = _run(case, gpu, fp8, 2, window=37, layout="HND")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = _run(case, gpu, fp8, 2)
    o4, l4 = _run(case, gpu, fp8, 2, window=400)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


def test_fp8_window_paged_config(gpu):
    """The batched paged GQA decode workload (B 64, Hq 32, Hkv 8, D 128) over an
    E4M3 cache with a 1024-key window, every request against the oracle."""
    case = workloads.make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                                 dtype=torch.bfloat16, seed=2, num_pages=20000)
    fp8 = case.fp8_pools()
    out, lse = _run(case, gpu, fp8, window=1024)
    ro, rl = _oracle(case, fp8, window=1024)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "fp8 paged decode window 1024")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (128, 8, 2), (64, 8, 8), (256, 16, 2),
                                      (128, 8, 1)])
@pytest.mark.parametrize("split_pages", [0, 2])
def test_small_fp8(gpu, D, Hq, Hkv, split_pages):
    lens = [1, 15, 16, 17, 300, 64, 1000, 3, 0]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=torch.bfloat16, seed=500 + D + Hq, extra_pages=5)
    fp8 = case.fp8_pools()
    out, lse = _run(case, gpu, fp8, split_pages)
    ro, rl = _oracle(case, fp8)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"fp8 D{D} Hq{Hq} Hkv{Hkv} split{split_pages}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_small_fp8_fp16_queries(gpu, D):
    lens = [7, 300, 16, 1, 129]
    case = workloads.make_decode(B=len(lens), Hq=16, Hkv=4, D=D, page_size=16, kv_lens=lens,
                                 dtype=torch.float16, seed=510 + D, extra_pages=3)
    fp8 = case.fp8_pools()
    out, lse = _run(case, gpu, fp8, split_pages=3)
    ro, rl = _oracle(case, fp8)
    assert_parity(out, lse, ro, rl, torch.float16, f"fp8 cache, fp16 queries D{D}")


def test_every_value_byte_is_exact(gpu):
    """One key per request and v_scale 1: the output row is the value row itself,
    so each E4M3 byte's conversion is seen exactly (NaN bytes give NaN columns)."""
    D = 64
    case = workloads.make_decode(B=4, Hq=2, Hkv=1, D=D, page_size=16, kv_lens=[1, 1, 1, 1],
                                 dtype=torch.bfloat16, seed=520, permute_pages=False,
                                 extra_pages=0)
    kb, vb, ks, _ = case.fp8_pools()
    for b in range(4):                       # request b's value row holds bytes 64b .. 64b+63
        vb[int(case.page_table[b, 0]), 0, 0] = torch.arange(64 * b, 64 * b + 64).to(torch.uint8)
    out, lse = _run(case, gpu, (kb, vb, ks, 1.0))
    want = torch.arange(256).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.bfloat16)
    got = out.cpu()
    for b in range(4):
        for h in range(2):
            g, w = got[b, h], want[64 * b:64 * b + 64]
            assert torch.equal(torch.isnan(g), torch.isnan(w)), (b, h)
            ok = ~torch.isnan(w)
            assert torch.equal(g[ok], w[ok]), (b, h)
    ro, rl = _oracle(case, (kb, vb, ks, 1.0))
    assert_parity(out[:, :, :0], lse, ro[:, :, :0], rl, torch.bfloat16, "single-key lse")


def test_scales_and_large_logits(gpu):
    """Key scale 40x (logits in the hundreds) and a negative value scale."""
    case = workloads.make_decode(B=3, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=[700, 33, 2000],
                                 dtype=torch.bfloat16, seed=530)
    kb, vb, ks, vs = case.fp8_pools()
    fp8 = (kb, vb, 40.0 * ks, -0.5 * vs)
    out, lse = _run(case, gpu, fp8, split_pages=4)
    ro, rl = _oracle(case, fp8)
    assert torch.isfinite(out.float()).all() and rl.abs().max() > 100
    assert_parity(out, lse, ro, rl, torch.bfloat16, "fp8 scaled")


def test_fp8_empty_and_bad_requests(gpu):
    """kv_len 0 -> out 0, lse -inf; a page id outside the pool -> NaN for that request."""
    case = workloads.make_decode(B=3, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=[0, 40, 40],
                                 dtype=torch.bfloat16, seed=540, extra_pages=2)
    fp8 = case.fp8_pools()
    table = case.page_table.clone()
    table[2, 1] = case.num_pages + 5
    out, lse = _run(case, gpu, fp8, split_pages=1, table=table)
    ro, rl = _oracle(case, fp8)
    out, lse = out.cpu(), lse.cpu()
    assert torch.equal(out[0].float(), torch.zeros_like(out[0].float()))
    assert torch.isneginf(lse[0]).all()
    assert_parity(out[1:2], lse[1:2], ro[1:2], rl[1:2], torch.bfloat16, "neighbour")
    assert torch.isnan(out[2].float()).all() and torch.isnan(lse[2]).all()


def test_fp8_equals_16bit_on_exact_values(gpu):
    """A 16-bit cache holding exactly the dequantised E4M3 values (scales 1) gives the
    same result as the E4M3 cache up to the order of the fp32 sums (the E4M3 path
    feeds the head dimension to the matrix cores in another order): the
    conversion is exact and the rest of the path is shared."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16,
                                 kv_lens=[33, 400, 16, 1, 250], dtype=torch.bfloat16, seed=550,
                                 extra_pages=4, poison=False)
    kb, vb, _, _ = case.fp8_pools()
    out8, lse8 = _run(case, gpu, (kb, vb, 1.0, 1.0), split_pages=5)
    kp = kb.view(torch.float8_e4m3fn).to(torch.bfloat16).to(gpu)
    vp = vb.view(torch.float8_e4m3fn).to(torch.bfloat16).to(gpu)
    out16, lse16 = A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu),
                                  case.kv_lens.to(gpu), scale=case.scale,
                                  max_kv_len=case.max_kv_len, split_pages=5)
    torch.cuda.synchronize()
    assert (lse8 - lse16).abs().max().item() <= 1e-4
    assert (out8.float() - out16.float()).abs().max().item() <= 1e-2


def test_paged_config_fp8(gpu):
    """The batched paged GQA decode workload (B 64, Hq 32, Hkv 8, D 128, kv_len in
    [512, 4096]) over an E4M3 cache, every request against the oracle."""
    case = workloads.make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                                 dtype=torch.bfloat16, seed=2, num_pages=20000)
    fp8 = case.fp8_pools()
    for split in (0, 8):
        out, lse = _run(case, gpu, fp8, split_pages=split)
        ro, rl = _oracle(case, fp8)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"fp8 paged config split{split}")

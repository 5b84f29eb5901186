"""GPU parity of attn_decode_paged (split-KV decode + LSE combine) against the oracle."""
import math

import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _run(case, gpu, split_pages=0, pools=None, table=None):
    import attention_qk_online_amd as A
    kp, vp = pools if pools is not None else case.pools(gpu)
    t = (case.page_table if table is None else table).to(gpu)
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, t, case.kv_lens.to(gpu), scale=case.scale,
                              max_kv_len=case.max_kv_len, split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case):
    kp, vp = case.pools("cpu")
    return oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale)


def test_single_sequence_fp32(gpu):
    """fp32 decode, 1 token, 4 heads (MHA), head_dim 64, contiguous KV of 256 as pages."""
    case = workloads.make_config(1)
    out, lse = _run(case, gpu)
    ro, rl = _oracle(case)
    assert_parity(out, lse, ro, rl, torch.float32, case.name)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (128, 32, 8), (64, 8, 8), (256, 16, 2),
                                      (128, 8, 1)])
@pytest.mark.parametrize("split_pages", [0, 1, 2, 7])
def test_small_paged_bf16(gpu, D, Hq, Hkv, split_pages):
    lens = [1, 15, 16, 17, 300, 64, 1000, 3]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=torch.bfloat16, seed=100 + D + Hq, extra_pages=9)
    out, lse = _run(case, gpu, split_pages)
    ro, rl = _oracle(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"D{D} Hq{Hq} Hkv{Hkv} split{split_pages}")


def test_small_fp32_groups(gpu):
    for G in (1, 2, 4, 8):
        case = workloads.make_decode(B=3, Hq=8, Hkv=8 // G, D=128, page_size=16, kv_lens=[5, 77, 200],
                                     dtype=torch.float32, seed=7 + G)
        out, lse = _run(case, gpu, split_pages=3)
        ro, rl = _oracle(case)
        assert_parity(out, lse, ro, rl, torch.float32, f"fp32 G{G}")


def test_split_counts_agree(gpu):
    """Forced split counts (1 page .. whole request) agree with each other and the oracle."""
    case = workloads.make_decode(B=4, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[2000, 1, 513, 4096],
                                 dtype=torch.bfloat16, seed=9)
    ro, rl = _oracle(case)
    pools = case.pools(gpu)
    results = []
    for sp in (1, 2, 7, 64, 256):
        out, lse = _run(case, gpu, sp, pools=pools)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"split_pages={sp}")
        results.append(out.float())
    for r in results[1:]:
        assert (r - results[0]).abs().max().item() <= 2e-2


def test_page_permutation_bitwise(gpu):
    """Moving physical pages (and remapping the table) changes nothing, bit for bit."""
    case = workloads.make_decode(B=5, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=[33, 400, 16, 1, 250],
                                 dtype=torch.bfloat16, seed=11, extra_pages=20)
    kp, vp = case.pools(gpu)
    out1, lse1 = _run(case, gpu, pools=(kp, vp))
    perm = torch.randperm(case.num_pages, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(case.num_pages)
    pg = perm.to(gpu)
    out2, lse2 = _run(case, gpu, pools=(kp[pg].contiguous(), vp[pg].contiguous()),
                      table=inv[case.page_table.long()].to(torch.int32))
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_deterministic(gpu):
    case = workloads.make_decode(B=6, Hq=32, Hkv=8, D=128, page_size=16, len_range=(1, 3000),
                                 dtype=torch.bfloat16, seed=12)
    pools = case.pools(gpu)
    a = _run(case, gpu, pools=pools)
    b = _run(case, gpu, pools=pools)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_and_bad_requests(gpu):
    """kv_len 0 -> out 0, lse -inf; an out-of-range page id or an oversize kv_len
    poisons only that request with NaN; neighbours are unaffected."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=4, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=[0, 40, 40, 40],
                                 dtype=torch.bfloat16, seed=13, extra_pages=2)
    ro, rl = _oracle(case)
    kp, vp = case.pools(gpu)
    table = case.page_table.clone()
    table[2, 1] = case.num_pages + 5           # out of range
    lens = case.kv_lens.clone()
    lens[3] = 10 ** 6                          # above max_kv_len
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, table.to(gpu), lens.to(gpu), scale=case.scale,
                              max_kv_len=48, split_pages=1)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.equal(out[0].float(), torch.zeros_like(out[0].float()))
    assert torch.isneginf(lse[0]).all()
    assert_parity(out[1:2], lse[1:2], ro[1:2], rl[1:2], torch.bfloat16, "neighbour")
    assert torch.isnan(out[2].float()).all() and torch.isnan(lse[2]).all()
    assert torch.isnan(out[3].float()).all() and torch.isnan(lse[3]).all()


def test_large_logits(gpu):
    """Logits around 1000 (scale x q.k): the online rescaling keeps the result finite."""
    case = workloads.make_decode(B=2, Hq=4, Hkv=1, D=128, page_size=16, kv_lens=[700, 33],
                                 dtype=torch.bfloat16, seed=14, scale=40.0)
    out, lse = _run(case, gpu, split_pages=3)
    ro, rl = _oracle(case)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert rl.abs().max() > 500
    assert_parity(out, lse, ro, rl, torch.bfloat16, "large logits")


@pytest.fixture(scope="module")
def paged_config(gpu):
    """Batched paged GQA decode at full size: B 64, Hq 32, Hkv 8, D 128, page 16,
    kv_len in [512, 4096], pages scattered over a 300k-page pool (inputs on the
    GPU and the oracle's answer)."""
    case = workloads.make_config(2)
    pools = case.pools(gpu)
    ro, rl = _oracle(case)
    return case, pools, ro, rl


@pytest.mark.parametrize("split_pages", [0, 8, 64])
def test_paged_config_full(gpu, paged_config, split_pages):
    """Auto runs, and fixed runs that outnumber the waves of the grid (8 pages)."""
    case, pools, ro, rl = paged_config
    out, lse = _run(case, gpu, split_pages=split_pages, pools=pools)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"{case.name} split_pages={split_pages}")


def test_workspace_contents_do_not_matter(gpu):
    """One caller workspace, filled with NaN bit patterns, reused across bf16 calls
    of different shapes and run lengths: every result equals a fresh-workspace
    call bit for bit."""
    import attention_qk_online_amd as A
    c1 = workloads.make_decode(B=8, Hq=8, Hkv=2, D=128, page_size=16,
                               kv_lens=[700, 1, 33, 512, 0, 129, 64, 1000], dtype=torch.bfloat16,
                               seed=410, extra_pages=5)
    c2 = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=16, kv_lens=[300, 2048, 17, 5, 900],
                               dtype=torch.bfloat16, seed=411, extra_pages=3)
    calls = ((c1, 2), (c2, 0), (c1, 8), (c2, 1))
    need = max(A.decode_paged_workspace_size(torch.bfloat16, c.B, c.Hq, c.Hkv, c.D, 16, c.max_kv_len, s)
               for c, s in calls)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=gpu)
    for case, split in calls:
        kp, vp = case.pools(gpu)
        args = (case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu))
        kw = dict(scale=case.scale, max_kv_len=case.max_kv_len, split_pages=split)
        o_ref, l_ref = A.decode_paged(*args, **kw)
        out, lse = A.decode_paged(*args, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), (case.name, split)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_many_requests(gpu, dtype):
    """More than 64 requests: the device-side schedule scans kv_lens 64 at a time."""
    g = torch.Generator().manual_seed(420)
    lens = torch.randint(0, 300, (150,), generator=g).tolist()
    lens[7] = 0
    lens[100] = 1
    case = workloads.make_decode(B=150, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=lens, dtype=dtype,
                                 seed=421, extra_pages=4)
    for split in (0, 3):
        out, lse = _run(case, gpu, split)
        ro, rl = _oracle(case)
        assert_parity(out, lse, ro, rl, dtype, f"B150 {dtype} split{split}")


def test_more_than_512_requests(gpu):
    """700 requests: the schedule reads the lengths 512 at a time (two
    batches of eight 64-request chunks), in the unit count, the run's
    request search and the merge; an inconsistent length in the second
    batch poisons only its own request."""
    import attention_qk_online_amd as A
    g = torch.Generator().manual_seed(430)
    lens = torch.randint(0, 200, (700,), generator=g).tolist()
    lens[3] = 0
    lens[511] = 1
    lens[512] = 199
    case = workloads.make_decode(B=700, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=lens,
                                 dtype=torch.bfloat16, seed=431, extra_pages=4)
    ro, rl = _oracle(case)
    kp, vp = case.pools(gpu)
    for split in (0, 2):
        out, lse = _run(case, gpu, split, pools=(kp, vp))
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"B700 split{split}")
    kv = case.kv_lens.clone()
    kv[600] = case.max_kv_len + 1
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu), kv.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isnan(out[600].float()).all() and torch.isnan(lse[600]).all()
    keep = torch.arange(700) != 600
    assert_parity(out[keep], lse[keep], ro[keep], rl[keep], torch.bfloat16, "B700, request 600 bad")


def test_more_than_4096_requests(gpu):
    """4200 short requests: the unit count hands the run's request search the
    count at the end of each of the first 64 chunks of 64 requests; runs
    starting past them search on from chunk 64."""
    g = torch.Generator().manual_seed(440)
    lens = torch.randint(0, 48, (4200,), generator=g).tolist()
    case = workloads.make_decode(B=4200, Hq=4, Hkv=2, D=64, page_size=16, kv_lens=lens,
                                 dtype=torch.bfloat16, seed=441, extra_pages=2)
    ro, rl = _oracle(case)
    for split in (0, 1):
        out, lse = _run(case, gpu, split)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"B4200 split{split}")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 8), (256, 16, 2)])
@pytest.mark.parametrize("split_pages", [0, 2])
def test_small_paged_fp16(gpu, D, Hq, Hkv, split_pages):
    lens = [1, 15, 16, 17, 300, 64, 1000, 3, 0]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                 dtype=torch.float16, seed=430 + D + Hq, extra_pages=5)
    out, lse = _run(case, gpu, split_pages)
    ro, rl = _oracle(case)
    assert_parity(out, lse, ro, rl, torch.float16, f"fp16 D{D} Hq{Hq} Hkv{Hkv} split{split_pages}")


def test_paged_config_fp16(gpu):
    """The batched paged GQA decode workload with fp16 inputs."""
    case = workloads.make_decode(B=64, Hq=32, Hkv=8, D=128, page_size=16, len_range=(512, 4096),
                                 dtype=torch.float16, seed=2, num_pages=20000)
    out, lse = _run(case, gpu)
    ro, rl = _oracle(case)
    assert_parity(out, lse, ro, rl, torch.float16, "fp16 paged decode B64")


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 32, 8), (torch.bfloat16, 64, 8, 8),
                                            (torch.bfloat16, 256, 16, 2), (torch.float16, 128, 8, 4),
                                            (torch.bfloat16, 128, 4, 4)])
def test_few_long_requests(gpu, dtype, D, Hq, Hkv):
    """One to three long requests: each (request, head group) spans more than
    64 runs, so the merge folds its segments on several waves per head and
    combines them through LDS (G = 1, 2, 4, 8); an empty request among them
    gets out 0 and lse -inf."""
    for lens in ([20000], [9000, 0, 5000], [12001, 7777]):
        case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                     dtype=dtype, seed=900 + D + Hq + len(lens), extra_pages=3)
        out, lse = _run(case, gpu)
        ro, rl = _oracle(case)
        assert_parity(out, lse, ro, rl, dtype, f"{dtype} D{D} Hq{Hq} Hkv{Hkv} lens {lens}")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (256, 16, 2), (64, 8, 8)])
def test_many_segment_merge_chunks_and_idle_waves(gpu, D, Hq, Hkv):
    """The 16-wave merge with one-page runs: the long request leaves ~1250
    partial states per head, so each wave folds two chunks of 64; the short
    one leaves 3, so 13 of the 16 waves hold none.  The workspace starts as
    NaN bit patterns (the merge reads its first slots before it knows the
    segment count): the result equals a fresh-workspace call bit for bit and
    matches the oracle; the empty request gets out 0 and lse -inf."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=3, Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=[20000, 40, 0],
                                 dtype=torch.bfloat16, seed=960 + D, extra_pages=2)
    kp, vp = case.pools(gpu)
    args = (case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu))
    kw = dict(scale=case.scale, max_kv_len=case.max_kv_len, split_pages=1)
    need = A.decode_paged_workspace_size(torch.bfloat16, case.B, Hq, Hkv, D, 16, case.max_kv_len, 1)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=gpu)
    out, lse = A.decode_paged(*args, workspace=ws, **kw)
    o_ref, l_ref = A.decode_paged(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
    ro, rl = _oracle(case)
    assert_parity(out.cpu(), lse.cpu(), ro, rl, torch.bfloat16, f"D{D} Hq{Hq} Hkv{Hkv} split_pages 1")


def test_few_long_requests_bad_page(gpu):
    """A bad page id in one of two long requests poisons only that request."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=2, Hq=32, Hkv=8, D=128, page_size=16, kv_lens=[16000, 16000],
                                 dtype=torch.bfloat16, seed=950, extra_pages=2)
    ro, rl = _oracle(case)
    kp, vp = case.pools(gpu)
    table = case.page_table.clone()
    table[1, 700] = case.num_pages + 3
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert_parity(out[0:1], lse[0:1], ro[0:1], rl[0:1], torch.bfloat16, "clean request")
    assert torch.isnan(out[1].float()).all() and torch.isnan(lse[1]).all()


def _repage16(case, kp, vp):
    """The same NHD cache seen as 16-token pages (zero copy) and its page table."""
    m = case.page_size // 16
    kp16 = kp.reshape(kp.shape[0] * m, 16, *kp.shape[2:])
    vp16 = vp.reshape(vp.shape[0] * m, 16, *vp.shape[2:])
    t = case.page_table.long()
    j = torch.arange(t.shape[1] * m)
    return kp16, vp16, (t[:, j // m] * m + j % m).to(torch.int32)


@pytest.mark.parametrize("P", [32, 64, 128, 256])
@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 32, 8), (torch.float16, 64, 8, 8),
                                            (torch.bfloat16, 256, 16, 2)])
def test_larger_pages(gpu, P, dtype, D, Hq, Hkv):
    """Pages of 32 to 256 tokens: parity with the oracle, and the same cache seen
    as 16-token pages gives the same result bit for bit (the kernel walks
    16-token blocks either way)."""
    import attention_qk_online_amd as A
    lens = [1, 15, 16, 17, 300, 64, 1000, 0, 33, 257]
    case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=P, kv_lens=lens,
                                 dtype=dtype, seed=960 + P + D, extra_pages=3)
    ro, rl = _oracle(case)
    kp, vp = case.pools(gpu)
    kp16, vp16, t16 = _repage16(case, kp, vp)
    q, lens_d = case.q.to(gpu), case.kv_lens.to(gpu)
    for split in (0, 2):
        out, lse = A.decode_paged(q, kp, vp, case.page_table.to(gpu), lens_d, scale=case.scale,
                                  max_kv_len=case.max_kv_len, split_pages=split)
        o16, l16 = A.decode_paged(q, kp16, vp16, t16.to(gpu), lens_d, scale=case.scale,
                                  max_kv_len=case.max_kv_len, split_pages=split)
        torch.cuda.synchronize()
        assert_parity(out, lse, ro, rl, dtype, f"page {P} {dtype} D{D} split {split}")
        assert torch.equal(out, o16) and torch.equal(lse, l16)


def test_larger_pages_variants(gpu):
    """64-token pages with a sliding window (NHD and HND), the rotary
    embedding and an E4M3 cache, each against the oracle."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=5, Hq=16, Hkv=4, D=128, page_size=64, kv_lens=[33, 400, 16, 1, 250],
                                 dtype=torch.bfloat16, seed=970, extra_pages=3)
    kc, vc = case.pools("cpu")
    q, t, lens_d = case.q.to(gpu), case.page_table.to(gpu), case.kv_lens.to(gpu)
    for layout in ("NHD", "HND"):
        kp, vp = case.pools(gpu, layout=layout)
        out, lse = A.decode_paged(q, kp, vp, t, lens_d, scale=case.scale, max_kv_len=case.max_kv_len,
                                  kv_layout=layout, window_left=37)
        torch.cuda.synchronize()
        ro, rl = oracle.ref_decode_paged(case.q, kc, vc, case.page_table, case.kv_lens, case.scale,
                                         window_left=37)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"page 64 {layout} window 37")
    kp, vp = case.pools(gpu)
    out, lse = A.decode_paged(q, kp, vp, t, lens_d, scale=case.scale, max_kv_len=case.max_kv_len,
                              rope_theta=10000.0)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_decode_paged(case.q, kc, vc, case.page_table, case.kv_lens, case.scale,
                                     rope=(10000.0, 1.0))
    assert_parity(out, lse, ro, rl, torch.bfloat16, "page 64 rope")
    kb, vb, ks, vs = case.fp8_pools()
    out, lse = A.decode_paged_fp8(q, kb.to(gpu), vb.to(gpu), t, lens_d, ks, vs, scale=case.scale,
                                  max_kv_len=case.max_kv_len)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_decode_paged_fp8(case.q, kb, vb, ks, vs, case.page_table, case.kv_lens,
                                         case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "page 64 E4M3")


@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("split", [0, 2])
def test_larger_pages_bad_page(gpu, layout, split):
    """64-token pages: a table entry outside the pool poisons only its request
    (NaN out and lse); the others match the oracle."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=4, Hq=8, Hkv=2, D=128, page_size=64, kv_lens=[100, 300, 70, 1],
                                 dtype=torch.bfloat16, seed=975, extra_pages=2)
    ro, rl = _oracle(case)
    table = case.page_table.clone()
    table[1, 2] = case.num_pages + 5           # tokens 128..191 of request 1
    kp, vp = case.pools(gpu, layout=layout)
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len, split_pages=split,
                              kv_layout=layout)
    torch.cuda.synchronize()
    good = torch.tensor([0, 2, 3])
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"good requests ({layout}, split {split})",
                  rows=good)
    assert torch.isnan(out[1].float()).all() and torch.isnan(lse[1]).all()


def test_undersized_workspace_is_refused(gpu):
    """The binding raises on a caller workspace smaller than the size query
    instead of allocating behind the caller's back."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=2, Hq=8, Hkv=2, D=128, page_size=16, kv_lens=[300, 40],
                                 dtype=torch.bfloat16, seed=976)
    kp, vp = case.pools(gpu)
    need = A.decode_paged_workspace_size(torch.bfloat16, case.B, case.Hq, case.Hkv, case.D, 16,
                                         case.max_kv_len, 0)
    small = torch.empty(need - 1, dtype=torch.uint8, device=gpu)
    with pytest.raises(ValueError, match="workspace"):
        A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu),
                       scale=case.scale, max_kv_len=case.max_kv_len, workspace=small)



@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 32, 8), (torch.bfloat16, 64, 8, 8),
                                            (torch.float16, 256, 16, 2), (torch.bfloat16, 128, 16, 2)])
def test_many_segments_per_pair(gpu, dtype, D, Hq, Hkv):
    """Long requests among short ones (max_kv_len 8064): their (request, KV
    head) pairs span tens of runs of the balanced cut.  With four requests the
    merge folds them with one wave per head, in chunks of 64 lse values; with
    a single request it runs segment-parallel (16 waves per workgroup).
    G = 1, 2, 4, 8."""
    for lens in ([8064, 100, 0, 17], [8064], [5000, 8000, 1, 4097]):
        case = workloads.make_decode(B=len(lens), Hq=Hq, Hkv=Hkv, D=D, page_size=16, kv_lens=lens,
                                     dtype=dtype, seed=1200 + D + Hq + len(lens), extra_pages=3)
        out, lse = _run(case, gpu)
        ro, rl = _oracle(case)
        assert_parity(out, lse, ro, rl, dtype, f"{dtype} D{D} Hq{Hq} Hkv{Hkv} lens {lens}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_empty_cache(gpu, dtype):
    """max_kv_len 0 with an empty pool and page table (NULL pointers at the
    boundary): kv_len 0 gives out 0 and lse -inf; a kv_len above the bound
    gives NaN and reads nothing."""
    import attention_qk_online_amd as A
    D = 128
    q = torch.randn(3, 8, D, device=gpu).to(dtype)
    pool = torch.empty((0, 16, 2, D), dtype=dtype, device=gpu)
    table = torch.empty((3, 0), dtype=torch.int32, device=gpu)
    lens = torch.tensor([0, 5, 0], dtype=torch.int32, device=gpu)
    out, lse = A.decode_paged(q, pool, pool, table, lens, scale=0.1, max_kv_len=0)
    torch.cuda.synchronize()
    out, lse = out.float().cpu(), lse.cpu()
    for b in (0, 2):
        assert torch.equal(out[b], torch.zeros(8, D)) and torch.isneginf(lse[b]).all()
    assert torch.isnan(out[1]).all() and torch.isnan(lse[1]).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_batch_above_65535_requests(gpu, dtype):
    """A batch of 70 000 short requests (grid dimensions indexed by request go
    past 65 535): sampled requests match the oracle."""
    B = 70000
    case = workloads.make_decode(B=B, Hq=4, Hkv=2, D=64, page_size=16, len_range=(0, 40),
                                 dtype=dtype, seed=1600, extra_pages=3, poison=False)
    out, lse = _run(case, gpu, split_pages=1 if dtype == torch.float32 else 0)
    picks = sorted(set(list(range(40)) + list(range(B - 40, B)) + list(range(0, B, 997))))
    kp, vp = case.pools("cpu")
    ro, rl = oracle.ref_decode_paged(case.q, kp, vp, case.page_table, case.kv_lens, case.scale,
                                     requests=picks)
    assert_parity(out, lse, ro, rl, dtype, f"B {B}", rows=picks)


@pytest.mark.parametrize("Hkv,G", [(3, 4), (5, 2), (12, 2), (16, 1), (32, 2)])
@pytest.mark.parametrize("lens", [[1, 700, 33, 2048], [5000]])
def test_more_than_eight_kv_heads(gpu, Hkv, G, lens):
    """A workgroup folds up to eight KV heads of a unit; more heads form
    several head groups per request (the last one partial when Hkv is not a
    multiple of 8), and a single long request takes the merge that splits
    heads and d over workgroups."""
    import attention_qk_online_amd as A
    case = workloads.make_decode(B=len(lens), Hq=G * Hkv, Hkv=Hkv, D=128, page_size=16, kv_lens=lens,
                                 dtype=torch.bfloat16, seed=1900 + Hkv, extra_pages=2)
    kp, vp = case.pools(gpu)
    out, lse = A.decode_paged(case.q.to(gpu), kp, vp, case.page_table.to(gpu), case.kv_lens.to(gpu),
                              scale=case.scale, max_kv_len=case.max_kv_len)
    torch.cuda.synchronize()
    kc, vc = case.pools()
    ro, rl = oracle.ref_decode_paged(case.q, kc, vc, case.page_table, case.kv_lens, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"Hkv {Hkv} G {G} lens {lens}")

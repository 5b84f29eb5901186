"""GPU parity of attn_prefill_varlen / attn_prefill_paged against the oracle."""
import pytest
import torch

import oracle
import workloads
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def _varlen(case, gpu, causal=None):
    import attention_qk_online_amd as A
    causal = case.causal if causal is None else causal
    out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu),
                                case.max_seqlen_q, case.max_seqlen_k, causal=causal,
                                scale=case.scale)
    torch.cuda.synchronize()
    return out, lse


def _paged(case, gpu, pools=None, table=None):
    import attention_qk_online_amd as A
    kp, vp = pools if pools is not None else case.pools(gpu)
    t = case.page_table if table is None else table
    out, lse = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp, t.to(gpu),
                               case.kv_lens.to(gpu), case.max_seqlen_q, case.max_kv_len,
                               causal=case.causal, scale=case.scale)
    torch.cuda.synchronize()
    return out, lse


def _ref(case, causal=None, rows=None):
    causal = case.causal if causal is None else causal
    return oracle.ref_prefill_varlen(case.q, case.k, case.v, case.cu_seqlens_q, case.cu_seqlens_k,
                                     causal, case.scale, rows=rows)


def _sample_rows(cu, n, seed):
    """Rows to check at full size: first/last two rows of every sequence, the
    rows around each 128-row tile edge of the first sequence, plus random rows."""
    cu = [int(x) for x in cu]
    rows = set()
    for a, b in zip(cu[:-1], cu[1:]):
        rows.update(r for r in (a, a + 1, b - 2, b - 1) if a <= r < b)
    for t in range(cu[0] + 127, min(cu[1], cu[0] + 1024), 128):
        rows.update((t, t + 1))
    g = torch.Generator().manual_seed(seed)
    rows.update(torch.randint(0, cu[-1], (n,), generator=g).tolist())
    return torch.tensor(sorted(r for r in rows if r < cu[-1]))


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_small_varlen(gpu, D, causal):
    lens = [1, 17, 128, 129, 300, 64, 255]
    case = workloads.make_prefill(B=len(lens), Hq=8, Hkv=2, D=D, lens_q=lens, dtype=torch.bfloat16,
                                  seed=200 + D, causal=causal)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"D{D} causal{causal}")


@pytest.mark.parametrize("G", [1, 4, 8])
def test_group_sizes(gpu, G):
    case = workloads.make_prefill(B=2, Hq=8, Hkv=8 // G, D=128, lens_q=[200, 77], dtype=torch.bfloat16,
                                  seed=210 + G, causal=True)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"G{G}")


def test_bottom_right_causal(gpu):
    """Lq != Lk: queries are the last Lq positions; Lq > Lk leaves leading rows empty."""
    case = workloads.make_prefill(B=4, Hq=4, Hkv=4, D=128, lens_q=[100, 5, 300, 40],
                                  lens_k=[500, 5, 130, 0], dtype=torch.bfloat16, seed=220, causal=True)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "bottom-right")


def test_causal_row0_and_gqa_bitwise(gpu):
    """Causal row 0 is exactly v[0]; GQA equals MHA with repeated K/V, bit for bit."""
    case = workloads.make_prefill(B=1, Hq=8, Hkv=2, D=128, lens_q=[333], dtype=torch.bfloat16,
                                  seed=230, causal=True)
    out, lse = _varlen(case, gpu)
    v0 = case.v[0].repeat_interleave(4, dim=0)
    assert torch.equal(out[0].cpu(), v0)
    rep = workloads.PrefillCase(**{**case.__dict__, "Hkv": 8,
                                   "k": case.k.repeat_interleave(4, dim=1).contiguous(),
                                   "v": case.v.repeat_interleave(4, dim=1).contiguous()})
    out2, lse2 = _varlen(rep, gpu)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_large_logits(gpu):
    case = workloads.make_prefill(B=1, Hq=2, Hkv=1, D=128, lens_q=[400], dtype=torch.bfloat16,
                                  seed=240, causal=True, scale=40.0)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert torch.isfinite(out.float()).all()
    assert rl.abs().max() > 500
    assert_parity(out, lse, ro, rl, torch.bfloat16, "large logits")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_running_max_raised_across_tiles_and_key_halves(gpu, D, causal):
    """Keys scaled so that each row's maximum score jumps between 64-key tiles
    and between the two 32-key halves of a tile (head_dim 256 splits a
    tile's scores between two waves that must agree on the running max):
    the running max is raised many times, by different amounts per half."""
    case = workloads.make_prefill(B=2, Hq=4, Hkv=2, D=D, lens_q=[333, 200], lens_k=[333, 520],
                                  dtype=torch.bfloat16, seed=245, causal=causal)
    j = torch.arange(case.k.shape[0])
    pos = j - torch.repeat_interleave(case.cu_seqlens_k[:-1].long(), torch.diff(case.cu_seqlens_k.long()))
    f = 1.0 + 3.0 * ((pos % 64) >= 32).float() + 0.75 * (pos // 64).float()
    # every third tile puts its larger keys in the first half instead
    f = torch.where((pos // 64) % 3 == 1, 1.0 + 5.0 * ((pos % 64) < 32).float(), f)
    case.k = (case.k.float() * f[:, None, None]).to(case.k.dtype)
    case.scale = 4.0 / D ** 0.5
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert torch.isfinite(out.float()).all()
    assert rl.abs().max() > 100
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"raised max D{D} causal {causal}")


def test_deterministic(gpu):
    case = workloads.make_prefill(B=3, Hq=8, Hkv=1, D=128, len_range=(100, 700), dtype=torch.bfloat16,
                                  seed=250, causal=True)
    a = _varlen(case, gpu)
    b = _varlen(case, gpu)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("D", [128, 256])
def test_small_paged(gpu, D):
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=D, page_size=16, chunk=70, cached=200,
                                        shared_prefix=64, dtype=torch.bfloat16, seed=260 + D)
    out, lse = _paged(case, gpu)
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"paged D{D}")


def test_paged_equals_contiguous_bitwise(gpu):
    """The paged loader and the contiguous loader give identical bits."""
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=4, D=128, page_size=16, chunk=150, cached=333,
                                        shared_prefix=32, dtype=torch.bfloat16, seed=270)
    out, lse = _paged(case, gpu)
    ks, vs, ck = [], [], [0]
    for b in range(case.B):
        L = int(case.kv_lens[b])
        ks.append(oracle.gather_pages(case.pool_k, case.page_table[b], L))
        vs.append(oracle.gather_pages(case.pool_v, case.page_table[b], L))
        ck.append(ck[-1] + L)
    contig = workloads.PrefillCase(name="contig", seed=0, B=case.B, Hq=4, Hkv=4, D=128,
                                   dtype=torch.bfloat16, causal=True, scale=case.scale, q=case.q,
                                   k=torch.cat(ks), v=torch.cat(vs), cu_seqlens_q=case.cu_seqlens_q,
                                   cu_seqlens_k=torch.tensor(ck, dtype=torch.int32))
    out2, lse2 = _varlen(contig, gpu)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_ragged_config_all_rows(gpu):
    """Ragged causal prefill at full size (B 8, L in [1024, 4096], Hq 64, Hkv 8,
    D 128): every row of out and lse against the oracle."""
    case = workloads.make_config(3)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, case.name + " (all rows)")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_long_config_short_prefixes_all_rows(gpu):
    """The 1K and 4K prefixes of the 32768-token causal prefill (Hq 64, Hkv 8,
    D 128): every row against the oracle."""
    case = workloads.make_config(4)
    for L in (1024, 4096):
        sub = case.prefix(L)
        out, lse = _varlen(sub, gpu)
        ro, rl = _ref(sub)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"{sub.name} (all rows)")
        del out, lse


def test_long_config_16k_all_rows(gpu):
    """The 16K prefix of the 32768-token causal prefill: every row."""
    sub = workloads.make_config(4).prefix(16384)
    out, lse = _varlen(sub, gpu)
    ro, rl = _ref(sub)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"{sub.name} (all rows)")
    assert torch.isfinite(out.float()).all()


def test_long_config_32k_sampled(gpu):
    """The whole 32768-token causal prefill: the first and last rows, the rows
    around the first query tiles' edges and random rows against the oracle
    (every row would take the float64 oracle minutes); all rows finite."""
    case = workloads.make_config(4)
    out, lse = _varlen(case, gpu)
    rows = _sample_rows(case.cu_seqlens_q, 48, 32768)
    ro, rl = _ref(case, rows=rows)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"{case.name} (sampled rows)", rows=rows)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_chunked_paged_config_all_rows(gpu):
    """Chunked prefill on a paged cache: 16 requests x 512-token chunks over 8192 cached
    tokens, the first 4096 on shared pages; Hq = Hkv = 16, D 256, page 16: every row."""
    case = workloads.make_config(5)
    out, lse = _paged(case, gpu)
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, case.name + " (all rows)")
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_zero_and_negative_scale(gpu, scale):
    """scale 0: every visible key weighs the same; a negative scale flips the scores."""
    case = workloads.make_prefill(B=2, Hq=4, Hkv=2, D=128, lens_q=[200, 77], dtype=torch.bfloat16,
                                  seed=280, causal=True, scale=scale)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"scale {scale}")


@pytest.mark.parametrize("causal", [True, False])
def test_q_and_k_lengths_differ(gpu, causal):
    """Lq != Lk in both directions, with and without the (bottom-right) causal mask, D 256."""
    case = workloads.make_prefill(B=4, Hq=4, Hkv=1, D=256, lens_q=[50, 300, 129, 1],
                                  lens_k=[400, 140, 129, 33], dtype=torch.bfloat16, seed=290,
                                  causal=causal)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"Lq!=Lk causal={causal}")


def test_group_of_sixteen_and_many_sequences(gpu):
    """16 query heads per KV head; 100 short sequences (one work item per head and tile)."""
    g = torch.Generator().manual_seed(300)
    lens = torch.randint(1, 200, (100,), generator=g).tolist()
    case = workloads.make_prefill(B=100, Hq=32, Hkv=2, D=128, lens_q=lens, dtype=torch.bfloat16,
                                  seed=301, causal=True)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, "G16 B100")


def test_overlong_sequence_is_nan(gpu):
    """A sequence longer than max_seqlen_q: the rows the launch covers are NaN; other
    sequences are unaffected."""
    import attention_qk_online_amd as A
    case = workloads.make_prefill(B=2, Hq=4, Hkv=2, D=128, lens_q=[100, 300], dtype=torch.bfloat16,
                                  seed=310, causal=True)
    out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu), 256, 300,
                                causal=True, scale=case.scale)
    torch.cuda.synchronize()
    ro, rl = _ref(case)
    assert_parity(out[:100], lse[:100], ro[:100], rl[:100], torch.bfloat16, "good sequence")
    assert torch.isnan(out[100:356].float()).all() and torch.isnan(lse[100:356]).all()


def test_paged_bad_page_is_nan(gpu):
    """A page id outside the pool: rows whose keys reach it are NaN (here every row of
    that request, as its chunk sees all cached tokens); other requests are unaffected."""
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=2, D=128, page_size=16, chunk=40, cached=100,
                                        shared_prefix=0, dtype=torch.bfloat16, seed=320)
    table = case.page_table.clone()
    table[1, 2] = case.num_pages + 5
    out, lse = _paged(case, gpu, table=table)
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    n0 = int(case.cu_seqlens_q[1])
    assert_parity(out[:n0], lse[:n0], ro[:n0], rl[:n0], torch.bfloat16, "good request")
    assert torch.isnan(out[n0:].float()).all() and torch.isnan(lse[n0:]).all()


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_small_varlen_fp16(gpu, D, causal):
    lens = [1, 17, 128, 129, 300, 64, 255]
    case = workloads.make_prefill(B=len(lens), Hq=8, Hkv=2, D=D, lens_q=lens, dtype=torch.float16,
                                  seed=340 + D, causal=causal)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.float16, f"fp16 varlen D{D} causal={causal}")


@pytest.mark.parametrize("D", [128, 256])
def test_small_paged_fp16(gpu, D):
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=D, page_size=16, chunk=70, cached=200,
                                        shared_prefix=64, dtype=torch.float16, seed=350 + D)
    out, lse = _paged(case, gpu)
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    assert_parity(out, lse, ro, rl, torch.float16, f"fp16 paged D{D}")


def test_ragged_config_fp16_sampled(gpu):
    """The ragged causal prefill workload (B 8, L in [1024, 4096], Hq 64, Hkv 8, D 128) in fp16."""
    case = workloads.make_prefill(B=8, Hq=64, Hkv=8, D=128, len_range=(1024, 4096), dtype=torch.float16,
                                  seed=3, causal=True)
    out, lse = _varlen(case, gpu)
    rows = _sample_rows(case.cu_seqlens_q, 64, 33)
    ro, rl = _ref(case, rows=rows)
    assert_parity(out, lse, ro, rl, torch.float16, "fp16 ragged (sampled rows)", rows=rows)


def _repage16(case, kp, vp):
    """The same NHD pools seen as 16-token pages (zero copy) and the page table."""
    m = case.page_size // 16
    j = torch.arange(case.page_table.shape[1] * m)
    t = case.page_table.long()
    return (kp.reshape(kp.shape[0] * m, 16, *kp.shape[2:]), vp.reshape(vp.shape[0] * m, 16, *vp.shape[2:]),
            (t[:, j // m] * m + j % m).to(torch.int32))


@pytest.mark.parametrize("P", [32, 64, 128, 256])
@pytest.mark.parametrize("D", [128, 256])
def test_paged_larger_pages(gpu, P, D):
    """Pages of 32 to 256 tokens: parity with the oracle (causal, and with a
    sliding window that skips whole key tiles), bit-for-bit equality with the
    same cache seen as 16-token pages and with the HND layout, and the
    shared-prefix cascade."""
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=D, page_size=P, chunk=90, cached=422,
                                        shared_prefix=256, dtype=torch.bfloat16, seed=980 + P + D)
    kp, vp = case.pools(gpu)
    kh, vh = case.pools(gpu, layout="HND")
    kp16, vp16, t16 = _repage16(case, kp, vp)
    q, cq, lens = case.q.to(gpu), case.cu_seqlens_q.to(gpu), case.kv_lens.to(gpu)
    t = case.page_table.to(gpu)
    for window in (-1, 77):
        out, lse = A.prefill_paged(q, cq, kp, vp, t, lens, case.max_seqlen_q, case.max_kv_len,
                                   causal=True, scale=case.scale, window_left=window)
        o16, l16 = A.prefill_paged(q, cq, kp16, vp16, t16.to(gpu), lens, case.max_seqlen_q,
                                   case.max_kv_len, causal=True, scale=case.scale, window_left=window)
        oh, lh = A.prefill_paged(q, cq, kh, vh, t, lens, case.max_seqlen_q, case.max_kv_len,
                                 causal=True, scale=case.scale, kv_layout="HND", window_left=window)
        torch.cuda.synchronize()
        ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                          case.page_table, case.kv_lens, True, case.scale,
                                          window_left=window)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"page {P} D{D} window {window}")
        assert torch.equal(out, o16) and torch.equal(lse, l16)
        assert torch.equal(out, oh) and torch.equal(lse, lh)
    out, lse = A.prefill_paged_cascade(q, cq, kp, vp, t, lens, case.max_seqlen_q, case.max_kv_len, 256,
                                       causal=True, scale=case.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"page {P} D{D} cascade")


@pytest.mark.parametrize("P", [32, 64, 128, 256])
@pytest.mark.parametrize("D", [128, 256])
def test_paged_larger_pages_ragged(gpu, P, D):
    """Pages of 32 to 256 tokens with per-request lengths that are multiples of
    neither 16 nor the page size (partial last pages and partial 16-token
    blocks, chunks of 1 to 130 queries): parity with the oracle in both page
    layouts, with and without a sliding window, and through the shared-prefix
    cascade in both layouts."""
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=4, Hq=4, Hkv=2, D=D, page_size=P, chunk=[90, 17, 1, 130],
                                        cached=[601, 333, 259, 700], shared_prefix=256,
                                        dtype=torch.bfloat16, seed=1000 + P + D, spare_pages=2)
    assert all(int(L) % 16 for L in case.kv_lens)
    q, cq, lens = case.q.to(gpu), case.cu_seqlens_q.to(gpu), case.kv_lens.to(gpu)
    t = case.page_table.to(gpu)
    for layout in ("NHD", "HND"):
        kp, vp = case.pools(gpu, layout=layout)
        for window in (-1, 100):
            out, lse = A.prefill_paged(q, cq, kp, vp, t, lens, case.max_seqlen_q, case.max_kv_len,
                                       causal=True, scale=case.scale, kv_layout=layout,
                                       window_left=window)
            torch.cuda.synchronize()
            ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                              case.page_table, case.kv_lens, True, case.scale,
                                              window_left=window)
            assert_parity(out, lse, ro, rl, torch.bfloat16, f"ragged page {P} D{D} {layout} w{window}")
        out, lse = A.prefill_paged_cascade(q, cq, kp, vp, t, lens, case.max_seqlen_q, case.max_kv_len,
                                           256, causal=True, scale=case.scale, kv_layout=layout)
        torch.cuda.synchronize()
        ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                          case.page_table, case.kv_lens, True, case.scale)
        assert_parity(out, lse, ro, rl, torch.bfloat16, f"ragged page {P} D{D} {layout} cascade")
        del kp, vp


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_paged_bad_page_larger_pages(gpu, layout):
    """64-token pages: a table entry outside the pool (a page every row of that
    request sees) makes that request's rows NaN; the other requests match the
    oracle."""
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=3, Hq=4, Hkv=2, D=128, page_size=64, chunk=[40, 33, 70],
                                        cached=[100, 150, 90], shared_prefix=0,
                                        dtype=torch.bfloat16, seed=330, spare_pages=1)
    table = case.page_table.clone()
    table[1, 1] = case.num_pages + 5           # tokens 64..127 of request 1
    kp, vp = case.pools(gpu, layout=layout)
    out, lse = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp, table.to(gpu),
                               case.kv_lens.to(gpu), case.max_seqlen_q, case.max_kv_len, causal=True,
                               scale=case.scale, kv_layout=layout)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    c = [int(x) for x in case.cu_seqlens_q]
    good = torch.cat([torch.arange(c[0], c[1]), torch.arange(c[2], c[3])])
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"good requests ({layout})", rows=good)
    assert torch.isnan(out[c[1]:c[2]].float()).all() and torch.isnan(lse[c[1]:c[2]]).all()


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_no_keys_at_all(gpu, D, causal):
    """A ragged batch whose sequences all have zero keys (total_k 0: k and v are
    empty tensors, NULL pointers at the boundary): every row gets out 0 and
    lse -inf."""
    import attention_qk_online_amd as A
    case = workloads.make_prefill(B=3, Hq=8, Hkv=2, D=D, lens_q=[300, 1, 129], lens_k=[0, 0, 0],
                                  dtype=torch.bfloat16, seed=330, causal=causal)
    assert case.k.numel() == 0
    out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu), 300, 1,
                                causal=causal, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.float().cpu(), torch.zeros(out.shape))
    assert torch.isneginf(lse.cpu()).all()


def test_keys_above_max_seqlen_k_are_nan(gpu):
    """A sequence with more keys than the host bound max_seqlen_k: its rows are NaN;
    the other sequence is unaffected."""
    import attention_qk_online_amd as A
    case = workloads.make_prefill(B=2, Hq=4, Hkv=2, D=128, lens_q=[100, 60], lens_k=[200, 500],
                                  dtype=torch.bfloat16, seed=331, causal=True)
    out, lse = A.prefill_varlen(case.q.to(gpu), case.k.to(gpu), case.v.to(gpu),
                                case.cu_seqlens_q.to(gpu), case.cu_seqlens_k.to(gpu), 100, 300,
                                causal=True, scale=case.scale)
    torch.cuda.synchronize()
    ro, rl = _ref(case)
    assert_parity(out[:100], lse[:100], ro[:100], rl[:100], torch.bfloat16, "good sequence")
    assert torch.isnan(out[100:].float()).all() and torch.isnan(lse[100:]).all()


@pytest.mark.parametrize("D", [128, 256])
def test_paged_kv_len_above_max_kv_len_is_nan(gpu, D):
    """A request whose kv_len exceeds the host bound max_kv_len (but fits its
    page-table row): its rows are NaN and nothing of it is read; the other
    request is unaffected."""
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=2, Hq=4, Hkv=2, D=D, page_size=16, chunk=[40, 30],
                                        cached=[100, 300], dtype=torch.bfloat16, seed=332)
    kp, vp = case.pools(gpu)
    out, lse = A.prefill_paged(case.q.to(gpu), case.cu_seqlens_q.to(gpu), kp, vp,
                               case.page_table.to(gpu), case.kv_lens.to(gpu), 40, 140,
                               causal=True, scale=case.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    n0 = int(case.cu_seqlens_q[1])
    assert_parity(out[:n0], lse[:n0], ro[:n0], rl[:n0], torch.bfloat16, "good request")
    assert torch.isnan(out[n0:].float()).all() and torch.isnan(lse[n0:]).all()


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_paged_empty_cache(gpu, layout):
    """max_kv_len 0 with an empty pool and page table (NULL pointers at the
    boundary): rows with no key get out 0 and lse -inf; a request claiming keys
    (kv_len above max_kv_len) gets NaN and reads nothing."""
    import attention_qk_online_amd as A
    q = torch.randn(50, 8, 128, device=gpu).to(torch.bfloat16)
    cu = torch.tensor([0, 20, 50], dtype=torch.int32, device=gpu)
    lens = torch.tensor([0, 7], dtype=torch.int32, device=gpu)
    pool = torch.empty((0, 16, 2, 128) if layout == "NHD" else (0, 2, 16, 128), dtype=torch.bfloat16,
                       device=gpu)
    table = torch.empty((2, 0), dtype=torch.int32, device=gpu)
    out, lse = A.prefill_paged(q, cu, pool, pool, table, lens, 30, 0, causal=False, scale=0.1,
                               kv_layout=layout)
    torch.cuda.synchronize()
    out, lse = out.float().cpu(), lse.cpu()
    assert torch.equal(out[:20], torch.zeros(20, 8, 128)) and torch.isneginf(lse[:20]).all()
    assert torch.isnan(out[20:]).all() and torch.isnan(lse[20:]).all()


@pytest.mark.parametrize("D,layout", [(128, "NHD"), (256, "HND")])
def test_paged_pages_past_4gib(gpu, D, layout):
    """The pages of a chunked prefill placed at the top of a pool of more than
    4 GiB per tensor (byte offsets above 2^32): same result as the compact
    pool, bit for bit, and parity with the oracle."""
    import attention_qk_online_amd as A
    case = workloads.make_paged_prefill(B=3, Hq=8, Hkv=8, D=D, page_size=16, chunk=[100, 37, 64],
                                        cached=[300, 500, 129], dtype=torch.bfloat16, seed=340)
    page_bytes = 16 * 8 * D * 2
    big = (5 << 30) // page_bytes + 64                # > 5 GiB per pool
    print(f"pool of {big} pages ({big * page_bytes / 2**30:.1f} GiB each)", flush=True)
    kp, vp = case.pools(gpu, layout)
    # old id i -> big - 1 - 3 i: scattered over the top of the big pool
    remap = torch.arange(case.num_pages, device=gpu) * -3 + (big - 1)
    shape = (big,) + tuple(kp.shape[1:])
    kb = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=gpu)
    vb = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=gpu)
    kb.index_copy_(0, remap, kp)
    vb.index_copy_(0, remap, vp)
    table_big = remap[case.page_table.to(gpu).long()].to(torch.int32)
    args = (case.q.to(gpu), case.cu_seqlens_q.to(gpu))
    tail = (case.kv_lens.to(gpu), case.max_seqlen_q, case.max_kv_len)
    o_small, l_small = A.prefill_paged(*args, kp, vp, case.page_table.to(gpu), *tail, causal=True,
                                       scale=case.scale, kv_layout=layout)
    o_big, l_big = A.prefill_paged(*args, kb, vb, table_big, *tail, causal=True, scale=case.scale,
                                   kv_layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(o_small, o_big) and torch.equal(l_small, l_big)
    del kb, vb
    ro, rl = oracle.ref_prefill_paged(case.q, case.cu_seqlens_q, case.pool_k, case.pool_v,
                                      case.page_table, case.kv_lens, True, case.scale)
    assert_parity(o_big, l_big, ro, rl, torch.bfloat16, f"D{D} {layout} pool of {big} pages")


def test_varlen_keys_past_4gib(gpu):
    """A ragged batch whose second sequence starts more than 4 GiB into k and v
    (a first sequence of 2^20 keys, Hkv 8, head_dim 256): the second
    sequence's rows match the oracle on its own keys."""
    import attention_qk_online_amd as A
    Hq, Hkv, D, L0 = 8, 8, 256, 1 << 20
    lens_q, lens_k = [1, 200], [L0, 333]
    Tk = sum(lens_k)
    print(f"k, v of {Tk * Hkv * D * 2 / 2**30:.2f} GiB each", flush=True)
    g = torch.Generator(device=gpu).manual_seed(341)
    k = torch.randn(Tk, Hkv, D, generator=g, device=gpu).to(torch.bfloat16)
    v = torch.randn(Tk, Hkv, D, generator=g, device=gpu).to(torch.bfloat16)
    q = torch.randn(sum(lens_q), Hq, D, generator=g, device=gpu).to(torch.bfloat16)
    cu_q = torch.tensor([0, 1, 201], dtype=torch.int32, device=gpu)
    cu_k = torch.tensor([0, L0, Tk], dtype=torch.int32, device=gpu)
    scale = 1.0 / 16
    out, lse = A.prefill_varlen(q, k, v, cu_q, cu_k, 200, L0, causal=True, scale=scale)
    torch.cuda.synchronize()
    k1, v1 = k[L0:].cpu(), v[L0:].cpu()
    q1 = q[1:].cpu()
    del k, v
    ro, rl = oracle.ref_prefill_varlen(q1, k1, v1, torch.tensor([0, 200], dtype=torch.int32),
                                       torch.tensor([0, 333], dtype=torch.int32), True, scale)
    assert_parity(out[1:], lse[1:], ro, rl, torch.bfloat16, "sequence past 4 GiB")


@pytest.mark.parametrize("D", [128, 256])
def test_more_than_eight_kv_heads(gpu, D):
    """Twelve KV heads, two query heads each (the work order walks KV heads,
    sequences, tiles and the heads of a group)."""
    case = workloads.make_prefill(B=2, Hq=24, Hkv=12, D=D, lens_q=[150, 260], dtype=torch.bfloat16,
                                  seed=260, causal=True)
    out, lse = _varlen(case, gpu)
    ro, rl = _ref(case)
    assert_parity(out, lse, ro, rl, torch.bfloat16, f"Hkv 12 D{D}")

"""Pins for the CPU oracle (no GPU).

The oracle is trusted only because these checks tie it to something other
than itself: hand-derived closed forms (``tests/golden``), brute force with
explicit loops, PyTorch's own scaled_dot_product_attention in float64,
special cases with textbook answers, and invariants of the mathematics.
``test_planted_mistakes_are_caught`` edits the oracle's source on the CPU
(dropped scale, wrong head grouping, flipped mask offset, ...) and checks that
at least one pin fails for every edit.
"""
import json
import math
import os
import types

import pytest
import torch

import oracle
import oracle.ref as REF
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


def _ev(x):
    env = {"log": math.log, "sqrt": math.sqrt, "nan": math.nan, "inf": math.inf,
           "exp": math.exp, "cos": math.cos, "sin": math.sin}
    if isinstance(x, str) and x.strip() == "-0":
        return -0.0
    return float(eval(x, {"__builtins__": {}}, env)) if isinstance(x, str) else float(x)


def _tensor(nested):
    if isinstance(nested, list):
        return torch.stack([_tensor(x) for x in nested]) if isinstance(nested[0], list) \
            else torch.tensor([_ev(x) for x in nested], dtype=F64)
    return torch.tensor(_ev(nested), dtype=F64)


def _close(a, b, tol=1e-12):
    a, b = a.to(F64), b.to(F64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both_inf = torch.isinf(a) & torch.isinf(b) & (torch.sign(a) == torch.sign(b))
    d = torch.where(both_inf, torch.zeros_like(a), (a - b).abs())
    assert not torch.isnan(d).any(), "NaN mismatch"
    assert float(d.max()) <= tol, float(d.max())


# ---------------------------------------------------------------------------
# Pins, each a function of an oracle module R so planted mistakes can be tested
# ---------------------------------------------------------------------------
def pin_golden(R):
    for fn in sorted(os.listdir(GOLDEN)):
        if not fn.endswith(".json"):
            continue
        g = json.load(open(os.path.join(GOLDEN, fn)))
        if g["kind"] == "prefill":
            o, l = R.ref_prefill_varlen(_tensor(g["q"]), _tensor(g["k"]), _tensor(g["v"]),
                                        g["cu_seqlens_q"], g["cu_seqlens_k"], g["causal"],
                                        _ev(g["scale"]), window_left=g.get("window_left", -1))
        elif g["kind"] == "fp8_e4m3":
            got = R.fp8_e4m3_to_float(torch.tensor([b for b, _ in g["values"]], dtype=torch.uint8))
            want = torch.tensor([_ev(v) for _, v in g["values"]], dtype=F64)
            assert torch.equal(torch.isnan(got), torch.isnan(want)), fn
            ok = ~torch.isnan(want)
            assert torch.equal(got[ok], want[ok]), fn
            assert torch.equal(torch.signbit(got[ok]), torch.signbit(want[ok])), fn
            continue
        elif g["kind"] == "decode_fp8":
            o, l = R.ref_decode_paged_fp8(_tensor(g["q"]),
                                          torch.tensor(g["k_pages"], dtype=torch.uint8),
                                          torch.tensor(g["v_pages"], dtype=torch.uint8),
                                          _ev(g["k_scale"]), _ev(g["v_scale"]),
                                          torch.tensor(g["page_table"]), torch.tensor(g["kv_lens"]),
                                          _ev(g["scale"]))
        elif g["kind"] == "decode_rope":
            o, l = R.ref_decode_paged(_tensor(g["q"]), _tensor(g["k_pages"]), _tensor(g["v_pages"]),
                                      torch.tensor(g["page_table"]), torch.tensor(g["kv_lens"]),
                                      _ev(g["scale"]),
                                      rope=(_ev(g["rope_theta"]), _ev(g["rope_scale"])))
        elif g["kind"] == "decode":
            o, l = R.ref_decode_paged(_tensor(g["q"]), _tensor(g["k_pages"]), _tensor(g["v_pages"]),
                                      torch.tensor(g["page_table"]), torch.tensor(g["kv_lens"]),
                                      _ev(g["scale"]))
        else:
            states = [(_tensor(s["o"]), _tensor(s["lse"])) for s in g["states"]]
            o, l = R.merge_states(states)
        _close(o, _tensor(g["out"]), 1e-13)
        _close(l, _tensor(g["lse"]), 1e-13)


def _brute(q, k, v, cq, ck, causal, scale):
    """Explicit loops, exp without max subtraction (fine for these small logits)."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = torch.zeros((Tq, Hq, v.shape[2]), dtype=F64)
    lse = torch.zeros((Tq, Hq), dtype=F64)
    for b in range(len(cq) - 1):
        Lq, Lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for i in range(Lq):
            for h in range(Hq):
                g = h // G
                ws, tot = [], 0.0
                for j in range(Lk):
                    if causal and j > i + (Lk - Lq):
                        continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[cq[b] + i, h, d]) * float(k[ck[b] + j, g, d])
                    w = math.exp(s * scale)
                    ws.append((j, w))
                    tot += w
                if not ws:
                    lse[cq[b] + i, h] = -math.inf
                    continue
                lse[cq[b] + i, h] = math.log(tot)
                for j, w in ws:
                    for d in range(v.shape[2]):
                        out[cq[b] + i, h, d] += (w / tot) * float(v[ck[b] + j, g, d])
    return out, lse


def pin_brute_force(R):
    for causal in (False, True):
        c = workloads.make_prefill(B=3, Hq=4, Hkv=2, D=5, lens_q=[3, 1, 4], lens_k=[3, 4, 6],
                                   dtype=F64, seed=11, causal=causal)
        cq, ck = c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist()
        o, l = R.ref_prefill_varlen(c.q, c.k, c.v, cq, ck, causal, c.scale)
        ob, lb = _brute(c.q, c.k, c.v, cq, ck, causal, c.scale)
        _close(o, ob, 1e-12)
        _close(l, lb, 1e-12)


def pin_sdpa_library(R):
    """torch's own SDPA (float64, CPU) for Lq = Lk causal and Lq != Lk non-causal."""
    import torch.nn.functional as F
    for causal, lq, lk in ((True, 6, 6), (False, 3, 7)):
        c = workloads.make_prefill(B=1, Hq=6, Hkv=3, D=8, lens_q=[lq], lens_k=[lk], dtype=F64,
                                   seed=12, causal=causal, scale=0.37)
        o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, causal, c.scale)
        G = c.Hq // c.Hkv
        qh = c.q.permute(1, 0, 2).unsqueeze(0)
        kh = c.k.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
        vh = c.v.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
        ref = F.scaled_dot_product_attention(qh, kh, vh, is_causal=causal, scale=c.scale)
        _close(o, ref[0].permute(1, 0, 2), 1e-12)


def pin_single_key(R):
    c = workloads.make_decode(B=2, Hq=4, Hkv=2, D=8, page_size=4, kv_lens=[1, 1], dtype=F64, seed=13)
    kp, vp = c.pools()
    o, l = R.ref_decode_paged(c.q, kp, vp, c.page_table, c.kv_lens, c.scale)
    for b in range(2):
        for h in range(4):
            g = h // 2
            _close(o[b, h], c.v_tok[b, g], 0.0)
            _close(l[b, h], c.scale * (c.q[b, h] @ c.k_tok[b, g]), 1e-13)


def pin_constant_v(R):
    c = workloads.make_prefill(B=2, Hq=2, Hkv=1, D=4, lens_q=[5, 3], lens_k=[5, 6], dtype=F64,
                               seed=14, causal=True)
    row = torch.tensor([0.5, -1.25, 2.0, 3.0], dtype=F64)
    v = row.expand_as(c.v).clone()
    o, l = R.ref_prefill_varlen(c.q, c.k, v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale)
    _close(o, row.expand_as(o), 1e-13)


def pin_scale_zero_mean(R):
    """scale = 0: every visible key weighs the same, so out = mean of visible V rows
    and lse = ln(number visible); checks bottom-right visibility counts too."""
    lq, lk = [4, 2], [4, 5]
    c = workloads.make_prefill(B=2, Hq=2, Hkv=2, D=3, lens_q=lq, lens_k=lk, dtype=F64, seed=15,
                               causal=True, scale=0.0)
    o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, 0.0)
    cq, ck = c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist()
    for b in range(2):
        for i in range(lq[b]):
            n = i + (lk[b] - lq[b]) + 1
            for h in range(2):
                _close(o[cq[b] + i, h], c.v[ck[b]:ck[b] + n, h].mean(0), 1e-13)
                _close(l[cq[b] + i, h], torch.tensor(math.log(n), dtype=F64), 1e-13)


def pin_shift_invariance(R):
    """k_j <- k_j + w for every j: out unchanged, lse shifted by scale*q.w; with a
    large shift this also exercises overflow safety."""
    c = workloads.make_decode(B=2, Hq=2, Hkv=1, D=6, page_size=4, kv_lens=[7, 3], dtype=F64, seed=16,
                              poison=False)
    kp, vp = c.pools()
    o, l = R.ref_decode_paged(c.q, kp, vp, c.page_table, c.kv_lens, c.scale)
    w = torch.zeros(6, dtype=F64)
    w[0] = 1000.0 / max(1e-9, abs(float(c.q[0, 0, 0])) * c.scale)
    o2, l2 = R.ref_decode_paged(c.q, kp + w, vp, c.page_table, c.kv_lens, c.scale)
    assert torch.isfinite(o2).all() and torch.isfinite(l2).all()
    _close(o2, o, 1e-9)
    _close(l2, l + c.scale * (c.q @ w), 1e-9)


def pin_paging(R):
    """Physical page order is irrelevant; paged == contiguous; aliased pages ==
    de-aliased copies; poisoned slots never reach the output."""
    c = workloads.make_decode(B=3, Hq=4, Hkv=2, D=8, page_size=4, kv_lens=[9, 4, 13], dtype=F64,
                              seed=17, num_pages=20)
    kp, vp = c.pools()
    o, l = R.ref_decode_paged(c.q, kp, vp, c.page_table, c.kv_lens, c.scale)
    assert torch.isfinite(o).all() and torch.isfinite(l).all()
    # permute physical pages, remap the table
    perm = torch.randperm(c.num_pages, generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(c.num_pages)
    o2, l2 = R.ref_decode_paged(c.q, kp[perm], vp[perm], inv[c.page_table.long()], c.kv_lens, c.scale)
    _close(o2, o, 1e-13)
    _close(l2, l, 1e-13)
    # contiguous: the same request as a single-query non-causal prefill
    cu = torch.tensor([0] + torch.cumsum(c.kv_lens.long(), 0).tolist())
    o3, l3 = R.ref_prefill_varlen(c.q, c.k_tok, c.v_tok, torch.arange(4), cu, False, c.scale)
    _close(o3, o, 1e-13)
    _close(l3, l, 1e-13)
    # aliasing: two requests share their first page; de-aliased copy gives the same
    shared = workloads.make_decode(B=2, Hq=2, Hkv=1, D=4, page_size=2, kv_lens=[4, 4], dtype=F64,
                                   seed=18, poison=False)
    kp, vp = shared.pools()
    table = shared.page_table.clone()
    table[1, 0] = table[0, 0]
    oa, la = R.ref_decode_paged(shared.q, kp, vp, table, shared.kv_lens, 0.7)
    kd, vd = kp.clone(), vp.clone()
    kd[table[1, 1]] = kp[table[1, 1]]
    kd = torch.cat([kd, kp[table[0, 0]].unsqueeze(0)])
    vd = torch.cat([vd, vp[table[0, 0]].unsqueeze(0)])
    t2 = table.clone()
    t2[1, 0] = kd.shape[0] - 1
    od, ld = R.ref_decode_paged(shared.q, kd, vd, t2, shared.kv_lens, 0.7)
    _close(oa, od, 0.0)
    _close(la, ld, 0.0)


def pin_gqa_equals_repeated_mha(R):
    c = workloads.make_prefill(B=2, Hq=6, Hkv=2, D=4, lens_q=[4, 5], dtype=F64, seed=19, causal=True)
    o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale)
    k3, v3 = c.k.repeat_interleave(3, dim=1), c.v.repeat_interleave(3, dim=1)
    o2, l2 = R.ref_prefill_varlen(c.q, k3, v3, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale)
    _close(o, o2, 0.0)
    _close(l, l2, 0.0)


def pin_causal_rows(R):
    """Row 0 is v[0]; row i equals non-causal attention over keys 0..i; the last
    causal row equals a decode of that query over the whole KV."""
    c = workloads.make_prefill(B=1, Hq=2, Hkv=1, D=6, lens_q=[7], dtype=F64, seed=20, causal=True)
    o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale)
    _close(o[0], c.v[0].expand(2, 6), 1e-13)
    for i in range(7):
        oi, li = R.ref_prefill_varlen(c.q[i:i + 1], c.k[:i + 1], c.v[:i + 1], [0, 1], [0, i + 1],
                                      False, c.scale)
        _close(o[i], oi[0], 1e-13)
        _close(l[i], li[0], 1e-13)
    kp = c.k.reshape(7, 1, 1, 6)[:, 0].unsqueeze(1)  # 7 pages of one slot
    vp = c.v.reshape(7, 1, 1, 6)[:, 0].unsqueeze(1)
    od, ld = R.ref_decode_paged(c.q[6:7], kp, vp, torch.arange(7).unsqueeze(0), torch.tensor([7]),
                                c.scale)
    _close(o[6], od[0], 1e-13)
    _close(l[6], ld[0], 1e-13)


def pin_chunked_equals_full(R):
    """Chunk queries over a paged cache equal the matching rows of a full causal
    prefill over the whole sequence (bottom-right alignment)."""
    c = workloads.make_paged_prefill(B=2, Hq=2, Hkv=1, D=4, page_size=2, chunk=3, cached=5,
                                     shared_prefix=2, dtype=F64, seed=21)
    o, l = R.ref_prefill_paged(c.q, c.cu_seqlens_q, c.pool_k, c.pool_v, c.page_table, c.kv_lens,
                               True, c.scale)
    for b in range(2):
        L = int(c.kv_lens[b])
        kf = R.gather_pages(c.pool_k, c.page_table[b], L)
        vf = R.gather_pages(c.pool_v, c.page_table[b], L)
        qf = torch.zeros((L, 2, 4), dtype=F64)
        qf[L - 3:] = c.q[3 * b:3 * b + 3]
        of, lf = R.ref_prefill_varlen(qf, kf, vf, [0, L], [0, L], True, c.scale)
        _close(o[3 * b:3 * b + 3], of[L - 3:], 1e-13)
        _close(l[3 * b:3 * b + 3], lf[L - 3:], 1e-13)


def pin_merge_partition(R):
    """Attention over disjoint key blocks, merged by LSE, equals the unsplit result."""
    c = workloads.make_prefill(B=1, Hq=1, Hkv=1, D=5, lens_q=[3], lens_k=[11], dtype=F64, seed=22,
                               causal=False)
    full = R.ref_prefill_varlen(c.q, c.k, c.v, [0, 3], [0, 11], False, c.scale)
    cuts = [0, 2, 3, 9, 11]
    parts = [R.ref_prefill_varlen(c.q, c.k[a:b], c.v[a:b], [0, 3], [0, b - a], False, c.scale)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, l = R.merge_states(parts)
    _close(o, full[0], 1e-13)
    _close(l, full[1], 1e-13)
    # an empty block carries no weight
    o2, l2 = R.merge_states(parts + [(torch.zeros_like(full[0]), torch.full_like(full[1], -math.inf))])
    _close(o2, full[0], 1e-13)


def pin_empty_rows(R):
    """No visible key: out 0, lse -inf (decode kv_len 0; Lq > Lk bottom-right)."""
    c = workloads.make_decode(B=2, Hq=2, Hkv=1, D=4, page_size=2, kv_lens=[0, 3], dtype=F64, seed=23)
    kp, vp = c.pools()
    o, l = R.ref_decode_paged(c.q, kp, vp, c.page_table, c.kv_lens, c.scale)
    assert torch.equal(o[0], torch.zeros_like(o[0]))
    assert torch.isneginf(l[0]).all() and torch.isfinite(l[1]).all()
    p = workloads.make_prefill(B=1, Hq=1, Hkv=1, D=4, lens_q=[5], lens_k=[2], dtype=F64, seed=24)
    o, l = R.ref_prefill_varlen(p.q, p.k, p.v, [0, 5], [0, 2], True, p.scale)
    assert torch.equal(o[:3], torch.zeros_like(o[:3])) and torch.isneginf(l[:3]).all()
    _close(o[3, 0], p.v[0, 0], 0.0)


def pin_rows_subset(R):
    c = workloads.make_prefill(B=2, Hq=2, Hkv=1, D=4, lens_q=[6, 5], dtype=F64, seed=25, causal=True)
    o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale)
    rows = torch.tensor([0, 4, 6, 10])
    o2, l2 = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale,
                                  rows=rows)
    _close(o2[rows], o[rows], 0.0)
    assert torch.isnan(o2[1]).all()


def pin_fp8_decoder_library(R):
    """Every byte decodes as torch's float8_e4m3fn reads it."""
    b = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    got = R.fp8_e4m3_to_float(b)
    want = b.view(torch.float8_e4m3fn).to(F64)
    assert torch.equal(torch.isnan(got), torch.isnan(want))
    ok = ~torch.isnan(want)
    assert torch.equal(got[ok], want[ok])


def pin_fp8_decode_equals_dequantised(R):
    """Decode over E4M3 bytes equals plain decode over the same cache decoded by
    torch and scaled (k_scale on K, v_scale on V), including subnormal bytes."""
    c = workloads.make_decode(B=3, Hq=4, Hkv=2, D=8, page_size=4, kv_lens=[5, 9, 1], dtype=F64,
                              seed=30)
    kb, vb, ks, vs = c.fp8_pools()
    kb = kb.clone()
    kb[c.page_table[1, 0], 1, 0, :4] = torch.tensor([1, 3, 0x81, 0x87], dtype=torch.uint8)
    kf = kb.view(torch.float8_e4m3fn).to(F64) * ks
    vf = vb.view(torch.float8_e4m3fn).to(F64) * vs
    o, l = R.ref_decode_paged_fp8(c.q, kb, vb, ks, vs, c.page_table, c.kv_lens, c.scale)
    o2, l2 = R.ref_decode_paged(c.q, kf, vf, c.page_table, c.kv_lens, c.scale)
    _close(o, o2, 1e-13)
    _close(l, l2, 1e-13)
    # the scales are where they belong: k_scale * scale is one factor, v_scale is linear
    o3, l3 = R.ref_decode_paged_fp8(c.q, kb, vb, 2 * ks, 3 * vs, c.page_table, c.kv_lens,
                                    c.scale / 2)
    _close(o3, 3 * o, 1e-12)
    _close(l3, l, 1e-12)
    # with a sliding window: the windowed decode of the dequantised cache
    for left in (0, 3):
        o4, l4 = R.ref_decode_paged_fp8(c.q, kb, vb, ks, vs, c.page_table, c.kv_lens, c.scale,
                                        window_left=left)
        o5, l5 = R.ref_decode_paged(c.q, kf, vf, c.page_table, c.kv_lens, c.scale, window_left=left)
        _close(o4, o5, 1e-13)
        _close(l4, l5, 1e-13)


def pin_window_brute_force(R):
    """Sliding window against explicit loops over (i, j, d), causal and not,
    with Lq < Lk (bottom-right alignment), and its limits: a window as long
    as the keys is no window; window 0 with causal leaves each row its own key."""
    c = workloads.make_prefill(B=2, Hq=2, Hkv=1, D=3, lens_q=[4, 3], lens_k=[7, 3], dtype=F64,
                               seed=40, causal=True)
    for causal in (True, False):
        for left in (0, 2, 5):
            o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, causal,
                                        c.scale, window_left=left)
            cq, ck = c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist()
            for b in range(2):
                Lq, Lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
                for i in range(Lq):
                    for h in range(2):
                        js = [j for j in range(Lk) if j >= i + Lk - Lq - left and
                              (not causal or j <= i + Lk - Lq)]
                        sc = [c.scale * sum(float(c.q[cq[b] + i, h, d]) * float(c.k[ck[b] + j, 0, d])
                                            for d in range(3)) for j in js]
                        mx = max(sc)
                        w = [math.exp(x - mx) for x in sc]
                        z = sum(w)
                        for d in range(3):
                            want = sum(wj * float(c.v[ck[b] + j, 0, d]) for wj, j in zip(w, js)) / z
                            assert abs(float(o[cq[b] + i, h, d]) - want) < 1e-12
                        assert abs(float(l[cq[b] + i, h]) - (mx + math.log(z))) < 1e-12
    full = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale)
    wide = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale,
                                window_left=7)
    _close(full[0], wide[0], 0.0)
    o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, True, c.scale,
                                window_left=0)
    _close(o[3, 0], c.v[6, 0], 0.0)       # last row of sequence 0 sits on key 6


def pin_right_window_brute_force(R):
    """Right-side window (window_size's second half) against explicit loops
    over (i, j, d), alone and with a left window, with Lq < Lk and Lq > Lk
    (bottom-right alignment, empty rows); its limits: a right window of 0 is
    the causal mask, one as long as the keys is no bound, and the band
    (0, 0) leaves each row its own diagonal key."""
    c = workloads.make_prefill(B=3, Hq=2, Hkv=1, D=3, lens_q=[4, 3, 5], lens_k=[7, 3, 2], dtype=F64,
                               seed=41, causal=False)
    cq, ck = c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist()
    for left, right in ((-1, 0), (-1, 1), (-1, 3), (1, 1), (2, 0), (0, 2)):
        o, l = R.ref_prefill_varlen(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, False,
                                    c.scale, window_left=left, window_right=right)
        for b in range(3):
            Lq, Lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
            for i in range(Lq):
                for h in range(2):
                    js = [j for j in range(Lk) if j <= i + Lk - Lq + right and
                          (left < 0 or j >= i + Lk - Lq - left)]
                    if not js:
                        assert float(l[cq[b] + i, h]) == -math.inf
                        assert all(float(o[cq[b] + i, h, d]) == 0.0 for d in range(3))
                        continue
                    sc = [c.scale * sum(float(c.q[cq[b] + i, h, d]) * float(c.k[ck[b] + j, 0, d])
                                        for d in range(3)) for j in js]
                    mx = max(sc)
                    w = [math.exp(x - mx) for x in sc]
                    z = sum(w)
                    for d in range(3):
                        want = sum(wj * float(c.v[ck[b] + j, 0, d]) for wj, j in zip(w, js)) / z
                        assert abs(float(o[cq[b] + i, h, d]) - want) < 1e-12
                    assert abs(float(l[cq[b] + i, h]) - (mx + math.log(z))) < 1e-12
    args = (c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k)
    causal = R.ref_prefill_varlen(*args, True, c.scale)
    right0 = R.ref_prefill_varlen(*args, False, c.scale, window_right=0)
    _close(causal[0], right0[0], 0.0)
    _close(causal[1], right0[1], 0.0)
    plain = R.ref_prefill_varlen(*args, False, c.scale)
    wide = R.ref_prefill_varlen(*args, False, c.scale, window_right=7)
    _close(plain[0], wide[0], 0.0)
    # causal set: a right window adds nothing
    both = R.ref_prefill_varlen(*args, True, c.scale, window_right=2)
    _close(causal[0], both[0], 0.0)
    o, l = R.ref_prefill_varlen(*args, False, c.scale, window_left=0, window_right=0)
    _close(o[1, 0], c.v[4, 0], 0.0)        # row 1 of sequence 0 sits on key 4


def pin_decode_window(R):
    """Decode with a window is the last row of a causal windowed prefill over the
    same keys (one slices the keys, the other masks them), and a window of 0
    returns the last value row."""
    c = workloads.make_decode(B=3, Hq=4, Hkv=2, D=5, page_size=4, kv_lens=[9, 1, 6], dtype=F64,
                              seed=41)
    kp, vp = c.pools()
    for left in (0, 3, 20):
        o, l = R.ref_decode_paged(c.q, kp, vp, c.page_table, c.kv_lens, c.scale, window_left=left)
        for b in range(3):
            L = int(c.kv_lens[b])
            kf = R.gather_pages(kp, c.page_table[b], L)
            vf = R.gather_pages(vp, c.page_table[b], L)
            qf = torch.zeros((L, 4, 5), dtype=F64)
            qf[L - 1] = c.q[b]
            of, lf = R.ref_prefill_varlen(qf, kf, vf, [0, L], [0, L], True, c.scale,
                                          window_left=left)
            _close(o[b], of[L - 1], 1e-13)
            _close(l[b], lf[L - 1], 1e-13)
            if left == 0:
                _close(o[b, 0], vf[L - 1, 0], 0.0)


def pin_rope(R):
    """rope_rotate against complex multiplication (library complex128), its
    relative-position property, norm preservation and position 0; decode with
    rope equals plain decode on pre-rotated q and keys."""
    g = torch.Generator().manual_seed(42)
    x = torch.randn((3, 5, 8), generator=g, dtype=F64)
    pos = torch.tensor([0.0, 1.0, 7.0, 100.0, 4095.0], dtype=F64)
    theta, scale = 500.0, 2.0
    y = R.rope_rotate(x, pos, theta, scale)
    freq = theta ** (-2.0 * torch.arange(4, dtype=F64) / 8)
    z = torch.complex(x[..., :4], x[..., 4:]) * torch.polar(torch.ones(5, 4, dtype=F64),
                                                            pos.unsqueeze(1) / scale * freq)
    _close(y, torch.cat([z.real, z.imag], dim=-1), 1e-12)
    _close(y.norm(dim=-1), x.norm(dim=-1), 1e-12)
    _close(y[:, 0], x[:, 0], 0.0)
    q, k = x[0, :1], x[1, :1]
    for m, n, dl in ((3.0, 1.0, 10.0), (50.0, 70.0, -20.0)):
        a = (R.rope_rotate(q, torch.tensor([m]), theta) * R.rope_rotate(k, torch.tensor([n]), theta)).sum()
        b = (R.rope_rotate(q, torch.tensor([m + dl]), theta) *
             R.rope_rotate(k, torch.tensor([n + dl]), theta)).sum()
        assert abs(float(a - b)) < 1e-12
    c = workloads.make_decode(B=2, Hq=4, Hkv=2, D=8, page_size=4, kv_lens=[6, 3], dtype=F64, seed=43)
    kp, vp = c.pools()
    o, l = R.ref_decode_paged(c.q, kp, vp, c.page_table, c.kv_lens, c.scale, rope=(theta, scale))
    for b in range(2):
        L = int(c.kv_lens[b])
        kf = R.gather_pages(kp, c.page_table[b], L)
        vf = R.gather_pages(vp, c.page_table[b], L)
        zk = torch.complex(kf[..., :4], kf[..., 4:]) * torch.polar(
            torch.ones(L, 1, 4, dtype=F64), torch.arange(L, dtype=F64).view(L, 1, 1) / scale * freq)
        zq = torch.complex(c.q[b][..., :4], c.q[b][..., 4:]) * torch.polar(
            torch.ones(4, 4, dtype=F64), torch.full((4, 1), (L - 1) / scale, dtype=F64) * freq)
        kr = torch.cat([zk.real, zk.imag], dim=-1)
        qr = torch.cat([zq.real, zq.imag], dim=-1)
        for h in range(4):
            of, lf = R.softmax_attend(qr[h:h + 1], kr[:, h // 2], vf[:, h // 2], c.scale)
            _close(o[b, h], of[0], 1e-12)
            _close(l[b, h], lf[0], 1e-12)


PINS = [pin_golden, pin_brute_force, pin_sdpa_library, pin_single_key, pin_constant_v,
        pin_scale_zero_mean, pin_shift_invariance, pin_paging, pin_gqa_equals_repeated_mha,
        pin_causal_rows, pin_chunked_equals_full, pin_merge_partition, pin_empty_rows,
        pin_rows_subset, pin_fp8_decoder_library, pin_fp8_decode_equals_dequantised,
        pin_window_brute_force, pin_right_window_brute_force, pin_decode_window, pin_rope]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_holds(pin):
    pin(REF)


# Mistakes an implementer could plausibly make, planted in a copy of the oracle.
MUTANTS = {
    "dropped_scale": ("s = (q @ k.transpose(0, 1)) * scale", "s = (q @ k.transpose(0, 1))"),
    "gqa_modulo": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "mask_offset_sign": ("(rows.long().unsqueeze(1) + offset)", "(rows.long().unsqueeze(1) - offset)"),
    "top_left_causal": ("off = Lk - Lq", "off = 0"),
    "lse_without_max": ("lse = m + torch.log(", "lse = torch.log("),
    "page_slot_swapped": ("return pages[ids, t % P]", "return pages[t % P, ids]" ),
    "wrong_page_index": ("ids = table_row.long()[t // P]", "ids = table_row.long()[t % P]"),
    "pv_transposed": ("return p @ v, lse", "return (p @ v.flip(0)), lse"),
    "merge_linear_weights": ("w = torch.exp(lses - mx.unsqueeze(0))",
                             "w = torch.softmax(lses, dim=0) + 0 * mx"),
    "mask_strict": ("<= (rows.long().unsqueeze(1) + offset)", "< (rows.long().unsqueeze(1) + offset)"),
    "window_sign": ("(rows.long().unsqueeze(1) + offset - left)", "(rows.long().unsqueeze(1) - offset - left)"),
    "window_strict": (">= (rows.long().unsqueeze(1) + offset - left)", "> (rows.long().unsqueeze(1) + offset - left)"),
    "decode_window_off_by_one": ("return max(0, L - 1 - window_left) if", "return max(0, L - window_left) if"),
    "rope_turn_sign": ("return torch.cat([a * c - b * s, b * c + a * s], dim=-1)",
                       "return torch.cat([a * c + b * s, b * c - a * s], dim=-1)"),
    "rope_freq_exponent": ("-2.0 * torch.arange(h, dtype=F64) / D", "-1.0 * torch.arange(h, dtype=F64) / D"),
    "rope_query_position": ("torch.tensor([L - 1]), *rope)", "torch.tensor([L]), *rope)"),
    "right_window_ignored": ("    return window_right if window_right >= 0 else -1", "    return -1"),
    "right_window_overrides_causal": ("    if causal:\n        return 0", "    if causal and window_right < 0:\n        return 0"),
    "right_window_off_by_one": ("int(r.max()) + off + shift + 1))", "int(r.max()) + off + shift))"),
    "window_ignored": ("            vis = w if vis is None else vis & w", "            vis = vis"),
    "fp8_exponent_bias": ("(e - 7).to(F64)", "(e - 8).to(F64)"),
    "fp8_subnormal_as_normal": ("mag = torch.where(e == 0, sub, norm)", "mag = norm"),
    "fp8_nan_on_exponent_15": ("(e == 15) & ((x & 7) == 7)", "(e == 15)"),
    "fp8_window_ignored": ("k = fp8_e4m3_to_float(gather_pages(k_pages, page_table[b], L)) * float(k_scale)\n"
                           "        v = fp8_e4m3_to_float(gather_pages(v_pages, page_table[b], L)) * float(v_scale)\n"
                           "        first = decode_window_first(L, window_left)",
                           "k = fp8_e4m3_to_float(gather_pages(k_pages, page_table[b], L)) * float(k_scale)\n"
                           "        v = fp8_e4m3_to_float(gather_pages(v_pages, page_table[b], L)) * float(v_scale)\n"
                           "        first = 0"),
    "fp8_k_scale_on_values": ("* float(v_scale)", "* float(k_scale)"),
    "softmax_no_exp_shift": ("p = torch.exp(s - torch.where(empty, torch.zeros_like(lse), lse).unsqueeze(1))",
                             "p = torch.exp(s - torch.where(empty, torch.zeros_like(m), m).unsqueeze(1))"),
}


def _mutant(old, new):
    src = open(REF.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = REF.__file__
    exec(compile(src.replace(old, new), REF.__file__ + "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    R = _mutant(*MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin(R)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


def test_oracle_imports_no_product_code():
    """The oracle imports only torch and the standard library."""
    import ast
    for fn in os.listdir(os.path.dirname(REF.__file__)):
        if not fn.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(os.path.dirname(REF.__file__), fn)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""] if node.level == 0 else []
            else:
                continue
            for n in names:
                assert n.split(".")[0] in {"torch", "math", "typing", "__future__"}, (fn, n)


def test_error_stats_semantics():
    ref = torch.tensor([1.0, -2.0, -math.inf], dtype=F64)
    got = torch.tensor([1.01, -2.0, -math.inf], dtype=F64)
    st = oracle.error_stats(got, ref)
    assert abs(st["max_abs"] - 0.01) < 1e-12 and abs(st["max_rel"] - 0.005) < 1e-12 and st["inf_match"]
    st = oracle.error_stats(torch.tensor([1.0, -2.0, 0.0], dtype=F64), ref)
    assert not st["inf_match"]
    st = oracle.error_stats(torch.tensor([math.nan, -2.0, -math.inf], dtype=F64), ref)
    assert math.isnan(st["max_abs"])

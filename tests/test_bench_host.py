"""Host-side arithmetic behind the reported rates (no GPU): the visible-pair
counts that turn a prefill time into TFLOP/s, the source digest that ties a
committed HBM-traffic record to the kernel sources, and the one-GPU guard of
bench.py.  Each count is checked against an explicit loop over (query, key)
pairs written from the visibility rule: query i of a sequence with Lq
queries and Lk keys sees key j iff j <= i + (Lk - Lq) + right (causal:
right = 0) and j >= i + (Lk - Lq) - left, each side open when -1, and
0 <= j < Lk ("FlashAttention-3 内核在最新大模型推理中的集成实践", section 二:
causal masking of packed sequences; the bottom-right alignment is the
reading the oracle also takes)."""
import os
import random
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def brute_pairs(lens_q, lens_k, causal, left=-1, right=-1):
    right = 0 if causal else right
    tot = 0
    for lq, lk in zip(lens_q, lens_k):
        off = lk - lq
        for i in range(lq):
            for j in range(lk):
                if right >= 0 and j > i + off + right:
                    continue
                if left >= 0 and j < i + off - left:
                    continue
                tot += 1
    return tot


CASES = [([5], [5]), ([3], [9]), ([9], [3]), ([1, 7, 0, 4], [1, 7, 2, 11]), ([16, 33], [16, 40]),
         ([0], [0]), ([4], [0]), ([0], [6])]


@pytest.mark.parametrize("lens_q,lens_k", CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_pairs_brute_force(lens_q, lens_k, causal):
    assert workloads.prefill_pairs(lens_q, lens_k, causal) == brute_pairs(lens_q, lens_k, causal)


def test_prefill_pairs_random_and_closed_form():
    rng = random.Random(5)
    for _ in range(200):
        B = rng.randint(1, 4)
        lq = [rng.randint(0, 40) for _ in range(B)]
        lk = [rng.randint(0, 40) for _ in range(B)]
        for causal in (True, False):
            assert workloads.prefill_pairs(lq, lk, causal) == brute_pairs(lq, lk, causal), (lq, lk)
    # equal lengths, causal: L (L + 1) / 2 per sequence
    assert workloads.prefill_pairs([32768], [32768], True) == 32768 * 32769 // 2
    assert workloads.prefill_flops([1024], [1024], 64, 128, True) == 4 * 128 * 64 * 1024 * 1025 // 2


@pytest.mark.parametrize("causal,left,right", [(True, -1, -1), (True, 3, -1), (True, 0, -1),
                                               (False, -1, -1), (False, 4, 2), (False, -1, 0),
                                               (False, 2, -1), (False, 0, 0)])
def test_visible_pairs_brute_force(causal, left, right):
    rng = random.Random(11)
    for _ in range(40):
        B = rng.randint(1, 3)
        lq = [rng.randint(0, 25) for _ in range(B)]
        lk = [rng.randint(0, 25) for _ in range(B)]
        assert bench.visible_pairs(lq, lk, causal, left, right) == \
            brute_pairs(lq, lk, causal, left, right), (lq, lk)


def test_visible_pairs_without_window_is_prefill_pairs():
    lq, lk = [130, 47, 1], [130, 300, 9]
    for causal in (True, False):
        assert bench.visible_pairs(lq, lk, causal) == workloads.prefill_pairs(lq, lk, causal)


@pytest.mark.parametrize("causal", [True, False])
def test_sampled_pairs_brute_force(causal):
    """The CPU baseline's flop count for a row sample: every row, every 5th
    row, and a few single rows, against the explicit loop."""
    lq, lk = [7, 0, 12, 3], [9, 4, 12, 20]
    cu = [0]
    for L in lq:
        cu.append(cu[-1] + L)

    def rows_pairs(rows):
        tot = 0
        for r in rows:
            b = max(i for i in range(len(lq)) if cu[i] <= r < cu[i + 1])
            i, off = r - cu[b], lk[b] - lq[b]
            tot += sum(1 for j in range(lk[b]) if not causal or j <= i + off)
        return tot

    total = cu[-1]
    for rows in (list(range(total)), list(range(0, total, 5)), [0], [total - 1], [8, 9]):
        assert bench.sampled_pairs(lq, lk, rows, causal) == rows_pairs(rows), rows
    assert bench.sampled_pairs(lq, lk, list(range(total)), causal) == \
        workloads.prefill_pairs(lq, lk, causal)


def test_code_only_drops_comments_and_spacing():
    a = "int x = 1; // one\n/* block\n comment */ int y =  2;\n"
    b = "int x = 1;\nint y = 2; // two"
    assert bench._code_only(a) == bench._code_only(b) == "int x = 1; int y = 2;"
    assert bench._code_only("int x = 1;") != bench._code_only("int x = 2;")


def test_traffic_records_parse():
    """Every committed traffic record either matches the current kernel
    sources (then its bytes are at least the algorithmic bytes of a launch
    and below twice them) or is ignored."""
    algorithmic = {"decode_split": 576_114_688, "decode_fp8": 288_057_344,
                   "decode_rope": 576_114_688}
    for kind in bench.TRAFFIC_FILES:
        t = bench.measured_traffic(kind)
        assert t is None or isinstance(t, int)
        if t is not None and kind in algorithmic:
            assert algorithmic[kind] <= t < 2 * algorithmic[kind], (kind, t)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""

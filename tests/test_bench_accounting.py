"""CPU checks of the benchmark's work accounting: the flop and pair counts
it divides by are pinned to closed forms of the causal rule (a query at
absolute position p sees keys 0..p, ONNX GenAI Wiki "Chunked Prefill",
section 1.2) and to brute-force counts, independently of the formulas in
bench.py."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def brute_pairs(past, rows):
    return sum(1 for i in range(rows) for j in range(past + rows) if j <= past + i)


def test_chunk_pairs_brute_force():
    for past, rows in [(0, 1), (0, 7), (5, 3), (100, 17), (512, 416)]:
        assert bench.issued_pairs(past, rows) == brute_pairs(past, rows)
        assert bench.chunk_flops(past, rows, 3, 8) == 4 * 8 * 3 * brute_pairs(past, rows)


def test_chunked_total_equals_one_shot_closed_form():
    # 4000-token prompt in W=512 chunks: the pairs of all chunks sum to the
    # one-shot count sum_{p<4000} (p + 1) = 4000 * 4001 / 2
    chunks = [(512 * i, 512) for i in range(7)] + [(3584, 416)]
    total = sum(bench.chunk_flops(p, r, 32, 128) for p, r in chunks)
    assert total == 4 * 128 * 32 * (4000 * 4001 // 2)
    assert round(total / 1e9, 2) == 131.10
    per_chunk = [round(bench.chunk_flops(p, r, 32, 128) / 1e9, 3) for p, r in chunks]
    assert per_chunk == [2.152, 6.447, 10.742, 15.037, 19.332, 23.627, 27.921, 25.849]


def test_ladder_tail_useful_vs_issued():
    # the 1137-token prompt's last chunk: 113 real rows at past 1024,
    # padded to the 171 rung
    assert bench.issued_pairs(1024, 113) == 122153
    assert bench.issued_pairs(1024, 171) == 189810


def brute_rolling_pairs(L, C, c):
    # chunk j holds the window of the last C positions up to its end; query
    # position p sees the window positions a with a <= p (Horizon blog
    # "Chunk Prefill", sections 3-4, no left pad)
    n = 0
    for j in range(L // c):
        end = (j + 1) * c
        window = range(max(0, end - C), end)
        for i in range(c):
            p = j * c + i
            n += sum(1 for a in window if a <= p)
    return n


def test_rolling_pairs_brute_force_and_workload_total():
    for L, C, c in [(32, 8, 4), (48, 16, 8), (40, 40, 8), (24, 8, 8)]:
        assert bench.rolling_work(L, 1, 1, C, c, False)[0] == brute_rolling_pairs(L, C, c)
    # 4096 fp16 tokens, 16 heads, D 128, C 2048, c 256: 49.41 GFLOP visible
    pairs, _ = bench.rolling_work(4096, 16, 128, 2048, 256, False)
    assert round(4 * 128 * 16 * pairs / 1e9, 2) == 49.41


def test_rolling_bytes_closed_form():
    # per chunk: q + out (2 c rows), the window's K and V (2 min(C, end)
    # rows), the new K and V rows written (2 c rows); rows of H*D*2 bytes;
    # the explicit mask adds c*C*2 bytes per chunk
    L, H, D, C, c = 4096, 16, 128, 2048, 256
    row = H * D * 2
    rows = sum(4 * c + 2 * min(C, (j + 1) * c) for j in range(L // c))
    _, b0 = bench.rolling_work(L, H, D, C, c, False)
    _, b1 = bench.rolling_work(L, H, D, C, c, True)
    assert b0 == rows * row
    assert b1 - b0 == (L // c) * c * C * 2

"""The benchmark's work accounting against closed forms (no GPU)."""
import numpy as np

import bench


def test_prefill_pairs_closed_form():
    N, W, Hq = 1000, 64, 4
    for p in (0.0, 1.0):
        gate = np.full((1, N, 1), int(p), np.uint8)
        useful, band, far = bench.prefill_pairs(gate, W, Hq, 1)
        # window part: sum_i min(i+1, W) = W(W+1)/2 + (N-W)W per head
        assert band == Hq * (W * (W + 1) // 2 + (N - W) * W)
        # far part with every row routed: sum_{i>=W} (i+1-W) = (N-W)(N-W+1)/2 per head
        assert far == (Hq * (N - W) * (N - W + 1) // 2 if p else 0)
        assert useful == band + far
    # all-ones total equals the causal triangle
    u, _, _ = bench.prefill_pairs(np.ones((1, N, 1), np.uint8), W, Hq, 1)
    assert u == Hq * N * (N + 1) // 2
    # two gate groups: heads follow their own group
    gate = np.zeros((1, N, 2), np.uint8)
    gate[0, :, 1] = 1
    u2, b2, f2 = bench.prefill_pairs(gate, W, Hq, 2)
    assert f2 == 2 * (N - W) * (N - W + 1) // 2 and b2 == band


def test_decode_bytes_closed_form():
    B, Hq, Hkv, d, W = 4, 16, 4, 128, 1024
    lens = np.array([32768, 32768, 500, 1024])
    gate = np.array([[1], [0], [1], [0]], np.uint8)
    nbytes, keys = bench.decode_bytes(gate, lens, W, Hq, Hkv, d)
    assert keys == Hkv * (32768 + 1024 + 500 + 1024)
    assert nbytes == keys * d * 2 * 2 + B * Hq * d * 2 * 2


def test_profiled_traffic_is_tied_to_the_kernel_sources(tmp_path):
    """Counter figures are reported only for the sources they were taken on."""
    table = ("## HBM traffic\n\n| kernel | dispatches | FETCH KiB | WRITE KiB | HBM bytes/launch | work |\n"
             "|---|---|---|---|---|---|\n| `attn_kernel` | 4 | 1.0 | 2.0 | 12345 | x |\n\n"
             "## MFMA use\n\n| `attn_kernel` | 1 | 2 | 3 | 999 | 5 |\n")
    good = tmp_path / "good.md"
    good.write_text(f"kernel sources sha256: `{bench.kernel_source_hash()}`\n\n" + table)
    assert bench.profiled_traffic(str(good)) == {"attn_kernel": 12345.0}
    stale = tmp_path / "stale.md"
    stale.write_text("kernel sources sha256: `" + "0" * 64 + "`\n\n" + table)
    assert bench.profiled_traffic(str(stale)) == {}
    assert bench.profiled_traffic(str(tmp_path / "missing.md")) == {}


def test_anchored_accounting_closed_form():
    """Window rows past the window add min(A, i-W+1) anchor pairs; full rows
    are unchanged; decode window pairs read min(A, L-W) anchor rows more."""
    N, W, Hq, A = 1000, 64, 4, 100
    zeros = np.zeros((1, N, 1), np.uint8)
    u0, b0, f0 = bench.prefill_pairs(zeros, W, Hq, 1)
    uA, bA, fA = bench.prefill_pairs(zeros, W, Hq, 1, A)
    # sum over i >= W of min(A, i-W+1) = A(A+1)/2 + (N-W-A)A
    assert uA - u0 == Hq * (A * (A + 1) // 2 + (N - W - A) * A) and fA == 0
    ones = np.ones((1, N, 1), np.uint8)
    assert bench.prefill_pairs(ones, W, Hq, 1, A)[0] == Hq * N * (N + 1) // 2
    lens = np.array([32768, 32768, 500, 1100])
    gate = np.array([[1], [0], [0], [0]], np.uint8)
    _, keys = bench.decode_bytes(gate, lens, 1024, 16, 4, 128, A=256)
    assert keys == 4 * (32768 + (1024 + 256) + 500 + (1024 + 76))

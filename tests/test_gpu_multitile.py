"""Every-row GPU parity at shapes where the persistent window workers take
several tiles each.

The bf16 window branch runs min(tiles, 2 x CUs) resident workgroups that
claim window tiles from per-XCD queues, one tile ahead; the next tile's
first K/V block is copied and its queries loaded inside the current tile's
last block.  At N=8192 with 16 query / 4 KV heads there are 8192/32 x 4 =
1024 window tiles for 512 workers (256 CUs), so every worker hands over at
least once.  With W=16 the tiles alternate between two blocks and a single
block (tile 0 and every odd tile: the band [q0-15, q0+31] starts inside the
block that holds q0), which takes the one-block path of the handover.
Every row and head is compared against the float64 oracle on the same
stored bf16 values (max-abs 2e-2), as are the both-branch distance and the
anchored window branch.
"""
import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_router_amd import synth
from tests.gpu_util import TOL, dev, diff_tolerance, ensure_built, host, max_abs, say

pytestmark = pytest.mark.gpu

N, HQ, HKV = 8192, 16, 4


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    yield
    torch.cuda.empty_cache()


def swa():
    import sliding_window_attention_router_amd as m

    return m


def _window_tiles(N, Hq, Hkv, B=1):
    rows_per_tile = 128  # query rows of a window tile: (128 / (Hq/Hkv)) tokens x Hq/Hkv heads
    return B * Hkv * -(-N // (rows_per_tile // (Hq // Hkv)))


def _assert_handover(N, Hq, Hkv):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = _window_tiles(N, Hq, Hkv)
    say(f"  window tiles {tiles}, resident workers {2 * cus}")
    assert tiles > 2 * cus, "shape too small: no worker would take a second tile"


CASES = [
    # d,  W,    p,    A,   seed   (all: B=1, N=8192, Hq=16, Hkv=4, G=1, bf16)
    (128, 1024, 0.13, 0, 41),   # the long-prefill shape at a quarter of its length
    (128, 16, 0.13, 0, 42),     # one- and two-block window tiles
    (64, 32, 0.05, 0, 43),      # d=64: single-block tiles, sparse routing
    (128, 1024, 0.13, 256, 44), # anchored window branch (anchor blocks ahead of each tile)
]


@pytest.mark.parametrize("d,W,p,A,seed", CASES)
def test_every_row_multitile(d, W, p, A, seed):
    say(f"every-row parity N={N} Hq={HQ} Hkv={HKV} d={d} W={W} p={p} A={A} seed={seed}")
    _assert_handover(N, HQ, HKV)
    w = synth.long_prefill(seed=seed, N=N, Hq=HQ, Hkv=HKV, d=d, W=W, p=p)
    bf = torch.bfloat16
    Q, K, V, g = dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), dev(w.gate)
    O, _ = swa().prefill(Q, K, V, g, W, anchors=A)
    O2, _ = swa().prefill(Q, K, V, g, W, anchors=A)
    torch.cuda.synchronize()
    assert torch.equal(O, O2), "two runs differ"
    ref = oracle.prefill(w.Q, w.K, w.V, w.gate, W, anchors=A)["O"]
    err = np.abs(host(O) - ref)
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    say(f"  density {w.gate.mean():.4f}; all {N} rows x {HQ} heads: max-abs {err.max():.3e} "
        f"at (b, row, head, ch) {tuple(int(x) for x in worst)}")
    assert err.max() <= TOL["bf16"]


def test_every_row_multitile_both_branch():
    """Both-branch mode at the single-block shape: every row takes the far
    part, the merge writes the distance; O and diff on every row."""
    d, W, p = 64, 32, 0.05
    say(f"every-row both-branch N={N} Hq={HQ} Hkv={HKV} d={d} W={W} p={p}")
    _assert_handover(N, HQ, HKV)
    w = synth.long_prefill(seed=43, N=N, Hq=HQ, Hkv=HKV, d=d, W=W, p=p)
    bf = torch.bfloat16
    O, diff = swa().prefill(dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), dev(w.gate), W, both_branch=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(w.Q, w.K, w.V, w.gate, W, both_branch=True)
    err = max_abs(host(O), ref["O"])
    dg = host(diff)
    derr = np.abs(dg - ref["diff"])
    tol = diff_tolerance(ref["diff"], HQ * d, TOL["bf16"])
    say(f"  O max-abs {err:.3e}; diff max-abs {derr.max():.3e}, worst share of its bound "
        f"{np.max(derr / np.maximum(tol, 1e-30)):.3e}")
    assert err <= TOL["bf16"]
    assert np.all(derr <= tol)
    assert np.all(dg[:, :W] == 0.0)


def test_many_units_schedule_tables_in_global_memory():
    """B=33 sequences x 32 KV heads (MHA) at N=2048: 1056 (sequence, unit)
    pairs exceed the far schedule's per-unit LDS tables (1024 entries) and,
    with 5 chunk slots each, its (unit, chunk) tables, so the schedule builds
    all of them in global memory.  Sampled rows of every sequence against the
    oracle."""
    B, N, H, d, W, p = 33, 2048, 32, 64, 64, 0.1
    say(f"schedule in global memory: B={B} N={N} MHA {H} heads d={d} W={W} p={p}")
    w = synth.long_prefill(seed=46, B=B, N=N, Hq=H, Hkv=H, d=d, W=W, p=p)
    bf = torch.bfloat16
    O, _ = swa().prefill(dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), dev(w.gate), W)
    torch.cuda.synchronize()
    Oh = host(O)
    rows = np.unique(np.concatenate([np.arange(0, 80), np.arange(N - 40, N),
                                     np.random.default_rng(47).integers(0, N, 120)]))
    err = 0.0
    for b in range(B):
        ref = oracle.prefill(w.Q[b:b + 1], w.K[b:b + 1], w.V[b:b + 1], w.gate[b:b + 1], W, rows=rows)["O"]
        err = max(err, max_abs(Oh[b:b + 1, rows], ref))
    say(f"  {rows.size} rows x {B} sequences x {H} heads: max-abs {err:.3e}")
    assert err <= TOL["bf16"]


def test_dense_gate_near_the_item_bound():
    """Gate all 1 through the hard-gate path at N=8192 (GQA 16/4, W=1024):
    the far schedule cuts about 1900 items, close to the bound the plan sizes
    its far grid and partial buffers by for this shape (1024 + one per far
    tile = 2048).  Sampled rows of every head against the oracle."""
    d, W = 128, 1024
    say(f"dense gate near the item bound: N={N} Hq={HQ} Hkv={HKV} d={d} W={W}")
    w = synth.long_prefill(seed=48, N=N, Hq=HQ, Hkv=HKV, d=d, W=W, p=0.13)
    gate = np.ones_like(w.gate)
    bf = torch.bfloat16
    O, _ = swa().prefill(dev(w.Q, bf), dev(w.K, bf), dev(w.V, bf), dev(gate), W)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(W - 8, W + 72), np.arange(N - 80, N),
                                     np.random.default_rng(49).integers(0, N, 120)]))
    ref = oracle.prefill(w.Q, w.K, w.V, gate, W, rows=rows)["O"]
    err = max_abs(host(O)[:, rows], ref)
    say(f"  {rows.size} rows x {HQ} heads: max-abs {err:.3e}")
    assert err <= TOL["bf16"]


"""GPU parity of the index kernel's own output: the Block-Max score table
(msa_index_scores) against the oracle's index scores and block maxima
[hyper.ai paper page 2606.13392, 方法 (Method): dot-product index scores
max-pooled over fixed key blocks; Telegram review quant_prune_distill post
751, "Метод"].

Integer-valued index inputs give exact fp32 dot products, so the table must
match bit for bit.  On Gaussian inputs each score is a sum of d_idx exact
bf16 x bf16 products accumulated in fp32, so it lies within
d_idx * 2^-23 * sum_c |q_c k_c| of the exact value, and a block maximum within
the largest such bound over the block's keys."""
import numpy as np
import pytest
import torch

from block_sparse_long_02_amd import binding as bd
from block_sparse_long_02_amd import inputs
from oracle import msa_oracle as orc
from gpu_common import say

pytestmark = pytest.mark.gpu


def _gpu_scores(inp, B, t0, t1, row_stride, with_sm):
    b, T, G, di = inp.idx_q.shape
    dims = bd.make_dims(b, T, G, G, index_dim=di, block_size=B, topk=1)
    scores = torch.full((b, t1 - t0, G, row_stride), float("nan"), dtype=torch.float32, device="cuda")
    sm = None
    if with_sm:
        L = (t1 - 1) // B
        sm = torch.full((b, t1 - t0, G, max(1, (L + 15) // 16)), float("nan"), dtype=torch.float32,
                        device="cuda")
    bd.msa_index_scores(dims, inp.idx_q.cuda(), inp.idx_k.cuda(), scores, t0, t1, row_stride,
                        superblock_max=sm)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), (sm.cpu().numpy() if sm is not None else None)


def _check_rows(inp, B, t0, scores, sm, rows, exact):
    iq = inp.idx_q.to(torch.float64).numpy()
    ik = inp.idx_k.to(torch.float64).numpy()
    G, di = iq.shape[2], iq.shape[3]
    worst = 0.0
    n_checked = 0
    for s, t in rows:
        L = t // B
        if L == 0:
            continue
        for g in range(G):
            ref = orc.block_max(orc.index_scores(iq[s, t, g], ik[s], t), t, B)[:L]
            got = scores[s, t - t0, g, :L].astype(np.float64)
            if exact:
                assert np.array_equal(got, ref), (s, t, g, np.flatnonzero(got != ref)[:8])
            else:
                mag = np.abs(ik[s, : t + 1]) @ np.abs(iq[s, t, g])       # sum_c |q_c k_c| per key
                bound = orc.block_max(mag, t, B)[:L] * di * 2.0 ** -23
                err = np.abs(got - ref)
                assert (err <= bound).all(), (s, t, g, float((err - bound).max()))
                worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
            if sm is not None:
                nsb = (L + 15) // 16
                sref = np.array([got[16 * i: min(16 * i + 16, L)].max() for i in range(nsb)])
                assert np.array_equal(sm[s, t - t0, g, :nsb].astype(np.float64), sref), (s, t, g)
            n_checked += 1
    return n_checked, worst


@pytest.mark.parametrize("mode", ["integer", "gaussian"])
def test_index_scores_tiny_prefill_every_row(mode):
    """T = 2048, 4 groups, d_idx 64, B 128: every row of the table."""
    T, G, di, B = 2048, 4, 64, 128
    say(f"[index scores] T={T} G={G} di={di} B={B} {mode}")
    inp = inputs.make_prefill(T, G, G, 8, di, seed=81, idx_mode=mode)
    rs = bd.scores_row_stride(bd.make_dims(1, T, G, G, index_dim=di, block_size=B, topk=1), T)
    scores, _ = _gpu_scores(inp, B, 0, T, rs, False)
    n, worst = _check_rows(inp, B, 0, scores, None, [(0, t) for t in range(T)], mode == "integer")
    say(f"  rows x groups checked {n}, largest error / bound {worst:.3f}")


@pytest.mark.parametrize("mode,di,B", [("integer", 128, 64), ("gaussian", 128, 32), ("integer", 64, 32)])
def test_index_scores_offset_range_wide_stride_and_superblocks(mode, di, B):
    """A query range that starts inside the sequence and ends on a ragged
    token (t0 = 300, t1 = 1999), batch 2, a row stride wider than needed, and
    the kernel variant that also writes the 16-block run maxima."""
    T, G = 2100, 3
    t0, t1 = 300, 1999
    say(f"[index scores range] T={T} G={G} di={di} B={B} [{t0},{t1}) {mode}")
    inp = inputs.make_prefill(T, G, G, 8, di, batch=2, seed=82 + B, idx_mode=mode)
    L = (t1 - 1) // B
    rs = (L + 3) // 4 * 4 + 8
    rows = [(s, t) for s in range(2) for t in list(range(t0, t1, 7)) + [t1 - 1]]
    for with_sm in (False, True):
        scores, sm = _gpu_scores(inp, B, t0, t1, rs, with_sm)
        n, worst = _check_rows(inp, B, t0, scores, sm, rows, mode == "integer")
        say(f"  superblocks={with_sm}: rows x groups checked {n}, largest error / bound {worst:.3f}")


def test_index_scores_rows_beyond_1024_candidates():
    """B = 32, query tokens [32768, 36000): rows of up to 1124 candidate
    blocks, the range the selection serves through the 16-block run maxima.
    Integer inputs, exact; sampled rows plus the first and last."""
    T, G, di, B = 36000, 2, 64, 32
    t0, t1 = 32768, 36000
    say(f"[index scores long rows] T={T} B={B} [{t0},{t1})")
    inp = inputs.make_prefill(T, G, G, 8, di, seed=84, idx_mode="integer")
    L = (t1 - 1) // B
    assert L > 1024
    rs = (L + 3) // 4 * 4
    scores, sm = _gpu_scores(inp, B, t0, t1, rs, True)
    rows = [(0, t) for t in [t0, t0 + 1, t0 + 31, t0 + 32] + list(range(t0 + 45, t1, 97)) + [t1 - 1]]
    n, _ = _check_rows(inp, B, t0, scores, sm, rows, True)
    say(f"  rows x groups checked {n}")

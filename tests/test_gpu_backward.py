"""GPU parity of msa_prefill_backward against the oracle's attention_backward.

The forward runs on the GPU (its selection and lse feed the backward, as in
training); the oracle recomputes the gradients in fp64 from the same bf16
inputs and the GPU's selection.  Bounds: max-abs <= 1e-2 of the largest
reference value and mean-relative (sum |diff| / sum |ref|) <= 5e-3 per
gradient.  P and dS enter the MFMA products rounded to bf16 (at most 2^-8 relative)
and dq is summed from bf16 partials, one per selected block; over the
hundreds to thousands of keys of a row these roundings average out to a few
1e-3 of the values, which is what the bounds allow.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_02_amd import binding as bd
from block_sparse_long_02_amd import inputs
from oracle import msa_oracle as orc

from gpu_common import gpu_prefill, say

pytestmark = pytest.mark.gpu


def _dout(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def gpu_backward(inp, out, lse, bidx, dout, B, k, query_chunk=0):
    b, T, Hq, d = inp.q.shape
    G = inp.k.shape[2]
    dims = bd.make_dims(b, T, Hq, G, head_dim=d, index_dim=inp.idx_q.shape[-1], block_size=B, topk=k,
                        query_chunk=query_chunk)
    dq = torch.full((b, T, Hq, d), float("nan"), device="cuda")
    dk = torch.full((b, T, G, d), float("nan"), device="cuda")
    dv = torch.full((b, T, G, d), float("nan"), device="cuda")
    bd.msa_prefill_backward(dims, inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), out.cuda(), lse.cuda(), dout.cuda(),
                            bidx.cuda().to(torch.int32).contiguous(), dq, dk, dv)
    torch.cuda.synchronize()
    return dq.cpu().double().numpy(), dk.cpu().double().numpy(), dv.cpu().double().numpy()


def check_grad(got, ref, what):
    assert np.isfinite(got).all(), what
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    mr = err.sum() / max(np.abs(ref).sum(), 1e-300)
    say(f"  {what}: max-abs {err.max():.3e} (of {scale:.3e})  mean-rel {mr:.3e}")
    assert err.max() <= 1e-2 * scale, what
    assert mr <= 5e-3, what


CASES = [
    # T, Hq, G, B, k, query_chunk, batch
    (1000, 16, 4, 64, 6, 0, 1),       # R = 4, ragged tail
    (777, 8, 8, 32, 9, 256, 2),       # R = 1, three query chunks, batch 2
    (600, 24, 8, 128, 3, 0, 1),       # R = 3, partial last block
    (700, 64, 8, 128, 4, 0, 1),       # the 128K workload's heads and block size
    (300, 32, 2, 64, 12, 0, 1),       # R = 16, k beyond the number of blocks (all selected)
    (200, 128, 1, 32, 5, 0, 1),       # R = 128, the largest heads per group
]


def test_backward_one_token():
    """T = 1: each head attends to one key with P = 1, so dv = the sum of the
    group's dO rows and, exactly, dS = P (dP - Delta) = 0, hence dq = dk = 0.
    On the GPU dP (an MFMA dot product) and Delta (dO . out, out = v exactly)
    are two fp32 sums of the same 128 exact bf16 products in different orders,
    each within 128 * 2^-24 * sum_i |dO_i v_i| of the exact value, so |dS| is at
    most twice that, and dq, dk are bounded by the softmax scale times |dS|
    times |k| or |q| (plus the bf16 rounding of the dq partial)."""
    T, Hq, G, B, k, d = 1, 8, 2, 128, 4, 128
    say("[backward one token]")
    inp = inputs.make_prefill(T, Hq, G, d, 64, seed=77)
    out, lse, bidx = gpu_prefill(inp, B, k)
    dout = _dout((1, T, Hq, d), 78)
    dq, dk, dv = gpu_backward(inp, out, lse, bidx, dout, B, k)
    rq, rk, rv = orc.attention_backward(inp.q, inp.k, inp.v, dout, bidx, B)
    check_grad(dv, rv, "dv")
    assert np.abs(rq).max() == 0.0 and np.abs(rk).max() == 0.0
    R = Hq // G
    scale = 1.0 / np.sqrt(d)
    q64 = inp.q[0, 0].double().numpy()               # [Hq, d]
    k64 = inp.k[0, 0].double().numpy()               # [G, d]
    v64 = inp.v[0, 0].double().numpy()
    do64 = dout[0, 0].double().numpy()
    for h in range(Hq):
        g = h // R
        ds_bound = 2 * d * 2.0 ** -24 * np.abs(do64[h] * v64[g]).sum()
        assert (np.abs(dq[0, 0, h]) <= scale * ds_bound * np.abs(k64[g]) * (1 + 2.0 ** -8) + 1e-30).all(), h
    for g in range(G):
        ds_bounds = np.array([2 * d * 2.0 ** -24 * np.abs(do64[h] * v64[g]).sum() for h in range(g * R, g * R + R)])
        bound = scale * (ds_bounds[:, None] * np.abs(q64[g * R:(g + 1) * R])).sum(0)
        assert (np.abs(dk[0, 0, g]) <= bound * (1 + 1e-6) + 1e-30).all(), g
    say(f"  dq max {np.abs(dq).max():.2e}, dk max {np.abs(dk).max():.2e} (exact 0)")


@pytest.mark.parametrize("T,Hq,G,B,k,chunk,nb", CASES)
def test_backward_vs_oracle(T, Hq, G, B, k, chunk, nb):
    say(f"[backward] T={T} Hq={Hq} G={G} B={B} k={k} chunk={chunk} batch={nb}")
    inp = inputs.make_prefill(T, Hq, G, 128, 64, batch=nb, seed=900 + T)
    out, lse, bidx = gpu_prefill(inp, B, k)
    dout = _dout((nb, T, Hq, 128), 901 + T)
    dq, dk, dv = gpu_backward(inp, out, lse, bidx, dout, B, k, query_chunk=chunk)
    rq, rk, rv = orc.attention_backward(inp.q, inp.k, inp.v, dout, bidx, B)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_backward_given_selection_edge_rows():
    """A given selection with rows missing their local block, out-of-range
    entries and rows that attend nothing (dq = 0 there)."""
    T, Hq, G, B, k = 500, 8, 2, 32, 4
    say("[backward given selection]")
    inp = inputs.make_prefill(T, Hq, G, 128, 64, seed=911)
    rng = np.random.default_rng(912)
    sel = np.full((1, T, G, k), -1, dtype=np.int32)
    for t in range(T):
        L = t // B
        for g in range(G):
            if t % 11 == 5:
                continue                                   # nothing to attend
            c = list(rng.permutation(L)[: k - 1]) if L > 0 else []
            row = ([] if t % 7 == 3 and c else [L]) + c
            if len(row) < k and t % 3 == 0:
                row.append(L + 1 + t % 5)                   # out of range: ignored
            sel[0, t, g, : len(row)] = rng.permutation(row)
    bidx = torch.from_numpy(sel)
    out, lse, _ = gpu_prefill(inp, B, k, flags=bd.MSA_GIVEN_INDICES, block_idx=bidx)
    dout = _dout((1, T, Hq, 128), 913)
    dq, dk, dv = gpu_backward(inp, out, lse, bidx, dout, B, k)
    rq, rk, rv = orc.attention_backward(inp.q, inp.k, inp.v, dout, bidx, B)
    empty = np.array([t % 11 == 5 for t in range(T)])
    assert (dq[0, empty] == 0).all()
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_backward_bitwise_deterministic():
    T, Hq, G, B, k = 2100, 16, 2, 64, 8
    say("[backward determinism]")
    inp = inputs.make_prefill(T, Hq, G, 128, 64, seed=921)
    out, lse, bidx = gpu_prefill(inp, B, k)
    dout = _dout((1, T, Hq, 128), 922)
    a = gpu_backward(inp, out, lse, bidx, dout, B, k)
    b = gpu_backward(inp, out, lse, bidx, dout, B, k)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_several_list_windows():
    """T beyond two 8192-token list windows: lists of one key block in several
    windows, their dk/dv partials summed across windows; then the same in four
    query chunks, dk/dv accumulated across chunks."""
    T, Hq, G, B, k = 16500, 4, 2, 64, 4
    inp = inputs.make_prefill(T, Hq, G, 128, 64, seed=931)
    out, lse, bidx = gpu_prefill(inp, B, k)
    dout = _dout((1, T, Hq, 128), 932)
    rq, rk, rv = orc.attention_backward(inp.q, inp.k, inp.v, dout, bidx, B)
    for chunk in (0, 5120):
        say(f"[backward multi-window] T={T} query_chunk={chunk}")
        dq, dk, dv = gpu_backward(inp, out, lse, bidx, dout, B, k, query_chunk=chunk)
        check_grad(dq, rq, "dq")
        check_grad(dk, rk, "dk")
        check_grad(dv, rv, "dv")


def test_backward_and_indexer_kl_on_a_forced_sink_selection():
    """The forced-sink prefill's selection (block 0 beside the local block in
    every row) fed to the backward and to the indexer KL: both against the
    oracle on that selection."""
    T, Hq, G, B, k = 900, 16, 4, 64, 5
    say(f"[backward + KL on a sink selection] T={T} B={B} k={k}")
    inp = inputs.make_prefill(T, Hq, G, 128, 64, seed=930)
    out, lse, bidx = gpu_prefill(inp, B, k, flags=bd.MSA_FORCE_SINK)
    sel = bidx.numpy()
    assert all(0 in sel[0, t, g] for t in range(B, T) for g in range(G)), "block 0 in every row past the first block"
    dout = _dout((1, T, Hq, 128), 931)
    dq, dk, dv = gpu_backward(inp, out, lse, bidx, dout, B, k)
    rq, rk, rv = orc.attention_backward(inp.q, inp.k, inp.v, dout, bidx, B)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")
    dims = bd.make_dims(1, T, Hq, G, index_dim=64, block_size=B, topk=k)
    kl = torch.empty((1, T, G), device="cuda")
    diq = torch.empty((1, T, G, 64), device="cuda")
    dik = torch.empty((1, T, 64), device="cuda")
    bd.msa_indexer_kl(dims, inp.q.cuda(), inp.k.cuda(), inp.idx_q.cuda(), inp.idx_k.cuda(), bidx.cuda(),
                      lse.cuda(), kl, diq, dik)
    torch.cuda.synchronize()
    ores = orc.indexer_kl(inp.q, inp.k, inp.idx_q, inp.idx_k, bidx, B)
    kl_ref = np.array([ores["kl"][(0, t)] for t in range(T)])
    assert (np.abs(kl.cpu().double().numpy()[0] - kl_ref) <= 1e-3 * np.abs(kl_ref) + 1e-4).all()
    check_grad(diq.cpu().double().numpy(), np.stack([ores["d_idx_q"][(0, t)] for t in range(T)])[None], "d idx_q")
    check_grad(dik.cpu().double().numpy(), ores["d_idx_k"], "d idx_k")


def test_duplicate_blocks_in_a_selection_keep_the_fallback_sort():
    """A selection that repeats a block within a row is invalid input; the
    list sort detects the repeated token and falls back to its sorting
    network.  The calls must stay finite and bitwise repeatable."""
    T, Hq, G, B, k = 700, 8, 2, 64, 4
    say("[duplicate blocks in a given selection]")
    inp = inputs.make_prefill(T, Hq, G, 128, 64, seed=940)
    _, _, bidx = gpu_prefill(inp, B, k)
    sel = bidx.numpy().copy()
    for t in range(2 * B, T, 7):
        for g in range(G):
            if sel[0, t, g, 1] >= 0:
                sel[0, t, g, 2] = sel[0, t, g, 1]          # the same block twice
    bsel = torch.from_numpy(sel)
    out, lse, _ = gpu_prefill(inp, B, k, flags=bd.MSA_GIVEN_INDICES, block_idx=bsel)
    dout = _dout((1, T, Hq, 128), 941)
    runs = [gpu_backward(inp, out, lse, bsel, dout, B, k) for _ in range(2)]
    for a_, b_ in zip(*runs):
        assert np.isfinite(a_).all() and np.array_equal(a_, b_)
    dims = bd.make_dims(1, T, Hq, G, index_dim=64, block_size=B, topk=k)
    res = []
    for _ in range(2):
        kl = torch.empty((1, T, G), device="cuda")
        diq = torch.empty((1, T, G, 64), device="cuda")
        dik = torch.empty((1, T, 64), device="cuda")
        bd.msa_indexer_kl(dims, inp.q.cuda(), inp.k.cuda(), inp.idx_q.cuda(), inp.idx_k.cuda(), bsel.cuda(),
                          lse.cuda(), kl, diq, dik)
        torch.cuda.synchronize()
        res.append([x.cpu().numpy() for x in (kl, diq, dik)])
    for a_, b_ in zip(*res):
        assert np.isfinite(a_).all() and np.array_equal(a_, b_)

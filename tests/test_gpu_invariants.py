"""Properties of the method checked on the GPU path at sizes the oracle cannot
run whole [hyper.ai paper page 2606.13392, 方法 (Method): top-k of the block
maxima with the local block kept, then softmax attention over the gathered
keys]:

- nesting: the top-k is a total order on the blocks (score descending, lower
  block first), so the k-selection of a row is contained in its
  (k + 1)-selection, with and without the forced sink block;
- q = 0: every selected key gets the same weight, so each output row is the
  mean of the V rows its selection gathers;
- V constant: the output is that constant (the weights sum to one);
- every output coordinate lies between the smallest and largest value of
  that coordinate over the gathered V rows (a convex combination), up to the
  bf16 rounding of the output.

Outputs are checked on the GPU's own selection, gathered with torch."""
import pytest
import torch

from block_sparse_long_02_amd import binding as bd
from block_sparse_long_02_amd import inputs
from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.load_library()


def _index_topk(idx_q, idx_k, B, k, flags=0):
    b, T, G, di = idx_q.shape
    dims = bd.make_dims(b, T, G, G, index_dim=di, block_size=B, topk=k, flags=flags)
    bidx = torch.full((b, T, G, k), -7, dtype=torch.int32, device="cuda")
    bd.msa_index_topk(dims, idx_q, idx_k, bidx)
    torch.cuda.synchronize()
    return bidx


def _contained(small, big):
    """Every valid entry of each row of small appears in the same row of big."""
    hit = (small.unsqueeze(-1) == big.unsqueeze(-2)).any(-1)
    return bool((hit | (small < 0)).all())


@pytest.mark.parametrize("sink", [False, True])
def test_selection_nesting_128k(sink):
    T, G, di, B = 131072, 8, 128, 128
    say(f"[nesting 128K] sink={sink}")
    dev = torch.device("cuda")
    x = inputs.make_prefill(T, G, G, 8, di, seed=21, device=dev, block_size=B, skew_std=0.5)
    fl = bd.MSA_FORCE_SINK if sink else 0
    sels = {k: _index_topk(x.idx_q, x.idx_k, B, k, fl) for k in (8, 9, 16, 21)}
    for k, kb in ((8, 9), (9, 16), (16, 21)):
        for t0 in range(0, T, 16384):   # in slices, to bound the comparison's memory
            assert _contained(sels[k][:, t0:t0 + 16384], sels[kb][:, t0:t0 + 16384]), (k, kb, t0)


def _gather_rows(bidx, t, g, B):
    """Token indices of row (t, g)'s selection, keys <= t."""
    blocks = bidx[0, t, g]
    blocks = blocks[blocks >= 0]
    toks = (blocks.view(-1, 1) * B + torch.arange(B, device=blocks.device).view(1, -1)).reshape(-1)
    return toks[toks <= t]


def test_zero_queries_give_the_mean_of_the_selected_values():
    T, Hq, G, d, di, B, k = 20000, 16, 4, 128, 64, 64, 8
    say(f"[q = 0] T={T} B={B} k={k}")
    dev = torch.device("cuda")
    x = inputs.make_prefill(T, Hq, G, d, di, seed=22, device=dev)
    q = torch.zeros_like(x.q)
    dims = bd.make_dims(1, T, Hq, G, index_dim=di, block_size=B, topk=k)
    out = torch.empty_like(q)
    bidx = torch.empty((1, T, G, k), dtype=torch.int32, device=dev)
    bd.msa_prefill(dims, q, x.k, x.v, x.idx_q, x.idx_k, out, block_idx=bidx)
    torch.cuda.synchronize()
    R = Hq // G
    gen = torch.Generator().manual_seed(5)
    rows = torch.randint(0, T, (200,), generator=gen).tolist() + [0, 1, B - 1, B, T - 1]
    worst = 0.0
    for t in rows:
        for g in range(G):
            toks = _gather_rows(bidx, t, g, B)
            ref = x.v[0, toks, g].float().mean(0)
            got = out[0, t, g * R:(g + 1) * R].float()
            # bf16 output rounding (half an ulp: at most 2^-8 relative) with room for
            # the fp32 sums and the fp16 partials of the block-major pass
            err = (got - ref).abs() / (2.0 ** -8 * ref.abs() + 1e-3)
            worst = max(worst, float(err.max()))
    say(f"  largest |out - mean of gathered V| / (2^-8 |mean| + 1e-3): {worst:.3f}")
    assert worst <= 1.0


def test_constant_values_and_convex_hull():
    T, Hq, G, d, di, B, k = 20000, 16, 4, 128, 64, 128, 6
    say(f"[V constant, convex hull] T={T} B={B} k={k}")
    dev = torch.device("cuda")
    x = inputs.make_prefill(T, Hq, G, d, di, seed=23, device=dev)
    dims = bd.make_dims(1, T, Hq, G, index_dim=di, block_size=B, topk=k)
    # a constant V per (group, coordinate): the output must equal it exactly
    c = torch.linspace(-3.0, 3.0, G * d, device=dev).view(1, 1, G, d).to(torch.bfloat16)
    vc = c.expand(1, T, G, d).contiguous()
    out = torch.empty_like(x.q)
    bd.msa_prefill(dims, x.q, x.k, vc, x.idx_q, x.idx_k, out)
    torch.cuda.synchronize()
    R = Hq // G
    want = c[0, 0].repeat_interleave(R, dim=0)          # [Hq, d]
    assert torch.equal(out[0], want.unsqueeze(0).expand(T, Hq, d)), "constant V"
    # random V: every coordinate within the range of the gathered rows
    bidx = torch.empty((1, T, G, k), dtype=torch.int32, device=dev)
    bd.msa_prefill(dims, x.q, x.k, x.v, x.idx_q, x.idx_k, out, block_idx=bidx)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(6)
    rows = torch.randint(0, T, (300,), generator=gen).tolist() + [0, T - 1]
    for t in rows:
        for g in range(G):
            vg = x.v[0, _gather_rows(bidx, t, g, B), g].float()
            lo, hi = vg.min(0).values, vg.max(0).values
            o = out[0, t, g * R:(g + 1) * R].float()
            slack = 2.0 ** -8 * torch.maximum(lo.abs(), hi.abs())   # the output's bf16 rounding
            assert bool(((o >= lo - slack) & (o <= hi + slack)).all()), (t, g)

"""GPU parity of the one-pass Index Branch (MSA_ONE_PASS_INDEX): scores,
Block-Max and the Top-k with the forced blocks in one kernel with no score
table [hyper.ai paper page 2606.13392, 方法 (Method)].

Its selection must equal the default two-pass path's bit for bit (the same
fp32 block maxima, the same order and tie rule), on Gaussian inputs and on
integer inputs full of exact ties; on integer inputs it is also compared with
the oracle's selection row by row.  Prefill with the flag must then give the
default path's outputs bit for bit, since the main branch sees the same lists.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_02_amd import binding as bd
from block_sparse_long_02_amd import inputs
from oracle import msa_oracle as orc

from gpu_common import check_selection_invariants, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.load_library()


def _index_topk(inp, B, k, flags, chunk=0):
    b, T, G, di = inp.idx_q.shape
    dims = bd.make_dims(b, T, G, G, index_dim=di, block_size=B, topk=k, flags=flags, query_chunk=chunk)
    bidx = torch.full((b, T, G, k), -7, dtype=torch.int32, device="cuda")
    bd.msa_index_topk(dims, inp.idx_q.cuda(), inp.idx_k.cuda(), bidx)
    torch.cuda.synchronize()
    return bidx


CASES = [
    # T, G, di, B, k, sink, batch, query_chunk, idx inputs
    (2048, 4, 64, 128, 16, False, 2, 0, "gaussian"),
    (5000, 3, 128, 64, 8, True, 1, 0, "integer"),
    (9000, 8, 128, 32, 17, False, 1, 4096, "integer"),   # the largest topk, several chunks
    (3000, 2, 64, 128, 1, False, 1, 0, "gaussian"),      # the local block alone
    (20000, 8, 128, 128, 16, True, 1, 0, "gaussian"),
    (6000, 4, 128, 32, 17, True, 2, 2048, "integer"),
    (4100, 8, 128, 128, 16, False, 1, 0, "integer"),
    (40000, 8, 64, 32, 2, True, 1, 0, "integer"),        # sink + local block only
    (100, 2, 64, 128, 4, True, 1, 0, "gaussian"),        # no candidate block in any row
    (700, 2, 64, 64, 17, False, 1, 0, "integer"),        # k beyond the block count
]


@pytest.mark.parametrize("T,G,di,B,k,sink,nb,chunk,mode", CASES)
def test_one_pass_matches_two_pass(T, G, di, B, k, sink, nb, chunk, mode):
    say(f"[one-pass index] T={T} G={G} di={di} B={B} k={k} sink={sink} batch={nb} chunk={chunk} {mode}")
    inp = inputs.make_prefill(T, G, G, 8, di, batch=nb, seed=T + k, idx_mode=mode)
    sinkf = bd.MSA_FORCE_SINK if sink else 0
    two = _index_topk(inp, B, k, sinkf, chunk)
    one = _index_topk(inp, B, k, sinkf | bd.MSA_ONE_PASS_INDEX, chunk)
    assert not (one == -7).any(), "entries left unwritten"
    neq = (one != two).nonzero()
    assert neq.numel() == 0, f"{neq.shape[0]} entries differ, first {neq[:4].tolist()}"
    got = one.cpu()
    if not sink:
        check_selection_invariants(got, T, G, B, k)
    if mode == "integer":   # exact scores: the oracle's selection, row by row
        iq = inp.idx_q.to(torch.float64).numpy()
        ik = inp.idx_k.to(torch.float64).numpy()
        rng = np.random.default_rng(T)
        rows = sorted(set([(s, int(t)) for s in range(nb) for t in rng.integers(0, T, 40)] + [(nb - 1, T - 1)]))
        for s, t in rows:
            for g in range(G):
                S = orc.block_max(orc.index_scores(iq[s, t, g], ik[s], t), t, B)
                exp = orc.select_blocks(S, t, B, k, sink=sink)
                assert got[s, t, g].tolist() == exp.tolist(), (s, t, g)


def test_one_pass_all_ties():
    """Every score equal: the tie rule alone decides, blocks 0..m-2 (the
    lowest candidates) beside the local block, with the sink and without."""
    T, G, di, B, k = 9000, 2, 64, 32, 9
    say(f"[one-pass index all ties] T={T} B={B} k={k}")
    base = inputs.make_prefill(T, G, G, 8, di, seed=3)
    inp = inputs.PrefillInputs(base.q, base.k, base.v, torch.zeros_like(base.idx_q), torch.zeros_like(base.idx_k))
    for sink in (False, True):
        got = _index_topk(inp, B, k, bd.MSA_ONE_PASS_INDEX | (bd.MSA_FORCE_SINK if sink else 0)).cpu().numpy()
        for t in list(range(0, T, 89)) + [T - 1]:
            L = t // B
            m = min(k, L + 1)
            exp = list(range(m - 1)) + [L] + [-1] * (k - m)   # block 0 is the lowest candidate either way
            for g in range(G):
                assert got[0, t, g].tolist() == exp, (t, g, sink)


@pytest.mark.parametrize("with_bidx,chunk", [(True, 0), (False, 1024)])
def test_one_pass_prefill_outputs_identical(with_bidx, chunk):
    """Prefill with the flag: out, lse and block_idx equal the default path's
    bit for bit, with the selection written to the caller's block_idx or kept
    in the workspace (query chunks of 1024 tokens)."""
    T, Hq, G, d, di, B, k = 5000, 16, 4, 128, 64, 64, 12
    say(f"[one-pass prefill] T={T} B={B} k={k} block_idx={with_bidx} chunk={chunk}")
    inp = inputs.make_prefill(T, Hq, G, d, di, seed=77)
    res = []
    for flags in (0, bd.MSA_ONE_PASS_INDEX):
        dims = bd.make_dims(1, T, Hq, G, head_dim=d, index_dim=di, block_size=B, topk=k, flags=flags,
                            query_chunk=chunk)
        out = torch.empty((1, T, Hq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1, T, Hq), dtype=torch.float32, device="cuda")
        bidx = torch.full((1, T, G, k), -7, dtype=torch.int32, device="cuda") if with_bidx else None
        bd.msa_prefill(dims, inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.idx_q.cuda(), inp.idx_k.cuda(), out,
                       lse=lse, block_idx=bidx)
        torch.cuda.synchronize()
        res.append((out, lse, bidx))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    if with_bidx:
        assert torch.equal(res[0][2], res[1][2])


def test_one_pass_128k_headline_shape():
    """The 128K-token prefill shape (8 groups, d_idx 128, B 128, k 16): the
    whole selection equals the two-pass path's."""
    T, G, di, B, k = 131072, 8, 128, 128, 16
    say(f"[one-pass index 128K] T={T} G={G} B={B} k={k}")
    dev = torch.device("cuda:0")
    inp = inputs.make_prefill(T, G, G, 8, di, seed=5, device=dev)
    two = _index_topk(inp, B, k, 0)
    one = _index_topk(inp, B, k, bd.MSA_ONE_PASS_INDEX)
    assert torch.equal(one, two)

"""HIP graph capture of the library's calls.

The prefill, the decode and the allocation-free decode only launch kernels on
the caller's stream (no allocation, no memset, no host synchronisation), so a
caller can capture them into a graph.  Each graph here is replayed several
times with new inputs copied into its static tensors in between (eager work,
an eager call of the library and a synchronisation between replays), and
every replay must equal an eager call on the same inputs bit for bit: the
kernels are deterministic, so any difference means a replay read stale or
wrong memory."""
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


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("flags", [0, bd.MSA_ONE_PASS_INDEX])
def test_prefill_graph_replays(flags):
    """Prefill in three query chunks (T = 3000, B 64, k 8), selection and lse
    written to the caller's buffers; four replays on four seeds."""
    T, Hq, G, d, di, B, k = 3000, 16, 4, 128, 64, 64, 8
    say(f"[graph prefill] T={T} B={B} k={k} flags={flags}")
    dev = torch.device("cuda")
    dims = bd.make_dims(1, T, Hq, G, head_dim=d, index_dim=di, block_size=B, topk=k, flags=flags, query_chunk=1024)
    x = inputs.make_prefill(T, Hq, G, d, di, seed=0, device=dev)
    q, kk, v, iq, ik = (t.clone() for t in (x.q, x.k, x.v, x.idx_q, x.idx_k))
    out = torch.empty_like(q)
    lse = torch.empty((1, T, Hq), dtype=torch.float32, device=dev)
    bidx = torch.empty((1, T, G, k), dtype=torch.int32, device=dev)
    nws = bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    g = _capture(lambda: bd.msa_prefill(dims, q, kk, v, iq, ik, out, lse=lse, block_idx=bidx, workspace=ws))
    ws2 = torch.empty_like(ws)
    for seed in (1, 2, 3, 4):
        y = inputs.make_prefill(T, Hq, G, d, di, seed=seed, device=dev)
        for dst, src in ((q, y.q), (kk, y.k), (v, y.v), (iq, y.idx_q), (ik, y.idx_k)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), bidx.clone())
        out2, lse2, bidx2 = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(bidx)
        bd.msa_prefill(dims, y.q, y.k, y.v, y.idx_q, y.idx_k, out2, lse=lse2, block_idx=bidx2, workspace=ws2)
        torch.cuda.synchronize()
        assert torch.equal(got[2], bidx2), f"selection, seed {seed}"
        assert torch.equal(got[0], out2) and torch.equal(got[1], lse2), f"outputs, seed {seed}"


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays(noalloc):
    """Decode of 3 sequences (cache capacity 5000, B 64, k 8); the cache
    lengths change between replays, so each replay must read them from
    device memory."""
    b, L, Hq, G, d, di, B, k = 3, 5000, 16, 4, 128, 64, 64, 8
    say(f"[graph decode] batch={b} L={L} noalloc={noalloc}")
    dev = torch.device("cuda")
    dims = bd.make_dims(b, L, Hq, G, head_dim=d, index_dim=di, block_size=B, topk=k)
    x = inputs.make_decode(b, L, Hq, G, d, di, seed=0, device=dev, cache_lens=[L, 1, 2049])
    q, kc, vc, iq, ikc, lens = (t.clone() for t in (x.q, x.k_cache, x.v_cache, x.idx_q, x.idx_k_cache, x.cache_lens))
    out = torch.empty((b, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, Hq), dtype=torch.float32, device=dev)
    bidx = torch.empty((b, G, k), dtype=torch.int32, device=dev)
    ws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_DECODE, dims), dtype=torch.uint8, device=dev)

    def call(qq, kk_, vv, iqq, ikk, ll, o, ls, bi, w):
        if noalloc:
            bd.msa_decode_noalloc(dims, qq, kk_, vv, iqq, ikk, ll, o, lse=ls, block_idx=bi)
        else:
            bd.msa_decode(dims, qq, kk_, vv, iqq, ikk, ll, o, lse=ls, block_idx=bi, workspace=w)

    g = _capture(lambda: call(q, kc, vc, iq, ikc, lens, out, lse, bidx, ws))
    ws2 = torch.empty_like(ws)
    for seed, ln in ((1, [4999, 64, 129]), (2, [2, 5000, 777]), (3, [1, 1, 1]), (4, [3333, 2048, 4097])):
        y = inputs.make_decode(b, L, Hq, G, d, di, seed=seed, device=dev, cache_lens=ln)
        for dst, src in ((q, y.q), (kc, y.k_cache), (vc, y.v_cache), (iq, y.idx_q), (ikc, y.idx_k_cache),
                         (lens, y.cache_lens)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), bidx.clone())
        out2, lse2, bidx2 = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(bidx)
        call(y.q, y.k_cache, y.v_cache, y.idx_q, y.idx_k_cache, y.cache_lens, out2, lse2, bidx2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(got[2], bidx2), f"selection, lens {ln}"
        assert torch.equal(got[0], out2) and torch.equal(got[1], lse2), f"outputs, lens {ln}"


def test_indexer_kl_and_backward_graph_replays():
    """The indexer KL and the main-branch backward, each over three query
    chunks (T = 3000, B 64, k 8, chunks of 1024: the later chunks add onto
    d idx_k, dk and dv), captured into graphs and replayed on four seeds: each
    replay equals an eager call bit for bit."""
    T, Hq, G, d, di, B, k = 3000, 16, 4, 128, 64, 64, 8
    say(f"[graph KL + backward] T={T} B={B} k={k} chunks of 1024")
    dev = torch.device("cuda")
    dims = bd.make_dims(1, T, Hq, G, head_dim=d, index_dim=di, block_size=B, topk=k, query_chunk=1024)
    pdims = bd.make_dims(1, T, Hq, G, head_dim=d, index_dim=di, block_size=B, topk=k)

    def forward(y):
        out = torch.empty_like(y.q)
        lse = torch.empty((1, T, Hq), dtype=torch.float32, device=dev)
        bidx = torch.empty((1, T, G, k), dtype=torch.int32, device=dev)
        bd.msa_prefill(pdims, y.q, y.k, y.v, y.idx_q, y.idx_k, out, lse=lse, block_idx=bidx)
        gen = torch.Generator(device=dev).manual_seed(int(y.q[0, 0, 0, 0].float().item() * 1000) % 1000)
        dout = torch.randn(y.q.shape, generator=gen, device=dev).to(torch.bfloat16)
        return out, lse, bidx, dout

    x = inputs.make_prefill(T, Hq, G, d, di, seed=0, device=dev)
    out0, lse0, bidx0, dout0 = forward(x)
    st = [t.clone() for t in (x.q, x.k, x.v, x.idx_q, x.idx_k, out0, lse0, bidx0, dout0)]
    q, kk_, v, iq, ik, out, lse, bidx, dout = st
    kl = torch.empty((1, T, G), dtype=torch.float32, device=dev)
    diq = torch.empty((1, T, G, di), dtype=torch.float32, device=dev)
    dik = torch.empty((1, T, di), dtype=torch.float32, device=dev)
    dq = torch.empty((1, T, Hq, d), dtype=torch.float32, device=dev)
    dk = torch.empty((1, T, G, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    wk = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_INDEXER_KL, dims), dtype=torch.uint8, device=dev)
    wb = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_BACKWARD, dims), dtype=torch.uint8, device=dev)

    def both(ws_k, ws_b, outs):
        bd.msa_indexer_kl(dims, q, kk_, iq, ik, bidx, lse, outs[0], outs[1], outs[2], workspace=ws_k)
        bd.msa_prefill_backward(dims, q, kk_, v, out, lse, dout, bidx, outs[3], outs[4], outs[5], workspace=ws_b)

    g = _capture(lambda: both(wk, wb, (kl, diq, dik, dq, dk, dv)))
    wk2, wb2 = torch.empty_like(wk), torch.empty_like(wb)
    for seed in (1, 2, 3, 4):
        y = inputs.make_prefill(T, Hq, G, d, di, seed=seed, device=dev)
        o, l_, b_, do = forward(y)
        for dst, src in zip(st, (y.q, y.k, y.v, y.idx_q, y.idx_k, o, l_, b_, do)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (kl, diq, dik, dq, dk, dv)]
        ref = [torch.empty_like(t) for t in got]
        both(wk2, wb2, ref)
        torch.cuda.synchronize()
        for name, a_, b2 in zip(("kl", "d idx_q", "d idx_k", "dq", "dk", "dv"), got, ref):
            assert torch.equal(a_, b2), f"{name}, seed {seed}"

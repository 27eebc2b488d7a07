"""Library calls from several host threads at once.

Each thread has its own stream and workspaces and runs prefills and decodes
on its own inputs; calls on different streams with disjoint workspaces may
run concurrently, so every result must equal, bit for bit, the same call made
alone beforehand (the kernels are deterministic)."""
from concurrent.futures import ThreadPoolExecutor

import pytest
import torch

from block_sparse_long_02_amd import binding as bd
from block_sparse_long_02_amd import inputs
from gpu_common import say

pytestmark = pytest.mark.gpu

T, HQ, G, D, DI, B, K = 1500, 16, 4, 128, 64, 64, 6
L = 3000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.load_library()


def _job(seed, stream):
    """One thread's work on its stream: a prefill and a decode of its own
    inputs, into fresh outputs and workspaces."""
    dev = torch.device("cuda")
    with torch.cuda.stream(stream):
        x = inputs.make_prefill(T, HQ, G, D, DI, seed=seed, device=dev)
        pd = bd.make_dims(1, T, HQ, G, index_dim=DI, block_size=B, topk=K, query_chunk=512)
        out = torch.empty_like(x.q)
        lse = torch.empty((1, T, HQ), dtype=torch.float32, device=dev)
        bidx = torch.empty((1, T, G, K), dtype=torch.int32, device=dev)
        pws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, pd), dtype=torch.uint8, device=dev)
        bd.msa_prefill(pd, x.q, x.k, x.v, x.idx_q, x.idx_k, out, lse=lse, block_idx=bidx, workspace=pws)
        y = inputs.make_decode(3, L, HQ, G, D, DI, seed=seed + 1, device=dev, cache_lens=[L, 1 + seed % 700, 2049])
        dd = bd.make_dims(3, L, HQ, G, index_dim=DI, block_size=B, topk=K)
        dout = torch.empty((3, HQ, D), dtype=torch.bfloat16, device=dev)
        dws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_DECODE, dd), dtype=torch.uint8, device=dev)
        bd.msa_decode(dd, y.q, y.k_cache, y.v_cache, y.idx_q, y.idx_k_cache, y.cache_lens, dout, workspace=dws)
    stream.synchronize()
    return out, lse, bidx, dout


def test_concurrent_calls_from_host_threads():
    seeds = list(range(11, 19))
    say(f"[threads] {len(seeds)} jobs, each alone, then on 8 threads at once")
    alone = [_job(sd, torch.cuda.Stream()) for sd in seeds]
    streams = [torch.cuda.Stream() for _ in seeds]
    for rnd in range(3):
        with ThreadPoolExecutor(len(seeds)) as ex:
            together = list(ex.map(_job, seeds, streams))
        torch.cuda.synchronize()
        for sd, a, b in zip(seeds, alone, together):
            for name, u, v in zip(("out", "lse", "block_idx", "decode out"), a, b):
                assert torch.equal(u, v), f"round {rnd}, seed {sd}: {name}"

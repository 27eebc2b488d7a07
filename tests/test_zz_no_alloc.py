"""The allocation-free decode entry point (msa_decode_noalloc), called through
the C ABI, against msa_decode with a caller workspace: the same kernels, so
outputs, lse and selections must be bitwise equal.  Two calls in a row, the
second smaller, both after the array already holds another call's contents;
a shape whose workspace exceeds the array is rejected before any launch."""
import numpy as np
import pytest
import torch

from block_sparse_long_02_amd import binding as bd
from block_sparse_long_02_amd import inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _both(dec, dims):
    b, Hq, d = dec.q.shape
    G = dec.k_cache.shape[2]
    k = dims.topk
    res = []
    for fn in (bd.msa_decode, bd.msa_decode_noalloc):
        out = torch.full((b, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((b, Hq), float("nan"), dtype=torch.float32, device="cuda")
        bidx = torch.full((b, G, k), -7, dtype=torch.int32, device="cuda")
        fn(dims, dec.q, dec.k_cache, dec.v_cache, dec.idx_q, dec.idx_k_cache, dec.cache_lens, out,
           lse=lse, block_idx=bidx)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu(), bidx.cpu()))
    return res


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    lib = bd.load_library()
    assert lib.msa_decode_noalloc_limit() == 32 << 20
    dev = torch.device("cuda")
    cases = [
        # (batch, L, lens, B, k): the second call is the smaller one
        (8, 1 << 18, [1 << 18, 200001, 777, 1 << 17, 65537, 2, 4096, 99999], 128, 16),
        (3, 5000, [5000, 1, 2049], 64, 6),
    ]
    for batch, L, lens, B, k in cases:
        _say(f"[decode noalloc] batch={batch} L={L} B={B} k={k}")
        dec = inputs.make_decode(batch, L, 64, 8, 128, 128, seed=L % 97, device=dev, cache_lens=lens)
        dims = bd.make_dims(batch, L, 64, 8, index_dim=128, block_size=B, topk=k)
        need = bd.msa_workspace_bytes(bd.MSA_OP_DECODE, dims)
        assert 0 < need <= lib.msa_decode_noalloc_limit()
        (o1, l1, b1), (o2, l2, b2) = _both(dec, dims)
        assert torch.equal(b1, b2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
        assert not torch.isnan(o2.float()).any()
        del dec


def test_noalloc_decode_rejects_shapes_beyond_its_array():
    dev = torch.device("cuda")
    batch, L = 2, 1 << 20
    dims = bd.make_dims(batch, L, 64, 8, index_dim=128, block_size=128, topk=16, flags=bd.MSA_DENSE)
    assert bd.msa_workspace_bytes(bd.MSA_OP_DECODE, dims) > (32 << 20)
    q = torch.zeros((batch, 64, 128), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((batch, 1, 8, 128), dtype=torch.bfloat16, device=dev).expand(batch, L, 8, 128)
    lens = torch.full((batch,), L, dtype=torch.int32, device=dev)
    out = torch.zeros_like(q)
    lib = bd.load_library()
    import ctypes
    st = lib.msa_decode_noalloc(ctypes.byref(dims), q.data_ptr(), kv.data_ptr(), kv.data_ptr(), None, None,
                                lens.data_ptr(), out.data_ptr(), None, None, None)
    assert st == bd.MSA_ERR_WORKSPACE

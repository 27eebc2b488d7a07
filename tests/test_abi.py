"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/msa.h declares, and rejects bad arguments with the
documented status before touching the device.  Pointers passed here are fake
addresses that the library never dereferences (validation fails first)."""
import ctypes
import os
import re

import pytest

from block_sparse_long_02_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("libmsa.so not built")
    return bd.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(bd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.msa_abi_version() == 1


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define (MSA_[A-Z_]+) (0x[0-9a-f]+|\d+)u?", src))
    for name, val in consts.items():
        assert getattr(bd, name) == int(val, 0), name


def test_dims_struct_layout():
    # the ctypes mirror must match the C struct: 12 x 4-byte fields
    assert ctypes.sizeof(bd.msa_dims) == 48
    assert bd.msa_dims.flags.offset == 36 and bd.msa_dims.query_chunk.offset == 40


def test_status_strings(lib):
    for st in range(0, 6):
        s = lib.msa_status_string(st).decode()
        assert s.startswith("MSA_")
    assert lib.msa_status_string(99).decode() == "unknown msa status"


def _dims(**kw):
    base = dict(batch=1, seqlen=2048, num_q_heads=16, num_kv_heads=4, head_dim=128, index_dim=64,
                block_size=128, topk=4)
    base.update(kw)
    b = base
    return bd.make_dims(b.pop("batch"), b.pop("seqlen"), b.pop("num_q_heads"), b.pop("num_kv_heads"), **b)


def _ws(lib, op, d):
    return lib.msa_workspace_bytes(op, ctypes.byref(d))


BAD = ctypes.c_size_t(-1).value


def test_workspace_bytes(lib):
    d = _dims()
    n_pre = _ws(lib, bd.MSA_OP_PREFILL, d)
    n_idx = _ws(lib, bd.MSA_OP_INDEX_TOPK, d)
    n_dec = _ws(lib, bd.MSA_OP_DECODE, d)
    assert 0 < n_idx < n_pre != BAD and n_dec not in (0, BAD)
    assert _ws(lib, bd.MSA_OP_PREFILL, _dims(flags=bd.MSA_DENSE)) == 0
    assert _ws(lib, 7, d) == BAD
    assert lib.msa_workspace_bytes(bd.MSA_OP_PREFILL, None) == BAD
    # a forced small chunk shrinks the workspace
    assert _ws(lib, bd.MSA_OP_PREFILL, _dims(query_chunk=256)) < n_pre
    # 128K and 1M prefill, 64 q heads / 8 groups: default chunking keeps the workspace near 80 GiB
    big = _dims(seqlen=131072, num_q_heads=64, num_kv_heads=8, index_dim=128, topk=16)
    assert _ws(lib, bd.MSA_OP_PREFILL, big) < (81 << 30)
    big1m = _dims(seqlen=1 << 20, num_q_heads=64, num_kv_heads=8, index_dim=128, topk=16)
    assert _ws(lib, bd.MSA_OP_PREFILL, big1m) < (81 << 30)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, bd.MSA_ERR_INVALID_ARG),
    ("seqlen", -1, bd.MSA_ERR_INVALID_ARG),
    ("num_q_heads", 10, bd.MSA_ERR_INVALID_ARG),      # 10 % 4 != 0
    ("topk", 0, bd.MSA_ERR_INVALID_ARG),
    ("reserved", 1, bd.MSA_ERR_INVALID_ARG),
    ("flags", 0x3, bd.MSA_ERR_INVALID_ARG),            # dense and given together
    ("flags", 0x8, bd.MSA_ERR_INVALID_ARG),            # unknown flag
    ("flags", 0x5, bd.MSA_ERR_INVALID_ARG),            # sink with dense
    ("flags", 0x6, bd.MSA_ERR_INVALID_ARG),            # sink with given indices
    ("query_chunk", 100, bd.MSA_ERR_INVALID_ARG),      # not a multiple of block_size
    ("softmax_scale", float("nan"), bd.MSA_ERR_INVALID_ARG),
    ("head_dim", 64, bd.MSA_ERR_UNSUPPORTED),
    ("index_dim", 96, bd.MSA_ERR_UNSUPPORTED),
    ("block_size", 16, bd.MSA_ERR_UNSUPPORTED),
    ("block_size", 256, bd.MSA_ERR_UNSUPPORTED),
])
def test_prefill_rejects_bad_dims(lib, field, value, status):
    d = _dims()
    setattr(d, field, value)
    fake = 0x10000
    st = lib.msa_prefill(ctypes.byref(d), fake, fake, fake, fake, fake, fake, None, None,
                         fake, 1 << 40, None)
    assert st == status
    assert _ws(lib, bd.MSA_OP_PREFILL, d) == BAD


def test_decode_head_limit(lib):
    d = _dims(num_q_heads=68, num_kv_heads=2)  # 34 heads per group > 16
    assert _ws(lib, bd.MSA_OP_DECODE, d) == BAD
    assert _ws(lib, bd.MSA_OP_PREFILL, d) != BAD
    fake = 0x10000
    st = lib.msa_decode(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None, None,
                        fake, 1 << 40, None)
    assert st == bd.MSA_ERR_UNSUPPORTED


def test_null_misaligned_and_workspace(lib):
    d = _dims()
    fake = 0x10000
    need = _ws(lib, bd.MSA_OP_PREFILL, d)
    call = lambda *a: lib.msa_prefill(ctypes.byref(d), *a)
    # null q
    assert call(None, fake, fake, fake, fake, fake, None, None, fake, need, None) == bd.MSA_ERR_INVALID_ARG
    # null idx without DENSE/GIVEN
    assert call(fake, fake, fake, None, fake, fake, None, None, fake, need, None) == bd.MSA_ERR_INVALID_ARG
    # misaligned bf16 tensor
    assert call(fake + 2, fake, fake, fake, fake, fake, None, None, fake, need, None) == bd.MSA_ERR_ALIGNMENT
    # misaligned workspace
    assert call(fake, fake, fake, fake, fake, fake, None, None, fake + 16, need, None) == bd.MSA_ERR_ALIGNMENT
    # workspace too small / missing
    assert call(fake, fake, fake, fake, fake, fake, None, None, fake, need - 1, None) == bd.MSA_ERR_WORKSPACE
    assert call(fake, fake, fake, fake, fake, fake, None, None, None, need, None) == bd.MSA_ERR_INVALID_ARG
    # dense mode forbids block_idx; given mode needs it
    dd = _dims(flags=bd.MSA_DENSE)
    assert lib.msa_prefill(ctypes.byref(dd), fake, fake, fake, None, None, fake, None, fake, None, 0,
                           None) == bd.MSA_ERR_INVALID_ARG
    dg = _dims(flags=bd.MSA_GIVEN_INDICES)
    ng = _ws(lib, bd.MSA_OP_PREFILL, dg)
    assert lib.msa_prefill(ctypes.byref(dg), fake, fake, fake, None, None, fake, None, None, fake, ng,
                           None) == bd.MSA_ERR_INVALID_ARG
    # index_topk takes no flags and needs block_idx
    assert lib.msa_index_topk(ctypes.byref(dd), fake, fake, fake, fake, 1 << 40, None) == bd.MSA_ERR_INVALID_ARG
    ni = _ws(lib, bd.MSA_OP_INDEX_TOPK, d)
    assert lib.msa_index_topk(ctypes.byref(d), fake, fake, None, fake, ni, None) == bd.MSA_ERR_INVALID_ARG
    # decode: null cache_lens
    nd = _ws(lib, bd.MSA_OP_DECODE, d)
    assert lib.msa_decode(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, None, None, fake, nd,
                          None) == bd.MSA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import torch
    d = _dims(seqlen=256)
    q = torch.zeros(1, 256, 16, 128, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        bd.msa_prefill(d, q, q, q, q, q, q)


def test_profile_calls_without_gpu_work(lib):
    """Profiling with no recorded calls: every stage reports zero launches;
    bad arguments are rejected and leave profiling off."""
    assert lib.msa_profile_begin() == bd.MSA_OK
    arr = (bd.msa_stage_time * bd.MSA_STAGE_COUNT)()
    n = ctypes.c_int32(-1)
    assert lib.msa_profile_end(arr, bd.MSA_STAGE_COUNT, ctypes.byref(n)) == bd.MSA_OK
    assert n.value == bd.MSA_STAGE_COUNT
    assert [r.stage for r in arr] == list(range(bd.MSA_STAGE_COUNT))
    assert all(r.launches == 0 and r.total_ms == 0.0 for r in arr)
    assert lib.msa_profile_end(arr, bd.MSA_STAGE_COUNT - 1, ctypes.byref(n)) == bd.MSA_ERR_INVALID_ARG
    assert lib.msa_profile_end(None, bd.MSA_STAGE_COUNT, ctypes.byref(n)) == bd.MSA_ERR_INVALID_ARG
    names = [lib.msa_stage_name(i).decode() for i in range(bd.MSA_STAGE_COUNT)]
    assert len(set(names)) == bd.MSA_STAGE_COUNT and "kv_outer_kernel" in names
    assert lib.msa_stage_name(99).decode() == "unknown stage"


def test_sink_flag_accepted_with_the_index_branch(lib):
    d = bd.make_dims(1, 4096, 16, 4, index_dim=64, block_size=64, topk=8, flags=bd.MSA_FORCE_SINK)
    plain = bd.make_dims(1, 4096, 16, 4, index_dim=64, block_size=64, topk=8)
    for op in (bd.MSA_OP_INDEX_TOPK, bd.MSA_OP_PREFILL, bd.MSA_OP_DECODE):
        assert lib.msa_workspace_bytes(op, ctypes.byref(d)) == lib.msa_workspace_bytes(op, ctypes.byref(plain))


def test_indexer_kl_shape_limits(lib):
    ok = bd.make_dims(1, 2048, 16, 4, index_dim=64, block_size=64, topk=8)
    assert lib.msa_workspace_bytes(bd.MSA_OP_INDEXER_KL, ctypes.byref(ok)) > 0
    # any head ratio the prefill takes: the heads are visited in turn per entry
    for hq, g in ((12, 4), (64, 1), (128, 1)):
        d = bd.make_dims(1, 2048, hq, g, index_dim=64, block_size=64, topk=8)
        assert lib.msa_workspace_bytes(bd.MSA_OP_INDEXER_KL, ctypes.byref(d)) > 0, (hq, g)
    r256 = bd.make_dims(1, 2048, 256, 1, index_dim=64, block_size=64, topk=8)  # beyond the prefill's 128
    fl = bd.make_dims(1, 2048, 16, 4, index_dim=64, block_size=64, topk=8, flags=bd.MSA_DENSE)
    for d in (r256, fl):
        assert lib.msa_workspace_bytes(bd.MSA_OP_INDEXER_KL, ctypes.byref(d)) == ctypes.c_size_t(-1).value



def test_backward_shape_limits(lib):
    ok = bd.make_dims(1, 2048, 12, 4, index_dim=64, block_size=64, topk=8)  # R = 3 is fine
    assert lib.msa_workspace_bytes(bd.MSA_OP_BACKWARD, ctypes.byref(ok)) > 0
    for fl in (bd.MSA_DENSE, bd.MSA_GIVEN_INDICES, bd.MSA_FORCE_SINK):
        d = bd.make_dims(1, 2048, 16, 4, index_dim=64, block_size=64, topk=8, flags=fl)
        assert lib.msa_workspace_bytes(bd.MSA_OP_BACKWARD, ctypes.byref(d)) == ctypes.c_size_t(-1).value
    # the selection is an input: null pointers and a short workspace are rejected before any launch
    d = bd.make_dims(1, 256, 8, 2, index_dim=64, block_size=64, topk=2)
    need = lib.msa_workspace_bytes(bd.MSA_OP_BACKWARD, ctypes.byref(d))
    buf = ctypes.create_string_buffer(1024)
    addr = (ctypes.addressof(buf) + 255) // 256 * 256  # every pointer 256-byte aligned
    p = ctypes.c_void_p(addr)
    args = [p] * 10
    assert lib.msa_prefill_backward(ctypes.byref(d), *args[:6], None, *args[7:], p, need, None) == \
        bd.MSA_ERR_INVALID_ARG
    assert lib.msa_prefill_backward(ctypes.byref(d), *args, p, need - 1, None) == bd.MSA_ERR_WORKSPACE


def test_backward_workspace_fits_128k_in_one_chunk(lib):
    d = bd.make_dims(1, 131072, 64, 8, index_dim=128, block_size=128, topk=16)
    ws = lib.msa_workspace_bytes(bd.MSA_OP_BACKWARD, ctypes.byref(d))
    assert 0 < ws <= 64 << 30


def test_index_scores_rejects_bad_ranges(lib):
    """msa_index_scores validates the token range, the row strides and the
    alignment before any launch."""
    d = _dims()                                   # T 2048, B 128: L(2047) = 15
    fake = 0x10000
    call = lambda t0, t1, rs, sm, sbs, sc=fake: lib.msa_index_scores(ctypes.byref(d), fake, fake, sc, t0, t1, rs,
                                                                      sm, sbs, None)
    assert call(0, 0, 16, None, 0) == bd.MSA_ERR_INVALID_ARG        # empty range
    assert call(-1, 100, 16, None, 0) == bd.MSA_ERR_INVALID_ARG
    assert call(0, 2049, 16, None, 0) == bd.MSA_ERR_INVALID_ARG     # past T
    assert call(0, 2048, 12, None, 0) == bd.MSA_ERR_INVALID_ARG     # row_stride < L(t1 - 1)
    assert call(0, 2048, 18, None, 0) == bd.MSA_ERR_INVALID_ARG     # not a multiple of 4
    assert call(0, 2048, 16, fake, 0) == bd.MSA_ERR_INVALID_ARG     # sb_stride < ceil(15 / 16)
    assert call(0, 2048, 16, None, 0, sc=fake + 4) == bd.MSA_ERR_ALIGNMENT
    assert call(0, 2048, 16, fake + 2, 1) == bd.MSA_ERR_ALIGNMENT
    dd = _dims(flags=bd.MSA_DENSE)
    assert lib.msa_index_scores(ctypes.byref(dd), fake, fake, fake, 0, 2048, 16, None, 0, None) == \
        bd.MSA_ERR_INVALID_ARG


def test_check_lens_flag_is_decode_only(lib):
    """MSA_CHECK_LENS is accepted by decode (same workspace) and rejected by
    every prefill-shaped operation and by the allocation-free decode."""
    plain = _dims()
    chk = _dims(flags=bd.MSA_CHECK_LENS)
    assert _ws(lib, bd.MSA_OP_DECODE, chk) == _ws(lib, bd.MSA_OP_DECODE, plain)
    for op in (bd.MSA_OP_INDEX_TOPK, bd.MSA_OP_PREFILL, bd.MSA_OP_INDEXER_KL, bd.MSA_OP_BACKWARD):
        assert _ws(lib, op, chk) == BAD
    fake = 0x10000
    assert lib.msa_prefill(ctypes.byref(chk), fake, fake, fake, fake, fake, fake, None, None, fake, 1 << 40,
                           None) == bd.MSA_ERR_INVALID_ARG
    assert lib.msa_decode_noalloc(ctypes.byref(chk), fake, fake, fake, fake, fake, fake, fake, None, None,
                                  None) == bd.MSA_ERR_INVALID_ARG


def test_one_pass_index_flag(lib):
    """MSA_ONE_PASS_INDEX: msa_index_topk needs no workspace and prefill a
    smaller one (no score table); topk above 17 is unsupported; the flag is
    rejected by decode, the KL loss, the backward, msa_index_scores and
    together with MSA_DENSE or MSA_GIVEN_INDICES."""
    one = bd.MSA_ONE_PASS_INDEX
    plain = _dims(topk=16)
    fused = _dims(topk=16, flags=one)
    assert _ws(lib, bd.MSA_OP_INDEX_TOPK, fused) == 0 < _ws(lib, bd.MSA_OP_INDEX_TOPK, plain)
    assert 0 < _ws(lib, bd.MSA_OP_PREFILL, fused) < _ws(lib, bd.MSA_OP_PREFILL, plain)
    assert _ws(lib, bd.MSA_OP_PREFILL, _dims(topk=16, flags=one | bd.MSA_FORCE_SINK)) == \
        _ws(lib, bd.MSA_OP_PREFILL, fused)
    # at 128K the table is most of the index branch's share of the prefill workspace
    big = dict(seqlen=131072, num_q_heads=64, num_kv_heads=8, index_dim=128, topk=16)
    assert _ws(lib, bd.MSA_OP_INDEX_TOPK, _dims(**big, flags=one)) == 0
    assert _ws(lib, bd.MSA_OP_INDEX_TOPK, _dims(**big)) > (4 << 30)
    assert _ws(lib, bd.MSA_OP_INDEX_TOPK, _dims(topk=17, flags=one)) == 0
    assert _ws(lib, bd.MSA_OP_INDEX_TOPK, _dims(topk=18, flags=one)) == BAD
    for op in (bd.MSA_OP_DECODE, bd.MSA_OP_INDEXER_KL, bd.MSA_OP_BACKWARD):
        assert _ws(lib, op, fused) == BAD
    for fl in (bd.MSA_DENSE, bd.MSA_GIVEN_INDICES, bd.MSA_CHECK_LENS):
        assert _ws(lib, bd.MSA_OP_PREFILL, _dims(topk=16, flags=one | fl)) == BAD
    fake = 0x10000
    assert lib.msa_index_topk(ctypes.byref(_dims(topk=18, flags=one)), fake, fake, fake, None, 0, None) == \
        bd.MSA_ERR_UNSUPPORTED
    assert lib.msa_index_scores(ctypes.byref(fused), fake, fake, fake, 0, 2048, 16, None, 0, None) == \
        bd.MSA_ERR_INVALID_ARG
    assert lib.msa_decode_noalloc(ctypes.byref(fused), fake, fake, fake, fake, fake, fake, fake, None, None,
                                  None) == bd.MSA_ERR_INVALID_ARG


def test_host_validation_from_many_threads(lib):
    """The host side is thread-safe: 16 threads sizing workspaces and having
    invalid calls rejected at the same time get the answers one thread gets."""
    from concurrent.futures import ThreadPoolExecutor
    shapes = [_dims(), _dims(topk=16, flags=bd.MSA_ONE_PASS_INDEX), _dims(seqlen=131072, num_q_heads=64,
              num_kv_heads=8, index_dim=128, topk=16), _dims(flags=bd.MSA_DENSE), _dims(query_chunk=256)]
    ops = (bd.MSA_OP_INDEX_TOPK, bd.MSA_OP_PREFILL, bd.MSA_OP_DECODE, bd.MSA_OP_INDEXER_KL, bd.MSA_OP_BACKWARD)
    want = [[_ws(lib, op, d) for op in ops] for d in shapes]
    bad = _dims(num_q_heads=10)
    fake = 0x10000

    def work(i):
        out = []
        for _ in range(200):
            out.append([[_ws(lib, op, d) for op in ops] for d in shapes] == want)
            out.append(lib.msa_prefill(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None, None, fake,
                                       1 << 40, None) == bd.MSA_ERR_INVALID_ARG)
        return all(out)

    with ThreadPoolExecutor(16) as ex:
        assert all(ex.map(work, range(16)))

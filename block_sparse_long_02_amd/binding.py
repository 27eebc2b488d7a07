"""Thin ctypes binding of libmsa.so (include/msa.h).

The functions carry the C ABI's names and only marshal arguments: they check
that each torch tensor is a contiguous device tensor of the dtype and shape
the ABI documents, pass its data pointer, take the current HIP stream, and
allocate the workspace with torch when the caller gives none.  Every step of
the computation runs in the HIP kernels of libmsa.so; there is no fallback,
and a missing library raises at the first call.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = 1
MSA_ERR_UNSUPPORTED = 2
MSA_ERR_ALIGNMENT = 3
MSA_ERR_WORKSPACE = 4
MSA_ERR_HIP = 5

MSA_DENSE = 0x1
MSA_GIVEN_INDICES = 0x2
MSA_FORCE_SINK = 0x4
MSA_CHECK_LENS = 0x8
MSA_ONE_PASS_INDEX = 0x10

MSA_OP_INDEX_TOPK = 0
MSA_OP_PREFILL = 1
MSA_OP_DECODE = 2
MSA_OP_INDEXER_KL = 3
MSA_OP_BACKWARD = 4

MSA_STAGE_INDEX_PREFILL = 0
MSA_STAGE_TOPK_PREFILL = 1
MSA_STAGE_BLOCK_LISTS = 2
MSA_STAGE_KV_OUTER = 3
MSA_STAGE_QUERY_MAJOR = 4
MSA_STAGE_QUERY_MAJOR_DENSE = 5
MSA_STAGE_INDEX_DECODE = 6
MSA_STAGE_TOPK_DECODE = 7
MSA_STAGE_DECODE_ATTN = 8
MSA_STAGE_DECODE_COMBINE = 9
MSA_STAGE_INDEXER_KL = 10
MSA_STAGE_BWD_PREP = 11
MSA_STAGE_BWD_LISTS = 12
MSA_STAGE_BWD_MERGE = 13
MSA_STAGE_INDEX_ONE_PASS = 14
MSA_STAGE_COUNT = 15

EXPORTED = ("msa_index_scores", "msa_index_topk", "msa_prefill", "msa_decode", "msa_decode_noalloc",
            "msa_decode_noalloc_limit", "msa_workspace_bytes",
            "msa_status_string", "msa_last_hip_error", "msa_abi_version", "msa_profile_begin",
            "msa_profile_end", "msa_stage_name", "msa_indexer_kl", "msa_prefill_backward")


class msa_stage_time(ctypes.Structure):
    _fields_ = [("stage", ctypes.c_int32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class msa_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("query_chunk", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def make_dims(batch, seqlen, num_q_heads, num_kv_heads, *, head_dim=128, index_dim=128,
              block_size=128, topk=16, softmax_scale=0.0, flags=0, query_chunk=0) -> msa_dims:
    return msa_dims(batch, seqlen, num_q_heads, num_kv_heads, head_dim, index_dim, block_size,
                    topk, softmax_scale, flags, query_chunk, 0)


class MSAError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{text} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmsa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmsa.so not found at {path}; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    pd = ctypes.POINTER(msa_dims)
    lib.msa_index_scores.argtypes = [pd, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp,
                                      ctypes.c_int32, vp]
    lib.msa_index_scores.restype = i32
    lib.msa_index_topk.argtypes = [pd, vp, vp, vp, vp, sz, vp]
    lib.msa_index_topk.restype = i32
    lib.msa_prefill.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_prefill.restype = i32
    lib.msa_decode.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_decode.restype = i32
    lib.msa_decode_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.msa_decode_noalloc.restype = i32
    lib.msa_decode_noalloc_limit.argtypes = []
    lib.msa_decode_noalloc_limit.restype = sz
    lib.msa_workspace_bytes.argtypes = [i32, pd]
    lib.msa_workspace_bytes.restype = sz
    lib.msa_status_string.argtypes = [i32]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_last_hip_error.argtypes = []
    lib.msa_last_hip_error.restype = ctypes.c_char_p
    lib.msa_abi_version.argtypes = []
    lib.msa_abi_version.restype = i32
    lib.msa_indexer_kl.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_indexer_kl.restype = i32
    lib.msa_prefill_backward.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_prefill_backward.restype = i32
    lib.msa_profile_begin.argtypes = []
    lib.msa_profile_begin.restype = i32
    lib.msa_profile_end.argtypes = [ctypes.POINTER(msa_stage_time), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.msa_profile_end.restype = i32
    lib.msa_stage_name.argtypes = [ctypes.c_int32]
    lib.msa_stage_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t, name, dtype, shape, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(lib, status):
    if status != MSA_OK:
        text = lib.msa_status_string(status).decode()
        if status == MSA_ERR_HIP:
            text += ": " + lib.msa_last_hip_error().decode()
        raise MSAError(status, text)


def msa_abi_version() -> int:
    return load_library().msa_abi_version()


def msa_status_string(status: int) -> str:
    return load_library().msa_status_string(status).decode()


def msa_workspace_bytes(op: int, dims: msa_dims) -> int:
    """Workspace bytes for op; raises MSAError(INVALID_ARG) on invalid dims."""
    n = load_library().msa_workspace_bytes(op, ctypes.byref(dims))
    if n == ctypes.c_size_t(-1).value:
        raise MSAError(MSA_ERR_INVALID_ARG, "invalid or unsupported dims")
    return n


def _workspace(op, dims, workspace, device):
    need = msa_workspace_bytes(op, dims)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device.type != "cuda":
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    return workspace.data_ptr(), workspace.numel()


def scores_row_stride(dims: msa_dims, t1: int) -> int:
    """Smallest valid row_stride of msa_index_scores for query tokens < t1."""
    L = (t1 - 1) // dims.block_size
    return max(4, (L + 3) // 4 * 4)


def msa_index_scores(dims: msa_dims, idx_q, idx_k, scores, t0: int, t1: int, row_stride: int,
                     superblock_max=None, stream=None):
    lib = load_library()
    b, T, G, di = dims.batch, dims.seqlen, dims.num_kv_heads, dims.index_dim
    p_iq = _ptr(idx_q, "idx_q", torch.bfloat16, (b, T, G, di))
    p_ik = _ptr(idx_k, "idx_k", torch.bfloat16, (b, T, di))
    p_s = _ptr(scores, "scores", torch.float32, (b, t1 - t0, G, row_stride))
    sb_stride = 0
    if superblock_max is not None:
        sb_stride = int(superblock_max.shape[-1])
    p_sm = _ptr(superblock_max, "superblock_max", torch.float32, (b, t1 - t0, G, sb_stride), optional=True)
    _check(lib, lib.msa_index_scores(ctypes.byref(dims), p_iq, p_ik, p_s, t0, t1, row_stride, p_sm, sb_stride,
                                     _stream(stream)))
    return scores


def msa_index_topk(dims: msa_dims, idx_q, idx_k, block_idx, workspace=None, stream=None):
    lib = load_library()
    b, T, G, di, k = dims.batch, dims.seqlen, dims.num_kv_heads, dims.index_dim, dims.topk
    p_iq = _ptr(idx_q, "idx_q", torch.bfloat16, (b, T, G, di))
    p_ik = _ptr(idx_k, "idx_k", torch.bfloat16, (b, T, di))
    p_bi = _ptr(block_idx, "block_idx", torch.int32, (b, T, G, k))
    ws, nws = _workspace(MSA_OP_INDEX_TOPK, dims, workspace, idx_q.device)
    _check(lib, lib.msa_index_topk(ctypes.byref(dims), p_iq, p_ik, p_bi, ws, nws, _stream(stream)))
    return block_idx


def msa_prefill(dims: msa_dims, q, k, v, idx_q, idx_k, out, lse=None, block_idx=None,
                workspace=None, stream=None):
    lib = load_library()
    b, T, Hq, G, d, di, kk = (dims.batch, dims.seqlen, dims.num_q_heads, dims.num_kv_heads,
                             dims.head_dim, dims.index_dim, dims.topk)
    idx_needed = not (dims.flags & (MSA_DENSE | MSA_GIVEN_INDICES))
    p_q = _ptr(q, "q", torch.bfloat16, (b, T, Hq, d))
    p_k = _ptr(k, "k", torch.bfloat16, (b, T, G, d))
    p_v = _ptr(v, "v", torch.bfloat16, (b, T, G, d))
    p_iq = _ptr(idx_q, "idx_q", torch.bfloat16, (b, T, G, di), optional=not idx_needed)
    p_ik = _ptr(idx_k, "idx_k", torch.bfloat16, (b, T, di), optional=not idx_needed)
    p_o = _ptr(out, "out", torch.bfloat16, (b, T, Hq, d))
    p_l = _ptr(lse, "lse", torch.float32, (b, T, Hq), optional=True)
    p_bi = _ptr(block_idx, "block_idx", torch.int32, (b, T, G, kk), optional=True)
    ws, nws = _workspace(MSA_OP_PREFILL, dims, workspace, q.device)
    _check(lib, lib.msa_prefill(ctypes.byref(dims), p_q, p_k, p_v, p_iq, p_ik, p_o, p_l, p_bi,
                                ws, nws, _stream(stream)))
    return out


def msa_indexer_kl(dims: msa_dims, q, k, idx_q, idx_k, block_idx, lse, kl, d_idx_q, d_idx_k,
                   workspace=None, stream=None):
    """Indexer KL loss per (token, group) row and its gradient into idx_q and
    idx_k (see include/msa.h); outputs are written into kl, d_idx_q, d_idx_k."""
    lib = load_library()
    b, T, Hq, G, d, di, kk = (dims.batch, dims.seqlen, dims.num_q_heads, dims.num_kv_heads,
                             dims.head_dim, dims.index_dim, dims.topk)
    p_q = _ptr(q, "q", torch.bfloat16, (b, T, Hq, d))
    p_k = _ptr(k, "k", torch.bfloat16, (b, T, G, d))
    p_iq = _ptr(idx_q, "idx_q", torch.bfloat16, (b, T, G, di))
    p_ik = _ptr(idx_k, "idx_k", torch.bfloat16, (b, T, di))
    p_bi = _ptr(block_idx, "block_idx", torch.int32, (b, T, G, kk))
    p_l = _ptr(lse, "lse", torch.float32, (b, T, Hq))
    p_kl = _ptr(kl, "kl", torch.float32, (b, T, G))
    p_dq = _ptr(d_idx_q, "d_idx_q", torch.float32, (b, T, G, di))
    p_dk = _ptr(d_idx_k, "d_idx_k", torch.float32, (b, T, di))
    ws, nws = _workspace(MSA_OP_INDEXER_KL, dims, workspace, q.device)
    _check(lib, lib.msa_indexer_kl(ctypes.byref(dims), p_q, p_k, p_iq, p_ik, p_bi, p_l, p_kl, p_dq, p_dk,
                                   ws, nws, _stream(stream)))
    return kl, d_idx_q, d_idx_k


def msa_prefill_backward(dims: msa_dims, q, k, v, out, lse, dout, block_idx, dq, dk, dv,
                         workspace=None, stream=None):
    """Gradient of the main branch's output into q, k and v with the selection
    held fixed (see include/msa.h); written into dq, dk, dv (fp32)."""
    lib = load_library()
    b, T, Hq, G, d, kk = (dims.batch, dims.seqlen, dims.num_q_heads, dims.num_kv_heads, dims.head_dim,
                          dims.topk)
    p_q = _ptr(q, "q", torch.bfloat16, (b, T, Hq, d))
    p_k = _ptr(k, "k", torch.bfloat16, (b, T, G, d))
    p_v = _ptr(v, "v", torch.bfloat16, (b, T, G, d))
    p_o = _ptr(out, "out", torch.bfloat16, (b, T, Hq, d))
    p_l = _ptr(lse, "lse", torch.float32, (b, T, Hq))
    p_do = _ptr(dout, "dout", torch.bfloat16, (b, T, Hq, d))
    p_bi = _ptr(block_idx, "block_idx", torch.int32, (b, T, G, kk))
    p_dq = _ptr(dq, "dq", torch.float32, (b, T, Hq, d))
    p_dk = _ptr(dk, "dk", torch.float32, (b, T, G, d))
    p_dv = _ptr(dv, "dv", torch.float32, (b, T, G, d))
    ws, nws = _workspace(MSA_OP_BACKWARD, dims, workspace, q.device)
    _check(lib, lib.msa_prefill_backward(ctypes.byref(dims), p_q, p_k, p_v, p_o, p_l, p_do, p_bi, p_dq, p_dk,
                                         p_dv, ws, nws, _stream(stream)))
    return dq, dk, dv


def msa_decode(dims: msa_dims, q, k_cache, v_cache, idx_q, idx_k_cache, cache_lens, out,
               lse=None, block_idx=None, workspace=None, stream=None):
    lib = load_library()
    b, L, Hq, G, d, di, kk = (dims.batch, dims.seqlen, dims.num_q_heads, dims.num_kv_heads,
                             dims.head_dim, dims.index_dim, dims.topk)
    idx_needed = not (dims.flags & (MSA_DENSE | MSA_GIVEN_INDICES))
    p_q = _ptr(q, "q", torch.bfloat16, (b, Hq, d))
    p_k = _ptr(k_cache, "k_cache", torch.bfloat16, (b, L, G, d))
    p_v = _ptr(v_cache, "v_cache", torch.bfloat16, (b, L, G, d))
    p_iq = _ptr(idx_q, "idx_q", torch.bfloat16, (b, G, di), optional=not idx_needed)
    p_ik = _ptr(idx_k_cache, "idx_k_cache", torch.bfloat16, (b, L, di), optional=not idx_needed)
    p_len = _ptr(cache_lens, "cache_lens", torch.int32, (b,))
    p_o = _ptr(out, "out", torch.bfloat16, (b, Hq, d))
    p_l = _ptr(lse, "lse", torch.float32, (b, Hq), optional=True)
    p_bi = _ptr(block_idx, "block_idx", torch.int32, (b, G, kk), optional=True)
    ws, nws = _workspace(MSA_OP_DECODE, dims, workspace, q.device)
    _check(lib, lib.msa_decode(ctypes.byref(dims), p_q, p_k, p_v, p_iq, p_ik, p_len, p_o, p_l, p_bi,
                               ws, nws, _stream(stream)))
    return out


def msa_decode_noalloc(dims: msa_dims, q, k_cache, v_cache, idx_q, idx_k_cache, cache_lens, out,
                       lse=None, block_idx=None, stream=None):
    """msa_decode on the library's own per-GPU scratch array: no workspace
    argument and no allocation (shapes beyond msa_decode_noalloc_limit()
    bytes of workspace are rejected)."""
    lib = load_library()
    b, L, Hq, G, d, di, kk = (dims.batch, dims.seqlen, dims.num_q_heads, dims.num_kv_heads,
                             dims.head_dim, dims.index_dim, dims.topk)
    idx_needed = not (dims.flags & (MSA_DENSE | MSA_GIVEN_INDICES))
    p_q = _ptr(q, "q", torch.bfloat16, (b, Hq, d))
    p_k = _ptr(k_cache, "k_cache", torch.bfloat16, (b, L, G, d))
    p_v = _ptr(v_cache, "v_cache", torch.bfloat16, (b, L, G, d))
    p_iq = _ptr(idx_q, "idx_q", torch.bfloat16, (b, G, di), optional=not idx_needed)
    p_ik = _ptr(idx_k_cache, "idx_k_cache", torch.bfloat16, (b, L, di), optional=not idx_needed)
    p_len = _ptr(cache_lens, "cache_lens", torch.int32, (b,))
    p_o = _ptr(out, "out", torch.bfloat16, (b, Hq, d))
    p_l = _ptr(lse, "lse", torch.float32, (b, Hq), optional=True)
    p_bi = _ptr(block_idx, "block_idx", torch.int32, (b, G, kk), optional=True)
    _check(lib, lib.msa_decode_noalloc(ctypes.byref(dims), p_q, p_k, p_v, p_iq, p_ik, p_len, p_o, p_l, p_bi,
                                       _stream(stream)))
    return out


def msa_profile_begin() -> None:
    """Start recording per-stage HIP events of the library's calls."""
    lib = load_library()
    _check(lib, lib.msa_profile_begin())


def msa_profile_end() -> dict:
    """Stop recording; {stage name: (launches, total ms)} for stages that ran."""
    lib = load_library()
    arr = (msa_stage_time * MSA_STAGE_COUNT)()
    n = ctypes.c_int32(0)
    _check(lib, lib.msa_profile_end(arr, MSA_STAGE_COUNT, ctypes.byref(n)))
    return {msa_stage_name(r.stage): (r.launches, r.total_ms) for r in arr[: n.value] if r.launches > 0}


def msa_stage_name(stage: int) -> str:
    return load_library().msa_stage_name(stage).decode()

"""Shared helpers of the GPU parity tests: running the library through its
binding and comparing against the CPU oracle to the stated tolerances."""
import sys

import numpy as np
import torch

from block_sparse_long_02_amd import binding as bd
from oracle import msa_oracle as orc

# Attention tolerances for bf16 inputs, fp32 accumulation and bf16 outputs.
ATOL_MAX = 2e-2
MEAN_REL = 5e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_prefill(inp, B, k, *, flags=0, query_chunk=0, block_idx=None, want_lse=True, scale=0.0):
    q = inp.q.cuda()
    b, T, Hq, d = q.shape
    G = inp.k.shape[2]
    di = inp.idx_q.shape[-1]
    dims = bd.make_dims(b, T, Hq, G, head_dim=d, index_dim=di, block_size=B, topk=k,
                        flags=flags, query_chunk=query_chunk, softmax_scale=scale)
    out = torch.empty_like(q)
    lse = torch.empty((b, T, Hq), dtype=torch.float32, device="cuda") if want_lse else None
    if flags & bd.MSA_DENSE:
        bidx = None
    elif block_idx is not None:
        bidx = block_idx.cuda().to(torch.int32).contiguous()
    else:
        bidx = torch.full((b, T, G, k), -7, dtype=torch.int32, device="cuda")
    bd.msa_prefill(dims, q, inp.k.cuda(), inp.v.cuda(), inp.idx_q.cuda(), inp.idx_k.cuda(), out,
                   lse=lse, block_idx=bidx)
    torch.cuda.synchronize()
    return out.cpu(), (lse.cpu() if lse is not None else None), (bidx.cpu() if bidx is not None else None)


def gpu_index_topk(inp, B, k, query_chunk=0):
    b, T, G, di = inp.idx_q.shape
    dims = bd.make_dims(b, T, G, G, index_dim=di, block_size=B, topk=k, query_chunk=query_chunk)
    bidx = torch.full((b, T, G, k), -7, dtype=torch.int32, device="cuda")
    bd.msa_index_topk(dims, inp.idx_q.cuda(), inp.idx_k.cuda(), bidx)
    torch.cuda.synchronize()
    return bidx.cpu()


def attn_error(got, ref):
    """(max-abs, mean-relative) of got vs ref (float64 arrays)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    return float(diff.max()), float(diff.sum() / max(np.abs(ref).sum(), 1e-300))


def check_attention(got, ref, what=""):
    mx, mr = attn_error(got, ref)
    say(f"  {what}: max-abs {mx:.3e}  mean-rel {mr:.3e}")
    assert mx <= ATOL_MAX, f"{what}: max-abs {mx}"
    assert mr <= MEAN_REL, f"{what}: mean-rel {mr}"


def check_selection_invariants(bidx, T, G, B, k, rows=None):
    """P4 on GPU output: local block present, exact count, ascending, in range, -1 padding."""
    bidx = bidx.numpy() if hasattr(bidx, "numpy") else bidx
    nbatch = bidx.shape[0]
    t = np.arange(T)
    L = t // B
    m = np.minimum(k, L + 1)
    for s in range(nbatch):
        sel = bidx[s]  # [T, G, k]
        pos = np.arange(k)[None, None, :]
        live = pos < m[:, None, None]
        assert (sel[~np.broadcast_to(live, sel.shape)] == -1).all(), "padding"
        lv = np.where(live, sel, 0)
        assert (np.where(live, sel >= 0, True)).all() and (np.where(live, sel <= L[:, None, None], True)).all()
        # last live entry is the local block (ascending order puts it last)
        last = np.take_along_axis(sel, (m - 1)[:, None, None].repeat(G, 1), axis=2)[..., 0]
        assert (last == L[:, None]).all(), "local block"
        dif = np.diff(lv, axis=2)
        live2 = live[..., 1:]
        assert (np.where(np.broadcast_to(live2, dif.shape), dif > 0, True)).all(), "ascending"


def compare_selection(gpu_bidx, ores, B, k, exact):
    """Compare GPU selection rows with the oracle's; returns the number of
    mismatching rows.  exact=True demands equality; otherwise a mismatch must
    be a near-tie under the oracle's scores."""
    mism = 0
    for (s, t), sel in ores["block_idx"].items():
        G = sel.shape[0]
        for g in range(G):
            got = gpu_bidx[s, t, g].numpy()
            if np.array_equal(got, sel[g]):
                continue
            mism += 1
            if exact:
                raise AssertionError(f"selection mismatch at s={s} t={t} g={g}: {got} vs {sel[g]}")
            S_g = ores["S"][(s, t)][g]
            assert orc.near_tie(S_g, t, B, k), f"non-tie mismatch s={s} t={t} g={g}: {got} vs {sel[g]}"
    return mism


def oracle_rows_out(ores, rows):
    out = np.stack([ores["out"][r] for r in rows])
    lse = np.stack([ores["lse"][r] for r in rows])
    return out, lse


def oracle_rows_gathered(q, k, v, idx_q, idx_k, B, topk, rows, gpu_bidx, s=0):
    """Oracle selection and attention for sampled prefill rows of a large
    workload, using the oracle's own steps but converting to float64 only the
    index keys up to t and the K/V rows the selection gathers.  Attention is
    computed on the GPU's selection (conditioned), selection compared apart.
    Tensors may live on the GPU.  Returns (sel_ok_rows, near_tie_rows,
    bad_rows, out_ref {t: [Hq, d]} for rows whose selection matched)."""
    import math
    G = k.shape[2]
    Hq, d = q.shape[2], q.shape[3]
    R = Hq // G
    scale = 1.0 / math.sqrt(d)
    res = {"equal": 0, "near_tie": 0, "bad": [], "out": {}}
    t_max = max(t for t in rows)
    IK = idx_k[s, : t_max + 1].cpu().to(torch.float64).numpy()
    for t in rows:
        IQ = idx_q[s, t].cpu().to(torch.float64).numpy()
        Q = q[s, t].cpu().to(torch.float64).numpy()
        o_t = np.zeros((Hq, d))
        for g in range(G):
            S = orc.block_max(orc.index_scores(IQ[g], IK, t), t, B)
            sel = orc.select_blocks(S, t, B, topk)
            got = np.asarray(gpu_bidx[s, t, g])
            if np.array_equal(got, sel):
                res["equal"] += 1
            elif orc.near_tie(S, t, B, topk):
                res["near_tie"] += 1
            else:
                res["bad"].append((t, g, got.tolist(), sel.tolist()))
            toks = orc.selected_tokens(got, t, B)
            tk = torch.from_numpy(toks).to(k.device)
            Kg = k[s, tk, g].cpu().to(torch.float64).numpy()
            Vg = v[s, tk, g].cpu().to(torch.float64).numpy()
            o, _ = orc.attention_row(Q[g * R:(g + 1) * R], Kg, Vg, np.arange(len(toks)), scale)
            o_t[g * R:(g + 1) * R] = o
        res["out"][t] = o_t
    return res

"""Plain, slow CPU oracle of the MiniMax Sparse Attention (MSA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module; the library and
its Python binding never do.  It shares no code with the HIP path.

Sources (the pages this follows; cited by title and section):
  [HA]  hyper.ai paper page 2606.13392, "MiniMax Sparse Attention" summary,
        sections 核心贡献 (Contributions) and 方法 (Method).
  [TG]  Telegram review, channel quant_prune_distill, post 751, sections
        "Метод" (Method) and "Эксперименты" (Experiments).
  [HN]  hamidun.com news "MiniMax выпустила MSA …", section "Как устроен MSA".

What is computed (everything in float64 from the bf16 input values, which
are exact in float64):
  index_scores   s[j] = idx_q[t,g] . idx_k[j]  for visible keys j <= t
                 (a raw, pre-softmax dot product)            [HA 方法; TG Метод]
  block_max      S[b] = max of s over the aligned block b (tokens [bB, (b+1)B)),
                 clipped to j <= t                            [HA 方法; TG Метод]
  select_blocks  the local block L(t) = floor(t/B) is always kept; the other
                 min(k, L(t)+1) - 1 blocks are the highest S among blocks
                 0..L(t)-1, equal scores broken by the lower block index;
                 output ascending, padded with -1             [HA 方法, 核心贡献; TG Метод]
                 variant sink=True: block 0 (sequence start) is kept too
                 when there is room for it                    [HA 实验]
  attention_row  exact softmax attention of each query head h of group
                 g = floor(h / R) over the keys of the selected blocks that
                 are <= t, scale 1/sqrt(d)                    [HA 方法; HN]
  decode_row     the same for the one new token at position len-1 of a cache
  attention_backward
                 the gradient of the main branch's output with the selection
                 held fixed: dq, dk, dv from d out       [HA 方法; TG Метод]
  indexer_kl     KL(p_M || p_I) per (token, group) row over the selected tokens,
                 p_I the softmax of the index scores, p_M the main branch's
                 head-averaged attention (held constant), and its gradient
                 into idx_q and idx_k                         [TG Метод; HA 方法]

Readings where the pages are silent (the plainest reading the rest supports):
  - no scale or activation on the index score; a positive scale would not
    change the selection anyway;
  - blocks are aligned at token 0; the last one may be partial;
  - the local block is the aligned block holding the query and counts inside k;
  - ties between equal block maxima go to the lower block index;
  - query head h belongs to group floor(h / R), R = Hq / G;
  - a decode cache of length len holds the new token at position len - 1.
Parity of this module is pinned by tests/test_oracle_pins.py (dense
equivalence through torch's SDPA, closed-form selections, exhaustive subset
enumeration, invariants, special inputs, the 16 x 128 = 2048-token budget).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    """torch tensor (any float dtype, any device) or array -> float64 ndarray."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: only to convert bf16 tensors
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def local_block(t: int, B: int) -> int:
    """The aligned block holding position t [HA 方法: the block containing the
    current query position is always included]."""
    return t // B


def index_scores(idx_q_tg: np.ndarray, idx_k: np.ndarray, t: int) -> np.ndarray:
    """Pre-softmax index scores of one (token, group) row against the visible
    keys 0..t: one index-query head per group, one index-key head shared by
    the layer, plain dot product [TG Метод; HA 方法]."""
    return idx_k[: t + 1] @ idx_q_tg


def block_max(scores: np.ndarray, t: int, B: int) -> np.ndarray:
    """Block Max Pooling: the maximum token score in each aligned block of the
    visible range, blocks 0..L(t) [HA 核心贡献, 方法; TG Метод]."""
    L = local_block(t, B)
    out = np.empty(L + 1, dtype=np.float64)
    for b in range(L + 1):
        lo, hi = b * B, min((b + 1) * B, t + 1)
        out[b] = scores[lo:hi].max()
    return out


def forced_blocks(t: int, B: int, k: int, sink: bool = False) -> list:
    """Blocks kept whatever their scores: the local block L(t) always [HA 方法];
    with sink=True also block 0, the start of the sequence, when the row has
    room for a second block (m = min(k, L+1) >= 2) -- the forced
    sequence-start variant the pages ablate [HA 实验: hard-coded selection of
    the sequence start and of the local window]."""
    L = local_block(t, B)
    m = min(k, L + 1)
    return [L, 0] if (sink and L >= 1 and m >= 2) else [L]


def select_blocks(S: np.ndarray, t: int, B: int, k: int, sink: bool = False) -> np.ndarray:
    """Top-k block selection with the forced block(s).

    m = min(k, L+1) blocks are kept: the forced blocks (the local block L, and
    with sink=True block 0) and the highest of the remaining candidate blocks
    below L, ordered by score (descending) then block id (ascending).
    Returned ascending and padded with -1 to length k [HA 方法: top-k per
    query group, local block always included; TG Метод; HA 实验 for sink]."""
    L = local_block(t, B)
    m = min(k, L + 1)
    forced = forced_blocks(t, B, k, sink)
    cand = np.array([b for b in range(L) if b not in forced], dtype=np.int64)
    order = np.lexsort((cand, -S[cand]))  # primary: -score, secondary: block id
    chosen = np.concatenate([cand[order[: m - len(forced)]], forced]).astype(np.int64)
    chosen.sort()
    out = np.full(k, -1, dtype=np.int64)
    out[:m] = chosen
    return out


def selected_tokens(sel: np.ndarray, t: int, B: int) -> np.ndarray:
    """Key positions covered by the selected blocks, clipped to j <= t."""
    toks = []
    for b in sel:
        if b < 0:
            continue
        toks.append(np.arange(b * B, min((b + 1) * B, t + 1)))
    return np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)


def attention_row(q_t: np.ndarray, K: np.ndarray, V: np.ndarray, toks: np.ndarray,
                  scale: float):
    """Exact softmax attention of query rows q_t [R, d] over the gathered
    keys/values K[toks], V[toks] ([n, d]) [HA 方法: standard scaled dot-product
    attention over the Key/Value vectors gathered from the selected blocks].
    Returns (o [R, d], lse [R]) with lse = ln sum_j exp(x_j).  A row with no
    key to attend (a given selection that keeps none of its visible blocks)
    is defined as o = 0, lse = -inf."""
    if len(toks) == 0:
        return np.zeros((q_t.shape[0], V.shape[-1])), np.full(q_t.shape[0], -np.inf)
    Kg, Vg = K[toks], V[toks]
    x = scale * (q_t @ Kg.T)                      # [R, n]
    mx = x.max(axis=1, keepdims=True)
    w = np.exp(x - mx)
    den = w.sum(axis=1, keepdims=True)
    o = (w @ Vg) / den
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def prefill(q, k, v, idx_q, idx_k, B: int, topk: int, scale: float | None = None,
            rows=None, dense: bool = False, block_idx=None, sink: bool = False):
    """MSA prefill over a batch.

    q [b,T,Hq,d], k/v [b,T,G,d], idx_q [b,T,G,di], idx_k [b,T,di] (any float
    type; converted to float64).  rows: iterable of (batch, t) to compute, or
    None for all.  dense: select every visible block (index branch skipped).
    block_idx: optional given selection [b,T,G,topk] (main branch only).
    sink: also force block 0 into every selection (see forced_blocks).

    Returns dict with 'out' {(s,t): [Hq,d]}, 'lse' {(s,t): [Hq]},
    'block_idx' {(s,t): [G,topk]} (None in dense mode) for the rows computed,
    plus 'S' {(s,t): list of per-group block-max arrays}.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    idx_q, idx_k = _f64(idx_q), _f64(idx_k)
    nbatch, T, Hq, d = q.shape
    G = k.shape[2]
    R = Hq // G
    if scale is None:
        scale = default_scale(d)
    if rows is None:
        rows = [(s, t) for s in range(nbatch) for t in range(T)]
    given = None if block_idx is None else np.asarray(_f64(block_idx), dtype=np.int64)
    res = {"out": {}, "lse": {}, "block_idx": {} if not dense else None, "S": {}}
    for s, t in rows:
        o_t = np.empty((Hq, d))
        lse_t = np.empty(Hq)
        sel_t = np.full((G, topk), -1, dtype=np.int64)
        S_t = []
        for g in range(G):
            if dense:
                sel = np.arange(local_block(t, B) + 1)
            elif given is not None:
                sel = given[s, t, g]
            else:
                sc = index_scores(idx_q[s, t, g], idx_k[s], t)
                Sg = block_max(sc, t, B)
                S_t.append(Sg)
                sel = select_blocks(Sg, t, B, topk, sink)
            if not dense:
                sel_t[g] = sel
            toks = selected_tokens(sel, t, B)
            heads = slice(g * R, (g + 1) * R)
            o, lse = attention_row(q[s, t, heads], k[s, :, g], v[s, :, g], toks, scale)
            o_t[heads] = o
            lse_t[heads] = lse
        res["out"][(s, t)] = o_t
        res["lse"][(s, t)] = lse_t
        if not dense:
            res["block_idx"][(s, t)] = sel_t
        res["S"][(s, t)] = S_t
    return res


def decode(q, k_cache, v_cache, idx_q, idx_k_cache, cache_lens, B: int, topk: int,
           scale: float | None = None, dense: bool = False, block_idx=None, sink: bool = False):
    """One decode step per sequence: the new token sits at position len-1 of
    its cache and runs the same index branch and main branch against cache
    positions 0..len-1 [HA 方法; the pages' decode speed-up at 1M context].

    q [b,Hq,d], k/v_cache [b,L,G,d], idx_q [b,G,di], idx_k_cache [b,L,di],
    cache_lens [b].  Returns dict with 'out' [b,Hq,d], 'lse' [b,Hq],
    'block_idx' [b,G,topk] (None in dense mode), 'S' list per sequence."""
    q, k_cache, v_cache = _f64(q), _f64(k_cache), _f64(v_cache)
    idx_q, idx_k_cache = _f64(idx_q), _f64(idx_k_cache)
    lens = [int(x) for x in (cache_lens.tolist() if hasattr(cache_lens, "tolist") else cache_lens)]
    nbatch, Hq, d = q.shape
    G = k_cache.shape[2]
    R = Hq // G
    if scale is None:
        scale = default_scale(d)
    given = None if block_idx is None else np.asarray(_f64(block_idx), dtype=np.int64)
    out = np.empty((nbatch, Hq, d))
    lse = np.empty((nbatch, Hq))
    sel_all = np.full((nbatch, G, topk), -1, dtype=np.int64)
    S_all = []
    for s in range(nbatch):
        t = lens[s] - 1
        S_s = []
        for g in range(G):
            if dense:
                sel = np.arange(local_block(t, B) + 1)
            elif given is not None:
                sel = given[s, g]
            else:
                sc = index_scores(idx_q[s, g], idx_k_cache[s], t)
                Sg = block_max(sc, t, B)
                S_s.append(Sg)
                sel = select_blocks(Sg, t, B, topk, sink)
                sel_all[s, g] = sel
            toks = selected_tokens(sel, t, B)
            heads = slice(g * R, (g + 1) * R)
            o, l = attention_row(q[s, heads], k_cache[s, :, g], v_cache[s, :, g], toks, scale)
            out[s, heads] = o
            lse[s, heads] = l
        S_all.append(S_s)
    return {"out": out, "lse": lse, "block_idx": None if dense else sel_all, "S": S_all}


def near_tie(S_g: np.ndarray, t: int, B: int, k: int, rel: float = 1e-3, sink: bool = False) -> bool:
    """True when the selection of this (token, group) row is decided by a
    near-tie: the last selected candidate and the first unselected one (in
    the oracle's score order, forced blocks excluded) differ by less than rel
    relative."""
    L = local_block(t, B)
    m = min(k, L + 1)
    forced = forced_blocks(t, B, k, sink)
    cand = np.array([b for b in range(L) if b not in forced], dtype=np.int64)
    want = m - len(forced)
    if want == 0 or want >= len(cand):
        return False          # nothing chosen among candidates, or all of them
    order = np.lexsort((cand, -S_g[cand]))
    sc = S_g[cand][order]
    a, b = sc[want - 1], sc[want]
    return abs(a - b) < rel * max(abs(a), abs(b), 1e-30)


def indexer_kl(q, k, idx_q, idx_k, block_idx, B: int, scale: float | None = None, rows=None):
    """Indexer KL loss and its gradient into the index branch inputs.

    The index branch is trained by aligning its distribution with the main
    branch's on the selected tokens: a KL divergence between the index
    branch's distribution and the main branch's head-averaged one, with a
    stop-gradient through the main branch's probabilities and the index
    inputs detached, so that only the index projections learn [TG Метод: KL
    between the index branch's outputs and the averaged main-branch outputs,
    stopgrad through the main-branch probabilities and on the index inputs;
    HA 方法: KL loss aligning the Index Branch with the Main Branch on the
    selected tokens, gradient detach on the Index Branch inputs].

    Per (s, t, g) row, J = the tokens <= t of the row's selected blocks:
      p_I(j) = softmax_j(idx_q[t,g] . idx_k[j])            (raw index score)
      p_M(j) = mean over the R heads h of group g of softmax_j(scale q[t,h] . k[j,g])
      KL     = sum_j p_M(j) (log p_M(j) - log p_I(j))
    and, for L = sum of KL over the rows computed, with p_M held constant,
      dL/d idx_q[t,g] = sum_j (p_I(j) - p_M(j)) idx_k[j]
      dL/d idx_k[j]  += (p_I(j) - p_M(j)) idx_q[t,g]       (over every row using j)

    q [b,T,Hq,d], k [b,T,G,d], idx_q [b,T,G,di], idx_k [b,T,di], block_idx
    [b,T,G,topk] (entries outside [0, L(t)] ignored).  rows: iterable of
    (batch, t), default all.  Returns {'kl': {(s,t): [G]}, 'd_idx_q':
    {(s,t): [G,di]}, 'd_idx_k': [b,T,di] accumulated over the rows computed}.
    """
    q, k = _f64(q), _f64(k)
    idx_q, idx_k = _f64(idx_q), _f64(idx_k)
    sel_all = np.asarray(_f64(block_idx), dtype=np.int64)
    nbatch, T, Hq, d = q.shape
    G = k.shape[2]
    R = Hq // G
    if scale is None:
        scale = default_scale(d)
    if rows is None:
        rows = [(s, t) for s in range(nbatch) for t in range(T)]
    res = {"kl": {}, "d_idx_q": {}, "d_idx_k": np.zeros(idx_k.shape)}
    for s, t in rows:
        L = local_block(t, B)
        kl_t = np.zeros(G)
        dq_t = np.zeros((G, idx_q.shape[-1]))
        for g in range(G):
            sel = [b for b in sel_all[s, t, g] if 0 <= b <= L]
            toks = selected_tokens(np.array(sorted(set(sel)), dtype=np.int64), t, B)
            if len(toks) == 0:
                continue
            sI = idx_k[s, toks] @ idx_q[s, t, g]
            log_pI = sI - (sI.max() + np.log(np.exp(sI - sI.max()).sum()))
            pM = np.zeros(len(toks))
            for h in range(g * R, (g + 1) * R):
                x = scale * (k[s, toks, g] @ q[s, t, h])
                a = np.exp(x - x.max())
                pM += a / a.sum()
            pM /= R
            nz = pM > 0
            kl_t[g] = float((pM[nz] * (np.log(pM[nz]) - log_pI[nz])).sum())
            ds = np.exp(log_pI) - pM
            dq_t[g] = ds @ idx_k[s, toks]
            res["d_idx_k"][s, toks] += ds[:, None] * idx_q[s, t, g][None, :]
        res["kl"][(s, t)] = kl_t
        res["d_idx_q"][(s, t)] = dq_t
    return res


def indexer_kl_rows(q, k, idx_q, idx_k, block_idx, B: int, rows, scale: float | None = None):
    """kl and d idx_q of the rows (s, t) given, as indexer_kl defines them,
    reading only those rows and their selected keys (for sampled checks at
    sizes where the whole inputs do not fit in float64).  Returns
    {'kl': {(s,t): [G]}, 'd_idx_q': {(s,t): [G, di]}}."""
    nbatch, T, Hq, d = q.shape
    G = k.shape[2]
    R = Hq // G
    if scale is None:
        scale = default_scale(d)
    res = {"kl": {}, "d_idx_q": {}}
    for s, t in rows:
        L = local_block(t, B)
        sel_t = np.asarray(_f64(block_idx[s, t]), dtype=np.int64)
        q_t, iq_t = _f64(q[s, t]), _f64(idx_q[s, t])
        kl_t = np.zeros(G)
        dq_t = np.zeros((G, iq_t.shape[-1]))
        for g in range(G):
            sel = [b for b in sel_t[g] if 0 <= b <= L]
            toks = selected_tokens(np.array(sorted(set(sel)), dtype=np.int64), t, B)
            if len(toks) == 0:
                continue
            lo, hi = int(toks.min()), int(toks.max()) + 1
            Kw = _f64(k[s, lo:hi, g])[toks - lo]
            IKw = _f64(idx_k[s, lo:hi])[toks - lo]
            sI = IKw @ iq_t[g]
            log_pI = sI - (sI.max() + np.log(np.exp(sI - sI.max()).sum()))
            pM = np.zeros(len(toks))
            for h in range(g * R, (g + 1) * R):
                x = scale * (Kw @ q_t[h])
                a = np.exp(x - x.max())
                pM += a / a.sum()
            pM /= R
            nz = pM > 0
            kl_t[g] = float((pM[nz] * (np.log(pM[nz]) - log_pI[nz])).sum())
            dq_t[g] = (np.exp(log_pI) - pM) @ IKw
        res["kl"][(s, t)] = kl_t
        res["d_idx_q"][(s, t)] = dq_t
    return res


def _backward_row(q_rows, Kg, Vg, dO, scale: float):
    """One (token, group) row of the backward: R query heads q_rows [R, d]
    over the gathered keys/values Kg, Vg [n, d], upstream gradient dO [R, d].
    Returns (dq [R, d], dk [n, d], dv [n, d]) of this row."""
    x = scale * (q_rows @ Kg.T)                        # [R, n]
    P = np.exp(x - x.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dP = dO @ Vg.T                                     # [R, n]
    dx = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    return scale * (dx @ Kg), scale * (dx.T @ q_rows), P.T @ dO


def attention_backward(q, k, v, dout, block_idx, B: int, scale: float | None = None):
    """Gradient of the main branch's output with respect to q, k and v, the
    selection held fixed.

    The selection is a top-k of block maxima, piecewise constant in the index
    inputs, and the index branch is trained only through its own loss with
    its inputs detached [TG Метод: stop-gradient on the index branch; HA 方法:
    gradient detach on the Index Branch inputs].  So the main branch is
    differentiated as the plain softmax attention it is on the fixed token set
    J of each row [HA 方法: standard scaled dot-product attention over the
    gathered Key/Value vectors].  Per (s, t, h), g = floor(h / R), J = the
    tokens <= t of the row's selected blocks (entries outside [0, L(t)]
    ignored, as in the given-selection prefill), x_j = scale q[t,h] . k[j,g],
    P = softmax_J(x), o = sum_j P_j v[j,g]; for a loss with d loss / d o = dO:
      dv[j,g] += P_j dO
      dP_j     = dO . v[j,g]
      dx_j     = P_j (dP_j - sum_i P_i dP_i)
      dq[t,h]  = scale sum_j dx_j k[j,g]
      dk[j,g] += scale dx_j q[t,h]
    A row with nothing to attend contributes nothing.

    q, dout [b,T,Hq,d]; k, v [b,T,G,d]; block_idx [b,T,G,topk].
    Returns (dq [b,T,Hq,d], dk [b,T,G,d], dv [b,T,G,d]) in float64.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    sel_all = np.asarray(_f64(block_idx), dtype=np.int64)
    nbatch, T, Hq, d = q.shape
    G = k.shape[2]
    R = Hq // G
    if scale is None:
        scale = default_scale(d)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for s in range(nbatch):
        for t in range(T):
            for g in range(G):
                toks = selected_tokens(sel_all[s, t, g], t, B)
                if len(toks) == 0:
                    continue
                heads = slice(g * R, (g + 1) * R)
                dq_r, dk_r, dv_r = _backward_row(q[s, t, heads], k[s, toks, g], v[s, toks, g],
                                                 dout[s, t, heads], scale)
                dq[s, t, heads] = dq_r
                np.add.at(dk[s, :, g], toks, dk_r)
                np.add.at(dv[s, :, g], toks, dv_r)
    return dq, dk, dv


def attention_backward_dq(q, k, v, dout, block_idx, B: int, rows, scale: float | None = None):
    """dq of the rows (s, t) given, as attention_backward defines it, reading
    only those rows and their selected keys (for sampled checks at sizes
    where the whole gradient does not fit in float64).  Returns
    {(s, t): dq [Hq, d]}."""
    nbatch, T, Hq, d = q.shape
    G = k.shape[2]
    R = Hq // G
    if scale is None:
        scale = default_scale(d)
    res = {}
    for s, t in rows:
        dq_t = np.zeros((Hq, d))
        sel_t = np.asarray(_f64(block_idx[s, t]), dtype=np.int64)
        q_t, do_t = _f64(q[s, t]), _f64(dout[s, t])
        for g in range(G):
            toks = selected_tokens(sel_t[g], t, B)
            if len(toks) == 0:
                continue
            lo, hi = int(toks.min()), int(toks.max()) + 1
            Kw, Vw = _f64(k[s, lo:hi, g]), _f64(v[s, lo:hi, g])
            heads = slice(g * R, (g + 1) * R)
            dq_t[heads] = _backward_row(q_t[heads], Kw[toks - lo], Vw[toks - lo], do_t[heads], scale)[0]
        res[(s, t)] = dq_t
    return res

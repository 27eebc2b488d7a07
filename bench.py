"""Benchmark of the MSA forward path on one MI355X.

One step = one MSA layer prefill over T = 131072 tokens (64 query heads in 8
GQA groups, head_dim 128, index_dim 128, block 128, top-k 16, idx_k with a
per-block random mean offset) followed by one decode step for 8 sequences at
1,048,576 tokens of context (same head layout).  Inputs are seeded synthetic
bf16 tensors resident in HBM before timing starts.

Prints one JSON line: `value` is prefill tokens/s; the decode rate, the dense
(all-blocks) comparison, a sampled parity check against the CPU oracle, the
roofline of the dominant prefill kernel (the stage with the largest time,
timed live with the library's per-stage HIP events over the timed steps), the
rooflines of the other main kernels, and the oracle's own rate on the host
cores are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_long_02_amd import binding as bd  # noqa: E402
from block_sparse_long_02_amd import inputs  # noqa: E402

METRIC = "MSA layer prefill tok/s @128K & decode tok/s @1M ctx; % MFMA/HBM roofline"
PEAK_MFMA_BF16 = 2.5e15   # MI355X dense bf16, FLOP/s
PEAK_HBM = 8.0e12         # MI355X HBM3E, B/s

PF = dict(T=131072, Hq=64, G=8, d=128, di=128, B=128, k=16, skew=0.5, seed=0)
DC = dict(batch=8, L=1 << 20, Hq=64, G=8, d=128, di=128, B=128, k=16, seed=1)

COPY_BYTES = 1 << 30   # calibration copy for the --pmc passes


def traffic_file(kernel):
    workload = ("decode_8x1m" if kernel.startswith("decode_") else
                "backward_t131072" if kernel.startswith("bwd_") else "prefill_t131072")
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def n_att(t, B, k):
    return (t % B) + 1 + B * min(k - 1, t // B)


def prefill_flops(T, Hq, G, d, di, B, k):
    t = np.arange(T, dtype=np.float64)
    index = 2.0 * G * di * (t + 1).sum()
    L = np.floor(t / B)
    att = (t % B) + 1 + B * np.minimum(k - 1, L)
    main = 4.0 * Hq * d * att.sum()
    return index, main


def indexer_kl_flops(T, Hq, G, d, di, B, k):
    """Per (row, attended token): the index score (2 di), the R heads' logits
    (2 d R), and the two gradient products (2 di each)."""
    t = np.arange(T, dtype=np.float64)
    L = np.floor(t / B)
    att = (t % B) + 1 + B * np.minimum(k - 1, L)
    return G * (6.0 * di + 2.0 * d * (Hq // G)) * att.sum()


def indexer_kl_ms(pin, bidx, lse, dev, stream, reps, keep=False):
    """Mean ms of the indexer KL on the prefill's selection and lse (and its
    outputs kl, d_idx_q, d_idx_k when keep)."""
    T, Hq, G, di = PF["T"], PF["Hq"], PF["G"], PF["di"]
    kd = bd.make_dims(1, T, Hq, G, index_dim=di, block_size=PF["B"], topk=PF["k"])
    kl = torch.empty((1, T, G), dtype=torch.float32, device=dev)
    dq = torch.empty((1, T, G, di), dtype=torch.float32, device=dev)
    dk = torch.empty((1, T, di), dtype=torch.float32, device=dev)
    kws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_INDEXER_KL, kd), dtype=torch.uint8, device=dev)
    fn = lambda: bd.msa_indexer_kl(kd, pin.q, pin.k, pin.idx_q, pin.idx_k, bidx, lse, kl, dq, dk,  # noqa: E731
                                   workspace=kws)
    fn()
    ms, _ = timed(fn, reps, stream)
    return (ms, (kl, dq, dk)) if keep else ms


def indexer_kl_checks(pin, pbidx, tensors, n_rows=24):
    """Full-size checks of the indexer KL: kl and d idx_q on seeded sampled
    rows against the oracle (row by row), and for d idx_k the property that
    holds at any size (summed over all keys it vanishes: each row's
    p_I - p_M sums to zero)."""
    from oracle import msa_oracle as orc
    kl, dq, dk = tensors
    T, B = PF["T"], PF["B"]
    rng = np.random.default_rng(79)
    ts = sorted(set([0, B - 1, B, T - 1] + [int(x) for x in rng.integers(0, T, n_rows - 4)]))
    rows = [(0, t) for t in ts]
    ref = orc.indexer_kl_rows(pin.q.cpu(), pin.k.cpu(), pin.idx_q.cpu(), pin.idx_k.cpu(), pbidx.cpu(), B, rows)
    klg, dqg = kl.cpu().double().numpy(), dq.cpu().double().numpy()
    kl_ok = all(bool((np.abs(klg[r] - ref["kl"][r]) <= 1e-3 * np.abs(ref["kl"][r]) + 1e-4).all()) for r in rows)
    err = sum(float(np.abs(dqg[r] - ref["d_idx_q"][r]).sum()) for r in rows)
    tot = sum(float(np.abs(ref["d_idx_q"][r]).sum()) for r in rows)
    mx = max(float(np.abs(dqg[r] - ref["d_idx_q"][r]).max()) for r in rows)
    scale = max(float(np.abs(ref["d_idx_q"][r]).max()) for r in rows)
    dk64 = dk.double()
    inv = float((dk64.sum(dim=1).abs().max() / dk64.abs().sum(dim=1).max()).item())
    return {"rows": len(rows), "kl_within_bound": kl_ok, "d_idx_q_max_abs": mx, "d_idx_q_ref_max": scale,
            "d_idx_q_mean_rel": err / max(tot, 1e-300), "d_idx_k_sum_rel": inv,
            "ok": bool(kl_ok and mx <= 1e-2 * scale and err / max(tot, 1e-300) <= 5e-3 and inv <= 1e-4)}


def backward_flops(T, Hq, d, B, k):
    """Per (token, head, attended key) the backward's five products (S, dP,
    dv, dk, dq), 2d flop each."""
    t = np.arange(T, dtype=np.float64)
    att = (t % B) + 1 + B * np.minimum(k - 1, np.floor(t / B))
    return 10.0 * d * Hq * att.sum()


def bwd_list_bytes(bidx, T, Hq, G, d, B, window=8192):
    """Algorithmic bytes of one bwd_list_kernel launch over the whole prefill:
    per (token, group, selected block) entry, the local block included, the
    group's R q and dO rows are read and R bf16 dq partial rows written, plus
    each row's lse and dO.out (8 bytes) and the 4-byte entry; per non-empty
    (group, 8192-token window, block) list the K/V block is read once and its
    fp32 dk/dv partial block written."""
    R = Hq // G
    t = torch.arange(T, device=bidx.device).view(1, T, 1, 1)
    sel = bidx.long()
    valid = (sel >= 0) & (sel <= t // B)
    entries = int(valid.sum().item())
    nb = (T + B - 1) // B
    nwin = (T + window - 1) // window
    g = torch.arange(G, device=bidx.device).view(1, 1, G, 1)
    key = ((g * nwin + t // window) * nb + sel)[valid]
    lists = int(torch.unique(key).numel())
    per_entry = R * (3 * d * 2 + 8) + 4
    return entries * per_entry + lists * (2 * B * d * 2 + 2 * B * d * 4), entries, lists


def backward_run(pin, pout, plse, pbidx, dev, stream, reps, profile=True):
    """The main-branch backward on the headline prefill's output, lse and
    selection with a seeded d out: (mean ms, stage ms, tensors)."""
    T, Hq, G = PF["T"], PF["Hq"], PF["G"]
    bdims = bd.make_dims(1, T, Hq, G, index_dim=PF["di"], block_size=PF["B"], topk=PF["k"])
    gen = torch.Generator(device=dev).manual_seed(77)
    dout = torch.randn((1, T, Hq, PF["d"]), generator=gen, device=dev).to(torch.bfloat16)
    dq = torch.empty((1, T, Hq, PF["d"]), dtype=torch.float32, device=dev)
    dk = torch.empty((1, T, G, PF["d"]), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_BACKWARD, bdims), dtype=torch.uint8, device=dev)
    fn = lambda: bd.msa_prefill_backward(bdims, pin.q, pin.k, pin.v, pout, plse, dout, pbidx,  # noqa: E731
                                         dq, dk, dv, workspace=ws)
    fn()
    ms, per = timed(fn, reps, stream)
    stages = None
    if profile:
        bd.msa_profile_begin()
        fn()
        torch.cuda.synchronize()
        stages = {n: t_ / c for n, (c, t_) in bd.msa_profile_end().items()}
    del ws
    return ms, per, stages, (dout, dq, dk, dv)


def backward_checks(pin, pbidx, tensors, n_rows=24):
    """Full-size checks of the backward: dq on seeded sampled rows against the
    oracle (row by row), and for dk / dv the properties that hold at any size
    (per group the key gradients sum to zero, the value gradients to the
    summed d out, every row attending at least its local block)."""
    from oracle import msa_oracle as orc
    dout, dq, dk, dv = tensors
    T, Hq, G, B = PF["T"], PF["Hq"], PF["G"], PF["B"]
    rng = np.random.default_rng(78)
    ts = sorted(set([0, B - 1, B, T - 1] + [int(x) for x in rng.integers(0, T, n_rows - 4)]))
    rows = [(0, t) for t in ts]
    bidx_c = pbidx.cpu()
    ref = orc.attention_backward_dq(pin.q.cpu(), pin.k.cpu(), pin.v.cpu(), dout.cpu(), bidx_c, B, rows)
    got = dq.cpu().double().numpy()
    err = sum(float(np.abs(got[r] - ref[r]).sum()) for r in rows)
    tot = sum(float(np.abs(ref[r]).sum()) for r in rows)
    mx = max(float(np.abs(got[r] - ref[r]).max()) for r in rows)
    scale = max(float(np.abs(ref[r]).max()) for r in rows)
    R = Hq // G
    dk64, dv64 = dk.double(), dv.double()
    dsum = dout.double().view(1, T, G, R, -1).sum(dim=(1, 3))        # [1, G, d]
    inv_k = float((dk64.sum(dim=1).abs().max() / dk64.abs().sum(dim=1).max()).item())
    inv_v = float(((dv64.sum(dim=1) - dsum).abs().max() / dsum.abs().max()).item())
    return {"rows": len(rows), "dq_max_abs": mx, "dq_ref_max": scale, "dq_mean_rel": err / max(tot, 1e-300),
            "dk_sum_rel": inv_k, "dv_sum_minus_dout_rel": inv_v,
            "ok": bool(mx <= 1e-2 * scale and err / max(tot, 1e-300) <= 5e-3 and inv_k <= 1e-4 and inv_v <= 1e-4)}


def dense_prefill_flops(T, Hq, d):
    return 4.0 * Hq * d * T * (T + 1) / 2


def decode_bytes(batch, L, Hq, G, d, di, B, k):
    t = L - 1
    per_seq = L * di * 2 + G * n_att(t, B, k) * d * 2 * 2 + Hq * d * 2 * 2 + G * di * 2
    return batch * per_seq


def measured_traffic(kernel):
    """Per-launch HBM bytes of a kernel from the committed --pmc summary, or
    None when absent or taken on different kernel sources."""
    from block_sparse_long_02_amd import profiling
    try:
        with open(traffic_file(kernel)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != profiling.source_hash(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def kv_outer_bytes(bidx, T, Hq, G, d, B, k):
    """Algorithmic bytes of one block-major launch over the whole prefill:
    per (token, group, selected non-local block) entry the group's R q rows
    are read and R partial rows (fp16 values + 8-byte statistics) written,
    plus the 4-byte list entry; every distinct selected (group, block) K/V
    block is read once."""
    R = Hq // G
    t = torch.arange(T, device=bidx.device).view(1, T, 1, 1)
    sel = bidx.long()
    valid = (sel >= 0) & (sel < t // B)
    entries = int(valid.sum().item())
    gb = (torch.arange(G, device=bidx.device).view(1, 1, G, 1) * ((T + B - 1) // B) + sel)[valid]
    blocks = int(torch.unique(gb).numel())
    per_entry = R * d * 2 + R * (d * 2 + 8) + 4
    return entries * per_entry + blocks * 2 * B * d * 2, entries, blocks


def compulsory_prefill_bytes(T, Hq, G, d, di, k):
    """Bytes no prefill schedule can avoid: every input read once (q, k, v,
    idx_q, idx_k) and every output written once (out bf16, lse fp32, the
    selection int32).  About 5.2 GB at T = 131072, 64 q heads, 8 groups."""
    return (T * Hq * d * 2 + 2 * T * G * d * 2 + T * G * di * 2 + T * di * 2
            + T * Hq * d * 2 + T * Hq * 4 + T * G * k * 4)


def kv_outer_flops(entries, Hq, G, d, B):
    """Method flops of the block-major launch: per non-local (token, group,
    block) entry, QK^T and PV over the block's B keys for the group's R
    heads, 4 d B R."""
    return 4.0 * d * B * (Hq // G) * entries


def local_block_flops(T, Hq, d, B):
    """Method flops of the local blocks: 4 Hq d (t mod B + 1) per token."""
    t = np.arange(T, dtype=np.float64)
    return 4.0 * Hq * d * ((t % B) + 1).sum()


def query_major_bytes(entries, T, Hq, G, d, B):
    """Algorithmic bytes of the query-major launch: per (token, head) the q row
    is read and the output row and lse written; per partial the fp16 row,
    its statistics and its list position are read; the local blocks' K/V
    (each block once per group)."""
    R = Hq // G
    nb = (T + B - 1) // B
    return T * Hq * (d * 2 + d * 2 + 4) + entries * (R * (d * 2 + 8) + 4) + G * nb * 2 * B * d * 2


def measured_peaks(dev):
    """Context only: a vendor bf16 GEMM and a device copy on this GPU."""
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        a @ b
    ms, _ = timed(lambda: a @ b, 10, torch.cuda.current_stream())
    x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    cms, _ = timed(lambda: y.copy_(x), 10, torch.cuda.current_stream())
    del a, b, x, y
    return {"bf16_gemm_8192_tflops": round(2 * 8192 ** 3 / (ms * 1e-3) / 1e12, 1),
            "device_copy_gbs": round(2 * (1 << 30) / (cms * 1e-3) / 1e9, 1)}


def profile_kernels_only(args, dev):
    """The 128K prefill's inputs, one calibration copy of COPY_BYTES, then
    --steps prefills, --steps indexer KL calls, --steps msa_index_topk calls
    in each of its two forms (two-pass, one-pass) and --steps main-branch
    backward calls on the last prefill's output (each +1 warmup), --steps
    all-blocks prefills of the same inputs (+1 warmup) and --steps
    decode steps (8 x 1M context), every kernel
    launched as in the timed steps: the workload of the --pmc counter passes
    and of the kernel-trace summary."""
    stream = torch.cuda.current_stream()
    pin = inputs.make_prefill(PF["T"], PF["Hq"], PF["G"], PF["d"], PF["di"], seed=PF["seed"], device=dev,
                              block_size=PF["B"], skew_std=PF["skew"])
    pdims = bd.make_dims(1, PF["T"], PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"])
    pout = torch.empty_like(pin.q)
    pws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, pdims), dtype=torch.uint8, device=dev)
    x = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    plse = torch.empty((1, PF["T"], PF["Hq"]), dtype=torch.float32, device=dev)
    pbidx = torch.empty((1, PF["T"], PF["G"], PF["k"]), dtype=torch.int32, device=dev)
    bd.msa_profile_begin()
    ms, _ = timed(lambda: bd.msa_prefill(pdims, pin.q, pin.k, pin.v, pin.idx_q, pin.idx_k, pout, lse=plse,
                                         block_idx=pbidx, workspace=pws), args.steps, stream)
    del pws
    kms = indexer_kl_ms(pin, pbidx, plse, dev, stream, args.steps)
    iforms = index_topk_forms(pin, pbidx, dev, stream, args.steps)
    bms, _, _, btens = backward_run(pin, pout, plse, pbidx, dev, stream, args.steps, profile=False)
    del btens
    # the all-blocks (dense) prefill of the same inputs
    ddn = bd.make_dims(1, PF["T"], PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"],
                       flags=bd.MSA_DENSE)
    dense_out = torch.empty_like(pin.q)
    bd.msa_prefill(ddn, pin.q, pin.k, pin.v, None, None, dense_out)
    dnms, _ = timed(lambda: bd.msa_prefill(ddn, pin.q, pin.k, pin.v, None, None, dense_out), args.steps, stream)
    del dense_out
    dec = inputs.make_decode(DC["batch"], DC["L"], DC["Hq"], DC["G"], DC["d"], DC["di"], seed=DC["seed"],
                             device=dev)
    ddims = bd.make_dims(DC["batch"], DC["L"], DC["Hq"], DC["G"], index_dim=DC["di"], block_size=DC["B"],
                         topk=DC["k"])
    dout = torch.empty((DC["batch"], DC["Hq"], DC["d"]), dtype=torch.bfloat16, device=dev)
    dws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_DECODE, ddims), dtype=torch.uint8, device=dev)
    dfn = lambda: bd.msa_decode(ddims, dec.q, dec.k_cache, dec.v_cache, dec.idx_q, dec.idx_k_cache,  # noqa: E731
                                dec.cache_lens, dout, workspace=dws)
    dms, _ = timed(dfn, args.steps, stream)
    stages = bd.msa_profile_end()
    print(json.dumps({"profile_steps": args.steps, "prefill_ms": round(ms, 4), "decode_ms": round(dms, 4),
                      "indexer_kl_ms": round(kms, 4), "backward_ms": round(bms, 4), "dense_ms": round(dnms, 4),
                      "index_topk": iforms,
                      "copy_bytes": COPY_BYTES,
                      "stage_ms": {n: round(t / c, 4) for n, (c, t) in stages.items()}}), flush=True)


def prefill_1m_run(dev, stream):
    """The long prefill of the pages' 1M-token setting: T = 1,048,576, 64 q heads
    in 8 groups, block 128, top-k 16, with 64 needle blocks (separable preset);
    one warmup, the mean of 2 timed calls, and the per-prefill stage totals of a
    third (the call runs in query chunks, so stages launch several times)."""
    T = 1 << 20
    pin = inputs.make_prefill(T, PF["Hq"], PF["G"], PF["d"], PF["di"], seed=5, device=dev, block_size=PF["B"],
                              needles=64)
    dims = bd.make_dims(1, T, PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"])
    out = torch.empty_like(pin.q)
    ws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, dims), dtype=torch.uint8, device=dev)
    fn = lambda: bd.msa_prefill(dims, pin.q, pin.k, pin.v, pin.idx_q, pin.idx_k, out, workspace=ws)  # noqa: E731
    fn()
    ms, _ = timed(fn, 2, stream)
    bd.msa_profile_begin()
    fn()
    torch.cuda.synchronize()
    stages = {n: {"launches": c, "ms": round(t, 3)} for n, (c, t) in bd.msa_profile_end().items()}
    f_index, f_main = prefill_flops(T, PF["Hq"], PF["G"], PF["d"], PF["di"], PF["B"], PF["k"])
    res = {"ms": round(ms, 2), "tok_s": round(T / (ms * 1e-3), 1),
           "algorithmic_tflop": round((f_index + f_main) / 1e12, 2),
           "tflops": round((f_index + f_main) / (ms * 1e-3) / 1e12, 2),
           "needles": 64, "workspace_gbytes": round(ws.numel() / 1e9, 2), "stages_per_prefill": stages}
    del pin, out, ws
    torch.cuda.empty_cache()
    return res


def index_topk_forms(pin, pbidx, dev, stream, reps):
    """The Index Branch alone on the headline inputs, in its default two-pass
    form (score table, then top-k) and as the one-pass option
    (MSA_ONE_PASS_INDEX, no table): ms per call (one warmup, then reps),
    workspace bytes, and whether both selections equal the prefill's."""
    res = {}
    for name, fl in (("two_pass", 0), ("one_pass", bd.MSA_ONE_PASS_INDEX)):
        idd = bd.make_dims(1, PF["T"], PF["G"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"],
                           flags=fl)
        nws = bd.msa_workspace_bytes(bd.MSA_OP_INDEX_TOPK, idd)
        iws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        ib = torch.empty((1, PF["T"], PF["G"], PF["k"]), dtype=torch.int32, device=dev)
        fn = lambda: bd.msa_index_topk(idd, pin.idx_q, pin.idx_k, ib, workspace=iws)  # noqa: E731
        fn()
        ms, _ = timed(fn, reps, stream)
        res[f"{name}_ms"] = round(ms, 3)
        res[f"{name}_workspace_bytes"] = int(nws)
        res[f"{name}_equals_prefill_selection"] = bool(torch.equal(ib, pbidx))
        del iws, ib
    return res


def timed(fn, reps, stream):
    """Mean ms of reps launches of fn, HIP events on the launch stream."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return float(np.mean(per)), per


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a stratified sample of tokens
# ---------------------------------------------------------------------------
def cpu_baseline_and_parity(pin, out_gpu, bidx_gpu, n_tokens, time_budget_s):
    from oracle import msa_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    T, Hq, G, d, B, k = PF["T"], PF["Hq"], PF["G"], PF["d"], PF["B"], PF["k"]
    R = Hq // G
    scale = 1.0 / math.sqrt(d)
    # stratified over t, visited in a seeded random order so that any prefix
    # (when the time budget ends the loop early) is still a uniform sample
    ts = [int((i + 0.5) * T / n_tokens) for i in range(n_tokens)]
    ts = [ts[j] for j in np.random.default_rng(0).permutation(n_tokens)]
    # inputs to float64 on the host (not timed)
    K = pin.k[0].cpu().to(torch.float64).numpy()
    V = pin.v[0].cpu().to(torch.float64).numpy()
    IK = pin.idx_k[0].cpu().to(torch.float64).numpy()
    Q = pin.q[0, ts].cpu().to(torch.float64).numpy()
    IQ = pin.idx_q[0, ts].cpu().to(torch.float64).numpy()
    og = out_gpu[0, ts].cpu().to(torch.float64).numpy()
    bg = bidx_gpu[0, ts].cpu().numpy()
    done, spent = 0, 0.0
    sel_equal = sel_neartie = sel_other = 0
    err_abs, err_sum, ref_sum = 0.0, 0.0, 0.0
    for i, t in enumerate(ts):
        t0 = time.perf_counter()
        o_t = np.empty((Hq, d))
        sels, Ss = [], []
        for g in range(G):
            S = orc.block_max(orc.index_scores(IQ[i, g], IK, t), t, B)
            sel = orc.select_blocks(S, t, B, k)
            toks = orc.selected_tokens(sel, t, B)
            o, _ = orc.attention_row(Q[i, g * R:(g + 1) * R], K[:, g], V[:, g], toks, scale)
            o_t[g * R:(g + 1) * R] = o
            sels.append(sel)
            Ss.append(S)
        spent += time.perf_counter() - t0
        done += 1
        for g in range(G):
            if np.array_equal(bg[i, g], sels[g]):
                sel_equal += 1
                diff = np.abs(og[i, g * R:(g + 1) * R] - o_t[g * R:(g + 1) * R])
                err_abs = max(err_abs, float(diff.max()))
                err_sum += float(diff.sum())
                ref_sum += float(np.abs(o_t[g * R:(g + 1) * R]).sum())
            elif orc.near_tie(Ss[g], t, B, k):
                sel_neartie += 1
            else:
                sel_other += 1
        if spent > time_budget_s and done >= 8:
            break
    # stratified sample over t: the mean per-token time estimates the mean
    # over the whole sequence (the oracle's cost is linear in t)
    used = ts[:done]
    cover = (f"stratified over t" if done == n_tokens
             else f"{done} of {n_tokens} stratified positions, in seeded random order")
    cpu = {
        "value": round(done / spent, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
        "sample": f"{done} query tokens ({cover}) of the T=131072 prefill, all 8 groups and 64 heads "
                  f"each: index scores, block max, top-k, gathered fp64 attention; "
                  f"{spent:.1f} s of CPU work; tok/s = tokens / time",
    }
    parity = {
        "rows_checked": done * G, "selection_equal": sel_equal, "selection_near_tie": sel_neartie,
        "selection_other": sel_other, "out_max_abs": err_abs,
        "out_mean_rel": err_sum / max(ref_sum, 1e-300), "t_range": [min(used), max(used)],
    }
    parity["ok"] = bool(sel_other == 0 and err_abs <= 2e-2 and parity["out_mean_rel"] <= 5e-3)
    return cpu, parity


def decode_parity(dec, out_gpu, bidx_gpu, seqs):
    """Oracle check of sampled decode sequences, built from the oracle's own
    steps; only the gathered K/V rows are converted to float64."""
    from oracle import msa_oracle as orc
    B, k, G, Hq, d = DC["B"], DC["k"], DC["G"], DC["Hq"], DC["d"]
    R = Hq // G
    scale = 1.0 / math.sqrt(d)
    worst_abs, sel_ok, near_ties = 0.0, True, 0
    num = den = 0.0
    for s in seqs:
        t = int(dec.cache_lens[s]) - 1
        IK = dec.idx_k_cache[s, : t + 1].cpu().to(torch.float64).numpy()
        IQ = dec.idx_q[s].cpu().to(torch.float64).numpy()
        Q = dec.q[s].cpu().to(torch.float64).numpy()
        og = out_gpu[s].cpu().to(torch.float64).numpy()
        for g in range(G):
            S = orc.block_max(orc.index_scores(IQ[g], IK, t), t, B)
            sel = orc.select_blocks(S, t, B, k)
            got = bidx_gpu[s, g].cpu().numpy()
            if not np.array_equal(sel, got):
                tie = orc.near_tie(S, t, B, k)
                near_ties += int(tie)
                sel_ok = sel_ok and tie
            # attention conditioned on the GPU's own selection
            toks = orc.selected_tokens(got, t, B)
            tk = torch.from_numpy(toks).to(dec.k_cache.device)
            Kg = dec.k_cache[s, tk, g].cpu().to(torch.float64).numpy()
            Vg = dec.v_cache[s, tk, g].cpu().to(torch.float64).numpy()
            o, _ = orc.attention_row(Q[g * R:(g + 1) * R], Kg, Vg, np.arange(len(toks)), scale)
            diff = np.abs(og[g * R:(g + 1) * R] - o)
            worst_abs = max(worst_abs, float(diff.max()))
            num += float(diff.sum())
            den += float(np.abs(o).sum())
    mean_rel = num / max(den, 1e-300)
    return {"sequences_checked": list(seqs), "selection_ok": bool(sel_ok), "near_tie_groups": near_ties,
            "out_max_abs": worst_abs, "out_mean_rel": mean_rel,
            "ok": bool(sel_ok and worst_abs <= 2e-2 and mean_rel <= 5e-3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true", help="skip the all-blocks comparison")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (CPU baseline + parity)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the block-size sweep, 32K prefill and forced-sink timings")
    ap.add_argument("--no-backward", action="store_true", help="skip the main-branch backward at 128K")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--profile-1m", action="store_true",
                    help="run only the 1M-token prefill (one warmup, two timed, one staged) for a rocprofv3 pass")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="run only prefills and decode steps (plus a calibration copy) for rocprofv3 passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    bd.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.profile_kernels:
        profile_kernels_only(args, dev)
        return
    if args.profile_1m:
        print(json.dumps({"prefill_t1048576_b128_k16_needles": prefill_1m_run(dev, torch.cuda.current_stream())}),
              flush=True)
        return

    log("generating prefill inputs (T=131072)")
    pin = inputs.make_prefill(PF["T"], PF["Hq"], PF["G"], PF["d"], PF["di"], seed=PF["seed"], device=dev,
                              block_size=PF["B"], skew_std=PF["skew"])
    pdims = bd.make_dims(1, PF["T"], PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"])
    pout = torch.empty_like(pin.q)
    plse = torch.empty((1, PF["T"], PF["Hq"]), dtype=torch.float32, device=dev)
    pbidx = torch.empty((1, PF["T"], PF["G"], PF["k"]), dtype=torch.int32, device=dev)
    pws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, pdims), dtype=torch.uint8, device=dev)

    log("generating decode inputs (8 x 1M context)")
    dec = inputs.make_decode(DC["batch"], DC["L"], DC["Hq"], DC["G"], DC["d"], DC["di"], seed=DC["seed"],
                             device=dev)
    ddims = bd.make_dims(DC["batch"], DC["L"], DC["Hq"], DC["G"], index_dim=DC["di"], block_size=DC["B"],
                         topk=DC["k"])
    dout = torch.empty((DC["batch"], DC["Hq"], DC["d"]), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((DC["batch"], DC["Hq"]), dtype=torch.float32, device=dev)
    dbidx = torch.empty((DC["batch"], DC["G"], DC["k"]), dtype=torch.int32, device=dev)
    dws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_DECODE, ddims), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        bd.msa_prefill(pdims, pin.q, pin.k, pin.v, pin.idx_q, pin.idx_k, pout, lse=plse, block_idx=pbidx,
                       workspace=pws)

    def decode():
        bd.msa_decode(ddims, dec.q, dec.k_cache, dec.v_cache, dec.idx_q, dec.idx_k_cache, dec.cache_lens,
                      dout, lse=dlse, block_idx=dbidx, workspace=dws)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        prefill()
        evs[i][1].record(stream)
        decode()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0

    # A second pass of the same steps with the library's per-stage HIP events
    # (recorded on the launch stream around every kernel stage) gives each
    # kernel's live launch time; the events cost ~16 us per decode step, so
    # they stay out of the pass above.
    bd.msa_profile_begin()
    for i in range(args.steps):
        prefill()
        decode()
    torch.cuda.synchronize()
    stage = {n: t / c for n, (c, t) in bd.msa_profile_end().items()}
    log("stage ms: " + ", ".join(f"{n} {v:.3f}" for n, v in stage.items()))
    p_all = [e[0].elapsed_time(e[1]) for e in evs]
    d_all = [e[1].elapsed_time(e[2]) for e in evs]
    p_ms, d_ms = float(np.mean(p_all)), float(np.mean(d_all))
    log(f"prefill {p_ms:.3f} ms  decode {d_ms:.3f} ms  wall/step {1e3 * wall / args.steps:.3f} ms")

    # per-kernel rooflines of the prefill (one query chunk covers T=131072,
    # so each stage is one launch per prefill)
    f_index, f_main = prefill_flops(PF["T"], PF["Hq"], PF["G"], PF["d"], PF["di"], PF["B"], PF["k"])
    dbytes = decode_bytes(DC["batch"], DC["L"], DC["Hq"], DC["G"], DC["d"], DC["di"], DC["B"], DC["k"])
    kvb, n_entries, n_blocks = kv_outer_bytes(pbidx, PF["T"], PF["Hq"], PF["G"], PF["d"], PF["B"], PF["k"])
    qmb = query_major_bytes(n_entries, PF["T"], PF["Hq"], PF["G"], PF["d"], PF["B"])
    rooflines = {}
    name_idx, name_kv, name_qm = (bd.msa_stage_name(bd.MSA_STAGE_INDEX_PREFILL), bd.msa_stage_name(bd.MSA_STAGE_KV_OUTER),
                                  bd.msa_stage_name(bd.MSA_STAGE_QUERY_MAJOR))
    compulsory = compulsory_prefill_bytes(PF["T"], PF["Hq"], PF["G"], PF["d"], PF["di"], PF["k"])
    f_kv = kv_outer_flops(n_entries, PF["Hq"], PF["G"], PF["d"], PF["B"])
    f_loc = local_block_flops(PF["T"], PF["Hq"], PF["d"], PF["B"])

    def mfma_roofline(name, kernel, flops, impl_bytes=None):
        # every prefill kernel is held to the bf16 MFMA peak on the method's
        # own flops (the prefill is MFMA-bound once K/V are reused); the bytes
        # the design itself moves are reported beside it, as is the ratio of
        # the counter-measured traffic to the prefill's compulsory bytes
        ms = stage[name]
        a = flops / (ms * 1e-3)
        traffic = measured_traffic(kernel)
        r = {"bound": "mfma", "achieved": round(a / 1e12, 2), "peak": 2500.0, "unit": "TFLOP/s",
             "frac": round(a / PEAK_MFMA_BF16, 4), "traffic": traffic, "launch_ms": round(ms, 4),
             "algorithmic_tflop_per_launch": round(flops / 1e12, 4),
             "traffic_ratio": None if traffic is None else round(traffic / compulsory, 2)}
        if impl_bytes is not None:
            r["implementation_gbytes_per_launch"] = round(impl_bytes / 1e9, 3)
            r["implementation_gbs"] = round(impl_bytes / (ms * 1e-3) / 1e9, 1)
            r["implementation_hbm_frac"] = round(impl_bytes / (ms * 1e-3) / PEAK_HBM, 4)
        return r

    if name_idx in stage:
        rooflines[name_idx] = mfma_roofline(name_idx, "index_blockmax_prefill_kernel", f_index)
    if name_kv in stage:
        rooflines[name_kv] = mfma_roofline(name_kv, "kv_outer_kernel", f_kv, kvb)
        rooflines[name_kv].update(entries=n_entries, distinct_blocks=n_blocks)
    if name_qm in stage:
        rooflines[name_qm] = mfma_roofline(name_qm, "query_major_kernel", f_loc, qmb)
    prefill_stages = [n for n in stage if n in rooflines]
    dominant = max(prefill_stages, key=lambda n: stage[n]) if prefill_stages else None

    dense = None
    if not args.no_dense:
        log("dense (all blocks) comparison")
        dpd = bd.make_dims(1, PF["T"], PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"],
                           topk=PF["k"], flags=bd.MSA_DENSE)
        dout2 = torch.empty_like(pout)
        pd_fn = lambda: bd.msa_prefill(dpd, pin.q, pin.k, pin.v, None, None, dout2)  # noqa: E731
        pd_fn()
        pd_ms, _ = timed(pd_fn, 2, stream)
        ddd = bd.make_dims(DC["batch"], DC["L"], DC["Hq"], DC["G"], index_dim=DC["di"], block_size=DC["B"],
                           topk=DC["k"], flags=bd.MSA_DENSE)
        dws2 = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_DECODE, ddd), dtype=torch.uint8, device=dev)
        dd_fn = lambda: bd.msa_decode(ddd, dec.q, dec.k_cache, dec.v_cache, None, None, dec.cache_lens,  # noqa: E731
                                      torch.empty_like(dout), workspace=dws2)
        dd_fn()
        dd_ms, _ = timed(dd_fn, 3, stream)
        del dout2, dws2
        dense = {
            "prefill_ms": round(pd_ms, 3), "decode_ms": round(dd_ms, 4),
            "prefill_speedup": round(pd_ms / p_ms, 3), "decode_speedup": round(dd_ms / d_ms, 3),
            "prefill_tflops": round(dense_prefill_flops(PF["T"], PF["Hq"], PF["d"]) / (pd_ms * 1e-3) / 1e12, 2),
            "analytic_prefill_cap": round(dense_prefill_flops(PF["T"], PF["Hq"], PF["d"]) / (f_index + f_main), 3),
        }
        log(f"dense prefill {pd_ms:.2f} ms, dense decode {dd_ms:.3f} ms")

    # The other prefill workloads of the pages' shapes, one timing each (not
    # the headline): the 128K block-size sweep (same 2048 attended tokens),
    # the 32K prefill, and the forced-sink variant of the headline workloads.
    variants = None
    if not args.no_variants:
        log("variant workloads")
        variants = {}
        vbuf = torch.empty_like(pout)  # the headline output stays intact for the checks below
        for B_, k_ in ((64, 32), (32, 64)):
            vd = bd.make_dims(1, PF["T"], PF["Hq"], PF["G"], index_dim=PF["di"], block_size=B_, topk=k_)
            vin = inputs.make_prefill(PF["T"], PF["Hq"], PF["G"], PF["d"], PF["di"], seed=PF["seed"], device=dev,
                                      block_size=B_, skew_std=PF["skew"])
            vws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, vd), dtype=torch.uint8, device=dev)
            fn = lambda: bd.msa_prefill(vd, vin.q, vin.k, vin.v, vin.idx_q, vin.idx_k, vbuf, workspace=vws)  # noqa: E731
            fn()
            ms, _ = timed(fn, 3, stream)
            variants[f"prefill_t131072_b{B_}_k{k_}"] = {"ms": round(ms, 3),
                                                        "tok_s": round(PF["T"] / (ms * 1e-3), 1)}
            del vin, vws
        T2 = 32768
        vd = bd.make_dims(1, T2, PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"])
        vin = inputs.make_prefill(T2, PF["Hq"], PF["G"], PF["d"], PF["di"], seed=2, device=dev, block_size=PF["B"])
        vout = torch.empty_like(vin.q)
        vws = torch.empty(bd.msa_workspace_bytes(bd.MSA_OP_PREFILL, vd), dtype=torch.uint8, device=dev)
        fn = lambda: bd.msa_prefill(vd, vin.q, vin.k, vin.v, vin.idx_q, vin.idx_k, vout, workspace=vws)  # noqa: E731
        fn()
        ms, _ = timed(fn, 5, stream)
        fi2, fm2 = prefill_flops(T2, PF["Hq"], PF["G"], PF["d"], PF["di"], PF["B"], PF["k"])
        variants["prefill_t32768_b128_k16"] = {"ms": round(ms, 3), "tok_s": round(T2 / (ms * 1e-3), 1),
                                               "tflops": round((fi2 + fm2) / (ms * 1e-3) / 1e12, 2)}
        del vin, vout, vws
        sd = bd.make_dims(1, PF["T"], PF["Hq"], PF["G"], index_dim=PF["di"], block_size=PF["B"], topk=PF["k"],
                          flags=bd.MSA_FORCE_SINK)
        fn = lambda: bd.msa_prefill(sd, pin.q, pin.k, pin.v, pin.idx_q, pin.idx_k, vbuf, workspace=pws)  # noqa: E731
        fn()
        ms, _ = timed(fn, 3, stream)
        variants["prefill_t131072_sink"] = {"ms": round(ms, 3), "tok_s": round(PF["T"] / (ms * 1e-3), 1)}
        sdd = bd.make_dims(DC["batch"], DC["L"], DC["Hq"], DC["G"], index_dim=DC["di"], block_size=DC["B"],
                           topk=DC["k"], flags=bd.MSA_FORCE_SINK)
        sink_out = torch.empty_like(dout)   # the headline decode output stays intact for the checks below
        fn = lambda: bd.msa_decode(sdd, dec.q, dec.k_cache, dec.v_cache, dec.idx_q, dec.idx_k_cache,  # noqa: E731
                                   dec.cache_lens, sink_out, workspace=dws)
        fn()
        ms, _ = timed(fn, 10, stream)
        variants["decode_8x1m_sink"] = {"ms": round(ms, 4), "tok_s": round(DC["batch"] / (ms * 1e-3), 1)}
        # indexer KL loss + gradient on the headline prefill's own selection and lse
        ms, kl_out = indexer_kl_ms(pin, pbidx, plse, dev, stream, 3, keep=True)
        kl_flops = indexer_kl_flops(PF["T"], PF["Hq"], PF["G"], PF["d"], PF["di"], PF["B"], PF["k"])
        variants["indexer_kl_t131072"] = {"ms": round(ms, 3), "tok_s": round(PF["T"] / (ms * 1e-3), 1),
                                          "algorithmic_tflop": round(kl_flops / 1e12, 3),
                                          "tflops": round(kl_flops / (ms * 1e-3) / 1e12, 2)}
        if not args.no_cpu:
            variants["indexer_kl_t131072"]["sampled_check"] = indexer_kl_checks(pin, pbidx, kl_out)
        del kl_out
        # the Index Branch alone, two-pass (default) and one-pass
        variants["index_topk_t131072"] = index_topk_forms(pin, pbidx, dev, stream, 3)
        del vbuf
        log(f"variants: {variants}")

    # The main-branch backward (selection held fixed) on the headline
    # prefill's output: a second workload of the same shapes, not in `value`.
    backward = None
    if not args.no_backward:
        log("main-branch backward at 128K")
        bms, bper, bst, btens = backward_run(pin, pout, plse, pbidx, dev, stream, 3)
        bflops = backward_flops(PF["T"], PF["Hq"], PF["d"], PF["B"], PF["k"])
        bbytes, b_entries, b_lists = bwd_list_bytes(pbidx, PF["T"], PF["Hq"], PF["G"], PF["d"], PF["B"])
        name_bl = bd.msa_stage_name(bd.MSA_STAGE_BWD_LISTS)
        bl_ms = bst.get(name_bl)
        backward = {
            "workload": "MSA main-branch backward T=131072 (B=128, k=16) on the prefill's own output and "
                        "selection, seeded d out",
            "ms": round(bms, 3), "median_ms": round(float(np.median(bper)), 3),
            "tok_s": round(PF["T"] / (bms * 1e-3), 1),
            "algorithmic_tflop": round(bflops / 1e12, 3),
            "tflops": round(bflops / (bms * 1e-3) / 1e12, 2),
            "stage_ms": {n: round(v, 4) for n, v in bst.items()},
            "roofline": None if bl_ms is None else {
                "kernel": name_bl, "bound": "hbm", "achieved": round(bbytes / (bl_ms * 1e-3) / 1e9, 1),
                "peak": 8000.0, "unit": "GB/s", "frac": round(bbytes / (bl_ms * 1e-3) / PEAK_HBM, 4),
                "traffic": measured_traffic("bwd_list_kernel"), "launch_ms": round(bl_ms, 4),
                "algorithmic_gbytes_per_launch": round(bbytes / 1e9, 3), "entries": b_entries, "lists": b_lists,
                "mfma_tflops": round(bflops / (bl_ms * 1e-3) / 1e12, 1)},
        }
        if not args.no_cpu:
            backward["sampled_check"] = backward_checks(pin, pbidx, btens)
        del btens
        log(f"backward: {backward}")

    peaks = measured_peaks(dev)
    cpu, parity, dparity = None, None, None
    if not args.no_cpu:
        log("oracle leg on host cores")
        cpu, parity = cpu_baseline_and_parity(pin, pout, pbidx, args.cpu_tokens, args.cpu_seconds)
        dparity = decode_parity(dec, dout, dbidx, seqs=list(range(DC["batch"])))

    if variants is not None:
        # the 1M-token prefill last, after the decode caches and the 128K
        # workspace are released
        del dec, dws, pws
        torch.cuda.empty_cache()
        log("prefill at T=1,048,576 (64 needle blocks)")
        variants["prefill_t1048576_b128_k16_needles"] = prefill_1m_run(dev, stream)
        log(f"1M prefill: {variants['prefill_t1048576_b128_k16_needles']}")

    prefill_tok_s = PF["T"] / (p_ms * 1e-3)
    decode_tok_s = DC["batch"] / (d_ms * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(prefill_tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "MSA prefill T=131072 (B=128, k=16, per-block skewed idx_k) + MSA decode 8 seq x 1,048,576 ctx (B=128, k=16)",
            "batch": 1, "seq_len": PF["T"], "q_heads": PF["Hq"], "kv_heads": PF["G"], "head_dim": PF["d"],
            "index_dim": PF["di"], "block_size": PF["B"], "topk": PF["k"],
            "decode_batch": DC["batch"], "decode_context": DC["L"],
        },
        "prefill": {
            "compulsory_gbytes": round(compulsory / 1e9, 3),
            "ms": round(p_ms, 4), "median_ms": round(float(np.median(p_all)), 4), "tok_s": round(prefill_tok_s, 1),
            "algorithmic_tflop": round((f_index + f_main) / 1e12, 3),
            "tflops": round((f_index + f_main) / (p_ms * 1e-3) / 1e12, 2),
            "mfma_frac": round((f_index + f_main) / (p_ms * 1e-3) / PEAK_MFMA_BF16, 4),
            "frac_of_measured_gemm": round((f_index + f_main) / (p_ms * 1e-3) / 1e12
                                           / peaks["bf16_gemm_8192_tflops"], 4),
        },
        "decode": {
            "ms": round(d_ms, 4), "median_ms": round(float(np.median(d_all)), 4), "tok_s": round(decode_tok_s, 1),
            "algorithmic_gbytes": round(dbytes / 1e9, 4),
            "roofline": {"bound": "hbm", "scope": "whole decode step (all kernels)",
                         "achieved": round(dbytes / (d_ms * 1e-3) / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
                         "frac": round(dbytes / (d_ms * 1e-3) / PEAK_HBM, 4),
                         "frac_of_measured_copy": round(dbytes / (d_ms * 1e-3) / 1e9 / peaks["device_copy_gbs"], 4),
                         "traffic": {k_: measured_traffic(k_) for k_ in ("decode_index_kernel", "decode_attn_kernel")}},
        },
        "roofline": dict(kernel=dominant, **rooflines[dominant]) if dominant else None,
        "kernel_rooflines": rooflines,
        "stage_ms": {n: round(v, 4) for n, v in stage.items()},
        "dense": dense,
        "variants": variants,
        "backward": backward,
        "measured_peaks": peaks,
        "parity": {"prefill_sampled": parity, "decode_sampled": dparity},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

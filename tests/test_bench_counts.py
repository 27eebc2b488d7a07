"""Host-side checks of the algorithmic counts bench.py divides by time for its
rooflines: closed forms against brute-force enumeration on small shapes, and
the totals at the benchmark's 128K prefill and 8 x 1M decode."""
import numpy as np
import torch

import bench


def _attended_keys(t, B, sel):
    """Visible keys of the selected blocks of query t (keys j <= t)."""
    return sum(len([j for j in range(b * B, (b + 1) * B) if j <= t]) for b in sel)


def test_prefill_flops_brute_force():
    T, Hq, G, d, di, B, k = 700, 6, 3, 16, 8, 32, 5
    rng = np.random.default_rng(0)
    idx_ref = main_ref = 0.0
    for t in range(T):
        L = t // B
        nonlocal_ = rng.choice(L, size=min(k - 1, L), replace=False) if L > 0 else []
        sel = list(nonlocal_) + [L]
        idx_ref += 2.0 * G * di * (t + 1)                      # every visible key scored per group
        main_ref += 4.0 * Hq * d * _attended_keys(t, B, sel)  # QK^T and PV per head and attended key
    idx, main = bench.prefill_flops(T, Hq, G, d, di, B, k)
    assert idx == idx_ref and main == main_ref


def test_prefill_flops_at_128k():
    idx, main = bench.prefill_flops(131072, 64, 8, 128, 128, 128, 16)
    assert abs(idx - 1.759e13) / 1.759e13 < 1e-3
    assert abs(main - 8.46e12) / 8.46e12 < 2e-3


def test_decode_bytes_brute_force_and_8x1m():
    batch, L, Hq, G, d, di, B, k = 3, 1000, 8, 2, 16, 8, 64, 4
    t = L - 1
    sel = list(range(k - 1)) + [t // B]           # any k-1 full blocks plus the local one
    att = _attended_keys(t, B, sel)
    per_seq = L * di * 2 + G * att * d * 2 * 2 + Hq * d * 2 * 2 + G * di * 2  # idx_k, K and V, q and out, idx_q
    assert bench.decode_bytes(batch, L, Hq, G, d, di, B, k) == batch * per_seq
    total = bench.decode_bytes(8, 1 << 20, 64, 8, 128, 128, 128, 16)
    assert abs(total - 2.2149e9) / 2.2149e9 < 1e-3


def test_kv_outer_and_query_major_bytes_count_entries():
    T, Hq, G, d, B, k = 300, 4, 2, 16, 32, 3
    rng = np.random.default_rng(1)
    bidx = torch.full((1, T, G, k), -1, dtype=torch.int32)
    for t in range(T):
        L = t // B
        for g in range(G):
            pick = sorted(rng.choice(L, size=min(k - 1, L), replace=False).tolist()) if L > 0 else []
            row = pick + [L]
            bidx[0, t, g, :len(row)] = torch.tensor(row, dtype=torch.int32)
    got, entries, blocks = bench.kv_outer_bytes(bidx, T, Hq, G, d, B, k)
    ref_entries = sum(int(((bidx[0, t] >= 0) & (bidx[0, t] < t // B)).sum()) for t in range(T))
    ref_blocks = len({(g, int(b)) for t in range(T) for g in range(G) for b in bidx[0, t, g].tolist()
                      if 0 <= b < t // B})
    R = Hq // G
    assert entries == ref_entries and blocks == ref_blocks
    assert got == entries * (R * d * 2 + R * (d * 2 + 8) + 4) + blocks * 2 * B * d * 2
    qm = bench.query_major_bytes(entries, T, Hq, G, d, B)
    nb = (T + B - 1) // B
    assert qm == T * Hq * (4 * d + 4) + entries * (R * (2 * d + 8) + 4) + G * nb * 4 * B * d


def test_compulsory_bytes_and_kv_outer_flops():
    # every input read once and every output written once, tensor by tensor
    T, Hq, G, d, di, k = 131072, 64, 8, 128, 128, 16
    tensors = {"q": T * Hq * d * 2, "k": T * G * d * 2, "v": T * G * d * 2, "idx_q": T * G * di * 2,
               "idx_k": T * di * 2, "out": T * Hq * d * 2, "lse": T * Hq * 4, "block_idx": T * G * k * 4}
    assert bench.compulsory_prefill_bytes(T, Hq, G, d, di, k) == sum(tensors.values())
    assert abs(sum(tensors.values()) - 5.23e9) / 5.23e9 < 5e-3
    # one entry: a 128-key block against R = 8 heads, QK^T and PV, 2 flops per MAC
    assert bench.kv_outer_flops(1, 64, 8, 128, 128) == 2 * 2 * 128 * 128 * 8
    # local blocks: brute force over a small case
    T, Hq, d, B = 300, 4, 16, 32
    ref = sum(4.0 * Hq * d * len(range((t // B) * B, t + 1)) for t in range(T))
    assert bench.local_block_flops(T, Hq, d, B) == ref

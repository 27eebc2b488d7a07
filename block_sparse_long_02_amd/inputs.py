"""Seeded synthetic inputs for the MSA forward path.

This module is shared by the tests, the benchmark and the oracle checks.  It
only draws random tensors and places them in the library's layouts; it holds
none of the method's arithmetic (no scores, no pooling, no selection, no
softmax).  Every value is rounded to bfloat16 (round-to-nearest-even) by
torch's own conversion, so the same bits feed the HIP path (as bf16) and the
oracle (as exactly representable float64).

Layouts (row-major, innermost last), as the C ABI declares them:
  prefill  q [b,T,Hq,d]  k,v [b,T,G,d]  idx_q [b,T,G,di]  idx_k [b,T,di]
  decode   q [b,Hq,d]    k_cache,v_cache [b,L,G,d]  idx_q [b,G,di]
           idx_k_cache [b,L,di]  cache_lens [b] int32

Generation runs chunk by chunk along the token axis with one generator, so a
given (seed, device, chunk size) always yields the same tensors while the fp32
staging buffer stays small (the 1M-token workloads need this on the GPU).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Elements drawn per randn call; part of the definition of the stream.
_DRAW = 1 << 24
# Token rows per draw for the per-row loops below.
_CHUNK = 1 << 14


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian_bf16(shape, gen, device, scale: float = 1.0) -> torch.Tensor:
    """iid N(0, scale^2) rounded to bf16, drawn in row chunks of the tensor
    flattened to [-1, last_dim]."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, *shape[-1:]) if len(shape) > 1 else out.view(1, -1)
    rows = flat.shape[0]
    step = max(1, _DRAW // max(1, flat.shape[1]))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                        dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[r0:r1].copy_(x)
    return out


def integer_bf16(shape, gen, device, lo: int = -3, hi: int = 3) -> torch.Tensor:
    """Uniform integers in [lo, hi], exact in bf16."""
    x = torch.randint(lo, hi + 1, shape, generator=gen, device=device, dtype=torch.int32)
    return x.to(torch.bfloat16)


@dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    idx_q: torch.Tensor
    idx_k: torch.Tensor
    meta: dict = field(default_factory=dict)


@dataclass
class DecodeInputs:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    idx_q: torch.Tensor
    idx_k_cache: torch.Tensor
    cache_lens: torch.Tensor
    meta: dict = field(default_factory=dict)


def make_prefill(T: int, Hq: int, G: int, d: int, di: int, *, batch: int = 1,
                 seed: int = 0, device="cpu", idx_mode: str = "gaussian",
                 block_size: int | None = None, skew_std: float = 0.0,
                 needles: int = 0, needle_preset: str = "separable",
                 needle_q_mean: float = 8.0) -> PrefillInputs:
    """Prefill tensors.

    idx_mode   'gaussian' (iid N(0,1)) or 'integer' (uniform in [-3, 3]; exact
               index dot products in fp32, for bit-exact selection checks).
    skew_std   > 0: every aligned block b of idx_k gets its own mean vector
               mu_b ~ N(0, skew_std^2 I) added to all its rows (skewed block
               popularity).  Needs block_size.
    needles    number of distinct aligned blocks whose idx_k rows are shifted
               along a direction u.  'separable': u is a seeded unit vector,
               idx_q = N(0,1) + needle_q_mean u (so u is idx_q's mean direction;
               at the default 8 every row's projection q.u = 8 + N(0,1) stays
               well above 0 even over millions of rows, at 4 about 1 row in
               4 000 falls below 0.5) and needle keys = N(0,1) + 2 sqrt(di) u.
               'literal': idx_q iid N(0,1), u = normalised mean of the drawn
               idx_q rows, needle keys += 2u.
    """
    gen = _gen(seed, device)
    q = gaussian_bf16((batch, T, Hq, d), gen, device)
    k = gaussian_bf16((batch, T, G, d), gen, device)
    v = gaussian_bf16((batch, T, G, d), gen, device)
    meta = {"T": T, "Hq": Hq, "G": G, "d": d, "di": di, "batch": batch,
            "seed": seed, "idx_mode": idx_mode}
    if idx_mode == "integer":
        idx_q = integer_bf16((batch, T, G, di), gen, device)
        idx_k = integer_bf16((batch, T, di), gen, device)
        return PrefillInputs(q, k, v, idx_q, idx_k, meta)
    if idx_mode != "gaussian":
        raise ValueError(f"unknown idx_mode {idx_mode!r}")

    if needles and needle_preset == "separable":
        u = torch.randn((di,), generator=gen, device=device, dtype=torch.float32)
        u = u / u.norm()
        idx_q = torch.empty((batch, T, G, di), dtype=torch.bfloat16, device=device)
        fq = idx_q.view(-1, di)
        step = _CHUNK * 8
        for r0 in range(0, fq.shape[0], step):
            r1 = min(fq.shape[0], r0 + step)
            x = torch.randn((r1 - r0, di), generator=gen, device=device, dtype=torch.float32)
            fq[r0:r1].copy_(x + needle_q_mean * u)
        meta["needle_dir"] = u.cpu()
        meta["needle_q_mean"] = needle_q_mean
    else:
        idx_q = gaussian_bf16((batch, T, G, di), gen, device)

    if skew_std > 0.0 or needles:
        if block_size is None:
            raise ValueError("skew / needles need block_size")
        B = block_size
        nb = (T + B - 1) // B
        idx_k = torch.empty((batch, T, di), dtype=torch.bfloat16, device=device)
        mu = None
        if skew_std > 0.0:
            mu = torch.randn((batch, nb, di), generator=gen, device=device,
                             dtype=torch.float32) * skew_std
            meta["skew_std"] = skew_std
        needle_blocks = None
        if needles:
            perm = torch.randperm(nb, generator=gen, device=device)[:needles]
            needle_blocks = torch.sort(perm).values
            meta["needle_blocks"] = needle_blocks.cpu()
            meta["needle_preset"] = needle_preset
            if needle_preset == "separable":
                shift = (2.0 * math.sqrt(di)) * meta["needle_dir"].to(device)
            elif needle_preset == "literal":
                mean = idx_q.float().view(-1, di).mean(0)
                shift = 2.0 * mean / mean.norm()
                meta["needle_dir"] = (mean / mean.norm()).cpu()
            else:
                raise ValueError(f"unknown needle_preset {needle_preset!r}")
            is_needle = torch.zeros((nb,), dtype=torch.bool, device=device)
            is_needle[needle_blocks] = True
        step = max(B, (_CHUNK // B) * B)
        for bi in range(batch):
            for t0 in range(0, T, step):
                t1 = min(T, t0 + step)
                x = torch.randn((t1 - t0, di), generator=gen, device=device,
                                dtype=torch.float32)
                blk = torch.arange(t0, t1, device=device) // B
                if mu is not None:
                    x += mu[bi, blk]
                if needle_blocks is not None:
                    x += is_needle[blk].to(torch.float32)[:, None] * shift[None, :]
                idx_k[bi, t0:t1].copy_(x)
    else:
        idx_k = gaussian_bf16((batch, T, di), gen, device)
    return PrefillInputs(q, k, v, idx_q, idx_k, meta)


def make_decode(batch: int, L: int, Hq: int, G: int, d: int, di: int, *, seed: int = 0,
                device="cpu", cache_lens=None, idx_mode: str = "gaussian") -> DecodeInputs:
    """Decode tensors: caches of capacity L per sequence and one new query
    token per sequence.  cache_lens (each including the new token) defaults
    to L for every sequence."""
    gen = _gen(seed, device)
    q = gaussian_bf16((batch, Hq, d), gen, device)
    k_cache = gaussian_bf16((batch, L, G, d), gen, device)
    v_cache = gaussian_bf16((batch, L, G, d), gen, device)
    if idx_mode == "integer":
        idx_q = integer_bf16((batch, G, di), gen, device)
        idx_k = integer_bf16((batch, L, di), gen, device)
    else:
        idx_q = gaussian_bf16((batch, G, di), gen, device)
        idx_k = gaussian_bf16((batch, L, di), gen, device)
    if cache_lens is None:
        cache_lens = [L] * batch
    lens = torch.tensor(list(cache_lens), dtype=torch.int32, device=device)
    meta = {"batch": batch, "L": L, "Hq": Hq, "G": G, "d": d, "di": di, "seed": seed}
    return DecodeInputs(q, k_cache, v_cache, idx_q, idx_k, lens, meta)

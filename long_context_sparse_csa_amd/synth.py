"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module draws random numbers and stores them in the input formats the
library consumes (bf16, fp32, packed E4M3|bf16 rows via torch's own casts).
It contains none of the attention method's arithmetic: no pooling, scoring,
selection, normalisation or rotation.

Every tensor is drawn from its own torch.Generator whose seed is derived from
(workload seed, tensor name), so a tensor does not change when another one is
added or resized.  The same seed gives the same values on the same device
type; the oracle always reads the bytes the GPU reads (copied to host).
"""

import zlib

import torch


def _seed(seed, name):
    return (int(seed) * 1_000_003 + zlib.crc32(name.encode())) % (2 ** 62)


def _gen(seed, name, device):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name))
    return g


def normal(shape, seed, name, device="cpu", std=1.0, mean=0.0,
           dtype=torch.float32):
    """N(mean, std^2) values, drawn in float32 and cast (RNE) to dtype."""
    g = _gen(seed, name, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def integers(shape, lo, hi, seed, name, device="cpu", dtype=torch.float32):
    """Uniform integers in [lo, hi], stored exactly in dtype."""
    g = _gen(seed, name, device)
    x = torch.randint(lo, hi + 1, shape, generator=g, device=device)
    return x.to(dtype)


def e4m3_codes(shape, seed, name, device="cpu"):
    """Uniform random finite OCP E4M3FN codes, uint8 (the NaN codes 0x7F and
    0xFF are never drawn)."""
    g = _gen(seed, name, device)
    x = torch.randint(0, 254, shape, generator=g, device=device)
    x = x + (x >= 0x7F).to(x.dtype)
    return x.to(torch.uint8)


def e4m3_rows(shape, seed, name, device="cpu", chunk_rows=1 << 20):
    """N(0,1) rows stored as E4M3FN codes with one fp32 scale per row (the
    row's largest magnitude / 448, so the largest value maps to 448): codes
    uint8 [*shape], scales float32 [*shape[:-1]] (torch casts)."""
    d = shape[-1]
    rows = 1
    for s in shape[:-1]:
        rows *= s
    codes = torch.empty((rows, d), dtype=torch.uint8, device=device)
    scales = torch.empty((rows,), dtype=torch.float32, device=device)
    g = _gen(seed, name, device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = torch.randn((r1 - r0, d), generator=g, device=device)
        sc = v.abs().amax(dim=1).clamp_min(1e-30) / 448.0
        codes[r0:r1] = (v / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scales[r0:r1] = sc
    return codes.view(*shape), scales.view(*shape[:-1])


def mxfp4_codes(shape, d, seed, name, device="cpu", scale_lo=120, scale_hi=134):
    """Uniform random MXFP4 rows: packed E2M1 codes uint8 [*shape, d/2] (every
    nibble is a valid code) and E8M0 scales uint8 [*shape, d/32] uniform in
    [scale_lo, scale_hi]."""
    g = _gen(seed, name, device)
    codes = torch.randint(0, 256, (*shape, d // 2), generator=g, device=device).to(torch.uint8)
    scales = torch.randint(scale_lo, scale_hi + 1, (*shape, d // 32), generator=g,
                           device=device).to(torch.uint8)
    return codes, scales


def mxfp4_rows(shape, seed, name, device="cpu", chunk_rows=1 << 18):
    """N(0,1) rows [*shape] (last dim d) in the OCP MX FP4 format: per block of
    32 values the E8M0 scale 2^(floor(log2(amax)) - 2) (the largest magnitude
    lands in [4, 8) and saturates at 6), elements rounded half-to-even onto
    the E2M1 grid.  Returns packed codes uint8 [..., d/2] and scales uint8
    [..., d/32]."""
    d = shape[-1]
    rows = 1
    for s_ in shape[:-1]:
        rows *= s_
    codes = torch.empty((rows, d // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, d // 32), dtype=torch.uint8, device=device)
    g = _gen(seed, name, device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = torch.randn((r1 - r0, d // 32, 32), generator=g, device=device)
        amax = v.abs().amax(dim=2).clamp_min(2.0 ** -100)
        x = torch.floor(torch.log2(amax)) - 2.0
        a = (v.abs() / torch.exp2(x)[..., None]).clamp_max(6.0)
        q = torch.where(a < 2.0, torch.round(a * 2.0) / 2.0,
                        torch.where(a < 4.0, torch.round(a), torch.round(a / 2.0) * 2.0))
        q = q.clamp_max(6.0)
        # magnitude -> code: 0, .5, 1, 1.5 -> 0..3; 2, 3 -> 4, 5; 4, 6 -> 6, 7
        mag = torch.where(q < 2.0, q * 2.0, torch.where(q < 4.0, q + 2.0, q / 2.0 + 4.0))
        c = mag.to(torch.int32) | ((v < 0) & (mag > 0)).to(torch.int32) * 8
        c = c.view(r1 - r0, d)
        codes[r0:r1] = (c[:, 0::2] | (c[:, 1::2] << 4)).to(torch.uint8)
        scales[r0:r1] = (x + 127.0).to(torch.uint8)
    return codes.view(*shape[:-1], d // 2), scales.view(*shape[:-1], d // 32)


def pack_values(vals, R):
    """float32 [..., D] -> uint8 [..., D+R]: E4M3FN codes of dims [0, D-R)
    followed by little-endian bf16 of dims [D-R, D) (torch casts)."""
    D = vals.shape[-1]
    lo = vals[..., : D - R].to(torch.float8_e4m3fn).view(torch.uint8)
    hi = vals[..., D - R:].contiguous().to(torch.bfloat16).view(torch.uint8)
    return torch.cat([lo, hi], dim=-1).contiguous()


def packed_rows(shape, D, R, seed, name, device="cpu", chunk_rows=1 << 20):
    """Packed rows whose D values are N(0,1): uint8 [*shape, D+R].

    Drawn in row chunks so that very large caches need little scratch."""
    rows = 1
    for s in shape:
        rows *= s
    out = torch.empty((rows, D + R), dtype=torch.uint8, device=device)
    g = _gen(seed, name, device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = torch.randn((r1 - r0, D), generator=g, device=device)
        out[r0:r1] = pack_values(v, R)
    return out.view(*shape, D + R)

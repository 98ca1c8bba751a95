"""Seeded synthetic inputs for the selective scan and its decode step.

This module only draws numbers. It holds none of the scan's arithmetic, and both
the fp64 oracle (tests, CPU baseline) and the HIP path (tests, bench, smoke) read
the exact same bits from it: the oracle widens the stored bf16/fp32 values to
fp64 exactly, the GPU reads them as they are.

Shapes follow the Mamba layer sizes the pages name (Mamba 130M and 2.8B from
"Mamba: How Selective State Spaces Achieve 5x Faster Inference Than
Transformers", section "What the numbers show: throughput and quality";
million-length sequences from "Mamba: Linear-Time Sequence Modeling with
Selective State Spaces", "Key points"; d_state = 16 from "Mamba Architecture
Explained", section "The Architecture in Practice").

Recipe (per configuration, all seeded):
  x, z, B, C  ~ N(0, 1)
  delta_raw   ~ N(0, 0.1^2)
  dt          ~ loguniform[lo, hi] per channel, dt_bias = softplus^-1(dt) in fp64
  A[d, n]     = -(n + 1) exactly, D = 1
  decode state ~ N(0, 1) in fp32
bf16 configurations draw in fp32 and round once to bf16 (round to nearest even).

Layouts: x, delta, z, y are [batch][dim][seqlen] (channel-major, contiguous in
time); B and C are [batch][seqlen][dstate] and shared by every channel; A is
[dim][dstate]; D and dt_bias are [dim]; states are [batch][dim][dstate].
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

# Tensor-stream identifiers: each tensor gets its own generator stream.
STREAM_X, STREAM_DELTA, STREAM_Z, STREAM_B, STREAM_C, STREAM_DT, STREAM_STATE = range(7)


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int = 16
    io: str = "bf16"  # "f32" or "bf16"
    seed: int = 0
    dt_lo: float = 1e-3
    dt_hi: float = 1e-1
    use_z: bool = True
    use_D: bool = True
    final_state: bool = True

    @property
    def io_dtype(self) -> torch.dtype:
        return torch.float32 if self.io == "f32" else torch.bfloat16

    @property
    def tokch(self) -> int:
        return self.batch * self.seqlen * self.dim

    def algorithmic_bytes(self) -> int:
        """Bytes one forward call must move at minimum: every input read once,
        every output written once (no (b, L, d, N) expansion)."""
        e = 4 if self.io == "f32" else 2
        tc = self.tokch
        n_io = 2 + (1 if self.use_z else 0) + 1          # x, delta, [z], y
        total = n_io * tc * e
        total += 2 * self.batch * self.seqlen * self.dstate * e  # B, C
        total += self.dim * self.dstate * 4                    # A
        total += self.dim * 4                                   # dt_bias
        total += (self.dim * 4) if self.use_D else 0            # D
        if self.final_state:
            total += self.batch * self.dim * self.dstate * 4
        return total


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int = 16
    steps: int = 64
    io: str = "bf16"
    seed: int = 0
    dt_lo: float = 1e-3
    dt_hi: float = 1e-1

    @property
    def io_dtype(self) -> torch.dtype:
        return torch.float32 if self.io == "f32" else torch.bfloat16

    def algorithmic_bytes_per_step(self) -> int:
        e = 4 if self.io == "f32" else 2
        bd = self.batch * self.dim
        total = 2 * bd * self.dstate * 4          # state read + write
        total += 4 * bd * e                       # x, delta, z, y
        total += 2 * self.batch * self.dstate * e # B, C
        total += self.dim * self.dstate * 4 + 2 * self.dim * 4  # A, D, dt_bias
        return total


CONFIGS = {
    "tiny": ScanConfig("tiny", 1, 256, 16, io="f32", seed=1),
    "m130": ScanConfig("m130", 8, 2048, 1536, io="bf16", seed=2, final_state=False),
    "m2p8": ScanConfig("m2p8", 4, 2048, 5120, io="bf16", seed=3),
    "long": ScanConfig("long", 1, 1 << 20, 1536, io="bf16", seed=4, dt_lo=1e-4, dt_hi=1e-2),
}
DECODE = DecodeConfig("decode", 256, 5120, io="bf16", seed=5)


def _gen(device, seed: int, stream: int, step: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream * 7_919 + step * 104_729) & ((1 << 62) - 1))
    return g


def _normal(shape, std, dtype, device, seed, stream, step=0, chunk_elems=1 << 28):
    """N(0, std^2) drawn in fp32 and rounded once to `dtype`; big tensors are
    drawn in slices so the fp32 temporary stays bounded."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    g = _gen(device, seed, stream, step)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        tmp = torch.randn(e - s, generator=g, dtype=torch.float32, device=device)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:e].copy_(tmp)
    return out


def channel_params(dim: int, dstate: int, dt_lo: float, dt_hi: float, seed: int):
    """A, D, dt_bias for `dim` channels, drawn on the CPU (small) in fp64 and
    stored as fp32."""
    g = _gen("cpu", seed, STREAM_DT)
    u = torch.rand(dim, generator=g, dtype=torch.float64)
    dt = torch.exp(math.log(dt_lo) + u * (math.log(dt_hi) - math.log(dt_lo)))
    dt_bias = (dt + torch.log(-torch.expm1(-dt))).to(torch.float32)
    A = -torch.arange(1, dstate + 1, dtype=torch.float32).repeat(dim, 1).contiguous()
    D = torch.ones(dim, dtype=torch.float32)
    return A, D, dt_bias


def scan_inputs(cfg: ScanConfig, device="cpu", seed: int | None = None) -> dict:
    """All inputs of one forward scan call, on `device`."""
    seed = cfg.seed if seed is None else seed
    b, L, d, N = cfg.batch, cfg.seqlen, cfg.dim, cfg.dstate
    dt = cfg.io_dtype
    A, D, dt_bias = channel_params(d, N, cfg.dt_lo, cfg.dt_hi, seed)
    out = {
        "x": _normal((b, d, L), 1.0, dt, device, seed, STREAM_X),
        "delta": _normal((b, d, L), 0.1, dt, device, seed, STREAM_DELTA),
        "z": _normal((b, d, L), 1.0, dt, device, seed, STREAM_Z) if cfg.use_z else None,
        "B": _normal((b, L, N), 1.0, dt, device, seed, STREAM_B),
        "C": _normal((b, L, N), 1.0, dt, device, seed, STREAM_C),
        "A": A.to(device),
        "D": D.to(device) if cfg.use_D else None,
        "delta_bias": dt_bias.to(device),
    }
    return out


def decode_state(cfg: DecodeConfig, device="cpu", seed: int | None = None, layer: int = 0):
    seed = cfg.seed if seed is None else seed
    return _normal((cfg.batch, cfg.dim, cfg.dstate), 1.0, torch.float32, device,
                   seed + 7 * layer, STREAM_STATE)


def decode_params(cfg: DecodeConfig, seed: int | None = None):
    seed = cfg.seed if seed is None else seed
    return channel_params(cfg.dim, cfg.dstate, cfg.dt_lo, cfg.dt_hi, seed)


def decode_token(cfg: DecodeConfig, step: int, device="cpu", seed: int | None = None) -> dict:
    """Per-token inputs of decode step `step` (fresh draws per step)."""
    seed = cfg.seed if seed is None else seed
    b, d, N = cfg.batch, cfg.dim, cfg.dstate
    dt = cfg.io_dtype
    return {
        "x": _normal((b, d), 1.0, dt, device, seed, STREAM_X, step + 1),
        "delta": _normal((b, d), 0.1, dt, device, seed, STREAM_DELTA, step + 1),
        "z": _normal((b, d), 1.0, dt, device, seed, STREAM_Z, step + 1),
        "B": _normal((b, N), 1.0, dt, device, seed, STREAM_B, step + 1),
        "C": _normal((b, N), 1.0, dt, device, seed, STREAM_C, step + 1),
    }


def length_mix(total: int, lo: int, hi: int, seed: int, empties: int = 0) -> list:
    """Sequence lengths for packed input: log-uniform integers in [lo, hi] until
    `total` tokens are used (the last one cut to fit), then `empties` zero-length
    sequences inserted at seeded positions."""
    g = _gen("cpu", seed, STREAM_STATE, 99)
    lens = []
    used = 0
    while used < total:
        u = float(torch.rand(1, generator=g, dtype=torch.float64))
        n = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
        n = max(1, min(n, total - used))
        lens.append(n)
        used += n
    for _ in range(empties):
        pos = int(torch.randint(0, len(lens) + 1, (1,), generator=g))
        lens.insert(pos, 0)
    return lens


def cu_seqlens(lens, device="cpu") -> torch.Tensor:
    """int32 offsets [0, l0, l0+l1, ...] of packed sequences."""
    out = [0]
    for n in lens:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32, device=device)


def packed_inputs(cfg: ScanConfig, total: int, device="cpu", seed: int | None = None) -> dict:
    """Inputs of one packed call with `total` tokens: x, delta, z [dim][total];
    B, C [total][dstate]; the same distributions as scan_inputs (drawn as one row)."""
    one = scan_inputs(shrink(cfg, batch=1, seqlen=total), device, seed)
    return {k: (v[0] if k in ("x", "delta", "z", "B", "C") and v is not None else v)
            for k, v in one.items()}


def conv_params(dim: int, width: int, seed: int):
    """Weights [dim][width] ~ N(0, 0.5^2) and bias [dim] ~ N(0, 0.2^2) in fp32 for the
    causal convolution in front of the scan, drawn on the CPU."""
    g = _gen("cpu", seed, STREAM_DT, 7)
    w = (torch.randn((dim, width), generator=g, dtype=torch.float32) * 0.5).contiguous()
    b = torch.randn(dim, generator=g, dtype=torch.float32) * 0.2
    return w, b


def conv_state(batch: int, dim: int, width: int, dtype, device="cpu", seed: int = 0):
    """A conv state [batch][dim][width-1] ~ N(0, 1) in `dtype` (the inputs before t = 0)."""
    return _normal((batch, dim, width - 1), 1.0, dtype, device, seed, STREAM_STATE, 11)


def shrink(cfg: ScanConfig, **kw) -> ScanConfig:
    """A copy of `cfg` with some sizes replaced (same distributions)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return ScanConfig(**d)

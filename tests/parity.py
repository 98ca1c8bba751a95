"""Helpers for GPU-vs-oracle parity: run the HIP path through the C ABI binding,
run the fp64 oracle on the same bits (all rows, or sampled rows at full size),
and compare with the per-row normwise metric.

Metric: for a tensor T with rows r (a (batch, channel) pair over tokens for y,
over states for h), err = max_r ||T_r - Tref_r||_inf / ||Tref_r||_inf; a row whose
reference is all zero must be exactly zero. Tolerances: 1e-5 for fp32 inputs and
outputs, 2e-2 for bf16 (the bf16 output rounding alone is <= 2^-9 relative).
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-5, "bf16": 2e-2}


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rowwise_err(got, ref) -> float:
    got = oracle.f64(got)
    ref = oracle.f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    L = ref.shape[-1]
    g = got.reshape(-1, L)
    r = ref.reshape(-1, L)
    scale = np.max(np.abs(r), axis=1)
    diff = np.max(np.abs(g - r), axis=1)
    zero = scale == 0
    if np.any(zero):
        assert np.all(diff[zero] == 0), "a row with an all-zero reference is not exactly zero"
    if np.all(zero):
        return 0.0
    return float(np.max(diff[~zero] / scale[~zero]))


def per_token_err(got, ref, floor_frac=0.1) -> float:
    """Per-token error of a [batch][L][N] gradient that is a sum over channels (dB, dC):
    for each (b, t) the max-norm error over the N states divided by the max-norm of the
    reference at that token -- or, where that sum cancelled, by a floor of floor_frac
    times the median per-token max-norm of its batch row."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape and g.ndim == 3, (g.shape, r.shape)
    scale = np.max(np.abs(r), axis=2)                               # [b][L]
    floor = floor_frac * np.median(scale, axis=1, keepdims=True)    # [b][1]
    den = np.maximum(scale, floor)
    if np.all(den == 0):
        return float(np.max(np.abs(g - r)))
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.max(np.abs(g - r), axis=2) / den))


def boundary_rows(batch, dim, cg, nspread, seed=0):
    """(b, d) rows on both sides of every boundary between groups of cg channels (the
    last channel of a group and the first of the next, plus channel 0 and the last
    channel), in every batch row, plus nspread random rows."""
    ch = {0, dim - 1}
    for k in range(1, (dim + cg - 1) // cg):
        ch.update((k * cg - 1, k * cg))
    picks = {(b, d) for b in range(batch) for d in ch if d < dim}
    rng = np.random.default_rng(seed)
    target = len(picks) + nspread
    while len(picks) < min(target, batch * dim):
        picks.add((int(rng.integers(batch)), int(rng.integers(dim))))
    rows = sorted(picks)
    return np.array([r[0] for r in rows]), np.array([r[1] for r in rows])


def gpu_scan(inp: dict, use_z=True, use_D=True, h0=None, final=True, plan=0, chunk_len=0,
             softplus=True, bias=True, group_channels=0, reverse=False, structured_a=False):
    from selective_state_space_53_amd import binding
    return binding.ssm_scan_fwd(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"] if bias else None, delta_softplus=softplus, h0=h0,
        return_final_state=final, plan=plan, chunk_len=chunk_len,
        group_channels=group_channels, reverse=reverse, structured_a=structured_a)


def oracle_full(inp: dict, use_z=True, use_D=True, h0=None, softplus=True, bias=True):
    return oracle.Oracle().scan(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"] if bias else None, delta_softplus=softplus, h0=h0,
        nthreads=threads())


def sample_rows(batch, dim, n, seed=0):
    """Deterministic (b, d) sample of about n rows: the first and last row, channels 63 and
    64 (the 64-channel boundary), and random rows. (Tests that must cover the channel
    groups of a plan use boundary_rows.)"""
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (batch - 1, dim - 1), (0, min(63, dim - 1)), (batch - 1, min(64, dim - 1))}
    while len(picks) < min(n, batch * dim):
        picks.add((int(rng.integers(batch)), int(rng.integers(dim))))
    rows = sorted(picks)
    return np.array([r[0] for r in rows]), np.array([r[1] for r in rows])


def oracle_rows(inp: dict, rb, rd, use_z=True, use_D=True, h0=None, softplus=True, bias=True):
    """Oracle on sampled rows only: copies just those rows (and B, C) to the host."""
    rb_t = torch.as_tensor(rb, device=inp["x"].device)
    rd_t = torch.as_tensor(rd, device=inp["x"].device)
    x = inp["x"][rb_t, rd_t]
    dl = inp["delta"][rb_t, rd_t]
    z = inp["z"][rb_t, rd_t] if use_z else None
    h0r = h0[rb_t, rd_t] if h0 is not None else None
    return oracle.Oracle().scan_rows(
        x, dl, inp["A"], inp["B"], inp["C"], rb, rd, z_rows=z, D=inp["D"] if use_D else None,
        delta_bias=inp["delta_bias"] if bias else None, delta_softplus=softplus, h0_rows=h0r,
        nthreads=threads())


def oracle_reverse_rows(inp: dict, rb, rd, use_z=True, use_D=True, h0=None):
    """Reverse-scan oracle on sampled rows: the causal oracle of the time-reversed
    rows (the reverse scan's definition), flipped back."""
    rb_t = torch.as_tensor(rb, device=inp["x"].device)
    rd_t = torch.as_tensor(rd, device=inp["x"].device)
    fl = lambda t: None if t is None else np.ascontiguousarray(oracle.f64(t)[..., ::-1])
    x = fl(inp["x"][rb_t, rd_t])
    dl = fl(inp["delta"][rb_t, rd_t])
    z = fl(inp["z"][rb_t, rd_t]) if use_z else None
    B = np.ascontiguousarray(oracle.f64(inp["B"])[:, ::-1])
    C = np.ascontiguousarray(oracle.f64(inp["C"])[:, ::-1])
    h0r = h0[rb_t, rd_t] if h0 is not None else None
    y, hf = oracle.Oracle().scan_rows(
        x, dl, inp["A"], B, C, rb, rd, z_rows=z, D=inp["D"] if use_D else None,
        delta_bias=inp["delta_bias"], delta_softplus=True, h0_rows=h0r, nthreads=threads())
    return np.ascontiguousarray(y[:, ::-1]), hf


def gpu_varlen(inp: dict, cu, use_z=True, use_D=True, h0=None, final=True, plan=0, chunk_len=0,
               reverse=False, group_channels=0):
    from selective_state_space_53_amd import binding
    return binding.ssm_scan_varlen_fwd(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], cu,
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"], h0=h0, return_final_state=final, plan=plan,
        chunk_len=chunk_len, reverse=reverse, group_channels=group_channels)


def oracle_varlen(inp: dict, cu, use_z=True, use_D=True, h0=None, reverse=False, channels=None):
    """Packed-sequence oracle, on every channel or on the listed ones."""
    sel = slice(None) if channels is None else torch.as_tensor(channels, device=inp["x"].device)
    pick = lambda t: None if t is None else t[sel]
    return oracle.Oracle().scan_varlen(
        pick(inp["x"]), pick(inp["delta"]), pick(inp["A"]), inp["B"], inp["C"],
        oracle.f64(cu).astype(np.int64), D=pick(inp["D"]) if use_D else None,
        z=pick(inp["z"]) if use_z else None, delta_bias=pick(inp["delta_bias"]),
        h0=None if h0 is None else h0[:, sel], reverse=reverse, nthreads=threads())

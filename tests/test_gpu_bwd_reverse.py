"""GPU parity of the backward of the anti-causal scan (ssm_scan_bwd with reverse, through
the C ABI) against the fp64 oracle's reverse gradients: every output on ragged shapes in
each checkpoint and backward plan, an integer-exact case bit for bit, the Mamba-2.8B
layer in full, and the training pair (the reverse forward saving its checkpoints, the
backward from them) bit for bit against the recomputing backward."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OUTS = ["dx", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"]
OKEY = {"ddelta_bias": "dbias"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_53_amd import binding  # noqa: F401  (fails loudly if unbuilt)


def _randn(shape, seed, dtype=torch.float32):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).to(DEV)


def _compare(g, ref, io):
    """As for the causal backward: per-token gradients per (batch, channel) row; dB, dC
    normwise per batch row; dA, dD, d_bias over the tensor; dh0 per row."""
    errs = {}
    for k in OUTS:
        if g.get(k) is None:
            continue
        r = np.asarray(ref[OKEY.get(k, k)])
        got = oracle.f64(g[k])
        if k in ("dB", "dC"):
            got, r = got.reshape(got.shape[0], -1), r.reshape(r.shape[0], -1)
        elif k in ("dA", "dD", "ddelta_bias"):
            got, r = got.reshape(1, -1), r.reshape(1, -1)
        errs[k] = parity.rowwise_err(got, r)
    say("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= parity.TOL[io]}
    assert not bad, bad


def _run(inp, dy, use_z=True, use_D=True, use_bias=True, h0=None, dhf=None, **plan):
    from selective_state_space_53_amd import binding
    g = binding.ssm_scan_bwd(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"] if use_bias else None, h0=h0, dh_final=dhf,
        want_dh0=True, reverse=True, **plan)
    torch.cuda.synchronize()
    ref = oracle.Oracle().scan_reverse_bwd(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"] if use_bias else None, h0=h0, dh_final=dhf,
        nthreads=parity.threads())
    return g, ref


SHAPES = [(1, 256, 16, "f32"), (2, 1000, 200, "bf16"), (1, 333, 70, "bf16"), (3, 1, 5, "f32"),
          (1, 17, 65, "f32"), (2, 65, 130, "bf16"), (1, 4103, 96, "bf16")]
PLANS = [dict(plan=1), dict(plan=2, chunk_len=64), dict(bwd_chunk_len=32, bwd_group_channels=32),
         dict(plan=2, chunk_len=96, bwd_chunk_len=64, bwd_group_channels=48)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}_L{}_d{}_{}".format(*s))
@pytest.mark.parametrize("plan", PLANS, ids=["single", "c64", "bwd_c32_g32", "c96_bwd_c64_g48"])
def test_reverse_bwd_all_outputs(shape, plan):
    batch, L, dim, io = shape
    cfg = synth.ScanConfig("revbwd", batch, L, dim, io=io, seed=1300 + L)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _randn((batch, dim, L), 1400 + L, cfg.io_dtype)
    h0 = _randn((batch, dim, 16), 11)
    dhf = _randn((batch, dim, 16), 12)
    for var in [dict(use_z=True, use_D=True, use_bias=True, h0=h0, dhf=dhf),
                dict(use_z=False, use_D=False, use_bias=False, h0=None, dhf=None)]:
        say("case reverse bwd", shape, plan, {k: (v is not None) if not isinstance(v, bool)
                                              else v for k, v in var.items()})
        g, ref = _run(inp, dy, **var, **plan)
        _compare(g, ref, io)


def test_reverse_bwd_integer_exact():
    """A = 0, Delta = 1 (softplus off), no gate, small integers: every intermediate is an
    exact integer, so the reverse gradients equal the oracle's bit for bit -- across the
    16-token tiles walked from the first, the checkpoint pass's tiles and chunks, the
    backward chunks and the reductions."""
    from selective_state_space_53_amd import binding
    rng = np.random.default_rng(18)
    batch, L, dim = 2, 97, 70
    x = np.zeros((batch, dim, L))
    for b in range(batch):
        for d in range(dim):
            idx = rng.choice(L, size=6, replace=False)
            x[b, d, idx] = rng.choice([-1.0, 1.0], size=6)
    t = lambda a: torch.tensor(a, dtype=torch.float32, device=DEV)
    inp = {"x": t(x), "delta": torch.ones((batch, dim, L), device=DEV),
           "B": t(rng.integers(-1, 2, size=(batch, L, 16))),
           "C": t(rng.integers(-1, 2, size=(batch, L, 16))),
           "A": torch.zeros((dim, 16), device=DEV), "D": t(rng.integers(-2, 3, size=dim))}
    dy = t(rng.integers(-1, 2, size=(batch, dim, L)))
    h0 = t(rng.integers(-2, 3, size=(batch, dim, 16)))
    dhf = t(rng.integers(-2, 3, size=(batch, dim, 16)))
    ref = oracle.Oracle().scan_reverse_bwd(inp["x"], inp["delta"], inp["A"], inp["B"],
                                           inp["C"], dy, D=inp["D"], delta_softplus=False,
                                           h0=h0, dh_final=dhf)
    for plan in PLANS + [dict(plan=2, chunk_len=32, bwd_chunk_len=32, bwd_group_channels=64)]:
        say("case reverse bwd integer", plan)
        g = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                                 D=inp["D"], delta_softplus=False, h0=h0, dh_final=dhf,
                                 want_dh0=True, reverse=True, **plan)
        torch.cuda.synchronize()
        for k in ["dx", "ddelta", "dA", "dB", "dC", "dD", "dh0"]:
            assert np.array_equal(oracle.f64(g[k]), ref[k]), k


def test_reverse_bwd_full_size():
    """The Mamba-2.8B layer shape (batch 4, 2048 tokens, d_inner 5120, bf16), every
    gradient of the anti-causal scan against the full fp64 oracle."""
    cfg = synth.CONFIGS["m2p8"]
    inp = synth.scan_inputs(cfg, DEV)
    dy = _randn((cfg.batch, cfg.dim, cfg.seqlen), 19, cfg.io_dtype)
    say("case reverse bwd full size")
    g, ref = _run(inp, dy)
    _compare(g, ref, cfg.io)


@pytest.mark.parametrize("shape", [(2, 1000, 200, "bf16"), (1, 333, 70, "f32"),
                                   (3, 17, 33, "f32")],
                         ids=lambda s: "b{}_L{}_d{}_{}".format(*s))
@pytest.mark.parametrize("plan", [dict(), dict(plan=2, chunk_len=64),
                                  dict(bwd_chunk_len=96)], ids=["auto", "c64", "bwd_c96"])
def test_reverse_training_pair(shape, plan):
    """The anti-causal forward with save_for_backward writes the same y and h_final as the
    plain anti-causal forward, and the backward from what it saved equals, bit for bit,
    the backward that recomputes the checkpoints."""
    from selective_state_space_53_amd import binding
    batch, L, dim, io = shape
    cfg = synth.ScanConfig("revtrain", batch, L, dim, io=io, seed=1500 + L)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _randn((batch, dim, L), L + 17, cfg.io_dtype)
    h0 = _randn((batch, dim, 16), 15)
    dhf = _randn((batch, dim, 16), 16)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    kw = dict(D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], h0=h0)
    fplan = {k: v for k, v in plan.items() if k in ("plan", "chunk_len")}
    say("case reverse training pair", shape, plan)
    ws = torch.empty(binding.ssm_scan_bwd_workspace_bytes(batch, L, dim, 16, cfg.io_dtype,
                                                          **plan),
                     dtype=torch.uint8, device=DEV)
    ys, hs = binding.ssm_scan_fwd(*args, **kw, return_final_state=True, reverse=True,
                                  save_for_backward=ws, **fplan)
    yp, hp = binding.ssm_scan_fwd(*args, **kw, return_final_state=True, reverse=True, **fplan)
    gs = binding.ssm_scan_bwd(*args, dy, **kw, dh_final=dhf, want_dh0=True, reverse=True,
                              workspace=ws, saved=True, **plan)
    gr = binding.ssm_scan_bwd(*args, dy, **kw, dh_final=dhf, want_dh0=True, reverse=True,
                              **plan)
    torch.cuda.synchronize()
    assert torch.equal(ys, yp) and torch.equal(hs, hp)
    for k in OUTS:
        assert torch.equal(gs[k], gr[k]), k
    ref = oracle.Oracle().scan_reverse_bwd(*args, dy, **kw, dh_final=dhf,
                                           nthreads=parity.threads())
    _compare(gs, ref, io)

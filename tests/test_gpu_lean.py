"""The lean and the general form of the scan kernels give the same bits.

A bf16 launch of batch rows (either direction) on whole aligned tiles with every channel
group in range and softplus on runs the kernels' lean form (straight-line tile loops,
buffer accesses); any other launch runs the general form. The two do the same arithmetic in the
same order, so a shape run once with a channel grouping that qualifies and once with one
that does not (the last group ragged) must agree bit for bit wherever the grouping does not
change a summation order: y and h_final of the forward; dx, ddelta, dz, dA, dD,
ddelta_bias and dh0 of the backward (dB and dC are sums over channels, grouped
differently, and are checked against the oracle instead). Both are also checked against
the fp64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_53_amd import binding  # noqa: F401  (fails loudly if unbuilt)


def _same(a, b, what):
    a, b = a.cpu(), b.cpu()
    diff = (a.float() - b.float()).abs().max().item() if a.numel() else 0.0
    assert torch.equal(a, b), f"{what}: lean and general forms differ (max {diff:.3e})"


@pytest.mark.parametrize("reverse", [False, True], ids=["causal", "anticausal"])
@pytest.mark.parametrize("use_z", [True, False], ids=["gated", "scan_only"])
@pytest.mark.parametrize("plan,chunk", [(1, 0), (2, 64)], ids=["single", "c64"])
def test_forward_lean_equals_general(use_z, plan, chunk, reverse):
    # 96 channels: groups of 16 (every group whole: lean) or 64 (a ragged last group:
    # general); 256 tokens = 8 whole tiles
    cfg = synth.ScanConfig("lean", 2, 256, 96, io="bf16", seed=901)
    say("case lean forward", use_z, plan, chunk, reverse)
    inp = synth.scan_inputs(cfg, DEV)
    gen = torch.Generator(device="cpu").manual_seed(902)
    h0 = torch.randn((2, 96, 16), generator=gen).to(DEV)
    yl, hl = parity.gpu_scan(inp, use_z=use_z, h0=h0, plan=plan, chunk_len=chunk,
                             group_channels=16, reverse=reverse)
    yg, hg = parity.gpu_scan(inp, use_z=use_z, h0=h0, plan=plan, chunk_len=chunk,
                             group_channels=64, reverse=reverse)
    torch.cuda.synchronize()
    _same(yl, yg, "y")
    _same(hl, hg, "h_final")
    if reverse:
        # the oracle of the anti-causal scan: the causal one on time-reversed inputs
        flip = {k: (v.flip(-1) if k in ("x", "delta", "z") else v.flip(1) if k in ("B", "C") else v)
                for k, v in inp.items()}
        yr, hr = parity.oracle_full(flip, use_z=use_z, h0=h0)
        yr = np.ascontiguousarray(np.asarray(yr)[..., ::-1])
    else:
        yr, hr = parity.oracle_full(inp, use_z=use_z, h0=h0)
    ey, eh = parity.rowwise_err(yl, yr), parity.rowwise_err(hl, hr)
    say(f"  y err {ey:.3e}  h_final err {eh:.3e}")
    assert ey <= parity.TOL["bf16"] and eh <= parity.TOL["bf16"]


def test_bidirectional_accumulate_lean_equals_general():
    """The causal scan, then the anti-causal one accumulated into the same y."""
    from selective_state_space_53_amd import binding
    cfg = synth.ScanConfig("leanacc", 2, 256, 96, io="bf16", seed=921)
    say("case lean accumulate")
    inp = synth.scan_inputs(cfg, DEV)
    outs = []
    for cg in (16, 64):
        y = parity.gpu_scan(inp, final=False, group_channels=cg)
        y = y[0] if isinstance(y, tuple) else y
        binding.ssm_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                             z=inp["z"], delta_bias=inp["delta_bias"], y=y, reverse=True,
                             accumulate=True, group_channels=cg)
        torch.cuda.synchronize()
        outs.append(y.clone())
    _same(outs[0], outs[1], "y (both directions)")


@pytest.mark.parametrize("reverse", [False, True], ids=["causal", "anticausal"])
@pytest.mark.parametrize("L,bwd_chunk", [(256, 0), (272, 0), (512, 128), (512, 96), (512, 192)],
                         ids=["L256", "L272", "L512_c128", "L512_c96", "L512_c192"])
def test_backward_lean_equals_general(reverse, L, bwd_chunk):
    # 64 channels: backward groups of 32 (lean) or 48 (a ragged last group: general); the
    # forward checkpoint pass likewise in groups of 16 (lean) or 48 (general). The lean
    # kernel loads the input rows of four 16-token tiles together when its chunk starts on
    # a 64-token line and holds a multiple of four tiles (L256; L512 with chunks of 128 or
    # 192 tokens, the last one 128), and tile by tile otherwise (L272: 17 tiles; chunks of
    # 96 tokens: 6 tiles, every other one starting mid-line).
    from selective_state_space_53_amd import binding
    batch, dim = 2, 64
    cfg = synth.ScanConfig("leanb", batch, L, dim, io="bf16", seed=911)
    say("case lean backward", reverse, L, bwd_chunk)
    inp = synth.scan_inputs(cfg, DEV)
    dy = synth.scan_inputs(cfg, DEV, seed=912)["z"]
    gen = torch.Generator(device="cpu").manual_seed(913)
    h0 = torch.randn((batch, dim, 16), generator=gen).to(DEV)
    dhf = torch.randn((batch, dim, 16), generator=gen).to(DEV)

    def run(fwd_cg, bwd_cg):
        g = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                                 D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], h0=h0,
                                 dh_final=dhf, want_dh0=True, plan=1, group_channels=fwd_cg,
                                 bwd_group_channels=bwd_cg, bwd_chunk_len=bwd_chunk,
                                 reverse=reverse)
        torch.cuda.synchronize()
        return g

    gl, gg = run(16, 32), run(48, 48)
    for k in ("dx", "ddelta", "dz", "dA", "dD", "ddelta_bias", "dh0"):
        _same(gl[k], gg[k], k)
    if reverse:   # time-reversed inputs through the causal oracle, gradients reversed back
        fl = lambda t: t.flip(-1)
        ref = oracle.Oracle().scan_bwd(fl(inp["x"]), fl(inp["delta"]), inp["A"], inp["B"].flip(1),
                                       inp["C"].flip(1), fl(dy), D=inp["D"], z=fl(inp["z"]),
                                       delta_bias=inp["delta_bias"], h0=h0, dh_final=dhf,
                                       nthreads=parity.threads())
        ref = {k: (np.asarray(v)[:, ::-1] if k in ("dB", "dC") else v) for k, v in ref.items()}
    else:
        ref = oracle.Oracle().scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                                       D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                       h0=h0, dh_final=dhf, nthreads=parity.threads())
    for g in (gl, gg):
        for k in ("dB", "dC"):
            got = oracle.f64(g[k]).reshape(batch, -1)
            r = np.ascontiguousarray(np.asarray(ref[k])).reshape(batch, -1)
            e = parity.rowwise_err(got, r)
            say(f"  {k} err {e:.3e}")
            assert e <= parity.TOL["bf16"]


@pytest.mark.parametrize("reverse", [False, True], ids=["causal", "anticausal"])
@pytest.mark.parametrize("plan,chunk", [(1, 0), (2, 64)], ids=["single", "c64"])
def test_packed_lean_equals_general(plan, chunk, reverse):
    """Packed sequences (sequences starting and ending inside tiles, empty ones among
    them): forward and backward, lean against general form."""
    from selective_state_space_53_amd import binding
    total, dim = 512, 96
    cfg = synth.ScanConfig("leanp", 1, total, dim, io="bf16", seed=931)
    say("case lean packed", plan, chunk, reverse)
    lens = synth.length_mix(total, 5, 200, seed=932, empties=2)
    cu = synth.cu_seqlens(lens, DEV)
    inp = synth.packed_inputs(cfg, total, DEV, seed=933)
    dy = synth.packed_inputs(cfg, total, DEV, seed=934)["z"]
    gen = torch.Generator(device="cpu").manual_seed(935)
    h0 = torch.randn((len(lens), dim, 16), generator=gen).to(DEV)
    dhf = torch.randn((len(lens), dim, 16), generator=gen).to(DEV)
    fw, bw = [], []
    for fcg, bcg in ((16, 32), (64, 64)):   # 96 channels: 16 and 32 whole, 64 ragged
        y, hf = binding.ssm_scan_varlen_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], cu,
                                            D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                            h0=h0, return_final_state=True, plan=plan,
                                            chunk_len=chunk, group_channels=fcg, reverse=reverse)
        g = binding.ssm_scan_varlen_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy, cu,
                                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                        h0=h0, dh_final=dhf, want_dh0=True, plan=plan,
                                        chunk_len=chunk, group_channels=fcg,
                                        bwd_group_channels=bcg, reverse=reverse)
        torch.cuda.synchronize()
        fw.append((y, hf))
        bw.append(g)
    _same(fw[0][0], fw[1][0], "y")
    _same(fw[0][1], fw[1][1], "h_final")
    for k in ("dx", "ddelta", "dz", "dA", "dD", "ddelta_bias", "dh0"):
        _same(bw[0][k], bw[1][k], k)
    for k in ("dB", "dC"):
        a, b = bw[0][k].double(), bw[1][k].double()
        rel = ((a - b).abs().max() / b.abs().max().clamp_min(1e-30)).item()
        say(f"  {k} lean vs general (channel grouping differs) {rel:.2e}")
        assert rel <= 1e-5

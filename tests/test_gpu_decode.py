"""GPU parity of ssm_state_update (one recurrent token per call, through the C ABI)
against the fp64 oracle, at the full decode shape (batch 256, 5120 channels, 64
steps, checked on sampled rows) and on small ragged shapes (every row); plus
decode == scan on the GPU."""
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
    from selective_state_space_53_amd import binding  # noqa: F401


def _run_steps(cfg, nrows_sample, use_z=True, use_D=True, bias=True, softplus=True):
    from selective_state_space_53_amd import binding
    A, D, dt_bias = (t.to(DEV) for t in synth.decode_params(cfg))
    state = synth.decode_state(cfg, DEV)
    b, d = cfg.batch, cfg.dim
    if nrows_sample is None:
        rb = np.repeat(np.arange(b), d)
        rd = np.tile(np.arange(d), b)
    else:
        rb, rd = parity.sample_rows(b, d, nrows_sample, seed=cfg.seed)
    sel = (torch.as_tensor(rb, device=DEV), torch.as_tensor(rd, device=DEV))
    st_ref = oracle.f64(state[sel])                 # [R][16] fp64
    orc = oracle.Oracle()
    ys, yrs, errs_state = [], [], {}
    Af, Bias, Dd = oracle.f64(A), oracle.f64(dt_bias), oracle.f64(D)
    for s in range(cfg.steps):
        tok = synth.decode_token(cfg, s, DEV)
        y = binding.ssm_state_update(state, tok["x"], tok["delta"], A, tok["B"], tok["C"],
                                     D=D if use_D else None, z=tok["z"] if use_z else None,
                                     delta_bias=dt_bias if bias else None,
                                     delta_softplus=softplus)
        # the oracle step on the sampled rows, reading the same bits
        xs, dls = oracle.f64(tok["x"][sel]), oracle.f64(tok["delta"][sel])
        zs = oracle.f64(tok["z"][sel]) if use_z else None
        Bs, Cs = oracle.f64(tok["B"]), oracle.f64(tok["C"])
        yr = np.empty(len(rb))
        lib = orc._l
        rbi = np.ascontiguousarray(rb, dtype=np.int64)
        rdi = np.ascontiguousarray(rd, dtype=np.int64)
        rc = lib.ssm_oracle_step_rows(len(rb), 16, oracle._ptr_i(rbi), oracle._ptr_i(rdi),
                                      oracle._ptr(st_ref), oracle._ptr(xs), oracle._ptr(dls),
                                      oracle._ptr(zs), oracle._ptr(Af), oracle._ptr(Bs),
                                      oracle._ptr(Cs), oracle._ptr(Dd if use_D else None),
                                      oracle._ptr(Bias if bias else None), int(softplus),
                                      oracle._ptr(yr))
        assert rc == 0
        ys.append(y[sel].float().cpu().numpy())
        yrs.append(yr)
        if s + 1 in (1, 8, cfg.steps):
            torch.cuda.synchronize()
            errs_state[s + 1] = parity.rowwise_err(state[sel], st_ref)
    torch.cuda.synchronize()
    ey = parity.rowwise_err(np.stack(ys, axis=1), np.stack(yrs, axis=1))   # rows over steps
    return ey, errs_state


def test_decode_full_shape_64_steps_every_row():
    cfg = synth.DECODE
    say("case decode full, every row", cfg)
    ey, es = _run_steps(cfg, None)
    say(f"decode: y err (rows over 64 steps) {ey:.3e}; state err {es}")
    assert ey <= parity.TOL["bf16"]
    for k, v in es.items():
        assert v <= parity.TOL["bf16"], k


def test_decode_full_shape_fp32_io_sampled():
    """The decode batch (256 x 5120) with fp32 io for 16 steps, sampled rows, fp32 bar."""
    cfg = synth.DecodeConfig("decode_f32", batch=256, dim=5120, steps=16, io="f32", seed=23)
    say("case decode full fp32", cfg)
    ey, es = _run_steps(cfg, 2048)
    say(f"decode fp32: y err {ey:.3e}; state err {es}")
    assert ey <= 1e-5
    for k, v in es.items():
        assert v <= 1e-5, k


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("opts", [dict(), dict(use_z=False, use_D=False),
                                  dict(bias=False, softplus=False)],
                         ids=["gated", "scan_only", "raw_delta"])
def test_decode_small_all_rows(io, opts):
    cfg = synth.DecodeConfig("decode_small", batch=3, dim=70, steps=12, io=io, seed=21)
    ey, es = _run_steps(cfg, None, **opts)
    say(f"decode small {io} {opts}: y {ey:.3e} state {es}")
    tol = 1e-5 if io == "f32" else 2e-2
    assert ey <= tol and all(v <= tol for v in es.values())


def test_decode_equals_scan_on_gpu():
    """64 decode steps from S == one scan over the same 64 tokens with h0 = S."""
    from selective_state_space_53_amd import binding
    batch, dim, L = 4, 200, 64
    cfg = synth.ScanConfig("dec_vs_scan", batch, L, dim, io="f32", seed=31)
    inp = synth.scan_inputs(cfg, DEV)
    gen = torch.Generator(device="cpu").manual_seed(1)
    S = torch.randn((batch, dim, 16), generator=gen).to(DEV)
    y_scan, h_scan = binding.ssm_scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                          D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                          h0=S, return_final_state=True)
    st = S.clone()
    ys = []
    for t in range(L):
        ys.append(binding.ssm_state_update(
            st, inp["x"][:, :, t].contiguous(), inp["delta"][:, :, t].contiguous(), inp["A"],
            inp["B"][:, t].contiguous(), inp["C"][:, t].contiguous(), D=inp["D"],
            z=inp["z"][:, :, t].contiguous(), delta_bias=inp["delta_bias"]))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=2)
    assert parity.rowwise_err(y_dec, y_scan) <= 1e-5
    assert parity.rowwise_err(st, h_scan) <= 1e-5


def test_decode_steps_in_a_hip_graph():
    """The library allocates nothing and never synchronizes inside a call, so a run of
    decode steps (the conv update, then the scan's state update, per token) can be
    captured once into a HIP graph and replayed. Every replay, with eager work and a
    synchronization between replays, must give the states and outputs of the same steps
    run eagerly, bit for bit."""
    from selective_state_space_53_amd import binding
    batch, dim, T = 64, 1024, 6
    g = torch.Generator().manual_seed(41)
    A = -torch.rand((dim, 16), generator=g).add(0.1).to(DEV)
    D = torch.randn(dim, generator=g).to(DEV)
    bias = torch.randn(dim, generator=g).mul(0.3).to(DEV)
    w = torch.randn((dim, 4), generator=g).mul(0.5).to(DEV)
    cb = torch.randn(dim, generator=g).mul(0.2).to(DEV)
    bf = torch.bfloat16
    toks = [{k: torch.randn(shape, generator=g).to(bf).to(DEV)
             for k, shape in (("x", (batch, dim)), ("delta", (batch, dim)), ("z", (batch, dim)),
                              ("B", (batch, 16)), ("C", (batch, 16)))} for _ in range(T)]
    state0 = torch.randn((batch, dim, 16), generator=g).to(DEV)
    conv0 = torch.randn((batch, dim, 3), generator=g).to(bf).to(DEV)
    ys = [torch.empty((batch, dim), dtype=bf, device=DEV) for _ in range(T)]
    xc = [torch.empty((batch, dim), dtype=bf, device=DEV) for _ in range(T)]

    def steps(state, conv):
        for t, tok in enumerate(toks):
            binding.ssm_causal_conv1d_update(conv, tok["x"], w, cb, y=xc[t])
            binding.ssm_state_update(state, xc[t], tok["delta"], A, tok["B"], tok["C"], D=D,
                                     z=tok["z"], delta_bias=bias, y=ys[t])

    # eager reference
    st_e, cv_e = state0.clone(), conv0.clone()
    steps(st_e, cv_e)
    torch.cuda.synchronize()
    y_e = [y.clone() for y in ys]
    # capture (on a side stream, as torch requires), then replay three times
    st_g, cv_g = state0.clone(), conv0.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        steps(st_g.clone(), cv_g.clone())       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        steps(st_g, cv_g)
    for rep in range(3):
        st_g.copy_(state0)
        cv_g.copy_(conv0)
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  graph replay {rep}")
        assert torch.equal(st_g, st_e) and torch.equal(cv_g, cv_e), rep
        for t in range(T):
            assert torch.equal(ys[t], y_e[t]), (rep, t)
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()   # eager work between replays

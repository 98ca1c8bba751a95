"""GPU parity of the backward selective scan (ssm_scan_bwd, through the C ABI)
against the fp64 gradient oracle: every output on ragged shapes with each
backward group size and both plans of the checkpoint pass, the Mamba-2.8B layer
shape in full, and an integer-exact case that checks tile boundaries and the
reductions over channels and batch rows bit for bit."""
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
# oracle key for each GPU output
OKEY = {"ddelta_bias": "dbias"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from selective_state_space_53_amd import binding  # noqa: F401  (fails loudly if unbuilt)


def _dy(shape, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).to(DEV)


def _compare(g, ref, io, tol=None):
    tol = parity.TOL[io] if tol is None else tol
    errs = {}
    for k in OUTS:
        if g.get(k) is None:
            continue
        r = np.asarray(ref[OKEY.get(k, k)])
        got = oracle.f64(g[k])
        # per-token gradients: per (batch, channel) row, as y. Sums over channels (dB,
        # dC): normwise over each batch row (all tokens and states), since one token's
        # sum over channels can cancel far below the terms it adds. Sums over batch and
        # time (dA, dD, ddelta_bias): normwise over the tensor.
        if k in ("dB", "dC"):
            got, r = got.reshape(got.shape[0], -1), r.reshape(r.shape[0], -1)
        elif k in ("dA", "dD", "ddelta_bias"):
            got, r = got.reshape(1, -1), r.reshape(1, -1)
        errs[k] = parity.rowwise_err(got, r)
        if k in ("dB", "dC"):
            errs[k + "/token"] = parity.per_token_err(oracle.f64(g[k]), np.asarray(ref[OKEY.get(k, k)]))
    say("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def _run(inp, dy, io, use_z=True, use_D=True, use_bias=True, h0=None, dhf=None, plan=0,
         chunk=0, bwd_cg=0, bwd_chunk=0):
    from selective_state_space_53_amd import binding
    g = binding.ssm_scan_bwd(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"] if use_bias else None, h0=h0, dh_final=dhf,
        want_dh0=True, plan=plan, chunk_len=chunk, bwd_group_channels=bwd_cg,
        bwd_chunk_len=bwd_chunk)
    torch.cuda.synchronize()
    ref = oracle.Oracle().scan_bwd(
        inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
        D=inp["D"] if use_D else None, z=inp["z"] if use_z else None,
        delta_bias=inp["delta_bias"] if use_bias else None, h0=h0, dh_final=dhf,
        nthreads=parity.threads())
    return g, ref


SHAPES = [(1, 256, 16, "f32"), (2, 1000, 200, "bf16"), (1, 333, 70, "bf16"), (3, 1, 5, "f32"),
          (1, 17, 65, "f32"), (2, 65, 130, "bf16"), (1, 4103, 96, "bf16")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}_L{}_d{}_{}".format(*s))
@pytest.mark.parametrize("plan,chunk", [(1, 0), (2, 64)], ids=["single", "c64"])
def test_bwd_all_outputs(shape, plan, chunk):
    batch, L, dim, io = shape
    cfg = synth.ScanConfig("bwd", batch, L, dim, io=io, seed=300 + L)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((batch, dim, L), cfg.io_dtype, L)
    h0 = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(1)).to(DEV)
    dhf = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(2)).to(DEV)
    for var in [dict(use_z=True, use_D=True, use_bias=True, h0=h0, dhf=dhf),
                dict(use_z=False, use_D=False, use_bias=False, h0=None, dhf=None)]:
        say("case bwd", shape, plan, chunk, {k: v is not None if not isinstance(v, bool) else v
                                             for k, v in var.items()})
        g, ref = _run(inp, dy, io, plan=plan, chunk=chunk, **var)
        _compare(g, ref, io)


@pytest.mark.parametrize("cg", [32, 48, 64])
def test_bwd_every_group_size(cg):
    batch, L, dim = 2, 150, 150      # ragged last group and ragged last tile
    cfg = synth.ScanConfig("bwdcg", batch, L, dim, io="f32", seed=400 + cg)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((batch, dim, L), torch.float32, cg)
    dhf = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(cg)).to(DEV)
    say("case bwd group", cg)
    g, ref = _run(inp, dy, "f32", dhf=dhf, bwd_cg=cg)
    _compare(g, ref, "f32")


@pytest.mark.parametrize("shape", [(1, 1000, 200, "bf16"), (2, 333, 70, "f32"),
                                   (1, 4103, 96, "bf16"), (1, 65, 33, "f32")],
                         ids=lambda s: "b{}_L{}_d{}_{}".format(*s))
@pytest.mark.parametrize("bwd_chunk", [32, 64, 96])
def test_bwd_chunked_all_outputs(shape, bwd_chunk):
    """The chunked backward (gradient chains of the chunks from zero, a carry from the
    last chunk backwards, then every chunk from its carried-in gradient), with ragged
    last chunks and tiles, against the oracle."""
    batch, L, dim, io = shape
    cfg = synth.ScanConfig("bwdch", batch, L, dim, io=io, seed=350 + L)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((batch, dim, L), cfg.io_dtype, L + 1)
    h0 = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(3)).to(DEV)
    dhf = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(4)).to(DEV)
    say("case bwd chunked", shape, bwd_chunk)
    g, ref = _run(inp, dy, io, h0=h0, dhf=dhf, bwd_chunk=bwd_chunk)
    _compare(g, ref, io)


def test_bwd_long_sequence():
    """One row of 65,536 tokens x 256 channels (bf16) in the library's own plan: the
    backward is chunked (the sequence is what gives parallelism here); every output
    against the full fp64 oracle."""
    cfg = synth.ScanConfig("bwdlong", 1, 65536, 256, io="bf16", seed=44, dt_lo=1e-4,
                           dt_hi=1e-2)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((1, 256, 65536), torch.bfloat16, 45)
    say("case bwd long")
    g, ref = _run(inp, dy, "bf16")
    _compare(g, ref, "bf16")


def test_bwd_full_size():
    """The Mamba-2.8B layer shape (batch 4, 2048 tokens, d_inner 5120, bf16), every
    output against the full fp64 oracle."""
    cfg = synth.CONFIGS["m2p8"]
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((cfg.batch, cfg.dim, cfg.seqlen), cfg.io_dtype, 9)
    say("case bwd full size")
    g, ref = _run(inp, dy, cfg.io)
    _compare(g, ref, cfg.io)


def test_bwd_m130_full_size():
    """The Mamba-130M layer shape (batch 8, 2048 tokens, d_inner 1536, bf16) in the
    library's own plan, which chunks the backward here (as the benchmark runs it): every
    output against the full fp64 oracle."""
    cfg = synth.CONFIGS["m130"]
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((cfg.batch, cfg.dim, cfg.seqlen), cfg.io_dtype, 13)
    say("case bwd m130 full size")
    g, ref = _run(inp, dy, cfg.io)
    _compare(g, ref, cfg.io)


def test_bwd_long_full_size_sampled_channels():
    """The million-token row (1 x 1,048,576 x 1536, bf16) in the library's own plan. Every
    gradient of a channel -- dx, ddelta, dz and dh0 of its row, and dA, dD, d_bias summed
    over its batch rows -- depends on that channel's inputs alone, so the fp64 oracle run
    on a few sampled channels gives them exactly; dB and dC (sums over all channels) are
    checked at the 2.8B and 65,536-token sizes."""
    from selective_state_space_53_amd import binding
    cfg = synth.CONFIGS["long"]
    inp = synth.scan_inputs(cfg, DEV)
    dy = torch.randn((1, cfg.dim, cfg.seqlen), generator=torch.Generator(device=DEV).manual_seed(17),
                     device=DEV).to(cfg.io_dtype)
    say("case bwd long full size")
    g = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                             D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                             want_dh0=True)
    torch.cuda.synchronize()
    chans = [0, 517, 1024, cfg.dim - 1]
    idx = torch.tensor(chans, device=DEV)
    sub = lambda t: t.index_select(1, idx).cpu()
    ref = oracle.Oracle().scan_bwd(
        sub(inp["x"]), sub(inp["delta"]), inp["A"][idx].cpu(), inp["B"].cpu(),
        inp["C"].cpu(), sub(dy), D=inp["D"][idx].cpu(), z=sub(inp["z"]),
        delta_bias=inp["delta_bias"][idx].cpu(), nthreads=parity.threads())
    got = {k: (g[k].index_select(1, idx) if k in ("dx", "ddelta", "dz", "dh0")
               else g[k].index_select(0, idx)) for k in OUTS if k not in ("dB", "dC")}
    errs = {}
    for k, v in got.items():
        r = np.asarray(ref[OKEY.get(k, k)])
        gv = oracle.f64(v)
        if k in ("dA", "dD", "ddelta_bias"):
            gv, r = gv.reshape(1, -1), r.reshape(1, -1)
        errs[k] = parity.rowwise_err(gv, r)
    say("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= parity.TOL["bf16"]}
    assert not bad, bad


@pytest.mark.parametrize("shape", [(2, 1000, 200, "bf16"), (1, 333, 70, "f32"),
                                   (1, 4103, 96, "bf16"), (3, 17, 33, "f32")],
                         ids=lambda s: "b{}_L{}_d{}_{}".format(*s))
@pytest.mark.parametrize("plan,chunk,bwd_chunk", [(0, 0, 0), (2, 64, 0), (0, 0, 96)],
                         ids=["auto", "c64", "bwd_c96"])
def test_training_forward_saves_for_backward(shape, plan, chunk, bwd_chunk):
    """Training pair: the forward with save_for_backward writes the same y and h_final as
    the plain forward, and the backward that starts from what it saved (saved=True, no
    checkpoint pass of its own) gives the same gradients, bit for bit, as the backward
    that recomputes them."""
    from selective_state_space_53_amd import binding
    batch, L, dim, io = shape
    cfg = synth.ScanConfig("train", batch, L, dim, io=io, seed=500 + L)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((batch, dim, L), cfg.io_dtype, L + 7)
    h0 = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(5)).to(DEV)
    dhf = torch.randn((batch, dim, 16), generator=torch.Generator().manual_seed(6)).to(DEV)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    kw = dict(D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], h0=h0)
    say("case training pair", shape, plan, chunk, bwd_chunk)
    ws = torch.empty(binding.ssm_scan_bwd_workspace_bytes(batch, L, dim, 16, cfg.io_dtype,
                                                          plan=plan, chunk_len=chunk,
                                                          bwd_chunk_len=bwd_chunk),
                     dtype=torch.uint8, device=DEV)
    ys, hs = binding.ssm_scan_fwd(*args, **kw, return_final_state=True, plan=plan,
                                  chunk_len=chunk, save_for_backward=ws)
    yp, hp = binding.ssm_scan_fwd(*args, **kw, return_final_state=True, plan=plan,
                                  chunk_len=chunk)
    gs = binding.ssm_scan_bwd(*args, dy, **kw, dh_final=dhf, want_dh0=True, plan=plan,
                              chunk_len=chunk, workspace=ws, saved=True, bwd_chunk_len=bwd_chunk)
    gr = binding.ssm_scan_bwd(*args, dy, **kw, dh_final=dhf, want_dh0=True, plan=plan,
                              chunk_len=chunk, bwd_chunk_len=bwd_chunk)
    torch.cuda.synchronize()
    assert torch.equal(ys, yp) and torch.equal(hs, hp)
    for k in OUTS:
        assert torch.equal(gs[k], gr[k]), k
    # and the saved path against the oracle
    ref = oracle.Oracle().scan_bwd(*args, dy, **kw, dh_final=dhf, nthreads=parity.threads())
    _compare(gs, ref, io)


def test_bwd_row_offsets_near_4gib():
    """64 channels of one bf16 row of 33,554,400 tokens in one 64-channel workgroup: the
    last channel's 32-bit byte offsets reach 98.7% of 2^32. The first and last channels'
    own gradients (dx, ddelta, dz, dh0, dA, dD, d_bias) against the fp64 oracle on those
    channels alone."""
    from selective_state_space_53_amd import binding
    L, dim = 33_554_400, 64
    cfg = synth.ScanConfig("near4g", 1, L, dim, io="bf16", seed=71, dt_lo=1e-4, dt_hi=1e-2)
    inp = synth.scan_inputs(cfg, DEV)
    dy = torch.randn((1, dim, L), generator=torch.Generator(device=DEV).manual_seed(19),
                     device=DEV).to(torch.bfloat16)
    say("case bwd offsets near 4 GiB")
    g = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                             D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                             want_dh0=True, bwd_group_channels=64)
    torch.cuda.synchronize()
    idx = torch.tensor([0, dim - 1], device=DEV)
    sub = lambda t: t.index_select(1, idx).cpu()
    ref = oracle.Oracle().scan_bwd(
        sub(inp["x"]), sub(inp["delta"]), inp["A"][idx].cpu(), inp["B"].cpu(),
        inp["C"].cpu(), sub(dy), D=inp["D"][idx].cpu(), z=sub(inp["z"]),
        delta_bias=inp["delta_bias"][idx].cpu(), nthreads=2)
    errs = {}
    for k in OUTS:
        if k in ("dB", "dC"):
            continue
        v = (g[k].index_select(1, idx) if k in ("dx", "ddelta", "dz", "dh0")
             else g[k].index_select(0, idx))
        r = np.asarray(ref[OKEY.get(k, k)])
        gv = oracle.f64(v)
        if k in ("dA", "dD", "ddelta_bias"):
            gv, r = gv.reshape(1, -1), r.reshape(1, -1)
        errs[k] = parity.rowwise_err(gv, r)
    say("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= parity.TOL["bf16"]}
    assert not bad, bad


def test_bwd_integer_exact():
    """A = 0, Delta = 1 (softplus off), no gate, small integers everywhere: every
    intermediate is an exact integer in fp32, so the GPU gradients equal the oracle's
    bit for bit -- across tile edges (16), checkpoint-pass tile and chunk edges, and
    the sums over channels, channel groups and batch rows."""
    from selective_state_space_53_amd import binding
    rng = np.random.default_rng(8)
    batch, L, dim = 2, 97, 70
    x = np.zeros((batch, dim, L))
    for b in range(batch):
        for d in range(dim):
            idx = rng.choice(L, size=6, replace=False)
            x[b, d, idx] = rng.choice([-1.0, 1.0], size=6)
    t = lambda a: torch.tensor(a, dtype=torch.float32, device=DEV)
    inp = {
        "x": t(x), "delta": torch.ones((batch, dim, L), device=DEV), "z": None,
        "B": t(rng.integers(-1, 2, size=(batch, L, 16))),
        "C": t(rng.integers(-1, 2, size=(batch, L, 16))),
        "A": torch.zeros((dim, 16), device=DEV),
        "D": t(rng.integers(-2, 3, size=dim)), "delta_bias": None,
    }
    dy = t(rng.integers(-1, 2, size=(batch, dim, L)))
    dhf = t(rng.integers(-2, 3, size=(batch, dim, 16)))
    for plan, chunk, cg, bch in [(1, 0, 48, 0), (2, 64, 32, 0), (2, 32, 64, 0), (1, 0, 48, 32),
                                 (2, 64, 32, 64)]:
        say("case bwd integer", plan, chunk, cg, bch)
        g = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                                 D=inp["D"], delta_softplus=False, dh_final=dhf, want_dh0=True,
                                 plan=plan, chunk_len=chunk, bwd_group_channels=cg,
                                 bwd_chunk_len=bch)
        torch.cuda.synchronize()
        ref = oracle.Oracle().scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                                       D=inp["D"], delta_softplus=False, dh_final=dhf)
        for k in ["dx", "ddelta", "dA", "dB", "dC", "dD", "dh0"]:
            assert np.array_equal(oracle.f64(g[k]), ref[k]), k
        assert g["ddelta_bias"] is None and g["dz"] is None


def test_bwd_deterministic():
    cfg = synth.ScanConfig("bwddet", 2, 300, 200, io="bf16", seed=5)
    inp = synth.scan_inputs(cfg, DEV)
    dy = _dy((2, 200, 300), torch.bfloat16, 5)
    from selective_state_space_53_amd import binding
    a = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                             D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"])
    b = binding.ssm_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], dy,
                             D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"])
    torch.cuda.synchronize()
    for k in OUTS:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k

"""ssm_scan_fwd_noalloc through the C ABI: the variant of ssm_scan_fwd whose workspace is
the library's static device scratch. Calls in a row, each smaller than the one before
(so each runs on what the previous call left in the scratch), must give outputs bit for
bit equal to ssm_scan_fwd with a workspace of its own (same kernels, same plan), and
match the fp64 oracle within the io tolerance.
"""
import sys

import pytest
import torch

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


# (config, plan, chunk_len, rows checked against the oracle; 0 = all): the Mamba-2.8B
# layer in the library's own plan (1 MiB of B/C workspace), then smaller shapes in
# forced chunked plans (chunk states and sums in the scratch too), the last one fp32
CASES = [
    (synth.CONFIGS["m2p8"], 0, 0, 96),
    (synth.ScanConfig("na_mid", 2, 3000, 200, io="bf16", seed=41), 2, 96, 0),
    (synth.ScanConfig("na_small", 1, 1000, 70, io="f32", seed=42), 2, 64, 0),
]


def _outputs(fn, inp, cfg, plan, chunk, h0):
    return fn(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
              delta_bias=inp["delta_bias"], h0=h0, return_final_state=True, plan=plan,
              chunk_len=chunk)


def test_noalloc_equals_fwd_calls_in_a_row():
    from selective_state_space_53_amd import binding
    for i, (cfg, plan, chunk, nrows) in enumerate(CASES):
        say(f"case noalloc call {i}: {cfg.name} b={cfg.batch} L={cfg.seqlen} d={cfg.dim} "
            f"{cfg.io} plan={plan} chunk={chunk}")
        inp = synth.scan_inputs(cfg, DEV)
        gen = torch.Generator(device="cpu").manual_seed(100 + i)
        h0 = torch.randn((cfg.batch, cfg.dim, 16), generator=gen).to(DEV)
        y_na, hf_na = _outputs(binding.ssm_scan_fwd_noalloc, inp, cfg, plan, chunk, h0)
        torch.cuda.synchronize()
        y_ws, hf_ws = _outputs(binding.ssm_scan_fwd, inp, cfg, plan, chunk, h0)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), cfg.name
        assert torch.equal(hf_na, hf_ws), cfg.name
        if nrows:
            rb, rd = parity.sample_rows(cfg.batch, cfg.dim, nrows, seed=cfg.seed)
            yr, hr = parity.oracle_rows(inp, rb, rd, h0=h0)
            sel = (torch.as_tensor(rb, device=DEV), torch.as_tensor(rd, device=DEV))
            ey, eh = parity.rowwise_err(y_na[sel], yr), parity.rowwise_err(hf_na[sel], hr)
        else:
            yr, hr = parity.oracle_full(inp, h0=h0)
            ey, eh = parity.rowwise_err(y_na, yr), parity.rowwise_err(hf_na, hr)
        say(f"  y err {ey:.3e}  h_final err {eh:.3e}")
        assert ey <= parity.TOL[cfg.io] and eh <= parity.TOL[cfg.io]


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    """A million-token row needs 128 MiB of B/C workspace: refused before any launch."""
    from selective_state_space_53_amd import binding
    cfg = synth.shrink(synth.CONFIGS["long"], dim=16)
    inp = synth.scan_inputs(cfg, DEV)
    y = torch.zeros_like(inp["x"])
    with pytest.raises(binding.SSMError) as ei:
        binding.ssm_scan_fwd_noalloc(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], y=y)
    assert ei.value.status == binding.SSM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0

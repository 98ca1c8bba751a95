"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/ssm_scan.h declares, and rejects bad calls on the host before
any HIP call (only failing calls are made here; pointers are fake but aligned)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")
LIB = os.path.join(ROOT, "selective_state_space_53_amd", "libssmscan.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libssmscan.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def b():
    from selective_state_space_53_amd import binding
    return binding


def test_exports_every_declared_symbol(b):
    names = declared_functions()
    assert set(names) == set(b.EXPORTS), names
    for n in names:
        assert hasattr(b.lib, n), n
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_strings(b):
    hdr = open(os.path.join(ROOT, "include", "ssm_scan.h")).read()
    declared = int(re.search(r"#define SSM_SCAN_ABI_VERSION (\d+)", hdr).group(1))
    assert b.ssm_abi_version() == declared == b.ABI_VERSION
    assert b.ssm_status_string(0) == "ok"
    assert b.ssm_status_string(3) == "workspace too small"
    assert b.ssm_status_string(99) == "unknown status"


# fake device addresses: far apart, 256-byte aligned
P = {k: 0x7f0000000000 + i * (1 << 36) for i, k in enumerate(
    ["x", "delta", "A", "B", "C", "D", "z", "bias", "h0", "y", "hf", "ws"])}


def _chunked(b):
    """Forced chunked plan (chunks of 32 tokens): the forward then needs a workspace, so
    every call here that should be refused has a workspace region to check against (the
    single-pass plan needs none)."""
    return ctypes.byref(b.ScanOptions(32, 2, 0))


def scan(b, batch=2, seqlen=64, dim=64, dstate=16, io=1, ws_bytes=None, opts=None, **over):
    p = dict(P)
    p.update(over)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    if opts is None:
        opts = _chunked(b)
    return b.lib.ssm_scan_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                              p["bias"], p.get("softplus", 1), p["h0"], p["y"], p["hf"], batch,
                              seqlen, dim, dstate, io, p["ws"], ws_bytes, opts, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(seqlen=0), 1), (dict(dim=-3), 1), (dict(dstate=0), 1),
    (dict(dstate=8), 2), (dict(dstate=32), 2), (dict(io=7), 1),
    (dict(x=None), 1), (dict(delta=None), 1), (dict(A=None), 1), (dict(B=None), 1),
    (dict(C=None), 1), (dict(y=None), 1), (dict(softplus=2), 1),
    (dict(x=P["x"] + 8), 2), (dict(y=P["y"] + 2), 2), (dict(A=P["A"] + 2), 2),
    (dict(h0=P["h0"] + 4), 2),
    (dict(y=P["x"]), 1), (dict(y=P["x"] + 16), 1), (dict(y=P["B"]), 1),
    (dict(hf=P["h0"] + 16), 1), (dict(ws=P["y"]), 1), (dict(hf=P["y"]), 1),
    (dict(ws=None), 3), (dict(ws_bytes=16), 3),
])
def test_scan_rejects(b, kw, status):
    assert scan(b, **kw) == status
    assert b.ssm_last_error() != ""


def test_scan_rejects_bad_options(b):
    assert scan(b, opts=ctypes.byref(b.ScanOptions(48, 2, 0))) == 1   # not a multiple of 32
    assert scan(b, opts=ctypes.byref(b.ScanOptions(0, 0, 0, None, None, 2, 0))) == 1  # reverse
    assert scan(b, opts=ctypes.byref(b.ScanOptions(0, 0, 0, None, None, 0, -1))) == 1  # accumulate
    assert scan(b, opts=ctypes.byref(b.ScanOptions(64, 4, 0))) == 1   # unknown plan
    assert scan(b, opts=ctypes.byref(b.ScanOptions(64, 2, 40))) == 1  # group size
    assert scan(b, opts=ctypes.byref(b.ScanOptions(64, 2, 112))) == 1
    assert scan(b, opts=ctypes.byref(b.ScanOptions(-32, 2, 0))) == 1
    # structured_a: 0 or 1, with any plan
    for plan in (0, 1, 2, 3):
        o = b.ScanOptions(0, plan, 0)
        o.structured_a = 2
        assert scan(b, opts=ctypes.byref(o)) == 1


def noalloc(b, batch=2, seqlen=64, dim=64, dstate=16, io=1, opts=None, **over):
    p = dict(P)
    p.update(over)
    if opts == "chunks of 64":
        opts = ctypes.byref(b.ScanOptions(64, 2, 0))
    return b.lib.ssm_scan_fwd_noalloc(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"],
                                      p["z"], p["bias"], p.get("softplus", 1), p["h0"], p["y"],
                                      p["hf"], batch, seqlen, dim, dstate, io, opts, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(dstate=8), 2), (dict(x=None), 1), (dict(y=None), 1),
    (dict(softplus=2), 1), (dict(x=P["x"] + 8), 2), (dict(y=P["x"]), 1),
    (dict(hf=P["h0"] + 16), 1),
    # workspaces beyond the 32 MiB scratch: a million-token row (B/C widened: 128 MiB),
    # and a forced chunked plan whose chunk states do not fit
    (dict(batch=1, seqlen=1 << 20, dim=1536), 2),
    (dict(batch=64, seqlen=4096, dim=1024, opts="chunks of 64"), 2),
])
def test_noalloc_rejects(b, kw, status):
    """ssm_scan_fwd_noalloc: the checks of ssm_scan_fwd, and shapes whose workspace would not
    fit the static scratch, are refused on the host before the scratch is looked up."""
    assert noalloc(b, **kw) == status
    assert b.ssm_last_error() != ""


def test_workspace_query(b):
    # single pass: B and C widened to fp32, per state quad, tokens padded to 32
    assert b.ssm_scan_workspace_bytes(4, 2048, 5120, 16, 1) == 4 * 2048 * 32 * 4
    import torch
    assert b.ssm_scan_workspace_bytes(4, 2048, 5120, 16, torch.bfloat16) == 4 * 2048 * 32 * 4
    with pytest.raises(TypeError):
        b.ssm_scan_workspace_bytes(4, 2048, 5120, 16, torch.float16)
    assert b.ssm_scan_workspace_bytes(1, 100, 16, 16, 0, plan=1) == 128 * 32 * 4
    # forced chunking adds one state (16 fp32) and one sum per (row, chunk)
    ws = b.ssm_scan_workspace_bytes(2, 1000, 70, 16, 1, plan=2, chunk_len=64)
    k = 16
    bcq = 2 * 1024 * 32 * 4
    st = 2 * 70 * k * 16 * 4
    sm = 2 * 70 * k * 4
    def up(v):
        return (v + 255) // 256 * 256
    assert ws == up(up(up(up(bcq) + st) + sm) + k * 4)
    assert b.ssm_scan_workspace_bytes(0, 10, 10, 16, 1) == 0
    assert b.ssm_scan_workspace_bytes(1, 10, 10, 8, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(dstate=4), 2), (dict(state=None), 1), (dict(y=None), 1),
    (dict(y=P["x"]), 1), (dict(state=P["B"]), 1), (dict(y=P["hf"] + 8), 2), (dict(io=3), 1),
])
def test_state_update_rejects(b, kw, status):
    p = dict(P, state=P["hf"])
    batch = kw.pop("batch", 4)
    dstate = kw.pop("dstate", 16)
    io = kw.pop("io", 1)
    p.update(kw)
    st = b.lib.ssm_state_update(p["state"], p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"],
                                p["z"], p["bias"], 1, p["y"], batch, 32, dstate, io, None)
    assert st == status


def varlen(b, total=100, dim=64, nseq=3, io=1, ws_bytes=None, **over):
    p = dict(P, cu=0x7e0000000000)
    p.update(over)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return b.lib.ssm_scan_varlen_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                     p["bias"], 1, p["cu"], nseq, p["h0"], p["y"], p["hf"], total,
                                     dim, 16, io, p["ws"], ws_bytes, _chunked(b), None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), 1), (dict(nseq=0), 1), (dict(total=-1), 1), (dict(total=1 << 31), 1),
    (dict(cu=0x7e0000000002), 2), (dict(dim=0), 1), (dict(ws=None), 3),
    (dict(hf=P["h0"] + 16), 1), (dict(y=P["x"]), 1), (dict(h0=P["h0"] + 4), 2),
    (dict(total=0, hf=P["h0"] + 16), 1), (dict(total=0, hf=P["hf"] + 4), 2),
    (dict(total=0, dim=0), 1), (dict(hf=P["h0"]), 2),
])
def test_varlen_rejects(b, kw, status):
    assert varlen(b, **kw) == status
    assert b.ssm_last_error() != ""


def test_varlen_workspace_query(b):
    assert b.ssm_scan_varlen_workspace_bytes(0, 64, 16, 1) == 0
    assert (b.ssm_scan_varlen_workspace_bytes(1000, 64, 16, 1, plan=2, chunk_len=64)
            == b.ssm_scan_workspace_bytes(1, 1000, 64, 16, 1, plan=2, chunk_len=64))
    # chunked: B/C staging, chunk states, chunk sums, one flag per chunk
    ws = b.ssm_scan_workspace_bytes(1, 1000, 64, 16, 1, plan=2, chunk_len=64)
    def up(v):
        return (v + 255) // 256 * 256
    k = 16
    assert ws == up(up(up(up(1024 * 32 * 4) + 64 * k * 16 * 4) + 64 * k * 4) + k * 4)


def conv(b, batch=2, seqlen=64, dim=64, width=4, act=1, io=1, **over):
    p = dict(P, cs=P["h0"], cso=P["hf"])
    p.update(over)
    return b.lib.ssm_causal_conv1d_fwd(p["x"], p["A"], p["D"], p["cs"], p["y"], p["cso"], batch,
                                       seqlen, dim, width, act, io, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(seqlen=0), 1), (dict(width=3), 2), (dict(width=0), 1),
    (dict(act=2), 1), (dict(io=5), 1), (dict(x=None), 1), (dict(A=None), 1), (dict(y=None), 1),
    (dict(x=P["x"] + 8), 2), (dict(A=P["A"] + 4), 2), (dict(cs=P["h0"] + 1), 2),
    (dict(y=P["x"]), 1), (dict(cso=P["h0"]), 1), (dict(cso=P["y"] + 64), 1),
])
def test_conv_rejects(b, kw, status):
    assert conv(b, **kw) == status
    assert b.ssm_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(width=5), 2), (dict(state=None), 1), (dict(y=None), 1),
    (dict(y=P["x"]), 1), (dict(state=P["x"]), 1), (dict(act=-1), 1),
])
def test_conv_update_rejects(b, kw, status):
    p = dict(P, state=P["hf"])
    batch = kw.pop("batch", 4)
    width = kw.pop("width", 4)
    act = kw.pop("act", 1)
    p.update(kw)
    assert b.lib.ssm_causal_conv1d_update(p["state"], p["x"], p["A"], p["D"], p["y"], batch, 32,
                                          width, act, 1, None) == status


def test_binding_wraps_every_export(b):
    for n in b.EXPORTS:
        assert callable(getattr(b, n)), n


def test_forward_group_channels(b):
    # channels per workgroup: multiples of 16 from 16 to 96, else refused
    for cg in (16, 32, 48, 64, 80, 96):
        assert b.ssm_scan_workspace_bytes(2, 100, 64, 16, 1, group_channels=cg) > 0, cg
    for cg in (8, 24, 112, -16):
        assert b.ssm_scan_workspace_bytes(2, 100, 64, 16, 1, group_channels=cg) == 0, cg


def test_bwd_workspace_and_rejects(b):
    ws = b.ssm_scan_bwd_workspace_bytes(2, 100, 64, 16, 1)
    assert ws > b.ssm_scan_workspace_bytes(2, 100, 64, 16, 1)
    assert b.ssm_scan_bwd_workspace_bytes(2, 100, 64, 8, 1) == 0
    assert b.ssm_scan_bwd_workspace_bytes(2, 100, 64, 16, 1, bwd_group_channels=40) == 0
    assert b.ssm_scan_bwd_workspace_bytes(2, 100, 64, 16, 1, bwd_chunk_len=48) == 0
    # chunking adds the carried gradients, sums of Delta and per-chunk partials
    assert (b.ssm_scan_bwd_workspace_bytes(2, 1000, 64, 16, 1, bwd_chunk_len=64)
            > b.ssm_scan_bwd_workspace_bytes(2, 1000, 64, 16, 1, bwd_chunk_len=1024))
    p = dict(P, dy=P["z"] + (1 << 35), dx=P["y"], dd=P["y"] + (1 << 34), dz=P["hf"] + (1 << 34),
             dA=P["ws"] + (1 << 35), dB=P["ws"] + (1 << 34), dC=P["ws"] + (3 << 33),
             dD=P["D"] + (1 << 34), dbias=P["bias"] + (1 << 34), dh0=P["h0"] + (1 << 34))

    def call(**over):
        q = dict(p)
        q.update(over)
        return b.lib.ssm_scan_bwd(q["x"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"],
                                  q["bias"], 1, q["h0"], q["dy"], None, q["dx"], q["dd"], q["dz"],
                                  q["dA"], q["dB"], q["dC"], q["dD"], q["dbias"], q["dh0"], 2,
                                  100, 64, 16, 1, q["ws"], 1 << 40, None, None)
    assert call(dy=None) == 1
    assert call(dz=None) == 1                  # z given, dz missing
    assert call(dx=P["x"]) == 1                # output overlaps an input
    assert call(dB=p["dC"]) == 1               # outputs overlap each other
    assert call(dx=P["y"] + 8) == 2            # misaligned
    assert call(ws=None) == 3
    opts = b.ScanOptions(0, 0, 0, None, None, 0, 1, 0, 0)   # accumulate: no backward
    q = dict(p)
    assert b.lib.ssm_scan_bwd(q["x"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"],
                              q["bias"], 1, q["h0"], q["dy"], None, q["dx"], q["dd"], q["dz"],
                              q["dA"], q["dB"], q["dC"], q["dD"], q["dbias"], q["dh0"], 2, 100,
                              64, 16, 1, q["ws"], 1 << 40, ctypes.byref(opts), None) == 2


def _save_opts(b, save, nbytes, saved=0, reverse=0, accumulate=0):
    # (chunked plan, so that the forward's own workspace is not empty: see _chunked)
    return ctypes.byref(b.ScanOptions(32, 2, 0, None, None, reverse, accumulate, 0, 0, save,
                                      nbytes, saved))


def test_training_forward_save_rejects(b):
    """ssm_scan_fwd with save_workspace (checkpoints and q for the backward): the size
    formula in the header, and every check before anything is launched."""
    batch, L, dim = 2, 64, 64
    need = (batch * dim * ((L + 15) // 16) * 64 + 255) // 256 * 256 + batch * dim * L * 2
    sv = 0x7d0000000000
    # one byte fewer than the header's formula is refused (every call here fails a check
    # before any launch: the addresses are not real)
    assert scan(b, opts=_save_opts(b, sv, need - 1)) == 3
    # the anti-causal scan saves too, the same bytes (one byte short is refused)
    assert scan(b, opts=_save_opts(b, sv, need - 1, reverse=1)) == 3
    assert scan(b, opts=_save_opts(b, sv, need, accumulate=1)) == 2
    assert scan(b, opts=_save_opts(b, sv + 8, need)) == 2             # misaligned
    assert scan(b, opts=_save_opts(b, P["x"], need)) == 1             # overlaps an input
    assert scan(b, opts=_save_opts(b, P["y"] - 64, need)) == 1        # overlaps y
    assert scan(b, opts=_save_opts(b, P["ws"], need)) == 1            # overlaps the workspace
    assert scan(b, opts=_save_opts(b, None, 0, saved=1)) == 1         # a backward option
    # packed sequences cannot save
    p = dict(P, cu=0x7e0000000000)
    assert b.lib.ssm_scan_varlen_fwd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"],
                                     p["z"], p["bias"], 1, p["cu"], 3, p["h0"], p["y"],
                                     p["hf"], 100, 64, 16, 1, p["ws"], 1 << 40,
                                     _save_opts(b, sv, 1 << 30), None) == 2
    # the backward workspace starts with that region
    assert b.ssm_scan_bwd_workspace_bytes(batch, L, dim, 16, 1) > need


def test_backward_saved_option_rejects(b):
    p = dict(P, dy=P["z"] + (1 << 35), dx=P["y"], dd=P["y"] + (1 << 34), dz=P["hf"] + (1 << 34),
             dA=P["ws"] + (1 << 35), dB=P["ws"] + (1 << 34), dC=P["ws"] + (3 << 33),
             dD=P["D"] + (1 << 34), dbias=P["bias"] + (1 << 34), dh0=P["h0"] + (1 << 34))

    def call(opts):
        q = p
        return b.lib.ssm_scan_bwd(q["x"], q["delta"], q["A"], q["B"], q["C"], q["D"], q["z"],
                                  q["bias"], 1, q["h0"], q["dy"], None, q["dx"], q["dd"], q["dz"],
                                  q["dA"], q["dB"], q["dC"], q["dD"], q["dbias"], q["dh0"], 2,
                                  100, 64, 16, 1, q["ws"], 1 << 40, opts, None)
    assert call(_save_opts(b, 0x7d0000000000, 1 << 30)) == 1   # save_workspace: forward only
    assert call(_save_opts(b, None, 0, saved=2)) == 1


def test_backward_sequence_length_limit(b):
    """The backward addresses one workgroup's rows with 32-bit offsets: the planner picks
    channels per workgroup (64, 48, 32) whose rows span less than 4 GiB, and refuses a
    row too long even for 32 channels."""
    f32, bf16 = 0, 1
    assert b.ssm_scan_bwd_workspace_bytes(1, (1 << 32) // 128 - 1, 16, 16, f32) > 0
    assert b.ssm_scan_bwd_workspace_bytes(1, (1 << 32) // 128, 16, 16, f32) == 0
    assert b.ssm_scan_bwd_workspace_bytes(1, 1 << 25, 16, 16, bf16) > 0          # 48 or 32
    assert b.ssm_scan_bwd_workspace_bytes(1, 1 << 25, 16, 16, bf16, bwd_group_channels=64) == 0
    assert b.ssm_scan_bwd_workspace_bytes(1, 1 << 26, 16, 16, bf16) == 0


def varlen_bwd(b, total=100, dim=64, nseq=3, io=1, ws_bytes=None, opts=None, **over):
    p = dict(P, cu=0x7e0000000000, dy=P["z"] + (1 << 35), dhf=P["hf"] + (1 << 35), dx=P["y"],
             dd=P["y"] + (1 << 34), dz=P["hf"] + (1 << 34), dA=P["ws"] + (1 << 35),
             dB=P["ws"] + (1 << 34), dC=P["ws"] + (3 << 33), dD=P["D"] + (1 << 34),
             dbias=P["bias"] + (1 << 34), dh0=P["h0"] + (1 << 34))
    p.update(over)
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return b.lib.ssm_scan_varlen_bwd(
        p["x"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["bias"], 1, p["cu"], nseq,
        p["h0"], p["dy"], p["dhf"], p["dx"], p["dd"], p["dz"], p["dA"], p["dB"], p["dC"],
        p["dD"], p["dbias"], p["dh0"], total, dim, 16, io, p["ws"], ws_bytes, opts, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), 1), (dict(nseq=0), 1), (dict(total=-1), 1), (dict(total=1 << 31), 1),
    (dict(cu=0x7e0000000002), 2), (dict(dim=0), 1), (dict(ws=None), 3), (dict(ws_bytes=64), 3),
    (dict(dy=None), 1), (dict(dz=None), 1), (dict(dx=P["x"]), 1), (dict(dB=P["ws"] + (3 << 33)), 1),
    (dict(dh0=P["h0"] + 4), 2), (dict(dh0=P["h0"]), 1),
    # dh0 [nseq][dim][16] overlapping dh_final, with no tokens and with tokens
    (dict(total=0, dh0=P["hf"] + (1 << 35) + 64), 1), (dict(dh0=P["hf"] + (1 << 35) + 64), 1),
    (dict(total=0, dA=P["hf"] + (1 << 35)), 1), (dict(total=0, dh0=P["h0"] + 8), 2),
    (dict(total=0, dim=0), 1), (dict(total=0, dA=None), 1),
    # one fp32 row of the backward must span less than 4 GiB even at 32 channels per group
    (dict(total=1 << 25, io=0), 2),
])
def test_varlen_bwd_rejects(b, kw, status):
    assert varlen_bwd(b, **kw) == status
    assert b.ssm_last_error() != ""


def test_varlen_bwd_workspace_and_options(b):
    assert b.ssm_scan_varlen_bwd_workspace_bytes(0, 64, 16, 1) == 0
    for kw in ({}, dict(bwd_chunk_len=64), dict(plan=2, chunk_len=64, bwd_group_channels=32)):
        assert (b.ssm_scan_varlen_bwd_workspace_bytes(1000, 64, 16, 1, **kw)
                == b.ssm_scan_bwd_workspace_bytes(1, 1000, 64, 16, 1, **kw))
    # the checkpoints are always recomputed: saved=1 is refused; the anti-causal
    # backward takes the same workspace (one short of it is refused)
    assert varlen_bwd(b, opts=_save_opts(b, None, 0, saved=1)) == 2
    rev = _save_opts(b, None, 0, reverse=1)
    need = b.lib.ssm_scan_varlen_bwd_workspace_bytes(100, 64, 16, 1, rev)
    assert need == b.ssm_scan_varlen_bwd_workspace_bytes(100, 64, 16, 1, plan=2,
                                                          chunk_len=32) > 0
    assert varlen_bwd(b, opts=rev, ws_bytes=need - 1) == 3
    assert varlen_bwd(b, opts=_save_opts(b, 0x7d0000000000, 1 << 30)) == 1


def test_reverse_backward_workspace(b):
    """The anti-causal backward uses the causal backward's workspace layout and size."""
    rev = ctypes.byref(b.ScanOptions(0, 0, 0, None, None, 1, 0, 0, 0))
    for L in (100, 4103):
        assert (b.lib.ssm_scan_bwd_workspace_bytes(2, L, 64, 16, 1, rev)
                == b.ssm_scan_bwd_workspace_bytes(2, L, 64, 16, 1) > 0)

"""fp64 CPU oracle for the selective scan -- TEST INFRASTRUCTURE.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package. The product path (the HIP library and its binding) never
does: it shares no code with it and fails loudly when its own library is missing.

The scan's arithmetic lives in `ssm_oracle.c` (plain C, fp64, one sequential loop
per row; see `ssm_oracle.h` for the recurrence and where each part of it comes
from on the pages). This module builds that file with gcc, widens inputs exactly
to fp64 and calls it through ctypes; the reverse-time and packed scans are defined
here from it, and the causal convolution before the scan is plain numpy in fp64.

Every oracle function is pinned by CPU tests against things other than itself
(closed forms, library routines, brute force, invariants): see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "ssm_oracle.c"), os.path.join(_HERE, "ssm_oracle_bwd.c")]
_LIB_PATH = os.path.join(_HERE, "libssmoracle.so")
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True, out: str | None = None, extra_flags=()) -> str:
    """Compile the oracle's C files with gcc (no fast-math: IEEE fp64 throughout)."""
    out = out or _LIB_PATH
    srcs = _SRCS
    if (not force and os.path.exists(out)
            and all(os.path.getmtime(out) >= os.path.getmtime(s) for s in srcs)):
        return out
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", *extra_flags, *srcs, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    return out


def _load(path: str | None = None):
    lib = ctypes.CDLL(path or _LIB_PATH)
    lib.ssm_oracle_softplus.restype = ctypes.c_double
    lib.ssm_oracle_softplus.argtypes = [ctypes.c_double]
    lib.ssm_oracle_silu.restype = ctypes.c_double
    lib.ssm_oracle_silu.argtypes = [ctypes.c_double]
    lib.ssm_oracle_scan_rows.restype = ctypes.c_int
    lib.ssm_oracle_scan_rows.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _ip, _ip,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, ctypes.c_int]
    lib.ssm_oracle_scan_bwd_rows.restype = ctypes.c_int
    lib.ssm_oracle_scan_bwd_rows.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _ip, _ip, ctypes.c_int64, ctypes.c_int64,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp,
        _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int]
    lib.ssm_oracle_step_rows.restype = ctypes.c_int
    lib.ssm_oracle_step_rows.argtypes = [
        ctypes.c_int64, ctypes.c_int64, _ip, _ip, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
        _dp, ctypes.c_int, _dp]
    return lib


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = _load()
        return _lib


class Oracle:
    """A handle on one built copy of the oracle (tests build planted-mistake
    copies of the same source to show the pins catch them)."""

    def __init__(self, path: str | None = None):
        self._l = _load(path) if path else lib()

    # ---- scalar helpers -------------------------------------------------
    def softplus(self, v: float) -> float:
        return self._l.ssm_oracle_softplus(float(v))

    def silu(self, z: float) -> float:
        return self._l.ssm_oracle_silu(float(z))

    # ---- scan -----------------------------------------------------------
    def scan_rows(self, x_rows, delta_rows, A, B, C, row_b, row_d, z_rows=None, D=None,
                  delta_bias=None, delta_softplus=True, h0_rows=None, nthreads=1,
                  want_final=True):
        """Rows given explicitly: x_rows/delta_rows/z_rows are [R][L]; B, C are
        [batch][L][N]; A is [dim][N]; row_b/row_d name each row's batch and channel."""
        x_rows = f64(x_rows)
        delta_rows = f64(delta_rows)
        R, L = x_rows.shape
        A = f64(A)
        N = A.shape[1]
        B = f64(B)
        C = f64(C)
        assert B.shape[1:] == (L, N) and C.shape == B.shape and delta_rows.shape == (R, L)
        rb = np.ascontiguousarray(np.asarray(row_b, dtype=np.int64).reshape(R))
        rd = np.ascontiguousarray(np.asarray(row_d, dtype=np.int64).reshape(R))
        assert rb.size == 0 or (rb.min() >= 0 and rb.max() < B.shape[0])
        assert rd.size == 0 or (rd.min() >= 0 and rd.max() < A.shape[0])
        z_rows = None if z_rows is None else f64(z_rows)
        if z_rows is not None:
            assert z_rows.shape == (R, L)
        D = None if D is None else f64(D)
        delta_bias = None if delta_bias is None else f64(delta_bias)
        h0_rows = None if h0_rows is None else f64(h0_rows).reshape(R, N)
        y = np.empty((R, L), dtype=np.float64)
        hf = np.empty((R, N), dtype=np.float64) if want_final else None
        rc = self._l.ssm_oracle_scan_rows(
            R, L, N, _ptr_i(rb), _ptr_i(rd), _ptr(x_rows), _ptr(delta_rows), _ptr(z_rows),
            _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(delta_bias), int(bool(delta_softplus)),
            _ptr(h0_rows), _ptr(y), _ptr(hf), int(nthreads))
        if rc != 0:
            raise RuntimeError("ssm_oracle_scan_rows failed")
        return y, hf

    def scan(self, x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
             h0=None, nthreads=1):
        """Full tensors: x, delta, z are [batch][dim][L]; h0 [batch][dim][N].
        Returns y [batch][dim][L] and h_final [batch][dim][N] in fp64."""
        x = f64(x)
        b, d, L = x.shape
        N = f64(A).shape[1]
        rb = np.repeat(np.arange(b, dtype=np.int64), d)
        rd = np.tile(np.arange(d, dtype=np.int64), b)
        y, hf = self.scan_rows(
            x.reshape(b * d, L), f64(delta).reshape(b * d, L), A, B, C, rb, rd,
            z_rows=None if z is None else f64(z).reshape(b * d, L), D=D,
            delta_bias=delta_bias, delta_softplus=delta_softplus,
            h0_rows=None if h0 is None else f64(h0).reshape(b * d, N), nthreads=nthreads)
        return y.reshape(b, d, L), hf.reshape(b, d, N)

    # ---- gradients ------------------------------------------------------
    def scan_bwd(self, x, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                 delta_softplus=True, h0=None, dh_final=None, nthreads=1):
        """Gradients of sum(dy * y) + sum(dh_final * h_final) for the forward scan with
        the same arguments (full tensors, [batch][dim][L] layouts). Returns a dict with
        dx, ddelta, dz ([batch][dim][L]), dA [dim][N], dB, dC [batch][L][N], dD, dbias
        [dim] and dh0 [batch][dim][N], in fp64; dz / dD are None without z / D."""
        x = f64(x)
        b, d, L = x.shape
        A = f64(A)
        N = A.shape[1]
        B = f64(B)
        C = f64(C)
        rb = np.repeat(np.arange(b, dtype=np.int64), d)
        rd = np.tile(np.arange(d, dtype=np.int64), b)
        R = b * d
        rows = lambda t: None if t is None else np.ascontiguousarray(f64(t).reshape(R, -1))
        xz, dl, zz, dyy = rows(x), rows(delta), rows(z), rows(dy)
        h0r, dhf = rows(h0), rows(dh_final)
        Df = None if D is None else f64(D)
        bias = None if delta_bias is None else f64(delta_bias)
        out = {k: np.empty((R, L)) for k in ("dx", "ddelta")}
        out["dz"] = np.empty((R, L)) if z is not None else None
        out["dA"] = np.empty((d, N))
        out["dB"] = np.empty((b, L, N))
        out["dC"] = np.empty((b, L, N))
        out["dD"] = np.empty(d) if D is not None else None
        out["dbias"] = np.empty(d)
        out["dh0"] = np.empty((R, N))
        rc = self._l.ssm_oracle_scan_bwd_rows(
            R, L, N, _ptr_i(rb), _ptr_i(rd), b, d, _ptr(xz), _ptr(dl), _ptr(zz), _ptr(A),
            _ptr(B), _ptr(C), _ptr(Df), _ptr(bias), int(bool(delta_softplus)), _ptr(h0r),
            _ptr(dyy), _ptr(dhf), _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dz"]),
            _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
            _ptr(out["dbias"]), _ptr(out["dh0"]), int(nthreads))
        if rc != 0:
            raise RuntimeError("ssm_oracle_scan_bwd_rows failed")
        for k in ("dx", "ddelta", "dz"):
            if out[k] is not None:
                out[k] = out[k].reshape(b, d, L)
        out["dh0"] = out["dh0"].reshape(b, d, N)
        return out

    # ---- reverse-time and packed (varlen) scans ---------------------------
    def scan_reverse(self, x, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=True, h0=None, nthreads=1):
        """The scan run backwards in time: h_t = exp(Delta_t A) h_{t+1} + Delta_t B_t x_t,
        h_L = h0. By definition the forward scan of the time-reversed inputs, with the
        outputs reversed back; h_final is the state after token 0."""
        rx = f64(x)[:, :, ::-1]
        rd = f64(delta)[:, :, ::-1]
        rz = None if z is None else f64(z)[:, :, ::-1]
        rB = f64(B)[:, ::-1]
        rC = f64(C)[:, ::-1]
        y, hf = self.scan(rx, rd, A, rB, rC, D=D, z=rz, delta_bias=delta_bias,
                          delta_softplus=delta_softplus, h0=h0, nthreads=nthreads)
        return np.ascontiguousarray(y[:, :, ::-1]), hf

    def scan_reverse_bwd(self, x, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                         delta_softplus=True, h0=None, dh_final=None, nthreads=1):
        """Gradients through scan_reverse. That scan is the forward scan of the
        time-reversed inputs with y reversed back, so its gradients are scan_bwd of the
        reversed inputs and the reversed dy, with the per-token gradients (dx, ddelta,
        dz, dB, dC) reversed back. dA, dD, dbias are sums over tokens, and h0 (the state
        entering at the last token) and h_final (the state after token 0) keep their
        meaning, so dh0 and dh_final need no relabelling."""
        rt = lambda v: None if v is None else np.ascontiguousarray(f64(v)[:, :, ::-1])
        rl = lambda v: np.ascontiguousarray(f64(v)[:, ::-1])
        g = self.scan_bwd(rt(x), rt(delta), A, rl(B), rl(C), rt(dy), D=D, z=rt(z),
                          delta_bias=delta_bias, delta_softplus=delta_softplus, h0=h0,
                          dh_final=dh_final, nthreads=nthreads)
        for k in ("dx", "ddelta", "dz"):
            if g[k] is not None:
                g[k] = np.ascontiguousarray(g[k][:, :, ::-1])
        g["dB"] = np.ascontiguousarray(g["dB"][:, ::-1])
        g["dC"] = np.ascontiguousarray(g["dC"][:, ::-1])
        return g

    def scan_varlen_bwd(self, x, delta, A, B, C, dy, cu_seqlens, D=None, z=None,
                        delta_bias=None, delta_softplus=True, h0=None, dh_final=None,
                        reverse=False, nthreads=1):
        """Gradients through scan_varlen: every sequence is its own scan, so its
        gradients are scan_bwd (reverse: scan_reverse_bwd) of that sequence alone (with
        its h0 and dh_final); the
        per-token gradients (dx, ddelta, dz [dim][total], dB, dC [total][N]) are placed
        at its tokens, the per-channel ones (dA, dD, dbias) summed over sequences, and
        dh0 [nseq][dim][N] is per sequence (an empty sequence passes dh_final through:
        its final state is its initial state)."""
        x = f64(x)
        dim, total = x.shape
        N = f64(A).shape[1]
        cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
        nseq = len(cu) - 1
        assert cu[0] == 0 and cu[-1] == total and all(a <= b for a, b in zip(cu, cu[1:]))
        dl, Bf, Cf, dyf = f64(delta), f64(B), f64(C), f64(dy)
        zf = None if z is None else f64(z)
        h0f = None if h0 is None else f64(h0)
        dhf = None if dh_final is None else f64(dh_final)
        out = {"dx": np.zeros((dim, total)), "ddelta": np.zeros((dim, total)),
               "dz": np.zeros((dim, total)) if z is not None else None,
               "dA": np.zeros((dim, N)), "dB": np.zeros((total, N)), "dC": np.zeros((total, N)),
               "dD": np.zeros(dim) if D is not None else None, "dbias": np.zeros(dim),
               "dh0": np.zeros((nseq, dim, N))}
        for i in range(nseq):
            a, b = cu[i], cu[i + 1]
            if b == a:
                out["dh0"][i] = 0.0 if dhf is None else dhf[i]
                continue
            fn = self.scan_reverse_bwd if reverse else self.scan_bwd
            g = fn(x[None, :, a:b], dl[None, :, a:b], A, Bf[None, a:b, :], Cf[None, a:b, :],
                   dyf[None, :, a:b], D=D, z=None if zf is None else zf[None, :, a:b],
                   delta_bias=delta_bias, delta_softplus=delta_softplus,
                   h0=None if h0f is None else h0f[i][None],
                   dh_final=None if dhf is None else dhf[i][None], nthreads=nthreads)
            for k in ("dx", "ddelta") + (("dz",) if z is not None else ()):
                out[k][:, a:b] = g[k][0]
            out["dB"][a:b] = g["dB"][0]
            out["dC"][a:b] = g["dC"][0]
            out["dA"] += g["dA"]
            out["dbias"] += g["dbias"]
            if D is not None:
                out["dD"] += g["dD"]
            out["dh0"][i] = g["dh0"][0]
        return out

    def scan_varlen(self, x, delta, A, B, C, cu_seqlens, D=None, z=None, delta_bias=None,
                    delta_softplus=True, h0=None, reverse=False, nthreads=1):
        """Packed sequences: x, delta, z are [dim][total], B, C [total][N]; sequence i is
        tokens cu_seqlens[i] .. cu_seqlens[i+1]-1 and starts from h0[i] (zeros when h0 is
        None). By definition each sequence is scanned on its own. Returns y [dim][total]
        and the final state of every sequence [nseq][dim][N]."""
        x = f64(x)
        dim, total = x.shape
        N = f64(A).shape[1]
        cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
        nseq = len(cu) - 1
        assert cu[0] == 0 and cu[-1] == total and all(a <= b for a, b in zip(cu, cu[1:]))
        dl, Bf, Cf = f64(delta), f64(B), f64(C)
        zf = None if z is None else f64(z)
        h0f = None if h0 is None else f64(h0)
        y = np.zeros((dim, total))
        hf = np.zeros((nseq, dim, N))
        fn = self.scan_reverse if reverse else self.scan
        for i in range(nseq):
            a, b = cu[i], cu[i + 1]
            start = None if h0f is None else h0f[i][None]
            if b == a:
                hf[i] = 0.0 if start is None else start[0]
                continue
            yi, hi = fn(x[None, :, a:b], dl[None, :, a:b], A, Bf[None, a:b], Cf[None, a:b], D=D,
                        z=None if zf is None else zf[None, :, a:b], delta_bias=delta_bias,
                        delta_softplus=delta_softplus, h0=start, nthreads=nthreads)
            y[:, a:b] = yi[0]
            hf[i] = hi[0]
        return y, hf

    # ---- causal depthwise convolution + SiLU (the step before the scan) ----
    @staticmethod
    def conv1d(x, weight, bias=None, state=None, silu=True):
        """Causal depthwise convolution of width K per channel, then SiLU:
            out[b,d,t] = silu(bias[d] + sum_{k<K} weight[d,k] * x[b,d,t-(K-1)+k])
        (the channel-wise Conv1d with groups = channels and the SiLU after it in the
        Mamba block: sivaro, "The Architecture in Practice"). Inputs before t = 0 come
        from `state` [b][d][K-1] (oldest first), zeros when None -- the left padding
        that keeps the layer causal and the output as long as the input.
        Returns (out [b][d][L], new state = the last K-1 inputs of [state, x])."""
        x = f64(x)
        w = f64(weight)
        b_, d_, L = x.shape
        K = w.shape[1]
        st = np.zeros((b_, d_, K - 1)) if state is None else f64(state)
        xp = np.concatenate([st, x], axis=2)            # xp[..., j] = x[..., j - (K-1)]
        acc = np.zeros((b_, d_, L))
        if bias is not None:
            acc += f64(bias)[None, :, None]
        for k in range(K):
            acc += w[None, :, k, None] * xp[:, :, k:k + L]
        out = acc / (1.0 + np.exp(-acc)) if silu else acc
        return out, np.ascontiguousarray(xp[:, :, L:])

    @staticmethod
    def conv1d_step(state, x, weight, bias=None, silu=True):
        """One decode token: state [b][d][K-1] holds the last K-1 inputs (oldest first),
        x [b][d]. Returns (out [b][d], state shifted by one with x appended)."""
        st = f64(state)
        x = f64(x)
        w = f64(weight)
        K = w.shape[1]
        window = np.concatenate([st, x[:, :, None]], axis=2)   # the last K inputs
        acc = np.zeros(x.shape)
        if bias is not None:
            acc += f64(bias)[None, :]
        for k in range(K):
            acc += w[None, :, k] * window[:, :, k]
        out = acc / (1.0 + np.exp(-acc)) if silu else acc
        return out, np.ascontiguousarray(window[:, :, 1:])

    # ---- decode step ----------------------------------------------------
    def step(self, state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
             delta_softplus=True):
        """One token for every (batch, channel): state [batch][dim][N] (fp64, updated
        and returned), x/delta/z [batch][dim], B/C [batch][N]. Returns (y, state)."""
        st = np.array(f64(state), dtype=np.float64, copy=True)
        b, d, N = st.shape
        rb = np.repeat(np.arange(b, dtype=np.int64), d)
        rd = np.tile(np.arange(d, dtype=np.int64), b)
        y = np.empty(b * d, dtype=np.float64)
        xs = f64(x).reshape(b * d)
        ds = f64(delta).reshape(b * d)
        zs = None if z is None else f64(z).reshape(b * d)
        rc = self._l.ssm_oracle_step_rows(
            b * d, N, _ptr_i(rb), _ptr_i(rd), _ptr(st), _ptr(xs), _ptr(ds), _ptr(zs),
            _ptr(f64(A)), _ptr(f64(B)), _ptr(f64(C)), _ptr(None if D is None else f64(D)),
            _ptr(None if delta_bias is None else f64(delta_bias)), int(bool(delta_softplus)),
            _ptr(y))
        if rc != 0:
            raise RuntimeError("ssm_oracle_step_rows failed")
        return y.reshape(b, d), st


def f64(a) -> np.ndarray:
    """Exact widening to a C-contiguous fp64 numpy array (torch bf16/fp32 tensors
    on any device, numpy arrays, Python sequences)."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu")
            if a.dtype in (torch.bfloat16, torch.float16):
                a = a.to(torch.float32)  # exact
            a = a.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _ptr_i(a):
    return a.ctypes.data_as(_ip)


def default() -> Oracle:
    return Oracle()

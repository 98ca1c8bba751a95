"""Pins for the fp64 oracle: each check ties the oracle to something other than
itself -- a closed form worked by hand, a library routine (numpy.cumsum,
numpy.convolve, numpy.fft, numpy.logaddexp), an O(L^2) brute force written
independently, or an exact invariant.

Every function takes an `oracle.Oracle` and raises AssertionError on a mismatch.
tests/test_oracle_pins.py runs them on the real oracle; tests/test_oracle_mutants.py
runs them on copies of the oracle with planted mistakes and requires each copy to
fail at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / den


def _rows(batch, dim):
    rb = np.repeat(np.arange(batch), dim)
    rd = np.tile(np.arange(dim), batch)
    return rb, rd


# ---------------------------------------------------------------------------
# P1: one token and two tokens worked by hand (closed forms).
# ---------------------------------------------------------------------------
def pin_hand_example(orc):
    """tests/golden/hand_two_tokens.json: N=2, A=(-1,-2), v = delta_raw + bias = 0
    so Delta = softplus(0) = ln 2 and exp(Delta*A) = (1/2, 1/4) exactly."""
    with open(os.path.join(GOLDEN, "hand_two_tokens.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    ln2 = math.log(2.0)
    e1 = math.exp(-1.0)
    # Closed forms derived in the fixture (evaluated here with math only).
    h1 = [0.5 + 2 * ln2, -0.25 + 4 * ln2]
    y1 = (2.75 + 2 * ln2) / (1 + e1)
    # token 2: x = 0, z = 2, same Delta -> h2 = (h1[0]/2, h1[1]/4)
    h2 = [h1[0] / 2, h1[1] / 4]
    s2 = -1.0 * h2[0] + 2.0 * h2[1]          # C_2 = (-1, 2), D*x = 0
    y2 = s2 * 2.0 / (1 + math.exp(-2.0))
    for got, want in zip(g["expected_decimal"]["h1"], h1):
        assert abs(got - want) < 1e-15 * max(1, abs(want)), (got, want)
    assert abs(g["expected_decimal"]["y1"] - y1) < 1e-15

    x = np.array([inp["x"]])
    dl = np.array([inp["delta_raw"]])
    z = np.array([inp["z"]])
    A = np.array([inp["A"]])
    B = np.array([inp["B"]])
    C = np.array([inp["C"]])
    y, hf = orc.scan_rows(x, dl, A, B, C, [0], [0], z_rows=z, D=[inp["D"]],
                          delta_bias=[inp["delta_bias"]], delta_softplus=True,
                          h0_rows=np.array([inp["h0"]]))
    assert abs(y[0, 0] - y1) <= 1e-14 * abs(y1), (y[0, 0], y1)
    assert abs(y[0, 1] - y2) <= 1e-14 * abs(y2), (y[0, 1], y2)
    assert _rel(hf[0], h2) < 1e-15, (hf[0], h2)
    # the same first token through the decode step
    yy, st = orc.step(np.array([[inp["h0"]]]), [[inp["x"][0]]], [[inp["delta_raw"][0]]], A,
                      [inp["B"][0]], [inp["C"][0]], D=[inp["D"]], z=[[inp["z"][0]]],
                      delta_bias=[inp["delta_bias"]], delta_softplus=True)
    assert abs(yy[0, 0] - y1) <= 1e-14 * abs(y1)
    assert _rel(st[0, 0], h1) < 1e-15


# ---------------------------------------------------------------------------
# P2: A = 0 -> exp(Delta*A) = 1, the state is a cumulative sum (numpy.cumsum).
# ---------------------------------------------------------------------------
def pin_cumsum(orc):
    rng = np.random.default_rng(11)
    batch, dim, L, N = 2, 3, 50, 4
    x = rng.integers(-3, 4, size=(batch, dim, L)).astype(np.float64)
    dr = rng.choice([0.25, 0.5, 1.0, 2.0], size=(batch, dim, L))
    bias = np.array([0.0, 0.5, -0.125])
    B = rng.integers(-2, 3, size=(batch, L, N)).astype(np.float64)
    C = rng.integers(-2, 3, size=(batch, L, N)).astype(np.float64)
    D = np.array([1.0, -2.0, 0.5])
    A = np.zeros((dim, N))
    y, hf = orc.scan(x, dr, A, B, C, D=D, delta_bias=bias, delta_softplus=False)
    delta = dr + bias[None, :, None]
    # contributions Delta_s * x_s * B_s[n], accumulated with the library cumsum
    contrib = (delta * x)[:, :, :, None] * B[:, None, :, :]
    h = np.cumsum(contrib, axis=2)
    y_ref = np.einsum("btn,bdtn->bdt", C, h) + D[None, :, None] * x
    assert np.array_equal(y, y_ref), _rel(y, y_ref)
    assert np.array_equal(hf, h[:, :, -1, :])


# ---------------------------------------------------------------------------
# P3: Delta, B, C constant -> the LTI SSM is a convolution (the S4 view).
# ---------------------------------------------------------------------------
def pin_lti_convolution(orc):
    rng = np.random.default_rng(12)
    dim, L, N = 2, 300, 6
    A = -rng.uniform(0.2, 3.0, size=(dim, N))
    delta_c = np.array([0.07, 0.31])          # constant step per channel (softplus off)
    Bc = rng.standard_normal(N)
    Cc = rng.standard_normal(N)
    D = np.array([0.5, -1.25])
    x = rng.standard_normal((1, dim, L))
    B = np.tile(Bc, (1, L, 1))
    C = np.tile(Cc, (1, L, 1))
    dr = np.zeros((1, dim, L))
    y, _ = orc.scan(x, dr, A, B, C, D=D, delta_bias=delta_c, delta_softplus=False)
    k = np.arange(L)
    for d in range(dim):
        dl = delta_c[d]
        # closed-form kernel K_k = sum_n C_n * Delta * B_n * exp(k * Delta * A_n)
        K = (Cc * dl * Bc)[None, :] * np.exp(k[:, None] * dl * A[d][None, :])
        K = K.sum(axis=1)
        ref = np.convolve(x[0, d], K)[:L] + D[d] * x[0, d]
        assert _rel(y[0, d], ref) < 1e-12, _rel(y[0, d], ref)
        # and once more through an FFT convolution
        nfft = 2 * L
        ref_fft = np.fft.irfft(np.fft.rfft(x[0, d], nfft) * np.fft.rfft(K, nfft), nfft)[:L]
        ref_fft += D[d] * x[0, d]
        assert _rel(y[0, d], ref_fft) < 1e-10


def pin_step_response(orc):
    """N = 1, A = -1, Delta = softplus(0) = ln 2 (so r = exp(-ln 2) = 1/2), B = C = 1,
    D = 0, x_t = 1: y_t = ln2 * sum_{k<=t} 2^-k = 2 ln2 (1 - 2^-(t+1))."""
    with open(os.path.join(GOLDEN, "lti_step_response.json")) as f:
        g = json.load(f)
    L = len(g["y"])
    y, _ = orc.scan(np.ones((1, 1, L)), np.zeros((1, 1, L)), [[-1.0]], np.ones((1, L, 1)),
                    np.ones((1, L, 1)), delta_softplus=True)
    ln2 = math.log(2.0)
    for t in range(L):
        want = 2 * ln2 * (1 - 2.0 ** -(t + 1))
        assert abs(g["y"][t] - want) < 1e-15
        assert abs(y[0, 0, t] - want) < 1e-14, (t, y[0, 0, t], want)


# ---------------------------------------------------------------------------
# P4: x = 0, h0 != 0 -> pure decay with time-varying Delta, closed form.
# ---------------------------------------------------------------------------
def pin_free_decay(orc):
    rng = np.random.default_rng(13)
    batch, dim, L, N = 2, 3, 64, 5
    A = -rng.uniform(0.1, 4.0, size=(dim, N))
    dr = rng.uniform(0.001, 0.2, size=(batch, dim, L))
    bias = np.array([0.0, 0.01, 0.03])
    h0 = rng.standard_normal((batch, dim, N))
    C = rng.standard_normal((batch, L, N))
    B = rng.standard_normal((batch, L, N))
    x = np.zeros((batch, dim, L))
    y, hf = orc.scan(x, dr, A, B, C, D=np.ones(dim), delta_bias=bias, delta_softplus=False,
                     h0=h0)
    S = np.cumsum(dr + bias[None, :, None], axis=2)            # sum_{s<=t} Delta_s
    h = np.exp(A[None, :, None, :] * S[..., None]) * h0[:, :, None, :]
    y_ref = np.einsum("btn,bdtn->bdt", C, h)
    assert _rel(hf, h[:, :, -1, :]) < 1e-13
    for b in range(batch):
        for d in range(dim):
            assert _rel(y[b, d], y_ref[b, d]) < 1e-12


# ---------------------------------------------------------------------------
# P5: brute force, the recurrence unrolled into its O(L^2) closed form.
# ---------------------------------------------------------------------------
def brute_force(x, dr, A, B, C, D, z, bias, softplus, h0):
    """y_t = [sum_{s<=t} sum_n C_t[n] exp(A_n sum_{u=s+1..t} Delta_u) Delta_s B_s[n] x_s
              + sum_n C_t[n] exp(A_n sum_{u<=t} Delta_u) h0[n] + D x_t] * silu(z_t).
    Written from the unrolled recurrence; softplus via numpy.logaddexp, silu via
    numpy exp -- no code shared with the oracle."""
    batch, dim, L = x.shape
    N = A.shape[1]
    v = dr + (0 if bias is None else bias[None, :, None])
    delta = np.logaddexp(0.0, v) if softplus else v
    y = np.zeros_like(x)
    hf = np.zeros((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            S = np.concatenate([[0.0], np.cumsum(delta[b, d])])    # S[k] = sum_{u<k} Delta_u
            hs = np.zeros(N)
            for t in range(L):
                # state after token t, summed term by term
                hs = np.zeros(N)
                for s in range(t + 1):
                    hs += (np.exp(A[d] * (S[t + 1] - S[s + 1])) * delta[b, d, s] * B[b, s]
                           * x[b, d, s])
                if h0 is not None:
                    hs += np.exp(A[d] * S[t + 1]) * h0[b, d]
                val = float(np.dot(C[b, t], hs))
                if D is not None:
                    val += D[d] * x[b, d, t]
                if z is not None:
                    zz = z[b, d, t]
                    val *= zz / (1.0 + np.exp(-zz))
                y[b, d, t] = val
            hf[b, d] = hs
    return y, hf


def pin_brute_force(orc):
    rng = np.random.default_rng(14)
    batch, dim, L, N = 2, 3, 40, 5
    A = -rng.uniform(0.1, 3.0, size=(dim, N))
    x = rng.standard_normal((batch, dim, L))
    dr = rng.normal(0, 0.5, size=(batch, dim, L))
    bias = rng.normal(-1.0, 0.5, size=dim)
    z = rng.standard_normal((batch, dim, L)) * 2
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    D = rng.standard_normal(dim)
    h0 = rng.standard_normal((batch, dim, N))
    for use_z, use_D, use_h0, sp in [(True, True, True, True), (False, False, False, True),
                                     (True, False, True, False)]:
        dr_ = dr if sp else np.abs(dr) * 0.2
        args = dict(D=D if use_D else None, z=z if use_z else None, delta_bias=bias if sp else None,
                    delta_softplus=sp, h0=h0 if use_h0 else None)
        y, hf = orc.scan(x, dr_, A, B, C, **args)
        y_ref, hf_ref = brute_force(x, dr_, A, B, C, args["D"], args["z"], args["delta_bias"],
                                    sp, args["h0"])
        for b in range(batch):
            for d in range(dim):
                assert _rel(y[b, d], y_ref[b, d]) < 1e-11, (b, d, _rel(y[b, d], y_ref[b, d]))
        assert _rel(hf, hf_ref) < 1e-11


# ---------------------------------------------------------------------------
# P6 / P7 / P8: invariants (bitwise in fp64: same operations in the same order).
# ---------------------------------------------------------------------------
def _rand_problem(seed, batch=2, dim=3, L=97, N=16):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((batch, dim, L)),
        delta=rng.normal(0, 0.1, size=(batch, dim, L)),
        A=-np.tile(np.arange(1.0, N + 1), (dim, 1)) * rng.uniform(0.5, 1.5, size=(dim, 1)),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        D=rng.standard_normal(dim),
        z=rng.standard_normal((batch, dim, L)),
        delta_bias=rng.uniform(-6.9, -2.3, size=dim),
    )


def pin_chunked_equals_unchunked(orc):
    p = _rand_problem(15)
    L = p["x"].shape[2]
    y, hf = orc.scan(**p)
    for L1 in (1, 37, 64, 96):
        a = {k: (v[:, :, :L1] if k in ("x", "delta", "z") else v[:, :L1] if k in ("B", "C") else v)
             for k, v in p.items()}
        b_ = {k: (v[:, :, L1:] if k in ("x", "delta", "z") else v[:, L1:] if k in ("B", "C") else v)
              for k, v in p.items()}
        y1, h1 = orc.scan(**a)
        y2, h2 = orc.scan(**b_, h0=h1)
        assert np.array_equal(np.concatenate([y1, y2], axis=2), y), L1
        assert np.array_equal(h2, hf), L1


def pin_decode_equals_scan(orc):
    rng = np.random.default_rng(16)
    batch, dim, L, N = 3, 2, 10, 16           # batch >= dim on purpose
    p = _rand_problem(16, batch=batch, dim=dim, L=L, N=N)
    S = rng.standard_normal((batch, dim, N))
    y, hf = orc.scan(**p, h0=S)
    st = S.copy()
    for t in range(L):
        yt, st = orc.step(st, p["x"][:, :, t], p["delta"][:, :, t], p["A"], p["B"][:, t],
                          p["C"][:, t], D=p["D"], z=p["z"][:, :, t], delta_bias=p["delta_bias"])
        assert np.array_equal(yt, y[:, :, t]), t
    assert np.array_equal(st, hf)


def pin_linearity_and_causality(orc):
    p = _rand_problem(17)
    p.pop("z")
    rng = np.random.default_rng(17)
    h0 = rng.standard_normal((2, 3, 16))
    y, hf = orc.scan(**p, h0=h0)
    q = dict(p)
    q["x"] = p["x"] * 8.0
    y8, hf8 = orc.scan(**q, h0=h0 * 8.0)
    assert np.array_equal(y8, y * 8.0) and np.array_equal(hf8, hf * 8.0)
    # causality: a change at t0 leaves every earlier output bit-identical
    t0 = 50
    q = dict(p)
    q["x"] = p["x"].copy()
    q["x"][:, :, t0] += 1.0
    yc, _ = orc.scan(**q, h0=h0)
    assert np.array_equal(yc[:, :, :t0], y[:, :, :t0])
    assert not np.array_equal(yc[:, :, t0], y[:, :, t0])


# ---------------------------------------------------------------------------
# P10: the element-wise functions.
# ---------------------------------------------------------------------------
def pin_elementwise(orc):
    assert orc.softplus(0.0) == math.log(2.0)
    assert orc.silu(0.0) == 0.0
    vs = np.concatenate([np.linspace(-40, 40, 161), [-700.0, -1e-9, 1e-9, 700.0]])
    for v in vs:
        sp = orc.softplus(v)
        assert abs(sp - np.logaddexp(0.0, v)) <= 4e-16 * max(1.0, abs(sp)), v
        assert abs((orc.softplus(v) - orc.softplus(-v)) - v) <= 1e-14 * max(1.0, abs(v)), v
        s = orc.silu(v)
        ref = v * 0.5 * (1.0 + math.tanh(0.5 * v))   # sigma(v) = (1 + tanh(v/2)) / 2
        assert abs(s - ref) <= 1e-15 * max(1.0, abs(v)), (v, s, ref)
        assert abs((orc.silu(v) - orc.silu(-v)) - v) <= 1e-14 * max(1.0, abs(v)), v


# ---------------------------------------------------------------------------
# P11: the anti-causal (reverse-time) scan.
# ---------------------------------------------------------------------------
def pin_reverse_lti_convolution(orc):
    """Delta, B, C constant: the reverse scan is the anti-causal convolution
    y_t = sum_{s>=t} K_{s-t} x_s + D x_t, i.e. numpy.convolve on the reversed input."""
    rng = np.random.default_rng(31)
    dim, L, N = 2, 257, 6
    A = -rng.uniform(0.2, 3.0, size=(dim, N))
    delta_c = np.array([0.11, 0.43])
    Bc = rng.standard_normal(N)
    Cc = rng.standard_normal(N)
    D = np.array([-0.75, 2.0])
    x = rng.standard_normal((1, dim, L))
    y, _ = orc.scan_reverse(x, np.zeros((1, dim, L)), A, np.tile(Bc, (1, L, 1)),
                            np.tile(Cc, (1, L, 1)), D=D, delta_bias=delta_c,
                            delta_softplus=False)
    k = np.arange(L)
    for d in range(dim):
        dl = delta_c[d]
        K = ((Cc * dl * Bc)[None, :] * np.exp(k[:, None] * dl * A[d][None, :])).sum(axis=1)
        ref = np.convolve(x[0, d][::-1], K)[:L][::-1] + D[d] * x[0, d]
        assert _rel(y[0, d], ref) < 1e-12, _rel(y[0, d], ref)
        # y_t must not depend on x_s for s < t: the last output sees only the last input
        assert abs(y[0, d, -1] - (K[0] + D[d]) * x[0, d, -1]) < 1e-12 * max(1, abs(y[0, d, -1]))


def brute_force_reverse(x, dr, A, B, C, D, z, bias, softplus, h0):
    """Reverse recurrence h_t = exp(Delta_t A) h_{t+1} + Delta_t B_t x_t, h_L = h0,
    unrolled: with R_k = sum_{u>=k} Delta_u,
    h_t = sum_{s>=t} exp(A (R_t - R_s)) Delta_s B_s x_s + exp(A R_t) h0,
    y_t = (C_t . h_t + D x_t) silu(z_t); the final state is h_0."""
    batch, dim, L = x.shape
    N = A.shape[1]
    v = dr + (0 if bias is None else bias[None, :, None])
    delta = np.logaddexp(0.0, v) if softplus else v
    y = np.zeros_like(x)
    hf = np.zeros((batch, dim, N))
    for b in range(batch):
        for d in range(dim):
            R = np.concatenate([np.cumsum(delta[b, d][::-1])[::-1], [0.0]])
            for t in range(L):
                hs = np.zeros(N)
                for s in range(t, L):
                    hs += np.exp(A[d] * (R[t] - R[s])) * delta[b, d, s] * B[b, s] * x[b, d, s]
                if h0 is not None:
                    hs += np.exp(A[d] * R[t]) * h0[b, d]
                val = float(np.dot(C[b, t], hs))
                if D is not None:
                    val += D[d] * x[b, d, t]
                if z is not None:
                    zz = z[b, d, t]
                    val *= zz / (1.0 + np.exp(-zz))
                y[b, d, t] = val
                if t == 0:
                    hf[b, d] = hs
    return y, hf


def pin_reverse_brute_force(orc):
    rng = np.random.default_rng(32)
    batch, dim, L, N = 2, 2, 33, 4
    A = -rng.uniform(0.1, 3.0, size=(dim, N))
    x = rng.standard_normal((batch, dim, L))
    dr = rng.normal(0, 0.5, size=(batch, dim, L))
    bias = rng.normal(-1.0, 0.5, size=dim)
    z = rng.standard_normal((batch, dim, L)) * 2
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    D = rng.standard_normal(dim)
    h0 = rng.standard_normal((batch, dim, N))
    for use_z, use_h0 in [(True, True), (False, False)]:
        zz = z if use_z else None
        hh = h0 if use_h0 else None
        y, hf = orc.scan_reverse(x, dr, A, B, C, D=D, z=zz, delta_bias=bias, h0=hh)
        y_ref, hf_ref = brute_force_reverse(x, dr, A, B, C, D, zz, bias, True, hh)
        for b in range(batch):
            for d in range(dim):
                assert _rel(y[b, d], y_ref[b, d]) < 1e-11, (b, d)
        assert _rel(hf, hf_ref) < 1e-11


# ---------------------------------------------------------------------------
# P12: packed (variable-length) sequences.
# ---------------------------------------------------------------------------
def _packed_problem(seed, lens, dim=3, N=5):
    rng = np.random.default_rng(seed)
    total = int(sum(lens))
    return dict(
        x=rng.standard_normal((dim, total)),
        delta=rng.normal(0, 0.5, size=(dim, total)),
        A=-rng.uniform(0.1, 3.0, size=(dim, N)),
        B=rng.standard_normal((total, N)),
        C=rng.standard_normal((total, N)),
        D=rng.standard_normal(dim),
        z=rng.standard_normal((dim, total)),
        delta_bias=rng.normal(-1.0, 0.5, size=dim),
    ), np.concatenate([[0], np.cumsum(lens)]).astype(np.int64), rng.standard_normal(
        (len(lens), dim, N))


def pin_varlen_brute_force(orc):
    """Ragged lengths with empty and one-token sequences: each sequence against the
    brute-force closed forms (forward and reverse), starting from its own h0; an
    empty sequence's final state is its h0."""
    lens = [5, 0, 1, 17, 0, 0, 9, 2]
    p, cu, h0 = _packed_problem(33, lens)
    for reverse, bf in [(False, brute_force), (True, brute_force_reverse)]:
        y, hf = orc.scan_varlen(cu_seqlens=cu, h0=h0, reverse=reverse, **p)
        for i in range(len(lens)):
            a, b = int(cu[i]), int(cu[i + 1])
            if a == b:
                assert np.array_equal(hf[i], h0[i])
                continue
            yr, hr = bf(p["x"][None, :, a:b], p["delta"][None, :, a:b], p["A"],
                        p["B"][None, a:b], p["C"][None, a:b], p["D"], p["z"][None, :, a:b],
                        p["delta_bias"], True, h0[i][None])
            assert _rel(y[:, a:b], yr[0]) < 1e-11, (reverse, i)
            assert _rel(hf[i], hr[0]) < 1e-11, (reverse, i)


def pin_varlen_equals_batched(orc):
    """Equal lengths: packing is a relayout of a batch ([dim][b*L] <-> [b][dim][L])."""
    batch, L = 3, 21
    p, cu, h0 = _packed_problem(34, [L] * batch)
    dim = p["x"].shape[0]
    bt = {k: (v.reshape(dim, batch, L).transpose(1, 0, 2) if k in ("x", "delta", "z")
              else v.reshape(batch, L, -1) if k in ("B", "C") else v) for k, v in p.items()}
    for reverse in (False, True):
        fn = orc.scan_reverse if reverse else orc.scan
        yb, hb = fn(h0=h0, **bt)
        y, hf = orc.scan_varlen(cu_seqlens=cu, h0=h0, reverse=reverse, **p)
        assert np.array_equal(y, yb.transpose(1, 0, 2).reshape(dim, batch * L))
        assert np.array_equal(hf, hb)


def pin_varlen_isolation(orc):
    """Nothing crosses a boundary: changing one sequence's inputs changes its own
    outputs and leaves every other sequence's outputs bit-identical."""
    lens = [7, 12, 1, 9]
    p, cu, _ = _packed_problem(35, lens)
    for reverse in (False, True):
        y, hf = orc.scan_varlen(cu_seqlens=cu, reverse=reverse, **p)
        q = {k: v.copy() for k, v in p.items()}
        a, b = int(cu[1]), int(cu[2])
        q["x"][:, a:b] += 1.0
        q["B"][a:b] *= -1.0
        y2, hf2 = orc.scan_varlen(cu_seqlens=cu, reverse=reverse, **q)
        assert np.array_equal(y2[:, :a], y[:, :a]) and np.array_equal(y2[:, b:], y[:, b:])
        assert not np.array_equal(y2[:, a:b], y[:, a:b])
        assert np.array_equal(hf2[[0, 2, 3]], hf[[0, 2, 3]])
        assert not np.array_equal(hf2[1], hf[1])


# ---------------------------------------------------------------------------
# P13: the causal depthwise convolution + SiLU in front of the scan.
# ---------------------------------------------------------------------------
def _conv_problem(seed, batch=2, dim=3, L=40, K=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((batch, dim, L)), rng.standard_normal((dim, K)) * 0.5,
            rng.standard_normal(dim) * 0.3, rng.standard_normal((batch, dim, K - 1)))


def pin_conv_library(orc):
    """torch.nn.functional.conv1d (fp64, CPU) with groups = channels and K-1 zeros of
    padding on both sides, keeping the first L outputs, then torch's SiLU; and with a
    state, the same conv over [state, x] without padding."""
    import torch
    import torch.nn.functional as F
    x, w, b, st = _conv_problem(41)
    dim, K = w.shape
    tw = torch.tensor(w)[:, None, :]
    ref = F.conv1d(torch.tensor(x), tw, torch.tensor(b), padding=K - 1, groups=dim)
    ref = F.silu(ref[..., :x.shape[2]]).numpy()
    y, _ = orc.conv1d(x, w, b)
    assert _rel(y, ref) < 1e-14, _rel(y, ref)
    ref = F.silu(F.conv1d(torch.tensor(np.concatenate([st, x], axis=2)), tw, torch.tensor(b),
                          groups=dim)).numpy()
    y, _ = orc.conv1d(x, w, b, state=st)
    assert _rel(y, ref) < 1e-14


def pin_conv_np_convolve(orc):
    """Without SiLU and bias, each row is numpy.convolve with the reversed taps (Conv1d
    is a cross-correlation), truncated to the causal part."""
    x, w, _, _ = _conv_problem(42, batch=1, dim=2, L=33)
    y, _ = orc.conv1d(x, w, None, silu=False)
    for d in range(2):
        ref = np.convolve(x[0, d], w[d][::-1])[:33]
        assert _rel(y[0, d], ref) < 1e-14


def pin_conv_impulse(orc):
    """A unit impulse at t0: the pre-activation is bias + weight[K-1-(t-t0)] for
    0 <= t - t0 < K and bias elsewhere (the newest input meets the last tap)."""
    dim, L, K, t0 = 2, 12, 4, 5
    w = np.array([[1.0, 2.0, 3.0, 4.0], [-0.5, 0.25, -2.0, 8.0]])
    b = np.array([0.125, -1.0])
    x = np.zeros((1, dim, L))
    x[0, :, t0] = 1.0
    y, st = orc.conv1d(x, w, b, silu=False)
    for d in range(dim):
        for t in range(L):
            want = b[d] + (w[d, K - 1 - (t - t0)] if 0 <= t - t0 < K else 0.0)
            assert y[0, d, t] == want, (d, t, y[0, d, t], want)
    assert np.array_equal(st[0], np.zeros((dim, K - 1)))


def pin_conv_state_continuation(orc):
    """Splitting a sequence and carrying the state gives the same bits; a sequence
    shorter than K-1 keeps the tail of the old state."""
    x, w, b, st = _conv_problem(43, L=29)
    y, s_end = orc.conv1d(x, w, b, state=st)
    for cut in (1, 2, 3, 17):
        y1, s1 = orc.conv1d(x[:, :, :cut], w, b, state=st)
        y2, s2 = orc.conv1d(x[:, :, cut:], w, b, state=s1)
        assert np.array_equal(np.concatenate([y1, y2], axis=2), y), cut
        assert np.array_equal(s2, s_end), cut
    _, s1 = orc.conv1d(x[:, :, :1], w, b, state=st)
    assert np.array_equal(s1, np.concatenate([st[:, :, 1:], x[:, :, :1]], axis=2))


def pin_conv_decode_equals_prefill(orc):
    x, w, b, st = _conv_problem(44, L=9)
    y, s_end = orc.conv1d(x, w, b, state=st)
    s = st
    for t in range(x.shape[2]):
        yt, s = orc.conv1d_step(s, x[:, :, t], w, b)
        assert np.array_equal(yt, y[:, :, t]), t
    assert np.array_equal(s, s_end)


# ---------------------------------------------------------------------------
# P14: gradients (the backward scan).
# ---------------------------------------------------------------------------
def _bwd_problem(seed, batch=2, dim=3, L=23, N=4):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((batch, dim, L)),
        delta=rng.normal(0, 0.5, size=(batch, dim, L)),
        A=-rng.uniform(0.1, 2.0, size=(dim, N)),
        B=rng.standard_normal((batch, L, N)),
        C=rng.standard_normal((batch, L, N)),
        D=rng.standard_normal(dim),
        z=rng.standard_normal((batch, dim, L)),
        delta_bias=rng.normal(-0.5, 0.5, size=dim),
        h0=rng.standard_normal((batch, dim, N)),
    ), rng.standard_normal((batch, dim, L)), rng.standard_normal((batch, dim, N))


def _torch_forward(x, delta, A, B, C, D, z, delta_bias, softplus, h0):
    """The forward written a second time, in torch fp64 ops (softplus as logaddexp,
    silu as torch's), so that torch.autograd can differentiate it."""
    import torch
    import torch.nn.functional as F
    b, d, L = x.shape
    v = delta + (0 if delta_bias is None else delta_bias[None, :, None])
    dl = torch.logaddexp(v, torch.zeros_like(v)) if softplus else v
    h = h0 if h0 is not None else torch.zeros((b, d, A.shape[1]), dtype=x.dtype)
    ys = []
    for t in range(L):
        h = torch.exp(dl[:, :, t, None] * A[None]) * h + \
            (dl[:, :, t] * x[:, :, t])[..., None] * B[:, None, t, :]
        s = (C[:, None, t, :] * h).sum(-1)
        if D is not None:
            s = s + D[None, :] * x[:, :, t]
        if z is not None:
            s = s * F.silu(z[:, :, t])
        ys.append(s)
    return torch.stack(ys, dim=-1), h


def pin_bwd_autograd(orc):
    """Every gradient against torch.autograd of the torch forward, with and without
    the gate, skip, bias, softplus, initial and final states."""
    import torch
    p, dy, dhf = _bwd_problem(51)
    for use_z, use_D, sp, use_h, use_dhf in [(True, True, True, True, True),
                                             (False, False, True, False, False),
                                             (True, False, False, True, False)]:
        q = dict(p)
        if not sp:
            q["delta"] = np.abs(p["delta"]) * 0.3
            q["delta_bias"] = None
        names = ["x", "delta", "A", "B", "C"] + (["D"] if use_D else []) + \
                (["z"] if use_z else []) + (["delta_bias"] if sp else []) + \
                (["h0"] if use_h else [])
        tt = {k: torch.tensor(q[k], requires_grad=True) for k in names}
        y, hf = _torch_forward(tt["x"], tt["delta"], tt["A"], tt["B"], tt["C"], tt.get("D"),
                               tt.get("z"), tt.get("delta_bias"), sp, tt.get("h0"))
        loss = (y * torch.tensor(dy)).sum()
        if use_dhf:
            loss = loss + (hf * torch.tensor(dhf)).sum()
        loss.backward()
        g = orc.scan_bwd(q["x"], q["delta"], q["A"], q["B"], q["C"], dy,
                         D=q["D"] if use_D else None, z=q["z"] if use_z else None,
                         delta_bias=q["delta_bias"] if sp else None, delta_softplus=sp,
                         h0=q["h0"] if use_h else None, dh_final=dhf if use_dhf else None)
        pairs = [("dx", "x"), ("ddelta", "delta"), ("dA", "A"), ("dB", "B"), ("dC", "C")]
        pairs += [("dD", "D")] if use_D else []
        pairs += [("dz", "z")] if use_z else []
        pairs += [("dbias", "delta_bias")] if sp else []
        pairs += [("dh0", "h0")] if use_h else []
        for gk, tk in pairs:
            ref = tt[tk].grad.numpy()
            assert _rel(g[gk], ref) < 1e-11, (gk, _rel(g[gk], ref))


def pin_bwd_finite_differences(orc):
    """Directional derivatives of the (pinned) forward oracle by central differences:
    sum(grad * V) against (loss(P + eps V) - loss(P - eps V)) / (2 eps) for a random
    direction V of every input P."""
    p, dy, dhf = _bwd_problem(52, batch=2, dim=2, L=17, N=3)
    rng = np.random.default_rng(53)

    def loss(q):
        y, hf = orc.scan(q["x"], q["delta"], q["A"], q["B"], q["C"], D=q["D"], z=q["z"],
                         delta_bias=q["delta_bias"], h0=q["h0"])
        return float(np.sum(y * dy) + np.sum(hf * dhf))

    g = orc.scan_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dy, D=p["D"], z=p["z"],
                     delta_bias=p["delta_bias"], h0=p["h0"], dh_final=dhf)
    for gk, pk in [("dx", "x"), ("ddelta", "delta"), ("dz", "z"), ("dA", "A"), ("dB", "B"),
                   ("dC", "C"), ("dD", "D"), ("dbias", "delta_bias"), ("dh0", "h0")]:
        V = rng.standard_normal(p[pk].shape)
        eps = 1e-6
        qp = dict(p)
        qm = dict(p)
        qp[pk] = p[pk] + eps * V
        qm[pk] = p[pk] - eps * V
        fd = (loss(qp) - loss(qm)) / (2 * eps)
        an = float(np.sum(g[gk] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gk, fd, an)


def pin_bwd_cumsum_closed_form(orc):
    """A = 0, constant Delta, no gate: h_t = Delta sum_{s<=t} x_s B_s, so with
    R_s = sum_{t>=s} dy_t C_t (numpy reverse cumsum): dx_s = D dy_s + Delta B_s . R_s,
    dB_s = sum_d Delta x_s R_s, dC_t = sum_d dy_t h_t, dA = sum_t Delta R_t h_{t-1}."""
    rng = np.random.default_rng(54)
    b, d, L, N = 2, 3, 19, 4
    x = rng.standard_normal((b, d, L))
    dl = np.array([0.3, 0.7, 1.1])
    B = rng.standard_normal((b, L, N))
    C = rng.standard_normal((b, L, N))
    D = rng.standard_normal(d)
    dy = rng.standard_normal((b, d, L))
    g = orc.scan_bwd(x, np.zeros((b, d, L)), np.zeros((d, N)), B, C, dy, D=D, delta_bias=dl,
                     delta_softplus=False)
    R = np.cumsum((dy[..., None] * C[:, None])[:, :, ::-1], axis=2)[:, :, ::-1]  # [b,d,L,N]
    h = np.cumsum(dl[None, :, None, None] * x[..., None] * B[:, None], axis=2)     # h_t
    hprev = np.concatenate([np.zeros((b, d, 1, N)), h[:, :, :-1]], axis=2)
    dx = D[None, :, None] * dy + dl[None, :, None] * np.einsum("bln,bdln->bdl", B, R)
    dB = np.einsum("bdl,bdln->bln", dl[None, :, None] * x, R)
    dC = np.einsum("bdl,bdln->bln", dy, h)
    dA = np.einsum("bdln,bdln->dn", R, hprev) * dl[:, None]
    assert _rel(g["dx"], dx) < 1e-12 and _rel(g["dB"], dB) < 1e-12
    assert _rel(g["dC"], dC) < 1e-12 and _rel(g["dA"], dA) < 1e-12
    assert _rel(g["dD"], np.einsum("bdl,bdl->d", dy, x)) < 1e-12


def pin_varlen_bwd_autograd(orc):
    """Packed gradients against torch.autograd of the packed forward written again in
    torch ops (each sequence through the torch forward from its own h0; an empty
    sequence's final state is its h0), loss sum(dy y) + sum(dh_final h_final); ragged
    lengths with empty and one-token sequences."""
    import torch
    lens = [6, 0, 1, 11, 0, 4]
    p, cu, h0 = _packed_problem(61, lens, dim=3, N=4)
    rng = np.random.default_rng(62)
    dim, total = p["x"].shape
    dy = rng.standard_normal((dim, total))
    dhf = rng.standard_normal((len(lens), dim, 4))
    names = ["x", "delta", "A", "B", "C", "D", "z", "delta_bias"]
    tt = {k: torch.tensor(p[k], requires_grad=True) for k in names}
    th0 = torch.tensor(h0, requires_grad=True)
    ys, hfs = [], []
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            hfs.append(th0[i])
            continue
        y, hf = _torch_forward(tt["x"][None, :, a:b], tt["delta"][None, :, a:b], tt["A"],
                               tt["B"][None, a:b], tt["C"][None, a:b], tt["D"],
                               tt["z"][None, :, a:b], tt["delta_bias"], True, th0[i][None])
        ys.append(y[0])
        hfs.append(hf[0])
    loss = (torch.cat(ys, dim=1) * torch.tensor(dy)).sum() + \
        (torch.stack(hfs) * torch.tensor(dhf)).sum()
    loss.backward()
    g = orc.scan_varlen_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dy, cu, D=p["D"],
                            z=p["z"], delta_bias=p["delta_bias"], h0=h0, dh_final=dhf)
    for gk, tk in [("dx", "x"), ("ddelta", "delta"), ("dA", "A"), ("dB", "B"), ("dC", "C"),
                   ("dD", "D"), ("dz", "z"), ("dbias", "delta_bias")]:
        assert _rel(g[gk], tt[tk].grad.numpy()) < 1e-11, gk
    assert _rel(g["dh0"], th0.grad.numpy()) < 1e-11


def pin_varlen_reverse_bwd_autograd(orc):
    """Packed gradients of the anti-causal scan against torch.autograd of the packed
    anti-causal forward written in torch ops (each sequence through the direct
    anti-causal torch forward from its own h0), with empty and one-token sequences."""
    import torch
    lens = [5, 0, 1, 9, 0, 3]
    p, cu, h0 = _packed_problem(65, lens, dim=3, N=4)
    rng = np.random.default_rng(66)
    dim, total = p["x"].shape
    dy = rng.standard_normal((dim, total))
    dhf = rng.standard_normal((len(lens), dim, 4))
    names = ["x", "delta", "A", "B", "C", "D", "z", "delta_bias"]
    tt = {k: torch.tensor(p[k], requires_grad=True) for k in names}
    th0 = torch.tensor(h0, requires_grad=True)
    ys, hfs = [], []
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            hfs.append(th0[i])
            continue
        y, hf = _torch_forward_reverse(tt["x"][None, :, a:b], tt["delta"][None, :, a:b],
                                       tt["A"], tt["B"][None, a:b], tt["C"][None, a:b],
                                       tt["D"], tt["z"][None, :, a:b], tt["delta_bias"], True,
                                       th0[i][None])
        ys.append(y[0])
        hfs.append(hf[0])
    loss = (torch.cat(ys, dim=1) * torch.tensor(dy)).sum() + \
        (torch.stack(hfs) * torch.tensor(dhf)).sum()
    loss.backward()
    g = orc.scan_varlen_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dy, cu, D=p["D"],
                            z=p["z"], delta_bias=p["delta_bias"], h0=h0, dh_final=dhf,
                            reverse=True)
    for gk, tk in [("dx", "x"), ("ddelta", "delta"), ("dA", "A"), ("dB", "B"), ("dC", "C"),
                   ("dD", "D"), ("dz", "z"), ("dbias", "delta_bias")]:
        assert _rel(g[gk], tt[tk].grad.numpy()) < 1e-11, gk
    assert _rel(g["dh0"], th0.grad.numpy()) < 1e-11


def pin_varlen_bwd_equals_batched(orc):
    """Equal lengths: the packed gradients are the batch gradients, relayouted."""
    batch, L = 3, 13
    p, cu, h0 = _packed_problem(63, [L] * batch, dim=2, N=3)
    dim = p["x"].shape[0]
    rng = np.random.default_rng(64)
    dy = rng.standard_normal((dim, batch * L))
    dhf = rng.standard_normal((batch, dim, 3))
    tob = lambda v: v.reshape(dim, batch, L).transpose(1, 0, 2)
    gb = orc.scan_bwd(tob(p["x"]), tob(p["delta"]), p["A"], p["B"].reshape(batch, L, -1),
                      p["C"].reshape(batch, L, -1), tob(dy), D=p["D"], z=tob(p["z"]),
                      delta_bias=p["delta_bias"], h0=h0, dh_final=dhf)
    g = orc.scan_varlen_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dy, cu, D=p["D"],
                            z=p["z"], delta_bias=p["delta_bias"], h0=h0, dh_final=dhf)
    for k in ("dx", "ddelta", "dz"):
        assert np.array_equal(g[k], gb[k].transpose(1, 0, 2).reshape(dim, batch * L)), k
    for k in ("dB", "dC"):
        assert np.array_equal(g[k], gb[k].reshape(batch * L, -1)), k
    assert np.array_equal(g["dh0"], gb["dh0"])
    for k in ("dA", "dD", "dbias"):   # sums over batch rows in another order
        assert _rel(g[k], gb[k]) < 1e-13, k


def _torch_forward_reverse(x, delta, A, B, C, D, z, delta_bias, softplus, h0):
    """The anti-causal scan written directly in torch fp64 ops: the state runs from
    h_L = h0 down the tokens, h_t = exp(Delta_t A) h_{t+1} + Delta_t x_t B_t, and y_t is
    read from h_t (no reversal of arrays anywhere)."""
    import torch
    import torch.nn.functional as F
    b, d, L = x.shape
    v = delta + (0 if delta_bias is None else delta_bias[None, :, None])
    dl = torch.logaddexp(v, torch.zeros_like(v)) if softplus else v
    h = h0 if h0 is not None else torch.zeros((b, d, A.shape[1]), dtype=x.dtype)
    ys = [None] * L
    for t in range(L - 1, -1, -1):
        h = torch.exp(dl[:, :, t, None] * A[None]) * h + \
            (dl[:, :, t] * x[:, :, t])[..., None] * B[:, None, t, :]
        s = (C[:, None, t, :] * h).sum(-1)
        if D is not None:
            s = s + D[None, :] * x[:, :, t]
        if z is not None:
            s = s * F.silu(z[:, :, t])
        ys[t] = s
    return torch.stack(ys, dim=-1), h


def pin_reverse_bwd_autograd(orc):
    """Gradients through the anti-causal scan against torch.autograd of the anti-causal
    forward written directly in torch (loss sum(dy y) + sum(dh_final h_final)), with
    and without gate, skip, softplus, h0 and dh_final."""
    import torch
    p, dy, dhf = _bwd_problem(71, L=21)
    for use_z, use_D, sp, use_h, use_dhf in [(True, True, True, True, True),
                                             (False, False, False, False, True),
                                             (True, False, True, True, False)]:
        q = dict(p)
        if not sp:
            q["delta"] = np.abs(p["delta"]) * 0.3
            q["delta_bias"] = None
        names = ["x", "delta", "A", "B", "C"] + (["D"] if use_D else []) + \
                (["z"] if use_z else []) + (["delta_bias"] if sp else []) + \
                (["h0"] if use_h else [])
        tt = {k: torch.tensor(q[k], requires_grad=True) for k in names}
        y, hf = _torch_forward_reverse(tt["x"], tt["delta"], tt["A"], tt["B"], tt["C"],
                                       tt.get("D"), tt.get("z"), tt.get("delta_bias"), sp,
                                       tt.get("h0"))
        loss = (y * torch.tensor(dy)).sum()
        if use_dhf:
            loss = loss + (hf * torch.tensor(dhf)).sum()
        loss.backward()
        g = orc.scan_reverse_bwd(q["x"], q["delta"], q["A"], q["B"], q["C"], dy,
                                 D=q["D"] if use_D else None, z=q["z"] if use_z else None,
                                 delta_bias=q["delta_bias"] if sp else None,
                                 delta_softplus=sp, h0=q["h0"] if use_h else None,
                                 dh_final=dhf if use_dhf else None)
        pairs = [("dx", "x"), ("ddelta", "delta"), ("dA", "A"), ("dB", "B"), ("dC", "C")]
        pairs += [("dD", "D")] if use_D else []
        pairs += [("dz", "z")] if use_z else []
        pairs += [("dbias", "delta_bias")] if sp else []
        pairs += [("dh0", "h0")] if use_h else []
        for gk, tk in pairs:
            assert _rel(g[gk], tt[tk].grad.numpy()) < 1e-11, (gk, _rel(g[gk], tt[tk].grad.numpy()))


def pin_reverse_bwd_finite_differences(orc):
    """Directional derivatives of the (pinned) anti-causal forward oracle by central
    differences, for every input, against the reverse gradients."""
    p, dy, dhf = _bwd_problem(72, batch=2, dim=2, L=15, N=3)
    rng = np.random.default_rng(73)

    def loss(q):
        y, hf = orc.scan_reverse(q["x"], q["delta"], q["A"], q["B"], q["C"], D=q["D"],
                                 z=q["z"], delta_bias=q["delta_bias"], h0=q["h0"])
        return float(np.sum(y * dy) + np.sum(hf * dhf))

    g = orc.scan_reverse_bwd(p["x"], p["delta"], p["A"], p["B"], p["C"], dy, D=p["D"],
                             z=p["z"], delta_bias=p["delta_bias"], h0=p["h0"], dh_final=dhf)
    for gk, pk in [("dx", "x"), ("ddelta", "delta"), ("dz", "z"), ("dA", "A"), ("dB", "B"),
                   ("dC", "C"), ("dD", "D"), ("dbias", "delta_bias"), ("dh0", "h0")]:
        V = rng.standard_normal(p[pk].shape)
        eps = 1e-6
        qp = dict(p)
        qm = dict(p)
        qp[pk] = p[pk] + eps * V
        qm[pk] = p[pk] - eps * V
        fd = (loss(qp) - loss(qm)) / (2 * eps)
        an = float(np.sum(g[gk] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gk, fd, an)


ALL_PINS = [pin_hand_example, pin_cumsum, pin_lti_convolution, pin_step_response,
            pin_free_decay, pin_brute_force, pin_chunked_equals_unchunked,
            pin_decode_equals_scan, pin_linearity_and_causality, pin_elementwise,
            pin_reverse_lti_convolution, pin_reverse_brute_force, pin_varlen_brute_force,
            pin_varlen_equals_batched, pin_varlen_isolation, pin_conv_library,
            pin_conv_np_convolve, pin_conv_impulse, pin_conv_state_continuation,
            pin_conv_decode_equals_prefill, pin_bwd_autograd, pin_bwd_finite_differences,
            pin_bwd_cumsum_closed_form, pin_varlen_bwd_autograd, pin_varlen_bwd_equals_batched,
            pin_reverse_bwd_autograd, pin_reverse_bwd_finite_differences,
            pin_varlen_reverse_bwd_autograd]

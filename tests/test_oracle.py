"""Pins for the float64 oracle: closed forms, library routines, invariants, brute force.

Each pin_* function checks the oracle against something other than itself:
  - library routines computing the same special case (torch silu / linear /
    conv1d, and torch.autograd deriving the update from its loss);
  - closed forms of special cases (eta = 0 gives the ordinary gated MLP of the
    explainer page's §2.1; a single chunk gives a plain apply; the next-token
    conv of its §2.3 gives V_t = E_{t+1});
  - invariants (causality and serial equivalence of §3.2, associativity of
    §2.3 in prefix and masked dual form, batch independence, continuation);
  - a pure-Python scalar brute force on tiny shapes.
test_pins_catch_planted_mistakes plants plausible mistakes into a copy of the
oracle source and checks that every one of them fails at least one pin.
"""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from oracle import ipttt_oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ----------------------------------------------------------------------------
# small random cases (pages' orientation, float64)
# ----------------------------------------------------------------------------

def case(seed=0, N=1, L=37, d=6, F=10, Kc=4, scale=1.0):
    r = np.random.default_rng(seed)
    return dict(
        X=r.standard_normal((N, L, d)) * scale,
        E=r.standard_normal((N, L, d)),
        W_g=r.standard_normal((d, F)) / math.sqrt(d),
        W_u=r.standard_normal((d, F)) / math.sqrt(d),
        conv_w=r.standard_normal((d, Kc)) / math.sqrt(Kc),
        Proj=r.standard_normal((d, d)) / math.sqrt(d),
        W_0=r.standard_normal((F, d)) / math.sqrt(F),
    )


def run(orc, c, eta, B, update="linear", **kw):
    return orc.prefill(c["X"], c["E"], c["W_g"], c["W_u"], c["conv_w"], c["Proj"], c["W_0"],
                       eta, B, update=update, **kw)


def T(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.float64)


# ----------------------------------------------------------------------------
# independent model from library routines
# ----------------------------------------------------------------------------

def lib_Z(X, W_g, W_u):
    """Gated-MLP activation with torch's silu and linear (weight = out x in)."""
    x = T(X)
    return Fn.silu(Fn.linear(x, T(W_g).T)) * Fn.linear(x, T(W_u).T)


def lib_V(E_chunk, conv_w, Proj):
    """Depthwise conv with torch conv1d (a cross-correlation) and a right zero pad
    of Kc - 1 inside the chunk, then the projection."""
    e = T(E_chunk)                       # [T, d]
    w = T(conv_w)                        # [d, Kc]
    d, Kc = w.shape
    inp = Fn.pad(e.T[None], (0, Kc - 1))  # [1, d, T + Kc - 1]
    C = Fn.conv1d(inp, w[:, None, :], groups=d)[0].T
    return Fn.linear(C, T(Proj).T)


def lib_step(Z, V, W, eta, update):
    """One gradient-descent step on the chunk's loss, derived by autograd.
    linear: loss = -sum_t <z_t W, v_t>   mse: loss = 1/2 sum_t ||z_t W - v_t||^2."""
    W = W.clone().requires_grad_(True)
    if update == "linear":
        loss = -((Z @ W) * V).sum()
    else:
        loss = 0.5 * ((Z @ W - V) ** 2).sum()
    (g,) = torch.autograd.grad(loss, W)
    return (W - eta * g).detach()


def lib_scan(c, eta, B, update="linear"):
    X, E = c["X"], c["E"]
    N, L, _ = X.shape
    O = torch.zeros(X.shape, dtype=torch.float64)
    Wf = []
    for n in range(N):
        W = T(c["W_0"])
        for s in range(0, L, B):
            e_ = min(s + B, L)
            Z = lib_Z(X[n, s:e_], c["W_g"], c["W_u"])
            V = lib_V(E[n, s:e_], c["conv_w"], c["Proj"])
            O[n, s:e_] = Z @ W
            W = lib_step(Z, V, W, eta, update)
        Wf.append(W)
    return O.numpy(), torch.stack(Wf).numpy()


# ----------------------------------------------------------------------------
# pins (each raises AssertionError when the oracle disagrees)
# ----------------------------------------------------------------------------

def pin_gate_up_library(orc):
    c = case(1, L=23, d=7, F=13)
    Z = orc.gate_up(c["X"][0], c["W_g"], c["W_u"])
    np.testing.assert_allclose(Z, lib_Z(c["X"][0], c["W_g"], c["W_u"]).numpy(), rtol=1e-12, atol=1e-14)


def pin_conv_library(orc):
    for T_ in (1, 2, 3, 4, 5, 17):
        c = case(2, L=T_, d=5)
        C = orc.conv_chunk(c["E"][0], c["conv_w"])
        ref = lib_V(c["E"][0], c["conv_w"], np.eye(5)).numpy()
        np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-14)
        V = orc.target_chunk(c["E"][0], c["conv_w"], c["Proj"])
        np.testing.assert_allclose(V, lib_V(c["E"][0], c["conv_w"], c["Proj"]).numpy(),
                                   rtol=1e-12, atol=1e-14)


def pin_next_token_target(orc):
    """Conv kernel with its one at the next-token tap and a permutation Proj:
    V_t = E_{t+1} permuted inside the chunk, and 0 on the chunk's last row."""
    d, Tn = 6, 9
    r = np.random.default_rng(3)
    E = r.standard_normal((Tn, d))
    conv_w = np.zeros((d, 4))
    conv_w[:, 1] = 1.0
    perm = np.array([2, 0, 5, 1, 3, 4])
    P = np.zeros((d, d))
    P[np.arange(d), perm] = 1.0            # row vector e_c @ P = e_{perm[c]}
    V = orc.target_chunk(E, conv_w, P)
    expect = np.zeros((Tn, d))
    expect[:-1][:, perm] = E[1:]
    np.testing.assert_array_equal(V, expect)


def pin_eta0_textbook(orc):
    for B in (1, 4, 16, 100):
        c = case(4, N=2, L=29)
        O, Wf = run(orc, c, 0.0, B)
        for n in range(2):
            ref = Fn.linear(lib_Z(c["X"][n], c["W_g"], c["W_u"]), T(c["W_0"]).T).numpy()
            np.testing.assert_allclose(O[n], ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_array_equal(Wf[n], c["W_0"])


def pin_single_chunk(orc):
    """B >= L: one apply with W_0, and one update step over the whole sequence."""
    for update in ("linear", "mse"):
        c = case(5, L=21)
        for B in (21, 64):
            O, Wf = run(orc, c, 0.05, B, update)
            Z = lib_Z(c["X"][0], c["W_g"], c["W_u"])
            V = lib_V(c["E"][0], c["conv_w"], c["Proj"])
            np.testing.assert_allclose(O[0], (Z @ T(c["W_0"])).numpy(), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Wf[0], lib_step(Z, V, T(c["W_0"]), 0.05, update).numpy(),
                                       rtol=1e-12, atol=1e-13)


def pin_library_model(orc):
    for update in ("linear", "mse"):
        for B, L in ((1, 9), (3, 25), (4, 37), (8, 37), (37, 37)):
            c = case(6 + B, N=2, L=L)
            O, Wf = run(orc, c, 0.03, B, update)
            Or, Wr = lib_scan(c, 0.03, B, update)
            np.testing.assert_allclose(O, Or, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(Wf, Wr, rtol=1e-10, atol=1e-12)


def pin_prefix_form(orc):
    for B in (1, 5, 8, 40):
        c = case(7, N=2, L=40)
        O, Wf = run(orc, c, 0.02, B)
        Op, Wp = orc.prefill_prefix_form(c["X"], c["E"], c["W_g"], c["W_u"], c["conv_w"],
                                         c["Proj"], c["W_0"], 0.02, B)
        np.testing.assert_allclose(O, Op, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Wf, Wp, rtol=1e-11, atol=1e-12)


def pin_prefix_form_stream(orc):
    """The chunk-by-chunk prefix form against the all-at-once one (itself pinned
    against the scan above and the masked dual form below), with tails."""
    for B, L in ((1, 9), (5, 23), (8, 40), (40, 40), (64, 40)):
        c = case(17, N=1, L=L)
        Op, Wp = orc.prefill_prefix_form(c["X"], c["E"], c["W_g"], c["W_u"], c["conv_w"],
                                         c["Proj"], c["W_0"], 0.03, B)
        got = np.full_like(Op[0], np.nan)
        seen = []

        def put(s, e, Ok):
            seen.append((s, e))
            got[s:e] = Ok

        Wf = orc.prefill_prefix_form_stream(c["X"][0], c["E"][0], c["W_g"], c["W_u"], c["conv_w"],
                                            c["Proj"], c["W_0"], 0.03, B, put)
        assert seen == orc.chunk_ranges(L, B)
        np.testing.assert_allclose(got, Op[0], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Wf, Wp[0], rtol=1e-11, atol=1e-12)


def pin_dual_form(orc):
    """Linear: O = Z W_0 + eta (M * Z Z^T) V with M[t, s] = [chunk(s) < chunk(t)],
    Z and V from library routines (V chunk by chunk)."""
    L, B, eta = 30, 7, 0.04
    c = case(8, L=L)
    Z = lib_Z(c["X"][0], c["W_g"], c["W_u"])
    V = torch.cat([lib_V(c["E"][0, s:s + B], c["conv_w"], c["Proj"]) for s in range(0, L, B)])
    ch = torch.arange(L) // B
    M = (ch[None, :] < ch[:, None]).double()
    ref = Z @ T(c["W_0"]) + eta * ((M * (Z @ Z.T)) @ V)
    O, _ = run(orc, c, eta, B)
    np.testing.assert_allclose(O[0], ref.numpy(), rtol=1e-11, atol=1e-12)


def pin_final_state(orc):
    """Linear: W_final = W_0 + eta Z^T V over the whole sequence (associativity),
    and the per-entry evaluator agrees with the full scan."""
    L, B, eta = 33, 6, 0.05
    c = case(9, L=L)
    Z = lib_Z(c["X"][0], c["W_g"], c["W_u"])
    V = torch.cat([lib_V(c["E"][0, s:s + B], c["conv_w"], c["Proj"]) for s in range(0, L, B)])
    _, Wf = run(orc, c, eta, B)
    np.testing.assert_allclose(Wf[0], (T(c["W_0"]) + eta * Z.T @ V).numpy(), rtol=1e-11, atol=1e-12)
    rows = np.array([0, 3, 9, 9, 5])
    cols = np.array([0, 5, 2, 0, 4])
    got = orc.final_weight_entries(c["X"][0], c["E"][0], c["W_g"], c["W_u"], c["conv_w"], c["Proj"],
                                   c["W_0"], eta, B, rows, cols)
    np.testing.assert_allclose(got, Wf[0][rows, cols], rtol=1e-11, atol=1e-12)


def pin_causality(orc):
    """Perturbing X[p:] and E[p:] leaves O[:p] bit-identical; perturbing E inside
    chunk k leaves O up to the end of chunk k bit-identical (the target of a chunk
    is first used by the next one)."""
    L, B = 40, 8
    for update in ("linear", "mse"):
        c = case(10, L=L)
        O, _ = run(orc, c, 0.05, B, update)
        r = np.random.default_rng(11)
        for p in (0, 1, 7, 8, 9, 17, 39):
            c2 = dict(c, X=c["X"].copy(), E=c["E"].copy())
            c2["X"][:, p:] += r.standard_normal(c2["X"][:, p:].shape)
            c2["E"][:, p:] += r.standard_normal(c2["E"][:, p:].shape)
            O2, _ = run(orc, c2, 0.05, B, update)
            np.testing.assert_array_equal(O2[:, :p], O[:, :p])
            assert p == L or not np.array_equal(O2[:, p:], O[:, p:])
        for k in range(L // B):
            c3 = dict(c, E=c["E"].copy())
            c3["E"][:, k * B:(k + 1) * B] += 1.0
            O3, _ = run(orc, c3, 0.05, B, update)
            np.testing.assert_array_equal(O3[:, :(k + 1) * B], O[:, :(k + 1) * B])
            if k + 1 < L // B:
                assert not np.array_equal(O3[:, (k + 1) * B:], O[:, (k + 1) * B:])


def brute(X, E, W_g, W_u, conv_w, Proj, W_0, eta, B, update):
    """Scalar loops, no numpy arithmetic: one sequence."""
    L, d = len(X), len(X[0])
    F = len(W_g[0])
    Kc = len(conv_w[0])
    W = [[W_0[i][j] for j in range(d)] for i in range(F)]
    O = [[0.0] * d for _ in range(L)]
    s = 0
    while s < L:
        e = min(s + B, L)
        Z = []
        for t in range(s, e):
            row = []
            for f in range(F):
                a = sum(X[t][i] * W_g[i][f] for i in range(d))
                u = sum(X[t][i] * W_u[i][f] for i in range(d))
                row.append(a / (1.0 + math.exp(-a)) * u)
            Z.append(row)
        C = []
        for t in range(s, e):
            C.append([sum(conv_w[ch][j] * E[t + j][ch] for j in range(Kc) if t + j < e)
                      for ch in range(d)])
        V = [[sum(C[t][i] * Proj[i][o] for i in range(d)) for o in range(d)] for t in range(e - s)]
        Ok = [[sum(Z[t][f] * W[f][o] for f in range(F)) for o in range(d)] for t in range(e - s)]
        for t in range(e - s):
            O[s + t] = Ok[t]
        G = V if update == "linear" else [[V[t][o] - Ok[t][o] for o in range(d)] for t in range(e - s)]
        for f in range(F):
            for o in range(d):
                W[f][o] += eta * sum(Z[t][f] * G[t][o] for t in range(e - s))
        s = e
    return O, W


def pin_brute_force(orc):
    for update in ("linear", "mse"):
        for B in (1, 3, 4, 11, 16):
            c = case(12 + B, L=11, d=3, F=5)
            O, Wf = run(orc, c, 0.1, B, update)
            lists = {k: v[0].tolist() if k in ("X", "E") else v.tolist() for k, v in c.items()}
            Ob, Wb = brute(lists["X"], lists["E"], lists["W_g"], lists["W_u"], lists["conv_w"],
                           lists["Proj"], lists["W_0"], 0.1, B, update)
            np.testing.assert_allclose(O[0], np.array(Ob), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Wf[0], np.array(Wb), rtol=1e-12, atol=1e-13)


def pin_continuation(orc):
    """Two calls equal one call when the first ends on a chunk boundary (state carried)."""
    for update in ("linear", "mse"):
        c = case(13, N=2, L=40)
        O, Wf = run(orc, c, 0.03, 8, update)
        c1 = dict(c, X=c["X"][:, :16], E=c["E"][:, :16])
        O1, W1 = run(orc, c1, 0.03, 8, update)
        c2 = dict(c, X=c["X"][:, 16:], E=c["E"][:, 16:], W_0=W1)
        O2, W2 = run(orc, c2, 0.03, 8, update)
        np.testing.assert_array_equal(np.concatenate([O1, O2], axis=1), O)
        np.testing.assert_array_equal(W2, Wf)


def pin_batch_independence(orc):
    c = case(14, N=3, L=20)
    O, Wf = run(orc, c, 0.03, 6)
    c2 = dict(c, X=c["X"].copy(), E=c["E"].copy())
    c2["X"][[0, 2]] += 1.0
    c2["E"][[0, 2]] -= 1.0
    O2, W2 = run(orc, c2, 0.03, 6)
    np.testing.assert_array_equal(O2[1], O[1])
    np.testing.assert_array_equal(W2[1], Wf[1])


def pin_update_direction(orc):
    """Linear: each step raises the chunk's similarity sum <Z W, V>.
    MSE: with eta below 2 / lambda_max(Z^T Z) each step lowers ||Z W - V||."""
    c = case(15, L=8, d=4, F=6)
    Z = orc.gate_up(c["X"][0], c["W_g"], c["W_u"])
    V = orc.target_chunk(c["E"][0], c["conv_w"], c["Proj"])
    _, W1 = run(orc, c, 0.05, 8, "linear")
    assert np.sum((Z @ W1[0]) * V) > np.sum((Z @ c["W_0"]) * V)
    lam = np.linalg.eigvalsh(Z.T @ Z).max()
    _, W2 = run(orc, c, 1.0 / lam, 8, "mse")
    assert np.linalg.norm(Z @ W2[0] - V) < np.linalg.norm(Z @ c["W_0"] - V)


def pin_resets(orc):
    """Packed documents: each document's output equals a fresh scan of that document
    alone from W_0 (library model), and earlier documents do not affect it."""
    c = case(16, L=45)
    starts = [13, 30]
    X, E = c["X"][0], c["E"][0]
    O, Wf = orc.prefill_with_resets(X, E, c["W_g"], c["W_u"], c["conv_w"], c["Proj"], c["W_0"],
                                    0.03, 6, starts)
    bounds = [0, 13, 30, 45]
    for a, b in zip(bounds[:-1], bounds[1:]):
        cd = dict(c, X=c["X"][:, a:b], E=c["E"][:, a:b])
        Od, Wd = lib_scan(cd, 0.03, 6)
        np.testing.assert_allclose(O[a:b], Od[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Wf, Wd[0], rtol=1e-10, atol=1e-12)


def pin_decode_steps(orc):
    c = case(17, L=20)
    O, _ = run(orc, c, 0.03, 8)
    Od, Wd = orc.decode_steps(c["X"][0], c["E"][0], c["W_g"], c["W_u"], c["conv_w"], c["Proj"],
                              c["W_0"], 0.03, 8)
    np.testing.assert_array_equal(Od, O[0])
    c16 = dict(c, X=c["X"][:, :16], E=c["E"][:, :16])
    _, W16 = run(orc, c16, 0.03, 8)
    np.testing.assert_array_equal(Wd, W16[0])


# ---- backward through the scan ------------------------------------------------

GRAD_KEYS = ("dX", "dE", "dW_g", "dW_u", "dProj", "dconv_w", "dW_start")


def lib_scan_graph(p, eta, B, update):
    """The library model's scan kept on torch's autograd graph: the update step
    is derived by autograd from its loss with create_graph, so the gradient of
    anything downstream flows through every update."""
    X, E = p["X"], p["E"]
    N, L, _ = X.shape
    Os, Wf = [], []
    for n in range(N):
        W = p["W_0"]
        rows = []
        for s in range(0, L, B):
            e_ = min(s + B, L)
            x = X[n, s:e_]
            Z = Fn.silu(Fn.linear(x, p["W_g"].T)) * Fn.linear(x, p["W_u"].T)
            Kc = p["conv_w"].shape[1]
            inp = Fn.pad(E[n, s:e_].T[None], (0, Kc - 1))
            C = Fn.conv1d(inp, p["conv_w"][:, None, :], groups=p["conv_w"].shape[0])[0].T
            V = Fn.linear(C, p["Proj"].T)
            rows.append(Z @ W)
            loss = -((Z @ W) * V).sum() if update == "linear" else 0.5 * ((Z @ W - V) ** 2).sum()
            (g,) = torch.autograd.grad(loss, W, create_graph=True)
            W = W - eta * g
        Os.append(torch.cat(rows))
        Wf.append(W)
    return torch.stack(Os), torch.stack(Wf)


def grads_by_autograd(c, dO, dWf, eta, B, update):
    p = {k: T(v).requires_grad_(True) for k, v in c.items()}
    O, Wf = lib_scan_graph(p, eta, B, update)
    loss = (O * T(dO)).sum() + (Wf * T(dWf)).sum()
    names = ("X", "E", "W_g", "W_u", "Proj", "conv_w", "W_0")
    gs = torch.autograd.grad(loss, [p[k] for k in names])
    return {("d" + k if k != "W_0" else "dW_start"): g.numpy() for k, g in zip(names, gs)}


def orc_grads(orc, c, dO, dWf, eta, B, update):
    return orc.backward(c["X"], c["E"], c["W_g"], c["W_u"], c["conv_w"], c["Proj"], c["W_0"], eta,
                        B, dO, dW_final=dWf, update=update)


def pin_backward_autograd(orc):
    """Every gradient against torch.autograd through the library model (both
    rules, two sequences, a short last chunk, an upstream gradient on W_final)."""
    for update, eta in (("linear", 0.05), ("mse", 0.02)):
        c = case(31, N=2, L=23, d=5, F=7)
        r = np.random.default_rng(32)
        dO = r.standard_normal((2, 23, 5))
        dWf = r.standard_normal((2, 7, 5))
        got = orc_grads(orc, c, dO, dWf, eta, 5, update)
        ref = grads_by_autograd(c, dO, dWf, eta, 5, update)
        for k in GRAD_KEYS:
            np.testing.assert_allclose(got[k], ref[k], rtol=1e-9, atol=1e-11, err_msg=f"{update} {k}")


def pin_backward_finite_differences(orc):
    """Directional derivatives of the (separately pinned) forward by central
    differences: <grad, Delta> = (L(p + h Delta) - L(p - h Delta)) / 2h."""
    for update, eta in (("linear", 0.1), ("mse", 0.05)):
        c = case(41, N=1, L=11, d=4, F=6)
        r = np.random.default_rng(42)
        dO = r.standard_normal((1, 11, 4))
        dWf = r.standard_normal((1, 6, 4))
        g = orc_grads(orc, c, dO, dWf, eta, 3, update)

        def loss(cc):
            O, Wf = run(orc, cc, eta, 3, update)
            return float((O * dO).sum() + (Wf * dWf).sum())

        names = ("X", "E", "W_g", "W_u", "Proj", "conv_w", "W_0")
        for trial in range(3):
            delta = {k: r.standard_normal(c[k].shape) for k in names}
            h = 1e-5
            plus = {k: c[k] + h * delta[k] for k in names}
            minus = {k: c[k] - h * delta[k] for k in names}
            fd = (loss(plus) - loss(minus)) / (2 * h)
            an = sum(float((g["d" + k if k != "W_0" else "dW_start"] * delta[k]).sum()) for k in names)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (update, trial, fd, an)


def pin_backward_eta0(orc):
    """eta = 0: the textbook gated-MLP backward with the fixed weight W_0:
    dW_0 = sum Z^T dO + dW_final, dX from dZ = dO W_0^T, and no gradient reaches
    the target (E, Proj, conv)."""
    c = case(51, N=2, L=9, d=4, F=6)
    r = np.random.default_rng(52)
    dO = r.standard_normal((2, 9, 4))
    dWf = r.standard_normal((2, 6, 4))
    g = orc_grads(orc, c, dO, dWf, 0.0, 4, "linear")
    x = T(c["X"]).requires_grad_(True)
    wg, wu = T(c["W_g"]).requires_grad_(True), T(c["W_u"]).requires_grad_(True)
    Z = Fn.silu(x @ wg) * (x @ wu)
    dx, dwg, dwu = torch.autograd.grad((Z @ T(c["W_0"]) * T(dO)).sum(), [x, wg, wu])
    Zn = Z.detach().numpy()
    np.testing.assert_allclose(g["dW_start"], np.einsum("ntf,ntc->fc", Zn, dO) + dWf.sum(0), rtol=1e-11)
    np.testing.assert_allclose(g["dX"], dx.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dW_g"], dwg.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dW_u"], dwu.numpy(), rtol=1e-10, atol=1e-12)
    for k in ("dE", "dProj", "dconv_w"):
        assert np.abs(g[k]).max() == 0.0, k


def pin_backward_linear_in_upstream(orc):
    """The gradients are linear in the upstream gradients (dO, dW_final), and the
    per-sequence start weight gets each sequence's own dW_0."""
    c = case(61, N=2, L=10, d=4, F=6)
    r = np.random.default_rng(62)
    a = (r.standard_normal((2, 10, 4)), r.standard_normal((2, 6, 4)))
    b = (r.standard_normal((2, 10, 4)), r.standard_normal((2, 6, 4)))
    ga = orc_grads(orc, c, *a, 0.1, 3, "mse")
    gb = orc_grads(orc, c, *b, 0.1, 3, "mse")
    gs = orc_grads(orc, c, a[0] + 2 * b[0], a[1] + 2 * b[1], 0.1, 3, "mse")
    for k in GRAD_KEYS:
        np.testing.assert_allclose(gs[k], ga[k] + 2 * gb[k], rtol=1e-9, atol=1e-11)
    c3 = dict(c, W_0=np.stack([c["W_0"], c["W_0"]]))
    g3 = orc_grads(orc, c3, *a, 0.1, 3, "mse")
    np.testing.assert_allclose(g3["dW_start"].sum(0), ga["dW_start"], rtol=1e-12)


def pin_initial_weight_grad_entries(orc):
    """Sampled dL/dW_0 entries (linear rule) agree with the full backward."""
    c = case(71, N=1, L=17, d=5, F=7)
    r = np.random.default_rng(72)
    dO, dWf = r.standard_normal((1, 17, 5)), r.standard_normal((1, 7, 5))
    g = orc_grads(orc, c, dO, dWf, 0.07, 4, "linear")
    rows, cols = r.integers(0, 7, 12), r.integers(0, 5, 12)
    got = orc.initial_weight_grad_entries(c["X"][0], c["W_g"], c["W_u"], dO[0], dWf[0], rows, cols)
    np.testing.assert_allclose(got, g["dW_start"][rows, cols], rtol=1e-10, atol=1e-12)


PINS = [
    pin_gate_up_library, pin_conv_library, pin_next_token_target, pin_eta0_textbook,
    pin_single_chunk, pin_library_model, pin_prefix_form, pin_prefix_form_stream, pin_dual_form, pin_final_state,
    pin_causality, pin_brute_force, pin_continuation, pin_batch_independence,
    pin_update_direction, pin_resets, pin_decode_steps, pin_backward_autograd,
    pin_backward_finite_differences, pin_backward_eta0, pin_backward_linear_in_upstream,
    pin_initial_weight_grad_entries,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)


# ----------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------

MUTANTS = {
    "conv taps backward": ("C[: T - j] += conv_w[:, j][None, :] * E_chunk[j:]",
                           "C[j:] += conv_w[:, j][None, :] * E_chunk[: T - j]"),
    "conv kernel flipped": ("C[: T - j] += conv_w[:, j][None, :] * E_chunk[j:]",
                            "C[: T - j] += conv_w[:, -1 - j][None, :] * E_chunk[j:]"),
    "conv tap dropped": ("for j in range(conv_w.shape[1]):", "for j in range(conv_w.shape[1] - 1):"),
    "sigmoid sign": ("return a / (1.0 + np.exp(-a))", "return a / (1.0 + np.exp(a))"),
    "silu without sigmoid": ("return a / (1.0 + np.exp(-a))", "return a"),
    "gate and up swapped": ("return silu(X @ W_g) * (X @ W_u)", "return silu(X @ W_u) * (X @ W_g)"),
    "proj transposed": ("return conv_chunk(E_chunk, conv_w) @ _f64(Proj)",
                        "return conv_chunk(E_chunk, conv_w) @ _f64(Proj).T"),
    "linear update sign": ("W = W + eta * (Z.T @ V)", "W = W - eta * (Z.T @ V)"),
    "linear update drops eta": ("W = W + eta * (Z.T @ V)", "W = W + (Z.T @ V)"),
    "linear update mean not sum": ("W = W + eta * (Z.T @ V)", "W = W + eta * (Z.T @ V) / len(Z)"),
    "update before apply": ("O_k = Z @ W\n", "O_k = Z @ (W + eta * (Z.T @ V))\n"),
    "mse residual sign": ("W = W - eta * (Z.T @ (O_k - V))", "W = W - eta * (Z.T @ (O_k + V))"),
    "mse update sign": ("W = W - eta * (Z.T @ (O_k - V))", "W = W + eta * (Z.T @ (O_k - V))"),
    "chunk too short": ("return [(s, min(s + B, L)) for s in range(0, L, B)]",
                        "return [(s, min(s + B - 1, L)) for s in range(0, L, B)]"),
    "prefix form inclusive": ("O[n, s:e] = Zs[k] @ (W0 + eta * prefix)\n            prefix = prefix + S[k]",
                              "prefix = prefix + S[k]\n            O[n, s:e] = Zs[k] @ (W0 + eta * prefix)"),
    "streamed prefix form inclusive": ("on_chunk(s, e, Z @ W0 + eta * (Z @ P))\n        P += Z.T @ V",
                                       "P += Z.T @ V\n        on_chunk(s, e, Z @ W0 + eta * (Z @ P))"),
    "streamed prefix form drops eta": ("return W0 + eta * P", "return W0 + P"),
    "reset keeps state": ("            W = _f64(W_0).copy()\n", "            pass\n"),
    # backward
    "backward drops the update path of dZ": ("dZ = dOk @ Wk.T + eta * (V @ G.T)", "dZ = dOk @ Wk.T"),
    "backward uses G_k not G_k+1": (
        "dZ = dOk @ Wk.T + eta * (V @ G.T)\n                dV = eta * (Z @ G)\n                G = G + Z.T @ dOk",
        "G = G + Z.T @ dOk\n                dZ = dOk @ Wk.T + eta * (V @ G.T)\n                dV = eta * (Z @ G)"),
    "backward dV drops eta": ("dV = eta * (Z @ G)\n                G = G + Z.T @ dOk",
                              "dV = Z @ G\n                G = G + Z.T @ dOk"),
    "silu derivative drops a term": ("return s * (1.0 + a * (1.0 - s))", "return s"),
    "conv adjoint shifted the wrong way": ("dE[j:] += conv_w[:, j][None, :] * dC_chunk[: T - j]",
                                           "dE[: T - j] += conv_w[:, j][None, :] * dC_chunk[j:]"),
    "mse backward residual path sign": ("dY = dOk - eta * (Z @ G)", "dY = dOk + eta * (Z @ G)"),
    "mse backward drops R G^T": ("dZ = dY @ Wk.T - eta * (R @ G.T)", "dZ = dY @ Wk.T"),
    "dProj transposed": ('out["dProj"] += C.T @ dV', 'out["dProj"] += (C.T @ dV).T'),
}


def _mutant(old, new):
    src = inspect.getsource(ipttt_oracle)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, RuntimeError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{name}' passed every pin"


def test_chunk_ranges_edges():
    assert oracle.chunk_ranges(0, 4) == []
    assert oracle.chunk_ranges(4, 4) == [(0, 4)]
    assert oracle.chunk_ranges(5, 4) == [(0, 4), (4, 5)]
    with pytest.raises(ValueError):
        oracle.chunk_ranges(5, 0)


def test_empty_sequence():
    c = case(18, L=0)
    O, Wf = run(oracle, c, 0.1, 4)
    assert O.shape == (1, 0, 6)
    np.testing.assert_array_equal(Wf[0], c["W_0"])


# ----------------------------------------------------------------------------
# worked example (tests/golden): numbers stored by a script that calls only the
# oracle, checked here against the scalar loops above and per-step formulas
# ----------------------------------------------------------------------------

def _worked_example():
    import json
    import pathlib
    path = pathlib.Path(__file__).parent / "golden" / "worked_example_d2_F3.json"
    return json.loads(path.read_text(encoding="utf-8"))


@pytest.mark.parametrize("update", ["linear", "mse"])
def test_worked_example_scalar(update):
    """Every stored chunk of the worked example against scalar arithmetic:
    Z from the gated-MLP formula, V from the forward conv with its zero pad
    and Proj, O and the fast weight after each chunk from the scalar scan
    (brute) run on the prefix that ends with that chunk."""
    g = _worked_example()
    inp, eta, B = g["inputs"], g["eta"], g["chunk"]
    X, E, W_g, W_u = inp["X"], inp["E"], inp["W_g"], inp["W_u"]
    conv_w, Proj = inp["conv_w"], inp["Proj"]
    d, F, Kc = len(X[0]), len(W_g[0]), len(conv_w[0])
    chunks = g[update]["chunks"]
    assert [c["tokens"] for c in chunks] == [[0, 2], [2, 4], [4, 5]]
    for c in chunks:
        s, e = c["tokens"]
        for t in range(s, e):
            for f in range(F):
                a = sum(X[t][i] * W_g[i][f] for i in range(d))
                u = sum(X[t][i] * W_u[i][f] for i in range(d))
                assert c["Z"][t - s][f] == pytest.approx(a * u / (1.0 + math.exp(-a)), rel=1e-14,
                                                         abs=1e-15)
            conv = [sum(conv_w[ch][j] * E[t + j][ch] for j in range(Kc) if t + j < e)
                    for ch in range(d)]
            for o in range(d):
                v = sum(conv[i] * Proj[i][o] for i in range(d))
                assert c["V"][t - s][o] == pytest.approx(v, rel=1e-14, abs=1e-15)
        Ob, Wb = brute(X[:e], E[:e], W_g, W_u, conv_w, Proj, inp["W_0"], eta, B, update)
        np.testing.assert_allclose(np.array(c["O"]), np.array(Ob[s:e]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(np.array(c["W_after"]), np.array(Wb), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("update", ["linear", "mse"])
def test_worked_example_oracle(update):
    """The oracle still reproduces the stored worked example."""
    g = _worked_example()
    a = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
    O, Wf = oracle.prefill(a["X"][None], a["E"][None], a["W_g"], a["W_u"], a["conv_w"],
                           a["Proj"], a["W_0"][None], g["eta"], g["chunk"], update=update)
    chunks = g[update]["chunks"]
    np.testing.assert_allclose(O[0], np.concatenate([np.array(c["O"]) for c in chunks]),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(Wf[0], np.array(chunks[-1]["W_after"]), rtol=1e-13, atol=1e-15)

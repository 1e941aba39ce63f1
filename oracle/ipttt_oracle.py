"""Float64 CPU oracle for the In-Place Test-Time Training fast-weight prefill.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only the
test suite, the package smoke check and the benchmark's CPU-baseline leg may
import it. The HIP library and its Python binding never import, call or link
anything here, and this module imports nothing from them.

It is written to be read against the pages, step by step, in plain numpy
float64 with no blocking, fusion or reordering beyond what the method states.

Sources (web pages on the method, cited by title and section):
  [digest]    "论文日报 2026-04-14", entry "In-Place Test-Time Training for
              Large Language Models", sections 核心创新 and 方法论总结
  [explainer] "In-Place Test-Time Training：让大语言模型在推理时原地进化，
              长上下文任务准确率显著提升", sections 2.1, 2.2 (with Fig. 1),
              2.3, 3.2
  [analysis]  "大模型长文本核心架构全解析（非常详细），搞懂“边读边学”看这篇
              就够了！", sub-headings 第一板斧, 第二板斧, 第三板斧
  [abstract]  "Внутреннее тестовое обучение на месте" (English abstract)

Orientation (row vectors, as in the gated-MLP formula of [explainer] §2.1):
  X, E      [N, L, d]   layer input and token embeddings of N sequences
  W_g, W_u  [d, F]      frozen gate / up projections (slow weights)
  W  (W_o)  [F, d]      down projection, the fast weight, one per sequence
  conv_w    [d, Kc]     depthwise 1-D conv over tokens, Kc taps per channel
  Proj      [d, d]      target projection, V = Conv(E) @ Proj
  O         [N, L, d]   layer output

Readings taken where the pages leave a step open (each one is listed again,
with its justification, in the design notes of the repository):
  R1  Conv taps look forward: C[t] = sum_j conv_w[:, j] * E[t + j], j = 0..Kc-1.
      [explainer] §2.3 says the conv lets the target carry future-token
      information and gives the next-token target as the kernel with its one
      at the next position; tap j = 1 is that next position.
  R2  Zero padding at the chunk end: E[t + j] is taken as 0 when t + j falls
      past the end of the chunk, so a chunk's target reads only that chunk's
      embeddings and the scan stays causal ([explainer] §3.2 causal padding,
      [analysis] 第三板斧 strict causality).
  R3  The conv is a depthwise cross-correlation (no kernel flip), no bias.
  R4  Linear update: one gradient step on the negative similarity
      -sum_t <z_t W, v_t> over the chunk: W += eta * Z^T V (sum, no 1/B)
      ([explainer] §2.3: a simple similarity loss whose update is
      associative; §6: single-step gradient descent).
  R5  MSE update: one gradient step on 1/2 sum_t ||z_t W - v_t||^2 at the
      pre-update W: W -= eta * Z^T (Z W - V) ([analysis] 第二板斧: make
      W z_t close to v_t).
  R6  Apply then update: chunk k's output uses W_k; its own update is first
      visible to chunk k+1 ([explainer] §2.2 with Fig. 1, [analysis] 第三板斧).
  R7  SiLU(a) = a * sigmoid(a).
  R8  A last chunk shorter than B (L mod B != 0) is applied and then updated
      like any other chunk, with R2's zero padding at its own end.
  R9  State persists across calls; each call starts a new chunk at its first
      token. Reset puts the pretrained W_0 back ([explainer] §3.2 boundary
      reset).
  RB1 Training through the layer ([explainer] §4.1 continued training of a
      pretrained model, §4.2 pretraining from scratch) differentiates the scan
      as written, through every update (no stop-gradient). The trainable
      inputs are X, E, W_g, W_u, the projection (trainable by [explainer]
      §2.3), the conv weights and the fast weight's start value W_0 (the
      pretrained down projection); eta is a fixed hyper-parameter.

Parity: every function here is pinned by the not-gpu tests in
tests/test_oracle.py against closed forms, library routines (torch silu,
conv1d, autograd), invariants and a scalar brute force. Whether these readings
match the authors' own code is not pinned by anything on the pages, which
print no numeric example.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu",
    "gate_up",
    "conv_chunk",
    "target_chunk",
    "chunk_ranges",
    "prefill",
    "prefill_prefix_form",
    "prefill_prefix_form_stream",
    "prefill_with_resets",
    "final_weight_entries",
    "decode_steps",
    "silu_grad",
    "conv_chunk_backward",
    "backward",
    "initial_weight_grad_entries",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a)) (R7; [explainer] §2.1)."""
    return a / (1.0 + np.exp(-a))


def gate_up(X: np.ndarray, W_g: np.ndarray, W_u: np.ndarray) -> np.ndarray:
    """Intermediate activation Z = SiLU(X W_g) * (X W_u).

    The part of the gated MLP in front of the fast weight ([explainer] §2.1;
    the explainer's §2.2 calls it the intermediate activation A, [analysis]
    第一板斧 calls its rows z_t). X: [T, d], W_g / W_u: [d, F] -> [T, F].
    """
    X, W_g, W_u = _f64(X), _f64(W_g), _f64(W_u)
    return silu(X @ W_g) * (X @ W_u)


def conv_chunk(E_chunk: np.ndarray, conv_w: np.ndarray) -> np.ndarray:
    """Depthwise conv over the tokens of ONE chunk (R1-R3).

    C[t, c] = sum_j conv_w[c, j] * E[t + j, c], with E[t + j] = 0 when t + j is
    past the chunk's last token. E_chunk: [T, d], conv_w: [d, Kc] -> [T, d].
    """
    E_chunk, conv_w = _f64(E_chunk), _f64(conv_w)
    T, d = E_chunk.shape
    C = np.zeros((T, d), dtype=np.float64)
    for j in range(conv_w.shape[1]):
        if j >= T:
            break
        # rows t = 0 .. T-1-j read E[t + j]; rows past that read the zero pad
        C[: T - j] += conv_w[:, j][None, :] * E_chunk[j:]
    return C


def target_chunk(E_chunk: np.ndarray, conv_w: np.ndarray, Proj: np.ndarray) -> np.ndarray:
    """LM-aligned target V = Proj(Conv(E)) of one chunk, as V = Conv(E) @ Proj.

    [explainer] §2.3 (target built from token embeddings by a 1-D conv and a
    trainable projection); [analysis] 第二板斧.
    """
    return conv_chunk(E_chunk, conv_w) @ _f64(Proj)


def chunk_ranges(L: int, B: int):
    """Non-overlapping chunks [kB, min((k+1)B, L)), k ascending ([explainer] §2.2)."""
    if B <= 0:
        raise ValueError("chunk size must be positive")
    return [(s, min(s + B, L)) for s in range(0, L, B)]


def _check_update(update: str) -> None:
    if update not in ("linear", "mse"):
        raise ValueError(f"unknown update rule {update!r}")


def prefill(X, E, W_g, W_u, conv_w, Proj, W_start, eta, B, update="linear"):
    """Chunk-wise apply-then-update scan over N independent sequences.

    X, E: [N, L, d]. W_start: [F, d] (one W for all sequences) or [N, F, d].
    Returns (O [N, L, d], W_final [N, F, d]).

    For each chunk k with tokens s..e-1 ([explainer] §2.2 with Fig. 1,
    [analysis] 第三板斧):
      Z_k = SiLU(X_k W_g) * (X_k W_u)                 intermediate activation
      V_k = Conv(E_k) @ Proj                           target (R1-R3)
      O_k = Z_k W_k                                    apply with W_k (R6)
      W_{k+1} = W_k + eta Z_k^T V_k                    linear (R4)
      W_{k+1} = W_k - eta Z_k^T (Z_k W_k - V_k)        mse (R5)
    """
    _check_update(update)
    X, E = _f64(X), _f64(E)
    N, L, d = X.shape
    W_start = _f64(W_start)
    F = W_start.shape[-2]
    O = np.zeros((N, L, d), dtype=np.float64)
    W_final = np.zeros((N, F, d), dtype=np.float64)
    for n in range(N):
        W = (W_start[n] if W_start.ndim == 3 else W_start).copy()
        for s, e in chunk_ranges(L, B):
            Z = gate_up(X[n, s:e], W_g, W_u)
            V = target_chunk(E[n, s:e], conv_w, Proj)
            O_k = Z @ W
            O[n, s:e] = O_k
            if update == "linear":
                W = W + eta * (Z.T @ V)
            else:
                W = W - eta * (Z.T @ (O_k - V))
        W_final[n] = W
    return O, W_final


def prefill_prefix_form(X, E, W_g, W_u, conv_w, Proj, W_start, eta, B):
    """Linear update only: the prefix-sum form of the same scan.

    Because the linear update is associative ([explainer] §2.3), the weight
    that chunk k sees is W_k = W_0 + eta * sum_{j<k} Z_j^T V_j. This builds every
    chunk's S_j = Z_j^T V_j first, takes the exclusive prefix sum over j, and
    only then applies O_k = Z_k W_k. Returns (O, W_final) like prefill().
    """
    X, E = _f64(X), _f64(E)
    N, L, d = X.shape
    W_start = _f64(W_start)
    F = W_start.shape[-2]
    O = np.zeros((N, L, d), dtype=np.float64)
    W_final = np.zeros((N, F, d), dtype=np.float64)
    ranges = chunk_ranges(L, B)
    for n in range(N):
        W0 = W_start[n] if W_start.ndim == 3 else W_start
        Zs = [gate_up(X[n, s:e], W_g, W_u) for s, e in ranges]
        Vs = [target_chunk(E[n, s:e], conv_w, Proj) for s, e in ranges]
        S = [Zj.T @ Vj for Zj, Vj in zip(Zs, Vs)]
        prefix = np.zeros((F, d), dtype=np.float64)
        for k, (s, e) in enumerate(ranges):
            O[n, s:e] = Zs[k] @ (W0 + eta * prefix)
            prefix = prefix + S[k]
        W_final[n] = W0 + eta * prefix
    return O, W_final


def prefill_prefix_form_stream(X, E, W_g, W_u, conv_w, Proj, W_start, eta, B, on_chunk):
    """Linear update only: the prefix-sum form of ONE sequence, chunk by chunk.

    The same function as prefill_prefix_form (W_k = W_0 + eta * P_k with
    P_k = sum_{j<k} Z_j^T V_j, [explainer] §2.3 associativity), evaluated with
    one running P instead of every chunk's S_j at once, so that a long
    sequence fits in memory: O_k = Z_k W_0 + eta * (Z_k P_k), then
    P_{k+1} = P_k + Z_k^T V_k. X, E: [L, d]; W_start: [F, d]. Calls
    on_chunk(s, e, O_k) for each chunk in order and returns W_final [F, d].
    """
    X, E, W0 = _f64(X), _f64(E), _f64(W_start)
    P = np.zeros(W0.shape, dtype=np.float64)
    for s, e in chunk_ranges(X.shape[0], B):
        Z = gate_up(X[s:e], W_g, W_u)
        V = target_chunk(E[s:e], conv_w, Proj)
        on_chunk(s, e, Z @ W0 + eta * (Z @ P))
        P += Z.T @ V
    return W0 + eta * P


def prefill_with_resets(X, E, W_g, W_u, conv_w, Proj, W_0, eta, B, doc_starts, update="linear",
                        W_start=None):
    """One sequence of packed documents, with the fast weight reset at each boundary.

    [explainer] §3.2: at a document boundary the fast weight goes back to its
    pretrained value, so documents do not leak into each other. Reading: the
    scan restarts at each document start p in `doc_starts` (token positions,
    p = 0 implied): W := W_0 and a new chunk begins at p, so chunks never span
    two documents and a chunk's conv pad (R2) stops at the document end too.
    X, E: [L, d]. Returns (O [L, d], W_final [F, d]).
    """
    X, E = _f64(X), _f64(E)
    L = X.shape[0]
    bounds = sorted({0, *[int(p) for p in doc_starts if 0 < int(p) < L]}) + [L]
    W = _f64(W_0 if W_start is None else W_start).copy()
    O = np.zeros_like(X)
    for i in range(len(bounds) - 1):
        a, b = bounds[i], bounds[i + 1]
        if i > 0:
            W = _f64(W_0).copy()
        O_doc, W_doc = prefill(X[None, a:b], E[None, a:b], W_g, W_u, conv_w, Proj, W, eta, B,
                               update=update)
        O[a:b] = O_doc[0]
        W = W_doc[0]
    return O, W


def final_weight_entries(X, E, W_g, W_u, conv_w, Proj, W_0, eta, B, rows, cols):
    """Linear update only: selected entries of W_final for ONE long sequence.

    By associativity W_final = W_0 + eta * sum_k Z_k^T V_k, so entry (f, c) needs
    only column f of Z and column c of V over all tokens: O(L d) per entry.
    Lets a test check a full-length run at sampled entries. X, E: [L, d];
    rows / cols: equal-length integer arrays of F- and d-indices.
    Returns an array of len(rows) values.
    """
    X, E = _f64(X), _f64(E)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    W_g, W_u = _f64(W_g), _f64(W_u)
    ur, inv_r = np.unique(rows, return_inverse=True)
    uc, inv_c = np.unique(cols, return_inverse=True)
    Zcols = silu(X @ W_g[:, ur]) * (X @ W_u[:, ur])            # [L, |ur|]
    L = X.shape[0]
    Vcols = np.zeros((L, len(uc)), dtype=np.float64)
    Proj = _f64(Proj)
    for s, e in chunk_ranges(L, B):
        Vcols[s:e] = conv_chunk(E[s:e], conv_w) @ Proj[:, uc]
    acc = np.einsum("ti,ti->i", Zcols[:, inv_r], Vcols[:, inv_c])
    return _f64(W_0)[rows, cols] + eta * acc


def decode_steps(X, E, W_g, W_u, conv_w, Proj, W, eta, B, buffered=0, update="linear"):
    """Token-at-a-time continuation of a scan, one sequence.

    Reading of the step after prefill (the fast weights keep changing during
    inference, [explainer] §6 closing remarks): a generated token is applied
    with the current W at once; tokens are buffered until B of them close a
    chunk, and that chunk then updates W exactly as prefill would. The result
    therefore equals prefill() over the same tokens when the buffer starts
    empty. `buffered` > 0 is not modelled here (the buffer is explicit in the
    inputs): X, E hold the tokens of this call, W is the weight at a chunk
    start. Returns (O [T, d], W_after [F, d]).
    """
    X, E = _f64(X), _f64(E)
    if buffered:
        raise ValueError("decode_steps models a call that starts on a chunk boundary")
    O, W_after = prefill(X[None], E[None], W_g, W_u, conv_w, Proj, W, eta, B, update=update)
    # A trailing partial chunk has been applied but its update is still pending:
    # undo nothing; decoding keeps the pending tokens for the next call. The
    # weight returned is the one after the last COMPLETE chunk.
    T = X.shape[0]
    full = (T // B) * B
    if full != T:
        _, W_after = prefill(X[None, :full], E[None, :full], W_g, W_u, conv_w, Proj, W, eta, B,
                             update=update)
    return O[0], W_after[0]


def silu_grad(a: np.ndarray) -> np.ndarray:
    """Derivative of SiLU: d/da [a sigmoid(a)] = sigmoid(a) (1 + a (1 - sigmoid(a)))."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def conv_chunk_backward(dC_chunk, E_chunk, conv_w):
    """Adjoint of conv_chunk for one chunk: given dL/dC, returns (dL/dE, dL/dconv_w).

    C[t, c] += conv_w[c, j] E[t + j, c] for t + j inside the chunk, so each tap
    sends dC[t] back to E[t + j] and collects dC[t] * E[t + j] for its weight.
    """
    dC_chunk, E_chunk, conv_w = _f64(dC_chunk), _f64(E_chunk), _f64(conv_w)
    T, d = E_chunk.shape
    dE = np.zeros((T, d), dtype=np.float64)
    dw = np.zeros(conv_w.shape, dtype=np.float64)
    for j in range(conv_w.shape[1]):
        if j >= T:
            break
        dE[j:] += conv_w[:, j][None, :] * dC_chunk[: T - j]
        dw[:, j] += (dC_chunk[: T - j] * E_chunk[j:]).sum(axis=0)
    return dE, dw


def backward(X, E, W_g, W_u, conv_w, Proj, W_start, eta, B, dO, dW_final=None, update="linear"):
    """Gradients through the scan of prefill() (RB1), for the scalar loss whose
    gradient with respect to O is dO and with respect to W_final is dW_final
    (None: zero).

    X, E, dO: [N, L, d]; W_start: [F, d] shared by the sequences or [N, F, d];
    dW_final: [N, F, d] or None. Returns a dict with dX, dE [N, L, d], dW_g,
    dW_u [d, F], dProj [d, d], dconv_w [d, Kc] (summed over sequences) and
    dW_start (shape of W_start; summed over sequences when shared).

    The forward is rerun chunk by chunk, keeping each chunk's W_k, then the
    chain rule runs over the chunks in reverse with G = dL/dW_{k+1}:
      linear  W_{k+1} = W_k + eta Z^T V:
        dZ_k = dO_k W_k^T + eta V_k G^T     dV_k = eta Z_k G     G <- G + Z_k^T dO_k
      mse     W_{k+1} = W_k - eta Z^T R,  R_k = Z_k W_k - V_k:
        dY_k = dO_k - eta Z_k G             (gradient reaching Z_k W_k)
        dZ_k = dY_k W_k^T - eta R_k G^T     dV_k = eta Z_k G     G <- G + Z_k^T dY_k
    and on to the slow weights: with A = X W_g, U = X W_u, Z = SiLU(A) U,
      dA = dZ U SiLU'(A), dU = dZ SiLU(A), dX = dA W_g^T + dU W_u^T,
      dW_g = X^T dA, dW_u = X^T dU, dC = dV Proj^T, dProj = C^T dV, and the
      conv's adjoint inside the chunk (conv_chunk_backward).
    After the first chunk G is dL/dW_0.
    """
    _check_update(update)
    X, E, dO = _f64(X), _f64(E), _f64(dO)
    W_g, W_u, conv_w, Proj = _f64(W_g), _f64(W_u), _f64(conv_w), _f64(Proj)
    W_start = _f64(W_start)
    N, L, d = X.shape
    F = W_start.shape[-2]
    out = dict(dX=np.zeros_like(X), dE=np.zeros_like(E), dW_g=np.zeros_like(W_g),
               dW_u=np.zeros_like(W_u), dProj=np.zeros_like(Proj), dconv_w=np.zeros_like(conv_w),
               dW_start=np.zeros_like(W_start))
    for n in range(N):
        W = (W_start[n] if W_start.ndim == 3 else W_start).copy()
        saved = []
        for s, e in chunk_ranges(L, B):
            A = X[n, s:e] @ W_g
            U = X[n, s:e] @ W_u
            Z = silu(A) * U
            C = conv_chunk(E[n, s:e], conv_w)
            V = C @ Proj
            saved.append((s, e, A, U, Z, C, V, W))
            if update == "linear":
                W = W + eta * (Z.T @ V)
            else:
                W = W - eta * (Z.T @ (Z @ W - V))
        G = np.zeros((F, d)) if dW_final is None else _f64(dW_final)[n].copy()
        for s, e, A, U, Z, C, V, Wk in reversed(saved):
            dOk = dO[n, s:e]
            if update == "linear":
                dZ = dOk @ Wk.T + eta * (V @ G.T)
                dV = eta * (Z @ G)
                G = G + Z.T @ dOk
            else:
                R = Z @ Wk - V
                dY = dOk - eta * (Z @ G)
                dZ = dY @ Wk.T - eta * (R @ G.T)
                dV = eta * (Z @ G)
                G = G + Z.T @ dY
            dA = dZ * U * silu_grad(A)
            dU = dZ * silu(A)
            out["dX"][n, s:e] = dA @ W_g.T + dU @ W_u.T
            out["dW_g"] += X[n, s:e].T @ dA
            out["dW_u"] += X[n, s:e].T @ dU
            dC = dV @ Proj.T
            out["dProj"] += C.T @ dV
            dEk, dwk = conv_chunk_backward(dC, E[n, s:e], conv_w)
            out["dE"][n, s:e] = dEk
            out["dconv_w"] += dwk
        if W_start.ndim == 3:
            out["dW_start"][n] = G
        else:
            out["dW_start"] += G
    return out


def initial_weight_grad_entries(X, W_g, W_u, dO, dW_final, rows, cols):
    """Linear rule only: selected entries of dL/dW_0 for ONE long sequence.

    With the linear update G_k = G_{k+1} + Z_k^T dO_k, so dL/dW_0 = dL/dW_final +
    sum over all tokens of z_t^T dO_t: entry (f, c) needs one column of Z and
    one of dO, O(L d) each. X, dO: [L, d]; dW_final: [F, d] or None; rows /
    cols: equal-length F- and d-indices. Returns len(rows) values.
    """
    X, dO = _f64(X), _f64(dO)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    W_g, W_u = _f64(W_g), _f64(W_u)
    ur, inv_r = np.unique(rows, return_inverse=True)
    Zcols = gate_up(X, W_g[:, ur], W_u[:, ur])          # [L, |ur|]
    acc = np.einsum("ti,ti->i", Zcols[:, inv_r], dO[:, cols])
    base = np.zeros(len(rows)) if dW_final is None else _f64(dW_final)[rows, cols]
    return base + acc

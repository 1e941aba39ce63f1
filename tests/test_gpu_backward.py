"""GPU parity of the backward through the scan (ipttt_backward_layer, through the
C ABI) against the float64 oracle's backward.

Bar: relative Frobenius error 2e-2 per gradient (bf16 operands, fp32
accumulation; the oracle works in float64 on the exact bf16 input values).
Covered: both update rules; small, 4B and 1.5B layer shapes; chunk sizes that are and are not
multiples of 64 with ragged last chunks; two sequences; with and without an
upstream gradient on the final fast weight. At the 32k workload's full size,
in one call: an upstream gradient confined to the first two chunks must give
the oracle's two-chunk gradients and exact zeros for later tokens, and with a
dense upstream gradient sampled entries of dL/dW_0 follow from associativity.
Bitwise: a second run repeats the first.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from chunked_weight_mlp_amd import ipttt as B
from parity_check import report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def make_layer(w, weights, n_seq):
    dev = {k: v.to(DEV) for k, v in weights.items()}
    return B.Layer(**dev, chunk=w.chunk, eta=w.eta, update=w.update, max_batch=n_seq)


def to_pages(g):
    """Library gradient buffers -> the oracle's orientation (float64 numpy)."""
    f = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    return dict(dX=f(g["dx"]), dE=f(g["de"]), dW_g=f(g["dw_gate"]).T, dW_u=f(g["dw_up"]).T,
                dProj=f(g["dproj"]).T, dconv_w=f(g["dconv_w"]), dW_start=f(g["dw0"]).T)


def oracle_backward(w, weights, x, e, d_o, d_wf):
    ow = wl.to_oracle(weights)
    dwf = None if d_wf is None else d_wf.double().numpy().transpose(0, 2, 1)
    return oracle.backward(x.double().numpy(), e.double().numpy(), ow["W_g"], ow["W_u"],
                           ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, w.chunk,
                           d_o.double().numpy(), dW_final=dwf, update=w.update)


def compare(got, ref, label, keys=None):
    worst = 0.0
    for k in keys or ref:
        err = rel(got[k], ref[k])
        report(f"[backward] {label} {k}: rel_fro {err:.3e}")
        assert np.isfinite(got[k]).all(), k
        assert err <= TOL, (k, err)
        worst = max(worst, err)
    return worst


SMALL = wl.Workload("bf16_d256_f640", 2, 256, 640, 1000, 128, "bf16", 1e-2, "linear")


@pytest.mark.parametrize("Bc,L,N,with_dwf", [
    (128, 1000, 2, True),    # ragged last chunk, two sequences, upstream dW_final
    (96, 777, 1, False),     # chunk not a multiple of 64: padding rows in every chunk
    (64, 300, 2, True),      # short chunks (small-tile configuration)
    (256, 512, 1, False),
    (1024, 2148, 1, True),   # full-height tiles and a 100-token last chunk
])
def test_backward_small_shapes(Bc, L, N, with_dwf):
    w = SMALL.replace(chunk=Bc, seq_len=L, n_seq=N)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    if not with_dwf:
        d_wf = None
    say(f"[backward] d={w.d} F={w.d_ff} B={Bc} L={L} N={N} dW_final={with_dwf}")
    layer = make_layer(w, weights, N)
    g = layer.backward(x.to(DEV), e.to(DEV), d_o.to(DEV), None if d_wf is None else d_wf.to(DEV))
    torch.cuda.synchronize()
    compare(to_pages(g), oracle_backward(w, weights, x, e, d_o, d_wf), f"B={Bc}")


@pytest.mark.parametrize("Kc,Bc,L,update", [
    (1, 64, 194, "linear"),   # one tap: no window at all
    (3, 2, 41, "linear"),     # chunks of 2 tokens, shorter than the filter
    (8, 5, 67, "mse"),        # 8 taps over 5-token chunks, 2-token tail
    (8, 64, 130, "linear"),   # 2-token tail
])
def test_backward_conv_taps(Kc, Bc, L, update):
    """Conv adjoint with 1, 3 and 8 taps, including chunks shorter than the filter."""
    w = SMALL.replace(chunk=Bc, seq_len=L, n_seq=1, conv_k=Kc, update=update,
                      eta=1e-2 if update == "linear" else 2e-3)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    say(f"[backward] taps={Kc} B={Bc} L={L} {update}")
    layer = make_layer(w, weights, 1)
    g = layer.backward(x.to(DEV), e.to(DEV), d_o.to(DEV), d_wf.to(DEV))
    torch.cuda.synchronize()
    compare(to_pages(g), oracle_backward(w, weights, x, e, d_o, d_wf), f"taps={Kc} B={Bc}")


@pytest.mark.parametrize("Bc,L,N,with_dwf", [
    (128, 700, 2, True),     # ragged last chunk, two sequences
    (96, 500, 1, False),     # padding rows in every chunk
    (512, 1100, 1, True),    # full-height tiles
    (64, 3000, 2, True),     # the recompute in two chunk groups (32 and 15 chunks)
])
def test_backward_mse_small_shapes(Bc, L, N, with_dwf):
    """MSE rule: the forward is recomputed over chunk groups (a copy of W kept per
    chunk), the reverse pass runs chunk by chunk (dY_j = dO_j - eta Z_j G_{j+1})."""
    w = SMALL.replace(chunk=Bc, seq_len=L, n_seq=N, update="mse", eta=2e-3)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    if not with_dwf:
        d_wf = None
    say(f"[backward] mse d={w.d} F={w.d_ff} B={Bc} L={L} N={N} dW_final={with_dwf}")
    layer = make_layer(w, weights, N)
    g = layer.backward(x.to(DEV), e.to(DEV), d_o.to(DEV), None if d_wf is None else d_wf.to(DEV))
    torch.cuda.synchronize()
    compare(to_pages(g), oracle_backward(w, weights, x, e, d_o, d_wf), f"mse B={Bc}")


@pytest.mark.parametrize("update", ["linear", "mse"])
def test_backward_partial_tiles(update):
    """d 320 and d_ff 576 (multiples of 64, not of 128 or 256): the last row and
    column tiles of every backward GEMM, transpose and scan are partial."""
    w = SMALL.replace(d=320, d_ff=576, chunk=128, seq_len=600, n_seq=2, update=update,
                      eta=1e-2 if update == "linear" else 2e-3)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    say(f"[backward] partial tiles {update} d={w.d} F={w.d_ff} B=128 L=600 N=2")
    layer = make_layer(w, weights, 2)
    g = layer.backward(x.to(DEV), e.to(DEV), d_o.to(DEV), d_wf.to(DEV))
    torch.cuda.synchronize()
    compare(to_pages(g), oracle_backward(w, weights, x, e, d_o, d_wf), f"partial {update}")


def test_backward_mse_1p5b_shape():
    """The 1.5B pretraining layer (d 2048, d_ff 8192, MSE rule): two sequences of
    three chunks of 512 and a tail."""
    w = wl.WORKLOADS["pretrain_1p5b_8x16k_B512_mse"].replace(seq_len=3 * 512 + 77, n_seq=2)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    layer = make_layer(w, weights, 2)
    g = layer.backward(x.to(DEV), e.to(DEV), d_o.to(DEV), d_wf.to(DEV))
    torch.cuda.synchronize()
    say("[backward] 1.5B MSE: oracle")
    compare(to_pages(g), oracle_backward(w, weights, x, e, d_o, d_wf), "1.5B mse")


def test_backward_4b_shape():
    """4B-shaped layer (d 2560, d_ff 9728), four chunks of 512."""
    w = wl.WORKLOADS["qwen3_4b_L32k_B512"].replace(seq_len=2048)
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    layer = make_layer(w, weights, 1)
    g = layer.backward(x.to(DEV), e.to(DEV), d_o.to(DEV), d_wf.to(DEV))
    torch.cuda.synchronize()
    say("[backward] 4B shape: oracle on 2048 tokens")
    compare(to_pages(g), oracle_backward(w, weights, x, e, d_o, d_wf), "4B L=2048")


def test_backward_full_size_32k():
    """The 32k / B = 512 workload in one call, the configuration the benchmark
    times. (1) dO confined to the first two chunks, no dW_final: the gradients
    are the oracle's for those two chunks (nothing later reaches them) and
    exact zeros for later tokens. (2) Dense dO and dW_final: sampled entries of
    dL/dW_0 = dL/dW_final + sum_t z_t^T dO_t (linear rule, associativity).
    (3) A second run repeats the first bit for bit."""
    w = wl.WORKLOADS["qwen3_4b_L32k_B512"]
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, d_wf = wl.make_upstream(w)
    layer = make_layer(w, weights, 1)
    xd, ed = x.to(DEV), e.to(DEV)
    t2 = 2 * w.chunk
    d_o2 = torch.zeros_like(d_o)
    d_o2[:, :t2] = d_o[:, :t2]
    say("[backward] 32k: GPU run with dO on the first two chunks")
    g = layer.backward(xd, ed, d_o2.to(DEV), None)
    torch.cuda.synchronize()
    got = to_pages(g)
    for k in ("dX", "dE"):
        assert np.abs(got[k][:, t2:]).max() == 0.0, k
        got[k] = got[k][:, :t2]
    say("[backward] 32k: oracle on the first two chunks")
    ref = oracle_backward(w, weights, x[:, :t2], e[:, :t2], d_o[:, :t2], None)
    compare(got, ref, "32k first two chunks")

    say("[backward] 32k: dense dO, dW_final")
    g1 = {k: v.clone() for k, v in layer.backward(xd, ed, d_o.to(DEV), d_wf.to(DEV)).items()}
    g2 = layer.backward(xd, ed, d_o.to(DEV), d_wf.to(DEV))
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    r = np.random.default_rng(7)
    rows, cols = r.integers(0, w.d_ff, 48), r.integers(0, w.d, 48)
    ow = wl.to_oracle(weights)
    ref_e = oracle.initial_weight_grad_entries(x[0].double().numpy(), ow["W_g"], ow["W_u"],
                                               d_o[0].double().numpy(),
                                               d_wf[0].double().numpy().T, rows, cols)
    got_e = g1["dw0"].double().cpu().numpy()[cols, rows]
    err = rel(got_e, ref_e)
    report(f"[backward] 32k: sampled dW_0 rel err {err:.3e}")
    assert err <= TOL
    for k in ("dx", "de", "dw_gate", "dw_up", "dproj", "dconv_w"):
        assert torch.isfinite(g1[k]).all(), k


def test_backward_full_size_pretrain_mse():
    """The 8 x 16k / B = 512 MSE workload in one call. With dO confined to the
    first two chunks of each sequence and no dW_final, G stays zero past them,
    so the gradients equal the oracle's two-chunk backward and are exactly zero
    for later tokens."""
    w = wl.WORKLOADS["pretrain_1p5b_8x16k_B512_mse"]
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    d_o, _ = wl.make_upstream(w)
    t2 = 2 * w.chunk
    d_o2 = torch.zeros_like(d_o)
    d_o2[:, :t2] = d_o[:, :t2]
    layer = make_layer(w, weights, w.n_seq)
    say("[backward] 8x16k MSE: GPU run")
    g = layer.backward(x.to(DEV), e.to(DEV), d_o2.to(DEV), None)
    torch.cuda.synchronize()
    got = to_pages(g)
    for k in ("dX", "dE"):
        assert np.abs(got[k][:, t2:]).max() == 0.0, k
        got[k] = got[k][:, :t2]
    say("[backward] 8x16k MSE: oracle on the first two chunks of 8 sequences")
    ref = oracle_backward(w, weights, x[:, :t2], e[:, :t2], d_o[:, :t2], None)
    compare(got, ref, "8x16k mse first two chunks")

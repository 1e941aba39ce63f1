"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the whole sequence in one pass of the update scan).

The oracle cannot scan 128k tokens of a 4B-shaped layer in seconds, so it
checks what it can compute one by one:
  - O on the first chunks, two or, at small chunk sizes, one chunk group
    and two more (the oracle scans just those chunks; the HIP path's later
    chunks cannot change them, by causality);
  - sampled entries of the final fast weight (linear rule): by associativity
    W_final[f, c] = W_0[f, c] + eta sum_t Z[t, f] V[t, c] needs one column of
    Z and one of V, O(L d) each;
and properties that hold at any size: a run split into several passes over
the sequence equals the one-pass run bit for bit, and so does a second run.
Bar: relative Frobenius error 2e-2 (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from chunked_weight_mlp_amd import ipttt as B

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda:0"
TOL = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def run_full(w, weights, x, e, slab_chunks):
    dev = {k: v.to(DEV) for k, v in weights.items()}
    layer = B.Layer(**dev, chunk=w.chunk, eta=w.eta, update=w.update, max_batch=w.n_seq,
                    slab_chunks=slab_chunks)
    layer.reset()
    o = layer.prefill(x.to(DEV), e.to(DEV))
    torch.cuda.synchronize()
    ws = layer.w_state.clone()
    layer.close()
    del layer
    return o, ws


@pytest.mark.parametrize("name", ["qwen3_4b_L128k_B1024", "qwen3_4b_L32k_B512",
                                  "pretrain_1p5b_8x16k_B512_mse"])
def test_full_size(name):
    w = wl.WORKLOADS[name]
    say(f"[full] {name}: generating inputs")
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    say(f"[full] {name}: one-pass GPU run ({w.n_chunks} chunks)")
    o, ws = run_full(w, weights, x, e, w.n_chunks)
    assert torch.isfinite(o).all()
    ow = wl.to_oracle(weights)

    # first chunks of every sequence: two, plus one default chunk group
    # (about 1024 padded rows) for the linear rule
    group = max(1, 1024 // (-(-w.chunk // 64) * 64)) if w.update == "linear" else 0
    t2 = min(w.seq_len, (group + 2) * w.chunk)
    say(f"[full] {name}: oracle on the first {t2} tokens of {w.n_seq} sequence(s)")
    O2, _ = oracle.prefill(x[:, :t2].double().numpy(), e[:, :t2].double().numpy(), ow["W_g"], ow["W_u"],
                           ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, w.chunk, update=w.update)
    err_o = rel(o[:, :t2].double().cpu().numpy(), O2)
    say(f"[full] {name}: first-chunks rel_fro O = {err_o:.3e}")
    assert err_o <= TOL

    # sampled final-weight entries (linear rule), sequence 0
    if w.update == "linear":
        r = np.random.default_rng(5)
        rows = r.integers(0, w.d_ff, 48)
        cols = r.integers(0, w.d, 48)
        say(f"[full] {name}: oracle on 48 sampled final-weight entries")
        ref = oracle.final_weight_entries(x[0].double().numpy(), e[0].double().numpy(), ow["W_g"],
                                          ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"], w.eta,
                                          w.chunk, rows, cols)
        got = ws[0].double().cpu().numpy()[cols, rows]   # stored transposed: [d][d_ff]
        err_w = rel(got, ref)
        drift = rel(ow["W_0"][rows, cols], ref)
        say(f"[full] {name}: sampled W rel err = {err_w:.3e} (W_0 alone would be {drift:.2f})")
        assert err_w <= TOL

    # several passes over the sequence == one pass, bit for bit
    slab = max(1, w.n_chunks // 3)
    say(f"[full] {name}: multi-pass run ({slab} chunks per pass)")
    o2, ws2 = run_full(w, weights, x, e, slab)
    assert torch.equal(o2, o)
    assert torch.equal(ws2, ws)


@pytest.mark.parametrize("Bc", [64, 256, 512, 1024, 4096])
def test_chunk_sweep_full_size(Bc):
    """4B-shaped layer at L = 65536 and each chunk size: the first chunks (past
    the first chunk group) and sampled final-weight entries against the oracle
    (the prefix-sum form)."""
    w = wl.WORKLOADS[f"qwen3_4b_L64k_B{Bc}"]
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    slab = min(w.n_chunks, 256)  # B = 64: 1024 chunks in four passes
    say(f"[sweep-full] B={Bc}: GPU run, {slab} chunks per pass")
    o, ws = run_full(w, weights, x, e, slab)
    ow = wl.to_oracle(weights)
    # the default chunk group (about 1024 padded rows) plus two chunks: covers
    # the Gram term inside the first group and the second group's snapshot
    group = max(1, 1024 // (-(-Bc // 64) * 64))
    t2 = min(w.seq_len, (group + 2) * Bc)
    Op, _ = oracle.prefill_prefix_form(x[:, :t2].double().numpy(), e[:, :t2].double().numpy(),
                                       ow["W_g"], ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"],
                                       w.eta, Bc)
    err_o = rel(o[:, :t2].double().cpu().numpy(), Op)
    r = np.random.default_rng(6)
    rows, cols = r.integers(0, w.d_ff, 32), r.integers(0, w.d, 32)
    ref = oracle.final_weight_entries(x[0].double().numpy(), e[0].double().numpy(), ow["W_g"],
                                      ow["W_u"], ow["conv_w"], ow["Proj"], ow["W_0"], w.eta, Bc,
                                      rows, cols)
    err_w = rel(ws[0].double().cpu().numpy()[cols, rows], ref)
    say(f"[sweep-full] B={Bc}: rel O(first chunks)={err_o:.3e} W(sampled)={err_w:.3e}")
    assert err_o <= TOL and err_w <= TOL

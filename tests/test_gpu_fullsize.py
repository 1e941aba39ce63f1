"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the whole sequence in one pass of the update scan).

The oracle streams each sequence chunk by chunk, carrying W from one chunk to
the next (a continuation, pinned in the oracle tests), so host memory stays at
one chunk and one fast weight. Every chunk's O of every sequence is compared
with the oracle's on its own (relative Frobenius error), and so is the whole
final fast weight of every sequence, under both update rules. The explainer
page's §3.2 (the chunked algorithm equals the serial chunk loop) and §2.2
(apply, then update, per chunk) are what this checks at the lengths the
benchmark runs. The chunk-size sweep streams the prefix-sum form instead
(W_k = W_0 + eta * sum_{j<k} Z_j^T V_j), the form the chunk-parallel scan
evaluates.

Also at full size: a run split into several passes over the sequence equals
the one-pass run bit for bit. The longest case (256k tokens of the 4B-shaped
layer) puts more than 2^31 elements in each sequence's Zt and its chunk copies
of W, so every offset into them must be 64-bit.
Bar: relative Frobenius error 2e-2 per chunk (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from chunked_weight_mlp_amd import ipttt as B
from parity_check import ChunkErrors, check_weights, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda:0"
TOL = 2e-2


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


def stream_scan(w, ow, x, e, o_cpu, label):
    """The oracle's chunk scan over every sequence, chunk by chunk, each chunk's
    O checked as it comes; returns the final W of every sequence [N, F, d]."""
    ce = ChunkErrors(label)
    W_fin = []
    t0 = time.perf_counter()
    for n in range(w.n_seq):
        W = ow["W_0"]
        for k, (s, t) in enumerate(oracle.chunk_ranges(w.seq_len, w.chunk)):
            O_k, W_next = oracle.prefill(x[n:n + 1, s:t].double().numpy(),
                                         e[n:n + 1, s:t].double().numpy(), ow["W_g"], ow["W_u"],
                                         ow["conv_w"], ow["Proj"], W, w.eta, w.chunk,
                                         update=w.update)
            W = W_next[0]
            ce.add(n, k, s, o_cpu[n, s:t].double().numpy(), O_k[0])
        W_fin.append(W)
        say(f"[{label}] oracle: sequence {n} done ({time.perf_counter() - t0:.0f} s)")
    ce.check(TOL)
    return np.stack(W_fin)


@pytest.mark.parametrize("name", ["qwen3_4b_L128k_B1024", "qwen3_4b_L32k_B512",
                                  "pretrain_1p5b_8x16k_B512_mse", "qwen3_4b_L256k_B1024",
                                  "qwen3_4b_L32k_B512_mse"])
def test_full_size(name):
    w = wl.WORKLOADS[name]
    say(f"[full] {name}: generating inputs")
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    say(f"[full] {name}: one-pass GPU run ({w.n_chunks} chunks x {w.n_seq} sequence(s))")
    o, ws = run_full(w, weights, x, e, w.n_chunks)
    assert torch.isfinite(o).all()
    o_cpu = o.cpu()
    ow = wl.to_oracle(weights)
    say(f"[full] {name}: streaming the oracle over every chunk of every sequence")
    W_ref = stream_scan(w, ow, x, e, o_cpu, f"full {name}")
    W_gpu = ws.double().cpu().numpy().transpose(0, 2, 1)   # stored [n][d][d_ff]
    check_weights(W_gpu, W_ref, TOL, f"full {name}")
    drift = float(np.linalg.norm(W_ref[0] - ow["W_0"]) / np.linalg.norm(W_ref[0]))
    say(f"[full] {name}: the updates carry {drift:.2f} of the final weight's norm")

    # several passes over the sequence == one pass, bit for bit
    slab = max(1, w.n_chunks // 3)
    say(f"[full] {name}: multi-pass run ({slab} chunks per pass)")
    o2, ws2 = run_full(w, weights, x, e, slab)
    assert torch.equal(o2, o)
    assert torch.equal(ws2, ws)


@pytest.mark.parametrize("Bc", [64, 256, 512, 1024, 4096])
def test_chunk_sweep_full_size(Bc):
    """4B-shaped layer at L = 65536 and each chunk size: every chunk's O and the
    whole final weight against the oracle's prefix-sum form, streamed."""
    w = wl.WORKLOADS[f"qwen3_4b_L64k_B{Bc}"]
    weights = wl.make_weights(w)
    x, e = wl.make_inputs(w)
    slab = min(w.n_chunks, 256)  # B = 64: 1024 chunks in four passes
    say(f"[sweep-full] B={Bc}: GPU run, {slab} chunks per pass")
    o, ws = run_full(w, weights, x, e, slab)
    o_cpu = o.cpu()
    ow = wl.to_oracle(weights)
    ce = ChunkErrors(f"sweep-full B={Bc}")
    counter = iter(range(w.n_chunks))

    def on_chunk(s, t, O_k):
        ce.add(0, next(counter), s, o_cpu[0, s:t].double().numpy(), O_k)

    t0 = time.perf_counter()
    W_ref = oracle.prefill_prefix_form_stream(x[0].double().numpy(), e[0].double().numpy(),
                                              ow["W_g"], ow["W_u"], ow["conv_w"], ow["Proj"],
                                              ow["W_0"], w.eta, Bc, on_chunk)
    say(f"[sweep-full] B={Bc}: oracle {time.perf_counter() - t0:.0f} s")
    ce.check(TOL)
    check_weights(ws.double().cpu().numpy().transpose(0, 2, 1), W_ref[None], TOL,
                  f"sweep-full B={Bc}")

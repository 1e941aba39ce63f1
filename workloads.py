"""Seeded synthetic workloads for the fast-weight prefill.

This module only draws random numbers: it holds none of the method's
arithmetic, so both the HIP path and the float64 oracle can be fed from it.

Shapes follow the pages' settings: a Qwen3-4B-shaped MLP layer (d = 2560,
d_ff = 9728) at 32k / 64k / 128k context and chunk sizes 64 .. 4096, and a
1.5B-scale pretraining-shaped layer (d = 2048, d_ff = 8192) with 8 sequences of
16k. No dataset or trained weight is used; values are Gaussian:
  X, E                 ~ N(0, 1)
  W_g, W_u, Proj       ~ N(0, 1/d)       (fan-in d)
  W_0                  ~ N(0, 1/d_ff)    (fan-in d_ff)
  conv_w               ~ N(0, 1/Kc)      (fan-in Kc = 4)
Each tensor has its own torch CPU generator seed (X 17, E 18, W_g 19, W_u 20,
Proj 21, conv 22, W_0 23), the same for every chunk size. Values are drawn in
fp32 and rounded to nearest-even bf16 where the workload is bf16; the oracle
receives exactly those values widened to float64.

Storage layout (what the C library takes): every weight matrix is stored
output-major, row r holding the weights that produce output feature r (the
nn.Linear convention). In the pages' row-vector notation the stored array is
the transpose of the matrix written there:
  w_gate, w_up  [d_ff, d]  = W_g^T, W_u^T
  proj          [d, d]     = Proj^T          (V = C @ Proj)
  w0            [d, d_ff]  = W_0^T           (fast weight W_o^T, fp32)
  conv_w        [d, Kc]    tap j of channel c reads token t + j
"""
from __future__ import annotations

import dataclasses

import torch

SEEDS = dict(x=17, e=18, w_gate=19, w_up=20, proj=21, conv=22, w0=23, d_o=24, d_wfinal=25)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    d: int
    d_ff: int
    seq_len: int
    chunk: int
    dtype: str          # "f32" or "bf16": X, E, W_g, W_u, Proj, conv_w
    eta: float
    update: str         # "linear" or "mse"
    conv_k: int = 4

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk)

    def flops_per_token(self) -> int:
        """Algorithmic FLOPs per token: gate/up 4dF, conv 2*Kc*d, Proj 2d^2,
        apply 2dF, update 2dF (the MSE residual adds d, ignored)."""
        d, F = self.d, self.d_ff
        return 8 * d * F + 2 * d * d + 2 * self.conv_k * d

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(name, n, d, F, L, B, dtype, eta, update):
    return Workload(name, n, d, F, L, B, dtype, eta, update)


WORKLOADS = {
    w.name: w
    for w in [
        _w("tiny_d64_f256_L1024_B128_fp32", 1, 64, 256, 1024, 128, "f32", 1e-2, "linear"),
        _w("qwen3_4b_L32k_B512", 1, 2560, 9728, 32768, 512, "bf16", 1e-3, "linear"),
        _w("qwen3_4b_L128k_B1024", 1, 2560, 9728, 131072, 1024, "bf16", 1e-3, "linear"),
        _w("pretrain_1p5b_8x16k_B512_mse", 8, 2048, 8192, 16384, 512, "bf16", 1e-4, "mse"),
        # the longest parity case: d_ff x L (Zt elements per sequence) exceeds 2^31
        _w("qwen3_4b_L256k_B1024", 1, 2560, 9728, 262144, 1024, "bf16", 1e-3, "linear"),
        # parity case: the MSE rule on the 4B-shaped layer, one sequence
        _w("qwen3_4b_L32k_B512_mse", 1, 2560, 9728, 32768, 512, "bf16", 1e-4, "mse"),
    ]
    + [
        _w(f"qwen3_4b_L64k_B{B}", 1, 2560, 9728, 65536, B, "bf16", 1e-3, "linear")
        for B in (64, 256, 512, 1024, 4096)
    ]
}

HEADLINE = "qwen3_4b_L128k_B1024"


def _randn(shape, seed, std, dtype, device="cpu"):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device) if device != "cpu" else t


def make_weights(w: Workload, device="cpu", seed_offset=0):
    """Slow weights, conv, projection and W_0 in the storage layout above."""
    d, F, Kc = w.d, w.d_ff, w.conv_k
    so = seed_offset
    return dict(
        w_gate=_randn((F, d), SEEDS["w_gate"] + so, d ** -0.5, w.dtype, device),
        w_up=_randn((F, d), SEEDS["w_up"] + so, d ** -0.5, w.dtype, device),
        proj=_randn((d, d), SEEDS["proj"] + so, d ** -0.5, w.dtype, device),
        conv_w=_randn((d, Kc), SEEDS["conv"] + so, Kc ** -0.5, w.dtype, device),
        w0=_randn((d, F), SEEDS["w0"] + so, F ** -0.5, "f32", device),
    )


def make_inputs(w: Workload, device="cpu", seq_len=None, n_seq=None, seed_offset=0):
    """X and E, [n_seq, seq_len, d], drawn as one block per tensor."""
    L = w.seq_len if seq_len is None else seq_len
    N = w.n_seq if n_seq is None else n_seq
    so = seed_offset
    x = _randn((N, L, w.d), SEEDS["x"] + so, 1.0, w.dtype, device)
    e = _randn((N, L, w.d), SEEDS["e"] + so, 1.0, w.dtype, device)
    return x, e


def make_upstream(w: Workload, device="cpu", seq_len=None, n_seq=None, seed_offset=0,
                  wfinal_scale=0.1):
    """Upstream gradients for the backward: dL/dO [n_seq, seq_len, d] ~ N(0, 1)
    and dL/dW_final [n_seq, d, d_ff] ~ N(0, wfinal_scale^2) in the state layout,
    both fp32."""
    L = w.seq_len if seq_len is None else seq_len
    N = w.n_seq if n_seq is None else n_seq
    so = seed_offset
    d_o = _randn((N, L, w.d), SEEDS["d_o"] + so, 1.0, "f32", device)
    d_wf = _randn((N, w.d, w.d_ff), SEEDS["d_wfinal"] + so, wfinal_scale, "f32", device)
    return d_o, d_wf


def to_oracle(weights: dict):
    """The same values in the pages' orientation, float64 numpy (transposes only)."""
    f = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    return dict(
        W_g=f(weights["w_gate"]).T,
        W_u=f(weights["w_up"]).T,
        Proj=f(weights["proj"]).T,
        conv_w=f(weights["conv_w"]),
        W_0=f(weights["w0"]).T,
    )

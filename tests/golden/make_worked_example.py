"""Write worked_example_d2_F3.json: a hand-sized prefill worked chunk by chunk.

The pages print no numeric example of the method, so this file holds one of a
size a reader can follow on paper: d = 2, d_ff = 3, a 2-tap target conv, five
tokens in chunks of 2 (the last chunk short), eta = 1/2, all inputs dyadic
(exact in bfloat16). For each update rule it stores every chunk's Z, V, O and
the fast weight after the chunk. Steps, as the pages define them:
  Z = SiLU(X W_g) * (X W_u)                  explainer page §2.1
  V = Conv(E) Proj, conv zero past the chunk explainer page §2.3
  O_k = Z_k W_k, then W_{k+1} from chunk k   explainer page §2.2, Fig. 1
  linear: W + eta Z^T V                      explainer page §2.3
  MSE:    W - eta Z^T (Z W - V)              analysis page, 第二板斧

Every value comes from the oracle (this script calls nothing else). The test
that reads the file checks the numbers against scalar loops that do not use
the oracle, and checks that the oracle still reproduces them.

Run from the repository root: python tests/golden/make_worked_example.py
"""
from __future__ import annotations

import json
import os
import re
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))
from oracle import ipttt_oracle as orc  # noqa: E402

INPUTS = {
    "X": [[1.0, -0.75], [0.5, 2.0], [-1.0, 1.5], [2.0, 0.25], [-0.75, -1.0]],
    "E": [[0.75, 1.0], [-1.0, 0.5], [1.5, -0.5], [0.0, 2.0], [1.0, 1.0]],
    "W_g": [[0.5, -1.0, 0.25], [1.0, 0.5, -0.5]],
    "W_u": [[1.0, 0.25, -0.5], [-0.5, 1.0, 0.75]],
    "conv_w": [[1.0, 0.5], [0.25, -1.0]],
    "Proj": [[0.5, 0.25], [-0.25, 1.0]],
    "W_0": [[0.25, -0.5], [0.5, 0.125], [-0.25, 0.75]],
}
ETA, CHUNK = 0.5, 2


def worked(update: str) -> dict:
    a = {k: np.array(v, dtype=np.float64) for k, v in INPUTS.items()}
    X, E = a["X"][None], a["E"][None]
    chunks = []
    for s, e in orc.chunk_ranges(len(a["X"]), CHUNK):
        O, W_after = orc.prefill(X[:, :e], E[:, :e], a["W_g"], a["W_u"], a["conv_w"], a["Proj"],
                                 a["W_0"][None], ETA, CHUNK, update=update)
        chunks.append({
            "tokens": [s, e],
            "Z": orc.gate_up(a["X"][s:e], a["W_g"], a["W_u"]).tolist(),
            "V": orc.target_chunk(a["E"][s:e], a["conv_w"], a["Proj"]).tolist(),
            "O": O[0, s:e].tolist(),
            "W_after": W_after[0].tolist(),
        })
    return {"chunks": chunks}


def main() -> None:
    out = {
        "description": "hand-sized In-Place TTT prefill, one sequence, worked chunk by chunk",
        "source": ("steps: explainer page 'In-Place Test-Time Training：让大语言模型在推理时原地进化，"
                   "长上下文任务准确率显著提升' §2.1-§2.3 and Fig. 1; MSE rule: analysis page "
                   "'大模型长文本核心架构全解析（非常详细），搞懂“边读边学”看这篇就够了！' 第二板斧. "
                   "The pages print no numeric example: the numbers were computed by the oracle "
                   "(tests/golden/make_worked_example.py)."),
        "eta": ETA,
        "chunk": CHUNK,
        "inputs": INPUTS,
        "linear": worked("linear"),
        "mse": worked("mse"),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_example_d2_F3.json")
    text = json.dumps(out, indent=1, ensure_ascii=False)
    # one line per innermost list of numbers (a matrix row)
    text = re.sub(r"\[\s+([-+0-9.eE,\s]+?)\s+\]", lambda m: "[" + " ".join(m.group(1).split()) + "]",
                  text)
    with open(path, "w", encoding="utf-8") as fh:
        fh.write(text + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

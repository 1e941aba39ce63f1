"""Chunk-by-chunk comparison of the HIP path's outputs with the oracle's.

A single relative Frobenius error over a whole sequence is dominated by the
late chunks (their outputs carry the accumulated update), so an error confined
to early chunks or to a few tiles could hide under it. Every check here is per
(sequence, chunk): relative Frobenius error of that chunk's O against the
oracle's, each held to the bar on its own. Helpers only; no tests here.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle


# every check's summary line, printed again in pytest's terminal summary
# (tests/conftest.py), where captured output does not hide it
REPORT: list = []


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def report(line: str) -> None:
    REPORT.append(line)
    say(line)


def rel_fro(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


class ChunkErrors:
    """Collects per-(sequence, chunk) errors of O and reports the worst."""

    def __init__(self, label: str):
        self.label = label
        self.rows = []   # (seq, chunk, first token, rel_fro, max abs err)

    def add(self, n: int, k: int, s: int, got, ref) -> None:
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        self.rows.append((n, k, s, rel_fro(got, ref), float(np.max(np.abs(got - ref))) if got.size else 0.0))

    def add_sequence(self, n: int, got, ref, B: int) -> None:
        """All chunks of one sequence; got, ref: [L, d]."""
        for k, (s, e) in enumerate(oracle.chunk_ranges(ref.shape[0], B)):
            self.add(n, k, s, got[s:e], ref[s:e])

    def worst(self):
        return max(self.rows, key=lambda r: r[3])

    def check(self, tol: float) -> float:
        assert self.rows, "no chunks compared"
        n, k, s, err, _ = self.worst()
        mx = max(r[4] for r in self.rows)
        mean = float(np.mean([r[3] for r in self.rows]))
        report(f"[{self.label}] {len(self.rows)} chunks: worst rel_fro O = {err:.3e} (sequence {n}, "
               f"chunk {k}, tokens from {s}), mean {mean:.3e}, max |dO| = {mx:.3e} (tol {tol:.0e})")
        bad = [r for r in self.rows if not (r[3] <= tol)]
        assert not bad, f"{len(bad)} chunks above {tol}: first {bad[0]}"
        return err


def check_chunks(o, O_ref, B: int, tol: float, label: str) -> float:
    """o, O_ref: [N, L, d]. Asserts every chunk of every sequence within tol."""
    ce = ChunkErrors(label)
    for n in range(O_ref.shape[0]):
        ce.add_sequence(n, o[n], O_ref[n], B)
    return ce.check(tol)


def check_weights(W_gpu, W_ref, tol: float, label: str) -> float:
    """Final fast weights [N, F, d] (pages' orientation): every sequence within tol."""
    errs = [rel_fro(W_gpu[n], W_ref[n]) for n in range(W_ref.shape[0])]
    worst = int(np.argmax(errs))
    report(f"[{label}] final W: worst rel_fro {errs[worst]:.3e} (sequence {worst}) over {len(errs)} "
           f"sequence(s), max |dW| = {float(np.max(np.abs(np.asarray(W_gpu) - W_ref))):.3e}")
    assert all(e <= tol for e in errs), errs
    return errs[worst]

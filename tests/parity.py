"""Comparison helpers for GPU-vs-oracle parity (imported by the GPU tests).

Acceptance rules:
* block scores: |gpu - oracle| <= 1e-5 * max(1, |oracle|) on visible blocks,
  -inf past each query's last block;
* selection: the same set as the oracle, except that a block whose oracle
  score lies within 1e-4 (relative) of the k-th selected score may swap with
  another such block; the list is ascending, -1 padded, |S| equal;
* attention output, compared with the oracle's attention over the GPU's own
  selection: bf16 outputs max abs <= 2e-2 and mean abs <= 2e-3, float32
  outputs max abs <= 1e-4; lse within 1e-3 (bf16 inputs) or 1e-4 (float32).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

SCORE_RTOL = 1e-5
TIE_BAND = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-4


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def check_scores(gpu: np.ndarray, ora: np.ndarray, rows=None):
    """gpu/ora [T, Hidx, MB]."""
    fin = np.isfinite(ora)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ora)), "masked blocks differ"
    d = np.abs(gpu[fin] - ora[fin])
    lim = SCORE_RTOL * np.maximum(1.0, np.abs(ora[fin]))
    bad = d > lim
    assert not bad.any(), f"{bad.sum()} scores off; worst {d.max():.3g}"


def kth_score(scores_row, sel_row, forced):
    chosen = [j for j in sel_row if j not in forced]
    if not chosen:
        return None
    return min(scores_row[j] for j in chosen)


def check_selection(gpu_sel, gpu_cnt, ora_scores, ora_sel, ora_cnt, positions, init, local,
                    rows=None, abs_band=0.0):
    """Selections [T, Hidx, Kmax] / counts [T, Hidx]; positions: list of (b, p).
    abs_band widens the tie band to an absolute floor (scores near zero, whose
    own tolerance is absolute)."""
    T, H, K = ora_sel.shape
    n_band = 0
    rows = range(T) if rows is None else rows
    for t in rows:
        p = positions[t][1]
        nb = oracle.num_visible_blocks(p)
        F = set(oracle.forced_blocks(nb, init, local))
        for h in range(H):
            c = int(ora_cnt[t, h])
            assert int(gpu_cnt[t, h]) == c, f"count row {t},{h}: {gpu_cnt[t, h]} vs {c}"
            g = [int(x) for x in gpu_sel[t, h, :c]]
            assert all(x == -1 for x in gpu_sel[t, h, c:]), f"padding row {t},{h}"
            assert g == sorted(set(g)), f"not ascending/unique row {t},{h}: {g}"
            assert all(0 <= x < nb for x in g), f"out of range row {t},{h}"
            assert F <= set(g), f"forced block missing row {t},{h}"
            o = [int(x) for x in ora_sel[t, h, :c]]
            diff = set(g) ^ set(o)
            if diff:
                s = ora_scores[t, h]
                sk = kth_score(s, o, F)
                assert sk is not None
                lim = max(TIE_BAND * max(abs(sk), 1e-30), abs_band)
                for j in diff:
                    assert abs(s[j] - sk) <= lim, (
                        f"row {t},{h}: block {j} score {s[j]!r} vs k-th {sk!r}")
                n_band += 1
    return n_band


def check_output(gpu_out: np.ndarray, ora_out: np.ndarray, f32: bool):
    d = np.abs(gpu_out - ora_out)
    assert np.isfinite(gpu_out).all(), "non-finite output"
    if f32:
        assert d.max() <= F32_MAX, f"f32 max abs {d.max():.3g}"
    else:
        assert d.max() <= BF16_MAX, f"bf16 max abs {d.max():.3g}"
        assert d.mean() <= BF16_MEAN, f"bf16 mean abs {d.mean():.3g}"
    return float(d.max()), float(d.mean())


def check_lse(gpu_lse: np.ndarray, ora_lse: np.ndarray, f32: bool):
    assert np.array_equal(np.isneginf(gpu_lse), np.isneginf(ora_lse))
    fin = np.isfinite(ora_lse)
    d = np.abs(gpu_lse[fin] - ora_lse[fin])
    tol = 1e-4 if f32 else 1e-3
    assert d.size == 0 or d.max() <= tol, f"lse max abs {d.max():.3g}"

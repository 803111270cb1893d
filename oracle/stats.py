"""Statistics the benchmark pages report, computed from oracle outputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P2] section "MSE-Only vs QJL：bias 差異確認": a signed mean score error per
bit width; the pages give neither the pair count nor the exact statistic, so
both the signed mean and the multiplicative shrinkage are provided.
[P2] section "Needle-in-Haystack（Synthetic）": argmax of the estimated scores
must hit the planted key.
[P2] section "Lloyd-Max Codebook": distortion per coordinate, measured here as
the mean squared difference between rotated coordinates and their centroids.
"""
from __future__ import annotations

import numpy as np


def bias_signed(est: np.ndarray, exact: np.ndarray) -> float:
    """mean(est - exact) over pairs."""
    return float(np.mean(np.asarray(est) - np.asarray(exact)))


def bias_mult(est: np.ndarray, exact: np.ndarray) -> float:
    """1 - sum(est * exact) / sum(exact^2): the systematic shrinkage."""
    est = np.asarray(est, np.float64)
    exact = np.asarray(exact, np.float64)
    return float(1.0 - np.sum(est * exact) / np.sum(exact * exact))


def bias_mult_se(est: np.ndarray, exact: np.ndarray) -> float:
    """Delta-method standard error of bias_mult for independent pairs."""
    est = np.asarray(est, np.float64)
    exact = np.asarray(exact, np.float64)
    s2 = np.sum(exact * exact)
    b = np.sum(est * exact) / s2
    resid = exact * (est - b * exact)
    return float(np.sqrt(np.sum(resid * resid)) / s2)


def needle_hit(scores: np.ndarray, position: int) -> bool:
    """argmax (lowest index on ties) equals the needle position."""
    return int(np.argmax(scores)) == int(position)


def distortion_per_coord(y: np.ndarray, yhat: np.ndarray) -> float:
    """mean (y_i - c_i)^2 over all coordinates of all vectors."""
    return float(np.mean((np.asarray(y) - np.asarray(yhat)) ** 2))

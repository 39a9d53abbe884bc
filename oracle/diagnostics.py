"""Selector diagnostics of the oracle — TEST INFRASTRUCTURE ONLY.

Plain numpy definitions from "4.1.1 · 监督与联合训练" (selector supervision):
set recall R@k (eq. 2), teacher-mass coverage C (eq. 3) and the relative output
error E (eq. 14). Positions are 0-based here; the page numbers them from 1.
"""
from __future__ import annotations

from typing import Iterable

import numpy as np


def teacher_topk(p: np.ndarray, k: int) -> np.ndarray:
    """G = TopK(p, k): the k positions of largest teacher probability (lower index on ties)."""
    p = np.asarray(p, dtype=np.float64)
    order = sorted(range(p.shape[0]), key=lambda j: (-p[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def set_recall(selected: Iterable[int], p: np.ndarray, k: int) -> float:
    """eq. (2): |S ∩ G| / |G| with G the teacher's top-k."""
    G = set(teacher_topk(p, k).tolist())
    S = set(int(s) for s in selected)
    return len(S & G) / len(G)


def coverage(selected: Iterable[int], p: np.ndarray) -> float:
    """eq. (3): teacher probability mass on the selected positions."""
    p = np.asarray(p, dtype=np.float64)
    return float(sum(p[int(s)] for s in set(int(s) for s in selected)))


def relative_output_error(o_sparse: np.ndarray, o_dense: np.ndarray, eps: float = 1e-12) -> float:
    """eq. (14): ||o_sparse - o_dense|| / (||o_dense|| + eps)."""
    o_sparse = np.asarray(o_sparse, dtype=np.float64)
    o_dense = np.asarray(o_dense, dtype=np.float64)
    return float(np.linalg.norm(o_sparse - o_dense) / (np.linalg.norm(o_dense) + eps))

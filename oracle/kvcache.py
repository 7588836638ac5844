"""Plain growable K/V row storage for the oracle, one array per (layer, KV head)."""
from __future__ import annotations

import numpy as np


class RowStore:
    """Rows appended in absolute-position order; rows(l, j) returns the filled part."""

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int, cap: int = 64):
        self.L, self.H, self.D = n_layers, n_kv_heads, head_dim
        self.K = np.zeros((n_layers, n_kv_heads, cap, head_dim))
        self.V = np.zeros((n_layers, n_kv_heads, cap, head_dim))
        self.n = 0

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        """k, v: [L][Hkv][D] for one new position."""
        if self.n == self.K.shape[2]:
            grow = lambda A: np.concatenate([A, np.zeros_like(A)], axis=2)
            self.K, self.V = grow(self.K), grow(self.V)
        self.K[:, :, self.n] = k
        self.V[:, :, self.n] = v
        self.n += 1

    def rows(self, l: int, j: int):
        return self.K[l, j, : self.n], self.V[l, j, : self.n]

    def copy(self) -> "RowStore":
        c = RowStore(self.L, self.H, self.D, max(self.n, 1))
        c.K[:, :, : self.n] = self.K[:, :, : self.n]
        c.V[:, :, : self.n] = self.V[:, :, : self.n]
        c.n = self.n
        return c


def chain(*segments):
    """past(l, j) over several segments, concatenated in the given (position) order.

    A segment is anything with rows(l, j) -> (K, V)."""
    def past(l, j):
        parts = [s.rows(l, j) for s in segments]
        return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    return past


class FixedRows:
    """Per-(layer, head) row sets of possibly different lengths (token-drop keeps
    a different subset per head)."""

    def __init__(self, K: list, V: list):
        self.K, self.V = K, V          # K[l][j] : [n_lj][D]

    def rows(self, l: int, j: int):
        return self.K[l][j], self.V[l][j]

"""f64 brute force for tiny shapes: an independent restatement used to pin the oracle.

Nothing here is shared with the oracle or the library.  It is written as differently
from the oracle as the mathematics allows: explicit rotation matrices for RoPE, an
explicit additive mask matrix for causality, np.repeat for the GQA head mapping and a
whole-matrix softmax, all in f64.
"""
from __future__ import annotations

import numpy as np

NEOX, INTERLEAVED, NONE = 0, 1, 2


def pair_list(hd: int, style: int):
    half = hd // 2
    if style == NEOX:
        return [(i, i + half) for i in range(half)]
    if style == INTERLEAVED:
        return [(2 * i, 2 * i + 1) for i in range(half)]
    raise ValueError(style)


def rotation_matrix(hd: int, angles: np.ndarray, style: int) -> np.ndarray:
    """hd x hd block rotation in f64: subspace i turns by angles[i]."""
    R = np.zeros((hd, hd), np.float64)
    for i, (a, b) in enumerate(pair_list(hd, style)):
        c, s = np.cos(angles[i]), np.sin(angles[i])
        R[a, a], R[a, b] = c, -s
        R[b, a], R[b, b] = s, c
    return R


def f32_angles(hd: int, base: float, freq_scale: float, p: int) -> np.ndarray:
    """Angles as the pages form them: an f32 speed times an f32 position, in f32.

    The speed here comes from numpy's f64 power rounded to f32, not from the oracle."""
    i = np.arange(hd // 2, dtype=np.float64)
    speed = np.float32(np.float64(freq_scale) / np.power(np.float64(base), 2.0 * i / hd))
    return (np.float32(p) * speed.astype(np.float32)).astype(np.float64)


def rope_bf(x: np.ndarray, pos, base: float, freq_scale: float, style: int) -> np.ndarray:
    """x: [nt][nh][hd] -> f64 rotated copy (style NONE returns x in f64)."""
    x = np.asarray(x, np.float64)
    if style == NONE:
        return x.copy()
    nt, nh, hd = x.shape
    out = np.empty_like(x)
    for t in range(nt):
        R = rotation_matrix(hd, f32_angles(hd, base, freq_scale, int(pos[t])), style)
        out[t] = x[t] @ R.T
    return out


def attention_bf(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos, n_head_kv: int,
                 scale: float) -> np.ndarray:
    """q: [nt][n_head][hd]; K, V: [rows][n_head_kv * hd_kv] (one region).

    Returns [nt][n_head][hd_kv] in f64: softmax(q k^T * scale + mask) v per head, the
    mask holding -inf where key row > pos[t].  Query heads map onto kv heads by
    np.repeat (head h uses kv head h // group)."""
    q = np.asarray(q, np.float64)
    nt, n_head, hd = q.shape
    rows = K.shape[0]
    hd_kv = K.shape[1] // n_head_kv
    group = n_head // n_head_kv
    Kh = np.asarray(K, np.float64).reshape(rows, n_head_kv, hd_kv).transpose(1, 0, 2)
    Vh = np.asarray(V, np.float64).reshape(rows, n_head_kv, hd_kv).transpose(1, 0, 2)
    Kh = np.repeat(Kh, group, axis=0)   # [n_head][rows][hd_kv]
    Vh = np.repeat(Vh, group, axis=0)
    mask = np.where(np.arange(rows)[None, :] <= np.asarray(pos)[:, None], 0.0, -np.inf)
    out = np.empty((nt, n_head, hd_kv), np.float64)
    for h in range(n_head):
        S = q[:, h, :hd_kv] @ Kh[h].T * scale + mask          # [nt][rows]
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P = P / P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ Vh[h]
    return out

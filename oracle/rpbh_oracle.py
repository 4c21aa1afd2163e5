"""CPU oracle for the random-permuted block-Hadamard (RPBH) rotation.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product (libddg.so) shares no code with it.

Source: [ORQ] the OrbitQuant article (www.sumeiyu.com, news 221186).
  - §2.1 "旋转量化机制": the rotation Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi,
    H_h a Walsh-Hadamard matrix, D_i diagonal Rademacher signs, P_pi a random
    permutation; after it every coordinate of a unit vector has variance
    close to 1/d.
  - §2.2 "离线-在线协同量化": offline the weights are rotated into the shared
    basis, W <- W Pi_d^T, and quantized; online every activation is rotated by
    Pi_d, so the rotations cancel inside the product.

Readings where the section is silent:

R13  H_h is the Sylvester-ordered Walsh-Hadamard matrix of order h (a power of
     two), scaled by 1/sqrt(h) so that Pi_d is orthogonal (the variance 1/d of
     the section needs a norm-preserving rotation).
R14  (P_pi v)[i] = v[perm[i]]; the signs multiply after the permutation:
     (Pi_d v)[b h + j] = sum_t H_h[j, t] / sqrt(h) * signs[b h + t] * v[perm[b h + t]].
R15  A row vector is rotated as x' = x Pi_d^T, i.e. x'^T = Pi_d x^T: activation
     rows and weight rows (W Pi_d^T) go through the same map.
R16  The block size h is a parameter (the section gives none); the bench uses
     h = 128, one block per quantization group.
R17  The permutation and the signs are inputs (the random draws), so every
     implementation sees the same ones.
"""
from __future__ import annotations

import numpy as np

__all__ = ["hadamard", "rpbh_rotate", "rpbh_matrix"]


def hadamard(h: int) -> np.ndarray:
    """Sylvester Walsh-Hadamard matrix of order h (entries +-1), float64:
    H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    if h < 1 or h & (h - 1):
        raise ValueError("h must be a power of two")
    m = np.ones((1, 1), dtype=np.float64)
    while m.shape[0] < h:
        m = np.block([[m, m], [m, -m]])
    return m


def rpbh_rotate(x, perm, signs, h: int) -> np.ndarray:
    """Rows of x (n x d) mapped by Pi_d (R13-R15), in float64."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    perm = np.asarray(perm, dtype=np.int64)
    s = np.where(np.asarray(signs) < 0, -1.0, 1.0)
    if d % h or perm.shape != (d,) or s.shape != (d,):
        raise ValueError("shape")
    t = x[:, perm] * s[None, :]                       # D P_pi, per row
    hm = hadamard(h) / np.sqrt(float(h))
    blocks = t.reshape(n, d // h, h)
    return np.einsum("jt,nbt->nbj", hm, blocks).reshape(n, d)


def rpbh_matrix(perm, signs, h: int) -> np.ndarray:
    """Pi_d as a dense d x d matrix (tiny d only): column c is Pi_d e_c."""
    d = len(perm)
    return rpbh_rotate(np.eye(d), perm, signs, h).T

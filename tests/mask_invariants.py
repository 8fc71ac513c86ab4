"""Invariants of a chunk's decay mask L (page "State Space Duality and
Mamba-2", "The Mathematical Bridge": L_ij = prod_{k=j+1..i} a_k, a_k in
[0, 1]): entries in [0, 1], zero above the diagonal, and along each row
non-increasing away from the diagonal, L[i, j-1] <= L[i, j] for j <= i."""
import numpy as np


def check_mask_invariants(m):
    """m: [..., Q, Q] mask values (any float dtype)."""
    Q = m.shape[-1]
    assert np.all(m >= 0.0) and np.all(m <= 1.0), "mask outside [0, 1]"
    assert np.all(np.triu(m, 1) == 0.0), "nonzero above the diagonal"
    diffs = m[..., :, 1:] - m[..., :, :-1]          # diffs[i, j-1] = L[i, j] - L[i, j-1]
    lower = np.tril(np.ones((Q, Q - 1), dtype=bool), -1)   # pairs with j <= i
    assert np.all(diffs[..., lower] >= 0.0), "row monotonicity violated"

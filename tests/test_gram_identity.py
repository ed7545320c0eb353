"""The identity the G form of the loss rests on, checked in fp64 on the host.

||dW X^T||_F^2 = sum_r dW_r G dW_r^T with G = X^T X (the output error of the pages is
dW X, squared and summed).  The product runs over G' = G with its B x B blocks above the
diagonal doubled, those below zero and its diagonal zero, and adds the diagonal term
separately:

    sum_r dW_r G dW_r^T = sum_c (sum_r dW_rc^2) G_cc
                          + sum over tile rows a (channels) of sum_{c in a, r} dW_rc (G' dW^T)_cr

where tile row a only needs the columns of G' from block a on.  Inside each diagonal block
the same structure holds at half size (upper-right half block doubled, lower-left zero), so
the upper half of a tile row's channels needs the columns from its own half block on.  This is host logic (numpy,
fp64), independent of the GPU code; the GPU path is compared with the oracle's direct
definition in the GPU tests.
"""
import numpy as np
import pytest


def _g_prime(G, B):
    K = G.shape[0]
    Gp = np.zeros_like(G)
    for a0 in range(0, K, B):
        for b0 in range(0, K, B):
            blk = G[a0:a0 + B, b0:b0 + B]
            if b0 > a0:
                Gp[a0:a0 + B, b0:b0 + B] = 2.0 * blk
            elif b0 == a0:
                Gp[a0:a0 + B, b0:b0 + B] = blk
    np.fill_diagonal(Gp, 0.0)
    return Gp


def _g_form(dW, G, B):
    """The loss as the G-form product computes it: per tile row of channels, k from its own
    diagonal block on, plus the diagonal term."""
    K = G.shape[0]
    Gp = _g_prime(G, B)
    total = np.sum((dW * dW) @ np.diag(G))
    for a0 in range(0, K, B):
        a1 = min(K, a0 + B)
        C = Gp[a0:a1, a0:] @ dW[:, a0:].T          # channels of the tile row x rows of dW
        total += np.sum(dW[:, a0:a1].T * C)
    return total


@pytest.mark.parametrize("M,K,N,B", [(7, 12, 30, 4), (33, 64, 17, 16), (20, 96, 200, 32),
                                     (5, 40, 3, 16), (64, 256, 300, 256), (50, 300, 400, 256)])
def test_g_form_equals_direct(M, K, N, B):
    rng = np.random.default_rng(M * 1000 + K + N)
    dW = rng.standard_normal((M, K))
    X = rng.standard_normal((N, K)) * np.exp(rng.uniform(-2, 2, K))[None, :]
    direct = np.sum((dW @ X.T) ** 2)
    G = X.T @ X
    assert abs(_g_form(dW, G, B) - direct) <= 1e-11 * direct


def _g_prime_halves(G, B):
    """G' with the diagonal blocks restructured at half size: inside each B x B diagonal
    block, the upper-right (B/2) x (B/2) half block doubled and the lower-left one zero."""
    K = G.shape[0]
    Gp = _g_prime(G, B)
    h = B // 2
    for a0 in range(0, K, B):
        p1, q0, q1 = min(K, a0 + h), min(K, a0 + h), min(K, a0 + B)
        Gp[a0:p1, q0:q1] = 2.0 * G[a0:p1, q0:q1]
        Gp[q0:q1, a0:p1] = 0.0
    return Gp


def _g_form_halves(dW, G, B):
    """The G-form loss as the product computes it with half-size diagonal structure: the
    upper half of a tile row's channels starts at k = its own half block."""
    K = G.shape[0]
    Gp = _g_prime_halves(G, B)
    h = B // 2
    total = np.sum((dW * dW) @ np.diag(G))
    for a0 in range(0, K, B):
        for c0, c1 in ((a0, min(K, a0 + h)), (min(K, a0 + h), min(K, a0 + B))):
            if c0 >= c1:
                continue
            C = Gp[c0:c1, c0:] @ dW[:, c0:].T
            total += np.sum(dW[:, c0:c1].T * C)
    return total


@pytest.mark.parametrize("M,K,N,B", [(7, 12, 30, 4), (33, 64, 17, 16), (20, 96, 200, 32),
                                     (5, 40, 3, 16), (64, 256, 300, 256), (50, 300, 400, 256),
                                     (9, 448, 500, 256), (11, 704, 300, 256)])
def test_g_form_half_blocks_equal_direct(M, K, N, B):
    rng = np.random.default_rng(M * 1000 + K + N + 1)
    dW = rng.standard_normal((M, K))
    X = rng.standard_normal((N, K)) * np.exp(rng.uniform(-2, 2, K))[None, :]
    direct = np.sum((dW @ X.T) ** 2)
    G = X.T @ X
    assert abs(_g_form_halves(dW, G, B) - direct) <= 1e-11 * direct
    # the half-block structure is what makes skipping k < c0 exact: with the plain G'
    # (lower-left half block not zero, upper-right not doubled) the same skip is wrong
    Gp = _g_prime(G, B)
    h = B // 2
    wrong = np.sum((dW * dW) @ np.diag(G))
    for a0 in range(0, K, B):
        for c0, c1 in ((a0, min(K, a0 + h)), (min(K, a0 + h), min(K, a0 + B))):
            if c0 < c1:
                wrong += np.sum(dW[:, c0:c1].T * (Gp[c0:c1, c0:] @ dW[:, c0:].T))
    if K > h:
        assert abs(wrong - direct) > 1e-6 * direct


def test_g_form_diagonal_carries_the_independent_part():
    """For independent channels the diagonal term is most of the loss (the reason it is kept
    in fp32 while the off-diagonal entries go to fp16)."""
    rng = np.random.default_rng(3)
    M, K, N = 64, 128, 4096
    dW = rng.standard_normal((M, K))
    X = rng.standard_normal((N, K))
    G = X.T @ X
    diag = np.sum((dW * dW) @ np.diag(G))
    total = np.sum((dW @ X.T) ** 2)
    assert 0.9 < diag / total < 1.1


def test_g_form_planted_mistakes_are_caught():
    """Dropping the doubling, keeping the lower blocks, or leaving the diagonal in G' while
    also adding the diagonal term each break the identity."""
    rng = np.random.default_rng(5)
    M, K, N, B = 9, 48, 60, 16
    dW = rng.standard_normal((M, K))
    X = rng.standard_normal((N, K))
    G = X.T @ X
    direct = np.sum((dW @ X.T) ** 2)

    def variant(double, keep_lower, zero_diag):
        Gp = np.zeros_like(G)
        for a0 in range(0, K, B):
            for b0 in range(0, K, B):
                blk = G[a0:a0 + B, b0:b0 + B]
                if b0 > a0:
                    Gp[a0:a0 + B, b0:b0 + B] = (2.0 if double else 1.0) * blk
                elif b0 == a0 or keep_lower:
                    Gp[a0:a0 + B, b0:b0 + B] = blk
        if zero_diag:
            np.fill_diagonal(Gp, 0.0)
        total = np.sum((dW * dW) @ np.diag(G))
        for a0 in range(0, K, B):
            start = 0 if keep_lower else a0
            C = Gp[a0:a0 + B, start:] @ dW[:, start:].T
            total += np.sum(dW[:, a0:a0 + B].T * C)
        return total

    assert abs(variant(True, False, True) - direct) <= 1e-11 * direct
    for args in [(False, False, True), (True, True, True), (True, False, False)]:
        assert abs(variant(*args) - direct) > 1e-3 * direct, args

"""CPU oracle for the Walsh-Hadamard adapter (WHA) of QWHA -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module. The product path
(``quantization_aware_sparse_amd``) never does, and this module imports
nothing from it: the two share only the seeded input generators in ``synth``.

Everything is plain numpy in float64 on the CPU, with the Walsh-Hadamard
matrix built densely by Sylvester's construction. Where the method has a plain
definition (materialisation, forward, backward) the oracle is that definition
written out with dense matrix products; where it is a heuristic (the budget
allocation and the in-row selection of AdaAlloc) the oracle takes the steps in
the order the pages describe.

Sources (cited by page title and section):
  [PN]  QWHA notes, papernotes.org (ICLR 2026 model-compression notes):
        方法详解 › 整体框架; 关键设计 1 (WHA), 2 (AdaAlloc), 3 (Value Refinement);
        损失函数 / 训练策略.
  [GS]  QWHA technical summary, gist.science (arXiv 2509.17428):
        §2.1 Adapter Design, §2.2 Quantization-Aware Initialization.

Readings of points the pages leave open (all listed in the design notes):
  * H is the Sylvester (natural-order) +-1 matrix, unnormalised; H^-1 = H/n.
    For an input width d_in that is not a power of two, H is block-diagonal
    with Sylvester blocks of order b, the largest power of two dividing
    d_in, and H^-1 = H/b (``wht_matrix``).
  * AdaAlloc's budget formula is missing from the notes; it is read as
    p_i proportional to w_i^(1/t) (t = 1: proportional), floor rounding, a
    per-row floor m and cap d_in enforced by fix-and-reallocate passes (rows
    below the floor are fixed first; only when none are, rows above the cap
    are fixed and the floored rows released), i.e. the clamped proportional
    split, then the leftover (< d_out) goes one unit each to the rows
    with the smallest budget, lower row index first, rows at the cap skipped.
  * "Activation error magnitude" without calibration data is the row's l2
    norm of dW_Q (identity Hessian).
  * In-row selection orders columns by (-|C[i,j]|, j): ties go to the lower
    column; +0.0 and -0.0 are equal magnitudes. E is listed by (i, j).
  * Value Refinement with an identity Hessian (R = I) is exactly the identity
    on the dense solution, so c = fp32_RNE(C[i, E_i]) (see ``refine_ls``).
  * With calibration activations X the refinement is the normal equations of
    the pages' per-channel least squares, x G[S,S] = Q[i,S] with
    G = H Hs H / n^2, Q = dW_Q Hs H / n, Hs = X^T X (X token-major), solved by
    Cholesky; a pivot at or below 1e-10 times its diagonal entry marks G[S,S]
    as not positive definite and the row keeps the dense solution. AdaAlloc
    then allocates by sqrt(dW_Q[i] Hs dW_Q[i]^T). Optional damping adds
    damp * mean(diag Hs) to the diagonal (0 by default: the pages add none).
  * The ablation's selection variants: "magnitude" takes the global top-p of
    |C| (equal magnitudes in row-major order); "random" takes the p positions
    with the smallest SplitMix64 draws, the draw of position (i, j) being
    output i*d_in + j of the generator seeded with the caller's seed.

Parity pins: every public function here is pinned by tests under ``tests/``
against closed forms, library routines or brute force, except the parts of
``adaalloc`` that the pages do not print (the floor/cap passes, the leftover
tie rule and t != 1): those are pinned only to the reading above --
"parity unpinned" with respect to the pages.
"""

from __future__ import annotations

import functools
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "sylvester", "block_size", "wht_matrix", "wht", "transform", "row_norms", "adaalloc", "adaalloc_margins",
    "select", "values", "refine_ls", "csc", "init_select", "splitmix64", "magnitude_keys",
    "random_keys", "global_select", "init_select_global", "hessian", "damped",
    "activation_error_norms", "refine_system", "cholesky_lower", "refine_values",
    "init_select_calibrated", "layer_output_error", "unpack_codes", "dequantize",
    "merge_weights", "layer_forward", "scatter_dense",
    "materialize", "forward", "backward", "backward_dc_rows", "sign_update",
    "rel_err",
]


# --------------------------------------------------------------------------
# O1: the transform kernel H   ([PN] 关键设计 1; [GS] §2.1)
# --------------------------------------------------------------------------

@functools.lru_cache(maxsize=4)
def _sylvester_cached(n: int) -> np.ndarray:
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    H.setflags(write=False)
    return H


def sylvester(n: int) -> np.ndarray:
    """Dense fp64 Walsh-Hadamard matrix of order n by Sylvester's doubling
    H_{2m} = [[H_m, H_m], [H_m, -H_m]] from H_1 = [1]. Entries are +-1 (the
    square-wave basis of [PN] 关键设计 1); H is symmetric and H H = n I, so
    H^-1 = H / n."""
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError("n must be a power of two")
    return _sylvester_cached(int(n))


def block_size(d_in: int) -> int:
    """b = the largest power of two dividing d_in."""
    d_in = int(d_in)
    if d_in < 1:
        raise ValueError("d_in must be positive")
    return d_in & -d_in


def wht_matrix(d_in: int) -> np.ndarray:
    """The transform H for an input width d_in (dense, fp64). For a power of
    two it is the Sylvester matrix of that order. Otherwise, d_in = m * b
    with b the largest power of two dividing it and m odd, and H is
    block-diagonal with m copies of the Sylvester matrix of order b. This
    is the reading for widths the pages do not cover: it keeps +-1 entries,
    orthogonality (H H^T = b I, so H^-1 = H / b) and the add/subtract
    transform."""
    b = block_size(d_in)
    m = d_in // b
    Hb = sylvester(b)
    if m == 1:
        return Hb
    return np.kron(np.eye(m), Hb)


def wht(A: np.ndarray, d_in: int) -> np.ndarray:
    """A @ H for H = wht_matrix(d_in), fp64, applied block by block (the
    product with a block-diagonal matrix, without forming it)."""
    A = np.asarray(A, dtype=np.float64)
    b = block_size(d_in)
    m = d_in // b
    lead = A.shape[:-1]
    return (A.reshape(lead + (m, b)) @ sylvester(b)).reshape(lead + (d_in,))


# --------------------------------------------------------------------------
# O2, O3: dense solution and row error norms   ([PN] 关键设计 2, 3)
# --------------------------------------------------------------------------

def transform(dwq: np.ndarray) -> np.ndarray:
    """Dense solution C = dW_Q H (fp64 matmul). Row i is x0 = v B^-1 of the
    refinement sub-problem with R = I ([PN] 关键设计 3), the candidates AdaAlloc
    picks from ([PN] 关键设计 2)."""
    d_in = dwq.shape[1]
    return wht(dwq, d_in)


def row_norms(dwq: np.ndarray) -> np.ndarray:
    """w_i = ||dW_Q[i, :]||_2 in fp64: the per-output-channel error magnitude
    AdaAlloc allocates by ([PN] 关键设计 2; [GS] §2.2), identity Hessian."""
    a = np.asarray(dwq, dtype=np.float64)
    return np.sqrt(np.sum(a * a, axis=1))


# --------------------------------------------------------------------------
# O4: AdaAlloc budgets   ([PN] 关键设计 2; [GS] §2.2)
# --------------------------------------------------------------------------

def adaalloc(w: np.ndarray, p: int, d_in: int, m: int = 3,
             t: float = 1.0) -> np.ndarray:
    """Per-row budgets p_i with sum p_i = p.

    Proportional pass: share q_i = P * s_i / S over the rows U not yet fixed,
    with s_i = w_i^(1/t), P = p - (budgets of fixed rows), S = sum_U s_i
    (q_i = floor(P/|U|) when S = 0), and p_i = floor(q_i). Rows with q_i < m
    are fixed at m; if there are none, rows with q_i > d_in are fixed at
    d_in and every row fixed at the floor is
    released again (capping raises the others' share); repeat until a pass
    fixes nothing. This reaches the clamped proportional split
    p_i = clamp(lambda * s_i, m, d_in) before rounding.
    The leftover r = p - sum p_i goes one unit each to the rows with the
    smallest p_i (lower row index first), skipping rows at d_in; if r exceeds
    the eligible rows, it is handed out in further such rounds."""
    w = np.asarray(w, dtype=np.float64)
    d_out = w.shape[0]
    if not (m * d_out <= p <= d_in * d_out):
        raise ValueError("budget out of range")
    s = w if t == 1.0 else w ** (1.0 / t)
    budget = np.zeros(d_out, dtype=np.int64)
    fixed = np.zeros(d_out, dtype=bool)
    capped = np.zeros(d_out, dtype=bool)
    while not fixed.all():
        U = ~fixed
        P = int(p - budget[fixed].sum())
        S = float(np.sum(s[U]))
        share = np.zeros(d_out)
        if S > 0.0:
            share[U] = (float(P) * s[U]) / S
        else:
            share[U] = float(P // int(U.sum()))
        budget[U] = np.floor(share[U]).astype(np.int64)
        low = U & (share < m)
        if low.any():
            budget[low] = m
            fixed |= low
            continue
        high = U & (share > d_in)
        if high.any():
            budget[high] = d_in
            capped |= high
            fixed = capped.copy()          # release the rows fixed at the floor
            continue
        break
    r = int(p - budget.sum())
    while r > 0:
        elig = np.nonzero(budget < d_in)[0]
        order = elig[np.lexsort((elig, budget[elig]))]
        give = order[:r]
        budget[give] += 1
        r -= len(give)
    assert int(budget.sum()) == p
    return budget


def adaalloc_margins(w: np.ndarray, p: int, d_in: int, m: int = 3,
                     t: float = 1.0) -> np.ndarray:
    """Distance of P*s_i/S to the nearest integer in the final proportional
    pass, per row (inf for rows fixed at the floor or the cap). A small
    margin means fp64 rounding order could change that row's floor."""
    w = np.asarray(w, dtype=np.float64)
    d_out = w.shape[0]
    s = w if t == 1.0 else w ** (1.0 / t)
    budget = np.zeros(d_out, dtype=np.int64)
    fixed = np.zeros(d_out, dtype=bool)
    margin = np.full(d_out, np.inf)
    capped = np.zeros(d_out, dtype=bool)
    while not fixed.all():
        U = ~fixed
        P = int(p - budget[fixed].sum())
        S = float(np.sum(s[U]))
        share = np.zeros(d_out)
        if S > 0.0:
            share[U] = (float(P) * s[U]) / S
            margin[:] = np.inf
            margin[U] = np.abs(share[U] - np.rint(share[U]))
        else:
            share[U] = float(P // int(U.sum()))
        budget[U] = np.floor(share[U]).astype(np.int64)
        low = U & (share < m)
        if low.any():
            budget[low] = m
            fixed |= low
            continue
        high = U & (share > d_in)
        if high.any():
            budget[high] = d_in
            capped |= high
            fixed = capped.copy()
            continue
        break
    margin[fixed] = np.inf
    return margin


# --------------------------------------------------------------------------
# O5, O6: in-row top-magnitude selection and values   ([PN] 关键设计 2, 3)
# --------------------------------------------------------------------------

def select(C: np.ndarray, budgets: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """For each row take the p_i columns first in the order (-|C[i,j]|, j)
    (largest magnitude first, lower column on ties) and list them ascending.
    Returns (row_ptr int32 [d_out+1], E int32 [p][2] of (i, j))."""
    d_out, d_in = C.shape
    budgets = np.asarray(budgets, dtype=np.int64)
    row_ptr = np.zeros(d_out + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(budgets)
    E = np.zeros((int(row_ptr[-1]), 2), dtype=np.int64)
    for i in range(d_out):
        order = np.argsort(-np.abs(C[i]), kind="stable")
        cols = np.sort(order[: budgets[i]])
        E[row_ptr[i]:row_ptr[i + 1], 0] = i
        E[row_ptr[i]:row_ptr[i + 1], 1] = cols
    return row_ptr.astype(np.int32), E.astype(np.int32)


def values(C: np.ndarray, E: np.ndarray) -> np.ndarray:
    """c_k = fp32(C[i_k, j_k]), round to nearest even: the dense solution at
    the chosen positions, which is what refinement returns when R = I."""
    return C[E[:, 0], E[:, 1]].astype(np.float32)


def refine_ls(v: np.ndarray, B: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Value Refinement for one channel ([PN] 关键设计 3): least squares
    min_x ||v - x B'||^2 over the rows B' = B[cols, :], solved with
    numpy.linalg.lstsq. With R = I, B = H^-1 = H/n and the solution equals
    the dense solution at cols (pinned by a test); kept for that pin."""
    Bp = np.asarray(B, dtype=np.float64)[np.asarray(cols), :]
    sol, *_ = np.linalg.lstsq(Bp.T, np.asarray(v, dtype=np.float64), rcond=None)
    return sol


def csc(E: np.ndarray, d_in: int) -> Tuple[np.ndarray, np.ndarray]:
    """Column index of F: csc_perm lists the positions k of E column by
    column, ascending k within a column (a stable sort by j); col_ptr is its
    exclusive scan of column counts."""
    j = np.asarray(E[:, 1], dtype=np.int64)
    perm = np.argsort(j, kind="stable")
    counts = np.bincount(j, minlength=d_in)
    col_ptr = np.zeros(d_in + 1, dtype=np.int64)
    col_ptr[1:] = np.cumsum(counts)
    return col_ptr.astype(np.int32), perm.astype(np.int32)


def init_select(dwq: np.ndarray, p: int, m: int = 3, t: float = 1.0,
                with_diagnostics: bool = False) -> Dict[str, np.ndarray]:
    """Quantization-aware init: w -> budgets -> E, c (+ the column index).

    The pipeline of [PN] 方法详解 › 整体框架 under the identity Hessian:
    dense solution C = dW_Q H, AdaAlloc budgets from the row norms, in-row
    top-magnitude positions, values c = C at E (refinement with R = I)."""
    d_out, d_in = dwq.shape
    C = transform(dwq)
    w = row_norms(dwq)
    budgets = adaalloc(w, p, d_in, m, t)
    row_ptr, E = select(C, budgets)
    c = values(C, E)
    col_ptr, perm = csc(E, d_in)
    out = dict(row_ptr=row_ptr, E=E, c=c, col_ptr=col_ptr, csc_perm=perm,
               budgets=budgets, w=w)
    if with_diagnostics:
        gaps = np.full(d_out, np.inf)
        for i in range(d_out):
            a = np.sort(np.abs(C[i]))[::-1]
            k = int(budgets[i])
            if 0 < k < d_in and a[k - 1] > 0:
                gaps[i] = (a[k - 1] - a[k]) / a[k - 1]
        out["boundary_gap"] = gaps
        out["budget_margin"] = adaalloc_margins(w, p, d_in, m, t)
        out["C"] = C
    return out


# --------------------------------------------------------------------------
# Selection variants of the ablation: the global top-p of the dense solution
# by magnitude, and p positions drawn at random ([PN] 关键设计 2 describes
# the global magnitude pick that AdaAlloc improves on; 实验关键数据 ›
# 消融实验 (Table 4) compares both with AdaAlloc; [GS] §2.2). Values and
# refinement are as for AdaAlloc: c = fp32(C[E]) under R = I.
# --------------------------------------------------------------------------

_GAMMA = 0x9E3779B97F4A7C15
_U64 = (1 << 64) - 1


def splitmix64(seed: int, n: np.ndarray) -> np.ndarray:
    """Output n (n = 0, 1, ...) of the SplitMix64 generator seeded with
    `seed` (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): the state after n+1 steps is
    seed + (n+1)*gamma mod 2^64 with gamma = 0x9E3779B97F4A7C15, and the
    output is that state through the mix: z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
    z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31 (all mod 2^64).
    The state is a function of n alone, so any draw is computed directly."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _U64) + (n + np.uint64(1)) * np.uint64(_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def magnitude_keys(C: np.ndarray) -> np.ndarray:
    """|C| as fp64 bit patterns (uint64): ordered like |C|; -0.0 == +0.0."""
    return np.ascontiguousarray(np.abs(C)).view(np.uint64)


def random_keys(d_out: int, d_in: int, seed: int) -> np.ndarray:
    """The complement of the SplitMix64 draw of each position (flat index
    i*d_in + j): larger keys are smaller draws, so taking the largest keys
    takes the positions with the smallest draws."""
    n = np.arange(d_out * d_in, dtype=np.uint64)
    return (~splitmix64(seed, n)).reshape(d_out, d_in)


def global_select(keys: np.ndarray, p: int) -> Tuple[np.ndarray, np.ndarray]:
    """The p positions with the largest keys over the whole matrix, equal
    keys taken in row-major order; E listed by (i, j), row_ptr per row."""
    d_out, d_in = keys.shape
    flat = keys.ravel()
    if not 0 <= p <= flat.size:
        raise ValueError("p out of range")
    order = np.lexsort((np.arange(flat.size), ~flat))   # key descending, index ascending
    sel = np.sort(order[:p])
    E = np.stack([sel // d_in, sel % d_in], axis=1).astype(np.int32)
    counts = np.bincount(E[:, 0], minlength=d_out)
    row_ptr = np.zeros(d_out + 1, dtype=np.int32)
    np.cumsum(counts, out=row_ptr[1:])
    return row_ptr, E


def init_select_global(dwq: np.ndarray, p: int, strategy: str,
                       seed: int = 0) -> Dict[str, np.ndarray]:
    """Global selection variant ('magnitude' or 'random') of the init:
    E from global_select on the variant's keys, c = fp32(C[E])."""
    d_out, d_in = dwq.shape
    C = transform(dwq)
    if strategy == "magnitude":
        keys = magnitude_keys(C)
    elif strategy == "random":
        keys = random_keys(d_out, d_in, seed)
    else:
        raise ValueError(strategy)
    row_ptr, E = global_select(keys, p)
    c = values(C, E)
    col_ptr, perm = csc(E, d_in)
    return dict(row_ptr=row_ptr, E=E, c=c, col_ptr=col_ptr, csc_perm=perm, C=C, keys=keys)


# --------------------------------------------------------------------------
# O11-O14: Value Refinement with a calibration Hessian   ([PN] 关键设计 2, 3;
# 损失函数 / 训练策略; [GS] §2.2)
#
# The init's objective is the layer-output error ||dW_Q X - F H^-1 X||_F^2
# over calibration activations; with the Hessian XX^T = U S U^T and
# R = U S^(1/2) it becomes ||dW_Q R - F H^-1 R||_F^2, solved channel by
# channel: positions by AdaAlloc (budgets from the activation error
# magnitude ||dW_Q[i,:] R||, then the in-row top |C|), values by least
# squares min_x ||v - x B'||^2 with v = dW_Q[i,:] R and B' the rows of
# B = H^-1 R at the chosen positions. The closed form did not survive
# extraction; it is read as the normal equations of that problem,
#   x (B' B'^T) = v B'^T,  B' B'^T = G[S,S],  v B'^T = Q[i,S],
#   G = H Hs H / n^2,  Q = dW_Q Hs H / n,  Hs = XX^T,
# since R R^T = Hs and H^-1 = H/n is symmetric: no SVD is needed.
# Activations are stored token-major here (X is [N][d_in]), so Hs = X^T X.
# --------------------------------------------------------------------------

def hessian(X: np.ndarray) -> np.ndarray:
    """Hs = sum over calibration tokens of x^T x (fp64 [d_in][d_in]): the
    pages' XX^T with one column per token."""
    a = np.asarray(X, dtype=np.float64)
    return a.T @ a


def damped(Hs: np.ndarray, damp: float) -> np.ndarray:
    """Hs + damp * mean(diag Hs) * I. The pages add no damping (damp = 0 is
    the plain reading); a relative diagonal load is offered for calibration
    sets too small to make Hs definite."""
    Hs = np.asarray(Hs, dtype=np.float64)
    if damp == 0.0:
        return Hs.copy()
    return Hs + damp * float(np.mean(np.diag(Hs))) * np.eye(Hs.shape[0])


def activation_error_norms(dwq: np.ndarray, Hs: np.ndarray) -> np.ndarray:
    """w_i = ||dW_Q[i,:] R||_2 = sqrt(dW_Q[i,:] Hs dW_Q[i,:]^T): the
    activation error magnitude AdaAlloc allocates by ([PN] 关键设计 2)."""
    a = np.asarray(dwq, dtype=np.float64)
    q = np.einsum("ij,ij->i", a @ np.asarray(Hs, dtype=np.float64), a)
    return np.sqrt(np.maximum(q, 0.0))


def refine_system(dwq: np.ndarray, Hs: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """G = H Hs H / n^2 (the Gram matrix of the rows of B = H^-1 R) and
    Q = dW_Q Hs H / n (row i holds v B^T), both fp64 dense."""
    d_in = dwq.shape[1]
    b = float(block_size(d_in))
    Hs = np.asarray(Hs, dtype=np.float64)
    G = wht(wht(Hs, d_in).T, d_in) / b ** 2        # H Hs H (H and Hs symmetric)
    Q = wht(np.asarray(dwq, dtype=np.float64) @ Hs, d_in) / b
    return G, Q


def cholesky_lower(A: np.ndarray, pivot_tol: float = 1e-10) -> Tuple[np.ndarray, bool]:
    """Textbook Cholesky A = L L^T, column by column (outer-product form).
    A pivot (the diagonal before its square root) at or below pivot_tol times
    that diagonal entry of A marks A as not positive definite, returning
    (partial L, False)."""
    A = np.array(A, dtype=np.float64)
    n = A.shape[0]
    d0 = A.diagonal().copy()
    L = np.zeros_like(A)
    for k in range(n):
        piv = A[k, k]
        if not piv > pivot_tol * d0[k]:
            return L, False
        L[k, k] = np.sqrt(piv)
        L[k + 1:, k] = A[k + 1:, k] / L[k, k]
        A[k + 1:, k + 1:] -= np.outer(L[k + 1:, k], L[k + 1:, k])
    return L, True


def refine_values(G: np.ndarray, Q: np.ndarray, row_ptr: np.ndarray, E: np.ndarray,
                  pivot_tol: float = 1e-10) -> Tuple[np.ndarray, np.ndarray]:
    """Per row i with positions S = E_i: solve x G[S,S] = Q[i,S] by Cholesky
    of G[S,S] and two triangular solves ([PN] 关键设计 3). Returns x (fp64 [p];
    NaN on rows whose G[S,S] is not positive definite) and ok [d_out]."""
    import scipy.linalg as sla
    d_out = len(row_ptr) - 1
    x = np.full(len(E), np.nan)
    ok = np.ones(d_out, dtype=bool)
    for i in range(d_out):
        a, b = int(row_ptr[i]), int(row_ptr[i + 1])
        if a == b:
            continue
        S = np.asarray(E[a:b, 1], dtype=np.int64)
        A = G[np.ix_(S, S)]
        L, good = cholesky_lower(A, pivot_tol)
        if not good:
            ok[i] = False
            continue
        y = sla.solve_triangular(L, Q[i, S], lower=True)
        x[a:b] = sla.solve_triangular(L.T, y, lower=False)
    return x, ok


def init_select_calibrated(dwq: np.ndarray, Hs: np.ndarray, p: int, m: int = 3,
                           t: float = 1.0, damp: float = 0.0,
                           pivot_tol: float = 1e-10) -> Dict[str, np.ndarray]:
    """The init with calibration data ([PN] 方法详解 › 整体框架, 关键设计 2, 3):
    Hs' = damped(Hs), w = activation error norms under Hs', AdaAlloc budgets,
    in-row top |C| positions (C = dW_Q H does not depend on Hs), then refined
    values c = fp32(x); a row whose G[S,S] is not positive definite keeps the
    dense solution fp32(C[E])."""
    d_out, d_in = dwq.shape
    Hd = damped(Hs, damp)
    C = transform(dwq)
    w = activation_error_norms(dwq, Hd)
    budgets = adaalloc(w, p, d_in, m, t)
    row_ptr, E = select(C, budgets)
    c0 = values(C, E)
    G, Q = refine_system(dwq, Hd)
    x, ok = refine_values(G, Q, row_ptr, E, pivot_tol)
    bad = np.repeat(~ok, np.diff(row_ptr))
    c = np.where(bad, c0, x.astype(np.float32)).astype(np.float32)
    rhs = Q[E[:, 0], E[:, 1]] if len(E) else np.zeros(0)
    col_ptr, perm = csc(E, d_in)
    return dict(row_ptr=row_ptr, E=E, c=c, c_dense=c0, x=x, ok=ok, col_ptr=col_ptr,
                csc_perm=perm, budgets=budgets, w=w, G=G, rhs=rhs, C=C, Hs=Hd)


def layer_output_error(dwq: np.ndarray, X: np.ndarray, E: np.ndarray, c: np.ndarray) -> float:
    """||(dW_Q - F H^-1) X^T||_F^2 over calibration tokens X [N][d_in]: the
    init's objective ([PN] 损失函数 / 训练策略)."""
    d_out, d_in = dwq.shape
    F = scatter_dense(E, np.asarray(c, dtype=np.float64), d_out, d_in)
    resid = np.asarray(dwq, dtype=np.float64) - wht(F, d_in) / float(block_size(d_in))
    r = resid @ np.asarray(X, dtype=np.float64).T
    return float(np.sum(r * r))


# --------------------------------------------------------------------------
# O15-O17: the quantized base layer with the adapter (inference path):
# packed b-bit codes with per-group scale and zero ([PN] 损失函数 / 训练策略:
# the adapter is merged into the quantized model, group quantization), the
# merged weights W_Q + alpha dW, and y = x W_Q^T + alpha z F^T.
# --------------------------------------------------------------------------

def unpack_codes(words: np.ndarray, d_in: int, bits: int) -> np.ndarray:
    """Codes q [rows][d_in] from uint32 words: code j of a row sits in word
    j // cpw, cpw = floor(32 / bits), at bit (j % cpw) * bits."""
    cpw = 32 // bits
    words = np.asarray(words, dtype=np.uint64)
    j = np.arange(d_in)
    shift = ((j % cpw) * bits).astype(np.uint64)
    return ((words[:, j // cpw] >> shift) & np.uint64((1 << bits) - 1)).astype(np.int64)


def dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int) -> np.ndarray:
    """W_Q = (q - z) * s per group of `group` columns, in fp32 (the
    quantizer's own arithmetic)."""
    g = np.arange(q.shape[1]) // group
    z = np.asarray(zeros, dtype=np.float32)[:, g]
    s = np.asarray(scales, dtype=np.float32)[:, g]
    return ((q.astype(np.float32) - z) * s).astype(np.float32)


def merge_weights(W_Q: np.ndarray, E: np.ndarray, c: np.ndarray, alpha: float) -> np.ndarray:
    """W_Q + alpha F H^-1 (fp64): the adapter merged into the base weights."""
    d_out, d_in = W_Q.shape
    return np.asarray(W_Q, dtype=np.float64) + materialize(E, c, d_out, d_in, alpha)


def layer_forward(x: np.ndarray, W_Q: np.ndarray, E: np.ndarray, c: np.ndarray,
                  alpha: float) -> np.ndarray:
    """y = x W_Q^T + alpha z F^T (fp64): the quantized layer with its
    adapter, by the plain definition x (W_Q + alpha F H^-1)^T."""
    return np.asarray(x, dtype=np.float64) @ merge_weights(W_Q, E, c, alpha).T


# --------------------------------------------------------------------------
# O7-O10: materialisation, forward, backward, update
#         ([PN] 方法详解 › 整体框架, 损失函数 / 训练策略; [GS] §2.1)
# --------------------------------------------------------------------------

def scatter_dense(E: np.ndarray, c: np.ndarray, d_out: int,
                  d_in: int) -> np.ndarray:
    """F = Scatter(c, E) as a dense fp64 [d_out][d_in] matrix."""
    F = np.zeros((d_out, d_in), dtype=np.float64)
    F[E[:, 0], E[:, 1]] = np.asarray(c, dtype=np.float64)
    return F


def _scatter_sparse(E, c, d_out, d_in):
    import scipy.sparse as sp
    return sp.csr_matrix(
        (np.asarray(c, dtype=np.float64), (E[:, 0], E[:, 1])),
        shape=(d_out, d_in))


def materialize(E: np.ndarray, c: np.ndarray, d_out: int, d_in: int,
                alpha: float = 1.0) -> np.ndarray:
    """dW = alpha * F H^-1 = alpha * F H / n, F = Scatter(c, E).

    F is held as a scipy sparse matrix so the product skips its zeros; every
    output entry is the same sum as the dense product F @ H."""
    F = _scatter_sparse(E, c, d_out, d_in)
    if block_size(d_in) == d_in:
        return (alpha / d_in) * np.asarray(F @ sylvester(d_in))
    return (alpha / block_size(d_in)) * wht(F.toarray(), d_in)


def forward(x: np.ndarray, dW: np.ndarray) -> np.ndarray:
    """Adapter branch of the layer output: y = x dW^T (fp64)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(dW, dtype=np.float64).T


def backward(x: np.ndarray, dy: np.ndarray, E: np.ndarray, c: np.ndarray,
             d_out: int, d_in: int, alpha: float = 1.0,
             dW: Optional[np.ndarray] = None):
    """Gradients of the adapter branch with W_Q and H frozen and only c
    trainable ([PN] 损失函数 / 训练策略):
      dx = dy dW;  G = dy^T x;  dF = alpha * G H / n;  dc = dF[E]."""
    if dW is None:
        dW = materialize(E, c, d_out, d_in, alpha)
    x64 = np.asarray(x, dtype=np.float64)
    dy64 = np.asarray(dy, dtype=np.float64)
    dx = dy64 @ dW
    G = dy64.T @ x64
    dF = (alpha / block_size(d_in)) * wht(G, d_in)
    dc = dF[E[:, 0], E[:, 1]]
    return dx, dc


def backward_dc_rows(x: np.ndarray, dy: np.ndarray, E: np.ndarray,
                     rows: np.ndarray, d_in: int,
                     alpha: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """dc restricted to the nonzeros of the given rows of F: the same
    definition as ``backward`` (dF = alpha * (dy^T x) H / n, gathered at E)
    evaluated on those rows of G only. Returns (k indices, dc values)."""
    rows = np.asarray(rows, dtype=np.int64)
    x64 = np.asarray(x, dtype=np.float64)
    G = np.asarray(dy, dtype=np.float64)[:, rows].T @ x64   # [len(rows)][d_in]
    dF = (alpha / block_size(d_in)) * wht(G, d_in)
    where = {int(r): a for a, r in enumerate(rows)}
    ks = np.nonzero(np.isin(E[:, 0], rows))[0]
    vals = np.array([dF[where[int(E[k, 0])], int(E[k, 1])] for k in ks])
    return ks, vals


def sign_update(c: np.ndarray, dc: np.ndarray, step: float = 1e-3) -> np.ndarray:
    """c' = c + fp32(step) * sign(dc) in fp32 (sign(0) = 0): the synthetic
    coefficient update of the attention-block training step."""
    c32 = np.asarray(c, dtype=np.float32)
    sg = np.sign(np.asarray(dc, dtype=np.float32)).astype(np.float32)
    return (c32 + np.float32(step) * sg).astype(np.float32)


def rel_err(a: np.ndarray, b: np.ndarray) -> float:
    """Normwise relative error max|a - b| / max|b| (b is the reference)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if a.size else 0.0
    if den == 0.0:
        return num
    return num / den

"""Pins of the CPU oracle to things other than itself: closed forms, textbook
values, library routines (scipy.linalg.hadamard, numpy.linalg.lstsq/inv,
torch.autograd in fp64) and brute force on tiny inputs. Each test is chosen
so that a plausible slip in the oracle (a dropped term, a sign, an index, a
transposed operand) fails it."""

import itertools

import numpy as np
import pytest

import oracle as O
from tests.conftest import read_golden


# ---------------------------------------------------------------- H (O1)

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_sylvester_identities(n):
    H = O.sylvester(n)
    assert H.shape == (n, n)
    assert np.array_equal(H @ H.T, n * np.eye(n))          # H H^T = n I
    assert np.array_equal(H, H.T)                          # symmetric
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda a: bin(int(a)).count("1"))(i & j)
    assert np.array_equal(H, (-1.0) ** pc)                 # (-1)^popcount(i&j)


@pytest.mark.parametrize("n", [2, 4, 32, 512, 4096])
def test_sylvester_matches_scipy(n):
    from scipy.linalg import hadamard
    assert np.array_equal(O.sylvester(n), hadamard(n).astype(np.float64))


def test_sylvester_golden():
    g = read_golden("wht4.txt")
    assert np.array_equal(O.sylvester(4), g["H4"])
    assert np.array_equal(O.sylvester(2), np.array([[1.0, 1.0], [1.0, -1.0]]))
    C = O.transform(g["v"].astype(np.float32))
    assert np.array_equal(C, g["C"])


def test_sylvester_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.sylvester(12)


# --------------------------------------------------------- transform (O2/O3)

def _fwht_recursive(v):
    """Independent check: the textbook in-place butterfly recursion."""
    a = np.array(v, dtype=np.float64)
    h = 1
    n = a.shape[-1]
    while h < n:
        for s in range(0, n, 2 * h):
            x = a[..., s:s + h].copy()
            y = a[..., s + h:s + 2 * h].copy()
            a[..., s:s + h] = x + y
            a[..., s + h:s + 2 * h] = x - y
        h *= 2
    return a


def test_transform_matches_butterfly_recursion():
    rng = np.random.default_rng(1)
    dwq = rng.standard_normal((5, 64)).astype(np.float32)
    C = O.transform(dwq)
    assert np.allclose(C, _fwht_recursive(dwq.astype(np.float64)),
                       rtol=0, atol=1e-12)


def test_transform_parseval():
    rng = np.random.default_rng(2)
    dwq = (0.01 * rng.standard_normal((16, 256))).astype(np.float32)
    C = O.transform(dwq)
    w = O.row_norms(dwq)
    lhs = np.sum(C * C, axis=1)
    rhs = 256 * w * w
    assert np.max(np.abs(lhs - rhs) / rhs) < 1e-12


def test_transform_spike_and_constant():
    n = 32
    H = O.sylvester(n)
    for j in [0, 5, 31]:
        row = np.zeros((1, n), np.float32)
        row[0, j] = 0.75
        assert np.array_equal(O.transform(row)[0], 0.75 * H[j])
    const = np.full((1, n), 0.125, np.float32)
    C = O.transform(const)[0]
    assert C[0] == n * 0.125 and np.all(C[1:] == 0)


def test_row_norms():
    dwq = np.array([[3, 4, 0, 0], [0, 0, 0, 0], [1, 1, 1, 1]], np.float32)
    assert np.array_equal(O.row_norms(dwq), np.array([5.0, 0.0, 2.0]))


# --------------------------------------------------------------- AdaAlloc (O4)

def test_adaalloc_golden():
    g = read_golden("adaalloc_hand.txt")
    p, m, d_in = (int(v) for v in g["p m d_in"][0])
    b = O.adaalloc(g["w"][0], p, d_in, m=m)
    assert np.array_equal(b, g["budgets"][0].astype(np.int64))


def _expected_unbounded(w, p):
    """When neither the floor nor the cap binds the rule is a single
    proportional floor pass plus the leftover to the smallest budgets."""
    S = float(np.sum(w))
    b = np.floor(p * w / S).astype(np.int64)
    r = p - int(b.sum())
    order = np.lexsort((np.arange(len(w)), b))
    b[order[:r]] += 1
    return b


def test_adaalloc_reduces_to_proportional():
    rng = np.random.default_rng(3)
    w = rng.uniform(0.5, 2.0, size=257)
    p = 257 * 40 + 123
    b = O.adaalloc(w, p, 1024, m=3)
    assert np.array_equal(b, _expected_unbounded(w, p))
    assert b.sum() == p


def test_adaalloc_invariants_random():
    rng = np.random.default_rng(4)
    for trial in range(30):
        d_out = int(rng.integers(1, 200))
        d_in = int(2 ** rng.integers(2, 9))
        m = int(rng.integers(0, min(4, d_in) + 1))
        p = int(rng.integers(m * d_out, d_in * d_out + 1))
        w = rng.lognormal(0, 2, size=d_out) * (rng.random(d_out) > 0.1)
        b = O.adaalloc(w, p, d_in, m=m)
        assert b.sum() == p
        assert np.all(b >= m) and np.all(b <= d_in)


def test_adaalloc_floor_binds():
    b = O.adaalloc(np.array([1e-6, 1.0, 1.0, 1.0]), 12, 8, m=3)
    assert np.array_equal(b, [3, 3, 3, 3])


def test_adaalloc_cap_binds():
    # pass 1: floor(12*w/103) = (11, 0, 0, 0) -> rows 1..3 fixed at the floor 1
    # pass 2: U = {0}, P = 9 > d_in = 4 -> row 0 capped at 4, rows 1..3 released
    # pass 3: P = 8 over (1, 1, 1): floor(8/3) = 2 each; leftover 2 -> rows 1, 2
    b = O.adaalloc(np.array([100.0, 1.0, 1.0, 1.0]), 12, 4, m=1)
    assert np.array_equal(b, [4, 3, 3, 2])


def test_adaalloc_cap_keeps_others_proportional():
    # the capped row's excess is shared in proportion to the others' norms:
    # after capping row 0 at 8, P = 12 over w = (1, 2, 3): (2, 4, 6) exactly
    b = O.adaalloc(np.array([100.0, 1.0, 2.0, 3.0]), 20, 8, m=1)
    assert np.array_equal(b, [8, 2, 4, 6])


def test_adaalloc_is_clamped_proportional_split():
    """Brute-force pin of the floor/cap reading: before rounding the budgets
    are clamp(lambda s_i, m, d_in) with lambda solving sum = p (bisection)."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        d_out = int(rng.integers(2, 40))
        d_in = int(2 ** rng.integers(2, 7))
        m = int(rng.integers(0, 4))
        m = min(m, d_in)
        p = int(rng.integers(m * d_out, d_in * d_out + 1))
        w = rng.lognormal(0, 2.5, size=d_out)
        b = O.adaalloc(w, p, d_in, m=m)
        lo, hi = 0.0, 1e30
        for _ in range(400):
            lam = 0.5 * (lo + hi)
            if np.clip(lam * w, m, d_in).sum() < p:
                lo = lam
            else:
                hi = lam
        cont = np.clip(hi * w, m, d_in)
        # rounding moves each budget by less than one unit from the split
        assert np.all(np.abs(b - cont) < 1.0 + 1e-6), (b, cont)
        assert b.sum() == p


def test_adaalloc_zero_norms_split_evenly():
    b = O.adaalloc(np.zeros(4), 10, 8, m=1)
    # floor(10/4) = 2 each, leftover 2 to rows 0 and 1
    assert np.array_equal(b, [3, 3, 2, 2])


def test_adaalloc_temperature_flattens():
    w = np.array([1.0, 4.0, 16.0])
    b1 = O.adaalloc(w, 42, 64, m=0, t=1.0)
    b2 = O.adaalloc(w, 42, 64, m=0, t=2.0)   # w^(1/2) = (1, 2, 4)
    assert np.array_equal(b1, [2, 8, 32])
    assert np.array_equal(b2, [6, 12, 24])


def test_adaalloc_rejects_infeasible():
    with pytest.raises(ValueError):
        O.adaalloc(np.ones(4), 11, 8, m=3)       # p < m d_out
    with pytest.raises(ValueError):
        O.adaalloc(np.ones(4), 33, 8, m=3)       # p > d_in d_out


# ------------------------------------------- AdaAlloc rounding margins (O12)
# The margin of a row is the distance of its share P s_i / S in the final
# proportional pass to the nearest integer (inf for a row held at the floor
# or the cap). The values below are worked by hand.

def test_adaalloc_margin_half():
    # w = (1, 1), p = 7: both shares are 7/2 = 3.5, half-way between floors
    got = O.adaalloc_margins(np.array([1.0, 1.0]), 7, 100, m=3)
    assert np.array_equal(got, [0.5, 0.5])
    assert np.array_equal(O.adaalloc(np.array([1.0, 1.0]), 7, 100, m=3), [4, 3])


def test_adaalloc_margin_of_the_golden_case_and_the_floored_row():
    # w = (1, 2, 3, 4), p = 20, m = 3: row 0 is held at the floor in the first
    # pass; the second pass shares P = 17 over S = 9: 34/9, 51/9, 68/9, whose
    # distances to 4, 6, 8 are 2/9, 3/9, 4/9
    got = O.adaalloc_margins(np.array([1.0, 2.0, 3.0, 4.0]), 20, 100, m=3)
    assert got[0] == np.inf
    assert np.allclose(got[1:], [2 / 9, 3 / 9, 4 / 9], rtol=0, atol=1e-14)


def test_adaalloc_margin_near_an_integer():
    # w = (1, 2 + d), p = 30: the shares are 30/(3+d) and 30(2+d)/(3+d), both
    # 10 d / (3 + d) from the integers 10 and 20 (about 1e-12 for d = 3e-13)
    d = 3e-13
    w = np.array([1.0, 2.0 + d])
    dd = w[1] - 2.0                          # the d that fp64 actually holds
    want = 10.0 * dd / (3.0 + dd)
    got = O.adaalloc_margins(w, 30, 100, m=0)
    assert np.all(np.abs(got - want) <= 2e-15), (got, want)
    assert 0.9e-12 < got[0] < 1.1e-12
    # an exact split has margin 0 in every row
    assert np.array_equal(O.adaalloc_margins(np.array([1.0, 2.0, 1.0]), 40, 100, m=0),
                          [0.0, 0.0, 0.0])


def test_adaalloc_margin_after_the_cap_releases_the_floor():
    # w = (1, 1, 100), p = 40, d_in = 16, m = 1: rows 0, 1 fall below the
    # floor first (40/102 each); then row 2's share 38 exceeds the cap and is
    # held at 16, which releases rows 0 and 1; they split the remaining 24
    # evenly: shares 12, 12 (margin 0) and row 2 at the cap (inf)
    w = np.array([1.0, 1.0, 100.0])
    assert np.array_equal(O.adaalloc(w, 40, 16, m=1), [12, 12, 16])
    assert np.array_equal(O.adaalloc_margins(w, 40, 16, m=1), [0.0, 0.0, np.inf])


def test_adaalloc_margin_temperature():
    # t = 2 shares by sqrt(w): w = (1, 4) -> s = (1, 2), p = 10: shares
    # 10/3 and 20/3, both 1/3 from an integer
    got = O.adaalloc_margins(np.array([1.0, 4.0]), 10, 100, m=0, t=2.0)
    assert np.allclose(got, [1 / 3, 1 / 3], rtol=0, atol=1e-14)


# -------------------------------------------------------- selection (O5/O6)

@pytest.mark.parametrize("n", [4, 8, 16])
def test_select_is_best_sparse_approximation_bruteforce(n):
    """Within a row, the chosen p_i columns minimise the least-squares error
    ||v - x_S (H/n)[S,:]||^2 over all subsets of that size; the minimum is
    (1/n) sum_{j not in S} C_j^2 and the LS solution is C[S] (refinement with
    R = I is the identity)."""
    rng = np.random.default_rng(10 + n)
    H = O.sylvester(n)
    B = H / n
    for trial in range(4):
        v = rng.standard_normal(n).astype(np.float32)
        C = O.transform(v[None, :])[0]
        for k in range(1, min(4, n) + 1):
            _, E = O.select(C[None, :], np.array([k]))
            S_or = tuple(int(j) for j in E[:, 1])
            best, best_S = np.inf, None
            for S in itertools.combinations(range(n), k):
                x, *_ = np.linalg.lstsq(B[list(S)].T, v.astype(np.float64),
                                        rcond=None)
                res = float(np.sum((v - x @ B[list(S)]) ** 2))
                if res < best - 1e-12:
                    best, best_S = res, S
            x_or = O.refine_ls(v, B, np.array(S_or))
            res_or = float(np.sum((v - x_or @ B[list(S_or)]) ** 2))
            assert res_or <= best + 1e-10
            assert S_or == best_S
            rest = [j for j in range(n) if j not in S_or]
            assert abs(res_or - np.sum(C[rest] ** 2) / n) < 1e-10
            assert np.allclose(x_or, C[list(S_or)], rtol=0, atol=1e-10)
            assert np.array_equal(O.values(C[None, :], E),
                                  x_or.astype(np.float32)) or \
                np.allclose(O.values(C[None, :], E), x_or, rtol=1e-6)


def test_select_ties_go_to_lower_column():
    n = 16
    row = np.zeros((1, n), np.float32)
    row[0, 6] = 1.0            # spike: every |C| equals 1
    C = O.transform(row)
    for k in [1, 3, 16]:
        _, E = O.select(C, np.array([k]))
        assert np.array_equal(E[:, 1], np.arange(k))
    # signed zeros are equal magnitudes
    Cz = np.array([[0.0, -0.0, 0.0, -0.0]])
    _, E = O.select(Cz, np.array([2]))
    assert np.array_equal(E[:, 1], [0, 1])


def _row_with_transform(Crow):
    """A 1 x n error row whose dense solution dW_Q H is exactly Crow:
    dW_Q = Crow H / n (H H = n I); every value used here is exact in fp64."""
    n = len(Crow)
    return (np.asarray(Crow, dtype=np.float64) @ O.sylvester(n) / n)[None, :]


def test_boundary_gap_hand_worked():
    # C = (4, 3, 2, 1) by construction: the gap between the k-th and
    # (k+1)-th largest |C| over the k-th is 1/4 (k = 1), 1/3 (k = 2) and
    # 1/2 (k = 3); no boundary exists for k = 0 or k = n (inf)
    dwq = _row_with_transform([4.0, 3.0, 2.0, 1.0])
    assert np.array_equal(dwq, [[2.5, 0.5, 1.0, 0.0]])
    for k, want in ((0, np.inf), (1, 0.25), (2, 1 / 3), (3, 0.5), (4, np.inf)):
        r = O.init_select(dwq, k, m=0, with_diagnostics=True)
        assert np.array_equal(r["C"], [[4.0, 3.0, 2.0, 1.0]])
        assert r["boundary_gap"][0] == pytest.approx(want, rel=1e-15), k
    # the order of C's columns does not matter, signs neither
    dwq = _row_with_transform([-1.0, 3.0, -4.0, 2.0])
    r = O.init_select(dwq, 2, m=0, with_diagnostics=True)
    assert r["boundary_gap"][0] == pytest.approx(1 / 3, rel=1e-15)
    assert np.array_equal(r["E"][:, 1], [1, 2])


def test_boundary_gap_tie_and_near_tie():
    # a spike row has every |C| equal: the boundary sits inside a tie, gap 0
    spike = np.zeros((1, 16))
    spike[0, 5] = 0.75
    r = O.init_select(spike, 3, m=0, with_diagnostics=True)
    assert r["boundary_gap"][0] == 0.0
    # C = (4, 4 - 4e, 2, 1) with e = 2^-40: the first boundary is e wide
    e = 2.0 ** -40
    dwq = _row_with_transform([4.0, 4.0 - 4.0 * e, 2.0, 1.0])
    r = O.init_select(dwq, 1, m=0, with_diagnostics=True)
    assert r["boundary_gap"][0] == e
    # a row whose k-th largest |C| is zero has no boundary to measure (inf)
    r = O.init_select(_row_with_transform([8.0, 0.0, 0.0, 0.0]), 2, m=0,
                      with_diagnostics=True)
    assert r["boundary_gap"][0] == np.inf


def test_diagnostics_per_row():
    # two rows with hand-worked C and budgets 1 and 2 (w = (5, 5) splits
    # p = 3 into 1.5 and 1.5: floors 1, 1, leftover to row 0 -> (2, 1)).
    # Row 0 keeps |C| = 4, 3 and leaves 0: gap (3 - 0) / 3 = 1; row 1 keeps 4
    # and leaves 3: gap 1/4
    dwq = np.vstack([_row_with_transform([3.0, 4.0, 0.0, 0.0]),
                     _row_with_transform([0.0, 0.0, 4.0, 3.0])])
    r = O.init_select(dwq, 3, m=0, with_diagnostics=True)
    assert np.array_equal(r["budgets"], [2, 1])
    assert np.array_equal(r["boundary_gap"], [1.0, 0.25])
    assert np.array_equal(r["budget_margin"], [0.5, 0.5])


def test_select_orders_rows_and_columns():
    rng = np.random.default_rng(5)
    C = rng.standard_normal((6, 32))
    b = np.array([1, 5, 3, 32, 2, 7])
    row_ptr, E = O.select(C, b)
    assert np.array_equal(np.diff(row_ptr), b)
    for i in range(6):
        seg = E[row_ptr[i]:row_ptr[i + 1]]
        assert np.all(seg[:, 0] == i)
        assert np.all(np.diff(seg[:, 1]) > 0)
        chosen = np.abs(C[i, seg[:, 1]])
        other = np.delete(np.abs(C[i]), seg[:, 1])
        if other.size:
            assert chosen.min() >= other.max()


def test_csc_index():
    rng = np.random.default_rng(6)
    C = rng.standard_normal((20, 16))
    row_ptr, E = O.select(C, rng.integers(1, 8, size=20))
    col_ptr, perm = O.csc(E, 16)
    assert col_ptr[-1] == len(E)
    for j in range(16):
        ks = perm[col_ptr[j]:col_ptr[j + 1]]
        assert np.all(E[ks, 1] == j)
        assert np.all(np.diff(ks) > 0)
    assert np.array_equal(np.sort(perm), np.arange(len(E)))


# ---------------------------------------------------------- golden whole init

def test_init_materialize_fwd_bwd_golden():
    g = read_golden("init_hand_2x4.txt")
    dwq = g["dWq"].astype(np.float32)
    p, m = (int(v) for v in g["p m"][0])
    r = O.init_select(dwq, p, m=m)
    assert np.array_equal(r["budgets"], g["budgets"][0].astype(np.int64))
    assert np.array_equal(r["E"], g["E"].astype(np.int32))
    assert np.array_equal(r["c"], g["c"][0].astype(np.float32))
    dW = O.materialize(r["E"], r["c"], 2, 4, 1.0)
    assert np.array_equal(dW, g["dW"])
    y = O.forward(g["x"], dW)
    dx, dc = O.backward(g["x"], g["dy"], r["E"], r["c"], 2, 4, 1.0)
    assert np.allclose(y, g["y"], atol=1e-15)
    assert np.allclose(dx, g["dx"], atol=1e-15)
    assert np.allclose(dc, g["dc"][0], atol=1e-15)


# ------------------------------------------------------ materialize (O7)

def test_materialize_full_budget_reconstructs_error():
    rng = np.random.default_rng(7)
    d_out, n = 8, 32
    dwq = (0.01 * rng.standard_normal((d_out, n))).astype(np.float32)
    r = O.init_select(dwq, d_out * n, m=3)
    C = O.transform(dwq)
    dW = O.materialize(r["E"], C[r["E"][:, 0], r["E"][:, 1]], d_out, n, 1.0)
    assert np.max(np.abs(dW - dwq.astype(np.float64))) < 1e-12


def test_materialize_single_nonzero_and_alpha():
    n = 64
    H = O.sylvester(n)
    E = np.array([[2, 9]], np.int32)
    dW = O.materialize(E, np.array([0.5], np.float32), 4, n, alpha=2.0)
    expect = np.zeros((4, n))
    expect[2] = 2.0 * 0.5 / n * H[9]
    assert np.array_equal(dW, expect)


def test_materialize_matches_inverse():
    rng = np.random.default_rng(8)
    d_out, n = 6, 16
    C = rng.standard_normal((d_out, n))
    _, E = O.select(C, rng.integers(1, 6, size=d_out))
    c = rng.standard_normal(len(E)).astype(np.float32)
    F = O.scatter_dense(E, c, d_out, n)
    ref = F @ np.linalg.inv(O.sylvester(n))
    assert np.allclose(O.materialize(E, c, d_out, n), ref, rtol=0, atol=1e-13)


# --------------------------------------------------------- fwd / bwd (O8/O9)

def _small_adapter(seed, d_out=12, n=32, T=7, alpha=1.0):
    rng = np.random.default_rng(seed)
    C = rng.standard_normal((d_out, n))
    _, E = O.select(C, rng.integers(3, 9, size=d_out))
    c = rng.standard_normal(len(E)).astype(np.float32)
    x = rng.standard_normal((T, n))
    dy = rng.standard_normal((T, d_out))
    return E, c, x, dy


def test_fwd_bwd_bilinear_identities():
    for alpha in [1.0, 0.7]:
        E, c, x, dy = _small_adapter(11, alpha=alpha)
        dW = O.materialize(E, c, 12, 32, alpha)
        y = O.forward(x, dW)
        dx, dc = O.backward(x, dy, E, c, 12, 32, alpha)
        L = float(np.sum(dy * y))
        assert abs(float(np.sum(dx * x)) - L) < 1e-12 * max(1, abs(L))
        assert abs(float(np.dot(dc, c.astype(np.float64))) - L) < \
            1e-12 * max(1, abs(L))


def test_fwd_bwd_against_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    alpha = 0.9
    E, c, x, dy = _small_adapter(12, alpha=alpha)
    d_out, n = 12, 32
    H = torch.tensor(O.sylvester(n))
    ct = torch.tensor(c.astype(np.float64), requires_grad=True)
    xt = torch.tensor(x, requires_grad=True)
    F = torch.zeros(d_out, n, dtype=torch.float64)
    F = F.index_put((torch.tensor(E[:, 0]).long(), torch.tensor(E[:, 1]).long()),
                    ct)
    dW = alpha * F @ torch.linalg.inv(H)
    y = xt @ dW.T
    y.backward(torch.tensor(dy))
    dx, dc = O.backward(x, dy, E, c, d_out, n, alpha)
    assert np.allclose(y.detach().numpy(),
                       O.forward(x, O.materialize(E, c, d_out, n, alpha)),
                       rtol=0, atol=1e-12)
    assert np.allclose(xt.grad.numpy(), dx, rtol=0, atol=1e-12)
    assert np.allclose(ct.grad.numpy(), dc, rtol=0, atol=1e-12)


def test_dc_finite_difference():
    E, c, x, dy = _small_adapter(13)
    d_out, n = 12, 32

    def L(cv):
        return float(np.sum(dy * O.forward(x, O.materialize(E, cv, d_out, n))))
    _, dc = O.backward(x, dy, E, c, d_out, n)
    c64 = c.astype(np.float64)
    for k in [0, 3, len(c) - 1]:
        e = np.zeros_like(c64)
        e[k] = 0.5
        # L is linear in c: the difference quotient is exact up to rounding
        assert abs((L(c64 + e) - L(c64)) / 0.5 - dc[k]) < 1e-10


def test_backward_dc_rows_matches_full():
    E, c, x, dy = _small_adapter(14)
    _, dc = O.backward(x, dy, E, c, 12, 32, 0.5)
    ks, vals = O.backward_dc_rows(x, dy, E, np.array([0, 5, 11]), 32, 0.5)
    assert np.allclose(vals, dc[ks], rtol=0, atol=1e-13)
    assert set(E[ks, 0]) == {0, 5, 11}


def test_sign_update():
    c = np.array([1.0, -2.0, 0.5, 0.0], np.float32)
    dc = np.array([0.3, -1e-30, 0.0, -4.0], np.float32)
    out = O.sign_update(c, dc)
    expect = np.array([1.0 + np.float32(1e-3), -2.0 - np.float32(1e-3), 0.5,
                       -np.float32(1e-3)], np.float32)
    assert np.array_equal(out, expect)


def test_rel_err():
    assert O.rel_err(np.array([1.0, 2.0]), np.array([1.0, 4.0])) == 0.5
    assert O.rel_err(np.zeros(3), np.zeros(3)) == 0.0


# ------------------------------------------------------------ rank of F

_PRIME = 2147483647


def _rank_mod_p(A):
    """Exact rank over GF(2^31 - 1) by Gaussian elimination; a lower bound
    on the rank over the reals for integer matrices."""
    M = np.array(A, dtype=np.int64) % _PRIME
    rows, cols = M.shape
    r = 0
    for c in range(cols):
        piv = None
        for i in range(r, rows):
            if M[i, c] != 0:
                piv = i
                break
        if piv is None:
            continue
        M[[r, piv]] = M[[piv, r]]
        inv = pow(int(M[r, c]), _PRIME - 2, _PRIME)
        M[r] = (M[r] * inv) % _PRIME
        others = np.nonzero(M[:, c])[0]
        others = others[others != r]
        if len(others):
            f = M[others, c][:, None]
            M[others] = (M[others] - (f * M[r][None, :]) % _PRIME) % _PRIME
        r += 1
        if r == rows:
            break
    return r


@pytest.mark.parametrize("shape", [(48, 48), (24, 64), (64, 24)])
def test_rank_full_with_three_per_row_and_column(shape):
    """QWHA notes 关键设计 1: F is full rank with high probability once every
    row and column holds more than two nonzeros."""
    d_out, n = shape
    for seed in range(20):
        rng = np.random.default_rng(100 + seed)
        mask = np.zeros(shape, bool)
        for i in range(d_out):
            mask[i, rng.choice(n, 3, replace=False)] = True
        for j in range(n):
            need = 3 - int(mask[:, j].sum())
            if need > 0:
                free = np.nonzero(~mask[:, j])[0]
                mask[rng.choice(free, need, replace=False), j] = True
        F = np.where(mask, rng.integers(1, 1000, size=shape), 0)
        assert _rank_mod_p(F) == min(shape)


def test_rank_of_small_config_adapter():
    import synth
    spec = synth.config_specs("c1")[0]
    layer = synth.make_layer(spec, seed=0)
    r = O.init_select(layer.dwq, spec.p, m=3)
    F = np.zeros((spec.d_out, spec.d_in), np.int64)
    # integer surrogate with the same pattern (rank over GF(p) <= real rank)
    rng = np.random.default_rng(0)
    F[r["E"][:, 0], r["E"][:, 1]] = rng.integers(1, 1000, size=len(r["E"]))
    assert _rank_mod_p(F) == 256
    assert np.diff(r["row_ptr"]).min() >= 3


# ------------------------------------------------------------------ selection variants
# ([PN] 关键设计 2, 实验关键数据 › 消融实验 Table 4; [GS] §2.2)

def test_splitmix64_published_outputs():
    # first outputs of SplitMix64 from state 0 (Steele, Lea & Flood 2014; the
    # reference generator's well-known test values)
    got = [int(v) for v in O.splitmix64(0, np.arange(3))]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_counter_form_continues_a_stream():
    # draw n of seed s is draw 0 of the generator advanced by n steps
    n = np.arange(50, dtype=np.uint64)
    seed = 12345
    stepped = [int(O.splitmix64((seed + int(k) * 0x9E3779B97F4A7C15) & ((1 << 64) - 1), 0))
               for k in range(50)]
    assert [int(v) for v in O.splitmix64(seed, n)] == stepped


def test_splitmix64_bits_are_balanced():
    z = O.splitmix64(99, np.arange(200000))
    for b in (0, 17, 40, 63):
        frac = float(np.mean((z >> np.uint64(b)) & np.uint64(1)))
        assert abs(frac - 0.5) < 0.01


def _rand_dwq(d_out, d_in, seed):
    return np.random.default_rng(seed).standard_normal((d_out, d_in)).astype(np.float32)


@pytest.mark.parametrize("p", [0, 1, 7, 40, 128])
def test_magnitude_selection_is_a_threshold(p):
    dwq = _rand_dwq(8, 16, 3)
    r = O.init_select_global(dwq, p, "magnitude")
    C = O.transform(dwq)
    mask = np.zeros(C.shape, bool)
    mask[r["E"][:, 0], r["E"][:, 1]] = True
    assert mask.sum() == p
    if 0 < p < C.size:
        assert np.abs(C[mask]).min() >= np.abs(C[~mask]).max()
    assert np.array_equal(r["c"], C[mask].astype(np.float32))   # row-major = E order


def test_magnitude_captures_at_least_the_adaalloc_energy():
    dwq = _rand_dwq(32, 64, 5)
    p = 300
    C = O.transform(dwq)
    g = O.init_select_global(dwq, p, "magnitude")
    a = O.init_select(dwq, p)
    eg = np.sum(C[g["E"][:, 0], g["E"][:, 1]] ** 2)
    ea = np.sum(C[a["E"][:, 0], a["E"][:, 1]] ** 2)
    assert eg >= ea


def test_magnitude_bruteforce_tiny():
    # every p-subset of a 2x4 matrix: the selection has the largest sum of |C|
    dwq = np.array([[0.3, -1.0, 0.25, 0.5], [2.0, 0.1, -0.4, 0.05]], np.float32)
    C = np.abs(O.transform(dwq)).ravel()
    for p in range(9):
        r = O.init_select_global(dwq, p, "magnitude")
        got = sorted((r["E"][:, 0] * 4 + r["E"][:, 1]).tolist())
        best = max(itertools.combinations(range(8), p), key=lambda s: (sum(C[list(s)]), [-i for i in s]))
        assert np.isclose(sum(C[got]), sum(C[list(best)]), rtol=0, atol=1e-12)


def test_magnitude_ties_go_in_row_major_order():
    # one spike per row: every |C| of a row is equal; rows 1 and 2 share a value
    dwq = np.zeros((3, 8), np.float32)
    dwq[0, 5], dwq[1, 2], dwq[2, 7] = 0.5, 2.0, -2.0
    r = O.init_select_global(dwq, 11, "magnitude")
    flat = (r["E"][:, 0] * 8 + r["E"][:, 1]).tolist()
    assert flat == list(range(8, 19))     # all of row 1, then the first 3 of row 2
    assert r["row_ptr"].tolist() == [0, 0, 8, 11]


def test_random_selection_ignores_the_data_and_follows_the_draws():
    a = O.init_select_global(_rand_dwq(8, 16, 1), 30, "random", seed=11)
    b = O.init_select_global(_rand_dwq(8, 16, 2), 30, "random", seed=11)
    assert np.array_equal(a["E"], b["E"])
    c = O.init_select_global(_rand_dwq(8, 16, 1), 30, "random", seed=12)
    assert not np.array_equal(a["E"], c["E"])
    draws = O.splitmix64(11, np.arange(128)).reshape(8, 16)
    mask = np.zeros((8, 16), bool)
    mask[a["E"][:, 0], a["E"][:, 1]] = True
    assert draws[mask].max() < draws[~mask].min()     # the 30 smallest draws


def test_random_selection_is_uniform():
    counts = np.zeros(64)
    for seed in range(400):
        r = O.init_select_global(np.zeros((8, 8), np.float32), 16, "random", seed=seed)
        counts[r["E"][:, 0] * 8 + r["E"][:, 1]] += 1
    freq = counts / 400
    assert np.all(np.abs(freq - 0.25) < 0.1)


def test_global_selection_full_and_empty_budgets():
    dwq = _rand_dwq(4, 8, 9)
    for strategy in ("magnitude", "random"):
        full = O.init_select_global(dwq, 32, strategy, seed=1)
        assert full["E"].shape == (32, 2) and full["row_ptr"].tolist() == [0, 8, 16, 24, 32]
        empty = O.init_select_global(dwq, 0, strategy, seed=1)
        assert empty["E"].shape == (0, 2) and empty["col_ptr"].tolist() == [0] * 9


# ---------------------------------------------- refinement with a Hessian (O11-O14)

def _calib(N, d_in, seed, spread=1.0):
    """Calibration tokens with per-channel scales spread over e^(+-spread)."""
    rng = np.random.default_rng(seed)
    scale = np.exp(spread * rng.standard_normal(d_in))
    return rng.standard_normal((N, d_in)) * scale


def test_refine_golden():
    g = read_golden("refine_hand_2x2.txt")
    p, m = (int(v) for v in g["p m"][0])
    r = O.init_select_calibrated(g["dWq"].astype(np.float32), g["Hs"], p, m=m)
    assert np.allclose(r["w"] ** 2, g["w squared"][0], rtol=1e-14)
    assert r["budgets"].tolist() == g["budgets"][0].astype(int).tolist()
    assert np.array_equal(r["E"], g["E"].astype(np.int32))
    assert np.array_equal(r["c_dense"], g["c dense"][0].astype(np.float32))
    x = g["x numerator"][0] / g["x denominator"][0]
    assert np.allclose(r["x"], x, rtol=1e-14, atol=0)
    assert np.array_equal(r["c"], x.astype(np.float32))


def test_hessian_is_the_sum_of_token_outer_products():
    X = _calib(7, 8, 1)
    Hs = np.zeros((8, 8))
    for t in range(7):
        Hs += np.outer(X[t], X[t])
    assert np.allclose(O.hessian(X), Hs, rtol=1e-13, atol=1e-13)


def test_activation_error_norms_are_output_error_norms():
    dwq = _rand_dwq(9, 16, 2)
    X = _calib(40, 16, 3)
    direct = np.linalg.norm(dwq.astype(np.float64) @ X.T, axis=1)    # ||dW_Q[i] X||
    assert np.allclose(O.activation_error_norms(dwq, O.hessian(X)), direct, rtol=1e-12)
    # identity Hessian: the plain row norms
    assert np.allclose(O.activation_error_norms(dwq, np.eye(16)), O.row_norms(dwq), rtol=1e-14)


@pytest.mark.parametrize("s", [1.0, 4.0, 0.37])
def test_refine_with_isotropic_hessian_is_the_dense_solution(s):
    dwq = _rand_dwq(12, 32, 5)
    r = O.init_select_calibrated(dwq, s * np.eye(32), 120, m=3)
    base = O.init_select(dwq, 120, m=3)
    for key in ("row_ptr", "E", "col_ptr", "csc_perm"):
        assert np.array_equal(r[key], base[key]), key
    C = O.transform(dwq)
    assert np.allclose(r["x"], C[r["E"][:, 0], r["E"][:, 1]], rtol=1e-12, atol=1e-15)


def test_refine_matches_lstsq_on_the_unreduced_problem():
    # min_x ||(dW_Q[i] - x (H/n)[S,:]) X^T||: no Hessian, no normal equations
    d_out, d_in = 10, 32
    dwq = _rand_dwq(d_out, d_in, 6)
    X = _calib(96, d_in, 7, spread=1.5)
    r = O.init_select_calibrated(dwq, O.hessian(X), 130, m=3)
    H = O.sylvester(d_in)
    assert r["ok"].all()
    for i in range(d_out):
        a, b = r["row_ptr"][i], r["row_ptr"][i + 1]
        S = r["E"][a:b, 1]
        D = (H / d_in)[S, :] @ X.T
        target = dwq[i].astype(np.float64) @ X.T
        sol, *_ = np.linalg.lstsq(D.T, target, rcond=None)
        assert np.allclose(r["x"][a:b], sol, rtol=1e-9, atol=1e-12 * np.abs(sol).max())


def test_refine_never_raises_the_layer_error_and_usually_lowers_it():
    d_out, d_in = 16, 64
    dwq = _rand_dwq(d_out, d_in, 8)
    X = _calib(200, d_in, 9, spread=1.0)
    r = O.init_select_calibrated(dwq, O.hessian(X), 400, m=3)
    H = O.sylvester(d_in)
    lower = 0
    for i in range(d_out):     # per channel: refined x is optimal over its support
        a, b = r["row_ptr"][i], r["row_ptr"][i + 1]
        rows = slice(a, b)
        def err(vals):
            resid = dwq[i].astype(np.float64) - vals @ (H / d_in)[r["E"][rows, 1], :]
            return float(np.sum((resid @ X.T) ** 2))
        e_ref, e_dense = err(r["x"][rows]), err(r["c_dense"][rows].astype(np.float64))
        assert e_ref <= e_dense * (1 + 1e-12)
        lower += e_ref < 0.99 * e_dense
    assert lower >= d_out // 2
    assert O.layer_output_error(dwq, X, r["E"], r["c"]) < \
        O.layer_output_error(dwq, X, r["E"], r["c_dense"])


def test_refine_full_budget_reconstructs_for_any_hessian():
    d_out, d_in = 4, 16
    dwq = _rand_dwq(d_out, d_in, 10)
    X = _calib(50, d_in, 11, spread=2.0)
    r = O.init_select_calibrated(dwq, O.hessian(X), d_out * d_in, m=3)
    C = O.transform(dwq)
    assert np.allclose(r["x"], C.ravel(), rtol=1e-8, atol=1e-10 * np.abs(C).max())
    assert O.layer_output_error(dwq, X, r["E"], r["x"]) < 1e-14 * np.sum((dwq @ X.T) ** 2)


def test_refine_is_scale_invariant_in_the_calibration_set():
    dwq = _rand_dwq(8, 32, 12)
    X = _calib(80, 32, 13)
    a = O.init_select_calibrated(dwq, O.hessian(X), 90, m=3)
    b = O.init_select_calibrated(dwq, O.hessian(4.0 * X), 90, m=3)
    assert np.array_equal(a["E"], b["E"])
    assert np.allclose(b["w"], 4.0 * a["w"], rtol=1e-13)
    assert np.allclose(a["x"], b["x"], rtol=1e-10)


def test_cholesky_matches_numpy_and_flags_indefinite():
    rng = np.random.default_rng(14)
    B = rng.standard_normal((30, 12))
    A = B.T @ B
    L, ok = O.cholesky_lower(A)
    assert ok and np.allclose(L, np.linalg.cholesky(A), rtol=1e-12, atol=1e-13)
    low_rank = B[:5].T @ B[:5]             # rank 5 < 12: a pivot collapses to rounding
    assert not O.cholesky_lower(low_rank)[1]
    indef = A.copy()
    indef[3, 3] = -1.0
    assert not O.cholesky_lower(indef)[1]


def test_refine_rows_without_a_definite_system_keep_the_dense_solution():
    # 6 calibration tokens: rank(Hs) = 6, so rows with more than 6 positions
    # have a singular G[S,S]
    d_out, d_in = 6, 32
    dwq = _rand_dwq(d_out, d_in, 15)
    X = _calib(6, d_in, 16)
    r = O.init_select_calibrated(dwq, O.hessian(X), 40, m=3)
    big = r["budgets"] > 6
    assert big.any() and (~big).any()
    assert np.array_equal(r["ok"], ~big)
    rows = np.repeat(np.arange(d_out), r["budgets"])
    assert np.array_equal(r["c"][big[rows]], r["c_dense"][big[rows]])
    # damping makes every system definite
    d = O.init_select_calibrated(dwq, O.hessian(X), 40, m=3, damp=0.01)
    assert d["ok"].all()
    Hd = O.damped(O.hessian(X), 0.01)
    assert np.allclose(np.diag(Hd) - np.diag(O.hessian(X)),
                       0.01 * np.mean(np.diag(O.hessian(X))), rtol=1e-12)


# ---------------------------------------------- quantized base layer (O15-O17)

import synth  # noqa: E402  (the fixture's quantizer and code storage)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_unpack_codes_golden(bits):
    g = read_golden("packed_codes.txt")
    codes = g[f"b{bits} codes"][0].astype(np.int64)
    words = g[f"b{bits} words"][0].astype(np.uint64).astype(np.uint32)[None, :]
    assert np.array_equal(O.unpack_codes(words, len(codes), bits)[0], codes)
    assert np.array_equal(synth.pack_codes(codes[None, :].astype(np.uint8), bits), words)


def test_dequantize_golden():
    g = read_golden("packed_codes.txt")
    q = g["dq codes"].astype(np.int64)
    w = O.dequantize(q, g["dq scales"], g["dq zeros"], 2)
    assert np.array_equal(w, g["dq weights"].astype(np.float32))


@pytest.mark.parametrize("bits,group", [(2, 64), (3, 128), (4, 128), (4, 64), (8, 32)])
def test_dequantized_codes_are_the_quantizer_output(bits, group):
    rng = np.random.default_rng(bits * 100 + group)
    w0 = (0.02 * rng.standard_normal((12, 256))).astype(np.float32)
    q, s, z = synth.rtn_codes(w0, bits, group)
    words = synth.pack_codes(q, bits)
    got = O.dequantize(O.unpack_codes(words, 256, bits), s, z, group)
    assert np.array_equal(got, synth.rtn_quantize(w0, bits, group))     # bit for bit


def test_merge_and_layer_forward_definitions():
    rng = np.random.default_rng(3)
    d_out, d_in = 6, 16
    W_Q = rng.standard_normal((d_out, d_in)).astype(np.float32)
    dwq = _rand_dwq(d_out, d_in, 4)
    r = O.init_select(dwq, 30, m=3)
    F = O.scatter_dense(r["E"], r["c"], d_out, d_in)
    H = O.sylvester(d_in)
    merged = O.merge_weights(W_Q, r["E"], r["c"], 0.7)
    assert np.allclose(merged, W_Q + 0.7 * F @ H / d_in, rtol=1e-13, atol=1e-13)
    x = rng.standard_normal((5, d_in))
    y = O.layer_forward(x, W_Q, r["E"], r["c"], 0.7)
    # base GEMM plus the adapter's own forward (FWHT, then the sparse product)
    z = x @ H / d_in
    assert np.allclose(y, x @ W_Q.astype(np.float64).T + 0.7 * z @ F.T, rtol=1e-12, atol=1e-12)
    # no adapter: the plain quantized layer
    y0 = O.layer_forward(x, W_Q, r["E"], np.zeros_like(r["c"]), 0.7)
    assert np.allclose(y0, x @ W_Q.astype(np.float64).T, rtol=1e-13, atol=1e-13)


# ---------------------------------------------- widths that are not powers of two

@pytest.mark.parametrize("d_in", [12, 24, 40, 96, 112, 14336])
def test_block_size_and_structure(d_in):
    b = O.block_size(d_in)
    assert b & (b - 1) == 0 and d_in % b == 0 and (d_in // b) % 2 == 1
    if d_in <= 112:
        from scipy.linalg import block_diag, hadamard
        H = O.wht_matrix(d_in)
        assert np.array_equal(H, block_diag(*[hadamard(b).astype(np.float64)] * (d_in // b)))
        assert np.array_equal(H @ H.T, b * np.eye(d_in))        # H^-1 = H / b
        A = np.random.default_rng(d_in).standard_normal((5, d_in))
        assert np.allclose(O.wht(A, d_in), A @ H, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 64, 1024])
def test_wht_matrix_is_sylvester_for_powers_of_two(n):
    assert np.array_equal(O.wht_matrix(n), O.sylvester(n))


@pytest.mark.parametrize("d_in", [12, 40])
def test_full_budget_reconstructs_at_block_widths(d_in):
    dwq = _rand_dwq(5, d_in, d_in)
    r = O.init_select(dwq, 5 * d_in, m=3)
    C = O.transform(dwq)
    dW = O.materialize(r["E"], C[r["E"][:, 0], r["E"][:, 1]], 5, d_in, 1.0)
    assert np.allclose(dW, dwq.astype(np.float64), rtol=0, atol=1e-14)


def test_fwd_bwd_against_torch_autograd_at_a_block_width():
    torch = pytest.importorskip("torch")
    alpha, d_out, n = 0.7, 9, 24                    # b = 8, three blocks
    dwq = _rand_dwq(d_out, n, 31)
    r = O.init_select(dwq, 60, m=3)
    E, c = r["E"], r["c"]
    rng = np.random.default_rng(32)
    x = rng.standard_normal((7, n))
    dy = rng.standard_normal((7, d_out))
    H = torch.tensor(O.wht_matrix(n))
    ct = torch.tensor(c.astype(np.float64), requires_grad=True)
    xt = torch.tensor(x, requires_grad=True)
    F = torch.zeros(d_out, n, dtype=torch.float64)
    F = F.index_put((torch.tensor(E[:, 0]).long(), torch.tensor(E[:, 1]).long()), ct)
    y = xt @ (alpha * F @ torch.linalg.inv(H)).T
    y.backward(torch.tensor(dy))
    dx, dc = O.backward(x, dy, E, c, d_out, n, alpha)
    assert np.allclose(y.detach().numpy(), O.forward(x, O.materialize(E, c, d_out, n, alpha)),
                       rtol=0, atol=1e-12)
    assert np.allclose(xt.grad.numpy(), dx, rtol=0, atol=1e-12)
    assert np.allclose(ct.grad.numpy(), dc, rtol=0, atol=1e-12)


def test_refine_matches_lstsq_at_a_block_width():
    d_out, d_in = 6, 48                             # b = 16, three blocks
    dwq = _rand_dwq(d_out, d_in, 33)
    X = _calib(120, d_in, 34)
    r = O.init_select_calibrated(dwq, O.hessian(X), 80, m=3)
    H = O.wht_matrix(d_in)
    b = O.block_size(d_in)
    for i in range(d_out):
        a, e = r["row_ptr"][i], r["row_ptr"][i + 1]
        S = r["E"][a:e, 1]
        D = (H / b)[S, :] @ X.T
        sol, *_ = np.linalg.lstsq(D.T, dwq[i].astype(np.float64) @ X.T, rcond=None)
        assert np.allclose(r["x"][a:e], sol, rtol=1e-9, atol=1e-12 * np.abs(sol).max())

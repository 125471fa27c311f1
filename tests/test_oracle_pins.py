"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each pin is a hand-worked
value, an independent algorithm (the textbook Gram-Schmidt Babai, the GPTQ
solve form, exhaustive enumeration), a closed form, or an invariant the pages
state.  A dropped term, a wrong sign or index or a transposed operand in the
oracle breaks at least one of them.
"""
import numpy as np
import pytest

import oracle as O
from _golden import load

RNG = np.random.default_rng(12345)


def _rand_problem(rng, m, n, N, spread=0.5, outl=0):
    X = rng.standard_normal((n, N)) * rng.lognormal(0, spread, (n, 1))
    if outl:
        X[rng.choice(n, outl, replace=False)] *= 20
    W = rng.standard_normal((m, n)) * 0.02
    return W, X


# ---------------------------------------------------------------- golden


def test_golden_three_column_nearest_plane():
    g = load("handworked_nearest_plane_3col.txt")
    H, w = g["H"], g["w"]
    L, info = O.cholesky_lower(H)
    assert info == 0
    np.testing.assert_allclose(L, g["L"], atol=1e-15)
    res = O.quant_layer(w[None, :], H=H, grid_kind="sym", bits=int(g["bits"]),
                        group=0, damp=0.0)
    np.testing.assert_allclose(res["scales"][0, 0], g["step"], rtol=1e-15)
    np.testing.assert_array_equal(res["codes"][0], g["codes"])
    np.testing.assert_allclose(res["rho"][0], g["rho"], atol=1e-12)
    assert res["loss"] == pytest.approx(g["loss"], rel=1e-12)
    assert res["loss_damped"] == pytest.approx(g["loss"], rel=1e-12)
    assert res["bound"] == pytest.approx(g["bound"], rel=1e-12)
    s = np.full(3, g["step"])
    # round-to-nearest is the sweep without feedback
    np.testing.assert_array_equal(np.rint(w / s), g["rtn_codes"])
    assert O.proxy_loss(w[None], (s * g["rtn_codes"])[None], H) == \
        pytest.approx(g["rtn_loss"], rel=1e-12)
    # closest point, two ways
    z_fp, loss_fp = O.cvp_enumerate(L, w, s, res["loss_damped"])
    z_box, loss_box = O.cvp_box(H, w, s, np.rint(w / s), 3)
    assert loss_fp == pytest.approx(g["cvp_loss"], rel=1e-12)
    assert loss_box == pytest.approx(g["cvp_loss"], rel=1e-12)
    assert O.gamma_ratio(s, np.diag(L) ** 2) == pytest.approx(g["gamma"])
    # the other two sweep forms
    np.testing.assert_array_equal(O.gptq_obs_sweep(w[None], H, s[None])[0],
                                  g["codes"])
    np.testing.assert_array_equal(O.babai_gram_schmidt(L.T, w, s), g["codes"])
    # column spacing c = 1 gives alpha = 1/l_kk = 0.5
    rc = O.quant_layer(w[None, :], H=H, grid_kind="colspacing", c=1.0,
                       damp=0.0)
    np.testing.assert_allclose(rc["scales"], [0.5, 0.5, 0.5], rtol=1e-15)
    np.testing.assert_array_equal(rc["codes"][0], g["codes"])


def test_golden_asym_tie_rounds_to_even():
    g = load("handworked_asym_tie.txt")
    res = O.quant_layer(g["w"][None], H=g["H"], grid_kind="asym",
                        bits=int(g["bits"]), group=0, damp=0.0)
    assert res["scales"][0, 0] == g["step"]
    assert res["zeros"][0, 0] == g["zero"]
    np.testing.assert_array_equal(res["codes"][0], g["codes"])
    assert res["loss"] == g["loss"]


def test_step_closed_forms_per_group():
    W = np.array([[0.1, -0.7, 0.3, 0.2],
                  [0.0, 0.0, -0.5, 0.25]])
    # steps are stored (and computed) in float32: compare at that precision
    f32 = dict(rtol=2 ** -23)
    s, z = O.grid_steps(W, "sym", 4, 2)
    np.testing.assert_allclose(s, [[0.7 / 7, 0.3 / 7], [1.0, 0.5 / 7]], **f32)
    assert z is None
    s, z = O.grid_steps(W, "asym", 3, 2)
    # row0 g0: lo=-0.7 hi=0.1; g1: lo=0 hi=0.3; row1 g0 all zero; g1 lo=-.5 hi=.25
    np.testing.assert_allclose(s, [[0.8 / 7, 0.3 / 7], [1.0, 0.75 / 7]], **f32)
    np.testing.assert_array_equal(z, [[np.rint(0.7 / (0.8 / 7)), 0],
                                      [0, np.rint(0.5 / (0.75 / 7))]])
    s, _ = O.grid_steps(W, "sym", 2, 0)
    np.testing.assert_allclose(s, [[0.7], [0.5]], **f32)
    # the stored value is exactly the float32 quotient
    assert s[0, 0] == float(np.float32(np.float32(0.7) / np.float32(1)))


# ----------------------------------------------- three forms of one method


@pytest.mark.parametrize("grid_kind,bits,group", [
    ("sym", 4, 0), ("sym", 3, 4), ("asym", 4, 4), ("sym", 2, 2),
    ("colspacing", 0, 0)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_three_sweep_forms_agree(grid_kind, bits, group, seed):
    """[GEOM 2.2, Theorem 4 and the redundancy of an extra propagation]:
    the SIC form (original-weight error, Cholesky coefficients), the GPTQ
    form (running error, explicit H_FF^-1 H_Fk solve) and the textbook
    Gram-Schmidt Babai on the stacked tall basis give the same integers."""
    rng = np.random.default_rng(seed)
    m, n, N = 5, 12, 40
    W, X = _rand_problem(rng, m, n, N, outl=1)
    damp = 0.05
    res = O.quant_layer(W, X=X, grid_kind=grid_kind, bits=bits, group=group,
                        c=0.3, damp=damp)
    Sp = res["Sp"]
    zb = O.gptq_obs_sweep(res["Wp"], res["Hd"], Sp)
    np.testing.assert_array_equal(zb, res["Z"])
    # Theorem 1: the tall basis [sqrt2 X^T; sqrt(lam) I] spans the same
    # closest-vector instance as the square Cholesky factor.
    A = np.vstack([np.sqrt(2.0) * X.T, np.sqrt(res["lam"]) * np.eye(n)])
    for r in range(m):
        zg = O.babai_gram_schmidt(A, res["Wp"][r], Sp[r])
        np.testing.assert_array_equal(zg, res["Z"][r])


def test_tall_basis_qr_reproduces_cholesky_factor():
    """[GEOM 2.1, Theorem 1]: R of a QR of the tall basis equals L^T up to the
    signs of its rows."""
    rng = np.random.default_rng(7)
    n, N = 9, 30
    _, X = _rand_problem(rng, 1, n, N)
    lam = 0.3
    A = np.vstack([np.sqrt(2.0) * X.T, np.sqrt(lam) * np.eye(n)])
    R = np.linalg.qr(A, mode="r")
    Hd = O.hessian(X) + lam * np.eye(n)
    L, info = O.cholesky_lower(Hd)
    assert info == 0
    np.testing.assert_allclose(np.abs(R), np.abs(L.T), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------- loss and bound


def test_loss_is_output_error_and_identity():
    """[WSIC 1]: the objective is the output error ||W X - W^ X||^2; with
    H = 2 X X^T the proxy loss is 2 ||(W - W^) X||_F^2.  The damped loss
    equals sum rho^2 s^2 D (coordinates of R Delta), and each row stays under
    the Theorem 5 bound [GEOM 2.3]."""
    rng = np.random.default_rng(3)
    m, n, N = 16, 24, 200
    W, X = _rand_problem(rng, m, n, N)
    res = O.quant_layer(W, X=X, grid_kind="sym", bits=3, group=8, damp=0.01)
    Dl = res["W0"] - res["What"]
    assert res["loss"] == pytest.approx(2.0 * np.sum((Dl @ X) ** 2), rel=1e-10)
    ident = np.sum(res["rho"] ** 2 * res["Sp"] ** 2 * res["D"][None, :])
    assert res["loss_damped"] == pytest.approx(ident, rel=1e-10)
    assert res["loss"] == pytest.approx(
        res["loss_damped"] - res["lam"] * np.sum(Dl ** 2), rel=1e-10)
    Dp = Dl[:, res["pi"]]
    per_row = np.sum((Dp @ res["L"]) ** 2, axis=1)
    bound_row = 0.25 * np.sum(res["Sp"] ** 2 * res["D"][None, :], axis=1)
    assert np.all(per_row <= bound_row * (1 + 1e-12))
    assert res["loss_damped"] <= res["bound"]


def test_certificate_equals_residual():
    rng = np.random.default_rng(4)
    W, X = _rand_problem(rng, 10, 20, 100, outl=2)
    res = O.quant_layer(W, X=X, grid_kind="asym", bits=4, group=4, damp=0.01)
    Dp = (res["W0"] - res["What"])[:, res["pi"]]
    G = O.certificate(Dp, res["L"], res["Sp"])
    np.testing.assert_allclose(G, res["rho"], atol=1e-10)
    assert np.max(np.abs(G)) <= 0.5 + 1e-12


# ----------------------------------------------------- special cases


def test_diagonal_hessian_is_round_to_nearest():
    """A diagonal Hessian is an orthogonal lattice basis: nearest plane is
    coordinate-wise rounding [GEOM 2.2]."""
    rng = np.random.default_rng(5)
    m, n = 7, 16
    W = rng.standard_normal((m, n))
    H = np.diag(rng.uniform(0.5, 3.0, n))
    res = O.quant_layer(W, H=H, grid_kind="sym", bits=4, group=4, damp=0.0)
    S = O.expand_group_steps(res["scales"], n)
    np.testing.assert_array_equal(res["Z"], np.rint(W / S))


def test_lattice_points_are_fixed_points():
    rng = np.random.default_rng(6)
    m, n = 6, 16
    Z = rng.integers(-7, 8, (m, n)).astype(float)
    Z[:, 0] = 7.0  # max |z| = 7 in each row: the symmetric 4-bit step is s
    # dyadic steps: 7 s and 7 s / 7 are exact in float32, so the float32 step
    # recovered from W is s itself
    s = rng.integers(2 ** 12, 2 ** 16, (m, 1)) * 2.0 ** -20
    W = Z * s
    _, X = _rand_problem(rng, 1, n, 60)
    res = O.quant_layer(W, X=X, grid_kind="sym", bits=4, group=0, damp=0.01)
    np.testing.assert_array_equal(res["Z"], Z)
    assert abs(res["loss"]) < 1e-20


def test_hessian_scale_invariance():
    rng = np.random.default_rng(8)
    W, X = _rand_problem(rng, 8, 20, 80)
    H = O.hessian(X)
    a = O.quant_layer(W, H=H, grid_kind="sym", bits=3, group=4, damp=0.02)
    b = O.quant_layer(W, H=H * 37.5, grid_kind="sym", bits=3, group=4,
                      damp=0.02)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    assert b["loss"] == pytest.approx(37.5 * a["loss"], rel=1e-9)


def test_row_permutation_equivariance():
    rng = np.random.default_rng(9)
    W, X = _rand_problem(rng, 12, 16, 80)
    p = rng.permutation(12)
    a = O.quant_layer(W, X=X, grid_kind="asym", bits=3, group=8)
    b = O.quant_layer(W[p], X=X, grid_kind="asym", bits=3, group=8)
    np.testing.assert_array_equal(a["codes"][p], b["codes"])


@pytest.mark.parametrize("block", [1, 3, 8, 16, 64])
def test_blocked_equals_plain(block):
    rng = np.random.default_rng(10)
    W, X = _rand_problem(rng, 20, 40, 160, outl=2)
    a = O.quant_layer(W, X=X, grid_kind="sym", bits=4, group=8)
    b = O.quant_layer(W, X=X, grid_kind="sym", bits=4, group=8, block=block)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["rho"], b["rho"], atol=1e-9)


@pytest.mark.parametrize("seed", range(6))
def test_babai_against_exhaustive_closest_point(seed):
    """Babai is a heuristic for the closest-vector problem [GEOM 2.1-2.3]:
    exact enumeration is never worse than it, and Babai's loss
    stays within the Theorem 5 bound and the relative (gamma) bound."""
    rng = np.random.default_rng(100 + seed)
    n = 5 if seed % 2 else 6
    W, X = _rand_problem(rng, 6, n, 3 * n, spread=1.0)
    res = O.quant_layer(W, X=X, grid_kind="sym", bits=2, group=0, damp=0.05)
    L, D = res["L"], res["D"]
    for r in range(W.shape[0]):
        w, s = res["Wp"][r], res["Sp"][r]
        zp = res["Z"][r][res["pi"]]
        d = w - s * zp
        loss_b = float(d @ (L @ (L.T @ d)))
        z_c, loss_c = O.cvp_enumerate(L, w, s, loss_b)
        Hp = res["Hd"][np.ix_(res["pi"], res["pi"])]
        z_x, loss_x = O.cvp_box(Hp, w, s, zp, 2)
        assert loss_c <= loss_b * (1 + 1e-12)
        assert loss_c <= loss_x * (1 + 1e-12)
        if np.max(np.abs(z_c - zp)) <= 2:
            assert loss_x == pytest.approx(loss_c, rel=1e-10)
        assert loss_b <= 0.25 * np.sum(s ** 2 * D) * (1 + 1e-12)
        assert loss_b <= O.gamma_ratio(s, D) * loss_c * (1 + 1e-9) + 1e-300


# ------------------------------------------------------------- factor


def test_cholesky_pin():
    rng = np.random.default_rng(11)
    _, X = _rand_problem(rng, 1, 30, 100)
    Hd = O.hessian(X) + 0.1 * np.eye(30)
    L, info = O.cholesky_lower(Hd)
    assert info == 0
    assert np.all(np.triu(L, 1) == 0)
    assert np.all(np.diag(L) > 0)
    np.testing.assert_allclose(L @ L.T, Hd, rtol=1e-12, atol=1e-12 * np.max(Hd))


def test_cholesky_failure_reports_minor():
    A = np.diag([1.0, 2.0, -1.0, 1.0])
    _, info = O.cholesky_lower(A)
    assert info == 3
    B = np.array([[1.0, 2.0], [2.0, 1.0]])  # det < 0
    _, info = O.cholesky_lower(B)
    assert info == 2
    res = O.quant_layer(np.ones((2, 4)), H=np.zeros((4, 4)) - np.eye(4),
                        damp=0.0)
    assert res["info"] == 1
    # a NaN pivot is a failure at its column (reading; pages are silent)
    C = np.eye(6)
    C[4, 1] = C[1, 4] = np.nan
    _, info = O.cholesky_lower(C)
    assert info == 5


def test_spectral_hessian_closed_form_factor():
    """The given-H workload H = L0 diag(lam) L0^T has Cholesky factor
    L0 diag(sqrt lam) (uniqueness of the factor with positive diagonal)."""
    rng = np.random.default_rng(12)
    n = 64
    L0 = np.tril(rng.standard_normal((n, n)) / np.sqrt(n), -1) + np.eye(n)
    lam = np.arange(1, n + 1) ** -1.2
    H = (L0 * lam) @ L0.T
    L, info = O.cholesky_lower(H)
    assert info == 0
    np.testing.assert_allclose(L, L0 * np.sqrt(lam), rtol=1e-9, atol=1e-12)
    # WaterSIC spacing alpha = c / l_kk makes every Gram-Schmidt norm c:
    # damped loss = c^2 sum rho^2
    W = rng.standard_normal((8, n)) * 0.01
    res = O.quant_layer(W, H=H, grid_kind="colspacing", c=0.004, damp=0.0)
    np.testing.assert_allclose(res["scales"], 0.004 / np.sqrt(lam), rtol=1e-9)
    assert res["loss_damped"] == pytest.approx(
        0.004 ** 2 * np.sum(res["rho"] ** 2), rel=1e-9)


# ---------------------------------------------------------------- orders


def test_front_to_back_is_the_reversed_problem():
    rng = np.random.default_rng(13)
    W, X = _rand_problem(rng, 8, 16, 64)
    H = O.hessian(X)
    a = O.quant_layer(W, H=H, grid_kind="sym", bits=3, group=0,
                      order="front_to_back")
    b = O.quant_layer(W[:, ::-1], H=H[::-1, ::-1], grid_kind="sym", bits=3,
                      group=0)
    np.testing.assert_array_equal(a["codes"], b["codes"][:, ::-1])
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-10)


def test_explicit_perm_matches_permuted_problem():
    rng = np.random.default_rng(14)
    W, X = _rand_problem(rng, 8, 12, 64)
    H = O.hessian(X)
    p = rng.permutation(12)
    a = O.quant_layer(W, H=H, grid_kind="sym", bits=4, group=0, order="perm",
                      perm=p)
    b = O.quant_layer(W[:, p], H=H[np.ix_(p, p)], grid_kind="sym", bits=4,
                      group=0)
    np.testing.assert_array_equal(a["codes"][:, p], b["codes"])


def test_act_order_processes_largest_diagonal_first():
    H = np.diag([1.0, 5.0, 3.0, 5.0])
    p = O.order_permutation("act_order", 4, H)
    # first processed = last position: column 1 (5.0, lower index), then 3
    assert list(p[::-1]) == [1, 3, 2, 0]


def test_min_pivot_on_a_diagonal_matrix_sorts_ascending():
    """[GEOM 2.3] min-pivot order on a diagonal H: the Schur complement never
    changes, so the pivots are the diagonal in increasing order (ties by the
    lower index) and the largest entry is processed first."""
    H = np.diag([3.0, 1.0, 2.0, 1.0, 5.0])
    pi, piv, info = O.min_pivot_order(H)
    assert info == 0
    assert list(pi) == [1, 3, 2, 0, 4]
    np.testing.assert_array_equal(piv, [1.0, 1.0, 2.0, 3.0, 5.0])
    np.testing.assert_array_equal(O.order_permutation("min_pivot", 5, H), pi)


def test_min_pivot_handworked_3x3():
    """tests/golden/handworked_min_pivot_3x3.txt: the order, the pivots and
    the lower trace than the natural order, worked on paper."""
    g = load("handworked_min_pivot_3x3.txt")
    pi, piv, info = O.min_pivot_order(g["H"])
    assert info == 0
    np.testing.assert_array_equal(pi, g["order"].astype(np.int64))
    np.testing.assert_allclose(piv, g["pivots"], rtol=1e-15)
    L = O.cholesky_lower(g["H"])[0]
    np.testing.assert_allclose(np.diag(L) ** 2, g["natural_pivots"], rtol=1e-15)
    assert piv.sum() < g["natural_pivots"].sum()


def test_min_pivot_matches_greedy_determinant_ratios():
    """Brute force: the Schur-complement diagonal of candidate i after the
    chosen set S is det H[S+i] / det H[S] (a ratio of principal minors), so
    the greedy order and its pivots follow from determinants alone."""
    rng = np.random.default_rng(31)
    for n in (2, 3, 5, 7):
        _, X = _rand_problem(rng, 1, n, 3 * n, spread=0.8)
        H = O.hessian(X)
        chosen, ratios = [], []
        for _ in range(n):
            base = np.linalg.det(H[np.ix_(chosen, chosen)]) if chosen else 1.0
            cand = [(np.linalg.det(H[np.ix_(chosen + [i], chosen + [i])]) / base, i)
                    for i in range(n) if i not in chosen]
            r, q = min(cand)
            chosen.append(q)
            ratios.append(r)
        pi, piv, info = O.min_pivot_order(H)
        assert info == 0
        assert list(pi) == chosen, n
        np.testing.assert_allclose(piv, ratios, rtol=1e-9)


def test_min_pivot_pivots_are_the_permuted_factor():
    """The pivots are D of the LDL^T of the permuted Hessian, i.e. the squared
    diagonal of its Cholesky factor (numpy's), and each is the smallest
    Schur diagonal among the columns still open at its step."""
    rng = np.random.default_rng(32)
    _, X = _rand_problem(rng, 1, 40, 160, spread=0.7, outl=3)
    H = O.hessian(X)
    pi, piv, info = O.min_pivot_order(H)
    assert info == 0 and sorted(pi) == list(range(40))
    Lp = np.linalg.cholesky(H[np.ix_(pi, pi)])
    np.testing.assert_allclose(piv, np.diag(Lp) ** 2, rtol=1e-10)
    # Schur diagonal of position i at step k = Hp_ii - sum_{p<k} L_ip^2
    Hp = H[np.ix_(pi, pi)]
    sq = np.cumsum(Lp ** 2, axis=1)
    for k in range(40):
        schur = np.diag(Hp)[k:] - (sq[k:, k - 1] if k else 0.0)
        assert piv[k] <= schur.min() * (1 + 1e-12)


def test_min_pivot_2x2_takes_the_smaller_trace():
    """2 x 2 closed form: the trace of D is a + c - b^2 / (first pivot), so
    the smaller diagonal entry must go first."""
    a, b, c = 5.0, 1.5, 2.0
    H = np.array([[a, b], [b, c]])
    pi, piv, info = O.min_pivot_order(H)
    assert list(pi) == [1, 0]
    assert piv.sum() == pytest.approx(a + c - b * b / c, rel=1e-15)
    assert piv.sum() < a + c - b * b / a


def test_min_pivot_reports_the_failing_step():
    """A pivot that is not positive stops the factorization: info = step + 1;
    a NaN diagonal is taken first."""
    pi, piv, info = O.min_pivot_order(np.diag([2.0, -1.0, 3.0]))
    assert info == 1 and list(pi) == [1, 0, 2]
    assert piv[0] == -1.0 and np.all(np.isnan(piv[1:]))
    pi, piv, info = O.min_pivot_order(np.ones((2, 2)))
    assert info == 2 and list(pi) == [0, 1] and piv[0] == 1.0
    pi, _, info = O.min_pivot_order(np.diag([1.0, np.nan, 2.0]))
    assert info == 1 and pi[0] == 1
    # the layer's factor fails at the same leading minor
    W = np.ones((2, 3))
    out = O.quant_layer(W, H=np.diag([2.0, -1.0, 3.0]), order="min_pivot", damp=0.0)
    assert out["info"] == 1


def test_min_pivot_layer_is_the_layer_in_that_order():
    rng = np.random.default_rng(33)
    W, X = _rand_problem(rng, 8, 24, 96, outl=2)
    a = O.quant_layer(W, X=X, grid_kind="asym", bits=3, group=8, order="min_pivot")
    pi, _, _ = O.min_pivot_order(a["Hd"])
    b = O.quant_layer(W, X=X, grid_kind="asym", bits=3, group=8, order="perm", perm=pi)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["pi"], pi)


def test_dead_feature_is_erased():
    """[WSIC 2]: a zero-variance input is erased: its code is 0 and the other
    columns are quantized as if it were absent (damp 0 keeps lambda equal)."""
    rng = np.random.default_rng(15)
    W, X = _rand_problem(rng, 6, 10, 50)
    X[4] = 0.0
    a = O.quant_layer(W, X=X, grid_kind="sym", bits=3, group=0, damp=0.0)
    assert np.all(a["codes"][:, 4] == 0)
    keep = [i for i in range(10) if i != 4]
    W2 = W.copy()
    W2[:, 4] = 0.0
    # steps come from the zeroed W, so give the reduced problem the same rows
    b = O.quant_layer(W2[:, keep], X=X[keep], grid_kind="sym", bits=3,
                      group=0, damp=0.0)
    np.testing.assert_array_equal(a["codes"][:, keep], b["codes"])


# --------------------------------------------------------------- rate


def test_column_entropy():
    codes = np.array([[0, 1, 5], [1, 1, 5], [2, 1, 6], [3, 1, 6]])
    np.testing.assert_allclose(O.column_entropy_bits(codes), [2.0, 0.0, 1.0])


def test_huffman_cost_pins():
    """Huffman totals against closed forms: a dyadic distribution is coded at
    exactly its entropy; two symbols cost one bit each; one symbol costs
    nothing; a hand-built tree; and for any counts the mean length lies in
    [H, H + 1) (Shannon's bounds)."""
    assert O.huffman_cost([7]) == 0
    assert O.huffman_cost([3, 5]) == 8
    # p = 1/2, 1/4, 1/8, 1/8 -> lengths 1, 2, 3, 3
    assert O.huffman_cost([4, 2, 1, 1]) == 4 * 1 + 2 * 2 + 1 * 3 + 1 * 3
    # counts 5, 9, 12, 13, 16, 45 -> lengths 4, 4, 3, 3, 3, 1 (by hand)
    assert O.huffman_cost([5, 9, 12, 13, 16, 45]) == 5 * 4 + 9 * 4 + 12 * 3 + 13 * 3 + 16 * 3 + 45
    rng = np.random.default_rng(3)
    for _ in range(20):
        cnt = rng.integers(1, 1000, size=rng.integers(2, 40))
        m = cnt.sum()
        p = cnt / m
        H = -np.sum(p * np.log2(p))
        L = O.huffman_cost(cnt) / m
        assert H - 1e-12 <= L < H + 1
    codes = np.array([[0, 1, 5], [1, 1, 5], [2, 1, 6], [3, 1, 6]])
    np.testing.assert_array_equal(O.column_huffman_bits(codes), [8, 0, 4])


def test_damping_hand_example():
    """[OAEM 3] damped form H + lambda I; reading lambda = damp * mean diag H.
    By hand: mean diag of [[4,2,2],[2,5,3],[2,3,6]] is 5, damp 0.2 -> 1."""
    H = np.array([[4.0, 2, 2], [2, 5, 3], [2, 3, 6]])
    Hd, W0, lam, dead = O.fix_dead_and_damp(H, np.ones((1, 3)), 0.2)
    assert lam == pytest.approx(1.0, rel=1e-15)
    np.testing.assert_allclose(Hd, [[5, 2, 2], [2, 6, 3], [2, 3, 7]])
    assert not dead.any()


def test_dead_feature_diagonal_and_lambda():
    """Dead input k: H_kk becomes 1 before lambda is taken.  By hand:
    diag (2, 0, 4) -> (2, 1, 4), mean 7/3, damp 0.3 -> lambda 0.7."""
    H = np.diag([2.0, 0.0, 4.0])
    Hd, W0, lam, dead = O.fix_dead_and_damp(H, np.ones((2, 3)), 0.3)
    assert lam == pytest.approx(0.7, rel=1e-14)
    np.testing.assert_allclose(np.diag(Hd), [2.7, 1.7, 4.7])
    np.testing.assert_array_equal(W0, [[1, 0, 1], [1, 0, 1]])
    np.testing.assert_array_equal(dead, [False, True, False])


@pytest.mark.parametrize("grid_kind,group", [("sym", 4), ("asym", 3),
                                             ("colspacing", 0)])
def test_perm_with_grouped_and_column_steps(grid_kind, group):
    """Steps belong to ORIGINAL columns (groups of consecutive original
    columns; spacing c / l_kk of the position a column is processed at).
    Checked with the textbook Gram-Schmidt Babai run on the permuted tall
    basis with independently permuted steps."""
    rng = np.random.default_rng(16)
    m, n, N = 4, 12, 48
    W, X = _rand_problem(rng, m, n, N, outl=1)
    p = rng.permutation(n)
    res = O.quant_layer(W, X=X, grid_kind=grid_kind, bits=3, group=group,
                        c=0.05, damp=0.02, order="perm", perm=p)
    A = np.vstack([np.sqrt(2.0) * X.T, np.sqrt(res["lam"]) * np.eye(n)])
    Ap = A[:, p]
    if grid_kind == "colspacing":
        # l_kk of the permuted problem = norm of the k-th Gram-Schmidt vector
        Lp, _ = O.cholesky_lower(Ap.T @ Ap)
        alpha_pos = 0.05 / np.diag(Lp)
        np.testing.assert_allclose(res["scales"][p], alpha_pos, rtol=1e-12)
        S_pos = np.broadcast_to(alpha_pos, (m, n))
    else:
        s_grp, _ = O.grid_steps(W, grid_kind, 3, group)
        S_pos = np.repeat(s_grp, group, axis=1)[:, p]
    for r in range(m):
        zg = O.babai_gram_schmidt(Ap, W[r, p], S_pos[r])
        np.testing.assert_array_equal(res["Z"][r, p], zg)


# ---------------------------------------------------------------- SSQR (GEOM 3)

def test_ssqr_step_scale_and_code_range():
    rng = np.random.default_rng(41)
    W = rng.standard_normal((6, 32)).astype(np.float32).astype(np.float64)
    for kind, bits in (("sym", 4), ("asym", 3)):
        s1, z1 = O.grid_steps(W, kind, bits, 16)
        s2, z2 = O.grid_steps(W, kind, bits, 16, step_scale=0.5)
        assert np.array_equal(s2, s1 * 0.5)          # a power of two scales exactly
        if kind == "asym":
            lo = np.minimum(W.reshape(6, 2, 16).min(axis=2), 0).astype(np.float32)
            assert np.array_equal(z2, np.rint(-lo / (s1 * 0.5).astype(np.float32)).astype(np.int64))
    assert O.code_range("sym", 4) == (-8, 7)
    assert O.code_range("asym", 2) == (0, 3)


def test_ssqr_overflow_split_reconstructs_the_dequantized_weights():
    rng = np.random.default_rng(42)
    m, n, G = 5, 24, 8
    scales = rng.uniform(0.01, 0.1, (m, n // G)).astype(np.float32).astype(np.float64)
    zeros = rng.integers(0, 16, (m, n // G))
    codes = rng.integers(-20, 36, (m, n))
    rows, cols, vals = O.overflow_entries(codes, scales, zeros, "asym", 4)
    lo, hi = O.code_range("asym", 4)
    inside = (codes >= lo) & (codes <= hi)
    assert len(rows) == int(np.sum(~inside))
    order = rows * n + cols
    assert np.all(np.diff(order) > 0)                 # row-major, no repeats
    assert not np.any(inside[rows, cols])
    S = np.repeat(scales, G, axis=1).astype(np.float32)
    Z = (codes - np.repeat(zeros, G, axis=1)).astype(np.float32)
    full = S * Z
    recon = np.where(inside, full, np.float32(0))
    recon[rows, cols] = vals
    assert np.array_equal(recon, full)


def _rtn_count(W0, kind, bits, group, kappa):
    """Outliers of plain round-to-nearest at steps s * kappa (no sweep)."""
    s, z = O.grid_steps(W0, kind, bits, group, step_scale=kappa)
    S = O.expand_group_steps(s, W0.shape[1])
    codes = np.rint(W0 / S).astype(np.int64)
    if z is not None:
        codes = codes + O.expand_group_steps(z.astype(np.float64), W0.shape[1]).astype(np.int64)
    lo, hi = O.code_range(kind, bits)
    return int(np.sum((codes < lo) | (codes > hi)))


def test_ssqr_search_on_a_diagonal_hessian_equals_brute_force():
    """A diagonal H makes the sweep plain rounding, whose outlier count never
    increases with kappa: the bisection must land on the smallest point of
    its dyadic grid that meets the target."""
    rng = np.random.default_rng(43)
    m, n = 12, 64
    W = (0.02 * rng.standard_t(3, (m, n))).astype(np.float32).astype(np.float64)
    H = np.diag(rng.uniform(0.5, 2.0, n))
    iters, lo = 6, -4.0
    for kind, bits, group, density in (("sym", 3, 32, 0.05), ("asym", 2, 16, 0.10)):
        def count_at(k):
            r = O.quant_layer(W, H=H, grid_kind=kind, bits=bits, group=group, damp=0.0,
                              step_scale=k)
            rows, _, _ = O.overflow_entries(r["codes"], r["scales"], r["zeros"], kind, bits)
            assert len(rows) == _rtn_count(W, kind, bits, group, k)
            return len(rows)
        kappa, evals = O.ssqr_search(count_at, m, n, density, iters=iters, log2_lo=lo)
        target = int(np.floor(density * m * n))
        grid = [lo + (0.0 - lo) * k / 2 ** iters for k in range(2 ** iters + 1)]
        best = min(x for x in grid
                   if _rtn_count(W, kind, bits, group, float(np.float32(2.0 ** x))) <= target)
        assert kappa == float(np.float32(2.0 ** best))
        assert len(evals) == iters + 2


def test_ssqr_search_edges():
    calls = []

    def always(c):
        return lambda k: (calls.append(k), c)[1]
    k, ev = O.ssqr_search(always(0), 4, 4, 0.0, iters=5, log2_lo=-3.0)
    assert k == 0.125 and len(ev) == 2                # the lower end already meets it
    k, ev = O.ssqr_search(always(100), 4, 4, 0.5, iters=5, log2_lo=-3.0)
    assert k == 1.0 and len(ev) == 1                  # unreachable: kappa stays 1


# ---------------------------------------------------------------- OA-EM


def _blobs(rng, K, per, g, spread=0.05):
    means = rng.standard_normal((K, g)) * 3.0
    pts = np.concatenate([mu + spread * rng.standard_normal((per, g)) for mu in means])
    return pts[rng.permutation(len(pts))], means


def _as_layer(pts, g, ng):
    """Group vectors (in index order r * ng + i) as an m x (ng g) matrix."""
    m = len(pts) // ng
    return pts[:m * ng].reshape(m, ng * g)


def _kmeans(X, C0, iters):
    from sklearn.cluster import KMeans
    km = KMeans(n_clusters=len(C0), init=C0, n_init=1, max_iter=iters, algorithm="lloyd",
                tol=0.0).fit(X)
    return km.cluster_centers_, km.labels_


def test_oaem_handworked_scalar_round():
    """tests/golden/handworked_oaem_scalar.txt: one E/M round and the final
    E-step with scalar groups, worked on paper."""
    gd = load("handworked_oaem_scalar.txt")
    books, codes, objs, R = O.oaem_init(gd["W"], gd["H"], 1,
                                        gd["seeds"].astype(np.int64)[None], iters=1)
    np.testing.assert_allclose(books[0][:, 0], gd["codebook"], rtol=1e-15)
    np.testing.assert_array_equal(codes[0], gd["codes"].astype(np.int64))
    assert objs[0] == pytest.approx(gd["objective"], rel=1e-15)


def test_oaem_identity_metric_is_lloyd_kmeans():
    """[OAEM 3] with every H_i = I the Mahalanobis E-step is the nearest
    centroid and the M-step the mean: Lloyd's k-means (scikit-learn's, from
    the same initial centroids, on blobs where no cluster empties)."""
    rng = np.random.default_rng(41)
    g, ng, K = 4, 6, 5
    pts, means = _blobs(rng, K, 24, g)
    W = _as_layer(pts, g, ng)
    m = W.shape[0]
    vec = W.reshape(m * ng, g)
    # one seed per blob: the group vector nearest to each blob centre
    seeds = np.array([[int(np.argmin(np.linalg.norm(vec - mu, axis=1))) for mu in means]])
    books, codes, objs, R = O.oaem_init(W, np.eye(ng * g), g, seeds, iters=6)
    C_ref, lab_ref = _kmeans(vec, vec[seeds[0]], 6)
    np.testing.assert_allclose(books[0], C_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(codes[0].reshape(-1), lab_ref)


def test_oaem_common_metric_is_kmeans_in_whitened_coordinates():
    """With one metric H_0 = L L^T for every group, distances are Euclidean
    in y = L^T w, so OA-EM is k-means on the whitened vectors."""
    rng = np.random.default_rng(42)
    g, ng, K = 3, 5, 4
    pts, means = _blobs(rng, K, 20, g, spread=0.3)
    W = _as_layer(pts, g, ng)
    m = W.shape[0]
    B = rng.standard_normal((g, g))
    H0 = B @ B.T + 0.5 * np.eye(g)
    Hd = np.kron(np.eye(ng), H0)
    vec = W.reshape(m * ng, g)
    seeds = np.array([[int(np.argmin(np.linalg.norm(vec - mu, axis=1))) for mu in means]])
    books, codes, _, _ = O.oaem_init(W, Hd, g, seeds, iters=5)
    L = np.linalg.cholesky(H0)
    Y = vec @ L
    Cy, lab = _kmeans(Y, Y[seeds[0]], 5)
    np.testing.assert_array_equal(codes[0].reshape(-1), lab)
    np.testing.assert_allclose(books[0] @ L, Cy, rtol=1e-9, atol=1e-12)


def test_oaem_mstep_minimises_the_weighted_error():
    """The M-step centroid of each cluster is the minimiser of
    sum (w - c)^T H_i (w - c) over its groups (scipy's BFGS from zero)."""
    from scipy.optimize import minimize
    rng = np.random.default_rng(43)
    g, ng, m, K = 4, 7, 9, 3
    X = rng.standard_normal((ng * g, 200)) * rng.lognormal(0, 0.7, (ng * g, 1))
    Hb = O.oaem_blocks(O.hessian(X), g)
    R = rng.standard_normal((m, ng * g))
    a = rng.integers(0, K, (m, ng))
    a[0, 0] = 0
    C0 = rng.standard_normal((K + 1, g))          # centroid K gets no group
    C = O.oaem_mstep(R, Hb, a, C0)
    np.testing.assert_array_equal(C[K], C0[K])
    for k in range(K):
        grp = [(r, i) for r in range(m) for i in range(ng) if a[r, i] == k]

        def f(c):
            return sum((R[r, i * g:(i + 1) * g] - c) @ Hb[i] @ (R[r, i * g:(i + 1) * g] - c)
                       for r, i in grp)
        opt = minimize(f, np.zeros(g), method="BFGS", options={"gtol": 1e-10})
        np.testing.assert_allclose(C[k], opt.x, rtol=1e-5, atol=1e-6)
        assert f(C[k]) <= opt.fun * (1 + 1e-12)


def test_oaem_objective_falls_with_rounds_and_stages_reconstruct():
    """E and M steps each minimise the same objective, so more rounds never
    raise it; the residual is W minus every stage's chosen centroids."""
    rng = np.random.default_rng(44)
    g, ng, m, K = 4, 8, 12, 6
    X = rng.standard_normal((ng * g, 300)) * rng.lognormal(0, 0.5, (ng * g, 1))
    Hd, _, _, _ = O.fix_dead_and_damp(O.hessian(X), np.zeros((1, ng * g)), 0.01)
    W = rng.standard_normal((m, ng * g)) * 0.02
    seeds = np.stack([rng.choice(m * ng, K, replace=False) for _ in range(2)])
    prev = np.inf
    for it in range(5):
        _, _, objs, _ = O.oaem_init(W, Hd, g, seeds[:1], iters=it)
        assert objs[0] <= prev * (1 + 1e-12)
        prev = objs[0]
    books, codes, objs, R = O.oaem_init(W, Hd, g, seeds, iters=3)
    rec = np.zeros_like(W)
    for t in range(2):
        for i in range(ng):
            rec[:, i * g:(i + 1) * g] += books[t][codes[t][:, i]]
    np.testing.assert_allclose(W - rec, R, atol=1e-14)
    Hb = O.oaem_blocks(Hd, g)
    assert objs[1] == pytest.approx(O.oaem_objective(R, Hb), rel=1e-12)
    assert objs[1] < objs[0]

"""Pins for the fp64 oracle: each test ties an oracle function to something
other than itself (a closed form, a library routine, an invariance, brute
force), chosen so that a plausible slip - a dropped term, a wrong sign, a
transposed operand, a wrong index - fails at least one of them."""
import numpy as np
import pytest
import scipy.linalg

from oracle import muon_oracle as O

RNG = np.random.default_rng(12345)


def _gauss(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _phi_scalar(sig, sched):
    """The scalar odd polynomial each singular value follows: s <- a s + b s^3 + c s^5."""
    s = np.array(sig, dtype=np.float64)
    for a, b, c in sched:
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def _ns_by_svd(X0, sched):
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    return (U * _phi_scalar(S, sched)) @ Vt


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


SHAPES = [(4, 7), (7, 4), (16, 16), (32, 8), (64, 256), (1, 5), (5, 1), (3, 3)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("T", [0, 1, 2, 5])
def test_direct_ns_equals_svd_closed_form(shape, T):
    M = _gauss(shape, hash((shape, T)) % 2**32)
    X0, _ = O.frobenius_normalize(M)
    sched = O.coeff_schedule(O.QUINTIC, T)
    got = O.ns_direct(X0, T, O.QUINTIC)
    want = _ns_by_svd(X0, sched)
    assert got.shape == shape
    assert _rel(got, want) < 1e-12


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (12, 12)])
def test_per_step_schedule_equals_svd_closed_form(shape):
    sched = np.array([[3.4445, -4.7750, 2.0315], [1.5, -0.5, 0.0], [2.0, -1.5, 0.5],
                      [3.4445, -4.7750, 2.0315]])
    M = _gauss(shape, 7)
    X0, _ = O.frobenius_normalize(M)
    assert _rel(O.ns_direct(X0, 4, sched), _ns_by_svd(X0, sched)) < 1e-12
    assert _rel(O.ns_gram(X0, 4, sched), _ns_by_svd(X0, sched)) < 1e-11


@pytest.mark.parametrize("shape", [(8, 12), (12, 8), (10, 10)])
def test_cubic_iteration_converges_to_scipy_polar_factor(shape):
    M = _gauss(shape, 99)
    X0, _ = O.frobenius_normalize(M)
    X = O.ns_direct(X0, 60, O.CUBIC)
    if shape[0] <= shape[1]:
        Upol, _ = scipy.linalg.polar(M, side="left")   # M = P U, U has orthonormal rows
    else:
        Upol, _ = scipy.linalg.polar(M, side="right")  # M = U P, U has orthonormal cols
    assert _rel(X, Upol) < 1e-12
    Xg = O.ns_gram(X0, 60, O.CUBIC)
    assert _rel(Xg, Upol) < 1e-10


@pytest.mark.parametrize("shape", [(4, 7), (7, 4), (16, 16), (8, 64), (64, 8), (2, 50)])
@pytest.mark.parametrize("T", [0, 1, 2, 3, 5, 6])
def test_gram_space_equals_direct(shape, T):
    M = _gauss(shape, 1000 + T)
    X0, _ = O.frobenius_normalize(M)
    d = O.ns_direct(X0, T)
    g = O.ns_gram(X0, T)
    assert _rel(g, d) < 1e-11
    assert _rel(g, _ns_by_svd(X0, O.coeff_schedule(O.QUINTIC, T))) < 1e-11


def test_orientation_right_multiplied_form():
    """p(X X^T) X == X p(X^T X): iterate a tall matrix on its large side by hand."""
    M = _gauss((24, 10), 5)
    X0, _ = O.frobenius_normalize(M)
    X = X0.copy()
    for a, b, c in O.coeff_schedule(O.QUINTIC, 5):
        S = X.T @ X
        X = a * X + X @ (b * S + c * (S @ S))
    assert _rel(O.ns_direct(X0, 5), X) < 1e-12
    assert _rel(O.ns_direct(X0.T, 5), X.T) < 1e-12


def test_orthogonal_equivariance_oddness_scale():
    M = _gauss((9, 14), 11)
    P, _ = np.linalg.qr(_gauss((9, 9), 12))
    R, _ = np.linalg.qr(_gauss((14, 14), 13))
    X0, _ = O.frobenius_normalize(M)
    base = O.ns_direct(X0, 5)
    assert _rel(O.ns_direct(P @ X0 @ R, 5), P @ base @ R) < 1e-12
    assert _rel(O.ns_direct(-X0, 5), -base) < 1e-13
    # scale invariance of normalize + NS: exact with eps = 0, within O(eps/nu) otherwise
    X0e, _ = O.frobenius_normalize(M, eps=0.0)
    Xa, _ = O.frobenius_normalize(3.7 * M, eps=0.0)
    assert _rel(O.ns_direct(Xa, 5), O.ns_direct(X0e, 5)) < 1e-13
    Xb, nu = O.frobenius_normalize(3.7 * M)
    assert _rel(O.ns_direct(Xb, 5), base) < 50 * 1e-7 / nu


def test_scaled_identity_reduces_to_scalar_map():
    """M = sigma [I 0]: every singular value equals sigma/(sigma sqrt(m) + eps)."""
    m, n, sig, eps = 4, 9, 0.3, 1e-7
    M = np.zeros((m, n))
    M[:, :m] = sig * np.eye(m)
    X0, nu = O.frobenius_normalize(M, eps)
    assert nu == pytest.approx(sig * np.sqrt(m), rel=1e-15)
    x = sig / (sig * np.sqrt(m) + eps)
    # five quintic steps by hand: x <- 3.4445 x - 4.7750 x^3 + 2.0315 x^5
    for _ in range(5):
        x = 3.4445 * x - 4.7750 * x ** 3 + 2.0315 * x ** 5
    want = np.zeros((m, n))
    want[:, :m] = x * np.eye(m)
    assert np.max(np.abs(O.ns_direct(X0, 5) - want)) < 1e-14
    assert np.max(np.abs(O.ns_gram(X0, 5) - want)) < 1e-14


def _matmul_loops(A, B):
    n, k = len(A), len(A[0])
    p = len(B[0])
    return [[sum(A[i][t] * B[t][j] for t in range(k)) for j in range(p)] for i in range(n)]


def test_brute_force_loops_tiny():
    """Pure-Python loops for a 2x3 matrix, three steps."""
    M = [[0.3, -0.1, 0.25], [0.05, 0.4, -0.2]]
    nu = sum(v * v for row in M for v in row) ** 0.5
    X = [[v / (nu + 1e-7) for v in row] for row in M]
    a, b, c = O.QUINTIC
    for _ in range(3):
        Xt = [list(r) for r in zip(*X)]
        A = _matmul_loops(X, Xt)
        AA = _matmul_loops(A, A)
        B = [[b * A[i][j] + c * AA[i][j] for j in range(2)] for i in range(2)]
        BX = _matmul_loops(B, X)
        X = [[a * X[i][j] + BX[i][j] for j in range(3)] for i in range(2)]
    X0, _ = O.frobenius_normalize(np.array(M))
    assert np.max(np.abs(O.ns_direct(X0, 3) - np.array(X))) < 1e-14


def test_momentum_closed_form():
    beta = 0.95
    gs = [_gauss((5, 6), 20 + k) for k in range(6)]
    buf = np.zeros((5, 6))
    for k, g in enumerate(gs):
        buf, d = O.nesterov_momentum(buf, g, beta)
        closed = sum(beta ** (k - j) * gs[j] for j in range(k + 1))
        assert np.max(np.abs(buf - closed)) < 1e-13
        assert np.max(np.abs(d - (gs[k] + beta * closed))) < 1e-13


def test_plain_momentum_closed_form():
    """Plain momentum from zero: buf_k = d_k = sum_j beta^(k-j) g_j (no Nesterov look-ahead)."""
    rng = np.random.default_rng(42)
    beta = 0.9
    gs = [rng.standard_normal((5, 7)) for _ in range(4)]
    buf = np.zeros((5, 7))
    for k, g in enumerate(gs):
        buf, d = O.plain_momentum(buf, g, beta)
        closed = sum(beta ** (k - j) * gs[j] for j in range(k + 1))
        assert np.allclose(buf, closed, rtol=1e-14, atol=1e-14)
        assert np.array_equal(d, buf)


def test_nesterov_ema_variant_gives_same_update():
    """Reading of 'momentum-based update': the EMA form differs only by (1-beta),
    which the Frobenius normalization removes (up to eps)."""
    beta = 0.95
    gs = [_gauss((7, 5), 40 + k) for k in range(4)]
    buf, ema = np.zeros((7, 5)), np.zeros((7, 5))
    for g in gs:
        buf, d = O.nesterov_momentum(buf, g, beta)
        ema = beta * ema + (1 - beta) * g
        d_ema = (1 - beta) * g + beta * ema
        assert np.max(np.abs(d_ema - (1 - beta) * d)) < 1e-14
    x1, _ = O.frobenius_normalize(d)
    x2, _ = O.frobenius_normalize(d_ema)
    assert _rel(x2, x1) < 1e-6


def test_rms_matching_scale():
    M = _gauss((256, 512), 3)
    Upol, _ = scipy.linalg.polar(M, side="left")
    s = O.rms_scale(256, 512)
    assert s == pytest.approx(0.2 * np.sqrt(512), rel=1e-15)
    assert np.sqrt(np.mean((s * Upol) ** 2)) == pytest.approx(0.2, abs=1e-12)
    X0, _ = O.frobenius_normalize(M)
    rms = np.sqrt(np.mean((s * O.ns_direct(X0, 5)) ** 2))
    assert 0.17 < rms < 0.205   # the quintic does not converge; singular values land in ~[0.7, 1.1]
    # tall matrix uses max(rows, cols) as well
    assert O.rms_scale(512, 256) == O.rms_scale(256, 512)


def test_zero_gradient_is_pure_decoupled_decay():
    W = _gauss((6, 10), 8) * 0.02
    r = O.muon_step_ref(W, np.zeros_like(W), np.zeros_like(W), lr=0.02, wd=0.01)
    assert np.array_equal(r["X"], np.zeros_like(W))
    assert _rel(r["U"], -0.02 * 0.01 * W) < 1e-15
    assert r["nu"] == 0.0


def test_lr_zero_leaves_weights_and_updates_momentum():
    W = _gauss((6, 10), 8) * 0.02
    g = _gauss((6, 10), 9) * 0.02
    r = O.muon_step_ref(W, g, np.zeros_like(W), lr=0.0)
    assert np.array_equal(r["W_new"], W)
    assert np.max(np.abs(r["buf_new"] - g)) == 0.0


def test_ns_steps_zero_is_normalized_nesterov():
    W = _gauss((5, 8), 1) * 0.02
    g = _gauss((5, 8), 2) * 0.02
    r = O.muon_step_ref(W, g, np.zeros_like(W), ns_steps=0, beta=0.9)
    d = g + 0.9 * g
    assert _rel(r["X"], d / (np.linalg.norm(d) + 1e-7)) < 1e-15
    s = 0.2 * np.sqrt(8)
    assert _rel(r["U"], -0.02 * (0.01 * W + s * r["X"])) < 1e-15


def test_full_step_gram_form_matches_direct():
    W = _gauss((16, 40), 30) * 0.02
    g = _gauss((16, 40), 31) * 0.02
    buf = _gauss((16, 40), 32) * 0.01
    a = O.muon_step_ref(W, g, buf, form="direct")
    b = O.muon_step_ref(W, g, buf, form="gram")
    assert _rel(b["U"], a["U"]) < 1e-12


def test_round_to_bf16_matches_torch_on_fp32_values_and_ties():
    import torch
    x32 = (np.random.default_rng(0).standard_normal(10000) * 0.02).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_bf16(x32.astype(np.float64)), want)
    # exact ties go to the even neighbour
    one = 1.0
    assert O.round_to_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    assert O.round_to_bf16(np.array([-(one + 2.0 ** -8 + 2.0 ** -30)]))[0] == -(one + 2.0 ** -7)


def test_multi_step_driver_carries_state():
    Ws = [_gauss((4, 6), 50) * 0.02]
    bufs = [np.zeros((4, 6))]
    g1, g2 = _gauss((4, 6), 51) * 0.02, _gauss((4, 6), 52) * 0.02
    last, Ws2, bufs2 = O.muon_steps_ref(Ws, [[g1], [g2]], bufs, param_dtype="f32")
    r1 = O.muon_step_ref(Ws[0], g1, bufs[0])
    r2 = O.muon_step_ref(r1["W_new_stored"], g2, O.round_to_f32(r1["buf_new"]))
    assert np.array_equal(last[0]["U"], r2["U"])
    assert np.array_equal(bufs2[0], O.round_to_f32(r2["buf_new"]))


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (20, 20), (1, 7)])
@pytest.mark.parametrize("T", [0, 1, 5])
def test_orthogonalize_equals_svd_of_the_normalized_input(shape, T):
    """orthogonalize_ref(M) = U phi^T(S / (||M||_F + eps)) V^T, from numpy's SVD of
    M itself (the normalization written out by hand here, not the oracle's)."""
    M = _gauss(shape, 31 + T) * 3.0
    U, S, Vt = np.linalg.svd(M, full_matrices=False)
    nu = np.sqrt(np.sum(S ** 2))          # ||M||_F from the singular values
    want = (U * _phi_scalar(S / (nu + 1e-7), O.coeff_schedule(O.QUINTIC, T))) @ Vt
    assert _rel(O.orthogonalize_ref(M, T), want) < 1e-12
    assert _rel(O.orthogonalize_ref(M, T, form="gram"), want) < 1e-11
    # a different eps and a cubic schedule
    want2 = (U * _phi_scalar(S / (nu + 0.5), O.coeff_schedule((1.5, -0.5, 0.0), T))) @ Vt
    assert _rel(O.orthogonalize_ref(M, T, (1.5, -0.5, 0.0), eps=0.5), want2) < 1e-12


def test_orthogonalize_of_zero_is_zero():
    assert np.all(O.orthogonalize_ref(np.zeros((4, 6)), 5) == 0.0)


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (16, 16)])
@pytest.mark.parametrize("form", ["direct", "gram"])
def test_whole_step_equals_closed_form_on_shared_singular_vectors(shape, form):
    """The whole step (momentum, normalization, orientation, NS, RMS scale,
    decoupled decay, apply) against a closed form: with the gradient and the
    momentum built on the same singular vectors, g = P diag(gam) Q^T and
    buf = P diag(mu) Q^T, the Nesterov direction is P diag(delta) Q^T with
    delta = (1 + beta) gam + beta^2 mu, its Frobenius norm is ||delta||_2, and
    NS sends each singular value through the scalar odd polynomial, so
    U = -lr (wd W + s P diag(phi(delta / (||delta||_2 + eps))) Q^T) with
    s = 0.2 sqrt(max(rows, cols)).  No matrix product of the oracle is reused."""
    rows, cols = shape
    k = min(rows, cols)
    rng = np.random.default_rng(2024 + rows * 100 + cols)
    P, _ = np.linalg.qr(rng.standard_normal((rows, k)))
    Q, _ = np.linalg.qr(rng.standard_normal((cols, k)))
    gam = rng.uniform(0.05, 1.0, k) * 1e-2
    mu = rng.uniform(-1.0, 1.0, k) * 1e-2
    g = (P * gam) @ Q.T
    buf = (P * mu) @ Q.T
    W = rng.standard_normal(shape) * 0.02
    lr, beta, wd, eps, T = 0.02, 0.95, 0.01, 1e-7, 5
    r = O.muon_step_ref(W, g, buf, lr=lr, beta=beta, wd=wd, ns_steps=T, eps=eps, form=form)
    delta = (1.0 + beta) * gam + beta * beta * mu
    sig = np.abs(delta) / (np.sqrt(np.sum(delta ** 2)) + eps)
    phi = _phi_scalar(sig, O.coeff_schedule(O.QUINTIC, T)) * np.sign(delta)
    X = (P * phi) @ Q.T
    s = 0.2 * np.sqrt(max(rows, cols))
    U = -lr * (wd * W + s * X)
    assert _rel(r["buf_new"], beta * buf + g) < 1e-14
    assert abs(r["nu"] - np.sqrt(np.sum(delta ** 2))) <= 1e-14 * r["nu"]
    assert _rel(r["X"], X) < 1e-11
    assert _rel(r["U"], U) < 1e-11
    assert _rel(r["W_new"], W + U) < 1e-14
    # plain momentum: the direction is the new buffer itself, P diag(gam + beta mu) Q^T
    rp = O.muon_step_ref(W, g, buf, lr=lr, beta=beta, wd=wd, ns_steps=T, eps=eps, form=form,
                         nesterov=False)
    dp = gam + beta * mu
    sp = np.abs(dp) / (np.sqrt(np.sum(dp ** 2)) + eps)
    Xp = (P * (_phi_scalar(sp, O.coeff_schedule(O.QUINTIC, T)) * np.sign(dp))) @ Q.T
    assert abs(rp["nu"] - np.sqrt(np.sum(dp ** 2))) <= 1e-14 * rp["nu"]
    assert _rel(rp["U"], -lr * (wd * W + s * Xp)) < 1e-11
    assert _rel(rp["buf_new"], beta * buf + g) < 1e-14

"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-worked examples
stored under tests/golden/ (each file names the passage it follows), closed
forms (isometry and Pythagoras with orthonormal A), special cases that reduce
to numpy's textbook row norm, brute force over tiny random layers, finite
differences, and torch CPU fp64 autograd of a dense DoRA layer with a detached
norm.  The last test plants mistakes in copies of the oracle's formulas and
checks that these pins catch each one.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dora_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def arr(x):
    return np.asarray(x, dtype=np.float64)


def rand_layer(rng, d_out, d_in, r, b_std=0.3):
    W0 = rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    A = rng.uniform(-1, 1, (r, d_in)) / np.sqrt(d_in)
    B = rng.standard_normal((d_out, r)) * b_std
    return W0, A, B


# ---------------------------------------------------------------- golden pins

def test_arrow_example():
    c = load("arrow_example.json")
    wn = oracle.dense_row_norm(c["W0"], c["A"], c["B"], c["s"])
    np.testing.assert_allclose(wn, c["wnorm"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.factored_row_norm(c["W0"], c["A"], c["B"], c["s"]), c["wnorm"],
                               rtol=0, atol=1e-15)
    g = oracle.magnitude_scale(c["m"], wn, c["eps"])
    np.testing.assert_allclose(g, c["g"], rtol=0, atol=1e-15)
    Wm = oracle.merged_weight(c["W0"], c["A"], c["B"], c["m"], c["s"], c["eps"])
    np.testing.assert_allclose(Wm, c["merged"], rtol=0, atol=1e-15)
    Ws = oracle.merge_with_scale(c["W0"], c["A"], c["B"], c["g"], c["s"])
    np.testing.assert_allclose(Ws, c["merged"], rtol=0, atol=1e-15)
    assert abs(np.linalg.norm(Wm[0]) - 2.0) < 1e-15  # length set by m


def test_pythagoras_rows():
    c = load("pythagoras_rows.json")
    for f in (oracle.dense_row_norm, oracle.factored_row_norm):
        np.testing.assert_array_equal(f(c["W0"], c["A"], c["B"], c["s"]), arr(c["wnorm"]))


def test_collinear_rows_cross_term_and_sign():
    c = load("collinear_rows.json")
    for case in c["cases"]:
        for f in (oracle.dense_row_norm, oracle.factored_row_norm):
            np.testing.assert_allclose(f(c["W0"], c["A"], c["B"], case["s"]), case["wnorm"],
                                       rtol=0, atol=1e-14)


def test_eps_clamp():
    c = load("eps_clamp.json")
    wn = oracle.dense_row_norm(c["W0"], c["A"], c["B"], c["s"])
    np.testing.assert_array_equal(wn, arr(c["wnorm"]))
    np.testing.assert_array_equal(oracle.magnitude_scale(c["m"], wn, c["eps"]), arr(c["g"]))


def test_compose_small_forward_backward():
    c = load("compose_small.json")
    y = oracle.compose_forward(c["base_out"], c["lora_out"], c["g"], c["s"])
    np.testing.assert_array_equal(y, arr(c["y"]))
    d = oracle.compose_forward(c["base_out"], c["lora_out"], c["g"], c["s"], delta_only=True)
    np.testing.assert_array_equal(d, arr(c["delta"]))
    db, dl, dm = oracle.compose_backward(c["dy"], c["base_out"], c["lora_out"], c["g"], c["wnorm"],
                                         c["s"], c["eps"])
    np.testing.assert_array_equal(db, arr(c["d_base"]))
    np.testing.assert_array_equal(dl, arr(c["d_lora"]))
    np.testing.assert_array_equal(dm, arr(c["d_m"]))
    db2, dl2, dm2 = oracle.compose_backward(c["dy"], c["base_out"], c["lora_out"], c["g"], c["wnorm"],
                                            c["s"], c["eps"], delta_only=True)
    np.testing.assert_array_equal(db2, arr(c["d_base_delta"]))
    np.testing.assert_array_equal(dl2, dl)
    np.testing.assert_array_equal(dm2, dm)


def test_compose_inner_small():
    # the dual-output forward and the (dy, inner) backward on a hand-worked layer
    c = load("compose_inner_small.json")
    y, inner = oracle.compose_forward_inner(c["base_out"], c["lora_out"], c["g"], c["s"])
    np.testing.assert_array_equal(inner, arr(c["inner"]))
    np.testing.assert_array_equal(y, arr(c["y"]))
    db, dl, dm = oracle.compose_backward_inner(c["dy"], c["inner"], c["g"], c["wnorm"], c["s"], c["eps"])
    np.testing.assert_array_equal(db, arr(c["d_base"]))
    np.testing.assert_array_equal(dl, arr(c["d_lora"]))
    np.testing.assert_array_equal(dm, arr(c["d_m"]))
    db2, _, _ = oracle.compose_backward_inner(c["dy"], c["inner"], c["g"], c["wnorm"], c["s"], c["eps"],
                                              delta_only=True)
    np.testing.assert_array_equal(db2, arr(c["d_base_delta"]))


def test_inner_backward_finite_differences():
    # L = sum(dy * (m / max(wnorm, eps)) * inner), wnorm fixed: d_m by central
    # differences in m; d_base and d_lora through inner = base + s lora
    rng = np.random.default_rng(21)
    T, d_out, s, eps = 6, 5, 1.3, 1e-12
    base, lora, dy = (rng.standard_normal((T, d_out)) for _ in range(3))
    wnorm, m = rng.uniform(0.5, 2.0, d_out), rng.uniform(0.5, 2.0, d_out)

    def loss(b, l, mm):
        return float(np.sum(dy * (mm / np.maximum(wnorm, eps)) * (b + s * l)))

    db, dl, dm = oracle.compose_backward_inner(dy, base + s * lora, m / wnorm, wnorm, s, eps)
    h = 1e-6
    for j in range(d_out):
        e = np.zeros(d_out); e[j] = h
        assert abs((loss(base, lora, m + e) - loss(base, lora, m - e)) / (2 * h) - dm[j]) < 1e-7
    for (i, j) in [(0, 0), (5, 4), (2, 3)]:
        e = np.zeros((T, d_out)); e[i, j] = h
        assert abs((loss(base + e, lora, m) - loss(base - e, lora, m)) / (2 * h) - db[i, j]) < 1e-7
        assert abs((loss(base, lora + e, m) - loss(base, lora - e, m)) / (2 * h) - dl[i, j]) < 1e-7


# ------------------------------------------------- special cases / closed forms

@pytest.mark.parametrize("shape", [(7, 5, 3), (1, 9, 2), (12, 4, 6), (33, 17, 1)])
def test_b_zero_and_s_zero_reduce_to_row_norm(shape):
    rng = np.random.default_rng(1)
    W0, A, B = rand_layer(rng, *shape)
    ref = np.linalg.norm(W0, axis=1)
    for f in (oracle.dense_row_norm, oracle.factored_row_norm):
        np.testing.assert_allclose(f(W0, A, np.zeros_like(B), 1.7), ref, rtol=1e-14)
        np.testing.assert_allclose(f(W0, A, B, 0.0), ref, rtol=1e-14)


def _orthonormal_rows(rng, r, d_in):
    Q, _ = np.linalg.qr(rng.standard_normal((d_in, r)))
    return Q.T  # [r, d_in], orthonormal rows


@pytest.mark.parametrize("s", [1.0, -2.5, 0.3])
def test_orthonormal_a_isometry_and_pythagoras(s):
    rng = np.random.default_rng(2)
    d_out, d_in, r = 11, 20, 6
    A = _orthonormal_rows(rng, r, d_in)
    B = rng.standard_normal((d_out, r))
    # W0 = 0: ||s B_i A|| = |s| ||B_i|| because A^T is an isometry.
    for f in (oracle.dense_row_norm, oracle.factored_row_norm):
        np.testing.assert_allclose(f(np.zeros((d_out, d_in)), A, B, s),
                                   abs(s) * np.linalg.norm(B, axis=1), rtol=1e-13)
    # W0 orthogonal to A's row space: n^2 = ||W0_i||^2 + s^2 ||B_i||^2.
    W0 = rng.standard_normal((d_out, d_in))
    W0 = W0 - (W0 @ A.T) @ A
    ref = np.sqrt(np.linalg.norm(W0, axis=1) ** 2 + s * s * np.linalg.norm(B, axis=1) ** 2)
    for f in (oracle.dense_row_norm, oracle.factored_row_norm):
        np.testing.assert_allclose(f(W0, A, B, s), ref, rtol=1e-13)


def test_rank_one_zero_base_closed_form():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((1, 13))
    B = rng.standard_normal((9, 1))
    ref = np.abs(2.0 * B[:, 0]) * np.linalg.norm(a)
    for f in (oracle.dense_row_norm, oracle.factored_row_norm):
        np.testing.assert_allclose(f(np.zeros((9, 13)), a, B, 2.0), ref, rtol=1e-13)


@pytest.mark.parametrize("shape", [(64, 48, 8), (5, 3, 7), (1, 16, 4), (17, 1, 3), (40, 30, 1)])
def test_factored_equals_dense_brute_force(shape):
    rng = np.random.default_rng(4)
    W0, A, B = rand_layer(rng, *shape, b_std=1.0)
    for s in (2.0, -0.7):
        d = oracle.dense_row_norm(W0, A, B, s)
        f = oracle.factored_row_norm(W0, A, B, s)
        # the factored sum cancels when a row norm is small, so its error is
        # relative to the size of the three terms, not to n^2 itself
        scale = np.sum(W0 * W0, 1) + s * s * np.sum((B @ A) ** 2, 1) + 2 * abs(s) * np.abs(
            np.einsum("ij,ij->i", B, W0 @ A.T))
        np.testing.assert_allclose(f * f, d * d, rtol=0, atol=1e-13 * scale.max())
        np.testing.assert_allclose(f, d, rtol=1e-9)


def test_row_subset_matches_full():
    rng = np.random.default_rng(5)
    W0, A, B = rand_layer(rng, 50, 20, 4)
    rows = [0, 7, 49, 13]
    np.testing.assert_array_equal(oracle.dense_row_norm(W0, A, B, 1.3, rows=rows),
                                  oracle.dense_row_norm(W0, A, B, 1.3)[rows])


def test_dense_norm_by_loop_brute_force():
    # pure-Python loops on a tiny layer: V'_ik = W0_ik + s * sum_j B_ij A_jk
    rng = np.random.default_rng(6)
    W0, A, B = rand_layer(rng, 4, 3, 2, b_std=1.0)
    s = 1.5
    ref = []
    for i in range(4):
        acc = 0.0
        for k in range(3):
            v = W0[i, k] + s * sum(B[i, j] * A[j, k] for j in range(2))
            acc += v * v
        ref.append(acc ** 0.5)
    np.testing.assert_allclose(oracle.dense_row_norm(W0, A, B, s), ref, rtol=1e-14)


# ----------------------------------------------------------- compose pins

def test_init_invariant_exact():
    # m0 = ||W0||_row and B = 0 => g = 1 and the layer reproduces the base output
    # exactly (LoRA & DoRA section 2: W'_init = W0; DoRA (aiwiki): training
    # starts exactly at W0).
    rng = np.random.default_rng(7)
    W0, A, _ = rand_layer(rng, 16, 12, 4)
    B = np.zeros((16, 4))
    m = np.linalg.norm(W0, axis=1)
    wn = oracle.dense_row_norm(W0, A, B, 2.0)
    g = oracle.magnitude_scale(m, wn, 1e-12)
    np.testing.assert_array_equal(g, np.ones(16))
    x = rng.standard_normal((5, 12))
    base, lora = x @ W0.T, (x @ A.T) @ B.T
    np.testing.assert_array_equal(oracle.compose_forward(base, lora, g, 2.0), base)
    np.testing.assert_array_equal(oracle.compose_forward(base, lora, g, 2.0, delta_only=True),
                                  np.zeros_like(base))


def test_compose_matches_weight_space_dora_layer():
    rng = np.random.default_rng(8)
    d_out, d_in, r, T, s, eps = 24, 18, 5, 9, 2.0, 1e-12
    W0, A, B = rand_layer(rng, d_out, d_in, r, b_std=0.5)
    m = np.linalg.norm(W0, axis=1) * (1 + 0.1 * rng.standard_normal(d_out))
    x = rng.standard_normal((T, d_in))
    g = oracle.magnitude_scale(m, oracle.dense_row_norm(W0, A, B, s), eps)
    y = oracle.compose_forward(x @ W0.T, (x @ A.T) @ B.T, g, s)
    np.testing.assert_allclose(y, oracle.dora_linear_forward(x, W0, A, B, m, s, eps), rtol=1e-12,
                               atol=1e-13)
    # merged weight serves the same layer
    Wm = oracle.merged_weight(W0, A, B, m, s, eps)
    np.testing.assert_allclose(x @ Wm.T, y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(Wm, axis=1), np.abs(m), rtol=1e-13)


def test_unit_g_is_plain_lora_and_zero_s_is_rescale():
    rng = np.random.default_rng(9)
    W0, A, B = rand_layer(rng, 10, 8, 3, b_std=1.0)
    x = rng.standard_normal((6, 8))
    base, lora = x @ W0.T, (x @ A.T) @ B.T
    # g = 1: y = W0 x + s B (A x) = x (W0 + sBA)^T  (LoRA & DoRA section 1)
    np.testing.assert_allclose(oracle.compose_forward(base, lora, np.ones(10), 1.5),
                               x @ (W0 + 1.5 * B @ A).T, rtol=1e-12, atol=1e-13)
    g = rng.uniform(0.5, 1.5, 10)
    np.testing.assert_allclose(oracle.compose_forward(base, lora, g, 0.0), g * base, rtol=1e-15)


def test_backward_finite_differences():
    # L = sum(dy * compose(base, lora, m / max(wnorm, eps))) with wnorm held fixed.
    rng = np.random.default_rng(10)
    T, d_out, s, eps = 5, 7, 1.7, 1e-12
    base, lora, dy = (rng.standard_normal((T, d_out)) for _ in range(3))
    wnorm = rng.uniform(0.5, 2.0, d_out)
    m = rng.uniform(0.5, 2.0, d_out)

    def loss(b, l, mm, delta):
        g = mm / np.maximum(wnorm, eps)
        return float(np.sum(dy * oracle.compose_forward(b, l, g, s, delta_only=delta)))

    for delta in (False, True):
        g = m / wnorm
        db, dl, dm = oracle.compose_backward(dy, base, lora, g, wnorm, s, eps, delta_only=delta)
        h = 1e-6
        for (t, i, j) in [(0, 0, 0), (3, 2, 5), (4, 4, 6)]:
            e = np.zeros((T, d_out)); e[i, j] = h
            fd_b = (loss(base + e, lora, m, delta) - loss(base - e, lora, m, delta)) / (2 * h)
            fd_l = (loss(base, lora + e, m, delta) - loss(base, lora - e, m, delta)) / (2 * h)
            assert abs(fd_b - db[i, j]) < 1e-7
            assert abs(fd_l - dl[i, j]) < 1e-7
        for j in range(d_out):
            e = np.zeros(d_out); e[j] = h
            fd_m = (loss(base, lora, m + e, delta) - loss(base, lora, m - e, delta)) / (2 * h)
            assert abs(fd_m - dm[j]) < 1e-7


def test_backward_matches_torch_autograd_of_dense_layer():
    # A dense DoRA layer (weight space, norm detached) differentiated by torch
    # CPU fp64 autograd: magnitude.grad equals the oracle's d_m and B.grad equals
    # d_lora^T (x A^T), the chain rule through lora_out = (x A^T) B^T.
    rng = np.random.default_rng(11)
    d_out, d_in, r, T, s, eps = 12, 10, 3, 8, 2.0, 1e-12
    W0, A, B = rand_layer(rng, d_out, d_in, r, b_std=0.5)
    m = np.linalg.norm(W0, axis=1) * (1 + 0.05 * rng.standard_normal(d_out))
    x = rng.standard_normal((T, d_in))
    dy = rng.standard_normal((T, d_out))
    tW0 = torch.tensor(W0)
    tA = torch.tensor(A)
    tB = torch.tensor(B, requires_grad=True)
    tm = torch.tensor(m, requires_grad=True)
    tx = torch.tensor(x)
    weight = tW0 + (tB @ tA) * s
    direction = weight / weight.norm(dim=1, keepdim=True).detach()
    y = torch.nn.functional.linear(tx, tm[:, None] * direction)
    y.backward(torch.tensor(dy))

    wn = oracle.dense_row_norm(W0, A, B, s)
    g = oracle.magnitude_scale(m, wn, eps)
    base, lora = x @ W0.T, (x @ A.T) @ B.T
    np.testing.assert_allclose(oracle.compose_forward(base, lora, g, s), y.detach().numpy(),
                               rtol=1e-12, atol=1e-13)
    _, dl, dm = oracle.compose_backward(dy, base, lora, g, wn, s, eps)
    np.testing.assert_allclose(dm, tm.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dl.T @ (x @ A.T), tB.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_as_f64_is_exact_for_bf16():
    t = torch.randn(100).to(torch.bfloat16)
    a = oracle.as_f64(t)
    assert a.dtype == np.float64
    np.testing.assert_array_equal(a, t.float().numpy().astype(np.float64))


# ------------------------------------------- the pins catch planted mistakes

def _mutants():
    def drop_cross(W0, A, B, s):
        W0, A, B = arr(W0), arr(A), arr(B)
        n2 = np.sum(W0 * W0, 1) + s * s * np.einsum("ij,ij->i", B @ (A @ A.T), B)
        return np.sqrt(np.maximum(n2, 0))

    def flip_cross(W0, A, B, s):
        W0, A, B = arr(W0), arr(A), arr(B)
        n2 = np.sum(W0 * W0, 1) - 2 * s * np.einsum("ij,ij->i", B, W0 @ A.T) + \
            s * s * np.einsum("ij,ij->i", B @ (A @ A.T), B)
        return np.sqrt(np.maximum(n2, 0))

    def s_not_squared(W0, A, B, s):
        W0, A, B = arr(W0), arr(A), arr(B)
        n2 = np.sum(W0 * W0, 1) + 2 * s * np.einsum("ij,ij->i", B, W0 @ A.T) + \
            s * np.einsum("ij,ij->i", B @ (A @ A.T), B)
        return np.sqrt(np.maximum(n2, 0))

    def gram_transposed(W0, A, B, s):
        W0, A, B = arr(W0), arr(A), arr(B)
        r = A.shape[0]
        G = (A.T @ A)[:r, :r]  # wrong contraction axis (needs d_in >= r)
        n2 = np.sum(W0 * W0, 1) + 2 * s * np.einsum("ij,ij->i", B, W0 @ A.T) + \
            s * s * np.einsum("ij,ij->i", B @ G, B)
        return np.sqrt(np.maximum(n2, 0))

    def column_norm(W0, A, B, s):
        V = arr(W0) + s * arr(B) @ arr(A)
        n = np.linalg.norm(V, axis=0)
        return np.resize(n, V.shape[0])

    return [drop_cross, flip_cross, s_not_squared, gram_transposed, column_norm]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_norm_mistakes(mutant):
    caught = False
    c = load("collinear_rows.json")
    for case in c["cases"]:
        if not np.allclose(mutant(c["W0"], c["A"], c["B"], case["s"]), case["wnorm"], atol=1e-12):
            caught = True
    rng = np.random.default_rng(12)
    for shape in [(7, 5, 3), (6, 6, 6), (9, 4, 2)]:
        W0, A, B = rand_layer(rng, *shape, b_std=1.0)
        ref = np.linalg.norm(arr(W0) + 1.3 * arr(B) @ arr(A), axis=1)
        if not np.allclose(mutant(W0, A, B, 1.3), ref, rtol=1e-10):
            caught = True
    assert caught


def test_merge_with_scale():
    rng = np.random.default_rng(12)
    d_out, d_in, r, s, eps = 20, 14, 4, 1.75, 1e-12
    W0, A, B = rand_layer(rng, d_out, d_in, r, b_std=0.6)
    m = rng.uniform(0.2, 2.0, d_out)
    # with the scale the norm produces, the merge is the pinned merged weight
    g = oracle.magnitude_scale(m, oracle.dense_row_norm(W0, A, B, s), eps)
    Ws = oracle.merge_with_scale(W0, A, B, g, s)
    np.testing.assert_allclose(Ws, oracle.merged_weight(W0, A, B, m, s, eps), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(Ws, axis=1), m, rtol=1e-13)
    # g = 1 and s = 0 reduce to the plain sum and to a row rescale of W0
    np.testing.assert_array_equal(oracle.merge_with_scale(W0, A, B, np.ones(d_out), 0.0), W0)
    np.testing.assert_allclose(oracle.merge_with_scale(W0, A, B, g, 0.0), g[:, None] * W0, rtol=1e-15)
    # brute force, element by element, on one row subset
    rows = [3, 0, 17]
    sub = oracle.merge_with_scale(W0, A, B, g, s, rows=rows)
    for a_, i in enumerate(rows):
        for j in range(d_in):
            v = W0[i, j] + s * sum(B[i, k] * A[k, j] for k in range(r))
            assert abs(sub[a_, j] - g[i] * v) <= 1e-14 * max(1.0, abs(g[i] * v))

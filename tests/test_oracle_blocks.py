"""Pins for the oracle's building blocks (CPU only).

Each block is checked against something other than itself: closed forms,
invariants, brute force, central finite differences in double, or an
independent library routine (numpy / torch CPU) computing the same textbook
operation.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

rng = np.random.default_rng(0)


def fd_check(f, x, analytic, h=1e-6, tol=1e-7):
    """Central differences of scalar f at x against an analytic gradient."""
    num = np.zeros_like(x)
    flat = x.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        fp = f()
        flat[i] = old - h
        fm = f()
        flat[i] = old
        num.reshape(-1)[i] = (fp - fm) / (2 * h)
    err = np.max(np.abs(num - analytic)) / max(1e-12, np.max(np.abs(analytic)))
    assert err < tol, err


# ---- linear -------------------------------------------------------------------

def test_linear_brute_force(oracle):
    x = rng.standard_normal((7, 13))
    W = rng.standard_normal((5, 13))
    b = rng.standard_normal(5)
    y = oracle.linear(x, W, b)
    ref = np.array([[b[n] + sum(x[m, k] * W[n, k] for k in range(13)) for n in range(5)] for m in range(7)])
    assert np.max(np.abs(y - ref)) < 1e-12
    assert np.max(np.abs(oracle.linear(x, W) - x @ W.T)) < 1e-12


def test_linear_bwd_finite_differences(oracle):
    x = rng.standard_normal((4, 6))
    W = rng.standard_normal((3, 6))
    b = rng.standard_normal(3)
    c = rng.standard_normal((4, 3))  # loss = sum(c * y)
    dx, dW, db = oracle.linear_bwd(c.copy(), x, W)
    loss = lambda: float(np.sum(c * oracle.linear(x, W, b)))
    fd_check(loss, x, dx)
    fd_check(loss, W, dW)
    fd_check(loss, b, db)


# ---- layernorm ----------------------------------------------------------------

def test_layernorm_unit_gain_gives_zero_mean_unit_variance(oracle):
    x = rng.standard_normal((9, 64)) * 3 + 1.5
    y, mean, rstd = oracle.layernorm(x, np.ones(64), np.zeros(64))
    assert np.max(np.abs(y.mean(axis=1))) < 1e-12
    # biased variance of the normalised row is var/(var+eps)
    var = x.var(axis=1)
    assert np.max(np.abs(y.var(axis=1) - var / (var + 1e-5))) < 1e-12
    assert np.max(np.abs(mean - x.mean(axis=1))) < 1e-12
    assert np.max(np.abs(rstd - 1 / np.sqrt(var + 1e-5))) < 1e-12


def test_layernorm_matches_torch(oracle):
    x = rng.standard_normal((5, 32))
    g = rng.standard_normal(32)
    b = rng.standard_normal(32)
    y, _, _ = oracle.layernorm(x, g, b)
    ref = F.layer_norm(torch.tensor(x), (32,), torch.tensor(g), torch.tensor(b), eps=1e-5).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


def test_layernorm_bwd_invariants_and_fd(oracle):
    M, C = 3, 16
    x = rng.standard_normal((M, C))
    g = rng.standard_normal(C)
    b = rng.standard_normal(C)
    c = rng.standard_normal((M, C))
    y, mean, rstd = oracle.layernorm(x, g, b)
    dx, dg, db = oracle.layernorm_bwd(c.copy(), x, mean, rstd, g)
    # LN output is invariant to shifting x: the gradient sums to zero per row.
    assert np.max(np.abs(dx.sum(axis=1))) < 1e-12
    # Scaling x - mean by a changes xhat only through eps:
    # d xhat/da at a=1 is xhat * eps/(var+eps), so
    # sum_c dx_c (x_c - mean) = sum_c dy_c g_c xhat_c * eps/(var+eps).
    var = x.var(axis=1)
    xhat = (x - mean[:, None]) * rstd[:, None]
    lhs = np.sum(dx * (x - mean[:, None]), axis=1)
    rhs = np.sum(c * g * xhat, axis=1) * 1e-5 / (var + 1e-5)
    assert np.max(np.abs(lhs - rhs)) < 1e-13
    loss = lambda: float(np.sum(c * oracle.layernorm(x, g, b)[0]))
    fd_check(loss, x, dx)
    fd_check(loss, g, dg)
    fd_check(loss, b, db)


def test_layernorm_bwd_accumulates_into_dx(oracle):
    x = rng.standard_normal((2, 8))
    g = np.ones(8)
    y, mean, rstd = oracle.layernorm(x, g, np.zeros(8))
    dy = rng.standard_normal((2, 8))
    dx1, _, _ = oracle.layernorm_bwd(dy.copy(), x, mean, rstd, g)
    # the C routine adds into dx: calling twice on the same buffer doubles it
    import ctypes
    dx = np.zeros_like(x)
    dg = np.zeros(8)
    db = np.zeros(8)
    f = oracle.lib().oracle_f64_layernorm_bwd
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    for _ in range(2):
        f(p(dx), p(dg), p(db), p(dy), p(x), p(mean), p(rstd), p(g), 2, 8)
    assert np.max(np.abs(dx - 2 * dx1)) < 1e-14


# ---- GELU (tanh approximation) -------------------------------------------------

def test_gelu_structure(oracle):
    x = np.linspace(-8, 8, 1601)
    y, _ = oracle.gelu(x)
    y_neg, _ = oracle.gelu(-x)
    # x * s(x) with s(x) + s(-x) = 1  =>  gelu(x) - gelu(-x) = x
    assert np.max(np.abs((y - y_neg) - x)) < 1e-12
    assert oracle.gelu(np.array([0.0]))[0][0] == 0.0
    big = np.array([10.0, 20.0])
    assert np.allclose(oracle.gelu(big)[0], big, atol=1e-12)
    assert np.allclose(oracle.gelu(-big)[0], 0.0, atol=1e-12)


def test_gelu_is_tanh_form_not_erf(oracle):
    # "Karpathy's four-hour GPT-2 reproduction in one post", what I checked
    # myself: GPT-2 uses the tanh approximation; the exact erf GELU differs.
    x = np.linspace(-6, 6, 2401)
    y, _ = oracle.gelu(x)
    exact = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    diff = np.max(np.abs(y - exact))
    assert 1e-5 < diff < 1e-3
    ref = F.gelu(torch.tensor(x), approximate="tanh").numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


def test_gelu_derivative_fd(oracle):
    x = np.linspace(-5, 5, 201)
    _, d = oracle.gelu(x)
    h = 1e-6
    num = (oracle.gelu(x + h)[0] - oracle.gelu(x - h)[0]) / (2 * h)
    assert np.max(np.abs(num - d)) < 1e-8


# ---- causal attention -----------------------------------------------------------

def test_attention_probs_rows_sum_to_one_and_are_causal(oracle):
    B, T, NH, hd = 2, 9, 3, 4
    qkv = rng.standard_normal((B * T, 3 * NH * hd))
    y, p = oracle.attention(qkv, B, T, NH, hd, want_probs=True)
    assert np.max(np.abs(p.sum(axis=-1) - 1)) < 1e-12
    assert np.all(np.triu(np.ones((T, T)), 1)[None, None] * p == 0)
    assert np.all(p >= 0)


def test_attention_special_cases(oracle):
    B, NH, hd = 2, 2, 4
    C = NH * hd
    # T = 1: each position attends only to itself, so y = v
    qkv = rng.standard_normal((B, 3 * C))
    y = oracle.attention(qkv, B, 1, NH, hd)
    assert np.max(np.abs(y - qkv[:, 2 * C:])) < 1e-14
    # q = k = 0: uniform weights over the causal prefix, y_i = mean_{j<=i} v_j
    T = 6
    qkv = rng.standard_normal((B * T, 3 * C))
    qkv[:, :2 * C] = 0
    y = oracle.attention(qkv, B, T, NH, hd).reshape(B, T, C)
    v = qkv[:, 2 * C:].reshape(B, T, C)
    ref = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert np.max(np.abs(y - ref)) < 1e-13


def test_attention_matches_torch_sdpa(oracle):
    B, T, NH, hd = 2, 11, 3, 8
    C = NH * hd
    qkv = rng.standard_normal((B * T, 3 * C))
    y = oracle.attention(qkv, B, T, NH, hd)
    t = torch.tensor(qkv).view(B, T, 3, NH, hd)
    q, k, v = (t[:, :, i].transpose(1, 2) for i in range(3))
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(1, 2).reshape(B * T, C).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


def test_attention_bwd_fd(oracle):
    B, T, NH, hd = 1, 5, 2, 3
    C = NH * hd
    qkv = rng.standard_normal((B * T, 3 * C))
    c = rng.standard_normal((B * T, C))
    dqkv = oracle.attention_bwd(c.copy(), qkv, B, T, NH, hd)
    loss = lambda: float(np.sum(c * oracle.attention(qkv, B, T, NH, hd)))
    fd_check(loss, qkv, dqkv)


# ---- cross-entropy ---------------------------------------------------------------

def test_cross_entropy_zero_logits_is_log_vocab(oracle):
    V = 509
    z = np.zeros((4, 512))
    rl, dz = oracle.cross_entropy(z, np.array([0, 1, 508, 200]), V)
    assert np.max(np.abs(rl - math.log(V))) < 1e-14
    assert np.all(dz[:, V:] == 0)


def test_cross_entropy_properties_and_torch(oracle):
    M, V, ld = 6, 37, 40
    z = rng.standard_normal((M, ld)) * 3
    z[:, V:] = 1e3  # padded columns must be ignored
    tgt = rng.integers(0, V, M)
    rl, dz = oracle.cross_entropy(z, tgt, V, scale=1.0)
    assert np.max(np.abs(dz[:, :V].sum(axis=1))) < 1e-14  # softmax - onehot sums to 0
    assert np.all(dz[:, V:] == 0)
    ref = F.cross_entropy(torch.tensor(z[:, :V]), torch.tensor(tgt), reduction="none").numpy()
    assert np.max(np.abs(rl - ref)) < 1e-12
    probs = torch.softmax(torch.tensor(z[:, :V]), dim=1).numpy()
    onehot = np.eye(V)[tgt]
    assert np.max(np.abs(dz[:, :V] - (probs - onehot))) < 1e-14


def test_cross_entropy_fd(oracle):
    M, V = 3, 7
    z = rng.standard_normal((M, V))
    tgt = np.array([1, 6, 0])
    _, dz = oracle.cross_entropy(z, tgt, V, scale=1.0 / M)
    loss = lambda: float(np.mean(oracle.cross_entropy(z, tgt, V, want_grad=False)))
    fd_check(loss, z, dz)


def test_float_instantiation_tracks_double(oracle):
    x = rng.standard_normal((8, 32))
    g = rng.standard_normal(32)
    b = rng.standard_normal(32)
    y64, _, _ = oracle.layernorm(x, g, b)
    y32, _, _ = oracle.layernorm(x.astype(np.float32), g.astype(np.float32), b.astype(np.float32), R=np.float32)
    assert np.max(np.abs(y64 - y32)) < 1e-5

"""GPU parity of the training tier: the dual-output forward (y and inner =
base + s*lora from one pass) and the backward that reads (dy, inner) only,
through the C ABI against the fp64 oracle.

The backward's oracle takes the GPU's stored inner (a host copy, exactly as
rounded to the activation dtype) as its input: that tensor is what the
backward is defined on.  Forward outputs are also checked bitwise against the
single-output compose, whose arithmetic they share.
"""
import sys

import numpy as np
import pytest
import torch

import dora_adapter_factored_amd as D
import dora_inputs as DI
import oracle
from parity_utils import check_act, host64, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


_layers = {}


def config_layer(cfg):
    if cfg not in _layers:
        _layers.clear()
        torch.cuda.empty_cache()
        say(f"[inner] generating config {cfg} ({DI.CONFIGS[cfg].name})")
        _layers[cfg] = DI.make_config(cfg, device=DEV)
        torch.cuda.synchronize()
    return _layers[cfg]


def gpu_norm(L):
    wn, g = D.factored_norm(L.W0, L.A, L.B, L.spec.s, L.m)
    torch.cuda.synchronize()
    return wn, g


def _tol_dtype(dt):
    return torch.bfloat16 if dt == torch.float16 else dt


def _dual_check(base, lora, g, s, rows=None, delta=False, tag=""):
    dt = base.dtype
    y, inner = D.compose_dual(base, lora, g, s, delta_only=delta)
    y1 = D.compose(base, lora, g, s, delta_only=delta)
    torch.cuda.synchronize()
    assert torch.equal(y, y1), f"{tag}: dual y differs from single-output compose"
    b64, l64 = host64(base), host64(lora)
    got_y, got_i = host64(y), host64(inner)
    if rows is not None:
        b64, l64, got_y, got_i = b64[rows], l64[rows], got_y[rows], got_i[rows]
    r_y, r_i = oracle.compose_forward_inner(b64, l64, host64(g), s, delta_only=delta)
    check_act(got_y, r_y, _tol_dtype(dt), f"{tag} y(delta={delta})")
    check_act(got_i, r_i, _tol_dtype(dt), f"{tag} inner")
    return y, inner


def _inner_bwd_check(dy, inner, g, wn, s, eps, rows=None, cols=None, delta=False, tag=""):
    dt = dy.dtype
    db, dl, dm = D.compose_backward_inner(dy, inner, g, wn, s, eps, delta_only=delta)
    torch.cuda.synchronize()
    csel = slice(None) if cols is None else cols
    d64, i64 = host64(dy)[:, csel], host64(inner)[:, csel]
    r_db, r_dl, r_dm = oracle.compose_backward_inner(d64, i64, host64(g)[csel], host64(wn)[csel], s, eps,
                                                     delta_only=delta)
    got_db, got_dl = host64(db)[:, csel], host64(dl)[:, csel]
    if rows is not None:
        got_db, got_dl, r_db, r_dl = got_db[rows], got_dl[rows], r_db[rows], r_dl[rows]
    td = _tol_dtype(dt)
    check_act(got_db, r_db, td, f"{tag} d_base")
    check_act(got_dl, r_dl, td, f"{tag} d_lora")
    check_act(host64(dm)[csel], r_dm, td, f"{tag} d_m")
    return db, dl, dm


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_dual_forward_config(cfg):
    L = config_layer(cfg)
    say(f"[inner] dual forward config {cfg}")
    _, g = gpu_norm(L)
    rows = None if cfg in (1, 2) else sample_rows(L.spec.T, 256, seed=60 + cfg)
    _dual_check(L.base_out, L.lora_out, g, L.spec.s, rows=rows, tag=f"cfg{cfg}")
    if cfg in (1, 3):
        _dual_check(L.base_out, L.lora_out, g, L.spec.s, rows=rows, delta=True, tag=f"cfg{cfg}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_inner_backward_config(cfg):
    L = config_layer(cfg)
    say(f"[inner] backward from (dy, inner) config {cfg}")
    wn, g = gpu_norm(L)
    s = L.spec.s
    eps = D.default_eps(L.dy.dtype)
    _, inner = D.compose_dual(L.base_out, L.lora_out, g, s)
    rows = None if cfg in (1, 2) else sample_rows(L.spec.T, 256, seed=70 + cfg)
    cols = None if cfg != 4 else sample_rows(L.spec.d_out, 256, seed=74)
    db, dl, _ = _inner_bwd_check(L.dy, inner, g, wn, s, eps, rows=rows, cols=cols, tag=f"cfg{cfg}")
    # d_base and d_lora do not depend on the activations: identical to the
    # two-activation backward's
    db2, dl2, _ = D.compose_backward(L.dy, L.base_out, L.lora_out, g, wn, s, eps)
    torch.cuda.synchronize()
    assert torch.equal(db, db2) and torch.equal(dl, dl2)
    if cfg in (1, 3):
        _inner_bwd_check(L.dy, inner, g, wn, s, eps, rows=rows, cols=cols, delta=True, tag=f"cfg{cfg}")


INNER_EDGE = [
    # T, d_out, dtype
    (1, 1000, "bf16"), (37, 1003, "bf16"), (5, 7, "f32"), (70, 517, "f32"), (33, 520, "f16"),
    (65, 8, "bf16"), (2, 1, "bf16"), (300, 4104, "bf16"), (129, 8200, "bf16"),
]


@pytest.mark.parametrize("T,d_out,dt", INNER_EDGE)
def test_inner_edge_shapes(T, d_out, dt):
    say(f"[inner] edge T={T} d_out={d_out} {dt}")
    torch.manual_seed(7 * T + d_out)
    dtype = DI.DTYPES[dt]
    base = torch.randn(T, d_out).to(dtype).to(DEV)
    lora = torch.randn(T, d_out).to(dtype).to(DEV)
    dy = torch.randn(T, d_out).to(dtype).to(DEV)
    g = (1.0 + 1e-3 * torch.randn(d_out)).float().to(DEV)
    wn = (1.0 + 0.1 * torch.rand(d_out)).float().to(DEV)
    s = 0.75
    _, inner = _dual_check(base, lora, g, s, tag="edge")
    _inner_bwd_check(dy, inner, g, wn, s, 1e-6, tag="edge")
    _inner_bwd_check(dy, inner, g, wn, s, 1e-6, delta=True, tag="edge")


def _misaligned(t):
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def test_inner_unaligned_pointers_take_the_scalar_path():
    say("[inner] unaligned pointers")
    L = DI.make_layer(DI.custom_spec(256, 512, 16, 64, dtype="bf16"), 22, device=DEV)
    wn, g = gpu_norm(L)
    s = L.spec.s
    y_a, i_a = D.compose_dual(L.base_out, L.lora_out, g, s)
    y_u, i_u = D.compose_dual(_misaligned(L.base_out), _misaligned(L.lora_out), g, s,
                              out=_misaligned(L.base_out), inner=_misaligned(L.lora_out))
    a = D.compose_backward_inner(L.dy, i_a, g, wn, s)
    u = D.compose_backward_inner(_misaligned(L.dy), _misaligned(i_a), g, wn, s)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_u) and torch.equal(i_a, i_u)
    # elementwise grads: same arithmetic on either path; d_m: a different
    # summation order, so against the oracle
    assert torch.equal(a[0], u[0]) and torch.equal(a[1], u[1])
    _, _, r_dm = oracle.compose_backward_inner(host64(L.dy), host64(i_a), host64(g), host64(wn), s,
                                               D.default_eps(torch.bfloat16))
    check_act(host64(u[2]), r_dm, torch.bfloat16, "d_m scalar path")


def test_dual_in_place():
    say("[inner] in-place y over base_out, inner over lora_out")
    L = DI.make_layer(DI.custom_spec(512, 256, 16, 96, dtype="bf16"), 42, device=DEV)
    _, g = gpu_norm(L)
    y_ref, i_ref = D.compose_dual(L.base_out, L.lora_out, g, L.spec.s)
    b, l = L.base_out.clone(), L.lora_out.clone()
    y, inner = D.compose_dual(b, l, g, L.spec.s, out=b, inner=l)
    torch.cuda.synchronize()
    assert y.data_ptr() == b.data_ptr() and inner.data_ptr() == l.data_ptr()
    assert torch.equal(y, y_ref) and torch.equal(inner, i_ref)


def test_inner_backward_frozen_magnitude_and_dy_alias():
    say("[inner] frozen m, d_base over dy")
    L = DI.make_layer(DI.custom_spec(512, 256, 16, 96, dtype="bf16"), 43, device=DEV)
    wn, g = gpu_norm(L)
    s = L.spec.s
    db, dl, dm = D.compose_backward_inner(L.dy, None, g, None, s, need_d_m=False)
    assert dm is None
    dyc = L.dy.clone()
    db2, _, _ = D.compose_backward_inner(dyc, None, g, None, s, need_d_m=False, need_d_lora=False, d_base=dyc)
    torch.cuda.synchronize()
    assert torch.equal(db2, db)
    r_db, r_dl, _ = oracle.compose_backward_inner(host64(L.dy), np.zeros_like(host64(L.dy)), host64(g),
                                                  np.ones(L.spec.d_out), s, 1e-6)
    check_act(host64(db), r_db, torch.bfloat16, "d_base frozen")
    check_act(host64(dl), r_dl, torch.bfloat16, "d_lora frozen")


def test_inner_t_zero():
    say("[inner] T = 0")
    g = torch.ones(64, device=DEV)
    empty = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    y, inner = D.compose_dual(empty, empty, g, 1.0)
    _, _, dm = D.compose_backward_inner(empty, empty, g, g, 1.0, 1e-6)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and inner.shape == (0, 64)
    assert torch.equal(dm, torch.zeros(64, device=DEV))


def test_inner_backward_deterministic():
    L = config_layer(3)
    say("[inner] backward determinism")
    wn, g = gpu_norm(L)
    _, inner = D.compose_dual(L.base_out, L.lora_out, g, L.spec.s)
    a = tuple(t.clone() for t in D.compose_backward_inner(L.dy, inner, g, wn, L.spec.s))
    b = D.compose_backward_inner(L.dy, inner, g, wn, L.spec.s)
    torch.cuda.synchronize()
    for x, z in zip(a, b):
        assert torch.equal(x, z)


def test_inner_autograd_function_matches_direct_calls():
    say("[inner] autograd wiring")
    L = DI.make_layer(DI.custom_spec(256, 128, 8, 40, dtype="bf16"), 52, device=DEV)
    wn, g = gpu_norm(L)
    eps = D.default_eps(torch.bfloat16)
    base = L.base_out.clone().requires_grad_(True)
    lora = L.lora_out.clone().requires_grad_(True)
    m = L.m.clone().requires_grad_(True)
    y = D.DoRAComposeInner.apply(base, lora, m, g, wn, L.spec.s, eps, False)
    y.backward(L.dy)
    y_ref, inner = D.compose_dual(L.base_out, L.lora_out, g, L.spec.s)
    db, dl, dm = D.compose_backward_inner(L.dy, inner, g, wn, L.spec.s, eps)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y_ref)
    assert torch.equal(base.grad, db) and torch.equal(lora.grad, dl) and torch.equal(m.grad, dm)
    # frozen magnitude: no d_m reduction, no inner needed for it
    base.grad = lora.grad = None
    y = D.DoRAComposeInner.apply(base, lora, m.detach(), g, wn, L.spec.s, eps, False)
    y.backward(L.dy)
    torch.cuda.synchronize()
    assert torch.equal(base.grad, db) and torch.equal(lora.grad, dl)

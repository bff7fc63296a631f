"""GPU parity of the grouped norm (several projections sharing r in one call,
each with its own d_out and d_in): every member's result is bitwise that of
its own single call, and agrees with the fp64 oracle on sampled rows."""
import sys

import numpy as np
import pytest
import torch

import dora_adapter_factored_amd as D
import dora_inputs as DI
import oracle
from parity_utils import check_rel, host64, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _members(layers, with_m=True):
    return [(L.W0, L.A, L.B, L.spec.s, L.m if with_m else None) for L in layers]


def _check_against_single_calls(layers, results, with_m=True):
    torch.cuda.synchronize()
    for L, (wn, g) in zip(layers, results):
        wn1, g1 = D.factored_norm(L.W0, L.A, L.B, L.spec.s, L.m if with_m else None)
        torch.cuda.synchronize()
        assert torch.equal(wn, wn1), L.spec.name
        if with_m:
            assert torch.equal(g, g1), L.spec.name
        else:
            assert g is None


def _check_oracle(L, wn, g, nrows, seed, rtol):
    rows = sample_rows(L.spec.d_out, nrows, seed=seed)
    ref = oracle.dense_row_norm(L.W0.cpu(), L.A.cpu(), L.B.cpu(), L.spec.s, rows=rows)
    check_rel(host64(wn)[rows], ref, rtol, f"{L.spec.name} wnorm")
    if g is not None:
        eps = D.default_eps(L.W0.dtype)
        check_rel(host64(g)[rows], oracle.magnitude_scale(host64(L.m)[rows], ref, eps), rtol, f"{L.spec.name} g")


def test_group_of_one_layer_of_the_sweep():
    # all seven projections of one layer: q, k, v, o, gate, up read the
    # 5120-wide input, down the 27648-wide one
    layers = []
    for proj in range(len(DI.SWEEP_PROJECTIONS)):
        spec = DI.sweep_spec(proj)
        say(f"[group] generating {spec.name}")
        layers.append(DI.make_layer(spec, DI.sweep_seed(3, proj), device=DEV, activations=False,
                                    gen_device="cuda"))
    say(f"[group] sweep layer, {len(layers)} members")
    res = D.factored_norm_group(_members(layers))
    _check_against_single_calls(layers, res)
    for j, (L, (wn, g)) in enumerate(zip(layers, res)):
        _check_oracle(L, wn, g, 64, 90 + j, 2e-3)


GROUP_CASES = [
    # (members as (d_out, d_in), r, dtype): grouped kernels when bf16, aligned, r > 128
    (((300, 4096), (1000, 4096), (520, 4096)), 256, "bf16"),
    (((64, 1024), (8, 1024), (1, 1024)), 384, "bf16"),
    (((257, 2048), (129, 2048)), 200, "bf16"),
    (((300, 1000), (520, 4096), (64, 2048), (96, 8200)), 256, "bf16"),   # different d_in
    (((64, 48), (40, 100)), 8, "f32"),             # member by member
    (((500, 640), (33, 640)), 16, "bf16"),         # r <= 128: member by member
    (((300, 2056), (40, 2056)), 136, "bf16"),      # grouped from r = 129
    (((200, 1024), (64, 1024)), 128, "bf16"),      # r = 128: member by member
    # 32 and 29 m-tiles in eight K-chunks beside a short member
    (((8000, 2048), (7200, 2048), (300, 2048)), 384, "bf16"),
]


@pytest.mark.parametrize("sizes,r,dt", GROUP_CASES)
def test_group_shapes(sizes, r, dt):
    say(f"[group] members={sizes} r={r} {dt}")
    layers = [DI.make_layer(DI.custom_spec(d_out, d_in, r, 1, dtype=dt, s=1.5, b_std=0.05), 700 + j, device=DEV,
                            activations=False) for j, (d_out, d_in) in enumerate(sizes)]
    res = D.factored_norm_group(_members(layers))
    _check_against_single_calls(layers, res)
    rtol = 2e-3 if dt == "bf16" else 1e-4
    for j, (L, (wn, g)) in enumerate(zip(layers, res)):
        _check_oracle(L, wn, g, 128, j, rtol)


def test_group_mixed_members_and_no_magnitude():
    say("[group] s = 0 member, m = None members, unaligned member")
    layers = [DI.make_layer(DI.custom_spec(d, 1024, 256, 1, s=1.0, b_std=0.05), 800 + j, device=DEV,
                            activations=False) for j, d in enumerate((256, 512, 384))]
    # wnorm only (m = None) for every member: the grouped kernels
    res = D.factored_norm_group(_members(layers, with_m=False))
    _check_against_single_calls(layers, res, with_m=False)
    # one member with s = 0 (base norm only): member by member
    members = _members(layers)
    members[1] = (layers[1].W0, layers[1].A, layers[1].B, 0.0, layers[1].m)
    res = D.factored_norm_group(members)
    torch.cuda.synchronize()
    wn1, _ = D.factored_norm(layers[1].W0, layers[1].A, layers[1].B, 0.0, layers[1].m)
    torch.cuda.synchronize()
    assert torch.equal(res[1][0], wn1)
    ref = torch.linalg.vector_norm(layers[1].W0.double(), dim=1).cpu().numpy()
    check_rel(host64(res[1][0]), ref, 2e-3, "s = 0 member")
    for j in (0, 2):
        wn, g = D.factored_norm(layers[j].W0, layers[j].A, layers[j].B, 1.0, layers[j].m)
        torch.cuda.synchronize()
        assert torch.equal(res[j][0], wn) and torch.equal(res[j][1], g)
    # one member whose W0 is not 16-byte aligned: member by member, same results
    buf = torch.empty(layers[2].W0.numel() + 1, dtype=torch.bfloat16, device=DEV)
    W0u = buf[1:].view(layers[2].W0.shape)
    W0u.copy_(layers[2].W0)
    members = _members(layers)
    members[2] = (W0u, layers[2].A, layers[2].B, 1.0, layers[2].m)
    res = D.factored_norm_group(members)
    torch.cuda.synchronize()
    for j, (W0, A, B, s, m) in enumerate(members):
        wn, g = D.factored_norm(W0, A, B, s, m)
        torch.cuda.synchronize()
        assert torch.equal(res[j][0], wn) and torch.equal(res[j][1], g), j
    _check_oracle(layers[2], res[2][0], res[2][1], 128, 7, 2e-3)


def test_group_of_eight_members_with_their_own_d_in():
    # the largest group, every member with its own [d_out, d_in], one of a
    # single row; members fall in four sizes of k-tiles per workgroup
    sizes = ((1, 4096), (300, 1000), (1024, 2048), (64, 8200), (513, 512), (2048, 3000), (257, 6144), (96, 1024))
    say(f"[group] eight members {sizes}")
    layers = [DI.make_layer(DI.custom_spec(d_out, d_in, 320, 1, s=0.75, b_std=0.05), 950 + j, device=DEV,
                            activations=False) for j, (d_out, d_in) in enumerate(sizes)]
    res = D.factored_norm_group(_members(layers))
    _check_against_single_calls(layers, res)
    for j, (L, (wn, g)) in enumerate(zip(layers, res)):
        _check_oracle(L, wn, g, 64, 30 + j, 2e-3)


def test_group_mixed_d_in_with_s_zero_and_no_magnitude():
    say("[group] different d_in; an s = 0 member; m = None members")
    layers = [DI.make_layer(DI.custom_spec(d_out, d_in, 256, 1, s=1.0, b_std=0.05), 990 + j, device=DEV,
                            activations=False) for j, (d_out, d_in) in enumerate(((384, 1024), (200, 5000), (640, 2048)))]
    members = [(L.W0, L.A, L.B, L.spec.s, None) for L in layers]
    members[1] = (layers[1].W0, layers[1].A, layers[1].B, 0.0, layers[1].m)
    res = D.factored_norm_group(members)
    torch.cuda.synchronize()
    for j, (W0, A, B, s, m) in enumerate(members):
        wn, g = D.factored_norm(W0, A, B, s, m)
        torch.cuda.synchronize()
        assert torch.equal(res[j][0], wn), j
        assert (res[j][1] is None) == (m is None) and (m is None or torch.equal(res[j][1], g)), j
    ref = torch.linalg.vector_norm(layers[1].W0.double(), dim=1).cpu().numpy()
    check_rel(host64(res[1][0]), ref, 2e-3, "s = 0 member")


def test_group_of_one_and_repeated_calls():
    say("[group] one member; repeated calls")
    L = DI.make_layer(DI.custom_spec(1024, 2048, 384, 1, b_std=0.05), 901, device=DEV, activations=False)
    a = D.factored_norm_group(_members([L]))
    a = [(w.clone(), g.clone()) for w, g in a]
    b = D.factored_norm_group(_members([L]))
    _check_against_single_calls([L], b)
    assert torch.equal(a[0][0], b[0][0]) and torch.equal(a[0][1], b[0][1])

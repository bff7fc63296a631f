"""Plain fp64 CPU oracle for the DoRA factored-norm / fused-compose hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links this file; only the tests, the
smoke check and the benchmark's CPU-baseline leg do.  It shares no code with
the GPU path.

Every function works on numpy float64 arrays (inputs are upcast exactly, so a
bf16 or fp32 tensor keeps its value) and follows the plain definition of the
quantity it returns, written out without blocking, fusion or reordering.

Sources, cited by short title and section:
  [ScalingDoRA]  "Scaling DoRA: High-Rank Adaptation via Factored Norms and
                 Fused Kernels" (Zelenin & Zhuravlyova, arXiv:2603.22276;
                 paperlayer.ai summary page).
  [DoRA-wiki]    "DoRA" (aiwiki.thehackersbrain.dev entry), DoRALinear listing.
  [LoRA&DoRA]    "LoRA & DoRA: The Math, Memory, and Trade-offs" (dev.to).
  [Lesson18]     "Lesson 18. DoRA: Magnitude and Direction".

Axis convention: W0 is stored [d_out, d_in] (the nn.Linear layout) and the
norm is taken over d_in for each of the d_out rows, one magnitude per output
feature, as in [DoRA-wiki] (weight.norm(dim=1)) and [ScalingDoRA] Abstract
("row-wise norm of W + sBA").  [Lesson18] and [LoRA&DoRA] §2 state the same
algorithm per column of the transposed matrix.

Parity pins: every function here is pinned by tests/test_oracle.py against
closed forms, hand-worked examples (tests/golden/), special cases that reduce
to a textbook routine, finite differences, or torch CPU fp64 autograd.
"""
from __future__ import annotations

import numpy as np

# Rows of the dense [rows, d_in] fp64 product materialised at once.
_ROW_CHUNK = 1024


def as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (any float dtype,
    bf16 included) to a numpy float64 array."""
    if hasattr(x, "detach"):  # torch tensor: upcast inside torch (bf16 -> f64 is exact)
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def adapted_weight_rows(W0, A, B, s, rows=None) -> np.ndarray:
    """V' = W0 + s * (B @ A), restricted to `rows` when given.

    The adapted (un-normalised) weight of DoRA: [LoRA&DoRA] §1 (W = W0 + sBA)
    and §2 (V' = W0 + sBA); [DoRA-wiki] forward (base.weight + (B @ A) * scale).
    """
    W0, A, B = as_f64(W0), as_f64(A), as_f64(B)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        W0, B = W0[rows], B[rows]
    return W0 + float(s) * (B @ A)


def dense_row_norm(W0, A, B, s, rows=None) -> np.ndarray:
    """wnorm_i = ||W0_i + s (BA)_i||_2 by materialising the dense product.

    This is the definition the factored norm reproduces: [ScalingDoRA]
    Abstract and §1 (row-wise norm of W + sBA, dense [d_out, d_in] product
    BA); [DoRA-wiki] forward (weight.norm(dim=1)).  Rows are materialised in
    chunks so that large layers fit in host memory; chunking over rows does not
    change any row's arithmetic.
    """
    W0 = as_f64(W0)
    idx = np.arange(W0.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty(idx.shape[0], dtype=np.float64)
    for c0 in range(0, idx.shape[0], _ROW_CHUNK):
        sel = idx[c0:c0 + _ROW_CHUNK]
        Wp = adapted_weight_rows(W0, A, B, s, rows=sel)
        out[c0:c0 + sel.shape[0]] = np.sqrt(np.sum(Wp * Wp, axis=1))
    return out


def factored_row_norm(W0, A, B, s, rows=None) -> np.ndarray:
    """wnorm from the three factored terms, never forming B @ A.

    [ScalingDoRA] §2 (squared row norm = base + cross + BA-norm terms; the
    cross term from row-wise inner products with W0 A^T, the BA-norm term
    through the Gram matrix A A^T) and App. B, norm assembly
    (max(base_sq + two_s*cross + s2*ba_sq, 0), then a square root).

      base_i  = sum_k W0_ik^2
      cross_i = B_i . (W0 A^T)_i
      ba_i    = B_i (A A^T) B_i^T
      n2_i    = base_i + 2 s cross_i + s^2 ba_i ;  wnorm_i = sqrt(max(n2_i, 0))

    Written independently of dense_row_norm; used as a cross-check of the
    algebra, not as the parity reference.
    """
    W0, A, B = as_f64(W0), as_f64(A), as_f64(B)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        W0, B = W0[rows], B[rows]
    s = float(s)
    base = np.einsum("ik,ik->i", W0, W0)
    U = W0 @ A.T                      # [rows, r]
    G = A @ A.T                       # [r, r]
    cross = np.einsum("ij,ij->i", B, U)
    ba = np.einsum("ij,ij->i", B @ G, B)
    n2 = base + (2.0 * s) * cross + (s * s) * ba
    return np.sqrt(np.maximum(n2, 0.0))


def magnitude_scale(m, wnorm, eps) -> np.ndarray:
    """g = m / max(wnorm, eps): [ScalingDoRA] §4 (Precision) and App. B
    (magnitude division)."""
    m, wnorm = as_f64(m), as_f64(wnorm)
    return m / np.maximum(wnorm, float(eps))


def compose_forward(base_out, lora_out, g, s, delta_only=False) -> np.ndarray:
    """DoRA output from the two branch outputs.

    y_tj = g_j * (base_tj + s * lora_tj), the activation-space form of
    x (diag(g) (W0 + sBA))^T with base = x W0^T and lora = (x A^T) B^T
    ([DoRA-wiki] forward; [LoRA&DoRA] §1 y = W0 x + sB(Ax)).

    delta_only returns the module contract of [ScalingDoRA] Data
    Availability: dY = g * (s lora) + (g - 1) * base, which the caller adds to
    the base output.  g broadcasts along the last (d_out) axis
    ([ScalingDoRA] App. B, kernel design).
    """
    base, lora, g = as_f64(base_out), as_f64(lora_out), as_f64(g)
    s = float(s)
    if delta_only:
        return g * (s * lora) + (g - 1.0) * base
    return g * (base + s * lora)


def compose_forward_inner(base_out, lora_out, g, s, delta_only=False):
    """Dual-output forward of the training tier ([ScalingDoRA] §4, Tier 1:
    one kernel produces the layer output and the inner term together).

    Returns (y, inner) with inner_tj = base_tj + s * lora_tj, the factor
    that g multiplies (y = g * inner) and the only activation the magnitude
    gradient needs; y is compose_forward's output (or the delta).
    """
    base, lora = as_f64(base_out), as_f64(lora_out)
    inner = base + float(s) * lora
    return compose_forward(base_out, lora_out, g, s, delta_only=delta_only), inner


def compose_backward_inner(dy, inner, g, wnorm, s, eps, delta_only=False):
    """Backward of the training tier from (dy, inner) alone, norm detached.

    With y = g * inner and inner = base + s lora ([ScalingDoRA] §4, Tier 1;
    the norm detached as in [DoRA-wiki] and [ScalingDoRA] Data Availability):
      d_base = g * dy          (delta_only: (g - 1) * dy)
      d_lora = g * s * dy
      d_m_j  = sum_t dy_tj * inner_tj / max(wnorm_j, eps)
    Returns (d_base, d_lora, d_m).
    """
    dy, inner, g, wnorm = as_f64(dy), as_f64(inner), as_f64(g), as_f64(wnorm)
    s = float(s)
    d_base = ((g - 1.0) if delta_only else g) * dy
    d_lora = (g * s) * dy
    d_m = np.sum(dy * inner, axis=0) / np.maximum(wnorm, eps)
    return d_base, d_lora, d_m


def compose_backward(dy, base_out, lora_out, g, wnorm, s, eps, delta_only=False):
    """Gradients of compose_forward with the norm detached.

    The norm is a constant for autograd ([DoRA-wiki] .detach() note;
    [ScalingDoRA] Data Availability: norm quantities detached; [LoRA&DoRA]
    §6).  With g = m / max(wnorm, eps) and y = g * (base + s lora):
      d_base = g * dy           (delta_only: (g - 1) * dy)
      d_lora = g * s * dy
      d_m_j  = sum_t dy_tj * (base_tj + s lora_tj) / max(wnorm_j, eps)
    d_m is the separate magnitude reduction of [ScalingDoRA] §3 (Backward
    Kernel) and App. B.  Returns (d_base, d_lora, d_m).
    """
    dy, base, lora = as_f64(dy), as_f64(base_out), as_f64(lora_out)
    g, wnorm = as_f64(g), as_f64(wnorm)
    s = float(s)
    d_base = (g - 1.0) * dy if delta_only else g * dy
    d_lora = (g * s) * dy
    d_m = np.sum(dy * (base + s * lora), axis=0) / np.maximum(wnorm, float(eps))
    return d_base, d_lora, d_m


def dora_linear_forward(x, W0, A, B, m, s, eps) -> np.ndarray:
    """Dense DoRA linear layer in weight space, bias-free:
    W' = diag(m / max(||V'_i||, eps)) V' with V' = W0 + sBA, then y = x W'^T.

    [DoRA-wiki] DoRALinear.forward; [LoRA&DoRA] §2 (w'_j = m_j v'_j/||v'_j||)
    and §6 (merged DoRA weight).  Used to tie the activation-space compose to
    the pages' weight-space definition.
    """
    x = as_f64(x)
    Vp = adapted_weight_rows(W0, A, B, s)
    n = np.sqrt(np.sum(Vp * Vp, axis=1))
    Wm = (as_f64(m) / np.maximum(n, float(eps)))[:, None] * Vp
    return x @ Wm.T


def merged_weight(W0, A, B, m, s, eps) -> np.ndarray:
    """DoRA merge for serving: W_merged = m * (W0 + sBA) / ||W0 + sBA||_row.

    [LoRA&DoRA] §6 (W_DoRA,merged); [Lesson18] "What it costs" (merged DoRA
    is an ordinary matrix).  Row convention as in the module docstring.
    """
    Vp = adapted_weight_rows(W0, A, B, s)
    n = np.sqrt(np.sum(Vp * Vp, axis=1))
    return (as_f64(m) / np.maximum(n, float(eps)))[:, None] * Vp


def merge_with_scale(W0, A, B, g, s, rows=None) -> np.ndarray:
    """The merge step given the scale: W_merged = diag(g) (W0 + sBA).

    With g = m / max(||W0 + sBA||_row, eps) this is merged_weight ([LoRA&DoRA]
    §6; [ScalingDoRA] §4 computes g once from the factored norm, so a merge
    for serving reuses it).  Restricted to `rows` when given (g is then
    indexed by the same rows).
    """
    g = as_f64(g)
    if rows is not None:
        g = g[np.asarray(rows, dtype=np.int64)]
    return g[:, None] * adapted_weight_rows(W0, A, B, s, rows=rows)

"""fp64 oracle of the Muon step for one or many 2D hidden weight matrices.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Layout: PyTorch's, a weight is ``(rows, cols) = (fan-out, fan-in)``
("About Muon: Why Not Adam", section "How Do We Turn It Into a Real
Optimizer?", the multiplier paragraph).  All arithmetic is numpy float64;
inputs arrive as whatever the GPU was given (fp32 or bf16 values) and are
upcast exactly.
"""

import numpy as np

from .storage import store

# Quintic coefficients (a, b, c) of p(s) = a s + b s^3 + c s^5, used for every
# iteration.  "The Optimizer Wars ...", section "What is Muon? Momentum
# orthogonalized by Newton-Schulz"; "About Muon: Why Not Adam", section
# "Making It Actually Run", subsection on why the iteration does not converge.
MUON_COEFFS = (3.4445, -4.7750, 2.0315)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def momentum_update(M, G, mu):
    """Momentum buffer as an exponential moving average of the gradient.

    The optimizer moves the buffer a fraction ``1 - mu`` of the way towards the
    new gradient, i.e. ``M <- mu*M + (1 - mu)*G``
    ("About Muon: Why Not Adam", section "The whole thing, in about forty
    lines": the buffer is interpolated towards the gradient by ``1 - mu``).
    """
    M = _f64(M)
    G = _f64(G)
    return mu * M + (1.0 - mu) * G


def nesterov_blend(G, M_new, mu, nesterov=True):
    """Input of the orthogonalisation.

    With Nesterov the gradient is interpolated towards the *updated* buffer by
    ``mu``: ``Y = (1 - mu)*G + mu*M_new``; without it ``Y = M_new``
    ("About Muon: Why Not Adam", section "The whole thing, in about forty
    lines"; Muon uses the Nesterov form per "Por qué AdamW ...", section
    "Momentum: recordar el paso anterior").
    """
    M_new = _f64(M_new)
    if not nesterov:
        return M_new.copy()
    return (1.0 - mu) * _f64(G) + mu * M_new


def _gram_polynomial(S, a, b, c):
    """``a I + b S + c S^2`` for a symmetric Gram matrix ``S``, in Horner form
    ``a I + S (b I + c S)``."""
    eye = np.eye(S.shape[0])
    return a * eye + S @ (b * eye + c * S)


def newton_schulz(G, steps=5, eps=1e-7, coeffs=None):
    """Approximate polar factor of ``G`` by iterated odd quintic polynomials.

    "About Muon: Why Not Adam", section "Making It Actually Run": after
    scaling by the Frobenius norm plus ``eps`` (the norm bounds the largest
    singular value, so every singular value lands in (0, 1]), each iteration
    replaces ``X`` by the odd matrix polynomial ``p(X) = a X + b X X^T X +
    c (X X^T)^2 X``, which maps each singular value ``s`` to ``a s + b s^3 +
    c s^5`` and leaves the singular vectors alone.  The polynomial only needs
    a Gram matrix, and the section takes it on the short side: for a wide
    ``X`` (rows <= cols), ``p(X) = q(X X^T) X``; for a tall one, ``p(X) =
    X q(X^T X)``, with ``q(S) = a I + b S + c S^2``.  Both are the same
    matrix; the short side only makes ``S`` small.

    ``coeffs`` is either one triple used for every iteration (default: the
    Muon triple) or a sequence of ``steps`` triples, one per iteration.
    """
    X = _f64(G)
    if X.ndim != 2:
        raise ValueError("newton_schulz expects a 2D matrix")
    if coeffs is None:
        coeffs = MUON_COEFFS
    coeffs = np.asarray(coeffs, dtype=np.float64)
    if coeffs.ndim == 1:
        schedule = [tuple(coeffs)] * steps
    else:
        if coeffs.shape != (steps, 3):
            raise ValueError("per-iteration coefficients must have shape (steps, 3)")
        schedule = [tuple(row) for row in coeffs]

    X = X / (np.sqrt(np.sum(X * X)) + eps)
    wide = X.shape[0] <= X.shape[1]
    for a, b, c in schedule:
        if wide:
            X = _gram_polynomial(X @ X.T, a, b, c) @ X
        else:
            X = X @ _gram_polynomial(X.T @ X, a, b, c)
    return np.ascontiguousarray(X)


def shape_scale(rows, cols, mode="moonlight"):
    """Per-matrix multiplier of the orthogonalised update.

    ``(rows, cols) = (fan-out, fan-in)``.  "About Muon: Why Not Adam":
    * ``moonlight``: ``0.2 * sqrt(max(rows, cols))`` -- entry RMS near 0.2 so
      the AdamW learning rate can be shared (section "Why Muon?", scaling
      paragraph; and the forty-line optimizer);
    * ``jordan``: ``sqrt(max(1, rows/cols))`` (section "How Do We Turn It Into
      a Real Optimizer?", the multiplier paragraph);
    * ``bernstein``: ``sqrt(fan-out / fan-in) = sqrt(rows/cols)``, the spectral
      condition's ratio (section "Why not Adam", problem 1);
    * ``none``: 1.
    """
    rows = float(rows)
    cols = float(cols)
    if mode == "moonlight":
        return 0.2 * np.sqrt(max(rows, cols))
    if mode == "jordan":
        return np.sqrt(max(1.0, rows / cols))
    if mode == "bernstein":
        return np.sqrt(rows / cols)
    if mode == "none":
        return 1.0
    raise ValueError("unknown scale mode %r" % (mode,))


def qk_clip(W, s_max, tau, block_rows):
    """QK-Clip of a query or key projection after its optimizer update.

    "The Optimizer Wars ...", section "What is MuonClip? Kimi K2's fix for
    exploding attention scores": for head h with maximum attention logit
    ``S_max^h``, ``gamma_h = min(1, tau / S_max^h)``; the head's query and key
    weights are each multiplied by ``sqrt(gamma_h)`` so their product, and the
    logits, shrink by ``gamma_h``.  Here ``W`` holds the heads as consecutive
    blocks of ``block_rows`` rows (PyTorch layout, one row per output
    feature) and ``s_max[h]`` is head h's maximum logit.  A head whose
    ``S_max`` does not exceed ``tau`` (including ``S_max <= 0``) is left alone.
    """
    W = _f64(W).copy()
    s_max = np.asarray(s_max, dtype=np.float64).reshape(-1)
    for h in range(s_max.size):
        rows = slice(h * block_rows, min((h + 1) * block_rows, W.shape[0]))
        if s_max[h] > tau:
            W[rows] *= np.sqrt(tau / s_max[h])
    return W


def muon_matrix_step(W, G, M, *, lr, mu=0.95, weight_decay=0.0, nesterov=True,
                     eps=1e-7, steps=5, coeffs=None, scale_mode="moonlight",
                     extra_scale=1.0, qk_smax=None, qk_block_rows=0, qk_tau=100.0,
                     param_dtype="fp32"):
    """One Muon step for one weight matrix; returns ``(W_new, M_new, O)``.

    Order of operations ("About Muon: Why Not Adam", section "The whole thing,
    in about forty lines"; decoupled decay from section "How Do We Turn It
    Into a Real Optimizer?"):

    1. ``M_new = mu M + (1 - mu) G``;
    2. ``Y`` = Nesterov blend of ``G`` towards ``M_new`` (or ``M_new``);
    3. ``O = newton_schulz(Y)``;
    4. ``s = shape_scale(rows, cols) * extra_scale`` (the extra factor is the
       starter configuration's extra scale knob, "Why Muon Works", 7.6);
    5. ``W <- (1 - lr*wd) W`` (decay uses the weight before the update), then
       ``W <- W - lr * s * O``;
    6. with ``qk_smax`` given, :func:`qk_clip` on the updated weight
       (MuonClip: the clip follows the ordinary Muon update);
    7. a ``param_dtype="bf16"`` weight stores the result of 5-6 rounded
       once to bfloat16 (:func:`oracle.storage.store`).

    ``O`` is the orthogonalised update before the multiplier, returned so
    tests can compare it directly.
    """
    W = _f64(W)
    rows, cols = W.shape
    M_new = momentum_update(M, G, mu)
    Y = nesterov_blend(G, M_new, mu, nesterov)
    O = newton_schulz(Y, steps=steps, eps=eps, coeffs=coeffs)
    s = shape_scale(rows, cols, scale_mode) * extra_scale
    W_new = (1.0 - lr * weight_decay) * W
    W_new = W_new - (lr * s) * O
    if qk_smax is not None:
        W_new = qk_clip(W_new, qk_smax, qk_tau, qk_block_rows)
    return store(W_new, param_dtype), M_new, O


def muon_step(weights, grads, moms, **hparams):
    """Muon over a list of matrices: each matrix is independent, so this is a
    plain loop of :func:`muon_matrix_step` (the forty-line optimizer loops
    over parameters one at a time).  Returns three lists ``(W, M, O)``."""
    Ws, Ms, Os = [], [], []
    for W, G, M in zip(weights, grads, moms):
        w, m, o = muon_matrix_step(W, G, M, **hparams)
        Ws.append(w)
        Ms.append(m)
        Os.append(o)
    return Ws, Ms, Os

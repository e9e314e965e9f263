"""Shared test helpers: run workloads through libmuon and the oracle.

The GPU side goes through the C ABI (the binding in muon_step_02_amd); the
reference side is the fp64 oracle fed with the exact values the GPU saw.
"""

import numpy as np
import torch

import oracle
import muon_step_02_amd as mu

# Tolerances (relative Frobenius error per matrix or tensor):
TOL_O_BF16 = 3e-2   # Newton-Schulz output with bf16 operands
TOL_O_F32 = 1e-4    # Newton-Schulz output in fp32
TOL_STATE = 1e-6    # fp32 momentum and AdamW state
# Largest error of one 256 x 256 block of the Newton-Schulz output, relative
# to the norm an average block of the reference has: a whole-matrix bound
# alone would let one wrong tile of a large matrix pass.
TOL_BLOCK_BF16 = 5e-2
TOL_BLOCK_F32 = 2e-4


def relF(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return num
    return num / den


def block_error(got, want, bs=256):
    """max over bs x bs blocks b of ||got_b - want_b||_F / (||want||_F *
    sqrt(|b| / |want|)): each block's error against the norm of an average
    block of the reference (blocks of a low-norm region are not held to a
    tighter bound than the rest)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    tot = np.linalg.norm(want)
    if tot == 0.0:
        return float(np.linalg.norm(got - want))
    worst = 0.0
    for i in range(0, want.shape[0], bs):
        for j in range(0, want.shape[1], bs):
            w = want[i:i + bs, j:j + bs]
            e = np.linalg.norm(got[i:i + bs, j:j + bs] - w)
            worst = max(worst, e / (tot * np.sqrt(w.size / want.size)))
    return worst


def check_output(got, want, tol, tol_block, what=""):
    """Whole-matrix and blockwise relative error of a Newton-Schulz output."""
    e = relF(got, want)
    eb = block_error(got, want)
    assert e <= tol, (what, "O", e, tol)
    assert eb <= tol_block, (what, "O block", eb, tol_block)
    return e, eb


def block_tol(tol_o):
    return TOL_BLOCK_F32 if tol_o <= TOL_O_F32 else TOL_BLOCK_BF16


def check_bf16_param(got, want, min_exact=0.97, what=""):
    """A bf16 parameter against the oracle's bf16 result: most elements equal
    bit for bit.  The rest differ where the kernels' fp32 step and the
    oracle's fp64 step (and the Newton-Schulz error) fall on opposite sides of
    a rounding boundary."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    exact = float(np.mean(got == want))
    assert exact >= min_exact, (what, "bf16 exact fraction", exact)
    return exact


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def w_tolerance(lr, s, O_ref, W_ref, tol_o):
    """Bound on the weight's relative error implied by the update's: the
    weight moves by lr*s*O, so an error tol_o*||O|| in O moves it by
    lr*s*tol_o*||O||; plus fp32 rounding of W itself."""
    return (lr * s * tol_o * np.linalg.norm(O_ref)) / max(np.linalg.norm(W_ref), 1e-30) + 2e-6


class Handle:
    _h = None

    @classmethod
    def get(cls):
        if cls._h is None:
            cls._h = mu.muon_init(0)
        return cls._h


def run_muon_step(mats, hp, stream=None, ws=None):
    """One batched step on the current stream; returns the workspace used."""
    h = Handle.get()
    need = mu.muon_workspace_size(h, mats, hp)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    mu.muon_step_batched(h, mats, hp, ws, stream)
    return ws


def hp_from(muon_hp, **over):
    d = dict(muon_hp)
    d.update(over)
    return mu.muon_hparams(lr=d["lr"], momentum=d["mu"], weight_decay=d["weight_decay"],
                           eps=d["eps"], extra_scale=d.get("extra_scale", 1.0),
                           nesterov=d["nesterov"], ns_steps=d["steps"], ns_dtype=d["ns_dtype"],
                           scale_mode=d["scale_mode"], coeffs=d.get("coeffs"))


def recipe_floor_output(Y, steps=5, eps=1e-7, coeffs=None):
    """The Newton-Schulz method as a plain bf16 implementation computes it:
    every tensor held in bf16, each product accumulated in fp32 and rounded,
    every elementwise result rounded ("About Muon: Why Not Adam", section
    "Making It Actually Run", in the bf16 that "The Optimizer Wars ...",
    section "What is Muon?" names).  The odd polynomial goes through the
    short-side Gram, q(X X^T) X for a wide X or X q(X^T X) for a tall one.
    On the CPU, on the NS input Y.  Its distance to the oracle is the error
    floor such an implementation has on this input; reported beside the
    kernels' error, never used as a reference."""
    def r(t):
        return t.to(torch.bfloat16).to(torch.float32)
    X = r(torch.from_numpy(np.ascontiguousarray(Y, dtype=np.float32)))
    X = r(X / (r(torch.linalg.norm(X)) + eps))
    wide = X.shape[0] <= X.shape[1]
    sched = ([tuple(c) for c in np.asarray(coeffs).reshape(-1, 3)] if coeffs is not None
             else [oracle.MUON_COEFFS] * steps)
    for a, b, c in sched:
        S = r(X @ X.T) if wide else r(X.T @ X)
        Q = r(r(b * S) + r(c * r(S @ S)))          # the polynomial's b and c terms
        QX = r(Q @ X) if wide else r(X @ Q)
        X = r(r(a * X) + QX)
    return X.double().numpy()


def oracle_kwargs(muon_hp, **over):
    d = dict(muon_hp)
    d.update(over)
    coeffs = d.get("coeffs")
    if coeffs is not None:
        coeffs = np.asarray(coeffs, dtype=np.float64).reshape(d["steps"], 3)
    return dict(lr=d["lr"], mu=d["mu"], weight_decay=d["weight_decay"], nesterov=d["nesterov"],
                eps=d["eps"], steps=d["steps"], coeffs=coeffs, scale_mode=d["scale_mode"],
                extra_scale=d.get("extra_scale", 1.0))


def compare_matrix(W0, G, M0, W1, M1, O_gpu, muon_hp, tol_o, report=None, name=""):
    """Oracle step for one matrix from the exact inputs; assert parity."""
    kw = oracle_kwargs(muon_hp)
    Wr, Mr, Or = oracle.muon_matrix_step(W0, G, M0, **kw)
    eo, _ = check_output(O_gpu, Or, tol_o, block_tol(tol_o), name)
    em = relF(M1, Mr)
    s = oracle.shape_scale(W0.shape[0], W0.shape[1], kw["scale_mode"]) * kw["extra_scale"]
    ew = relF(W1, Wr)
    tw = w_tolerance(kw["lr"], s, Or, Wr, tol_o)
    if report is not None:
        report.append((name, W0.shape, eo, em, ew, tw))
    assert em <= TOL_STATE, (name, "M", em)
    assert ew <= tw, (name, "W", ew, tw)
    return eo, em, ew

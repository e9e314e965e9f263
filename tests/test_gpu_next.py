"""GPU parity of the rows beyond the basic step: per-head (small) matrices in
the grouped launch, QK-Clip, coefficient schedules and global-norm gradient
clipping for AdamW.  All through the C ABI, against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import muon_step_02_amd as mu
from harness import (TOL_O_BF16, TOL_O_F32, TOL_STATE, Handle, f64, hp_from, oracle_kwargs, relF,
                     run_muon_step, w_tolerance)

pytestmark = pytest.mark.gpu
DEV = "cuda"

BASE_HP = dict(lr=2e-4, mu=0.95, weight_decay=0.1, nesterov=True, eps=1e-7, steps=5,
               scale_mode="moonlight", extra_scale=1.0, ns_dtype="bf16")


def _grad(rows, cols, seed, noise=0.3):
    g = torch.Generator(device=DEV).manual_seed(seed)
    r = min(8, rows, cols)
    U = torch.randn(rows, r, generator=g, device=DEV, dtype=torch.float64)
    V = torch.randn(r, cols, generator=g, device=DEV, dtype=torch.float64)
    s = 10.0 ** (-torch.arange(r, device=DEV, dtype=torch.float64) / 4)
    G = (U * s) @ V + noise * torch.randn(rows, cols, generator=g, device=DEV, dtype=torch.float64)
    return G.float()


def _weight(rows, cols, seed):
    g = torch.Generator(device=DEV).manual_seed(10_000 + seed)
    return torch.randn(rows, cols, generator=g, device=DEV) * 0.02


def test_per_head_blocks_with_large_matrices_in_one_call():
    # An MLA-style up-projection split per head (16 heads x 128 rows of a
    # 2048 x 1024 weight), an unsplit 512 x 1024 matrix, and a 64 x 2048 one:
    # the small class (short side <= 128) and the large class together.
    heads, dh, dm = 16, 128, 1024
    Wf, Gf, Mf = _weight(heads * dh, dm, 1), _grad(heads * dh, dm, 1), torch.zeros(heads * dh, dm, device=DEV)
    W2, G2, M2 = _weight(512, dm, 2), _grad(512, dm, 2), torch.zeros(512, dm, device=DEV)
    W3, G3, M3 = _weight(64, 2048, 3), _grad(64, 2048, 3), torch.zeros(64, 2048, device=DEV)
    W3t, G3t, M3t = _weight(2048, 96, 4), _grad(2048, 96, 4), torch.zeros(2048, 96, device=DEV)
    ins = [(f64(W), f64(G)) for W, G in ((Wf, Gf), (W2, G2), (W3, G3), (W3t, G3t))]
    mats, outs = [], []
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        O = torch.empty(dh, dm, device=DEV)
        outs.append(O)
        mats.append(mu.muon_matrix(Wf[sl], Gf[sl], Mf[sl], update_out=O))
    extra = []
    for W, G, M in ((W2, G2, M2), (W3, G3, M3), (W3t, G3t, M3t)):
        O = torch.empty_like(W)
        extra.append(O)
        mats.append(mu.muon_matrix(W, G, M, update_out=O))
    run_muon_step(mats, hp_from(BASE_HP))
    torch.cuda.synchronize()
    kw = oracle_kwargs(BASE_HP)
    W0, G0 = ins[0]
    Wg = f64(Wf)
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        Wr, Mr, Or = oracle.muon_matrix_step(W0[sl], G0[sl], np.zeros((dh, dm)), **kw)
        assert relF(f64(outs[h]), Or) <= TOL_O_BF16, h
        assert relF(f64(Mf[sl]), Mr) <= TOL_STATE
        assert relF(Wg[sl], Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(dh, dm), Or, Wr, TOL_O_BF16)
    for (W0, G0), W, M, O in zip(ins[1:], (W2, W3, W3t), (M2, M3, M3t), extra):
        Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), **kw)
        assert relF(f64(O), Or) <= TOL_O_BF16
        assert relF(f64(M), Mr) <= TOL_STATE
        assert relF(f64(W), Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(*W0.shape), Or, Wr,
                                               TOL_O_BF16)


@pytest.mark.parametrize("ns_dtype", ["bf16", "fp32"])
def test_qk_clip_after_update(ns_dtype):
    heads, dh, dm = 6, 64, 384
    tau = 100.0
    W, G, M = _weight(heads * dh, dm, 7), _grad(heads * dh, dm, 7), torch.zeros(heads * dh, dm, device=DEV)
    smax = torch.tensor([30.0, 100.0, 100.5, 400.0, 1e4, -5.0], device=DEV)
    W0, G0 = f64(W), f64(G)
    O = torch.empty_like(W)
    hpd = dict(BASE_HP, ns_dtype=ns_dtype, lr=0.02)
    hp = hp_from(hpd)
    hp.qk_tau = tau
    run_muon_step([mu.muon_matrix(W, G, M, update_out=O, qk_smax=smax, qk_block_rows=dh)], hp)
    torch.cuda.synchronize()
    kw = oracle_kwargs(hpd)
    Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), qk_smax=f64(smax),
                                         qk_block_rows=dh, qk_tau=tau, **kw)
    tol_o = TOL_O_F32 if ns_dtype == "fp32" else TOL_O_BF16
    assert relF(f64(O), Or) <= tol_o
    Wg = f64(W)
    for h in range(heads):
        sl = slice(h * dh, (h + 1) * dh)
        tw = w_tolerance(kw["lr"], oracle.shape_scale(heads * dh, dm), Or[sl], Wr[sl], tol_o)
        assert relF(Wg[sl], Wr[sl]) <= tw, h
    # the clipped heads really shrank: compare against the unclipped oracle
    Wu, _, _ = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), **kw)
    ratio = np.linalg.norm(Wg[3 * dh:4 * dh]) / np.linalg.norm(Wu[3 * dh:4 * dh])
    assert abs(ratio - 0.5) < 1e-4


def test_coefficient_schedule_reaches_polar_factor_fp32():
    # textbook quintic (15/8, -10/8, 3/8) iterated 25 times converges to U V^T
    rows, cols = 256, 384
    W, G, M = _weight(rows, cols, 9), _grad(rows, cols, 9, noise=1.0), torch.zeros(rows, cols, device=DEV)
    W0, G0 = f64(W), f64(G)
    O = torch.empty_like(W)
    steps = 25
    coeffs = [1.875, -1.25, 0.375] * steps
    hpd = dict(BASE_HP, ns_dtype="fp32", steps=steps, coeffs=coeffs)
    run_muon_step([mu.muon_matrix(W, G, M, update_out=O)], hp_from(hpd))
    torch.cuda.synchronize()
    Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), **oracle_kwargs(hpd))
    assert relF(f64(O), Or) <= TOL_O_F32
    Y = oracle.nesterov_blend(G0, oracle.momentum_update(np.zeros_like(G0), G0, 0.95), 0.95)
    U, _, Vt = np.linalg.svd(Y, full_matrices=False)
    assert relF(f64(O), U @ Vt) <= 1e-4


def test_three_step_schedule_and_per_iteration_coefficients_bf16():
    rows, cols = 512, 768
    W, G, M = _weight(rows, cols, 11), _grad(rows, cols, 11), torch.zeros(rows, cols, device=DEV)
    W0, G0 = f64(W), f64(G)
    O = torch.empty_like(W)
    coeffs = [3.4445, -4.7750, 2.0315, 2.5, -3.0, 1.2, 1.875, -1.25, 0.375]
    hpd = dict(BASE_HP, steps=3, coeffs=coeffs)
    run_muon_step([mu.muon_matrix(W, G, M, update_out=O)], hp_from(hpd))
    torch.cuda.synchronize()
    Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), **oracle_kwargs(hpd))
    assert relF(f64(O), Or) <= TOL_O_BF16


ADAMW_HP = dict(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@pytest.mark.parametrize("scale,gdt", [(1.0, torch.float32), (1e-4, torch.float32),
                                       (1.0, torch.bfloat16)])
def test_adamw_global_norm_clipping(scale, gdt):
    h = Handle.get()
    g = torch.Generator(device=DEV).manual_seed(21)
    sizes = [3, 4096, 70000, 1024 * 1024 + 5] + [999] * 35
    P = [torch.randn(n, generator=g, device=DEV) * 0.02 for n in sizes]
    Ms = [torch.zeros(n, device=DEV) for n in sizes]
    Vs = [torch.zeros(n, device=DEV) for n in sizes]
    ref = [[f64(p), np.zeros(n), np.zeros(n)] for p, n in zip(P, sizes)]
    norm_out = torch.zeros(1, device=DEV)
    ws = None
    for t in range(1, 4):
        grads = [(torch.randn(n, generator=g, device=DEV) * scale).to(gdt) for n in sizes]
        ts = [mu.adamw_tensor(p, gr, m, v) for p, gr, m, v in zip(P, grads, Ms, Vs)]
        if ws is None:
            # all-ones bytes: every partial sum must be written before it is read
            ws = torch.full((mu.adamw_workspace_size(h, ts),), 255, dtype=torch.uint8, device=DEV)
        mu.adamw_step_clipped(h, ts, mu.adamw_hparams(step=t, **ADAMW_HP), 1.0, ws, norm_out)
        torch.cuda.synchronize()
        G64 = [f64(gr) for gr in grads]
        clipped, norm = oracle.clip_by_global_norm(G64, 1.0)
        assert abs(norm_out.item() - norm) <= 1e-5 * norm
        for i in range(len(sizes)):
            ref[i] = list(oracle.adamw_tensor_step(ref[i][0], clipped[i], ref[i][1], ref[i][2],
                                                   step=t, **ADAMW_HP))
    for i in range(len(sizes)):
        assert relF(f64(P[i]), ref[i][0]) <= TOL_STATE, i
        assert relF(f64(Ms[i]), ref[i][1]) <= TOL_STATE, i
        assert relF(f64(Vs[i]), ref[i][2]) <= TOL_STATE, i


def test_adamw_clipping_below_threshold_equals_plain_step():
    h = Handle.get()
    g = torch.Generator(device=DEV).manual_seed(5)
    sizes = [5000, 12345]
    A = [torch.randn(n, generator=g, device=DEV) for n in sizes]
    grads = [torch.randn(n, generator=g, device=DEV) * 1e-4 for n in sizes]
    B = [a.clone() for a in A]
    st = {k: [torch.zeros(n, device=DEV) for n in sizes] for k in ("ma", "va", "mb", "vb")}
    hp = mu.adamw_hparams(step=1, **ADAMW_HP)
    ta = [mu.adamw_tensor(a, gr, m, v) for a, gr, m, v in zip(A, grads, st["ma"], st["va"])]
    tb = [mu.adamw_tensor(b, gr, m, v) for b, gr, m, v in zip(B, grads, st["mb"], st["vb"])]
    ws = torch.empty(mu.adamw_workspace_size(h, tb), dtype=torch.uint8, device=DEV)
    mu.adamw_step(h, ta, hp)
    mu.adamw_step_clipped(h, tb, hp, 1.0, ws)
    torch.cuda.synchronize()
    for a, b in zip(A, B):
        assert torch.equal(a, b)
    with pytest.raises(mu.MuonError):
        mu.adamw_step_clipped(h, tb, hp, 0.0, ws)
    with pytest.raises(mu.MuonError):
        mu.adamw_step_clipped(h, tb, hp, 1.0, ws[:8])

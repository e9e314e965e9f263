"""GPU parity of libmuon's kernels against the fp64 oracle (through the C ABI).

Marked ``gpu``: needs an MI355X and the built library.  Each GEMM phase is
checked against its plain definition in fp64 on the same bf16 inputs; whole
steps against ``oracle.muon_matrix_step`` / ``oracle.adamw_tensor_step``.
"""

import numpy as np
import pytest
import torch

import oracle
import muon_step_02_amd as mu
from harness import (TOL_BLOCK_BF16, TOL_O_BF16, TOL_O_F32, TOL_STATE, Handle, block_tol,
                     check_bf16_param, check_output, compare_matrix, f64, hp_from, oracle_kwargs,
                     relF, run_muon_step)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


def _sym_bf16(m, seed, scale):
    a = _bf16((m, m), seed, scale).float()
    return ((a + a.T) * 0.5).to(torch.bfloat16)


# ------------------------------------------------------------ GEMM phases --

@pytest.mark.parametrize("m,n", [(256, 256), (512, 768), (768, 1280)])
@pytest.mark.parametrize("s2", [1.0, 0.25])
def test_gram_phase(m, n, s2):
    h = Handle.get()
    X = _bf16((m, n), 1 + m + n, 1.0 / np.sqrt(n))
    A = torch.full((m, m), float("nan"), dtype=torch.bfloat16, device=DEV)
    mu.muon_test_gram_bf16(h, X, A, m, n, n, m, s2)
    torch.cuda.synchronize()
    X64 = f64(X)
    want = s2 * (X64 @ X64.T)
    got = f64(A)
    assert np.isfinite(got).all()
    assert relF(got, want) < 4e-3
    assert np.array_equal(got, got.T)  # mirrored triangle


@pytest.mark.parametrize("m", [256, 512, 1024])
def test_poly_phase(m):
    h = Handle.get()
    A = _sym_bf16(m, 7 + m, 1.0 / np.sqrt(m))
    B = torch.full((m, m), float("nan"), dtype=torch.bfloat16, device=DEV)
    a, b, c = 3.4445, -4.7750, 2.0315
    mu.muon_test_poly_bf16(h, A, B, m, m, a, b, c)
    torch.cuda.synchronize()
    A64 = f64(A)
    # the quintic's identity term sits on the diagonal: B X = a X + b A X + c A A X
    want = a * np.eye(m) + b * A64 + c * (A64 @ A64)
    got = f64(B)
    assert np.isfinite(got).all()
    assert relF(got, want) < 4e-3
    assert relF(np.diag(got), np.diag(want)) < 4e-3
    off = ~np.eye(m, dtype=bool)
    assert relF(got[off], want[off]) < 4e-3
    assert np.array_equal(got, got.T)


@pytest.mark.parametrize("m,n,ldx", [(256, 256, 256), (256, 768, 768), (512, 1024, 1024),
                                      (256, 512, 768)])
@pytest.mark.parametrize("s", [1.0, 0.5])
def test_update_phase(m, n, ldx, s):
    # X is read k-major (rows of X are the update's k); ldx > n checks that
    # the columns beyond n are neither read into the product nor written
    h = Handle.get()
    Xfull = _bf16((m, ldx), 3 + m, 1.0 / np.sqrt(n))
    X = Xfull[:, :n]
    B = _sym_bf16(m, 5 + n, 1.0 / np.sqrt(m))
    Xo = torch.full((m, ldx), float("nan"), dtype=torch.bfloat16, device=DEV)
    mu.muon_test_update_bf16(h, Xfull, B, Xo, m, n, ldx, m, s)
    torch.cuda.synchronize()
    X64, B64 = f64(X), f64(B)
    want = s * (B64 @ X64)
    got = f64(Xo[:, :n])
    assert np.isfinite(got).all()
    assert relF(got, want) < 4e-3
    assert np.isnan(f64(Xo[:, n:])).all()


# ------------------------------------------------------------ whole steps --

def _rand_matrix_inputs(rows, cols, seed, pdt=torch.float32, gdt=torch.float32, lowrank=True,
                        noise=0.3):
    # Eight decaying spikes over a Gaussian bulk whose normalised singular
    # values sit near 1e-2: ill-conditioned, yet above bf16 resolution.  (With
    # the bulk near 5e-4 the bf16 iteration itself is off by ~0.19, kernels or
    # not: small singular values are amplified up to p'(0)^5 ~ 485 times.)
    g = torch.Generator(device=DEV).manual_seed(seed)
    W = (torch.randn(rows, cols, generator=g, device=DEV) * 0.02).to(pdt)
    if lowrank:
        r = min(8, rows, cols)
        U = torch.randn(rows, r, generator=g, device=DEV, dtype=torch.float64)
        V = torch.randn(r, cols, generator=g, device=DEV, dtype=torch.float64)
        s = 10.0 ** (-torch.arange(r, device=DEV, dtype=torch.float64) / 4)
        G = (U * s) @ V + noise * torch.randn(rows, cols, generator=g, device=DEV, dtype=torch.float64)
        G = G.to(gdt)
    else:
        G = torch.randn(rows, cols, generator=g, device=DEV).to(gdt)
    M = torch.randn(rows, cols, generator=g, device=DEV) * 0.1
    return W, G, M


# (64, 300): short side <= 128 with a padded width of 384, not a multiple of 256,
# so its elementwise tiles go through LDS without a transpose; (1030, 513): a
# tall matrix whose rows are not 16-byte aligned (scalar path of the
# transposing tiles).
MIXED = [(256, 256), (300, 500), (500, 300), (1, 1), (1, 37), (37, 1), (7, 13), (1024, 256),
         (256, 1024), (513, 1030), (64, 64), (64, 300), (300, 64), (1030, 513)]

BASE_HP = dict(lr=2e-4, mu=0.95, weight_decay=0.1, nesterov=True, eps=1e-7, steps=5,
               scale_mode="moonlight", extra_scale=1.0, ns_dtype="bf16")


def _run_and_compare(shapes, hpd, tol_o, pdt=torch.float32, gdt=torch.float32, seed=0,
                     lowrank=True, tol_for=None):
    # tol_for(k, W0, G0, M0), if given, sets matrix k's output tolerance
    ins, mats, outs = [], [], []
    for k, (r, c) in enumerate(shapes):
        W, G, M = _rand_matrix_inputs(r, c, seed * 1000 + k, pdt, gdt, lowrank)
        ins.append((f64(W), f64(G), f64(M)))
        O = torch.full((r, c), float("nan"), device=DEV)
        nrm = torch.zeros(1, device=DEV)
        mats.append(mu.muon_matrix(W, G, M, update_out=O, norm_out=nrm))
        outs.append((W, M, O, nrm, G))  # G must outlive the call: the descriptor holds its address
    run_muon_step(mats, hp_from(hpd))
    torch.cuda.synchronize()
    report = []
    for k, ((W0, G0, M0), (W, M, O, nrm, _)) in enumerate(zip(ins, outs)):
        tol_k = tol_o if tol_for is None else tol_for(k, W0, G0, M0)
        if pdt == torch.bfloat16:
            # bf16 weights: the stored result is the step rounded once to bf16
            Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, M0, param_dtype="bf16", **_okw(hpd))
            check_output(f64(O), Or, tol_k, block_tol(tol_k), shapes[k])
            assert relF(f64(M), Mr) <= TOL_STATE
            check_bf16_param(f64(W), Wr, what=shapes[k])
            assert relF(f64(W), Wr) <= 5e-4
        else:
            compare_matrix(W0, G0, M0, f64(W), f64(M), f64(O), hpd, tol_k, report, str(shapes[k]))
        Mr = oracle.momentum_update(M0, G0, hpd["mu"])
        Yr = oracle.nesterov_blend(G0, Mr, hpd["mu"], hpd["nesterov"])
        assert abs(float(nrm.item()) - np.linalg.norm(Yr)) <= 1e-5 * np.linalg.norm(Yr) + 1e-30
    return report


def _okw(d):
    from harness import oracle_kwargs
    return oracle_kwargs(d)


@pytest.mark.parametrize("shape", MIXED)
def test_step_single_matrix_bf16(shape):
    _run_and_compare([shape], BASE_HP, TOL_O_BF16, seed=hash(shape) % 1000)


@pytest.mark.parametrize("shape", MIXED)
def test_step_single_matrix_f32(shape):
    _run_and_compare([shape], dict(BASE_HP, ns_dtype="fp32"), TOL_O_F32, seed=7)


def test_fp32_iteration_on_larger_matrices():
    # the fp32 iteration on the matrix cores: hundreds of triangle tiles with
    # mirrored stores, K up to 2048, both orientations, at the fp32 bound
    _run_and_compare([(1536, 2048), (2048, 1536), (704, 1984)], dict(BASE_HP, ns_dtype="fp32"),
                     TOL_O_F32, seed=19)


@pytest.mark.parametrize("shapes", [[(100, 150)], [(150, 100), (128, 192)], [(192, 130), (64, 200)]],
                         ids=["K 128 and 192", "K 128 and 192, two matrices", "K 192 and 256"])
def test_fp32_iteration_short_k(shapes):
    # launches whose K is at most 256 split each 64-tile into four 32 x 32
    # workgroups that divide K over their waves: K of 2, 3 and 4 slab pairs
    _run_and_compare(shapes, dict(BASE_HP, ns_dtype="fp32"), TOL_O_F32, seed=23)


def test_step_mixed_batch_bf16():
    _run_and_compare(MIXED, BASE_HP, TOL_O_BF16, seed=11)


def test_step_mixed_batch_f32():
    _run_and_compare(MIXED, dict(BASE_HP, ns_dtype="fp32"), TOL_O_F32, seed=12)


@pytest.mark.parametrize("shapes", [
    [(128, 7168)] * 3,                                   # small class, 3 tiles: 16 parts each
    [(1024, 4096), (1024, 1024), (4096, 1024)],          # large class, unequal K
    [(256, 20000), (100, 3000), (129, 129), (7, 9)],     # both classes split, plus fp32 tiny
    [(512, 65536)],                                      # one long matrix: 3 tiles x 16 parts
])
def test_k_split_gram_launches(shapes):
    # Gram launches with fewer tiles than compute units run K-split (fp32
    # partial tiles, then a reduce launch that sums them in part order,
    # scales, rounds and mirrors); outputs against the oracle as usual, and
    # the whole step is bitwise repeatable
    _run_and_compare(shapes, BASE_HP, TOL_O_BF16, seed=77)
    res = []
    for _ in range(2):
        W, G, M = _rand_matrix_inputs(*shapes[0], 5)
        O = torch.empty_like(W)
        run_muon_step([mu.muon_matrix(W, G, M, update_out=O)], hp_from(BASE_HP))
        torch.cuda.synchronize()
        res.append(O.clone())
    assert torch.equal(res[0], res[1])


@pytest.mark.parametrize("ns_dtype", ["bf16", "fp32"])
def test_strided_views_leave_the_rest_untouched(ns_dtype):
    # Column slices of wider buffers: param, grad and momentum each with its
    # own leading dimension, some of them odd (rows not 16-byte aligned), one
    # gradient in bf16.  Columns beyond the view hold a sentinel that must
    # survive the step.
    cases = [((300, 500), (512, 700, 600), torch.float32),
             ((500, 300), (301, 333, 450), torch.float32),
             ((64, 300), (303, 300, 320), torch.bfloat16),
             ((1030, 513), (600, 515, 513), torch.float32)]
    hpd = dict(BASE_HP, ns_dtype=ns_dtype)
    mats, keep = [], []
    for k, ((r, c), (lw, lg, lm), gdt) in enumerate(cases):
        W, G, M = _rand_matrix_inputs(r, c, 700 + k, gdt=gdt)
        bufs = [torch.full((r, ld), 7.0, dtype=t.dtype, device=DEV) for t, ld in
                ((W, lw), (G, lg), (M, lm))]
        views = [b[:, :c] for b in bufs]
        for v, t in zip(views, (W, G, M)):
            v.copy_(t)
        O = torch.empty(r, c, device=DEV)
        mats.append(mu.muon_matrix(*views, update_out=O))
        keep.append((tuple(f64(t) for t in (W, G, M)), bufs, views, O))
    run_muon_step(mats, hp_from(hpd))
    torch.cuda.synchronize()
    tol = TOL_O_BF16 if ns_dtype == "bf16" else TOL_O_F32
    for ((W0, G0, M0), bufs, (W, G, M), O), ((r, c), _, _) in zip(keep, cases):
        compare_matrix(W0, G0, M0, f64(W), f64(M), f64(O), hpd, tol)
        assert np.array_equal(f64(G), G0)
        for b in bufs:
            assert bool((b[:, c:] == 7.0).all())


@pytest.mark.parametrize("ns_dtype", ["bf16", "fp32"])
def test_small_and_large_class_boundary(ns_dtype):
    # short side 128 is the last of the 128-tile class, 129 the first of the
    # 256-tile class; both orientations, one call
    shapes = [(128, 700), (129, 700), (700, 128), (700, 129), (128, 128), (129, 129), (256, 129)]
    tol = TOL_O_BF16 if ns_dtype == "bf16" else TOL_O_F32
    _run_and_compare(shapes, dict(BASE_HP, ns_dtype=ns_dtype), tol, seed=31)


@pytest.mark.parametrize("ns_dtype,steps", [("bf16", 2), ("bf16", 4), ("fp32", 6)])
def test_even_iteration_counts(ns_dtype, steps):
    # after an even number of iterations the result sits in the other
    # ping-pong buffer than after an odd one; apply must read that one
    shapes = [(300, 500), (500, 300), (64, 300), (300, 64), (1030, 513)]
    tol = TOL_O_BF16 if ns_dtype == "bf16" else TOL_O_F32
    _run_and_compare(shapes, dict(BASE_HP, ns_dtype=ns_dtype, steps=steps), tol, seed=21 + steps)


@pytest.mark.parametrize("ns_dtype,count", [("bf16", 2500), ("fp32", 600)])
def test_step_thousands_of_tiny_matrices_in_one_call(ns_dtype, count):
    # Ragged matrices of at most 48 x 48 beside two large ones: the descriptor
    # table goes up in hundreds of chunks, the tile prefix search runs over
    # thousands of entries, and almost every matrix is one tile.  With the
    # bf16 iteration the matrices whose short side is at most 32 run the fp32
    # iteration in the same call (a bf16 iteration on that few singular values
    # misses 3e-2 on some inputs); every matrix is held to the plain bound.
    rng = np.random.default_rng(2024)
    shapes = [tuple(int(v) for v in rng.integers(1, 49, size=2)) for _ in range(count)]
    shapes[count // 2:count // 2] = [(300, 500)]
    shapes.append((1030, 513))
    hpd = dict(BASE_HP, ns_dtype=ns_dtype)
    _run_and_compare(shapes, hpd, TOL_O_F32 if ns_dtype == "fp32" else TOL_O_BF16, seed=13)


@pytest.mark.parametrize("short", [31, 32, 33, 48])
def test_tiny_class_boundary_bf16(short):
    # short side 32 is the last that runs in fp32 under a bf16 call, 33 the
    # first on bf16 operands (128-wide tiles); both orientations, long sides
    # from square to 40 times longer
    shapes = [(short, short), (short, 7 * short + 3), (40 * short, short), (short, 1000)]
    _run_and_compare(shapes, BASE_HP, TOL_O_BF16, seed=300 + short)


@pytest.mark.parametrize("mode", ["moonlight", "jordan", "bernstein", "none"])
def test_scale_modes_and_extra_scale(mode):
    _run_and_compare([(300, 700), (700, 300)], dict(BASE_HP, scale_mode=mode, extra_scale=1.5,
                                                    lr=0.02, weight_decay=0.01), TOL_O_BF16, seed=3)


def test_no_nesterov_and_other_coefficients():
    coeffs = [1.875, -1.25, 0.375] * 3
    _run_and_compare([(256, 512), (512, 256)],
                     dict(BASE_HP, nesterov=False, steps=3, coeffs=coeffs), TOL_O_BF16, seed=4)
    _run_and_compare([(256, 512)], dict(BASE_HP, steps=1), TOL_O_BF16, seed=5)


def test_bf16_grad_and_bf16_param():
    _run_and_compare([(256, 384), (384, 256)], BASE_HP, TOL_O_BF16, gdt=torch.bfloat16, seed=6)
    _run_and_compare([(256, 384), (384, 256)], BASE_HP, TOL_O_BF16, pdt=torch.bfloat16,
                     gdt=torch.bfloat16, seed=8)
    # rows not 16-byte aligned (scalar paths), the small class, both orientations
    ragged = [(37, 1), (7, 13), (1030, 513), (513, 1030), (64, 300), (300, 64)]
    _run_and_compare(ragged, BASE_HP, TOL_O_BF16, pdt=torch.bfloat16, gdt=torch.bfloat16, seed=9)
    _run_and_compare(ragged, dict(BASE_HP, ns_dtype="fp32"), TOL_O_F32, gdt=torch.bfloat16,
                     seed=10)


def test_bf16_param_large_step_moves_by_the_oracle_update():
    # At lr 0.02 a step moves a bf16 weight by far more than its rounding
    # (about 20% of an entry here), so the weight's change itself is checked:
    # ||(W1 - W0) - (Wr - W0)|| may hold the Newton-Schulz error (3e-2 of the
    # update) plus the bf16 rounding of W1 (half a unit in the last place of
    # each entry, 2^-9 relative), nothing more.  A kernel that skipped or
    # mis-signed the update, or stored W unrounded, fails by 50-200%.
    hpd = dict(BASE_HP, lr=0.02, weight_decay=0.01)
    shapes = [(256, 384), (384, 256), (1030, 513), (64, 300), (37, 1)]
    ins, mats, outs = [], [], []
    for k, (r, c) in enumerate(shapes):
        W, G, M = _rand_matrix_inputs(r, c, 4100 + k, torch.bfloat16, torch.bfloat16)
        ins.append((f64(W), f64(G), f64(M)))
        O = torch.empty(r, c, device=DEV)
        mats.append(mu.muon_matrix(W, G, M, update_out=O))
        outs.append((W, M, O, G))
    run_muon_step(mats, hp_from(hpd))
    torch.cuda.synchronize()
    for (W0, G0, M0), (W, M, O, _), shape in zip(ins, outs, shapes):
        Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, M0, param_dtype="bf16", **_okw(hpd))
        Wfull, _, _ = oracle.muon_matrix_step(W0, G0, M0, **_okw(hpd))
        check_output(f64(O), Or, TOL_O_BF16, TOL_BLOCK_BF16, shape)
        dW = Wfull - W0
        err = np.linalg.norm(f64(W) - Wfull) / np.linalg.norm(dW)
        bound = TOL_O_BF16 + 2.0 ** -9 * np.linalg.norm(Wfull) / np.linalg.norm(dW)
        assert err <= bound, (shape, err, bound)
        assert np.linalg.norm(dW) > 10 * 2.0 ** -9 * np.linalg.norm(Wfull)  # the step is resolved
        check_bf16_param(f64(W), Wr, min_exact=0.4, what=shape)


def test_resume_from_saved_state_is_bitwise():
    # The optimizer state is the caller's momentum buffer (and the weights):
    # three steps in a row equal two steps, a save of W and M to host memory,
    # a restore into fresh tensors, and a third step, bit for bit.
    shapes = [(512, 384), (384, 1024), (64, 300), (20, 9)]
    hp = hp_from(BASE_HP)
    grads = [[_rand_matrix_inputs(r, c, 900 + 10 * t + k)[1] for k, (r, c) in enumerate(shapes)]
             for t in range(3)]

    def fresh():
        return [(_rand_matrix_inputs(r, c, 800 + k)[0], torch.zeros(r, c, device=DEV))
                for k, (r, c) in enumerate(shapes)]

    def step(state, t):
        run_muon_step([mu.muon_matrix(W, G, M) for (W, M), G in zip(state, grads[t])], hp)

    straight = fresh()
    for t in range(3):
        step(straight, t)
    resumed = fresh()
    for t in range(2):
        step(resumed, t)
    torch.cuda.synchronize()
    saved = [(W.cpu().clone(), M.cpu().clone()) for W, M in resumed]
    del resumed
    restored = [(W.to(DEV), M.to(DEV)) for W, M in saved]
    step(restored, 2)
    torch.cuda.synchronize()
    for (W1, M1), (W2, M2) in zip(straight, restored):
        assert torch.equal(W1, W2) and torch.equal(M1, M2)


@pytest.mark.parametrize("ns_dtype", ["bf16", "fp32"])
def test_non_finite_gradient_propagates_to_its_matrix_only(ns_dtype):
    # IEEE semantics, no checks: a NaN or Inf in one matrix's gradient reaches
    # that matrix's momentum element and, through the norm, its whole update
    # and weight; every other matrix of the batch is bit-identical to a batch
    # without the bad one.
    hpd = dict(BASE_HP, ns_dtype=ns_dtype)
    hp = hp_from(hpd)
    shapes = [(300, 500), (256, 1024), (40, 40), (1030, 513)]
    for bad, val in ((1, float("nan")), (2, float("inf"))):
        runs = []
        for poison in (False, True):
            ts = [_rand_matrix_inputs(r, c, 600 + k) for k, (r, c) in enumerate(shapes)]
            if poison:
                ts[bad][1][3, 5] = val
            Os = [torch.empty(r, c, device=DEV) for r, c in shapes]
            run_muon_step([mu.muon_matrix(W, G, M, update_out=O) for (W, G, M), O in zip(ts, Os)], hp)
            torch.cuda.synchronize()
            runs.append((ts, Os))
        (clean, Oc), (dirty, Od) = runs
        for k in range(len(shapes)):
            if k == bad:
                assert not torch.isfinite(dirty[k][2][3, 5])
                assert torch.isfinite(dirty[k][2]).sum() == dirty[k][2].numel() - 1
                assert torch.isnan(Od[k]).all() and torch.isnan(dirty[k][0]).all()
            else:
                assert torch.equal(Oc[k], Od[k])
                assert torch.equal(clean[k][0], dirty[k][0]) and torch.equal(clean[k][2], dirty[k][2])


def test_row_blocks_of_fused_tensor():
    # Q, K, V row blocks of one fused (3d x d) weight, as separate matrices
    d = 256
    W, G, M = _rand_matrix_inputs(3 * d, d, 21)
    W0, G0, M0 = f64(W), f64(G), f64(M)
    mats, Os = [], []
    for j in range(3):
        O = torch.empty(d, d, device=DEV)
        Os.append(O)
        sl = slice(j * d, (j + 1) * d)
        mats.append(mu.muon_matrix(W[sl], G[sl], M[sl], update_out=O))
    run_muon_step(mats, hp_from(BASE_HP))
    torch.cuda.synchronize()
    Wg, Mg = f64(W), f64(M)
    for j in range(3):
        sl = slice(j * d, (j + 1) * d)
        compare_matrix(W0[sl], G0[sl], M0[sl], Wg[sl], Mg[sl], f64(Os[j]), BASE_HP, TOL_O_BF16)


def test_zero_gradient_is_pure_decay():
    W, _, _ = _rand_matrix_inputs(300, 200, 9)
    G = torch.zeros_like(W)
    M = torch.zeros_like(W)
    O = torch.full_like(W, float("nan"))
    W0 = W.clone()
    hpd = dict(BASE_HP, lr=0.02, weight_decay=0.01)
    run_muon_step([mu.muon_matrix(W, G, M, update_out=O)], hp_from(hpd))
    torch.cuda.synchronize()
    assert torch.all(O == 0) and torch.all(M == 0)
    assert torch.allclose(W, W0 * (1 - 0.02 * 0.01), rtol=1e-7, atol=0)


def test_repeatable_bitwise():
    res = []
    for _ in range(2):
        W, G, M = _rand_matrix_inputs(768, 512, 31)
        O = torch.empty_like(W)
        run_muon_step([mu.muon_matrix(W, G, M, update_out=O)], hp_from(BASE_HP))
        torch.cuda.synchronize()
        res.append((W.clone(), M.clone(), O.clone()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("ns_dtype", ["bf16", "fp32"])
def test_workspace_garbage_and_reuse_across_batches(ns_dtype):
    # The workspace starts as all-ones bytes (NaN in every float view) and
    # serves two differently shaped batches in a row.  The second batch must
    # match, bit for bit, the same batch run on a fresh zeroed workspace: no
    # kernel may read workspace memory that this call did not write first
    # (padding, partial sums, tables).
    h = Handle.get()
    hp = hp_from(dict(BASE_HP, ns_dtype=ns_dtype))
    shapes_a = [(300, 500), (64, 300), (1030, 513)]
    shapes_b = [(500, 300), (37, 1), (256, 1024), (300, 64)]

    def batch(shapes, seed):
        ts = [_rand_matrix_inputs(r, c, seed + k) for k, (r, c) in enumerate(shapes)]
        outs = [torch.empty_like(W) for W, _, _ in ts]
        mats = [mu.muon_matrix(W, G, M, update_out=O) for (W, G, M), O in zip(ts, outs)]
        return ts, outs, mats

    ta, oa, ma = batch(shapes_a, 500)
    tb, ob, mb = batch(shapes_b, 600)
    tb0 = [tuple(t.clone() for t in x) for x in tb]
    need = max(mu.muon_workspace_size(h, ma, hp), mu.muon_workspace_size(h, mb, hp))
    ws = torch.full((need,), 255, dtype=torch.uint8, device=DEV)
    run_muon_step(ma, hp, ws=ws)
    run_muon_step(mb, hp, ws=ws)
    torch.cuda.synchronize()

    tc = [tuple(t.clone() for t in x) for x in tb0]
    oc = [torch.empty_like(W) for W, _, _ in tc]
    mc = [mu.muon_matrix(W, G, M, update_out=O) for (W, G, M), O in zip(tc, oc)]
    run_muon_step(mc, hp, ws=torch.zeros(need, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    tol = TOL_O_BF16 if ns_dtype == "bf16" else TOL_O_F32
    for k in range(len(shapes_b)):
        assert torch.equal(ob[k], oc[k]) and torch.equal(tb[k][0], tc[k][0])
        assert torch.equal(tb[k][2], tc[k][2])
        W0, G0, M0 = (f64(t) for t in tb0[k])
        compare_matrix(W0, G0, M0, f64(tb[k][0]), f64(tb[k][2]), f64(ob[k]),
                       dict(BASE_HP, ns_dtype=ns_dtype), tol)


def test_consecutive_steps_carry_momentum():
    W, _, M = _rand_matrix_inputs(512, 256, 41)
    M.zero_()
    Wn, Mn = f64(W), f64(M)
    wtol = 0.0
    for step in range(3):
        _, G, _ = _rand_matrix_inputs(512, 256, 100 + step)
        O = torch.empty_like(W)
        run_muon_step([mu.muon_matrix(W, G, M, update_out=O)], hp_from(BASE_HP))
        torch.cuda.synchronize()
        Wn, Mn, On = oracle.muon_matrix_step(Wn, f64(G), Mn, **_okw(BASE_HP))
        assert relF(f64(O), On) <= TOL_O_BF16
        assert relF(f64(M), Mn) <= TOL_STATE
        # each step may move W by lr*s*TOL_O_BF16*||O|| more than the oracle does
        wtol += 2e-4 * oracle.shape_scale(512, 256) * TOL_O_BF16 * np.linalg.norm(On) / np.linalg.norm(Wn)
    assert relF(f64(W), Wn) <= wtol + 2e-6


def test_two_streams_run_independent_steps():
    # Two batches with their own workspaces, stepped three times on two
    # streams at once, end bit-identical to the same steps run one after the
    # other: the kernels share no device state beyond the caller's buffers.
    h = Handle.get()
    hp = hp_from(BASE_HP)
    shapes = {"a": [(512, 384), (384, 512), (64, 300)], "b": [(256, 1024), (1030, 513), (100, 100)]}

    def batch(name, seed):
        st = [_rand_matrix_inputs(r, c, seed + k) for k, (r, c) in enumerate(shapes[name])]
        mats = [mu.muon_matrix(W, G, M) for W, G, M in st]
        ws = torch.empty(mu.muon_workspace_size(h, mats, hp), dtype=torch.uint8, device=DEV)
        return st, mats, ws

    seq = {k: batch(k, 50 + i * 10) for i, k in enumerate("ab")}
    par = {k: batch(k, 50 + i * 10) for i, k in enumerate("ab")}
    cur = torch.cuda.current_stream()
    for _ in range(3):
        for k in "ab":
            mu.muon_step_batched(h, seq[k][1], hp, seq[k][2], cur)
    streams = {k: torch.cuda.Stream() for k in "ab"}
    for s in streams.values():
        s.wait_stream(cur)
    for _ in range(3):
        for k in "ab":
            mu.muon_step_batched(h, par[k][1], hp, par[k][2], streams[k])
    torch.cuda.synchronize()
    for k in "ab":
        for (W1, _, M1), (W2, _, M2) in zip(seq[k][0], par[k][0]):
            assert torch.equal(W1, W2) and torch.equal(M1, M2)


# -------------------------------------------------------------- validation --

def _status(fn):
    try:
        fn()
    except mu.MuonError as e:
        return e.status
    return 0


def test_largest_dimension():
    # the longest side the ABI accepts (2^20), as a row and as a column: one
    # 128-wide Gram tile with K = 2^20, and 8192 update tiles
    _run_and_compare([(1, 1 << 20), (1 << 20, 1)], BASE_HP, TOL_O_BF16, seed=9)
    h = Handle.get()
    W, G, M = (torch.zeros(1, (1 << 20) + 1, device=DEV) for _ in range(3))
    with pytest.raises(mu.MuonError) as e:
        mu.muon_workspace_size(h, [mu.muon_matrix(W, G, M)], hp_from(BASE_HP))
    assert e.value.status == 1


def test_abi_validation_rejects_and_enqueues_nothing():
    h = Handle.get()
    W, G, M = _rand_matrix_inputs(256, 256, 1)
    W0 = W.clone()
    hp = hp_from(BASE_HP)
    good = mu.muon_matrix(W, G, M)
    ws = torch.empty(mu.muon_workspace_size(h, [good], hp), dtype=torch.uint8, device=DEV)

    def step(m, hpx=hp, w=ws):
        return _status(lambda: mu.muon_step_batched(h, [m], hpx, w))

    bad = mu.muon_matrix(W, G, M); bad.rows = 0
    assert step(bad) == 1
    bad = mu.muon_matrix(W, G, M); bad.ld_grad = 100
    assert step(bad) == 1
    bad = mu.muon_matrix(W, G, M); bad.grad = None
    assert step(bad) == 1
    bad = mu.muon_matrix(W, G, M); bad.param_dtype = 7
    assert step(bad) == 1
    bad = mu.muon_matrix(W, W, M)
    assert step(bad) == 4
    bad = mu.muon_matrix(W, G, M); bad.param = W.data_ptr() + 2
    assert step(bad) == 6
    assert step(good, hp, ws[: ws.numel() - 256]) == 3
    for field, val in (("ns_steps", 0), ("ns_dtype", 5), ("scale_mode", 9), ("nesterov", 2)):
        hpx = hp_from(BASE_HP)
        setattr(hpx, field, val)
        assert step(good, hpx) == 1
    hpx = hp_from(BASE_HP); hpx.lr = float("nan")
    assert step(good, hpx) == 1
    assert _status(lambda: mu.muon_step_batched(h, [], hp, ws)) == 1
    torch.cuda.synchronize()
    assert torch.equal(W, W0)
    # AdamW validation
    p = torch.zeros(10, device=DEV)
    t = mu.adamw_tensor(p, p.clone(), p.clone(), p.clone())
    assert _status(lambda: mu.adamw_step(h, [t], mu.adamw_hparams(1e-3, step=0))) == 1
    t2 = mu.adamw_tensor(p, p.clone(), p.clone(), p.clone()); t2.numel = -1
    assert _status(lambda: mu.adamw_step(h, [t2], mu.adamw_hparams(1e-3, step=1))) == 1
    t3 = mu.adamw_tensor(p, p.clone(), p.clone(), p.clone()); t3.grad = None
    assert _status(lambda: mu.adamw_step(h, [t3], mu.adamw_hparams(1e-3, step=1))) == 1
    assert mu.load().muon_status_str(3) == b"workspace missing or too small"


# ------------------------------------------------------------------ AdamW --

ADAMW_HP = dict(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@pytest.mark.parametrize("pdt,gdt", [(torch.float32, torch.float32), (torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.float32), (torch.bfloat16, torch.bfloat16)])
def test_adamw_many_tensors_three_steps(pdt, gdt):
    h = Handle.get()
    # more tensors than one launch takes (256): two launch groups, the second
    # starting inside the run of small tensors
    sizes = ([1, 3, 4095, 4096, 4097, 10000, 65539, 0] + [257 * k for k in range(1, 33)] +
             [5 + 37 * (k % 11) for k in range(240)])
    g = torch.Generator(device=DEV).manual_seed(5)
    P, M, V, ref = [], [], [], []
    for n in sizes:
        p = (torch.randn(n, generator=g, device=DEV) * 0.02).to(pdt)
        P.append(p)
        M.append(torch.zeros(n, device=DEV))
        V.append(torch.zeros(n, device=DEV))
        ref.append([f64(p), np.zeros(n), np.zeros(n)])
    # an unaligned view (offset by one element) exercises the scalar path
    base = torch.randn(5001, generator=g, device=DEV).to(pdt) * 0.02
    P.append(base[1:])
    M.append(torch.zeros(5000, device=DEV))
    V.append(torch.zeros(5000, device=DEV))
    ref.append([f64(base[1:]), np.zeros(5000), np.zeros(5000)])
    for t in range(1, 4):
        grads = [(torch.randn(p.numel(), generator=g, device=DEV) * 1e-2).to(gdt) for p in P]
        ts = [mu.adamw_tensor(p, gr, m, v) for p, gr, m, v in zip(P, grads, M, V)]
        mu.adamw_step(h, ts, mu.adamw_hparams(step=t, **ADAMW_HP))
        torch.cuda.synchronize()
        for i, gr in enumerate(grads):
            th, m, v = oracle.adamw_tensor_step(ref[i][0], f64(gr), ref[i][1], ref[i][2], step=t,
                                                param_dtype="bf16" if pdt == torch.bfloat16 else "fp32",
                                                **ADAMW_HP)
            ref[i] = [th, m, v]
    for i in range(len(P)):
        if P[i].numel() == 0:
            continue
        # the moments do not depend on the parameter: fp32 state at 1e-6 always
        assert relF(f64(M[i]), ref[i][1]) <= TOL_STATE, i
        assert relF(f64(V[i]), ref[i][2]) <= TOL_STATE, i
        if pdt == torch.bfloat16:
            # the oracle keeps its own bf16 parameter (each step rounded once):
            # almost every element equal, the rest one rounding apart
            got, want = f64(P[i]), ref[i][0]
            exact = np.mean(got == want)
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
            assert exact >= 0.99, (i, exact)
            assert np.all(np.abs(got - want) <= 2 * ulp), i
        else:
            assert relF(f64(P[i]), ref[i][0]) <= TOL_STATE, i

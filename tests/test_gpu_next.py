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
    # 279 tensors: two launch groups (256 tensors each at most), so the sum of
    # squares of the second group lands after the first group's partials
    sizes = [3, 4096, 70000, 1024 * 1024 + 5] + [999] * 35 + [777] * 240
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


def test_mixed_class_call_equals_one_call_per_class():
    # One call over all three size classes (a 1024 x 768 matrix, four
    # 128 x 1536 blocks, two tiny matrices running the fp32 iteration) forks
    # the small and fp32 classes onto the handle's second stream after the
    # momentum launch and joins them before the apply.  The same matrices in
    # three calls of one class each (no fork) must give bitwise equal
    # weights, momenta and orthogonalised updates, over two steps.
    shapes = [(1024, 768)] + [(128, 1536)] * 4 + [(24, 700), (900, 17)]
    hp = hp_from(BASE_HP)

    def state():
        W = [_weight(r, c, 40 + i) for i, (r, c) in enumerate(shapes)]
        M = [torch.zeros(r, c, device=DEV) for r, c in shapes]
        O = [torch.empty(r, c, device=DEV) for r, c in shapes]
        return W, M, O

    (Wa, Ma, Oa), (Wb, Mb, Ob) = state(), state()
    groups = [[0], [1, 2, 3, 4], [5, 6]]   # large, small, fp32 classes
    for step in range(2):
        G = [_grad(r, c, 60 + 10 * step + i) for i, (r, c) in enumerate(shapes)]
        run_muon_step([mu.muon_matrix(Wa[i], G[i], Ma[i], update_out=Oa[i]) for i in range(len(shapes))], hp)
        for grp in groups:
            run_muon_step([mu.muon_matrix(Wb[i], G[i], Mb[i], update_out=Ob[i]) for i in grp], hp)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(Oa[i], Ob[i]), (step, i, "O")
            assert torch.equal(Ma[i], Mb[i]), (step, i, "M")
            assert torch.equal(Wa[i], Wb[i]), (step, i, "W")


@pytest.mark.parametrize("hpd", [BASE_HP, dict(BASE_HP, steps=3, coeffs=[3.0, -3.2, 1.2, 3.4445, -4.7750, 2.0315,
                                                                  1.875, -1.25, 0.375])],
                         ids=["5 steps", "3 steps, schedule"])
def test_small_class_update_in_strips(hpd):
    # 8 blocks of 100 x 4900 and 8 of 4900 x 100 (transposed): 16 x 39 column
    # tiles of 128 in the small class, more than two workgroups per compute
    # unit can take at once, so the update runs two tiles per workgroup and
    # the last strip of every matrix holds one tile.  Each strip forms its
    # matrix's B itself, with the iteration's coefficients.
    from harness import TOL_BLOCK_BF16, check_output
    shapes = [(100, 4900)] * 8 + [(4900, 100)] * 8
    W = [_weight(r, c, 80 + i) for i, (r, c) in enumerate(shapes)]
    G = [_grad(r, c, 120 + i) for i, (r, c) in enumerate(shapes)]
    M = [torch.zeros(r, c, device=DEV) for r, c in shapes]
    O = [torch.empty(r, c, device=DEV) for r, c in shapes]
    ins = [(f64(w), f64(g)) for w, g in zip(W, G)]
    run_muon_step([mu.muon_matrix(W[i], G[i], M[i], update_out=O[i]) for i in range(len(shapes))],
                  hp_from(hpd))
    torch.cuda.synchronize()
    kw = oracle_kwargs(hpd)
    for i, (W0, G0) in enumerate(ins):
        Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), **kw)
        check_output(f64(O[i]), Or, TOL_O_BF16, TOL_BLOCK_BF16, what="strip matrix %d" % i)
        assert relF(f64(M[i]), Mr) <= TOL_STATE, i
        assert relF(f64(W[i]), Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(*W0.shape), Or, Wr,
                                                  TOL_O_BF16), i


@pytest.mark.parametrize("hpd", [BASE_HP, dict(BASE_HP, steps=2),
                                 dict(BASE_HP, steps=3, coeffs=[3.4445, -4.7750, 2.0315,
                                                                3.0, -3.2, 1.2, 1.875, -1.25, 0.375])],
                         ids=["5 steps", "2 steps", "3 steps, schedule"])
def test_per_head_gram_parts_from_update_strips(hpd):
    # 64 heads of 128 x 3584 (rows of one 8192 x 3584 tensor): the small class
    # takes a K-split Gram of 7 parts and an update in 7 strips of 4 column
    # tiles per head, the same column ranges, so from the second iteration on
    # the update's strips store the Gram parts and no split Gram launch runs.
    # Sampled heads against the oracle over two steps (momentum carried), for
    # an odd and an even iteration count and a coefficient schedule.
    heads, dh, dm = 64, 128, 3584
    Wf = _weight(heads * dh, dm, 7)
    Mf = torch.zeros(heads * dh, dm, device=DEV)
    Of = torch.empty(heads * dh, dm, device=DEV)
    sample = [0, 1, 9, 31, 32, 47, 62, 63]
    ref = {h: [f64(Wf[h * dh:(h + 1) * dh]), np.zeros((dh, dm))] for h in sample}
    kw = oracle_kwargs(hpd)
    for step in range(2):
        Gf = _grad(heads * dh, dm, 200 + step)
        mats = [mu.muon_matrix(Wf[h * dh:(h + 1) * dh], Gf[h * dh:(h + 1) * dh], Mf[h * dh:(h + 1) * dh],
                               update_out=Of[h * dh:(h + 1) * dh]) for h in range(heads)]
        run_muon_step(mats, hp_from(hpd))
        torch.cuda.synchronize()
        for h in sample:
            sl = slice(h * dh, (h + 1) * dh)
            W0, M0 = ref[h]
            Wr, Mr, Or = oracle.muon_matrix_step(W0, f64(Gf[sl]), M0, **kw)
            assert relF(f64(Of[sl]), Or) <= TOL_O_BF16, (step, h)
            assert relF(f64(Mf[sl]), Mr) <= TOL_STATE, (step, h)
            assert relF(f64(Wf[sl]), Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(dh, dm), Or, Wr,
                                                       TOL_O_BF16), (step, h)
            # carry the GPU's own state, so each step is checked on its own
            ref[h] = [f64(Wf[sl]), f64(Mf[sl])]


def test_per_head_column_blocks_fused_strips():
    # Column blocks of a (3584, 64 x 128) tensor: 64 strided views of 3584 x 128
    # (leading dimension 8192), tall, so each is transposed to 128 x 3584: the
    # small class with 7 Gram parts and 7 strips per block, the fused strip
    # update, the momentum and apply transposing through LDS, and the other
    # columns of the tensor untouched.  Sampled blocks against the oracle.
    heads, dh, rows = 64, 128, 3584
    Wf = _weight(rows, heads * dh, 31)
    Gf = _grad(rows, heads * dh, 32)
    Mf = torch.zeros(rows, heads * dh, device=DEV)
    O = [torch.empty(rows, dh, device=DEV) for _ in range(heads)]
    W0f = Wf.clone()
    mats = [mu.muon_matrix(Wf[:, h * dh:(h + 1) * dh], Gf[:, h * dh:(h + 1) * dh], Mf[:, h * dh:(h + 1) * dh],
                           update_out=O[h]) for h in range(heads - 1)]  # the last block stays untouched
    run_muon_step(mats, hp_from(BASE_HP))
    torch.cuda.synchronize()
    kw = oracle_kwargs(BASE_HP)
    for h in [0, 1, 7, 31, 32, 62]:
        sl = slice(h * dh, (h + 1) * dh)
        W0, G0 = f64(W0f[:, sl]), f64(Gf[:, sl])
        Wr, Mr, Or = oracle.muon_matrix_step(W0, G0, np.zeros_like(W0), **kw)
        assert relF(f64(O[h]), Or) <= TOL_O_BF16, h
        assert relF(f64(Mf[:, sl]), Mr) <= TOL_STATE, h
        assert relF(f64(Wf[:, sl]), Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(rows, dh), Or, Wr,
                                                       TOL_O_BF16), h
    last = slice((heads - 1) * dh, heads * dh)
    assert torch.equal(Wf[:, last], W0f[:, last]) and torch.count_nonzero(Mf[:, last]) == 0


@pytest.mark.parametrize("blocks,tiles,tall", [(64, 5, False), (64, 10, True), (64, 23, False), (64, 31, False),
                                               (32, 36, False)],
                         ids=["strips 2-2-1", "tall, strips 3-3-3-1", "strips 6-6-6-5, fused",
                              "strips 8-8-8-7, fused", "strips 5 x 7 + 1, fused"])
def test_small_class_alone_streamed_strips(blocks, tiles, tall):
    # `blocks` blocks of 128 x 128*tiles (or their transposes), the small class
    # alone in the call: its update streams strips of ceil(blocks * tiles / 256)
    # column tiles at one workgroup per compute unit, the last strip of every
    # block shorter (down to one tile, whose strip copies its block twice).
    # The strip lengths reach every tail length of the streaming kernel's loop
    # (first tile, whole rounds of three, then 0-5 tiles); with parts of at
    # least 8 slabs the K-split Gram takes one part per strip and the strips
    # form the next Gram's parts (fused), else the Gram runs split each
    # iteration.  Sampled blocks against the oracle over two carried steps.
    from harness import TOL_BLOCK_BF16, check_output
    dh = 128
    dm = 128 * tiles
    shape = (dm, dh) if tall else (dh, dm)
    Ws = [_weight(*shape, 300 + i) for i in range(blocks)]
    Ms = [torch.zeros(*shape, device=DEV) for _ in range(blocks)]
    Os = [torch.empty(*shape, device=DEV) for _ in range(blocks)]
    sample = sorted({0, 1, 17, blocks // 2 - 1, blocks // 2, blocks - 2, blocks - 1})
    ref = {b: [f64(Ws[b]), np.zeros(shape)] for b in sample}
    kw = oracle_kwargs(BASE_HP)
    for step in range(2):
        Gs = [_grad(*shape, 400 + 100 * step + i) for i in range(blocks)]
        run_muon_step([mu.muon_matrix(Ws[i], Gs[i], Ms[i], update_out=Os[i]) for i in range(blocks)],
                      hp_from(BASE_HP))
        torch.cuda.synchronize()
        for b in sample:
            W0, M0 = ref[b]
            Wr, Mr, Or = oracle.muon_matrix_step(W0, f64(Gs[b]), M0, **kw)
            check_output(f64(Os[b]), Or, TOL_O_BF16, TOL_BLOCK_BF16, what="block %d step %d" % (b, step))
            assert relF(f64(Ms[b]), Mr) <= TOL_STATE, (step, b)
            assert relF(f64(Ws[b]), Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(*shape), Or, Wr,
                                                       TOL_O_BF16), (step, b)
            ref[b] = [f64(Ws[b]), f64(Ms[b])]


def test_streamed_strips_with_fused_gram_parts_are_repeatable():
    # The streamed strips form the next Gram's parts and the reduce sums them
    # in part order, so two runs from the same state give the same bits
    # (64 blocks of 128 x 2944: strips of 6 tiles, 4 parts per block).
    blocks, shape = 64, (128, 128 * 23)
    res = []
    for _ in range(2):
        Ws = [_weight(*shape, 700 + i) for i in range(blocks)]
        Gs = [_grad(*shape, 800 + i) for i in range(blocks)]
        Ms = [torch.zeros(*shape, device=DEV) for _ in range(blocks)]
        Os = [torch.empty(*shape, device=DEV) for _ in range(blocks)]
        run_muon_step([mu.muon_matrix(Ws[i], Gs[i], Ms[i], update_out=Os[i]) for i in range(blocks)],
                      hp_from(BASE_HP))
        torch.cuda.synchronize()
        res.append([t.clone() for t in Ws + Ms + Os])
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("blocks,tiles,extra,hpd",
                         [(64, 5, 0, BASE_HP), (32, 36, 0, BASE_HP), (64, 23, 256, BASE_HP),
                          (64, 23, 0, dict(BASE_HP, steps=1)), (64, 56, 0, dict(BASE_HP, steps=2))],
                         ids=["strips 2-2-1", "strips 5 x 7 + 1, fused", "ld > cols, fused",
                              "one iteration", "per-head 128 x 7168, two iterations"])
def test_streamed_strips_apply_the_step(blocks, tiles, extra, hpd):
    # Blocks of 128 x 128*tiles fp32 weights (rows of one tensor whose width
    # may exceed the blocks' by `extra` columns), the small class alone: the
    # last update's strips update W themselves and no apply launch runs.  The
    # same blocks with an update output take the apply launch instead; W and
    # M must agree bit for bit over two carried steps, the untouched columns
    # stay untouched, and sampled blocks match the oracle.
    from harness import TOL_BLOCK_BF16, check_output
    rows, cols = 128, 128 * tiles
    shape = (rows, cols)
    sample = sorted({0, 1, blocks // 2, blocks - 1})
    kw = oracle_kwargs(hpd)
    Wf = [_weight(blocks * rows, cols + extra, 900 + tiles) for _ in range(2)]
    Mf = [torch.zeros(blocks * rows, cols + extra, device=DEV) for _ in range(2)]
    W0_rest = Wf[0][:, cols:].clone()
    Os = [torch.empty(*shape, device=DEV) for _ in range(blocks)]
    ref = {b: [f64(Wf[0][b * rows:(b + 1) * rows, :cols]), np.zeros(shape)] for b in sample}
    for step in range(2):
        Gf = _grad(blocks * rows, cols + extra, 950 + step)
        for v in range(2):
            blk = [(Wf[v][b * rows:(b + 1) * rows, :cols], Gf[b * rows:(b + 1) * rows, :cols],
                    Mf[v][b * rows:(b + 1) * rows, :cols]) for b in range(blocks)]
            mats = [mu.muon_matrix(w, g, m, update_out=Os[b] if v == 0 else None)
                    for b, (w, g, m) in enumerate(blk)]
            run_muon_step(mats, hp_from(hpd))
        torch.cuda.synchronize()
        assert torch.equal(Wf[0], Wf[1]), step
        assert torch.equal(Mf[0], Mf[1]), step
        assert torch.equal(Wf[1][:, cols:], W0_rest) and torch.count_nonzero(Mf[1][:, cols:]) == 0
        for b in sample:
            sl = slice(b * rows, (b + 1) * rows)
            W0, M0 = ref[b]
            Wr, Mr, Or = oracle.muon_matrix_step(W0, f64(Gf[sl, :cols]), M0, **kw)
            check_output(f64(Os[b]), Or, TOL_O_BF16, TOL_BLOCK_BF16, what="block %d step %d" % (b, step))
            assert relF(f64(Mf[1][sl, :cols]), Mr) <= TOL_STATE, (step, b)
            assert relF(f64(Wf[1][sl, :cols]), Wr) <= w_tolerance(kw["lr"], oracle.shape_scale(*shape), Or, Wr,
                                                                 TOL_O_BF16), (step, b)
            ref[b] = [f64(Wf[1][sl, :cols]), f64(Mf[1][sl, :cols])]

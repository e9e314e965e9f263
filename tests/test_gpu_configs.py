"""Workload-level parity: the five configurations and the 8 x 4096^2 headline
workload, at full size, through muon_step_batched / adamw_step exactly as
bench.py calls them.  Every Muon matrix is updated on the GPU; the oracle
recomputes a sample of them (and sampled rows of the big AdamW tensors)
from the same inputs.  The sample always includes matrices whose tiles sit
where the grouped GEMM launches' per-XCD tile ranges start or end, or that
hold quarter tiles (the scheduler's own answer, muon_test_split_matrices),
and every sampled output is checked block by block as well as whole."""

import numpy as np
import pytest
import torch

import oracle
import synth
import muon_step_02_amd as mu
from harness import (TOL_O_BF16, TOL_O_F32, TOL_STATE, Handle, block_error, block_tol,
                     check_output, f64, hp_from, oracle_kwargs, recipe_floor_output, relF)

pytestmark = pytest.mark.gpu

DEV = "cuda"


class Materialised:
    """A workload's tensors on the GPU plus optimizer state."""

    def __init__(self, wl, keep_update=()):
        self.wl = wl
        self.W = [wl.make_weight(i, DEV) for i in range(len(wl.tensors))]
        self.G = [None] * len(wl.tensors)
        self.M = {}
        for v in wl.muon:
            if v.tensor not in self.M:
                self.M[v.tensor] = torch.zeros(wl.tensors[v.tensor].shape, device=DEV)
        self.m = {i: torch.zeros(wl.tensors[i].shape, device=DEV) for i in wl.adamw}
        self.v = {i: torch.zeros(wl.tensors[i].shape, device=DEV) for i in wl.adamw}
        self.O = {k: torch.empty(wl.muon[k].rows, wl.tensors[wl.muon[k].tensor].shape[1], device=DEV)
                  for k in keep_update}
        self.ws = None

    def view(self, t, k):
        v = self.wl.muon[k]
        return t[v.tensor][v.row0:v.row0 + v.rows]

    def new_grads(self, step):
        for i in range(len(self.wl.tensors)):
            self.G[i] = None
        for i in range(len(self.wl.tensors)):
            self.G[i] = self.wl.make_grad(i, step, DEV)

    def step(self, t, hp, adamw_hp=None):
        h = Handle.get()
        mats = []
        for k, v in enumerate(self.wl.muon):
            W = self.W[v.tensor][v.row0:v.row0 + v.rows]
            G = self.G[v.tensor][v.row0:v.row0 + v.rows]
            M = self.M[v.tensor][v.row0:v.row0 + v.rows]
            mats.append(mu.muon_matrix(W, G, M, update_out=self.O.get(k)))
        need = mu.muon_workspace_size(h, mats, hp)
        if self.ws is None or self.ws.numel() < need:
            self.ws = None
            self.ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        mu.muon_step_batched(h, mats, hp, self.ws)
        if self.wl.adamw:
            ts = [mu.adamw_tensor(self.W[i], self.G[i], self.m[i], self.v[i]) for i in self.wl.adamw]
            mu.adamw_step(h, ts, mu.adamw_hparams(step=t, **adamw_hp))


def split_sample(wl, hp, limit=8):
    """Up to `limit` matrices (evenly spread) of the scheduler's split list."""
    h = Handle.get()
    mats = []
    for v in wl.muon:
        shape = (v.rows, wl.tensors[v.tensor].shape[1])
        # shapes and dtypes are all the planner reads; pointers are not checked
        m = mu.MuonMatrix(rows=shape[0], cols=shape[1], ld_param=shape[1], ld_grad=shape[1],
                          ld_mom=shape[1], param_dtype=mu.MUON_F32,
                          grad_dtype=mu.MUON_BF16 if wl.tensors[v.tensor].grad_dtype == torch.bfloat16
                          else mu.MUON_F32)
        mats.append(m)
    idx = mu.muon_test_split_matrices(h, mats, hp)
    if len(idx) > limit:
        idx = [idx[int(round(i * (len(idx) - 1) / (limit - 1)))] for i in range(limit)]
    return idx


def _run(wl, steps, sample, adamw_rows=None, hp_over=None, report_name="", split_limit=8):
    hpd = dict(wl.muon_hp)
    hpd.update(hp_over or {})
    tol_o = TOL_O_F32 if hpd["ns_dtype"] == "fp32" else TOL_O_BF16
    hp = hp_from(hpd)
    extra = split_sample(wl, hp, split_limit)
    print(report_name, "matrices at XCD range boundaries / quarter tiles:", extra)
    sample = sorted(set(sample) | set(extra))
    st = Materialised(wl, keep_update=sample)
    # host copies of what the oracle needs
    ref_W = {k: f64(st.view(st.W, k)) for k in sample}
    ref_M = {k: np.zeros_like(ref_W[k]) for k in sample}
    ad_rows = {}
    for i in wl.adamw:
        rows = adamw_rows(i, wl.tensors[i].shape) if adamw_rows else slice(None)
        ad_rows[i] = rows
    ref_ad = {i: [f64(st.W[i][ad_rows[i]]), 0.0, 0.0] for i in wl.adamw}
    report = []
    for t in range(1, steps + 1):
        st.new_grads(t)
        G_host = {k: f64(st.view(st.G, k)) for k in sample}
        G_ad = {i: f64(st.G[i][ad_rows[i]]) for i in wl.adamw}
        st.step(t, hp, wl.adamw_hp)
        torch.cuda.synchronize()
        for k in sample:
            kw = oracle_kwargs(hpd)
            Wr, Mr, Or = oracle.muon_matrix_step(ref_W[k], G_host[k], ref_M[k], **kw)
            eo, eb = check_output(f64(st.O[k]), Or, tol_o, block_tol(tol_o), (report_name, t, k))
            em = relF(f64(st.view(st.M, k)), Mr)
            ew = relF(f64(st.view(st.W, k)), Wr)
            floor = float("nan")
            if hpd["ns_dtype"] == "bf16" and t == 1 and k == sample[0]:
                # the bf16 recipe's own error on this input (reported only)
                Y = oracle.nesterov_blend(G_host[k], Mr, kw["mu"], kw["nesterov"])
                Ob = recipe_floor_output(Y, kw["steps"], kw["eps"], kw["coeffs"])
                floor = relF(Ob, oracle.newton_schulz(Y, steps=kw["steps"], eps=kw["eps"],
                                                      coeffs=kw["coeffs"]))
            report.append((t, k, wl.muon_shapes()[k], eo, eb, floor, em, ew))
            assert em <= TOL_STATE, (report_name, t, k, "M", em)
            # open loop: the oracle continues from its own W and M
            ref_W[k], ref_M[k] = Wr, Mr
            s = oracle.shape_scale(*Wr.shape, kw["scale_mode"]) * kw["extra_scale"]
            tw = t * (kw["lr"] * s * tol_o * np.linalg.norm(Or)) / np.linalg.norm(Wr) + 2e-6
            assert ew <= tw, (report_name, t, k, "W", ew, tw)
        for i in wl.adamw:
            th, m, v = oracle.adamw_tensor_step(ref_ad[i][0], G_ad[i], ref_ad[i][1], ref_ad[i][2],
                                                step=t, **wl.adamw_hp)
            ref_ad[i] = [th, m, v]
            r = ad_rows[i]
            assert relF(f64(st.W[i][r]), th) <= TOL_STATE, (report_name, t, i, "theta")
            assert relF(f64(st.m[i][r]), m) <= TOL_STATE, (report_name, t, i, "m")
            assert relF(f64(st.v[i][r]), v) <= TOL_STATE, (report_name, t, i, "v")
    for line in report:
        print(report_name, "step %d matrix %d %s: O %.3e (worst block %.3e, bf16 recipe floor %.3e)"
              "  M %.3e  W %.3e" % line)
    return report


@pytest.mark.parametrize("mode", ["jordan", "moonlight"])
def test_config0_fp32_newton_schulz(mode):
    _run(synth.config0(), 1, [0], hp_over=dict(scale_mode=mode), report_name="c0-" + mode)


def test_config1_block_three_steps_with_adamw():
    wl = synth.config1()
    _run(wl, 3, list(range(len(wl.muon))), report_name="c1")


def test_config2_llama_layer():
    wl = synth.config2()
    _run(wl, 1, list(range(len(wl.muon))), report_name="c2")


def test_config3_moe_experts():
    wl = synth.config3()
    quiet = wl.quiet_experts[0]
    loud = next(e for e in range(64) if e not in wl.quiet_experts)
    sample = [3 * loud, 3 * loud + 2, 3 * quiet, 3 * quiet + 2]
    _run(wl, 1, sample, report_name="c3")


def test_config4_hybrid_decoder_two_steps():
    wl = synth.config4()
    # layer 0 and layer 23: Q, K, V, O, up, down
    sample = list(range(0, 6)) + list(range(6 * 23, 6 * 24))

    def rows(i, shape):
        if len(shape) == 2 and shape[0] > 8192:
            return slice(4096, 4096 + 512)   # 512 rows of the embedding / head
        return slice(None)
    _run(wl, 2, sample, adamw_rows=rows, report_name="c4")


def test_headline_workload():
    wl = synth.headline()
    _run(wl, 1, [0, 7], report_name="headline")


def test_perhead_workload():
    # 64 heads x 128 x 7168 (row blocks of one 8192 x 7168 query projection):
    # the 128-tile class with a K-split Gram (64 tiles of K = 7168 for 256
    # compute units); heads sampled at both ends and where the scheduler's
    # per-XCD ranges start or end
    wl = synth.perhead()
    _run(wl, 1, [0, 1, 31, 63], report_name="perhead", split_limit=12)


def test_perhead_mixed_workload():
    # per-head Q and K blocks (128 x 4096) beside whole 4096 x 4096 V and O
    wl = synth.perhead_mixed()
    _run(wl, 1, [0, 33, 64, 65], report_name="perhead-mixed")

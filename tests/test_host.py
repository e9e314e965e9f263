"""Host-side checks that need no GPU: the library loads and exports what the
header declares, the ctypes structures match the C layout the compiler
gives, parameter routing, and the synthetic workloads."""

import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

import muon_step_02_amd as mu
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:muon_status|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("muon_init", "muon_step_batched", "adamw_step", "muon_workspace_size",
                     "muon_destroy", "muon_status_str"):
        assert required in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(mu.LIB_PATH), "build first: python -m muon_step_02_amd.build"
    lib = mu.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert sorted(mu.exported_symbols()) == sorted(_declared_functions())
    out = subprocess.run(["nm", "-D", "--defined-only", mu.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


def test_status_strings_without_device():
    lib = mu.load()
    assert lib.muon_status_str(0) == b"ok"
    assert lib.muon_status_str(99) == b"unknown status"


STRUCTS = {
    "muon_matrix": mu.MuonMatrix,
    "muon_hparams": mu.MuonHparams,
    "adamw_tensor": mu.AdamwTensor,
    "adamw_hparams": mu.AdamwHparams,
    "muon_phase_times": mu.PhaseTimes,
}


def test_ctypes_layout_matches_c_compiler(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "muon.h"', "int main(void){"]
    for cname, cls in STRUCTS.items():
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for fname, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, fname, cname, fname))
    lines.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        k, _, v = line.rpartition(" ")
        got[k] = int(v)
    for cname, cls in STRUCTS.items():
        assert got["%s size" % cname] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got["%s.%s" % (cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_init_without_gpu_fails_cleanly():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(mu.MuonError) as e:
        mu.muon_init(0)
    assert e.value.status == 2


def test_hparams_helper():
    hp = mu.muon_hparams(lr=0.02, ns_dtype="fp32", scale_mode="jordan", nesterov=False,
                         coeffs=[1.0, 2.0, 3.0])
    assert hp.ns_dtype == mu.MUON_F32 and hp.scale_mode == 1 and hp.nesterov == 0
    assert [hp.coeffs[i] for i in range(3)] == [1.0, 2.0, 3.0]
    with pytest.raises(KeyError):
        mu.muon_hparams(lr=1.0, scale_mode="spectral")


def test_matrix_descriptor_from_row_block():
    W = torch.zeros(12, 5)
    G = torch.zeros(12, 5, dtype=torch.bfloat16)
    M = torch.zeros(12, 5)
    d = mu.muon_matrix(W[4:8], G[4:8], M[4:8])
    assert (d.rows, d.cols, d.ld_param, d.ld_grad) == (4, 5, 5, 5)
    assert d.param == W.data_ptr() + 4 * 5 * 4
    assert d.grad == G.data_ptr() + 4 * 5 * 2
    assert d.param_dtype == mu.MUON_F32 and d.grad_dtype == mu.MUON_BF16
    with pytest.raises(ValueError):
        mu.muon_matrix(W.T, G[:5, :5].T, M.T)
    with pytest.raises(TypeError):
        mu.muon_matrix(W, G, M.double())


# ------------------------------------------------------------------ routing --

def test_route_parameters():
    ps = {
        "embed.weight": torch.zeros(100, 16),
        "layers.0.attn.qkv.weight": torch.zeros(48, 16),
        "layers.0.attn.qkv.bias": torch.zeros(48),
        "layers.0.ln1.weight": torch.zeros(16),
        "layers.0.mlp.up.weight": torch.zeros(64, 16),
        "layers.0.mlp.router.weight": torch.zeros(8, 16),
        "final_norm.weight": torch.zeros(16),
        "lm_head.weight": torch.zeros(100, 16),
        "layers.0.attn.o.weight": torch.zeros(16, 16),
    }
    muon, adamw = mu.route_parameters(ps.items())
    assert [n for n, _ in muon] == ["layers.0.attn.qkv.weight", "layers.0.mlp.up.weight",
                                    "layers.0.attn.o.weight"]
    assert len(adamw) == len(ps) - 3
    muon, adamw = mu.route_parameters(ps.items(), exclude={"layers.0.attn.o.weight"})
    assert "layers.0.attn.o.weight" in [n for n, _ in adamw]


# ------------------------------------------------------- synthetic inputs --

def test_generators_are_seeded_and_shaped():
    w = synth.config1()
    a = w.make_grad(0, 1, "cpu")
    b = w.make_grad(0, 1, "cpu")
    c = w.make_grad(0, 2, "cpu")
    assert a.shape == (1024, 1024) and a.dtype == torch.float32
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert torch.equal(w.make_weight(1, "cpu"), w.make_weight(1, "cpu"))
    ln = w.make_weight(len(w.tensors) - 2, "cpu")
    assert torch.all(ln == 1.0)


def test_lowrank_generator_spectrum():
    ss = synth.seed_sequence(9, 0, 0)
    rec = synth.GradRecipe("lowrank", rank=8, decay=0.5, noise_std=0.0)
    G = synth.make_grad(rec, (64, 96), torch.float64, "cpu", ss).numpy()
    s = np.linalg.svd(G, compute_uv=False)
    assert np.allclose(s[:8], 10.0 ** (-np.arange(8) * 0.5), rtol=1e-10)
    assert s[8] < 1e-12


def test_workload_shapes_and_flops():
    c0, c1, c2, c3, c4 = (synth.config0(), synth.config1(), synth.config2(), synth.config3(),
                          synth.config4())
    assert c0.ns_flops()[0] == pytest.approx(0.3355e9, rel=1e-3)
    assert c1.ns_flops()[0] == pytest.approx(0.2952e12, rel=1e-3)
    assert c2.ns_flops()[0] == pytest.approx(14.74e12, rel=1e-3)
    assert c3.ns_flops()[0] == pytest.approx(94.83e12, rel=1e-3)
    assert c4.ns_flops()[0] == pytest.approx(43.29e12, rel=1e-3)
    h = synth.headline()
    assert h.ns_flops()[0] / 8 == pytest.approx(1.374e12, rel=1e-3)
    assert len(c3.muon) == 192 and len(c3.quiet_experts) == 16
    assert len(c4.muon) == 144
    n_params = sum(int(np.prod(t.shape)) for t in c4.tensors)
    assert n_params == pytest.approx(1.415e9, rel=1e-3)
    assert sum(int(np.prod(c4.tensors[i].shape)) for i in c4.adamw) == pytest.approx(206.6e6, rel=2e-3)


XCD_SPLIT_TEST = r"""
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <vector>
#include <algorithm>
namespace muon {
struct XcdSplit { int32_t b[9]; int32_t per; int32_t sub[8]; int32_t interleaved, rounds, cus; };
XcdSplit xcd_split(const int32_t* ntiles, const int64_t* weight, int n, int cus, int quarters,
                   int interleaved);
}
int main() {
    srand(7);
    for (int trial = 0; trial < 20000; ++trial) {
        int n = 1 + rand() % 12;
        const int cus = (trial & 1) ? 32 : 1 + rand() % 40;
        const int quarters = (trial >> 1) & 1;
        std::vector<int32_t> t(n);
        std::vector<int64_t> w(n);
        int64_t total_t = 0, total_w = 0, wmax = 0;
        for (int k = 0; k < n; ++k) {
            t[k] = (trial % 3 == 0) ? rand() % 3 : 1 + rand() % 300;
            w[k] = 1 + rand() % 256;
            total_t += t[k]; total_w += t[k] * w[k]; wmax = std::max(wmax, w[k]);
        }
        muon::XcdSplit xs = muon::xcd_split(t.data(), w.data(), n, cus, quarters, 0);
        if (xs.b[0] != 0 || xs.b[8] != total_t) { printf("bad ends %d\n", trial); return 1; }
        int per = 0;
        for (int x = 0; x < 8; ++x) {
            const int T = xs.b[x + 1] - xs.b[x];
            if (T < 0) { printf("not monotone %d\n", trial); return 1; }
            const int R = T % cus;
            // quarters only on the short last round, and only when asked for
            const int want = (quarters && R > 0 && 2 * R <= cus) ? R : 0;
            if (xs.sub[x] != want) { printf("sub %d x=%d %d/%d\n", trial, x, xs.sub[x], want); return 1; }
            per = std::max(per, T - xs.sub[x] + 4 * xs.sub[x]);
        }
        if (per != xs.per) { printf("per %d\n", trial); return 1; }
        // work of each range within one tile of the ideal eighth
        std::vector<int64_t> tw; for (int k = 0; k < n; ++k) for (int i = 0; i < t[k]; ++i) tw.push_back(w[k]);
        for (int x = 0; x < 8; ++x) {
            int64_t s = 0; for (int i = xs.b[x]; i < xs.b[x + 1]; ++i) s += tw[i];
            if (s * 8 > total_w + 8 * wmax) { printf("unbalanced %d x=%d %lld/%lld\n", trial, x, (long long)s, (long long)total_w); return 1; }
        }
    }
    printf("ok\n");
    return 0;
}
"""


def test_xcd_split_covers_every_tile_once_with_balanced_work(tmp_path):
    src = tmp_path / "xs.cpp"
    src.write_text(XCD_SPLIT_TEST)
    exe = tmp_path / "xs"
    libdir = os.path.dirname(mu.LIB_PATH)
    subprocess.run(["g++", "-O1", str(src), "-o", str(exe), "-L" + libdir, "-lmuon",
                    "-Wl,-rpath," + libdir], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_bench_roofline_choice_and_traffic_record(tmp_path):
    # bench.py's helpers: the HBM roofline applies below the ridge point only,
    # and a traffic record counts only for the kernel source it was taken on
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    m, n = 128, 7168                       # a per-head block: about 63 flop per byte
    flops, nbytes = 2 * m * m * n, (2 * m * n + m * m) * 2
    r = b.hbm_roofline(flops, nbytes, avg_ms=0.5, peak_tflops=2500.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - nbytes / 0.5e-3 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-3
    m = n = 4096                           # the headline's update: matrix-core bound
    assert b.hbm_roofline(2 * m * m * n, (2 * m * n + m * m) * 2, 0.1, 2500.0) is None
    src = tmp_path / "muon_step_02_amd" / "csrc"
    src.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (src / "gemm_bf16.hip").write_bytes(b"kernel source A")
    import hashlib
    sha = hashlib.sha256(b"kernel source A").hexdigest()
    rec = tmp_path / "profiles" / "traffic_k.md"
    rec.write_text("text\nsource_sha256: %s\nbytes_per_launch: 1.5e+09\n" % sha)
    assert b._traffic_record("k", root=str(tmp_path)) == 1.5e9
    (src / "gemm_bf16.hip").write_bytes(b"kernel source B")
    assert b._traffic_record("k", root=str(tmp_path)) is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

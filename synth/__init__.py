"""Seeded synthetic inputs for the Muon and AdamW workloads.

This module only *makes inputs*: weights, gradients and the lists of matrices
a workload holds.  It contains none of the optimizer's arithmetic and imports
neither the oracle nor the HIP library; both sides receive the same tensors
from here.

Gradient recipes (all seeded by ``numpy.random.SeedSequence([workload, step,
tensor])``):

* ``lowrank``: ``scale * (U_r diag(s) V_r^T + noise_std * N)`` with ``U_r``,
  ``V_r`` Haar-distributed orthonormal columns (QR of a Gaussian with the sign
  of R's diagonal fixed), ``s_i = 10^(-i*decay)`` for ``i = 0..r-1`` and ``N``
  iid standard normal: a few dominant directions over a noise floor, the very
  ill-conditioned update the pages describe (momentum updates "close to
  low-rank", "About Muon: Why Not Adam", section "Why not Adam", problem 2).
* ``hadamard``: ``scale * N o (P Q^T) / sqrt(r)``, Gaussian times low rank
  elementwise (full rank, heavy-tailed spectrum).
* ``gauss``: ``std * N`` (AdamW gradients).

The low-rank factors are drawn on the host with numpy (PCG64); the large
Gaussian fields with ``torch.randn`` on the target device from a generator
seeded by the same SeedSequence, so multi-gigabyte workloads are made on the
GPU in seconds.  Values are formed in float64 and rounded once to the
tensor's dtype.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch


def seed_sequence(workload_id, step, index):
    return np.random.SeedSequence([int(workload_id), int(step), int(index)])


def _torch_seed(ss):
    hi, lo = ss.generate_state(2, dtype=np.uint32)
    return ((int(hi) << 32) | int(lo)) & ((1 << 63) - 1)


def _generator(device, ss):
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    return g


def haar(rng, n, r):
    """n x r matrix with orthonormal columns, Haar distributed."""
    Z = rng.standard_normal((n, r))
    Q, R = np.linalg.qr(Z)
    Q = Q * np.sign(np.diag(R))[None, :]
    return Q


@dataclass
class GradRecipe:
    kind: str                 # "lowrank" | "hadamard" | "gauss" | "zero"
    rank: int = 0
    decay: float = 0.0        # s_i = 10^(-i*decay)
    noise_std: float = 0.0
    scale: float = 1.0
    std: float = 0.0


def make_grad(recipe, shape, dtype, device, ss):
    """Materialise one gradient tensor (rounded once to ``dtype``)."""
    rows, cols = (shape if len(shape) == 2 else (1, shape[0]))
    rng = np.random.Generator(np.random.PCG64(ss))
    gen = _generator(device, ss.spawn(1)[0])
    if recipe.kind == "zero":
        out = torch.zeros(rows, cols, dtype=torch.float64, device=device)
    elif recipe.kind == "lowrank":
        r = recipe.rank
        U = haar(rng, rows, r)
        V = haar(rng, cols, r)
        s = 10.0 ** (-np.arange(r) * recipe.decay)
        Us = torch.from_numpy(U * s[None, :]).to(device)
        Vt = torch.from_numpy(np.ascontiguousarray(V.T)).to(device)
        out = Us @ Vt
        if recipe.noise_std:
            noise = torch.randn(rows, cols, dtype=torch.float64, device=device, generator=gen)
            out.add_(noise, alpha=recipe.noise_std)
            del noise
        out.mul_(recipe.scale)
    elif recipe.kind == "hadamard":
        r = recipe.rank
        P = torch.from_numpy(rng.standard_normal((rows, r))).to(device)
        Qt = torch.from_numpy(np.ascontiguousarray(rng.standard_normal((cols, r)).T)).to(device)
        out = P @ Qt
        noise = torch.randn(rows, cols, dtype=torch.float64, device=device, generator=gen)
        out.mul_(noise)
        del noise
        out.mul_(recipe.scale / math.sqrt(r))
    elif recipe.kind == "gauss":
        out = torch.randn(rows, cols, dtype=torch.float64, device=device, generator=gen)
        out.mul_(recipe.std)
    else:
        raise ValueError(recipe.kind)
    out = out.to(dtype)
    return out.reshape(shape).contiguous()


@dataclass
class TensorSpec:
    name: str
    shape: tuple
    grad: GradRecipe
    init: str = "normal"      # "normal" (N(0, 0.02^2)) | "ones" | "zeros"
    param_dtype: torch.dtype = torch.float32
    grad_dtype: torch.dtype = torch.float32
    optimizer: str = "muon"   # "muon" | "adamw"


@dataclass
class MuonView:
    """A Muon matrix: rows [row0, row0+rows) of a 2D tensor of the workload."""
    tensor: int
    row0: int
    rows: int


@dataclass
class Workload:
    name: str
    workload_id: int
    tensors: list
    muon: list                # MuonView list
    adamw: list               # tensor indices
    steps: int = 1
    muon_hp: dict = field(default_factory=dict)
    adamw_hp: dict = field(default_factory=dict)

    def make_weight(self, i, device):
        spec = self.tensors[i]
        shape = spec.shape
        if spec.init == "ones":
            return torch.ones(shape, dtype=spec.param_dtype, device=device)
        if spec.init == "zeros":
            return torch.zeros(shape, dtype=spec.param_dtype, device=device)
        ss = seed_sequence(self.workload_id, 999, i)
        g = _generator(device, ss)
        w = torch.randn(shape, dtype=torch.float64, device=device, generator=g) * 0.02
        return w.to(spec.param_dtype).contiguous()

    def make_grad(self, i, step, device):
        spec = self.tensors[i]
        ss = seed_sequence(self.workload_id, step, i)
        return make_grad(spec.grad, spec.shape, spec.grad_dtype, device, ss)

    def muon_shapes(self):
        return [(v.rows, self.tensors[v.tensor].shape[1]) for v in self.muon]

    def ns_flops(self, ns_steps=5):
        """(triangle-aware, dense) Newton-Schulz flop counts per step."""
        alg = dense = 0
        for rows, cols in self.muon_shapes():
            m, n = min(rows, cols), max(rows, cols)
            alg += ns_steps * (3 * m * m * n + m ** 3)
            dense += ns_steps * (4 * m * m * n + 2 * m ** 3)
        return alg, dense


MUON_DEFAULT = dict(lr=2e-4, mu=0.95, weight_decay=0.1, nesterov=True, eps=1e-7,
                    steps=5, scale_mode="moonlight", extra_scale=1.0, ns_dtype="bf16")
ADAMW_DEFAULT = dict(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _muon_tensor(name, rows, cols, recipe, **kw):
    return TensorSpec(name, (rows, cols), recipe, **kw)


def config0():
    """One 256x256 fp32 matrix; 8 spikes 10^(-i/2) plus N(0, 1e-3) noise;
    lr 0.02, wd 0.01, fp32 Newton-Schulz."""
    t = [_muon_tensor("W", 256, 256, GradRecipe("lowrank", rank=8, decay=0.5, noise_std=1e-3))]
    hp = dict(MUON_DEFAULT, lr=0.02, weight_decay=0.01, ns_dtype="fp32", scale_mode="jordan")
    return Workload("c0: 256x256 fp32 matrix, fp32 Newton-Schulz", 0, t,
                    [MuonView(0, 0, 256)], [], steps=1, muon_hp=hp)


def config1():
    """d=1024 transformer block: Q,K,V,O 1024^2, up/gate 4096x1024, down
    1024x4096; rank-16 spikes 10^(-i/4) + noise; 3 steps; AdamW on two
    LayerNorms (weight and bias, 1024 each)."""
    rec = GradRecipe("lowrank", rank=16, decay=0.25, noise_std=1e-3)
    shapes = [("q", 1024, 1024), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 1024, 1024),
              ("up", 4096, 1024), ("gate", 4096, 1024), ("down", 1024, 4096)]
    t = [_muon_tensor(n, r, c, rec) for n, r, c in shapes]
    muon = [MuonView(i, 0, r) for i, (_, r, _) in enumerate(shapes)]
    ad = GradRecipe("gauss", std=1e-2)
    for j in range(2):
        t.append(TensorSpec("ln%d.weight" % j, (1024,), ad, init="ones", optimizer="adamw"))
        t.append(TensorSpec("ln%d.bias" % j, (1024,), ad, init="zeros", optimizer="adamw"))
    adamw = list(range(len(shapes), len(t)))
    return Workload("c1: d=1024 block, 3 steps, bf16 Newton-Schulz", 1, t, muon, adamw,
                    steps=3, muon_hp=dict(MUON_DEFAULT), adamw_hp=dict(ADAMW_DEFAULT))


def config2():
    """Llama-style d=4096 layer with GQA: Q,O 4096^2, K,V 1024x4096, up/gate
    14336x4096, down 4096x14336; bf16 gradients, fp32 master weights; rank-17
    spikes with sigma_1/sigma_17 = 1e4 plus noise."""
    rec = GradRecipe("lowrank", rank=17, decay=0.25, noise_std=1e-3)
    shapes = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
              ("up", 14336, 4096), ("gate", 14336, 4096), ("down", 4096, 14336)]
    t = [_muon_tensor(n, r, c, rec, grad_dtype=torch.bfloat16) for n, r, c in shapes]
    muon = [MuonView(i, 0, r) for i, (_, r, _) in enumerate(shapes)]
    return Workload("c2: Llama d=4096 layer (GQA), bf16 grads", 2, t, muon, [],
                    steps=1, muon_hp=dict(MUON_DEFAULT))


def config3(n_experts=64):
    """MoE expert batch at d=7168: per expert up/gate 2048x7168 and down
    7168x2048; rank-32 spikes 10^(-i/8) + noise, independent per expert; a
    seeded quarter of the experts has gradients scaled by 1e-6."""
    rng = np.random.Generator(np.random.PCG64(seed_sequence(3, 777, 0)))
    quiet = set(rng.choice(n_experts, size=n_experts // 4, replace=False).tolist())
    t, muon = [], []
    for e in range(n_experts):
        scale = 1e-6 if e in quiet else 1.0
        rec = GradRecipe("lowrank", rank=32, decay=0.125, noise_std=1e-3, scale=scale)
        for name, r, c in (("up", 2048, 7168), ("gate", 2048, 7168), ("down", 7168, 2048)):
            muon.append(MuonView(len(t), 0, r))
            t.append(_muon_tensor("e%d.%s" % (e, name), r, c, rec))
    w = Workload("c3: %d-expert MoE at d=7168" % n_experts, 3, t, muon, [],
                 steps=1, muon_hp=dict(MUON_DEFAULT))
    w.quiet_experts = sorted(quiet)
    return w


def config4(n_layers=24, d=2048, vocab=50304):
    """Hybrid step for a 24-layer d=2048 decoder: Muon on Q/K/V (row blocks
    of a fused 6144x2048 QKV), O, MLP up and down; AdamW on the untied
    embedding and head, the norms and the biases.  Gradients: Gaussian times
    rank-8, per-layer scale log-uniform in [1e-4, 1e-1]."""
    rng = np.random.Generator(np.random.PCG64(seed_sequence(4, 777, 0)))
    layer_scale = 10.0 ** rng.uniform(-4.0, -1.0, size=n_layers)
    t, muon, adamw = [], [], []
    ad = GradRecipe("gauss", std=1e-2)

    def add_adamw(name, shape, init="normal"):
        adamw.append(len(t))
        t.append(TensorSpec(name, shape, ad, init=init, optimizer="adamw"))

    add_adamw("embed", (vocab, d))
    for L in range(n_layers):
        rec = GradRecipe("hadamard", rank=8, scale=float(layer_scale[L]))
        qkv = len(t)
        t.append(_muon_tensor("l%d.qkv" % L, 3 * d, d, rec))
        for j in range(3):
            muon.append(MuonView(qkv, j * d, d))
        for name, r, c in (("o", d, d), ("up", 4 * d, d), ("down", d, 4 * d)):
            muon.append(MuonView(len(t), 0, r))
            t.append(_muon_tensor("l%d.%s" % (L, name), r, c, rec))
        add_adamw("l%d.ln1.weight" % L, (d,), "ones")
        add_adamw("l%d.ln1.bias" % L, (d,), "zeros")
        add_adamw("l%d.ln2.weight" % L, (d,), "ones")
        add_adamw("l%d.ln2.bias" % L, (d,), "zeros")
        add_adamw("l%d.qkv.bias" % L, (3 * d,), "zeros")
        add_adamw("l%d.o.bias" % L, (d,), "zeros")
        add_adamw("l%d.up.bias" % L, (4 * d,), "zeros")
        add_adamw("l%d.down.bias" % L, (d,), "zeros")
    add_adamw("final_ln.weight", (d,), "ones")
    add_adamw("final_ln.bias", (d,), "zeros")
    add_adamw("head", (vocab, d))
    return Workload("c4: 24-layer d=2048 decoder, hybrid Muon+AdamW", 4, t, muon, adamw,
                    steps=10, muon_hp=dict(MUON_DEFAULT), adamw_hp=dict(ADAMW_DEFAULT))


def headline(n=8, dim=4096):
    """n independent dim x dim fp32 weights, fp32 gradients (rank-16 spikes
    10^(-i/4) + noise), bf16 Newton-Schulz, Moonlight multiplier."""
    rec = GradRecipe("lowrank", rank=16, decay=0.25, noise_std=1e-3)
    t = [_muon_tensor("w%d" % i, dim, dim, rec) for i in range(n)]
    muon = [MuonView(i, 0, dim) for i in range(n)]
    return Workload("%dx %dx%d fp32 weights, bf16 Newton-Schulz" % (n, dim, dim), 100 + n, t,
                    muon, [], steps=1, muon_hp=dict(MUON_DEFAULT))


def headline_fp32(n=2, dim=4096):
    """The headline matrices with the fp32 iteration (its throughput at a
    size where it is not launch-bound)."""
    w = headline(n=n, dim=dim)
    w.muon_hp = dict(MUON_DEFAULT, ns_dtype="fp32")
    w.name = "%dx %dx%d fp32 weights, fp32 Newton-Schulz" % (n, dim, dim)
    return w


def perhead(n_heads=64, head_dim=128, d_model=7168):
    """Per-head Muon: the query projection of a d_model=7168, 64-head
    attention layer (8192 x 7168, Kimi K2's shape) orthogonalised one head at
    a time, i.e. 64 row blocks of 128 x 7168 of one fused tensor.  Gradient:
    rank-32 spikes 10^(-i/8) + noise over the fused tensor (as config 3)."""
    rec = GradRecipe("lowrank", rank=32, decay=0.125, noise_std=1e-3)
    t = [_muon_tensor("wq", n_heads * head_dim, d_model, rec)]
    muon = [MuonView(0, h * head_dim, head_dim) for h in range(n_heads)]
    return Workload("per-head Muon: %d heads x %dx%d (row blocks of a %dx%d query projection)"
                    % (n_heads, head_dim, d_model, n_heads * head_dim, d_model),
                    200, t, muon, [], steps=1, muon_hp=dict(MUON_DEFAULT))


def perhead_mixed(n_heads=32, head_dim=128, d_model=4096):
    """Per-head and whole matrices in one call: the query and key projections
    of a d_model=4096, 32-head layer split per head (64 blocks of 128 x 4096)
    beside the unsplit value and output projections (4096 x 4096 each)."""
    rec = GradRecipe("lowrank", rank=16, decay=0.25, noise_std=1e-3)
    t, muon = [], []
    for name in ("wq", "wk"):
        idx = len(t)
        t.append(_muon_tensor(name, n_heads * head_dim, d_model, rec))
        muon += [MuonView(idx, h * head_dim, head_dim) for h in range(n_heads)]
    for name in ("wv", "wo"):
        muon.append(MuonView(len(t), 0, d_model))
        t.append(_muon_tensor(name, d_model, d_model, rec))
    return Workload("per-head Q/K (%d x %dx%d each) + whole V, O (%dx%d)"
                    % (n_heads, head_dim, d_model, d_model, d_model),
                    201, t, muon, [], steps=1, muon_hp=dict(MUON_DEFAULT))


WORKLOADS = {"c0": config0, "c1": config1, "c2": config2, "c3": config3, "c4": config4,
             "headline": headline,
             # the same matrices, fewer of them: one 4096^2 matrix leaves most
             # of the chip idle (136 Gram tiles against 256 CUs)
             "headline-1": lambda: headline(n=1), "headline-2": lambda: headline(n=2),
             "headline-2-fp32": lambda: headline_fp32(n=2),
             "perhead": perhead, "perhead-mixed": perhead_mixed}

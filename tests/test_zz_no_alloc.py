"""The allocation-free clipped AdamW entry point (adamw_step_clipped_noalloc)
against the workspace one (adamw_step_clipped), through the C ABI: two calls
in a row on the same device, the second on smaller tensors than the first
(the fixed scratch keeps the first call's partial sums, which the second must
not read), each bit-identical to the workspace entry point on a copy of the
same state; and the size limit."""

import pytest
import torch

import muon_step_02_amd as mu
from harness import Handle

pytestmark = pytest.mark.gpu

DEV = "cuda"
HP = dict(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _state(sizes, seed, gdt=torch.float32):
    g = torch.Generator(device=DEV).manual_seed(seed)
    P = [torch.randn(n, generator=g, device=DEV) * 0.02 for n in sizes]
    G = [(torch.randn(n, generator=g, device=DEV) * 0.5).to(gdt) for n in sizes]
    M = [torch.randn(n, generator=g, device=DEV) * 1e-3 for n in sizes]
    V = [torch.rand(n, generator=g, device=DEV) * 1e-4 for n in sizes]
    return P, G, M, V


def _copy(st):
    return tuple([t.clone() for t in ts] for ts in st)


@pytest.mark.parametrize("gdt", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_entry_point_twice(gdt):
    h = Handle.get()
    calls = [([3, 4096, 70000, 1 << 20, 4097] + [999] * 260, 1),  # 1.3 M elements, 265 tensors
             ([5000, 12345, 1], 2)]                               # smaller: 3 tensors
    for sizes, step in calls:
        a = _state(sizes, 10 + step, gdt)
        b = _copy(a)
        hp = mu.adamw_hparams(step=step, **HP)
        ta = [mu.adamw_tensor(*x) for x in zip(*a)]
        tb = [mu.adamw_tensor(*x) for x in zip(*b)]
        na = torch.full((1,), -1.0, device=DEV)
        nb = torch.full((1,), -1.0, device=DEV)
        ws = torch.full((mu.adamw_workspace_size(h, tb),), 255, dtype=torch.uint8, device=DEV)
        mu.adamw_step_clipped_noalloc(h, ta, hp, 1.0, norm_out=na)
        mu.adamw_step_clipped(h, tb, hp, 1.0, ws, norm_out=nb)
        torch.cuda.synchronize()
        assert float(na) > 1.0  # the clip is active
        assert torch.equal(na, nb)
        for xa, xb in zip(a, b):
            for u, v in zip(xa, xb):
                assert torch.equal(u, v)


def test_noalloc_rejects_beyond_its_scratch_and_enqueues_nothing():
    h = Handle.get()
    p = torch.zeros(16, device=DEV)
    before = p.clone()
    big = mu.adamw_tensor(p, p.clone(), p.clone(), p.clone())
    big.numel = (1 << 30) + 1          # 2^18 + 1 chunks of 4096: one too many
    with pytest.raises(mu.MuonError) as e:
        mu.adamw_step_clipped_noalloc(h, [big], mu.adamw_hparams(step=1, **HP), 1.0)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.equal(p, before)
    assert mu.load().muon_status_str(7).startswith(b"problem larger than the fixed device scratch")

"""cp_ring_bwd_noalloc (the backward with its dvec scratch in the library's
own device array, for callers that cannot allocate) against cp_ring_bwd
(dvec in a caller buffer), through the C-ABI: two calls in a row on one
GPU, the second smaller, each bit-identical to cp_ring_bwd (the same
kernels on the same values), so nothing of the first call's scratch
contents reaches the second."""
import pytest
import torch

import context_parallelism_cp_amd as cp
from seeded_inputs import make_qkv

from test_gpu_parity import DEV, announce

pytestmark = pytest.mark.gpu


def _case(S, Hq, Hkv, P, layout, rank, seed):
    q, _, _ = make_qkv(S=S, H=Hq, D=128, seed=seed, dtype=torch.bfloat16)
    _, k, v = make_qkv(S=S, H=Hkv, D=128, seed=seed + 1, dtype=torch.bfloat16)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = cp.cp_ring_fwd(q, k, v, P, layout, rank)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 2)
    dout = torch.randn(out.shape, generator=g).to(torch.bfloat16).to(DEV)
    return q, k, v, out, lse, dout


def _grads(q, k, v, out):
    f32 = dict(device=DEV, dtype=torch.float32)
    return (torch.full(out.shape, float("nan"), **f32),
            torch.full((q.shape[0],) + tuple(k.shape[1:]), float("nan"), **f32),
            torch.full((q.shape[0],) + tuple(k.shape[1:]), float("nan"), **f32))


def test_ring_bwd_noalloc_matches_ring_bwd_twice():
    cases = [(32768, 32, 32, 8, "zigzag", -1, 11),    # 2^20 floats of dvec
             (4096, 8, 2, 4, "striped", 2, 21)]        # then a smaller call
    for S, Hq, Hkv, P, layout, rank, seed in cases:
        announce(f"ring bwd noalloc S={S} Hq={Hq} Hkv={Hkv} P={P} {layout} rank {rank}")
        q, k, v, out, lse, dout = _case(S, Hq, Hkv, P, layout, rank, seed)
        want = cp.cp_ring_bwd(q, k, v, out, lse, dout, P, layout, rank)
        got = _grads(q, k, v, out)
        cp.cp_ring_bwd_noalloc(q, k, v, out, lse, dout, *got, P, layout, rank)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert not torch.isnan(g).any(), name
            assert torch.equal(g, w), f"{name}: max diff {float((g - w).abs().max())}"
        print(f"    bit-identical to cp_ring_bwd", flush=True)


def test_ring_bwd_noalloc_refuses_past_its_array():
    q = torch.zeros(1, device=DEV)
    announce("ring bwd noalloc: 40 heads x 131072 rows of dvec refused")
    t = lambda *s, dt=torch.bfloat16: torch.zeros(*s, device=DEV, dtype=dt)
    S, Hq = 131072, 40
    with pytest.raises(cp.CpError) as e:
        cp.cp_ring_bwd_noalloc(t(S, Hq, 128), t(S, 8, 128), t(S, 8, 128),
                               t(S, Hq, 128, dt=torch.float32), t(Hq, S, dt=torch.float32),
                               t(S, Hq, 128), t(S, Hq, 128, dt=torch.float32),
                               t(S, 8, 128, dt=torch.float32), t(S, 8, 128, dt=torch.float32),
                               8, "zigzag", -1)
    assert e.value.code == cp.CP_ERR_WORKSPACE
    del q

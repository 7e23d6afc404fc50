"""GPU forward corruption: bit-exact against the oracle, small and at 2^28
tokens (sampled canvases plus whole-array statistics)."""
import numpy as np
import pytest

from oracle import corrupt
from tests.dg_harness import GpuModel
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_corrupt_bit_exact_with_model(name):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    cfg = get_config(name, B=3)
    inp = make_inputs(cfg, ["E", "Wq", "Wk", "Wv", "Wo", "x"])
    m = GpuModel(cfg, inp)
    x0 = torch.from_numpy(inp["x"]).cuda()
    out = torch.empty_like(x0)
    kappa = np.array([0.0, 0.37, 1.0], np.float32)
    for seed in [0, 1, 2**40 + 3]:
        dg.dg_corrupt(m.model, x0, kappa, seed, out)
        torch.cuda.synchronize()
        want = corrupt(inp["x"], kappa, seed, cfg.V)
        assert np.array_equal(out.cpu().numpy(), want)
    m.close()


# C % 4 == 0 takes the 16-byte quad kernel (4, 36, 260, and 1001 x 12 = 3003
# quads: three blocks of 1024, the last one partial); odd C and C % 4 == 2 the
# pair kernel
@pytest.mark.parametrize("B,C", [(5, 1), (5, 33), (5, 34), (5, 256), (5, 4), (5, 36), (5, 260), (1001, 12)])
def test_corrupt_batch_ragged_and_in_place(B, C):
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    V = 1000
    rng = np.random.default_rng(C)
    x0 = rng.integers(0, V, (B, C)).astype(np.int32)
    kappa = rng.random(B).astype(np.float32)
    xd = torch.from_numpy(x0).cuda()
    kd = torch.from_numpy(kappa).cuda()
    dg.dg_corrupt_batch(xd, kd, B, C, V, 99, xd)          # in place
    torch.cuda.synchronize()
    assert np.array_equal(xd.cpu().numpy(), corrupt(x0, kappa, 99, V))


@pytest.mark.parametrize("B,C", [(0, 256), (4, 0)])
def test_corrupt_batch_empty(B, C):
    # no tokens: nothing is read or written, and the call succeeds
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    x0 = torch.zeros(16, dtype=torch.int32, device="cuda")
    out = torch.full((16,), 7, dtype=torch.int32, device="cuda")
    kd = torch.zeros(max(B, 1), dtype=torch.float32, device="cuda")
    dg.dg_corrupt_batch(x0, kd, B, C, 1000, 3, out)
    torch.cuda.synchronize()
    assert (out == 7).all()


def test_corrupt_batch_unaligned_rows():
    # arrays 4 bytes past a 16-byte boundary: the quad kernel does not apply
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    B, C, V = 9, 20, 5000
    rng = np.random.default_rng(7)
    x0 = rng.integers(0, V, (B, C)).astype(np.int32)
    kappa = rng.random(B).astype(np.float32)
    buf = torch.zeros(B * C + 8, dtype=torch.int32, device="cuda")
    obuf = torch.zeros(B * C + 8, dtype=torch.int32, device="cuda")
    xd = buf[1:1 + B * C].view(B, C)
    od = obuf[3:3 + B * C].view(B, C)
    xd.copy_(torch.from_numpy(x0).cuda())
    assert xd.data_ptr() % 16 != 0 and od.data_ptr() % 16 != 0
    dg.dg_corrupt_batch(xd, torch.from_numpy(kappa).cuda(), B, C, V, 5, od)
    torch.cuda.synchronize()
    assert np.array_equal(od.cpu().numpy(), corrupt(x0, kappa, 5, V))
    assert (obuf[:3] == 0).all() and (obuf[3 + B * C:] == 0).all()


def test_corrupt_batch_at_bandwidth_size():
    import torch
    import discrete_diffusion_decoding_dg_amd as dg
    B, C, V = 1 << 20, 256, 262144
    print("[gpu] corrupt 2^28 tokens", flush=True)
    g = torch.Generator(device="cuda").manual_seed(0)
    x0 = torch.randint(0, V, (B, C), dtype=torch.int32, device="cuda", generator=g)
    kap = torch.rand((B,), dtype=torch.float32, device="cuda", generator=g)
    out = torch.empty_like(x0)
    dg.dg_corrupt_batch(x0, kap, B, C, V, 2024, out)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 12345, B // 2, B - 1])
    x0s = x0[torch.from_numpy(sel).cuda()].cpu().numpy()
    ks = kap[torch.from_numpy(sel).cuda()].cpu().numpy()
    want = corrupt(x0s, ks, 2024, V, canvas_ids=sel)
    assert np.array_equal(out[torch.from_numpy(sel).cuda()].cpu().numpy(), want)
    # whole-array statistics: kept fraction matches mean(kappa) + (1 - mean)/V
    kept = (out == x0).sum(dim=1).double()
    frac = (kept.sum() / (B * C)).item()
    expect = (kap.double().mean() + (1 - kap.double().mean()) / V).item()
    assert abs(frac - expect) < 5e-4

"""The measurement kernels behind the benchmark's measured peaks: the copy
moves every byte, the LDS probe reads the slots it should (its checksum against
a numpy recomputation), and the clock probe reports a plausible clock."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def test_copy_moves_every_byte(dev):
    from sphere_rasterization_amd import peaks as PK
    g = torch.Generator(device="cpu").manual_seed(7)
    for n in (4 * 3, 4 * 1000 + 4, (1 << 22) + 12):            # ragged tails past the unrolled rounds
        src = torch.randn(n, generator=g).to(dev)
        dst = torch.full_like(src, float("nan"))
        PK.copy(torch, dev, src, dst, blocks=64, reps=1)
        assert torch.equal(src.cpu(), dst.cpu())


def test_lds_probe_checksum(dev):
    from sphere_rasterization_amd import peaks as PK
    blocks, iters = 3, 11
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
    PK.lds(torch, dev, sink, blocks, iters)
    t = np.arange(256, dtype=np.int64)
    g, w = (t >> 4) & 3, t >> 6
    slot = np.arange(1024, dtype=np.uint64)
    s = np.stack([slot, 3 * slot, 5 * slot, 7 * slot], axis=1) & 0xFFFFFFFF
    a = np.zeros(256, np.uint64)
    b = np.zeros(256, np.uint64)
    for k in range(iters):
        for u in range(8):
            v = s[(k * 64 + u * 8 + g * 2 + w * 256) & 1023]
            a = (a + v[:, 0] + v[:, 1]) & 0xFFFFFFFF
            b = (b + v[:, 2] + v[:, 3]) & 0xFFFFFFFF
    want = (a ^ b).astype(np.uint32)
    got = sink.cpu().numpy().view(np.uint32).reshape(blocks, 256)
    assert (got == want[None, :]).all()


def test_clock_probe_is_plausible(dev):
    from sphere_rasterization_amd import peaks as PK
    for fp64 in (False, True):
        mhz, fma = PK.valu(torch, dev, blocks=512, iters=2000, fp64=fp64)
        assert 300.0 < mhz < 4000.0
        # at most two FMAs per lane per cycle on every SIMD of 256 CUs, at a clock below 4 GHz
        assert 0.0 < fma < 256 * 128 * 4.0e9

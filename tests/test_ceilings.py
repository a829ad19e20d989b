"""The chip-ceiling kernels through the C ABI: what they compute is checked
where it has a value (the copy is bit-exact, the read is deterministic), and
the timing loops return finite results and sane clock counts.  These kernels
compute nothing of attention; the bench reports the attention kernels
against them."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _fa():
    import io_aware_exact_03_amd as fa
    return fa


def test_copy_is_exact():
    fa = _fa()
    g = torch.Generator(device="cpu").manual_seed(11)
    src = torch.randint(-2**31, 2**31 - 1, (3 * (1 << 20) + 4,), generator=g, dtype=torch.int32).cuda()
    dst = torch.zeros_like(src)
    fa.ceiling_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_read_is_deterministic():
    """Every 16-byte chunk is folded into exactly one lane's XOR, so the XOR
    of the per-lane results is the XOR of every word of the source."""
    import numpy as np
    fa = _fa()
    src = torch.arange(1 << 22, dtype=torch.int32, device="cuda") * 2654435761
    a = fa.ceiling_read(src).clone()
    b = fa.ceiling_read(src)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    got = np.bitwise_xor.reduce(a.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert got == want


def test_mfma_loop_and_clocks():
    fa = _fa()
    sink, clk = fa.ceiling_mfma(8, 8, 50, clocks=True)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    c = clk.view(8, 2).cpu()
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()
    # shader clock over the 100 MHz constant clock: a plausible frequency
    ghz = (c[:, 0].double() / c[:, 1].double() * 0.1)
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), ghz


def test_valu_loop_counts():
    fa = _fa()
    exp_c, fma_c, mix_c = (fa.ceiling_valu(m, 2000) for m in (0, 1, 2))
    # 64 and 96 instructions per iteration take at least a few cycles each;
    # the mix issues both sets, so it takes at least as long as either
    assert exp_c > 64 and fma_c > 96
    assert mix_c >= 0.95 * max(exp_c, fma_c)


def test_mix_loop_runs_and_is_finite():
    """The forward-step mix loop in its three modes: finite sink values, and
    the same values from two launches (no atomics, fixed order)."""
    fa = _fa()
    for mode in (0, 1, 2):
        a = fa.ceiling_mix(mode, 4, 20)[0].clone()
        b, clk = fa.ceiling_mix(mode, 4, 20, clocks=True)
        torch.cuda.synchronize()
        assert torch.isfinite(a).all(), mode
        assert torch.equal(a, b), mode
        c = clk.view(4, 2).cpu()
        assert (c > 0).all(), mode

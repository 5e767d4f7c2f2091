"""Ceiling probes through the C ABI: the dense bf16 MFMA loop, the NT
contraction core (alone and with an output epilogue) and the HBM copy give
rates inside what the part can physically reach (published dense bf16 peak
about 2.5 PFLOP/s, HBM3E 8 TB/s), the core computes the product it times, and
the copy probe copies."""
import pytest

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 flop per clock
PEAK_HBM_GBS = 8000.0


@pytest.fixture(scope="module")
def M():
    import matrix_orthogonalizing_optimizer_muon_amd as mod
    return mod


def test_mfma_probe_rate_is_physical(M):
    tflops, flops = M.probe_mfma_bf16(iters=4000)
    print(f"mfma probe: {tflops:.1f} TFLOP/s", flush=True)
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == 2 * cus * 4 * 4000 * 4 * 32768
    assert 0.2 * PEAK_BF16_TFLOPS < tflops <= 1.02 * PEAK_BF16_TFLOPS


def test_mfma_probe_with_random_operands(M):
    # the same flop count; random operands switch more bits, so under the
    # part's power limit the rate is no higher than with fixed operands
    fixed, _ = M.probe_mfma_bf16(iters=40000)
    rnd, flops = M.probe_mfma_bf16(iters=40000, random_operands=True)
    print(f"mfma probe: fixed operands {fixed:.1f}, random operands {rnd:.1f} TFLOP/s", flush=True)
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == 2 * cus * 4 * 40000 * 4 * 32768
    assert 0.2 * PEAK_BF16_TFLOPS < rnd <= 1.05 * fixed


def test_hbm_copy_probe_copies_and_rate_is_physical(M):
    import torch
    n = (1 << 30) // 4 + 4   # 1 GiB + 16 bytes: the grid-stride tail runs too
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.zeros(n, dtype=torch.int32, device="cuda")
    gbs = M.probe_hbm_copy(dst, src, reps=3)
    torch.cuda.synchronize()
    print(f"copy probe: {gbs:.0f} GB/s", flush=True)
    assert torch.equal(dst, src)
    assert 0.1 * PEAK_HBM_GBS < gbs <= 1.05 * PEAK_HBM_GBS
    with pytest.raises(ValueError):
        M.probe_hbm_copy(dst[:-4], src)
    with pytest.raises(M.MuonError):
        M.probe_hbm_copy(dst[4:], dst[:-4])   # overlapping buffers


def test_nt_core_probe_with_output_writes_the_product(M):
    """The output epilogue of the core probe stores P Q^T rounded to bf16 once
    from its fp32 accumulators: against the fp64 product rounded to bf16, every
    element within one bf16 ulp and nearly all equal (positive operands, so
    only values on a rounding boundary can differ); the column pass stores
    exactly the transpose, with plain and with nontemporal stores."""
    import torch
    g = torch.Generator().manual_seed(6)
    m, n, k = 512, 768, 1024
    P = torch.rand(m, k, generator=g).to(torch.bfloat16)
    Q = torch.rand(n, k, generator=g).to(torch.bfloat16)
    ref = (P.double() @ Q.double().t()).to(torch.bfloat16).float()
    Pd, Qd = P.cuda(), Q.cuda()
    for mode in (1, 2, 3):
        C = torch.full((m, n), float("nan"), device="cuda", dtype=torch.bfloat16)
        CT = torch.full((n, m), float("nan"), device="cuda", dtype=torch.bfloat16) if mode >= 2 else None
        tf = M.probe_nt_out_bf16(Pd, Qd, C, CT, mode=mode, reps=2)
        got = C.float().cpu()
        ulp = torch.abs(ref) * 2.0 ** -7
        exact = float((got == ref).double().mean())
        print(f"nt core probe, output mode {mode}: {tf:.1f} TFLOP/s, {exact:.4%} equal to the rounded "
              f"fp64 product", flush=True)
        assert 0 < tf <= 1.02 * PEAK_BF16_TFLOPS
        assert bool(torch.all(torch.abs(got - ref) <= ulp)), "an element is more than one ulp off"
        assert exact >= 0.99
        if CT is not None:
            assert torch.equal(CT.cpu().view(torch.int16), C.cpu().t().contiguous().view(torch.int16))
    C = torch.empty((m, n), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(M.MuonError):   # no such mode
        M.probe_nt_out_bf16(Pd, Qd, C, None, mode=0)
    with pytest.raises(ValueError):    # the transposed copy needs CT
        M.probe_nt_out_bf16(Pd, Qd, C, None, mode=2)


def test_nt_core_probe_checksum_and_rate(M):
    """The NT core probe computes every 256x256 tile of P Q^T: its checksum is
    the sum of all entries of the product, which equals the dot product of the
    column sums of P and Q (positive operands: no cancellation)."""
    import torch
    g = torch.Generator().manual_seed(5)
    m, n, k = 512, 768, 1024
    P = torch.rand(m, k, generator=g).to(torch.bfloat16)
    Q = torch.rand(n, k, generator=g).to(torch.bfloat16)
    want = float((P.double().sum(0) * Q.double().sum(0)).sum())
    tf, cs = M.probe_nt_bf16(P.cuda(), Q.cuda(), reps=2)
    print(f"nt core probe: {tf:.1f} TFLOP/s, checksum {cs:.6e} against {want:.6e}", flush=True)
    assert 0 < tf <= 1.02 * PEAK_BF16_TFLOPS
    assert abs(cs - want) <= 1e-4 * abs(want), (cs, want)
    with pytest.raises(M.MuonError):   # k not a multiple of 64
        M.probe_nt_bf16(P[:, :1000].contiguous().cuda(), Q[:, :1000].contiguous().cuda())
    with pytest.raises(M.MuonError):   # m not a multiple of 256
        M.probe_nt_bf16(P[:500].contiguous().cuda(), Q.cuda())

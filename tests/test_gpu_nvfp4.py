"""GPU parity of the NVFP4 -> MXFP4 expert-weight re-encoding (lmoe_nvfp4_to_mxfp4)
against the CPU oracle: codes and scales are integers decided from the same FP32
values, so the comparison is bit-exact.

* Seeded inputs with the structure of NVFP4 expert weights (E2M1 codes, UE4M3
  block scales per 16 over a spread of exponents, one FP32 scale per matrix),
  plus rows of edge cases: scale bytes with the top bit set, subnormal scales,
  NaN scales, all-zero blocks, halves with scales far apart, matrix scales that
  are negative, tiny (subnormal products), non-finite, or large enough that
  some products overflow.
* The same conversion in place (out_codes = codes).
* Full size: all 256 experts' gate/up matrices (256 x 8192 x 4096) converted
  in one call, checked on a seeded sample of rows.
* End to end: NVFP4 weights converted on the GPU drive the MXFP4 forward, which
  matches the oracle run on the oracle's own conversion.
"""
import numpy as np
import pytest
import torch

import latent_moe_layer_router_amd as lmoe
import oracle
import synth
from tests import harness as H
from tests.pins import tiny
from tests.test_gpu_parity import run_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def nvfp4_inputs(M, R, C, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(M, R, C // 2), dtype=np.uint8)
    s16 = rng.integers(0x18, 0x60, size=(M, R, C // 16)).astype(np.uint8)   # 2^-4 .. 2^4
    g = np.array([0.0123, -3.5, 1.2e-38, 2.0e35, np.inf, 1.0][:M], np.float32)
    if R >= 8:
        s16[:, 0] |= 0x80                                         # top bit set (ignored)
        s16[:, 1] = rng.integers(0, 8, size=(M, C // 16))          # subnormal scales
        s16[:, 2, ::5] = 0x7F                                     # NaN scales
        codes[:, 3, :16] = rng.choice([0x00, 0x08, 0x80, 0x88], size=(M, 16))   # zero blocks
        s16[:, 4, 0::2], s16[:, 4, 1::2] = 0x08, 0x70             # halves 2^-6 and 2^7 apart
        s16[:, 5] = 0x7E                                          # 448: overflows with g = 2e35
        codes[:, 6] &= 0x77                                       # non-negative codes only
    return codes, s16, g


def gpu_convert(codes, s16, g, in_place=False):
    M, R, half = codes.shape
    C = 2 * half
    dc = torch.from_numpy(codes).to(DEV)
    ds = torch.from_numpy(s16).to(DEV)
    dg = torch.from_numpy(g).to(DEV)
    oc = dc if in_place else torch.empty_like(dc)
    os_ = torch.empty((M, R, C // 32), dtype=torch.uint8, device=DEV)
    lmoe.lmoe_nvfp4_to_mxfp4(dc.data_ptr(), ds.data_ptr(), dg.data_ptr(), M, R, C, oc.data_ptr(),
                             os_.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return oc.cpu().numpy(), os_.cpu().numpy()


def assert_same(got, want, what):
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} {what} differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("M,R,C", [(6, 16, 512), (1, 8, 32), (2, 33, 4096)])
def test_nvfp4_requant_bitexact(M, R, C):
    H.say(f"[gpu] nvfp4 -> mxfp4: {M} x {R} x {C}")
    codes, s16, g = nvfp4_inputs(M, R, C, seed=M * 1000 + R)
    want_c, want_s = oracle.default().nvfp4_to_mxfp4(codes, s16, g)
    got_c, got_s = gpu_convert(codes, s16, g)
    assert_same(got_s, want_s, "scales")
    assert_same(got_c, want_c, "code bytes")
    # the edge rows and matrix scales did what they are for
    if R >= 8:
        assert (want_s[:, 2] == 255).any() and (want_s[0, 5] != 255).all()
        if M >= 4:
            assert (want_s[3, 5] == 255).any()          # 6 * 448 * 2e35 overflows FP32
        if M >= 5:
            assert (want_s[4] == 255).all()             # matrix scale inf


def test_nvfp4_requant_in_place():
    codes, s16, g = nvfp4_inputs(4, 24, 1024, seed=5)
    want_c, want_s = oracle.default().nvfp4_to_mxfp4(codes, s16, g)
    H.say("[gpu] nvfp4 -> mxfp4 in place")
    got_c, got_s = gpu_convert(codes, s16, g, in_place=True)
    assert_same(got_s, want_s, "scales")
    assert_same(got_c, want_c, "code bytes")


def test_nvfp4_requant_full_size_sampled():
    """All 256 experts' gate/up weights (2F = 8192 rows of Dp = 4096) in one call;
    a seeded sample of 64 rows is compared with the oracle."""
    M, R, C = 256, 8192, 4096
    H.say(f"[gpu] nvfp4 -> mxfp4 full size {M} x {R} x {C}: generating")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(17)
    dc = torch.randint(0, 256, (M, R, C // 2), dtype=torch.uint8, device=DEV, generator=gen)
    ds = torch.randint(0x18, 0x60, (M, R, C // 16), dtype=torch.uint8, device=DEV, generator=gen)
    dg = (torch.rand(M, device=DEV, generator=gen) * 2.0 ** -6 + 2.0 ** -8).float()
    oc = torch.empty_like(dc)
    os_ = torch.empty((M, R, C // 32), dtype=torch.uint8, device=DEV)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    lmoe.lmoe_nvfp4_to_mxfp4(dc.data_ptr(), ds.data_ptr(), dg.data_ptr(), M, R, C, oc.data_ptr(),
                             os_.data_ptr(), s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    nbytes = M * R * (C // 2 + C // 16 + C // 2 + C // 32)
    H.say(f"[gpu]   converted in {ms:.2f} ms ({nbytes / ms / 1e6:.0f} GB/s of codes and scales moved)")
    rng = np.random.default_rng(3)
    rows = rng.choice(M * R, size=64, replace=False)
    mi, ri = torch.from_numpy(rows // R).to(DEV), torch.from_numpy(rows % R).to(DEV)
    codes = dc[mi, ri].cpu().numpy()[:, None, :]
    s16 = ds[mi, ri].cpu().numpy()[:, None, :]
    g = dg[mi].cpu().numpy()
    want_c, want_s = oracle.default().nvfp4_to_mxfp4(codes, s16, g)
    assert_same(os_[mi, ri].cpu().numpy()[:, None, :], want_s, "scales")
    assert_same(oc[mi, ri].cpu().numpy()[:, None, :], want_c, "code bytes")
    del dc, ds, oc, os_
    torch.cuda.empty_cache()


def test_nvfp4_checkpoint_through_mxfp4_forward():
    """NVFP4 expert weights, re-encoded on the GPU, run the MXFP4 forward and
    match the oracle on the oracle's own re-encoding (Dp = F = 1024, E = 4)."""
    w = tiny(T=100, D=256, Dp=1024, F_=1024, E=4, k=2, seed=230, act=synth.BF16, expert_w=synth.MXFP4)
    wts = synth.dense_weights(w)
    O = oracle.default()
    for name, sname, rows, cols, seed in (("w_gate_up", "s_gate_up", 2 * w.F, w.Dp, 1),
                                          ("w_down", "s_down", w.Dp, w.F, 2)):
        codes, s16, _ = nvfp4_inputs(w.E, rows, cols, seed)
        s16 = np.random.default_rng(seed).integers(0x30, 0x40, size=s16.shape).astype(np.uint8)
        g = np.full(w.E, cols ** -0.5 / 4, np.float32)       # weights of about N(0, 1/cols)
        want_c, want_s = O.nvfp4_to_mxfp4(codes, s16, g)
        got_c, got_s = gpu_convert(codes, s16, g)
        assert_same(got_s, want_s, f"{name} scales")
        assert_same(got_c, want_c, f"{name} code bytes")
        wts[name] = got_c
        wts[sname] = got_s
    run_case(w, wts=wts)

"""The C-ABI library without a GPU: it loads, exports every function that
include/lmoe.h declares, and its host-side checks answer without touching a device."""
import ctypes
import os
import re

import pytest

import latent_moe_layer_router_amd as lmoe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lmoe.h")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmoe_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(lmoe.EXPORTS)


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(lmoe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_null_destroy():
    for s in (lmoe.LMOE_OK, lmoe.LMOE_E_INVAL, lmoe.LMOE_E_UNSUPPORTED, lmoe.LMOE_E_NOMEM, lmoe.LMOE_E_HIP):
        assert lmoe.lmoe_status_str(s)
    lmoe.lmoe_destroy(None)


def test_workspace_bytes_full_size():
    cfg = lmoe.make_config(8192, 4096, 4096, 256, 8, 16384)
    n = lmoe.lmoe_workspace_bytes(cfg)
    # intermediates: P fp32 (256 MiB); xp one row per token (128 MiB, bf16); H, Y
    # in sorted order (1 GiB each); u (128 MiB), sum-of-squares partials, logits,
    # routing arrays
    assert 2.5 * 2 ** 30 < n < 2.65 * 2 ** 30


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 2, lmoe.LMOE_E_INVAL),
    ("d_model", 100, lmoe.LMOE_E_UNSUPPORTED),
    ("d_pooled", 0, lmoe.LMOE_E_UNSUPPORTED),
    ("n_experts", 1025, lmoe.LMOE_E_UNSUPPORTED),
    ("top_k", 0, lmoe.LMOE_E_UNSUPPORTED),
    ("top_k", 17, lmoe.LMOE_E_UNSUPPORTED),
    ("act_dtype", lmoe.LMOE_MXFP4, lmoe.LMOE_E_UNSUPPORTED),
    ("expert_wdtype", lmoe.LMOE_MXFP8_E4M3, lmoe.LMOE_E_UNSUPPORTED),
    ("d_ff", 4096 + 512, lmoe.LMOE_E_UNSUPPORTED),     # with MXFP4 experts: K % 1024
    ("max_tokens", 0, lmoe.LMOE_E_INVAL),
    ("eps_pool", -1.0, lmoe.LMOE_E_INVAL),
    ("eps_expert", float("nan"), lmoe.LMOE_E_INVAL),
    ("flags", 4, lmoe.LMOE_E_INVAL),
])
def test_config_validation(field, value, status):
    cfg = lmoe.make_config(8192, 4096, 4096, 256, 8, 128, experts="mxfp4" if field == "d_ff" else None)
    setattr(cfg, field, value)
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_workspace_bytes(cfg)
    assert e.value.status == status
    assert lmoe.lmoe_last_error()


@pytest.mark.parametrize("kw", [
    dict(act="f32"),                         # packed weights are bf16
    dict(experts="mxfp4"),                   # MXFP4 experts keep their layout
    dict(Dp=4096 + 128),                     # d_pooled not a multiple of 256
    dict(F=4096 + 64),                       # d_ff not a multiple of 128
    dict(max_tokens=1 << 16),                # 32-bit offsets of H at max_tokens
])
def test_packed_experts_flag_validation(kw):
    """The packed-layout flag is accepted only where every expert GEMM runs on
    the kernels that read that layout."""
    D, Dp, F = 8192, kw.pop("Dp", 4096), kw.pop("F", 4096)
    T = kw.pop("max_tokens", 128)
    lmoe.lmoe_workspace_bytes(lmoe.make_config(D, 4096, 4096, 256, 8, 128, packed=True))   # accepted
    cfg = lmoe.make_config(D, Dp, F, 256, 8, T, packed=True, **kw)
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_workspace_bytes(cfg)
    assert e.value.status == lmoe.LMOE_E_UNSUPPORTED
    assert "packed" in lmoe.lmoe_last_error()


@pytest.mark.parametrize("args", [
    (1, 32, 64), (1, 64, 96),                # rows, cols not multiples of 64
    (-1, 64, 64), (1, -64, 64),              # negative sizes
])
def test_pack_experts_rejects_bad_sizes(args):
    """Checked on the host before anything is enqueued (no GPU needed)."""
    m, r, c = args
    buf = 1 << 24
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_pack_experts(buf, buf + (1 << 20), m, r, c)
    assert e.value.status == lmoe.LMOE_E_INVAL


def test_pack_experts_rejects_bad_pointers():
    base = 1 << 24
    n = 2 * 64 * 128 * 2                     # bytes of two 64 x 128 matrices
    for src, dst in [(0, base), (base, 0), (base + 8, base + (1 << 20)), (base, base + (1 << 20) + 2),
                     (base, base + n - 16), (base + 16, base)]:
        with pytest.raises(lmoe.LmoeError) as e:
            lmoe.lmoe_pack_experts(src, dst, 2, 64, 128)
        assert e.value.status == lmoe.LMOE_E_INVAL, (src, dst)
    lmoe.lmoe_pack_experts(0, 0, 0, 64, 64)      # empty: nothing to do


def test_create_rejects_null_weights_before_touching_a_device():
    cfg = lmoe.make_config(256, 128, 128, 8, 2, 64)
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_create(cfg, lmoe.lmoe_weights())
    assert e.value.status == lmoe.LMOE_E_INVAL


def test_forward_rejects_null_handle():
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward(None, 0, 0, 1, 0)
    assert e.value.status == lmoe.LMOE_E_INVAL


def test_mxfp4_config():
    """MXFP4 experts: bf16 activations only; the expert inputs are held as MXFP8
    codes + scales (1 + 1/32 bytes per value instead of 2)."""
    bf = lmoe.lmoe_workspace_bytes(lmoe.make_config(8192, 4096, 4096, 256, 8, 16384))
    mx = lmoe.lmoe_workspace_bytes(lmoe.make_config(8192, 4096, 4096, 256, 8, 16384, experts="mxfp4"))
    T, A = 16384, 16384 * 8      # xp: one row per token; H: one per assignment
    assert bf - mx == pytest.approx((T * 4096 + A * 4096) * (2 - 1 - 1 / 32), abs=2 ** 20)
    cfg = lmoe.make_config(8192, 4096, 4096, 256, 8, 128, act="f32", experts="mxfp4")
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_workspace_bytes(cfg)
    assert e.value.status == lmoe.LMOE_E_UNSUPPORTED


@pytest.mark.parametrize("n,ptr", [(33, 16), (-32, 16), (64, 0)])
def test_mx_quantize_rejects_bad_arguments(n, ptr):
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_mx_quantize_e4m3(ptr, n, ptr, ptr)
    assert e.value.status == lmoe.LMOE_E_INVAL
    lmoe.lmoe_mx_quantize_e4m3(0, 0, 0, 0)     # empty: nothing to do


@pytest.mark.parametrize("args", [
    (1, 1, 48),                      # cols not a multiple of 32
    (-1, 1, 32), (1, -1, 32),        # negative sizes
])
def test_nvfp4_to_mxfp4_rejects_bad_sizes(args):
    """Checked on the host before anything is enqueued (no GPU needed)."""
    m, r, c = args
    buf = 1 << 20
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_nvfp4_to_mxfp4(buf, buf + 4096, buf + 8192, m, r, c, buf, buf + 16384)
    assert e.value.status == lmoe.LMOE_E_INVAL


def test_nvfp4_to_mxfp4_rejects_bad_pointers():
    base = 1 << 24
    codes, s16, g, oc, os_ = base, base + (1 << 16), base + (1 << 17), base + (1 << 18), base + (1 << 19)
    cases = [
        (0, s16, g, oc, os_),            # NULL codes
        (codes, s16, g, oc, 0),          # NULL out_scales
        (codes + 8, s16, g, oc, os_),    # codes misaligned
        (codes, s16 + 1, g, oc, os_),    # scales16 misaligned
        (codes, s16, g + 2, oc, os_),    # global_scale misaligned
        (codes, s16, g, codes + 16, os_),  # out_codes overlaps codes without being it
        (codes, s16, g, oc, codes + 4),  # out_scales inside codes
        (codes, s16, g, oc, s16),        # out_scales inside scales16
    ]
    for c in cases:
        with pytest.raises(lmoe.LmoeError) as e:
            lmoe.lmoe_nvfp4_to_mxfp4(c[0], c[1], c[2], 2, 4, 64, c[3], c[4])
        assert e.value.status == lmoe.LMOE_E_INVAL, c
    lmoe.lmoe_nvfp4_to_mxfp4(0, 0, 0, 0, 4, 64, 0, 0)   # empty: nothing to do


def test_forward_noalloc_checks_before_touching_a_device():
    """lmoe_forward_noalloc checks its configuration, weights and token count on
    the host: a T whose workspace exceeds the static scratch is refused (the
    limit at the full decode shape is T = 301), as are bad pointers, before any
    device call."""
    cfg = lmoe.make_config(8192, 4096, 4096, 256, 8, 1024)
    base = 1 << 30
    w = lmoe.lmoe_weights(*[base + (i << 20) for i in (0, 0, 1, 2, 3, 0, 4, 0, 5, 6)])
    w.b_router = None
    w.s_gate_up = None
    w.s_down = None
    x, out = base + (64 << 20), base + (256 << 20)
    for T in (302, 1024):
        with pytest.raises(lmoe.LmoeError) as e:
            lmoe.lmoe_forward_noalloc(cfg, w, x, out, T)
        assert e.value.status == lmoe.LMOE_E_INVAL and "scratch" in lmoe.lmoe_last_error()
    c = lmoe.make_config(8192, 4096, 4096, 256, 8, 301)
    assert lmoe.lmoe_workspace_bytes(c) <= lmoe.LMOE_NOALLOC_SCRATCH_BYTES
    c.max_tokens = 302
    assert lmoe.lmoe_workspace_bytes(c) > lmoe.LMOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward_noalloc(cfg, w, x, out, 2048)           # beyond max_tokens
    assert e.value.status == lmoe.LMOE_E_INVAL
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward_noalloc(cfg, lmoe.lmoe_weights(), x, out, 16)
    assert e.value.status == lmoe.LMOE_E_INVAL
    with pytest.raises(lmoe.LmoeError) as e:
        lmoe.lmoe_forward_noalloc(cfg, w, x + 8, out, 16)        # misaligned x
    assert e.value.status == lmoe.LMOE_E_INVAL
    lmoe.lmoe_forward_noalloc(cfg, w, x, out, 0)                  # T = 0: nothing to do

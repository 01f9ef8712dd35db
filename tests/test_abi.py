"""The C ABI library: it loads, exports every declared symbol, shares torch's HIP
runtime, and rejects bad arguments before launching anything (no GPU needed)."""

import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (load torch's HIP runtime first, as the binding does)

from causal_sliding_window_amd import swattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swattn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("swattn_fwd", "swattn_bwd", "swattn_decode", "swattn_fwd_f32", "swattn_bwd_f32",
              "swattn_decode_f32", "swattn_bwd_workspace_size", "swattn_decode_workspace_size",
              "swattn_status_string", "swattn_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = swattn.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_single_hip_runtime_in_process():
    swattn.lib()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) <= 1, paths


def test_status_strings_and_version():
    assert swattn.status_string(0) == "SWATTN_OK"
    assert swattn.status_string(1) == "SWATTN_ERR_INVALID_ARG"
    assert swattn.status_string(2) == "SWATTN_ERR_UNSUPPORTED"
    assert swattn.status_string(3) == "SWATTN_ERR_HIP"
    assert swattn.status_string(99) == "SWATTN_ERR_UNKNOWN"
    assert swattn.lib().swattn_version() >= 100


def test_workspace_sizes():
    assert swattn.swattn_bwd_workspace_size(8, 6, 2048, 128) == 8 * 6 * 2048 * 4
    assert swattn.swattn_bwd_workspace_size(1, 1, 3, 64) == 256
    assert swattn.swattn_bwd_workspace_size(1, 1, 3, 96) == 0
    assert swattn.swattn_bwd_workspace_size(0, 1, 3, 64) == 0
    # 4096 rows in chunks of 128 -> 32 splits; a 1024 window -> 8
    assert swattn.swattn_decode_workspace_size(32, 12, 128, 4096, -1) == 32 * 12 * 32 * 129 * 4
    assert swattn.swattn_decode_workspace_size(32, 12, 128, 4096, 1024) == 32 * 12 * 8 * 129 * 4
    assert swattn.swattn_decode_workspace_size(1, 1, 128, 4096, 0) == 0


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced (arguments fail first)
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 64, 0, 1.0, None), 1),        # window == 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 8, 64, -1, 1.0, None), 1),       # B == 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, -3, 64, -1, 1.0, None), 1),      # T < 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 96, -1, 1.0, None), 2),       # D unsupported
    ((None, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 64, -1, 1.0, None), 1),       # NULL q
    ((FAKE, FAKE, FAKE, FAKE, None, 1, 1, 8, 64, -1, 1.0, None), 1),       # NULL lse
    ((FAKE, MISALIGNED, FAKE, FAKE, FAKE, 1, 1, 8, 64, -1, 1.0, None), 1),  # misaligned k
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1 << 23, 128, -1, 1.0, None), 2),  # 2 GiB sequence
])
def test_fwd_argument_errors(args, expect):
    lib = swattn.lib()
    assert lib.swattn_fwd(*args) == expect
    assert lib.swattn_fwd_f32(*args) == expect


def test_bwd_and_decode_argument_errors():
    lib = swattn.lib()
    p9 = [FAKE] * 9
    assert lib.swattn_bwd(*p9, 1, 1, 8, 64, 0, 1.0, FAKE, None) == 1
    assert lib.swattn_bwd(*p9, 1, 1, 8, 64, -1, 1.0, None, None) == 1     # NULL workspace
    assert lib.swattn_bwd_f32(*p9, 1, 1, 8, 32, -1, 1.0, FAKE, None) == 2
    p6 = [FAKE] * 6
    assert lib.swattn_decode(*p6, 1, 1, 128, 0, -1, 1.0, FAKE, None) == 1  # Tmax == 0
    assert lib.swattn_decode(*p6, 1, 1, 128, 16, 0, 1.0, FAKE, None) == 1  # window == 0
    assert lib.swattn_decode(*p6, 1, 1, 80, 16, -1, 1.0, FAKE, None) == 2
    p6n = [FAKE, FAKE, FAKE, None, FAKE, FAKE]                               # NULL seqlens
    assert lib.swattn_decode_f32(*p6n, 1, 1, 128, 16, -1, 1.0, FAKE, None) == 1


def test_gqa_entry_points_declared_and_sized():
    names = declared_functions()
    for n in ("swattn_fwd_gqa", "swattn_bwd_gqa", "swattn_bwd_gqa_workspace_size",
              "swattn_decode_gqa"):
        assert n in names
    ws = swattn.swattn_bwd_gqa_workspace_size
    assert ws(8, 6, 6, 2048, 128) == swattn.swattn_bwd_workspace_size(8, 6, 2048, 128)
    # delta plus float32 dK and dV partials per query head
    assert ws(8, 6, 2, 2048, 128) == 8 * 6 * 2048 * 4 + 2 * 8 * 2048 * 6 * 128 * 4
    assert ws(8, 6, 4, 2048, 128) == 0       # 6 heads do not split into 4 groups
    assert ws(8, 6, 0, 2048, 128) == 0


def test_gqa_argument_errors():
    lib = swattn.lib()
    # q, k, v, o, lse, B, H, Hkv, T, D, window, scale, stream
    assert lib.swattn_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 6, 4, 8, 64, -1, 1.0, None) == 1
    assert lib.swattn_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 6, 0, 8, 64, -1, 1.0, None) == 1
    assert lib.swattn_fwd_gqa(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 6, 3, 8, 96, -1, 1.0, None) == 2
    p9 = [FAKE] * 9
    assert lib.swattn_bwd_gqa(*p9, 1, 6, 5, 8, 64, -1, 1.0, FAKE, None) == 1
    assert lib.swattn_bwd_gqa(*p9, 1, 6, 3, 8, 64, 0, 1.0, FAKE, None) == 1
    p6 = [FAKE] * 6
    assert lib.swattn_decode_gqa(*p6, 1, 6, 4, 128, 16, -1, 1.0, FAKE, None) == 1
    assert lib.swattn_decode_gqa(*p6, 1, 6, 2, 80, 16, -1, 1.0, FAKE, None) == 2


def test_prologue_argument_errors():
    """QK-norm + rotary prologue: sizes, D, base and eps are checked before any launch."""
    lib = swattn.lib()
    p4, p6 = [FAKE] * 4, [FAKE] * 6
    # q, k, q_out, k_out, pos_offset, B, T, H, Hkv, D, base, eps, stream
    assert lib.swattn_qk_norm_rope(*p4, None, 1, 8, 0, 0, 64, 1e4, 1e-6, None) == 1  # no side
    assert lib.swattn_qk_norm_rope(*p4, None, 1, 8, -1, 2, 64, 1e4, 1e-6, None) == 1
    # keys only (H = 0): q may be NULL, k may not
    assert lib.swattn_qk_norm_rope(None, None, None, None, None, 1, 8, 0, 2, 64, 1e4, 1e-6,
                                   None) == 1
    assert lib.swattn_qk_norm_rope(*p4, None, 0, 8, 6, 2, 64, 1e4, 1e-6, None) == 1
    assert lib.swattn_qk_norm_rope(*p4, None, 1, 8, 6, 2, 96, 1e4, 1e-6, None) == 2
    assert lib.swattn_qk_norm_rope(*p4, None, 1, 8, 6, 2, 64, 0.0, 1e-6, None) == 1
    assert lib.swattn_qk_norm_rope(*p4, None, 1, 8, 6, 2, 64, 1e4, -1.0, None) == 1
    assert lib.swattn_qk_norm_rope(*p4, None, 1, 8, 6, 2, 64, float("nan"), 1e-6, None) == 1
    assert lib.swattn_qk_norm_rope(None, FAKE, FAKE, FAKE, None, 1, 8, 6, 2, 64, 1e4, 1e-6,
                                   None) == 1
    assert lib.swattn_qk_norm_rope_bwd(*p6, None, 1, 8, 6, 2, 128, 1e4, float("inf"), None) == 1
    assert lib.swattn_qk_norm_rope_bwd(*p6, None, 1, 0, 6, 2, 128, 1e4, 1e-6, None) == 1


def test_binding_rejects_host_tensors():
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(swattn.SwattnError):
        swattn.fwd(q, q, q)


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf"), -0.0])
def test_scale_must_be_positive_and_finite(scale):
    """Every call that takes a softmax scale rejects one that is not a positive finite
    number, before anything launches (the kernels apply the mask before the scale)."""
    lib = swattn.lib()
    p5, p6, p8, p9 = [FAKE] * 5, [FAKE] * 6, [FAKE] * 8, [FAKE] * 9
    assert lib.swattn_fwd(*p5, 1, 1, 8, 64, -1, scale, None) == 1
    assert lib.swattn_fwd_f32(*p5, 1, 1, 8, 64, 4, scale, None) == 1
    assert lib.swattn_fwd_gqa(*p5, 1, 6, 3, 8, 64, -1, scale, None) == 1
    assert lib.swattn_bwd(*p9, 1, 1, 8, 64, -1, scale, FAKE, None) == 1
    assert lib.swattn_bwd_f32(*p9, 1, 1, 8, 64, -1, scale, FAKE, None) == 1
    assert lib.swattn_bwd_gqa(*p9, 1, 6, 3, 8, 64, -1, scale, FAKE, None) == 1
    assert lib.swattn_bwd_dq(*p8, 1, 1, 8, 64, -1, scale, None) == 1
    assert lib.swattn_bwd_dkdv(*p8, 1, 1, 8, 64, -1, scale, None) == 1
    assert lib.swattn_bwd_dq_f32(*p8, 1, 1, 8, 64, -1, scale, None) == 1
    assert lib.swattn_bwd_dkdv_f32(*p8, 1, 1, 8, 64, -1, scale, None) == 1
    assert lib.swattn_decode(*p6, 1, 1, 128, 16, -1, scale, FAKE, None) == 1
    assert lib.swattn_decode_f32(*p6, 1, 1, 128, 16, 8, scale, FAKE, None) == 1
    assert lib.swattn_decode_gqa(*p6, 1, 6, 2, 128, 16, -1, scale, FAKE, None) == 1
    # q, k_new, v_new, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, Tq, D, Tmax, W, scale
    assert lib.swattn_prefill(*p8, 1, 2, 2, 8, 64, 16, -1, scale, None) == 1



def test_noalloc_decode_checks_before_touching_the_gpu():
    """swattn_decode_noalloc validates its arguments and its scratch bound before any HIP
    call, so all of these return without a GPU."""
    lib = swattn.lib()
    p6 = [FAKE] * 6
    assert swattn.status_string(4) == "SWATTN_ERR_TOO_LARGE"
    # q, k_cache, v_cache, seqlens, o, lse, B, H, D, Tmax, window, scale, stream
    assert lib.swattn_decode_noalloc(*p6, 1, 1, 128, 16, 0, 1.0, None) == 1     # window 0
    assert lib.swattn_decode_noalloc(*p6, 1, 1, 96, 16, -1, 1.0, None) == 2     # D
    assert lib.swattn_decode_noalloc(*p6, 1, 1, 128, 16, -1, 0.0, None) == 1    # scale
    assert lib.swattn_decode_noalloc(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 1, 128, 16, -1, 1.0,
                                     None) == 1                                   # NULL seqlens
    # 32 x 12 heads, 20000-row caches: 157 splits of 129 floats each, 31 MB > 16 MiB
    assert swattn.swattn_decode_workspace_size(32, 12, 128, 20000, -1) > 16 << 20
    assert lib.swattn_decode_noalloc(*p6, 32, 12, 128, 20000, -1, 1.0, None) == 4
    # the decode workload (4096-row caches) fits: 6.3 MB
    assert swattn.swattn_decode_workspace_size(32, 12, 128, 4096, -1) <= 16 << 20


def test_fused_rope_argument_errors():
    """swattn_fwd_rope / swattn_bwd_rope check sizes, scale, base and eps before any launch."""
    lib = swattn.lib()
    p5 = [FAKE] * 5
    # q, k_rope, v, o, lse, q_rope, pos_offset, B, H, T, D, window, scale, base, eps, stream
    assert lib.swattn_fwd_rope(*p5, None, None, 1, 2, 8, 64, 0, 0.1, 1e4, 1e-6, None) == 1
    assert lib.swattn_fwd_rope(*p5, None, None, 1, 2, 8, 96, -1, 0.1, 1e4, 1e-6, None) == 2
    assert lib.swattn_fwd_rope(*p5, None, None, 1, 2, 8, 64, -1, 0.1, 0.0, 1e-6, None) == 1
    assert lib.swattn_fwd_rope(*p5, None, None, 1, 2, 8, 64, -1, 0.1, 1e4, -1.0, None) == 1
    assert lib.swattn_fwd_rope(*p5, MISALIGNED, None, 1, 2, 8, 64, -1, 0.1, 1e4, 0.0, None) == 1
    p11 = [FAKE] * 11
    # q, k, q_rope, k_rope, v, o, dO, lse, dq, dk, dv, pos_offset, B, H, T, D, window, scale,
    # base, eps, workspace, stream
    assert lib.swattn_bwd_rope(*p11, None, 1, 2, 8, 64, -1, 0.0, 1e4, 1e-6, FAKE, None) == 1
    assert lib.swattn_bwd_rope(*p11, None, 1, 2, 8, 64, -1, 0.1, float("nan"), 1e-6, FAKE,
                               None) == 1
    assert lib.swattn_bwd_rope(*p11, None, 1, 2, 8, 64, -1, 0.1, 1e4, 1e-6, None, None) == 1
    # the _gqa forms: Hkv after H, checked like swattn_fwd_gqa / swattn_bwd_gqa
    assert lib.swattn_fwd_rope_gqa(*p5, None, None, 1, 6, 4, 8, 64, -1, 0.1, 1e4, 1e-6,
                                   None) == 1
    assert lib.swattn_fwd_rope_gqa(*p5, None, None, 1, 6, 0, 8, 64, -1, 0.1, 1e4, 1e-6,
                                   None) == 1
    assert lib.swattn_fwd_rope_gqa(*p5, None, None, 1, 6, 3, 8, 96, -1, 0.1, 1e4, 1e-6,
                                   None) == 2
    assert lib.swattn_fwd_rope_gqa(*p5, None, None, 1, 6, 3, 8, 64, -1, 0.1, 1e4, float("inf"),
                                   None) == 1
    assert lib.swattn_bwd_rope_gqa(*p11, None, 1, 6, 5, 8, 64, -1, 0.1, 1e4, 1e-6, FAKE,
                                   None) == 1
    assert lib.swattn_bwd_rope_gqa(*p11, None, 1, 6, 3, 8, 64, -1, 0.1, 0.0, 1e-6, FAKE,
                                   None) == 1
    assert lib.swattn_bwd_rope_gqa(*p11, None, 1, 6, 3, 8, 64, -1, 0.1, 1e4, 1e-6, None,
                                   None) == 1


def test_probe_argument_errors():
    """The measurement probes check their arguments before anything is enqueued."""
    lib = swattn.lib()
    assert lib.swattn_probe_mfma(None, 1, 1, None) == 1                     # NULL out
    assert lib.swattn_probe_mfma(MISALIGNED, 1, 1, None) == 1               # misaligned out
    assert lib.swattn_probe_mfma(FAKE, 0, 1, None) == 1                     # no workgroups
    assert lib.swattn_probe_mfma(FAKE, (1 << 20) + 1, 1, None) == 1         # too many
    assert lib.swattn_probe_mfma(FAKE, 1, 0, None) == 1                     # no iterations
    assert lib.swattn_probe_mfma(FAKE, 1, (1 << 24) + 1, None) == 1         # past exactness
    assert lib.swattn_probe_read(None, 16, FAKE, 1, None) == 1              # NULL src
    assert lib.swattn_probe_read(FAKE, 16, None, 1, None) == 1              # NULL out
    assert lib.swattn_probe_read(ctypes.c_void_p((1 << 20) + 8), 16, FAKE, 1, None) == 1
    assert lib.swattn_probe_read(FAKE, 0, FAKE, 1, None) == 1               # nothing to read
    assert lib.swattn_probe_read(FAKE, 24, FAKE, 1, None) == 1              # not 16-byte pieces
    assert lib.swattn_probe_read(FAKE, 16, FAKE, 0, None) == 1              # no workgroups

"""The C-ABI library loads on the CPU, exports every symbol include/flexq.h declares,
and rejects bad arguments on the host before any HIP call (no kernel runs here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flexq.h")
LIB = os.path.join(ROOT, "w6a6_w6a8_integer_amd", "libflexq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libflexq.so not built")

SUCCESS, INVALID, UNSUPPORTED, LAUNCH = 0, 1, 2, 3
A16 = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced on error paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flexq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def flexq():
    import torch  # noqa: F401  (the HIP runtime must be the one torch loads)
    import w6a6_w6a8_integer_amd as fq
    return fq.lib()


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ["flexq_pack_w6", "flexq_quant_act", "flexq_gemm_w6ax"]:
        assert n in names


def test_every_declared_symbol_is_exported(flexq):
    out = subprocess.check_output(["nm", "-D", "--defined-only", LIB]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    import w6a6_w6a8_integer_amd as fq
    assert set(declared_functions()) == set(fq.SIGNATURES)


def test_peak_measurements_are_exported_and_check_arguments(flexq):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "flexq_peaks.h")).read(),
                  flags=re.S)
    names = set(re.findall(r"\b(flexq_[a-z0-9_]+)\s*\(", text))
    import w6a6_w6a8_integer_amd as fq
    assert names == set(fq.PEAK_SIGNATURES)
    out = subprocess.check_output(["nm", "-D", "--defined-only", LIB]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert names <= exported
    # argument errors return before any HIP call
    assert flexq.flexq_peak_hbm_read(None, 16, A16, None) == -1
    assert flexq.flexq_peak_hbm_read(A16, 24, 2 * A16, None) == -1
    assert flexq.flexq_peak_hbm_read(A16 + 8, 16, 2 * A16, None) == -1
    assert flexq.flexq_peak_mfma_i8(0, 0, A16, 2 * A16, None) == -1
    assert flexq.flexq_peak_mfma_i8(10, 5, A16, 2 * A16, None) == -1
    assert flexq.flexq_peak_mfma_i8(10, 0, None, 2 * A16, None) == -1
    assert flexq.flexq_peak_mfma_i8_rescale(0, A16, 2 * A16, None) == -1
    assert flexq.flexq_peak_mfma_i8_rescale(1 << 25, A16, 2 * A16, None) == -1
    assert flexq.flexq_peak_mfma_i8_rescale(10, A16, None, None) == -1
    assert flexq.flexq_peak_mfma_i8_rescale_waves() == 256 * 8     # 256 CUs without a GPU


def test_versions_and_status_strings(flexq):
    assert flexq.flexq_abi_version() == 1
    for s in range(4):
        assert flexq.flexq_status_string(s).decode().startswith("FLEXQ_")
    assert b"unknown" in flexq.flexq_status_string(99)
    assert flexq.flexq_packed_w6_bytes(4096, 4096) == 4096 * 4096 * 3 // 4
    assert flexq.flexq_packed_w6_bytes(16, 8) == 0
    assert flexq.flexq_packed_w6_bytes(0, 128) == 0


def test_pack_w6_rejects_bad_arguments(flexq):
    f = flexq.flexq_pack_w6
    assert f(None, 16, 128, 128, 2 * A16, 3 * A16, None) == INVALID
    assert f(A16, 16, 128, 128, None, 3 * A16, None) == INVALID
    assert f(A16, -16, 128, 128, 2 * A16, 3 * A16, None) == INVALID
    assert f(A16, 16, 0, 128, 2 * A16, 3 * A16, None) == INVALID
    assert f(A16, 16, 128, 64, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 16, 192, 128, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 24, 128, 128, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16 + 8, 16, 128, 128, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 16, 128, 128, 2 * A16 + 4, 3 * A16, None) == UNSUPPORTED
    # output overlapping the input
    assert f(A16, 16, 128, 128, A16 + 16, 3 * A16, None) == INVALID
    # empty weight: nothing to do, no pointer is looked at
    assert f(None, 0, 128, 128, None, None, None) == SUCCESS


def test_quant_act_rejects_bad_arguments(flexq):
    f = flexq.flexq_quant_act
    assert f(A16, 4, 128, 128, 7, 2 * A16, 3 * A16, None) == INVALID
    assert f(None, 4, 128, 128, 6, 2 * A16, 3 * A16, None) == INVALID
    assert f(A16, 4, 128, 128, 6, 2 * A16, None, None) == INVALID
    assert f(A16, -1, 128, 128, 6, 2 * A16, 3 * A16, None) == INVALID
    assert f(A16, 4, 100, 128, 6, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 4, 128, 32, 8, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16 + 2, 4, 128, 128, 6, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 4, 128, 128, 6, 2 * A16 + 4, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 4, 128, 128, 6, 2 * A16, 3 * A16 + 2, None) == UNSUPPORTED
    assert f(A16, 4, 128, 128, 6, A16 + 256, 3 * A16, None) == INVALID  # q_a inside x
    assert f(None, 0, 128, 128, 8, None, None, None) == SUCCESS
    assert f(A16, 1 << 21, 128, 128, 6, 2 * A16, 3 * A16, None) == UNSUPPORTED  # M limit


def test_a6_packed_entry_points_reject_bad_arguments(flexq):
    assert flexq.flexq_packed_a6_bytes(4, 4096) == 4 * 4096 * 3 // 4
    assert flexq.flexq_packed_a6_bytes(1, 8) == 0
    assert flexq.flexq_packed_a6_bytes(0, 128) == 0
    q = flexq.flexq_quant_act_a6_packed
    assert q(None, 4, 128, 128, 2 * A16, 3 * A16, None) == INVALID
    assert q(A16, 4, 128, 128, None, 3 * A16, None) == INVALID
    assert q(A16, 4, 128, 128, 2 * A16, None, None) == INVALID
    assert q(A16, -1, 128, 128, 2 * A16, 3 * A16, None) == INVALID
    assert q(A16, 4, 100, 128, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert q(A16, 4, 128, 64, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert q(A16 + 2, 4, 128, 128, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert q(A16, 4, 128, 128, 2 * A16 + 4, 3 * A16, None) == UNSUPPORTED
    assert q(A16, 4, 128, 128, 2 * A16, 3 * A16 + 2, None) == UNSUPPORTED
    assert q(A16, 4, 128, 128, A16 + 512, 3 * A16, None) == INVALID   # codes inside x
    assert q(A16, 4, 128, 128, 2 * A16, 2 * A16 + 368, None) == INVALID  # s_a inside codes
    assert q(None, 0, 128, 128, None, None, None) == SUCCESS
    g = flexq.flexq_gemm_w6a6_packed
    args = dict(qp=A16, sa=2 * A16, wp=3 * A16, sw=4 * A16, y=5 * A16)

    def call(M=4, N=16, K=128, group=128, **kw):
        a = {**args, **kw}
        return g(a["qp"], a["sa"], a["wp"], a["sw"], M, N, K, group, a["y"], None)

    for k in args:
        assert call(**{k: None}) == INVALID, k
    assert call(M=-1) == INVALID
    assert call(N=-16) == INVALID
    assert call(K=0) == INVALID
    assert call(K=130) == UNSUPPORTED
    assert call(N=24) == UNSUPPORTED
    assert call(group=256) == UNSUPPORTED
    assert call(qp=A16 + 4) == UNSUPPORTED
    assert call(wp=3 * A16 + 4) == UNSUPPORTED
    assert call(y=5 * A16 + 2) == UNSUPPORTED
    assert call(y=A16 + 256) == INVALID       # Y overlaps the packed codes (4 x 96 bytes)
    assert call(M=0, qp=None, y=None) == SUCCESS
    assert call(N=0, wp=None, y=None) == SUCCESS


def test_blocked_entry_points_reject_bad_arguments(flexq):
    assert flexq.flexq_blocked_act_bytes(1, 128) == 16 * 128
    assert flexq.flexq_blocked_act_bytes(17, 4096) == 32 * 4096
    assert flexq.flexq_blocked_act_bytes(16, 100) == 0
    assert flexq.flexq_blocked_act_bytes(0, 128) == 0
    q = flexq.flexq_quant_act_blocked
    assert q(A16, 4, 128, 128, 7, 2 * A16, 3 * A16, None) == INVALID
    assert q(None, 4, 128, 128, 6, 2 * A16, 3 * A16, None) == INVALID
    assert q(A16, 4, 128, 128, 6, None, 3 * A16, None) == INVALID
    assert q(A16, 4, 128, 128, 6, 2 * A16, None, None) == INVALID
    assert q(A16, -1, 128, 128, 6, 2 * A16, 3 * A16, None) == INVALID
    assert q(A16, 4, 100, 128, 6, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert q(A16, 4, 128, 64, 6, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert q(A16 + 2, 4, 128, 128, 6, 2 * A16, 3 * A16, None) == UNSUPPORTED
    assert q(A16, 4, 128, 128, 6, 2 * A16 + 8, 3 * A16, None) == UNSUPPORTED
    assert q(A16, 4, 128, 128, 6, 2 * A16, 3 * A16 + 2, None) == UNSUPPORTED
    assert q(A16, 4, 128, 128, 6, A16 + 512, 3 * A16, None) == INVALID      # codes inside x
    # the codes take 16 rows (2048 bytes) even for 4: scales 2000 bytes in overlap them
    assert q(A16, 4, 128, 128, 6, 2 * A16, 2 * A16 + 2000, None) == INVALID
    assert q(None, 0, 128, 128, 6, None, None, None) == SUCCESS
    g = flexq.flexq_gemm_w6ax_blocked
    args = dict(qb=A16, sa=2 * A16, wp=3 * A16, sw=4 * A16, y=5 * A16)

    def call(M=4, N=16, K=128, group=128, abits=8, **kw):
        a = {**args, **kw}
        return g(a["qb"], a["sa"], a["wp"], a["sw"], M, N, K, group, abits, a["y"], None)

    for k in args:
        assert call(**{k: None}) == INVALID, k
    assert call(abits=5) == INVALID
    assert call(M=-1) == INVALID
    assert call(K=0) == INVALID
    assert call(K=130) == UNSUPPORTED
    assert call(N=24) == UNSUPPORTED
    assert call(qb=A16 + 4) == UNSUPPORTED
    assert call(y=5 * A16 + 2) == UNSUPPORTED
    assert call(y=A16 + 1024) == INVALID      # Y overlaps the 16-row block of codes
    assert call(M=0, qb=None, y=None) == SUCCESS
    assert call(N=0, wp=None, y=None) == SUCCESS


def test_gemm_rejects_bad_arguments(flexq):
    f = flexq.flexq_gemm_w6ax
    g = flexq.flexq_gemm_w6ax_path
    args = dict(qa=A16, sa=2 * A16, wp=3 * A16, sw=4 * A16, y=5 * A16)

    def call(M=4, N=16, K=128, group=128, abits=6, **kw):
        a = {**args, **kw}
        return f(a["qa"], a["sa"], a["wp"], a["sw"], M, N, K, group, abits, a["y"], None)

    assert call(abits=4) == INVALID
    assert call(qa=None) == INVALID
    assert call(sa=None) == INVALID
    assert call(wp=None) == INVALID
    assert call(sw=None) == INVALID
    assert call(y=None) == INVALID
    assert call(M=-1) == INVALID
    assert call(N=-16) == INVALID
    assert call(K=0) == INVALID
    assert call(K=130) == UNSUPPORTED
    assert call(N=24) == UNSUPPORTED
    assert call(group=256) == UNSUPPORTED
    assert call(qa=A16 + 8) == UNSUPPORTED
    assert call(wp=3 * A16 + 4) == UNSUPPORTED
    assert call(sa=2 * A16 + 2) == UNSUPPORTED
    assert call(y=5 * A16 + 2) == UNSUPPORTED
    assert call(y=A16 + 64) == INVALID  # Y overlaps q_a
    assert call(y=3 * A16 + 32) == INVALID  # Y overlaps the packed weight
    assert call(M=0, qa=None, y=None) == SUCCESS
    assert call(N=0, wp=None, y=None) == SUCCESS
    assert g(A16, 2 * A16, 3 * A16, 4 * A16, 4, 16, 128, 128, 6, 8, 5 * A16, None) == INVALID


def test_group_dots_rejects_bad_arguments(flexq):
    f = flexq.flexq_gemm_w6ax_group_dots
    assert f(None, 2 * A16, 4, 16, 128, 128, 3 * A16, None) == INVALID
    assert f(A16, 2 * A16, 4, 16, 128, 128, None, None) == INVALID
    assert f(A16, 2 * A16, 4, 16, 128, 64, 3 * A16, None) == UNSUPPORTED
    assert f(A16, 2 * A16, 4, 16, 128, 128, 3 * A16 + 1, None) == UNSUPPORTED
    assert f(A16, 2 * A16, 4, 16, 128, 128, A16, None) == INVALID
    assert f(None, None, 0, 16, 128, 128, None, None) == SUCCESS


def test_linear_workspace_bytes(flexq):
    f = flexq.flexq_linear_w6ax_workspace_bytes
    # up to 64 rows the codes take whole 16-row blocks (the streaming kernel's layout)
    assert f(1, 128) == 16 * 128 + 4
    assert f(5, 128) == 16 * 128 + 5 * 4
    assert f(3, 8192) == 16 * 8192 + 3 * 64 * 4
    assert f(17, 384) == 32 * 384 + 17 * 3 * 4
    assert f(64, 8192) == 64 * 8192 + 64 * 64 * 4
    # above, M * K row-major codes rounded up to 256 bytes
    assert f(65, 128) == (65 * 128 + 255) // 256 * 256 + 65 * 4
    assert f(4096, 8192) == 4096 * 8192 + 4096 * 64 * 4
    assert f(0, 128) == 0 and f(-3, 128) == 0 and f(8, 100) == 0 and f(8, 0) == 0


def test_linear_rejects_bad_arguments(flexq):
    f = flexq.flexq_linear_w6ax
    ws = 6 * A16
    need = flexq.flexq_linear_w6ax_workspace_bytes(8, 128)

    def call(M=8, N=16, K=128, group=128, abits=6, x=A16, wp=3 * A16, sw=4 * A16, y=5 * A16,
             w=ws, wb=need):
        return f(x, wp, sw, M, N, K, group, abits, w, wb, y, None)

    assert call(abits=5) == INVALID
    assert call(x=None) == INVALID
    assert call(wp=None) == INVALID
    assert call(sw=None) == INVALID
    assert call(y=None) == INVALID
    assert call(M=-1) == INVALID
    assert call(K=0) == INVALID
    assert call(K=192) == UNSUPPORTED
    assert call(N=40) == UNSUPPORTED
    assert call(group=64) == UNSUPPORTED
    assert call(x=A16 + 8) == UNSUPPORTED
    assert call(wp=3 * A16 + 4) == UNSUPPORTED
    assert call(y=5 * A16 + 2) == UNSUPPORTED
    assert call(y=A16 + 64) == INVALID               # Y overlaps X
    assert call(y=3 * A16 + 16) == INVALID           # Y overlaps the packed weight
    assert call(w=None) == INVALID
    assert call(wb=need - 1) == INVALID              # workspace too small
    assert call(w=ws + 8) == UNSUPPORTED             # workspace not 16-byte aligned
    assert call(w=A16 + 16) == INVALID               # workspace overlaps X
    assert call(w=5 * A16) == INVALID                # workspace overlaps Y
    assert call(w=4 * A16) == INVALID                # workspace overlaps s_w
    assert call(M=0, x=None, y=None, w=None, wb=0) == SUCCESS
    assert call(N=0, wp=None, y=None, w=None, wb=0) == SUCCESS


def test_linear_noalloc_rejects_bad_arguments(flexq):
    """The allocation-free one-call layer checks its arguments like flexq_linear_w6ax
    and refuses shapes whose staging exceeds its per-GPU array, all on the host."""
    f = flexq.flexq_linear_w6ax_noalloc
    big = 1 << 32   # fake addresses 4 GiB apart: large shapes do not overlap

    def call(M=8, N=16, K=128, group=128, abits=6, x=A16, wp=3 * A16, sw=4 * A16, y=5 * A16):
        return f(x, wp, sw, M, N, K, group, abits, y, None)

    assert call(abits=7) == INVALID
    assert call(x=None) == INVALID
    assert call(y=None) == INVALID
    assert call(M=-1) == INVALID
    assert call(K=192) == UNSUPPORTED
    assert call(N=40) == UNSUPPORTED
    assert call(x=A16 + 8) == UNSUPPORTED
    assert call(y=A16 + 64) == INVALID               # Y overlaps X
    assert call(M=0, x=None, y=None) == SUCCESS
    limit = 64 << 20
    K = 28672
    M_ok = 2269
    assert flexq.flexq_linear_w6ax_workspace_bytes(M_ok, K) <= limit
    assert flexq.flexq_linear_w6ax_workspace_bytes(M_ok + 1, K) > limit
    assert call(M=M_ok + 1, K=K, x=big, wp=2 * big, sw=3 * big, y=4 * big) == UNSUPPORTED
    assert call(M=8192, K=8192, x=big, wp=2 * big, sw=3 * big, y=4 * big) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    import w6a6_w6a8_integer_amd as fq
    with pytest.raises(TypeError):
        fq.pack_w6(torch.zeros(16, 128, dtype=torch.float16))
    with pytest.raises(TypeError):
        fq.quant_act(torch.zeros(2, 128, dtype=torch.float16), 6)


def _good_gemm_args(M=3, N=32, K=256):
    import torch
    G = K // 128
    return dict(q_a=torch.zeros(M, K, dtype=torch.int8),
                s_a=torch.zeros(G, M, dtype=torch.float32),
                w_packed=torch.zeros(3 * N * K // 16, dtype=torch.int32),
                s_w=torch.zeros(G, N, dtype=torch.float16), N=N, abits=6,
                y=torch.zeros(M, N, dtype=torch.float16))


@pytest.mark.parametrize("field,bad,err,match", [
    ("s_a", ("zeros", (3, 2), "float32"), ValueError, "s_a must have shape"),   # [M][G]
    ("s_a", ("zeros", (2, 3), "float16"), TypeError, "s_a must be"),
    ("s_w", ("zeros", (32, 2), "float16"), ValueError, "s_w must have shape"),  # [N][G]
    ("s_w", ("zeros", (2, 32), "float32"), TypeError, "s_w must be"),
    ("w_packed", ("zeros", (3 * 32 * 256 // 16 - 1,), "int32"), ValueError, "w_packed holds"),
    ("w_packed", ("zeros", (3 * 32 * 256 // 16,), "uint8"), TypeError, "w_packed must be"),
    ("w_packed", ("zeros", (48, 32), "int32"), ValueError, "w_packed must be 1-D"),
    ("y", ("zeros", (3, 16), "float16"), ValueError, "y must have shape"),
    ("y", ("zeros", (3, 32), "float32"), TypeError, "y must be"),
    ("q_a", ("zeros", (3, 200), "int8"), ValueError, "multiple of 128"),
    ("q_a", ("zeros", (768,), "int8"), ValueError, "2-D"),
    ("N", 40, ValueError, "multiple of 16"),
])
def test_binding_checks_every_gemm_argument_before_any_call(field, bad, err, match):
    """Every tensor argument is checked (dtype, exact shape or size, contiguity,
    device) in Python before the C ABI sees a pointer: a wrong buffer raises instead
    of reading or writing out of bounds on the GPU."""
    import torch
    import w6a6_w6a8_integer_amd as fq
    args = _good_gemm_args()
    if isinstance(bad, tuple):
        _, shape, dt = bad
        args[field] = torch.zeros(shape, dtype=getattr(torch, dt))
    else:
        args[field] = bad
    with pytest.raises(err, match=match):
        fq.gemm_w6ax(**args)


def test_binding_checks_shapes_then_device():
    """With every shape right, the remaining objection to host tensors is the device."""
    import torch
    import w6a6_w6a8_integer_amd as fq
    with pytest.raises(TypeError, match="CUDA"):
        fq.gemm_w6ax(**_good_gemm_args())
    a = _good_gemm_args()
    nc = torch.zeros(a["N"], a["q_a"].shape[0], dtype=torch.float16).t()   # non-contiguous
    with pytest.raises(ValueError, match="contiguous"):
        fq.gemm_w6ax(**{**a, "y": nc})


def test_binding_checks_the_other_entry_points():
    import torch
    import w6a6_w6a8_integer_amd as fq
    f16, i8, i32, u8, f32 = torch.float16, torch.int8, torch.int32, torch.uint8, torch.float32
    x = torch.zeros(2, 256, dtype=f16)
    with pytest.raises(ValueError, match="q_a must have shape"):
        fq.quant_act(x, 6, q_a=torch.zeros(2, 128, dtype=i8))
    with pytest.raises(ValueError, match="s_a must have shape"):
        fq.quant_act(x, 6, q_a=torch.zeros(2, 256, dtype=i8), s_a=torch.zeros(2, 2, dtype=f32)[:1])
    with pytest.raises(ValueError, match="s_w must have shape"):
        fq.pack_w6(torch.zeros(32, 256, dtype=f16), s_w=torch.zeros(32, 2, dtype=f16))
    with pytest.raises(ValueError, match="w_packed holds"):
        fq.pack_w6(torch.zeros(32, 256, dtype=f16), w_packed=torch.zeros(10, dtype=i32))
    with pytest.raises(ValueError, match="multiple of 16"):
        fq.pack_w6(torch.zeros(24, 256, dtype=f16))
    wp = torch.zeros(3 * 32 * 256 // 16, dtype=i32)
    sw = torch.zeros(2, 32, dtype=f16)
    with pytest.raises(ValueError, match="workspace holds"):
        fq.linear_w6ax(x, wp, sw, 32, 6, workspace=torch.zeros(16, dtype=u8))
    with pytest.raises(ValueError, match="y must have shape"):
        fq.linear_w6ax(x, wp, sw, 32, 6, y=torch.zeros(32, 2, dtype=f16))
    with pytest.raises(ValueError, match="dots must have shape"):
        fq.gemm_w6ax_group_dots(torch.zeros(2, 256, dtype=i8), wp, 32,
                                dots=torch.zeros(2, 32, 1, dtype=i32))
    with pytest.raises(TypeError, match="CUDA"):
        fq.gemm_w6ax_group_dots(torch.zeros(2, 256, dtype=i8), wp, 32)
    # packed A6 activations: int32 [M][3K/16]
    with pytest.raises(ValueError, match="q_a6p must have shape"):
        fq.quant_act_a6_packed(x, q_a6p=torch.zeros(2, 32, dtype=i32))
    with pytest.raises(TypeError, match="q_a6p must be"):
        fq.quant_act_a6_packed(x, q_a6p=torch.zeros(2, 48, dtype=i8))
    with pytest.raises(TypeError, match="CUDA"):
        fq.quant_act_a6_packed(x)
    qp = torch.zeros(2, 48, dtype=i32)
    sa = torch.zeros(2, 2, dtype=f32)
    with pytest.raises(ValueError, match="multiple of 3"):
        fq.gemm_w6a6_packed(torch.zeros(2, 47, dtype=i32), sa, wp, sw, 32)
    with pytest.raises(ValueError, match="multiple of 128"):
        fq.gemm_w6a6_packed(torch.zeros(2, 45, dtype=i32), sa, wp, sw, 32)
    with pytest.raises(ValueError, match="s_a must have shape"):
        fq.gemm_w6a6_packed(qp, torch.zeros(2, 1, dtype=f32), wp, sw, 32)
    with pytest.raises(ValueError, match="w_packed holds"):
        fq.gemm_w6a6_packed(qp, sa, torch.zeros(10, dtype=i32), sw, 32)
    with pytest.raises(ValueError, match="y must have shape"):
        fq.gemm_w6a6_packed(qp, sa, wp, sw, 32, y=torch.zeros(2, 16, dtype=f16))
    with pytest.raises(TypeError, match="CUDA"):
        fq.gemm_w6a6_packed(qp, sa, wp, sw, 32)
    # blocked activation codes: int8, 1-D, ceil(M/16)*16*K bytes; M and K from s_a
    with pytest.raises(ValueError, match="q_a_blk holds"):
        fq.quant_act_blocked(x, 6, q_a_blk=torch.zeros(2 * 256, dtype=i8))
    with pytest.raises(ValueError, match="q_a_blk must be 1-D"):
        fq.quant_act_blocked(x, 6, q_a_blk=torch.zeros(16, 256, dtype=i8))
    with pytest.raises(TypeError, match="CUDA"):
        fq.quant_act_blocked(x, 6)
    qb = torch.zeros(16 * 256, dtype=i8)
    with pytest.raises(ValueError, match="q_a_blk holds"):
        fq.gemm_w6ax_blocked(torch.zeros(15 * 256, dtype=i8), sa, wp, sw, 32, 6)
    with pytest.raises(TypeError, match="q_a_blk must be"):
        fq.gemm_w6ax_blocked(qb.view(torch.uint8), sa, wp, sw, 32, 6)
    with pytest.raises(ValueError, match="s_w must have shape"):
        fq.gemm_w6ax_blocked(qb, sa, wp, torch.zeros(32, 2, dtype=f16), 32, 6)
    with pytest.raises(ValueError, match="y must have shape"):
        fq.gemm_w6ax_blocked(qb, sa, wp, sw, 32, 6, y=torch.zeros(32, 2, dtype=f16))
    with pytest.raises(TypeError, match="CUDA"):
        fq.gemm_w6ax_blocked(qb, sa, wp, sw, 32, 6)


def test_auto_path_rule(flexq):
    """The automatic kernel choice as flexq.h states it (256 CUs without a GPU): the
    streaming kernel up to one 64-row pass, the tiled kernel above; from 48 rows the
    tiled kernel also where the 64 x 128 tile's grid fills the GPU (at least 384
    128-column tiles)."""
    import w6a6_w6a8_integer_amd as fq
    DEC, PRE = fq.PATH_DECODE, fq.PATH_PREFILL
    assert fq.auto_path(1, 57344, 8192) == DEC
    assert fq.auto_path(32, 57344, 8192) == DEC
    assert fq.auto_path(47, 57344, 8192) == DEC
    assert fq.auto_path(48, 57344, 8192) == PRE       # 448 column tiles
    assert fq.auto_path(64, 57344, 8192) == PRE
    assert fq.auto_path(64, 10240, 8192) == DEC       # 80 column tiles
    assert fq.auto_path(64, 49152, 8192) == PRE       # 384: the boundary
    assert fq.auto_path(64, 49136, 8192) == PRE       # 384 tiles, the last one ragged
    assert fq.auto_path(64, 49024, 8192) == DEC       # 383
    assert fq.auto_path(64, 1 << 24, 128) == PRE
    assert fq.auto_path(65, 16, 128) == PRE
    assert fq.auto_path(65, 57344, 8192) == PRE
    assert fq.auto_path(4096, 16, 128) == PRE
    assert fq.auto_path(0, 128, 128) == DEC


def test_prefill_tile_rule(flexq):
    """The prefill tile choice as flexq.h states it (256 CUs without a GPU)."""
    import w6a6_w6a8_integer_amd as fq
    T256, T128, T64 = fq.PATH_PREFILL_256X128, fq.PATH_PREFILL_128X128, fq.PATH_PREFILL_128X64
    T64R = fq.PATH_PREFILL_64X128
    # LLaMA-2-70B layers
    assert fq.prefill_tile(4096, 57344, 8192) == T256    # 7168 vs 14336 tiles
    assert fq.prefill_tile(1024, 8192, 8192) == T256     # 1 round vs 2
    assert fq.prefill_tile(1024, 10240, 8192) == T256    # 2 rounds vs 3: 2.92 < 3
    assert fq.prefill_tile(256, 8192, 28672) == T64      # 128 tiles of 128 x 128 <= 256
    assert fq.prefill_tile(256, 10240, 8192) == T64      # 160 <= 256
    assert fq.prefill_tile(512, 8192, 8192) == T64       # 256 <= 256: one round either way
    assert fq.prefill_tile(512, 10240, 8192) == T256     # 1 round vs 2
    assert fq.prefill_tile(256, 57344, 8192) == T256     # 2 rounds vs 4
    assert fq.prefill_tile(64, 57344, 8192) == T64R      # 448 column tiles >= 1.5 per CU
    assert fq.prefill_tile(65, 57344, 8192) == T128      # two 64-row blocks: 128-row tiles
    assert fq.prefill_tile(16, 49024, 8192) == T128      # 383 column tiles: the 128-row rule
    # the boundary between the narrow and the square tile
    assert fq.prefill_tile(128, 32768, 256) == T64       # 256 tiles of 128 x 128
    assert fq.prefill_tile(128, 32784, 256) == T128      # 257
    assert fq.prefill_tile(0, 16, 128) == T64


def test_prefill_tail_split_rule(flexq):
    """The tail split as flexq.h states it (256 CUs without a GPU): whole rounds of
    256 x 128 tiles over the leading columns, 128 x 64 tiles for the rest, when the
    stated costs (a round 1.0; 128 x 64 tiles 0.48 up to one per CU, plus 0.6 per
    further CU's worth, at most two per CU) save 5 %."""
    import w6a6_w6a8_integer_amd as fq
    mc = fq.prefill_main_cols
    # 4 x 80 = 320 tiles: 256 in one round (64 column blocks), 2048 columns of
    # 128 x 64 tiles (8 x 32 = 256, one per CU): 1.48 rounds instead of 2
    assert mc(1024, 10240, 8192) == 8192
    assert mc(1024, 27648, 5120) == 24576                # 3 + 0.78 (1.5 per CU) vs 4
    assert mc(1000, 10192, 128) == 8192                  # ragged M and N
    assert mc(520, 33280, 128) == 32768                  # 3 row blocks: 85 column blocks
    assert mc(8192, 1280, 8192) == 1024                  # 64 x 10 tiles: 1 + 0.48 vs 3
    # whole rounds already, or a tail that costs more than it saves
    assert mc(4096, 57344, 8192) == 57344                # 7168 tiles = 28 rounds
    assert mc(1024, 8192, 8192) == 8192                  # 256 tiles, one round
    assert mc(256, 57344, 8192) == 57344                 # 1 + 2 x 0.685 > 2
    assert mc(512, 57344, 8192) == 57344                 # 3 + 1.08 (2 per CU) vs 4
    assert mc(4096, 7168, 8192) == 7168                  # 3 + 1.08 vs 4
    assert mc(2048, 10240, 8192) == 10240                # 2 + 1.08 vs 3
    # other tiles, empty shapes
    assert mc(256, 8192, 28672) == 8192                  # 128 x 64 grid
    assert mc(64, 57344, 8192) == 57344                  # 128 x 128 grid
    assert mc(0, 16, 128) == 16 and mc(16, 0, 128) == 0


def test_gemm_path_values(flexq):
    f = flexq.flexq_gemm_w6ax_path
    for bad in (-1, 8, 9):
        assert f(A16, 2 * A16, 3 * A16, 4 * A16, 4, 16, 128, 128, 6, bad, 5 * A16, None) == INVALID
    for p in range(8):  # every valid path with M = 0: a no-op
        assert f(None, None, 3 * A16, 4 * A16, 0, 16, 128, 128, 6, p, None, None) == SUCCESS


def test_splitk_workspace_bytes(flexq):
    f = flexq.flexq_gemm_w6ax_splitk_workspace_bytes
    assert f(64, 10240, 8192, 2) == 2 * 64 * 10240 * 4
    assert f(5, 16, 128, 1) == 5 * 16 * 4
    assert f(64, 10240, 8192, 0) == 3 * 64 * 10240 * 4     # the plan's 3 slices
    assert f(64, 10240, 8192, 64) == 64 * 64 * 10240 * 4   # K/128 = 64 slices at most
    assert f(64, 10240, 8192, 65) == 0
    assert f(64, 16, 256, 3) == 0                          # more slices than groups
    assert f(0, 16, 128, 1) == 0 and f(4, 0, 128, 1) == 0 and f(4, 16, 100, 1) == 0
    assert f(4, 16, 128, -1) == 0


def test_splitk_rejects_bad_arguments(flexq):
    f = flexq.flexq_gemm_w6ax_splitk
    big = 1 << 32   # fake addresses 4 GiB apart
    M, N, K = 8, 16, 256
    need = flexq.flexq_gemm_w6ax_splitk_workspace_bytes(M, N, K, 2)

    def call(M=M, N=N, K=K, group=128, abits=6, path=2, splits=2, qa=A16, sa=2 * A16,
             wp=3 * A16, sw=4 * A16, ws=big, wb=need, y=2 * big, acc=3 * big):
        return f(qa, sa, wp, sw, M, N, K, group, abits, path, splits, ws, wb, y, acc, None)

    assert call(abits=7) == INVALID
    for p in (0, 1, 6, 8, -1):
        assert call(path=p) == INVALID
    for p in (2, 3, 4, 5, 7):
        assert call(path=p, qa=None) == INVALID          # the path passes, the pointer not
    assert call(splits=-1) == INVALID
    assert call(splits=3) == INVALID                     # K = 256: at most 2 slices
    assert call(K=128 * 80, splits=65) == INVALID        # 64 slices at most
    assert call(qa=None) == INVALID
    assert call(y=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(wb=need - 1) == INVALID                  # workspace too small
    assert call(ws=big + 8) == UNSUPPORTED               # workspace not 16-byte aligned
    assert call(acc=3 * big + 4) == UNSUPPORTED          # accumulator not 16-byte aligned
    assert call(y=2 * big + 2) == UNSUPPORTED
    assert call(K=200) == UNSUPPORTED
    assert call(N=24) == UNSUPPORTED
    assert call(group=64) == UNSUPPORTED
    assert call(ws=A16) == INVALID                       # workspace overlaps q_a
    assert call(ws=4 * A16) == INVALID                   # workspace overlaps s_w
    assert call(acc=big + 64) == INVALID                 # accumulator overlaps the workspace
    assert call(acc=2 * big) == INVALID                  # accumulator overlaps Y
    assert call(acc=3 * A16) == INVALID                  # accumulator overlaps the weights
    assert call(y=big) == INVALID                        # Y overlaps the workspace
    assert call(M=0, qa=None, y=None, ws=None, wb=0) == SUCCESS
    assert call(N=0, wp=None, y=None, ws=None, wb=0) == SUCCESS


def test_splitk_plan_rule(flexq):
    """The slice plan on the LLaMA-2-70B layers (256 CUs without a GPU): split on
    narrow layers from 64 tokens up to a few hundred, never at 32 tokens or fewer,
    never on gate_up (its grid of tiles already fills the GPU), and not on o at 64
    tokens, where the streaming kernel on blocked codes is predicted as fast."""
    import w6a6_w6a8_integer_amd as fq
    T256, T128 = fq.PATH_PREFILL_256X128, fq.PATH_PREFILL_128X128
    L = {"qkv": (10240, 8192), "o": (8192, 8192), "gate_up": (57344, 8192), "down": (8192, 28672)}
    expect = {("qkv", 64): (3, T128), ("qkv", 128): (3, T128), ("qkv", 256): (3, T256),
              ("o", 128): (4, T128), ("o", 256): (4, T256),
              ("down", 64): (4, T128), ("down", 128): (4, T128), ("down", 256): (4, T256),
              ("down", 512): (2, T256)}
    for name, (N, K) in L.items():
        for M in (1, 16, 32, 64, 128, 256, 512, 1024, 4096):
            S, tile = fq.splitk_plan(M, N, K)
            if (name, M) in expect:
                assert (S, tile) == expect[(name, M)], (name, M, S, tile)
            else:
                assert S == 1, (name, M, S)
                assert tile == fq.prefill_tile(M, N, K)
    assert fq.splitk_plan(0, 16, 128) == (1, fq.PATH_PREFILL_128X64)
    assert fq.splitk_plan(64, 16, 128)[0] == 1           # one group: nothing to split


def test_splitk_plan_weighs_the_streaming_kernel(flexq):
    """At 33-64 tokens the plan splits only where split-K beat the weight-streaming
    kernel on blocked codes when both were timed on MI355X (20 launches, rotating
    weights; 256 CUs assumed without a GPU): the streaming kernel keeps the o-like
    layers and the narrow layers up to 48 tokens, split-K takes the long-K layers and
    70B qkv from 56 tokens."""
    import w6a6_w6a8_integer_amd as fq
    cases = {  # (N, K): {M: split?}
        (10240, 8192): {48: False, 56: True, 64: True},      # 70B qkv
        (8192, 8192): {33: False, 64: False},                # 70B o
        (8192, 28672): {48: False, 56: True, 64: True},      # 70B down
        (4096, 4096): {33: False, 64: False},                # 7B o
        (12288, 4096): {64: False},                          # 7B qkv
        (5120, 13824): {33: True, 64: True},                 # 13B down
        (8192, 1024): {33: False, 64: False},                # 70B o, 8-way share
        (8192, 3584): {64: False},                           # 70B down, 8-way share
        (7168, 8192): {64: False},                           # 70B gate_up, 8-way share
        (1280, 8192): {64: True},                            # 70B qkv, 8-way share
        (16384, 4096): {40: False, 64: False},
    }
    for (N, K), want in cases.items():
        for M, split in want.items():
            S, _ = fq.splitk_plan(M, N, K)
            assert (S > 1) == split, (N, K, M, S)

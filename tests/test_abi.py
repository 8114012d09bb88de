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
    assert g(A16, 2 * A16, 3 * A16, 4 * A16, 4, 16, 128, 128, 6, 7, 5 * A16, None) == INVALID


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
    assert f(1, 128) == 256 + 4         # q_a 128 B rounded up to 256, then s_a
    assert f(5, 128) == 768 + 5 * 4
    assert f(3, 8192) == 24576 + 3 * 64 * 4
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


def test_binding_refuses_cpu_tensors():
    import torch
    import w6a6_w6a8_integer_amd as fq
    with pytest.raises(TypeError):
        fq.pack_w6(torch.zeros(16, 128, dtype=torch.float16))
    with pytest.raises(TypeError):
        fq.quant_act(torch.zeros(2, 128, dtype=torch.float16), 6)


def test_auto_path_rule(flexq):
    """The automatic kernel choice as flexq.h states it: the streaming kernel up to
    one 64-row pass, the tiled kernel above, whatever the layer's width."""
    import w6a6_w6a8_integer_amd as fq
    DEC, PRE = fq.PATH_DECODE, fq.PATH_PREFILL
    assert fq.auto_path(1, 57344, 8192) == DEC
    assert fq.auto_path(32, 57344, 8192) == DEC
    assert fq.auto_path(48, 57344, 8192) == DEC
    assert fq.auto_path(64, 10240, 8192) == DEC
    assert fq.auto_path(64, 57344, 8192) == DEC
    assert fq.auto_path(64, 1 << 24, 128) == DEC
    assert fq.auto_path(65, 16, 128) == PRE
    assert fq.auto_path(65, 57344, 8192) == PRE
    assert fq.auto_path(4096, 16, 128) == PRE
    assert fq.auto_path(0, 128, 128) == DEC


def test_prefill_tile_rule(flexq):
    """The prefill tile choice as flexq.h states it (256 CUs without a GPU)."""
    import w6a6_w6a8_integer_amd as fq
    T256, T128, T64 = fq.PATH_PREFILL_256X128, fq.PATH_PREFILL_128X128, fq.PATH_PREFILL_128X64
    # LLaMA-2-70B layers
    assert fq.prefill_tile(4096, 57344, 8192) == T256    # 7168 vs 14336 tiles
    assert fq.prefill_tile(1024, 8192, 8192) == T256     # 1 round vs 2
    assert fq.prefill_tile(1024, 10240, 8192) == T256    # 2 rounds vs 3: 2.92 < 3
    assert fq.prefill_tile(256, 8192, 28672) == T64      # 128 tiles of 128 x 128 <= 256
    assert fq.prefill_tile(256, 10240, 8192) == T64      # 160 <= 256
    assert fq.prefill_tile(512, 8192, 8192) == T64       # 256 <= 256: one round either way
    assert fq.prefill_tile(512, 10240, 8192) == T256     # 1 round vs 2
    assert fq.prefill_tile(256, 57344, 8192) == T256     # 2 rounds vs 4
    assert fq.prefill_tile(64, 57344, 8192) == T128      # 448 tiles: 2 rounds either way
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
    for bad in (-1, 6, 7):
        assert f(A16, 2 * A16, 3 * A16, 4 * A16, 4, 16, 128, 128, 6, bad, 5 * A16, None) == INVALID
    for p in range(6):  # every valid path with M = 0: a no-op
        assert f(None, None, 3 * A16, 4 * A16, 0, 16, 128, 128, 6, p, None, None) == SUCCESS

"""The decode kernels' matrix instructions are inline asm, which the compiler
does not pad with the wait states the hardware requires.  Compile decode.hip
for gfx950 with the library's own flags and check every decode kernel's code
(tests/asm_hazards.py states the rules); also that the chunk loops hold no
scratch traffic (a spill reload there would wait for every copy in flight)."""
import os
import shutil
import subprocess

import pytest

import asm_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    from mla_latent_kv_07_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "decode.s")
    cmd = [hipcc, *B.common_flags(), *B.EXTRA_FLAGS.get("decode.hip", []), "--cuda-device-only",
           "-S", os.path.join(B.CSRC, "decode.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


def test_every_decode_kernel_is_compiled(decode_asm):
    ks = asm_hazards.kernels(decode_asm, r"decode")
    # four bf16 pipelined kernels (and the 128-row one over rows in place),
    # three FP8 pipelined kernels, the FP8 eight-wavefront kernel
    assert sum("decode_pipe_kernel" in k for k in ks) == 5, sorted(ks)
    assert sum("decode_pipe_f8_kernel" in k for k in ks) == 3, sorted(ks)
    assert sum("decode_kernel" in k for k in ks) == 1, sorted(ks)


def test_wait_states_around_matrix_instructions(decode_asm):
    bad = {}
    for name, body in asm_hazards.kernels(decode_asm, r"decode").items():
        v = asm_hazards.check(body)
        if v:
            bad[name] = v[:5]
    assert not bad, bad


def test_no_scratch_in_decode_kernels(decode_asm):
    for name, body in asm_hazards.kernels(decode_asm, r"decode").items():
        assert "scratch_" not in body, name


def test_checker_sees_a_missing_wait_state():
    """The scan flags a VALU write read by the next MFMA, a VALU read of a
    fresh MFMA result (per MFMA kind), and a VALU write reaching an MFMA
    through a branch; and accepts the padded forms."""
    bad = """
	v_cvt_pk_bf16_f32 v4, v0, v1
	v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]
"""
    assert asm_hazards.check(bad)
    ok = bad.replace("v_mfma", "s_nop 1\n\tv_mfma")
    assert not asm_hazards.check(ok)
    after_bf16 = """
	v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0
	s_nop 7
	v_mul_f32_e32 v0, v0, v12
"""
    assert not asm_hazards.check(after_bf16)  # 8 wait states after the bf16 16x16x32
    after_fp8 = after_bf16.replace("v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
                        "v_mfma_scale_f32_16x16x128_f8f6f4 v[0:3], v[4:11], v[12:19], 0, v20, v21")
    assert asm_hazards.check(after_fp8)  # 12 after the FP8 16x16x128
    assert not asm_hazards.check(after_fp8.replace("s_nop 7", "s_nop 7\n\ts_nop 3"))
    assert asm_hazards.check(after_bf16.replace("s_nop 7", "s_nop 6"))
    branchy = """
	v_mov_b32_e32 v5, 0
	s_cbranch_scc1 .LBB0_2
	s_nop 7
.LBB0_2:
	v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]
"""
    assert asm_hazards.check(branchy)

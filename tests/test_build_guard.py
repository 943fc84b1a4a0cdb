"""The build guard for untracked LDS copies (long_context_lm_amd/build.py), on the CPU.

Kernels that copy tiles into LDS with copy16_async_untracked wait for them with counted vmcnt
waits, which hold only while the kernel's own copies and stores are the only vector memory
operations in flight.  The guard reads the device assembly of those files and refuses scratch,
dynamic stacks, flat instructions, and memory instructions in called functions; and it refuses a
vmcnt wait of the compiler's own in a loop block that issues matrix-core products, which would
also wait for the next tile's copies in every iteration.
"""

import shutil

import pytest

from long_context_lm_amd import build as B

PLANTED = """\t.amdhsa_kernel k1
\t\t.amdhsa_private_segment_fixed_size 16
\t\t.amdhsa_uses_dynamic_stack 1
\t.end_amdhsa_kernel
k1:                                      ; @k1
\tflat_load_dword v0, v[2:3]
\tglobal_load_lds_dwordx4 v1, s[4:5]
\ts_swappc_b64 s[30:31], s[6:7]
helper:                                  ; @helper
\tglobal_load_dword v1, v[0:1], off
\tv_add_f32_e32 v0, v0, v1
\ts_setpc_b64 s[30:31]
pure:                                    ; @pure
\tv_exp_f32_e32 v0, v0
\ts_setpc_b64 s[30:31]
"""


def test_guard_flags_each_planted_hazard():
    bad = B.untracked_copy_violations(PLANTED)
    assert "k1: uses scratch (16 bytes per lane)" in bad
    assert "k1: dynamic stack" in bad
    assert "k1: flat instruction flat_load_dword" in bad
    assert "helper (called from a kernel): memory instruction global_load_dword" in bad
    assert not any(b.startswith("pure") for b in bad)  # a callee without memory instructions is fine
    assert not any("global_load_lds" in b for b in bad)  # the kernel's own copies are the counted ones


LOOPS = """k2:                                      ; @k2
\tglobal_load_dwordx4 v[0:3], v[4:5], off
\t;;#ASMSTART
\tglobal_load_lds_dwordx4 v6, s[4:5]
\t;;#ASMEND
.LBB0_1:                                ; =>This Inner Loop Header: Depth=1
\ts_waitcnt vmcnt(3)
\tv_mfma_f32_32x32x16_bf16 v[8:23], v[0:3], v[0:3], v[8:23]
\t;;#ASMSTART
\ts_waitcnt vmcnt(8)
\t;;#ASMEND
.LBB0_2:                                ;   in Loop: Header=BB0_1 Depth=1
\ts_waitcnt vmcnt(0) lgkmcnt(0)
\ts_barrier
\tv_mfma_f32_32x32x16_bf16 v[8:23], v[0:3], v[0:3], v[8:23]
.LBB0_3:                                ;   in Loop: Header=BB0_1 Depth=1
\ts_waitcnt vmcnt(0)
\tv_add_f32_e32 v0, v0, v1
.LBB0_4:
\ts_waitcnt vmcnt(0)
\tv_mfma_f32_32x32x16_bf16 v[8:23], v[0:3], v[0:3], v[8:23]
k3:                                      ; @k3
\tglobal_load_lds_dwordx4 v6, s[4:5]
.LBB1_1:                                ; =>This Inner Loop Header: Depth=1
\ts_waitcnt vmcnt(0)
\tv_mfma_f32_32x32x16_bf16 v[8:23], v[0:3], v[0:3], v[8:23]
"""


def test_loop_wait_check_flags_only_compiler_waits_in_product_loops():
    bad = B.loop_vmcnt_waits(LOOPS)
    assert bad == ["k2 .LBB0_1: s_waitcnt vmcnt(3)"], bad
    # not reported: the kernel's own counted wait (inline asm), a barrier's wait, a loop block
    # without products, a block outside any loop, and a kernel whose copies the compiler tracks
    # (k3: its wait is the one its copy needs)


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_library_sources_pass_the_guard():
    for src in B.UNTRACKED_COPY_SOURCES:
        asm = B._device_asm(src)
        assert B.untracked_copy_violations(asm) == [], src
        assert B.loop_vmcnt_waits(asm) == [], src

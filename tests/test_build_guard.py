"""The build guard for untracked LDS copies (long_context_lm_amd/build.py), on the CPU.

Kernels that copy tiles into LDS with copy16_async_untracked wait for them with counted vmcnt
waits, which hold only while the kernel's own copies and stores are the only vector memory
operations in flight.  The guard reads the device assembly of those files and refuses scratch,
dynamic stacks, flat instructions, and memory instructions in called functions.
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


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_library_sources_pass_the_guard():
    for src in B.UNTRACKED_COPY_SOURCES:
        assert B.untracked_copy_violations(B._device_asm(src)) == [], src

"""The issue-model script finds each attention kernel's main loop in the gfx950 assembly (CPU:
hipcc cross-compiles) and counts one slot's work per wave in it."""

import shutil

import pytest

from long_context_lm_amd import issue_model as M


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_main_loops_hold_one_or_two_slots():
    r = M.floors()
    # matrix-core instructions per wave and slot: S and P V for 64 queries (forward); S, dP' and
    # dQ for 32 queries (query-major); S, dP', dK and dV for 32 keys (key-major)
    assert r["attend_fwd"]["per_wave_slot"]["mfma"] == 32
    assert r["bwd_query"]["per_wave_slot"]["mfma"] == 24
    assert r["bwd_key"]["per_wave_slot"]["mfma"] == 32
    assert r["attend_fwd"]["slots_per_iteration"] == 1
    assert r["bwd_query"]["slots_per_iteration"] == 2   # unrolled twice (two fixed K buffers)
    assert r["bwd_key"]["slots_per_iteration"] == 2     # unrolled twice (two entry buffers)
    # one exponential per score element: 64 (forward: 64 queries x 64 keys / 64 lanes), 32 in
    # each backward pass (32 queries or keys per wave)
    assert r["attend_fwd"]["per_wave_slot"]["trans"] >= 64
    assert r["bwd_query"]["per_wave_slot"]["trans"] >= 32
    assert r["bwd_key"]["per_wave_slot"]["trans"] >= 32

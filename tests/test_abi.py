"""The C ABI on the host: the library loads, exports what include/gca.h declares, and rejects
invalid arguments with the documented status codes before touching the GPU."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from long_context_lm_amd import gca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gca.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, MISALIGNED, HIP = range(6)
FAKE = 0x100000  # never dereferenced: every call below fails validation first


@pytest.fixture(autouse=True)
def _no_launch_attempted():
    """Every call here must fail validation (or be an empty problem) before any HIP call; on a
    machine without a GPU an attempted launch would leave a HIP error behind."""
    yield
    assert gca.load().gca_last_hip_error() == 0, "a test call got past validation to a launch"


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gca_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = gca.load()
    names = declared_functions()
    assert set(gca.EXPORTS) == set(names)  # the binding knows every declared entry point
    for n in names:
        assert hasattr(lib, n), f"libgca.so does not export {n}"


def test_problem_struct_layout_matches_c():
    fields = [f for f, _ in gca.Problem._fields_]
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"gca.h\"\nint main(void){\n"
    prog += 'printf("%zu\\n", sizeof(gca_problem));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof(gca_problem, {f}));\n'
    prog += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(gca.Problem)
    assert out[1:] == [getattr(gca.Problem, f).offset for f in fields]


def good(**kw):
    c = gca.Config(B=2, G=2, H=3, n_q=8, n_kv=8, topk=4, dtype="bf16")
    p = c.problem()
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def ws_size(p, op):
    n = ctypes.c_size_t(0)
    st = gca.load().gca_workspace_size(op, ctypes.byref(p), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, INVALID), ("G", -1, INVALID), ("H", 0, INVALID), ("n_q_chunks", -1, INVALID),
    ("q_chunk_base", -3, INVALID), ("n_kv_chunks", -1, INVALID), ("topk", 0, INVALID),
    ("topk", 17, UNSUPPORTED), ("S", 32, UNSUPPORTED), ("d_head", 128, UNSUPPORTED),
    ("d_lmk", 32, UNSUPPORTED), ("dtype", 7, INVALID), ("use_gumbel", 2, INVALID),
    ("shift", 2, INVALID), ("reserved", 1, INVALID), ("attn_scale", float("inf"), INVALID),
    ("score_scale", float("nan"), INVALID), ("gumbel_tau", -1.0, INVALID),
    ("n_kv_chunks", 1 << 31, UNSUPPORTED), ("n_q_chunks", 1 << 40, UNSUPPORTED),
])
def test_problem_validation(field, value, status):
    p = good(**{field: value})
    lib = gca.load()
    for op in (0, 1, 2, 3, 4):
        assert ws_size(p, op)[0] == status
    z = ctypes.c_void_p(FAKE)
    assert lib.gca_retrieve(ctypes.byref(p), z, z, z, z, None, 0, None) == status
    assert lib.gca_forward(ctypes.byref(p), z, z, z, z, z, z, z, None, 0, None) == status
    assert lib.gca_backward(ctypes.byref(p), z, z, z, z, z, z, z, z, z, z, z, None, 0, None) == status
    assert lib.gca_landmark_backward(ctypes.byref(p), z, z, z, z, z, z, None, 0, None) == status
    assert lib.gca_fetch_chunks(ctypes.byref(p), z, z, z, z, z, z, None) == status
    assert lib.gca_decode_tokens(ctypes.byref(p), 1, z, z, z, z, z, z, None) == status


def test_null_problem_and_bad_op():
    lib = gca.load()
    n = ctypes.c_size_t(0)
    assert lib.gca_workspace_size(0, None, ctypes.byref(n)) == INVALID
    p = good()
    assert lib.gca_workspace_size(6, ctypes.byref(p), ctypes.byref(n)) == INVALID
    assert lib.gca_workspace_size(-1, ctypes.byref(p), ctypes.byref(n)) == INVALID
    assert lib.gca_workspace_size(0, ctypes.byref(p), None) == INVALID
    assert lib.gca_retrieve(None, None, None, None, None, None, 0, None) == INVALID


def test_workspace_sizes():
    # 16K training shape: retrieval fits one block per row; backward needs its index buffers
    c = gca.Config(B=8, G=2, H=12, n_q=256, n_kv=256, topk=8)
    assert gca.workspace_size(gca.OP_RETRIEVE, c) == 0
    assert gca.workspace_size(gca.OP_FORWARD, c) == 0
    bw = gca.workspace_size(gca.OP_BACKWARD, c)
    assert bw >= 2 * 8 * 12 * 256 * 64 * 8 * 4  # per-(token, slot) e values
    # 16M-token history: 256 blocks of 1024 candidates per row and group, 8 partial keys each
    c = gca.Config(B=1, G=2, H=12, n_q=1, n_kv=262144, topk=8, q_chunk_base=262144, shift=0)
    assert gca.workspace_size(gca.OP_RETRIEVE, c) == 2 * 256 * 8 * 8 + 2 * 256 * 8 * 4
    # more rows: blocks grow (cpt doubles) until the grid is at most 2048 waves
    c = gca.Config(B=8, G=2, H=12, n_q=1, n_kv=262144, topk=8, q_chunk_base=262144, shift=0)
    assert gca.workspace_size(gca.OP_RETRIEVE, c) == 16 * 32 * 8 * 8 + 16 * 32 * 8 * 4
    # landmark gradients: the inverse index over every row ({code, value} pairs) and its counts
    c = gca.Config(B=8, G=2, H=12, n_q=256, n_kv=256, topk=8)
    assert gca.workspace_size(gca.OP_LANDMARK_BACKWARD, c) == 8 * 256 * 2 * 256 * 2 * 4 + 8 * 256 * 4
    assert gca.workspace_size(gca.OP_LANDMARK_BACKWARD, gca.Config(B=1, G=1, H=1, n_q=3, n_kv=0, topk=2)) == 0
    # (group, row, slot) codes of the inverse index must fit in int32
    c = gca.Config(B=1, G=4, H=1, n_q=1 << 26, n_kv=1024, topk=16)
    with pytest.raises(gca.GcaError):
        gca.workspace_size(gca.OP_BACKWARD, c)


def test_pointer_checks():
    lib = gca.load()
    p = good()
    z = ctypes.c_void_p(FAKE)
    mis = ctypes.c_void_p(FAKE + 8)
    # retrieval: null and misaligned inputs/outputs
    assert lib.gca_retrieve(ctypes.byref(p), None, z, z, z, None, 0, None) == INVALID
    assert lib.gca_retrieve(ctypes.byref(p), z, z, None, z, None, 0, None) == INVALID
    assert lib.gca_retrieve(ctypes.byref(p), mis, z, z, z, None, 0, None) == MISALIGNED
    assert lib.gca_retrieve(ctypes.byref(p), z, z, ctypes.c_void_p(FAKE + 2), z, None, 0, None) == MISALIGNED
    # forward
    assert lib.gca_forward(ctypes.byref(p), z, z, z, z, z, None, None, None, 0, None) == INVALID
    assert lib.gca_forward(ctypes.byref(p), z, mis, z, z, z, z, z, None, 0, None) == MISALIGNED
    # backward: workspace checks come after the tensors
    st, need = ws_size(p, 2)
    assert st == OK and need > 0
    assert lib.gca_backward(ctypes.byref(p), z, z, z, z, z, z, z, z, z, z, z, z, need - 1, None) == WS_SMALL
    assert lib.gca_backward(ctypes.byref(p), z, z, z, z, z, z, z, z, z, z, z, None, need, None) == INVALID
    assert lib.gca_backward(ctypes.byref(p), z, z, z, z, z, z, z, z, z, z, z,
                            ctypes.c_void_p(FAKE + 16), need, None) == MISALIGNED
    assert lib.gca_backward(ctypes.byref(p), z, z, z, z, z, z, z, z, mis, z, z, z, need, None) == MISALIGNED
    # landmark gradients: tensors, then the workspace
    st, need = ws_size(p, 3)
    assert st == OK and need > 0
    assert lib.gca_landmark_backward(ctypes.byref(p), None, z, z, z, z, z, z, need, None) == INVALID
    assert lib.gca_landmark_backward(ctypes.byref(p), z, z, z, z, mis, z, z, need, None) == MISALIGNED
    assert lib.gca_landmark_backward(ctypes.byref(p), z, z, ctypes.c_void_p(FAKE + 2), z, z, z, z, need,
                                     None) == MISALIGNED
    assert lib.gca_landmark_backward(ctypes.byref(p), z, z, z, z, z, z, z, need - 1, None) == WS_SMALL
    assert lib.gca_landmark_backward(ctypes.byref(p), z, z, z, z, z, z, None, need, None) == INVALID
    # fetch of retrieved chunks: null and misaligned tensors are refused before any HIP call
    assert lib.gca_fetch_chunks(ctypes.byref(p), None, z, z, z, z, z, None) == INVALID
    assert lib.gca_fetch_chunks(ctypes.byref(p), z, None, z, z, z, z, None) == INVALID
    assert lib.gca_fetch_chunks(ctypes.byref(p), z, z, z, z, z, None, None) == INVALID
    assert lib.gca_fetch_chunks(ctypes.byref(p), z, mis, z, z, z, z, None) == MISALIGNED
    assert lib.gca_fetch_chunks(ctypes.byref(p), z, z, z, z, mis, z, None) == MISALIGNED
    assert lib.gca_fetch_chunks(ctypes.byref(p), ctypes.c_void_p(FAKE + 2), z, z, z, z, z, None) == MISALIGNED
    # token-level decode: one query chunk, 1..64 tokens, then the tensors
    one = good(n_q_chunks=1)
    assert lib.gca_decode_tokens(ctypes.byref(p), 1, z, z, z, z, z, z, None) == INVALID  # n_q_chunks = 8
    for n_tok in (0, -1, 65):
        assert lib.gca_decode_tokens(ctypes.byref(one), n_tok, z, z, z, z, z, z, None) == INVALID
    assert lib.gca_decode_tokens(ctypes.byref(one), 1, None, z, z, z, z, z, None) == INVALID
    assert lib.gca_decode_tokens(ctypes.byref(one), 1, z, z, z, z, z, None, None) == INVALID
    assert lib.gca_decode_tokens(ctypes.byref(one), 1, mis, z, z, z, z, z, None) == MISALIGNED
    assert lib.gca_decode_tokens(ctypes.byref(one), 1, z, z, z, ctypes.c_void_p(FAKE + 2), z, z, None) == MISALIGNED
    # sliding-window attention: one group, a query sequence that is its own key sequence, a
    # window that is a positive multiple of 64, bf16
    sw = gca.sw_config(2, 3, 8).problem()
    assert lib.gca_sw_forward(ctypes.byref(sw), 512, None, z, z, z, None, None) == INVALID
    assert lib.gca_sw_forward(ctypes.byref(sw), 512, mis, z, z, z, None, None) == MISALIGNED
    for window in (0, -64, 100):
        assert lib.gca_sw_forward(ctypes.byref(sw), window, z, z, z, z, None, None) == INVALID
    for field, value, status in (("G", 2, INVALID), ("n_kv_chunks", 9, INVALID), ("dtype", 2, INVALID)):
        bad = gca.sw_config(2, 3, 8).problem()
        setattr(bad, field, value)
        assert lib.gca_sw_forward(ctypes.byref(bad), 512, z, z, z, z, None, None) == status
    empty = gca.sw_config(2, 3, 0).problem()
    assert lib.gca_sw_forward(ctypes.byref(empty), 512, None, None, None, None, None, None) == OK
    assert lib.gca_sw_backward(ctypes.byref(empty), 512, *([None] * 9), None, 0, None) == OK
    st, need = ws_size(sw, 4)
    assert st == OK and need == 2 * 3 * 8 * 64 * 8
    args = [z] * 9
    assert lib.gca_sw_backward(ctypes.byref(sw), 512, *args, z, need - 1, None) == WS_SMALL
    assert lib.gca_sw_backward(ctypes.byref(sw), 512, *args, None, need, None) == INVALID
    assert lib.gca_sw_backward(ctypes.byref(sw), 512, *([z] * 5), ctypes.c_void_p(FAKE + 2), *([z] * 3), z, need,
                               None) == MISALIGNED
    assert lib.gca_sw_backward(ctypes.byref(sw), 512, *([z] * 6), None, z, z, z, need, None) == INVALID
    assert lib.gca_sw_backward(ctypes.byref(sw), 96, *args, z, need, None) == INVALID
    # fused layer attention: one group, a window that is a positive multiple of 64; its backward's
    # workspace is the GCA backward's plus 8 bytes per query token
    fz = good(G=1)
    assert lib.gca_fused_forward(ctypes.byref(good(G=2)), 512, *([z] * 10), None) == INVALID
    for window in (0, 32, 100):
        assert lib.gca_fused_forward(ctypes.byref(fz), window, *([z] * 10), None) == INVALID
    assert lib.gca_fused_forward(ctypes.byref(fz), 512, mis, *([z] * 9), None) == MISALIGNED
    assert lib.gca_fused_forward(ctypes.byref(fz), 512, *([z] * 7), None, None, None, None) == INVALID  # no o
    assert lib.gca_fused_forward(ctypes.byref(good(G=1, n_q_chunks=0)), 512, *([None] * 10), None) == OK
    st_f, need_f = ws_size(fz, 5)
    st_b, need_b = ws_size(fz, 2)
    assert st_f == OK and st_b == OK and need_f == need_b + 2 * 3 * 8 * 64 * 8
    fargs = [z] * 18
    assert lib.gca_fused_backward(ctypes.byref(fz), 512, *fargs, need_f - 1, None) == WS_SMALL
    assert lib.gca_fused_backward(ctypes.byref(fz), 512, *fargs[:17], None, need_f, None) == INVALID
    assert lib.gca_fused_backward(ctypes.byref(fz), 96, *fargs, need_f, None) == INVALID
    assert lib.gca_fused_backward(ctypes.byref(fz), 512, *fargs[:8], ctypes.c_void_p(FAKE + 2), *fargs[9:], need_f,
                                  None) == MISALIGNED  # lse_sw: 4-byte alignment
    assert lib.gca_fused_backward(ctypes.byref(fz), 512, *fargs[:9], ctypes.c_void_p(FAKE + 4), *fargs[10:], need_f,
                                  None) == MISALIGNED  # the GCA lse: 16-byte alignment
    # backward beyond the int32 range of inverse-index codes (G * n_q * K >= 2^31)
    big = good(n_q_chunks=1 << 28, n_kv_chunks=1025, H=1, B=1)
    assert lib.gca_backward(ctypes.byref(big), z, z, z, z, z, z, z, z, z, z, z, z, 1 << 40, None) == UNSUPPORTED


def test_empty_problem_is_a_noop_without_gpu():
    lib = gca.load()
    p = good(n_q_chunks=0)
    assert lib.gca_retrieve(ctypes.byref(p), None, None, None, None, None, 0, None) == OK
    assert lib.gca_forward(ctypes.byref(p), None, None, None, None, None, None, None, None, 0, None) == OK
    p = good(n_q_chunks=0, n_kv_chunks=0)
    assert lib.gca_backward(ctypes.byref(p), *([None] * 11), None, 0, None) == OK
    assert lib.gca_landmark_backward(ctypes.byref(p), *([None] * 6), None, 0, None) == OK
    assert lib.gca_fetch_chunks(ctypes.byref(p), *([None] * 6), None) == OK
    p = good(n_q_chunks=0)  # no rows: nothing to fetch, even from a history
    assert lib.gca_fetch_chunks(ctypes.byref(p), *([None] * 6), None) == OK


def test_status_strings_and_error_state():
    lib = gca.load()
    texts = [lib.gca_status_string(s).decode() for s in range(6)]
    assert len(set(texts)) == 6
    assert lib.gca_status_string(99).decode() == "unknown status"
    assert lib.gca_last_hip_error() == 0
    gca.profile_enable(False)
    assert gca.profile_collect() == {}

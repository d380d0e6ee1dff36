"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and its host-side validation returns the documented status
codes without launching anything (no GPU needed)."""
import ctypes
import re

import pytest

import quantized_gemv_argmax_amd as qg

OK, ENULL, ESHAPE, EALIGN, EWS, EDEV, EUNSUP = range(7)
# Fake, never-dereferenced device addresses with the alignment the checks look at.
A, B, C = 0x10000, 0x20000, 0x30000


@pytest.fixture(scope="module")
def L():
    return qg.lib()


def test_loads_and_version(L):
    assert L.qg_abi_version() == 2


def _declarations():
    """(return type, name, parameter list) of every function include/qgemv.h declares,
    parsed from the header text (comments stripped)."""
    text = open(qg.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    out = {}
    for m in re.finditer(r"(?:(?<=[;}])|^)\s*((?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\**)\s*([a-z_][a-z_0-9]*)\s*"
                         r"\(([^;{]*?)\)\s*;", text, flags=re.S | re.M):
        ret, name, params = m.group(1).strip(), m.group(2), " ".join(m.group(3).split())
        if name in ("if", "while", "return", "sizeof", "defined"):
            continue
        plist = [] if params in ("", "void") else [p.strip() for p in params.split(",")]
        out[name] = (ret, plist)
    return out


# The core boundary (names, return types and argument counts): the GEMV, small-N
# and fused argmax calls of the decode and verification steps, the block packers
# and size queries, and the error strings; the library may export more.
SCOPE_BOUNDARY = {
    "qg_abi_version": ("int", 0),
    "qg_status_string": ("const char*", 1),
    "qg_last_error": ("const char*", 0),
    "qg_q4k_bytes": ("size_t", 2),
    "qg_q8_0_bytes": ("size_t", 2),
    "qg_pack_q4k": ("qg_status", 5),
    "qg_pack_q8_0": ("qg_status", 5),
    "qgemv_q4k": ("qg_status", 6),
    "qgemv_q8_0": ("qg_status", 6),
    "qgemm_q4k_smalln": ("qg_status", 9),
    "lmhead_argmax_workspace_bytes": ("size_t", 2),
    "lmhead_argmax": ("qg_status", 9),
}


def test_scope_boundary_signatures():
    decl = _declarations()
    for name, (ret, nargs) in SCOPE_BOUNDARY.items():
        assert name in decl, name
        r, params = decl[name]
        assert r.replace(" ", "") == ret.replace(" ", ""), (name, r)
        assert len(params) == nargs, (name, params)
    # the products that need no workspace take none
    for name in ("qgemv_q4k", "qgemv_q8_0", "qgemm_q4k_smalln", "qgemv_q6k", "qgemv_q4k_q8_1",
                 "qgemm_q4k_q8_1_smalln", "qgemv_q4k_batch", "qgemm_q4k_smalln_batch"):
        assert not any("workspace" in p for p in decl[name][1]), name
        assert decl[name][1][-1].startswith("qg_stream_t"), name
    assert decl["qgemv_q4k"][1] == ["const void* w_packed", "const float* x", "float* y", "int64_t M", "int64_t K",
                                    "qg_stream_t stream"]
    assert decl["qgemm_q4k_smalln"][1][:3] == ["const void* w_packed", "const float* X", "int64_t ldx"]
    assert decl["lmhead_argmax"][1][6:8] == ["int32_t* out_index", "float* out_value"]
    # every entry point that launches work returns a status
    for name, (r, params) in decl.items():
        if params and params[-1].startswith("qg_stream_t"):
            assert r == "qg_status", name


def test_every_declaration_cites_its_passage():
    # each function declaration is preceded, within its block comment, by a
    # citation of the page section that defines it (or is a helper / override)
    text = open(qg.HEADER).read()
    blocks = re.split(r"\n(?=/\*)", text)
    cited = set()
    for b in blocks:
        m = re.match(r"/\*(.*?)\*/(.*)", b, flags=re.S)
        if not m:
            continue
        comment, body = m.group(1), m.group(2)
        names = re.findall(r"\b([a-z_][a-z_0-9]*)\s*\(", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
        if re.search(r"README|Why Local LLMs|Building a Fully Custom|tests and measurements|cannot allocate|"
                     r"host only|Size in bytes|Zero-fill", comment):
            cited.update(names)
    for name in _declarations():
        assert name in cited, name


def test_every_header_function_is_exported(L):
    names = qg.header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_status_strings(L):
    for s in range(7):
        assert qg.status_string(s) != "unknown status"
    assert qg.status_string(99) == "unknown status"


def test_sizes(L):
    assert L.qg_q4k_bytes(4096, 4096) == 9437184
    assert L.qg_q4k_bytes(3584, 18944) == 3584 * 74 * 144
    assert L.qg_q8_0_bytes(11008, 4096) == 47906816
    assert L.qg_q8_0_bytes(152064, 3584) == 579059712
    assert L.qg_q4k_bytes(4096, 4000) == 0
    assert L.qg_q4k_bytes(0, 256) == 0
    assert L.qg_q8_0_bytes(5, 48) == 0


def test_gemv_validation(L):
    f = L.qgemv_q4k
    assert f(None, A, B, 64, 256, None) == ENULL
    assert "NULL" in qg.last_error()
    assert f(C, A, B, 64, 300, None) == ESHAPE
    assert f(C, A, B, 0, 256, None) == ESHAPE
    assert f(C, A, B, 2**31, 256, None) == ESHAPE
    assert f(C + 4, A, B, 64, 256, None) == EALIGN
    assert f(C, A + 8, B, 64, 256, None) == EALIGN


def test_batch_validation(L):
    P = qg._Problem
    arr = (P * 9)()
    for i in range(9):
        arr[i] = P(C, A, B, 64, 256)
    assert L.qgemv_q4k_batch(arr, 0, None) == ESHAPE
    assert L.qgemv_q4k_batch(arr, 9, None) == ESHAPE
    arr[1] = P(C, None, B, 64, 256)
    assert L.qgemv_q4k_batch(arr, 2, None) == ENULL
    assert L.qgemv_q4k_batch(None, 1, None) == ENULL
    arr[1] = P(C, A, B, 64, 1000)
    assert L.qgemv_q4k_batch(arr, 2, None) == ESHAPE


def test_q8_0_and_lmhead_validation(L):
    assert L.qgemv_q8_0(C, A, B, 10, 33, None) == ESHAPE
    assert L.qgemv_q8_0(C, A, None, 10, 64, None) == ENULL
    assert L.lmhead_argmax(C, A, 1000, 3584, 0x40000, 1 << 20, None, None, None) == ENULL
    assert L.lmhead_argmax(C, A, 1000, 3584, None, 0, B, None, None) == EWS
    assert L.lmhead_argmax(C, A, 1000, 3584, 0x40000, 16, B, None, None) == EWS
    assert L.lmhead_argmax(C, A, 1000, 3584, 0x40000, 1 << 20, B + 2, None, None) == EALIGN
    assert L.lmhead_argmax(C, A, 2**31, 3584, 0x40000, 1 << 20, B, None, None) == ESHAPE
    assert L.lmhead_argmax_workspace_bytes(152064, 3584) == 152064 // 16 * 8


def test_noalloc_validation(L):
    f = L.lmhead_argmax_noalloc
    #  w, x, M, K, out_index, out_value, stream
    assert f(None, A, 1000, 3584, B, None, None) == ENULL
    assert f(C, A, 1000, 3584, None, None, None) == ENULL
    assert f(C, A, 1000, 3500, B, None, None) == ESHAPE
    assert f(C, A, 524289, 3584, B, None, None) == ESHAPE      # beyond the fixed partial array
    assert "524288" in qg.last_error()
    assert f(C, A, 1000, 3584, B + 2, None, None) == EALIGN
    assert f(C + 8, A, 1000, 3584, B, None, None) == EALIGN
    import torch
    if not torch.cuda.is_available():
        assert f(C, A, 524288, 3584, B, None, None) in (EDEV, EUNSUP)


def test_smalln_validation(L):
    f = L.qgemm_q4k_smalln
    assert f(C, A, 256, B, 64, 64, 256, 0, None) == ESHAPE
    assert f(C, A, 256, B, 64, 64, 256, 33, None) == ESHAPE
    assert f(C, A, 128, B, 64, 64, 256, 5, None) == ESHAPE   # ldx < K
    assert f(C, A, 256, B, 60, 64, 256, 5, None) == ESHAPE   # ldy < M
    assert f(C, A, 258, B, 64, 64, 256, 5, None) == ESHAPE   # ldx % 4
    assert f(C, A + 4, 256, B, 64, 64, 256, 5, None) == EALIGN
    # the activations must fit one 2^31-byte buffer range
    assert f(C, A, 1 << 26, B, 64, 64, 256, 32, None) == ESHAPE
    assert f(C, A, 1 << 26, B, 64, 64, 256, 1, None) != ESHAPE or "X extent" not in qg.last_error()


def test_pack_validation(L):
    assert L.qg_pack_q4k(None, A, 64, 256, None) == ENULL
    assert L.qg_pack_q4k(A, B, 64, 100, None) == ESHAPE
    assert L.qg_pack_q4k(A, A + 16, 64, 256, None) == ESHAPE  # overlap
    assert L.qg_pack_q8_0(A + 2, B, 64, 64, None) == EALIGN


def test_valid_call_without_gpu_reports_device_error(L):
    # all arguments valid: the only remaining check is the device query, which
    # fails here (no GPU visible) instead of launching anything
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    st = L.qgemv_q4k(C, A, B, 64, 256, None)
    assert st in (EDEV, EUNSUP)


def test_verify_validation(L):
    f = L.lmhead_argmax_verify
    out = 0x40000
    assert f(C, A, 512, 64, 500, 5, B, 1 << 20, out, None, None) == ESHAPE   # K % 256
    assert f(C, A, 512, 64, 512, 0, B, 1 << 20, out, None, None) == ESHAPE   # N = 0
    assert f(C, A, 512, 64, 512, 33, B, 1 << 20, out, None, None) == ESHAPE  # N > 32
    assert f(C, A, 500, 64, 512, 5, B, 1 << 20, out, None, None) == ESHAPE   # ldx < K
    assert f(C, A, 512, 64, 512, 5, None, 0, out, None, None) == EWS
    assert f(C, A, 512, 64, 512, 5, B, 1 << 20, None, None, None) == ENULL
    # 4 tiles x 5 columns x 8 bytes, rounded up to 256; for N <= 6 also the fp16
    # pairs (2K bytes) and block sums (K/8 bytes) of every column, rounded up to 256
    assert L.lmhead_argmax_verify_workspace_bytes(64, 512, 5) == 256 + 5632
    assert L.lmhead_argmax_verify_workspace_bytes(152064, 3584, 5) == 152064 // 16 * 5 * 8 + 38144
    assert L.lmhead_argmax_verify_workspace_bytes(152064, 3584, 7) == 152064 // 16 * 7 * 8


def test_q6k_sizes_and_validation(L):
    assert L.qg_q6k_bytes(3584, 18944) == 3584 * 74 * 210
    assert L.qg_q6k_bytes(152064, 3584) == 152064 * 14 * 210
    assert L.qg_q6k_bytes(10, 300) == 0
    assert L.qg_q6k_bytes(0, 256) == 0
    f = L.qgemv_q6k
    assert f(None, A, B, 64, 256, None) == ENULL
    assert f(C, A, B, 64, 300, None) == ESHAPE
    assert f(C, A, B, 0, 256, None) == ESHAPE
    assert f(C, A, B, 2**31 - 8, 256, None) == ESHAPE
    assert f(C, A, B, 64, 2**25, None) == ESHAPE
    assert f(C + 2, A, B, 64, 256, None) == EALIGN
    assert f(C, A, B + 4, 64, 256, None) == EALIGN
    assert L.qg_pack_q6k(None, A, 64, 256, None) == ENULL
    assert L.qg_pack_q6k(A, B, 64, 100, None) == ESHAPE
    assert L.qg_pack_q6k(A, A + 16, 64, 256, None) == ESHAPE  # overlap
    assert L.qg_pack_q6k(A + 2, B, 64, 256, None) == EALIGN


def test_topk_validation(L):
    O, S = qg._TopkOut, qg._Sampler
    D = 0x50000
    out = O(D, D + 256, D + 512, D + 768, D + 1024)
    ok_ws = 1 << 20
    f = L.logits_topk
    # 16 bytes per 16-row tile, then per group of 1024 tiles 64 eight-byte keys
    # and one (max, sum) pair, each part 256-byte aligned at its end
    def ws(M):
        tiles = -(-M // 16)
        groups = -(-tiles // 1024)
        up = lambda v: -(-v // 256) * 256
        return up(up(tiles * 16) + groups * 64 * 8 + groups * 8)
    assert L.logits_topk_workspace_bytes(152064) == ws(152064) == 157440
    assert L.logits_topk_workspace_bytes(262144) == ws(262144)
    assert L.logits_topk_workspace_bytes(262145) == 0
    assert L.lmhead_topk_workspace_bytes(152064, 3584) == ws(152064)
    assert L.lmhead_topk_workspace_bytes(152064, 3500) == 0
    assert f(None, 1000, 5, None, B, ok_ws, ctypes.byref(out), None) == ENULL
    assert f(A, 1000, 5, None, B, ok_ws, None, None) == ENULL
    assert f(A, 1000, 0, None, B, ok_ws, ctypes.byref(out), None) == ESHAPE
    assert f(A, 1000, 65, None, B, ok_ws, ctypes.byref(out), None) == ESHAPE
    assert f(A, 4, 5, None, B, ok_ws, ctypes.byref(out), None) == ESHAPE          # k > M
    assert f(A, 262145, 5, None, B, ok_ws, ctypes.byref(out), None) == ESHAPE     # M too large
    assert f(A, 1000, 5, None, None, 0, ctypes.byref(out), None) == EWS
    assert f(A, 1000, 5, None, B, 16, ctypes.byref(out), None) == EWS
    assert f(A + 4, 1000, 5, None, B, ok_ws, ctypes.byref(out), None) == EALIGN
    bad = O(D + 2, None, None, None, None)
    assert f(A, 1000, 5, None, B, ok_ws, ctypes.byref(bad), None) == EALIGN
    # a sampler needs u, a token output and sane parameters
    assert f(A, 1000, 5, ctypes.byref(S(1.0, 0.9, 0.0, None)), B, ok_ws, ctypes.byref(out), None) == ENULL
    no_tok = O(D, None, None, None, None)
    assert f(A, 1000, 5, ctypes.byref(S(1.0, 0.9, 0.0, C)), B, ok_ws, ctypes.byref(no_tok), None) == ENULL
    for T, p, m in [(1.0, 0.0, 0.0), (1.0, 1.5, 0.0), (1.0, 0.9, -0.1), (1.0, 0.9, 1.5), (float("nan"), 0.9, 0.0)]:
        assert f(A, 1000, 5, ctypes.byref(S(T, p, m, C)), B, ok_ws, ctypes.byref(out), None) == ESHAPE
    g = L.lmhead_topk
    assert g(C, A, 1000, 3584, 5, None, None, B, ok_ws, ctypes.byref(out), None) == ENULL   # logits
    assert g(C, A, 1000, 3500, 5, D, None, B, ok_ws, ctypes.byref(out), None) == ESHAPE
    assert g(C, A, 1000, 3584, 5, D + 4, None, B, ok_ws, ctypes.byref(out), None) == EALIGN


def test_q8_1_validation(L):
    assert L.qg_q8_1_bytes(3584) == 448 + 3584 + 224
    assert L.qg_q8_1_bytes(300) == 0
    assert L.qg_quantize_q8_1(None, 256, B, None) == ENULL
    assert L.qg_quantize_q8_1(A, 300, B, None) == ESHAPE
    assert L.qg_quantize_q8_1(A + 4, 256, B, None) == EALIGN
    assert L.qg_quantize_q8_1(A, 256, A + 512, None) == ESHAPE  # overlap
    f = L.qgemv_q4k_q8_1
    assert f(C, None, B, 64, 256, None) == ENULL
    assert f(C, A, B, 64, 300, None) == ESHAPE
    assert f(C, A, B, 0, 256, None) == ESHAPE
    assert f(C, A + 8, B, 64, 256, None) == EALIGN


def test_q8_1_batch_validation(L):
    P = qg._Problem
    arr = (P * 9)()
    for i in range(9):
        arr[i] = P(C, A, B, 64, 256)
    f = L.qgemv_q4k_q8_1_batch
    assert f(arr, 0, None) == ESHAPE
    assert f(arr, 9, None) == ESHAPE
    assert f(None, 1, None) == ENULL
    arr[1] = P(C, None, B, 64, 256)
    assert f(arr, 2, None) == ENULL
    arr[1] = P(C, A, B, 64, 1000)
    assert f(arr, 2, None) == ESHAPE
    arr[1] = P(C, A + 4, B, 64, 256)
    assert f(arr, 2, None) == EALIGN


def test_q8_1_smalln_validation(L):
    f = L.qgemm_q4k_q8_1_smalln
    #  w, xq, Y, ldy, M, K, N
    assert f(C, None, B, 64, 64, 256, 5, None) == ENULL
    assert f(C, A, B, 64, 64, 256, 0, None) == ESHAPE    # N < 1
    assert f(C, A, B, 64, 64, 256, 9, None) == ESHAPE    # N > 8
    assert f(C, A, B, 64, 64, 300, 5, None) == ESHAPE    # K % 256
    assert f(C, A, B, 60, 64, 256, 5, None) == ESHAPE    # ldy < M
    assert f(C, A, B, 66, 64, 256, 5, None) == ESHAPE    # ldy % 4
    assert f(C, A, B, 64, 0, 256, 5, None) == ESHAPE     # M < 1
    assert f(C, A + 8, B, 64, 64, 256, 5, None) == EALIGN
    P = qg._GemmQ81Problem
    arr = (P * 9)()
    for i in range(9):
        arr[i] = P(C, A, B, 64, 64, 256, 5)
    g = L.qgemm_q4k_q8_1_smalln_batch
    assert g(arr, 0, None) == ESHAPE
    assert g(arr, 9, None) == ESHAPE
    assert g(None, 1, None) == ENULL
    arr[1] = P(C, A, None, 64, 64, 256, 5)
    assert g(arr, 2, None) == ENULL


def test_smalln_forced_forms_keep_validation(L):
    # forcing a form does not relax the small-N argument checks
    f = L.qgemm_q4k_smalln
    for form in (qg.FORM_SMALLN_DOT, qg.FORM_SMALLN_REGS, qg.FORM_SMALLN_LDS, qg.FORM_SMALLN_LDS1,
                 qg.FORM_SMALLN_STREAM, qg.FORM_SMALLN_WALK, qg.FORM_SMALLN_SPLIT, qg.FORM_SMALLN_SLICE):
        with qg.launch_override(smalln_form=form):
            assert f(C, A, 256, B, 64, 64, 256, 0, None) == ESHAPE
            assert f(C, A, 128, B, 64, 64, 256, 3, None) == ESHAPE   # ldx < K
            assert f(C, A + 4, 256, B, 64, 64, 256, 3, None) == EALIGN
    assert qg.get_launch_override()["smalln_form"] == 0


def test_smalln_ws_sizes_and_validation(L):
    P = qg._GemmProblem
    arr = (P * 2)(P(C, A, 18944, B, 3584, 3584, 18944, 32), P(C, A, 3584, B, 4608, 4608, 3584, 32))
    assert L.qgemm_q4k_smalln_batch_workspace_bytes(arr, 0) == 0            # invalid count
    bad = (P * 1)(P(C, A, 100, B, 3584, 3584, 18944, 32))                    # ldx < K
    assert L.qgemm_q4k_smalln_batch_workspace_bytes(bad, 1) == 0
    with qg.launch_override(smalln_form=qg.FORM_SMALLN_SPLIT):
        need = L.qgemm_q4k_smalln_batch_workspace_bytes(arr, 2)
        assert need > 0 and need % 256 == 0
        # a fixed 4096-byte block for the tile groups' counters, then a partial sum
        # per K slice, tile and 16-column block, at most 16 slices
        assert need <= 4096 + 16 * (224 + 288) * 2 * 1024
    # the slice form's plan for the 7B down projection at N = 5: 56 groups of four
    # tiles, four K slices (18 or 19 super-blocks: 5 x 19 <= 160 staged groups)
    one = (P * 1)(P(C, A, 18944, B, 3584, 3584, 18944, 5))
    with qg.launch_override(smalln_form=qg.FORM_SMALLN_SLICE):
        assert L.qgemm_q4k_smalln_batch_workspace_bytes(one, 1) == 4096 + 4 * 224 * 1024
    # long K in the K-sliced walk: groups of 8 tiles at N = 32 (28 groups), the
    # slice count rounded down to a power of two (9 -> 8 slices of two 16-column
    # blocks); groups of 4 at N = 16 (56 groups, 4 slices)
    d32 = (P * 1)(P(C, A, 18944, B, 3584, 3584, 18944, 32))
    d16 = (P * 1)(P(C, A, 18944, B, 3584, 3584, 18944, 16))
    with qg.launch_override(smalln_form=qg.FORM_SMALLN_SPLIT):
        assert L.qgemm_q4k_smalln_batch_workspace_bytes(d32, 1) == 4096 + 8 * 224 * 2048
        assert L.qgemm_q4k_smalln_batch_workspace_bytes(d16, 1) == 4096 + 4 * 224 * 1024
    assert L.qgemm_q4k_smalln_batch_ws(None, 1, None, 0, None) == ENULL
    assert L.qgemm_q4k_smalln_batch_ws(bad, 1, None, 0, None) == ESHAPE


def test_launch_override_validation(L):
    O = qg._LaunchOverride
    assert L.qg_set_launch_override(None) == OK
    for field, bad in [("gemv_waves", 3), ("gemv_waves", 16), ("smalln_form", 9), ("smalln_waves", 16),
                       ("smalln_tiles", 3), ("smalln_depth", 1), ("verify_form", 4), ("verify_waves", 2),
                       ("verify_tiles", 8)]:
        o = O()
        setattr(o, field, bad)
        assert L.qg_set_launch_override(ctypes.byref(o)) == ESHAPE, field
        assert field in qg.last_error()
    assert all(v == 0 for v in qg.get_launch_override().values())
    with qg.launch_override(gemv_waves=2, verify_form=qg.FORM_VERIFY_MFMA):
        got = qg.get_launch_override()
        assert got["gemv_waves"] == 2 and got["verify_form"] == qg.FORM_VERIFY_MFMA
        with qg.launch_override(smalln_tiles=4):
            assert qg.get_launch_override()["gemv_waves"] == 0
        assert qg.get_launch_override()["gemv_waves"] == 2
    assert all(v == 0 for v in qg.get_launch_override().values())
    assert L.qg_get_launch_override(None) == ENULL


def test_quantize_columns_validation(L):
    f = L.qg_quantize_q8_1_columns
    #  X, ldx, K, N, xq, stream
    assert f(None, 256, 256, 2, B, None) == ENULL
    assert f(A, 256, 300, 2, B, None) == ESHAPE     # K % 256
    assert f(A, 256, 256, 0, B, None) == ESHAPE     # N < 1
    assert f(A, 256, 256, 33, B, None) == ESHAPE    # N > 32
    assert f(A, 128, 256, 2, B, None) == ESHAPE     # ldx < K
    assert f(A, 258, 256, 2, B, None) == ESHAPE     # ldx % 4
    assert f(A + 4, 256, 256, 2, B, None) == EALIGN
    assert f(A, 256, 256, 2, A + 1024, None) == ESHAPE  # overlap


def test_verify_q8_1_validation(L):
    f = L.lmhead_argmax_verify_q8_1
    out = 0x40000
    #  w, xq, M, K, N, ws, ws_bytes, out_index, out_value, stream
    assert f(C, None, 64, 512, 5, B, 1 << 20, out, None, None) == ENULL
    assert f(C, A, 64, 500, 5, B, 1 << 20, out, None, None) == ESHAPE   # K % 256
    assert f(C, A, 64, 512, 0, B, 1 << 20, out, None, None) == ESHAPE   # N = 0
    assert f(C, A, 64, 512, 9, B, 1 << 20, out, None, None) == ESHAPE   # N > 8
    assert f(C, A, 0, 512, 5, B, 1 << 20, out, None, None) == ESHAPE    # M < 1
    assert f(C + 8, A, 64, 512, 5, B, 1 << 20, out, None, None) == EALIGN
    assert f(C, A, 64, 512, 5, None, 0, out, None, None) == EWS
    assert f(C, A, 64, 512, 5, B, 255, out, None, None) == EWS
    assert f(C, A, 64, 512, 5, B, 1 << 20, None, None, None) == ENULL
    assert f(C, A, 64, 512, 5, B, 1 << 20, out + 2, None, None) == EALIGN
    assert L.lmhead_argmax_verify_q8_1_workspace_bytes(64, 512, 5) == 256
    assert L.lmhead_argmax_verify_q8_1_workspace_bytes(152064, 3584, 5) == 152064 // 16 * 5 * 8
    assert L.lmhead_argmax_verify_q8_1_workspace_bytes(64, 512, 9) == 0

"""The C-ABI library without a GPU: it loads, exports every function
include/qmm.h declares, agrees with the oracle and the generators on block
geometry, resolves exactly the eleven kinds by name, and refuses bad calls
with the documented status, in the documented order, before launching
anything."""
import ctypes
import os
import re
import subprocess

import pytest

import gguf_block_quantized_kind_amd as qmm
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

OK, EMPTY, KIND, KALIGN, DTYPE, ARG, HIP, WS = range(8)
FAKE = 0x1000  # never dereferenced: every call below is refused first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qmm.LIBRARY):
        import gguf_block_quantized_kind_amd._build as b
        b.build()
    return qmm.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qmm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("qmm_gemv", "qmm_gemm", "qmm_gemv_ex", "qmm_gemm_ex", "qmm_moe",
                     "qmm_moe_workspace_bytes", "qmm_dequant", "qmm_row_bytes"):
        assert required in names


def test_every_declared_function_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", qmm.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qmm_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(lib, n)


def test_geometry_matches_oracle_and_generators(lib, oracle_mod):
    for name, (kid, bb, be) in wl.KINDS.items():
        assert qmm.qmm_kind_from_name(name) == kid
        assert qmm.qmm_kind_name(kid) == name
        assert qmm.qmm_block_geometry(kid) == (bb, be) == oracle_mod.block_geometry(kid)
        for K in (be, 4096, 2048, 768):
            if K % be == 0:
                assert qmm.qmm_row_bytes(kid, K) == wl.row_bytes(name, K)
        assert qmm.qmm_row_bytes(kid, be + 16) == -1


def test_absent_kinds_do_not_resolve(lib):
    for absent in ("Q4_1", "Q5_1", "Q8_1", "IQ1_S", "IQ2_XXS", "IQ3_S", "q4_0", ""):
        assert qmm.qmm_kind_from_name(absent) == -1
    for kid in (0, 1, 3, 7, 9, 15, 16, 19, 21, 22, 40):
        assert qmm.qmm_kind_name(kid) is None
        assert lib.qmm_row_bytes(kid, 4096) == -1
        b, e = ctypes.c_int(), ctypes.c_int()
        assert lib.qmm_block_geometry(kid, ctypes.byref(b), ctypes.byref(e)) == KIND


def test_gemv_refusals_in_order(lib):
    g = lib.qmm_gemv_ex
    # empty beats everything else
    assert g(3, None, None, 9, None, 0, 10, 48, None) == EMPTY
    assert g(2, FAKE, FAKE, 0, FAKE, 1, 0, 4096, None) == EMPTY
    assert g(2, FAKE, FAKE, 0, FAKE, 1, 10, 0, None) == EMPTY
    # then the kind
    assert g(3, None, None, 9, None, 1, 10, 48, None) == KIND
    assert "kind 3" in qmm.qmm_last_error()
    # then K against the block
    assert g(2, None, None, 9, None, 1, 10, 48, None) == KALIGN
    assert g(12, None, None, 9, None, 1, 10, 512 + 32, None) == KALIGN
    # then the dtype
    assert g(2, None, None, 9, None, 1, 10, 64, None) == DTYPE
    # then pointers, alignment and M
    assert g(2, None, FAKE, 0, FAKE, 1, 10, 64, None) == ARG
    assert g(2, FAKE, None, 0, FAKE, 1, 10, 64, None) == ARG
    assert g(2, FAKE, FAKE, 0, None, 1, 10, 64, None) == ARG
    assert g(2, FAKE, FAKE + 2, 0, FAKE, 1, 10, 64, None) == ARG   # f32 x at 2 bytes
    assert g(2, FAKE, FAKE, 0, FAKE + 2, 1, 10, 64, None) == ARG   # y misaligned
    assert g(2, FAKE, FAKE, 0, FAKE, 9, 10, 64, None) == ARG       # M > 8
    assert lib.qmm_gemv(2, None, FAKE, FAKE, 10, 64) == ARG
    # sizes beyond the kernels' 32-bit row and element counts
    assert g(2, FAKE, FAKE, 0, FAKE, 1, 1 << 31, 64, None) == ARG   # N > INT32_MAX
    assert g(2, FAKE, FAKE, 0, FAKE, 1, 10, (1 << 30) + 32, None) == ARG  # K > 2^30


def test_matmul_packed_refusals(lib):
    m = lib.qmm_matmul_packed
    # above eight tokens, a kind the prefill GEMM over records does not take
    assert m(12, FAKE, FAKE, 1, FAKE, 9, 16, 256, None) == KIND
    # M * K at 2^31, for any token count
    assert m(8, FAKE, FAKE, 1, FAKE, 1 << 21, 16, 1024, None) == ARG
    # activation bytes at 2^31 (the GEMM's signed 32-bit offsets): 2^29
    # f32 values, 2^30 f16 values
    assert m(8, FAKE, FAKE, 0, FAKE, 1 << 18, 16, 2048, None) == ARG
    assert m(8, FAKE, FAKE, 1, FAKE, 1 << 19, 16, 2048, None) == ARG
    # repacked weights of 2 GiB or more (Q8_0: 272 bytes per row of 256)
    assert m(8, FAKE, FAKE, 1, FAKE, 16, (1 << 31) // 272 + 16, 256, None) == ARG


def test_gemm_refusals_in_order(lib):
    g = lib.qmm_gemm_ex
    assert g(2, FAKE, FAKE, 1, FAKE, 0, 10, 64, None) == EMPTY
    assert g(5, FAKE, FAKE, 1, FAKE, 10, 10, 64, None) == KIND
    assert g(14, FAKE, FAKE, 1, FAKE, 10, 10, 64, None) == KALIGN
    assert g(14, FAKE, FAKE, 2, FAKE, 10, 10, 256, None) == DTYPE
    assert g(14, FAKE, None, 1, FAKE, 10, 10, 256, None) == ARG
    assert g(14, FAKE, FAKE + 1, 1, FAKE, 10, 10, 256, None) == ARG  # f16 A at an odd address
    assert lib.qmm_gemm(14, FAKE, FAKE, None, 10, 10, 256) == ARG
    assert lib.qmm_matmul(39, FAKE, FAKE, 0, FAKE, 10, 10, 48, None) == KALIGN


def test_moe_refusals_in_order(lib):
    g = lib.qmm_moe
    ws_need = lib.qmm_moe_workspace_bytes(128, 16, 8)
    # int32 counts[E], offsets[E+1], order[P], item count, items[2 (P + min(E, P))]
    P = 16 * 8
    assert ws_need == (128 + 129 + P + 1 + 2 * (P + min(128, P))) * 4
    assert lib.qmm_moe_workspace_bytes(128, 1, 8) == (128 + 129 + 8 + 1 + 2 * (8 + 8)) * 4
    args = dict(kind=12, W=FAKE, E=128, ids=FAKE, topk=8, X=FAKE, dt=1, per=0, Y=FAKE, M=16, N=1536,
                K=2048, ws=FAKE, wsb=ws_need, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return g(a["kind"], a["W"], a["E"], a["ids"], a["topk"], a["X"], a["dt"], a["per"], a["Y"],
                 a["M"], a["N"], a["K"], a["ws"], a["wsb"], a["s"])

    assert call(E=0) == EMPTY
    assert call(topk=0) == EMPTY
    assert call(M=0) == EMPTY
    assert call(kind=1) == KIND
    assert call(K=2048 + 32) == KALIGN
    assert call(dt=5) == DTYPE
    assert call(ids=None) == ARG
    assert call(per=2) == ARG
    assert call(E=5000) == ARG
    assert call(ws=None) == WS
    assert call(wsb=ws_need - 1) == WS
    assert "workspace" in qmm.qmm_last_error()


def test_gemm_mx_refusals_in_order(lib):
    g = lib.qmm_gemm_mx
    need = lib.qmm_gemm_mx_workspace_bytes(10, 256)
    # Two terms of FP8 codes and E8M0 scales for M rounded up to 64 rows.
    assert need == 2 * (64 * 256 + 64 * 8)
    assert lib.qmm_gemm_mx_workspace_bytes(65, 4096) == 2 * 128 * 4096 * 33 // 32
    assert lib.qmm_gemm_mx_workspace_bytes(0, 256) == 0
    assert lib.qmm_gemm_mx_workspace_bytes(10, 48) == 0
    assert g(39, FAKE, FAKE, 1, FAKE, 0, 10, 256, FAKE, need, None) == EMPTY
    assert g(5, FAKE, FAKE, 1, FAKE, 10, 10, 256, FAKE, need, None) == KIND
    assert g(39, FAKE, FAKE, 1, FAKE, 10, 10, 48, FAKE, need, None) == KALIGN
    assert g(2, FAKE, FAKE, 1, FAKE, 10, 10, 256, FAKE, need, None) == KIND   # Q4_0: MXFP4 only
    assert "MXFP4" in qmm.qmm_last_error()
    assert g(39, FAKE, FAKE, 3, FAKE, 10, 10, 256, FAKE, need, None) == DTYPE
    assert g(39, None, FAKE, 1, FAKE, 10, 10, 256, FAKE, need, None) == ARG
    assert g(39, FAKE + 4, FAKE, 1, FAKE, 10, 10, 256, FAKE, need, None) == ARG  # W not 16-byte aligned
    assert g(39, FAKE, FAKE + 1, 1, FAKE, 10, 10, 256, FAKE, need, None) == ARG
    assert g(39, FAKE, FAKE, 1, FAKE, 65535 * 64 + 1, 10, 256, FAKE, 1 << 40, None) == ARG
    assert g(39, FAKE, FAKE, 1, FAKE, 10, 10, 256, None, need, None) == WS
    assert g(39, FAKE, FAKE, 1, FAKE, 10, 10, 256, FAKE, need - 1, None) == WS
    assert g(39, FAKE, FAKE, 1, FAKE, 10, 10, 256, FAKE + 8, need, None) == WS


def test_repack_sizes_and_refusals_in_order(lib, oracle_mod):
    from oracle import repack as rp
    for name in rp.KINDS:
        kid = qmm.kind_id(name)
        for N, K in ((130, 1024), (1, 256), (14336, 4096)):
            assert lib.qmm_packed_bytes(kid, N, K) == rp.packed_bytes(name, N, K)
        # Whole tiles: the native size exactly.
        assert lib.qmm_packed_bytes(kid, 32, 4096) == 32 * qmm.qmm_row_bytes(kid, 4096)
    assert len(rp.KINDS) == 11                     # every kind has a repacked layout
    assert lib.qmm_packed_bytes(99, 16, 256) == -1   # not a kind
    assert lib.qmm_packed_bytes(2, 16, 288) == -1
    assert lib.qmm_packed_bytes(2, 0, 256) == -1
    r = lib.qmm_repack
    assert r(2, FAKE, FAKE, 0, 256, None) == EMPTY
    assert r(99, FAKE, FAKE, 16, 256, None) == KIND
    assert r(2, FAKE, FAKE, 16, 48, None) == KALIGN     # not whole Q4_0 blocks
    assert r(2, FAKE, FAKE, 16, 288, None) == KALIGN    # whole blocks, not whole k-blocks
    assert "256" in qmm.qmm_last_error()
    assert r(2, None, FAKE, 16, 256, None) == ARG
    assert r(2, FAKE, FAKE + 8, 16, 256, None) == ARG   # P not 16-byte aligned
    g = lib.qmm_gemv_packed
    assert g(12, FAKE, FAKE, 0, FAKE, 0, 16, 256, None) == EMPTY
    assert g(99, FAKE, FAKE, 0, FAKE, 1, 16, 256, None) == KIND
    assert g(2, FAKE, FAKE, 0, FAKE, 1, 16, 256 + 32, None) == KALIGN
    assert g(12, FAKE, FAKE, 2, FAKE, 1, 16, 256, None) == DTYPE
    assert g(12, None, FAKE, 0, FAKE, 1, 16, 256, None) == ARG
    assert g(12, FAKE + 4, FAKE, 0, FAKE, 1, 16, 256, None) == ARG
    assert g(12, FAKE, FAKE + 2, 0, FAKE, 1, 16, 256, None) == ARG
    assert g(12, FAKE, FAKE, 0, FAKE + 2, 1, 16, 256, None) == ARG
    assert g(12, FAKE, FAKE, 0, FAKE, 9, 16, 256, None) == ARG
    assert g(12, FAKE, FAKE, 0, FAKE, 8, 16, 1 << 28, None) == ARG   # M * K >= 2^31


def test_gemv_i8_refusals_in_order(lib):
    g = lib.qmm_gemv_i8
    need = lib.qmm_gemv_i8_workspace_bytes(3, 512)
    assert need == 1536 + 2 * 256
    assert lib.qmm_gemv_i8_workspace_bytes(8, 4096) == 32768 + 2 * 4096
    assert lib.qmm_gemv_i8_workspace_bytes(0, 512) == 0 and lib.qmm_gemv_i8_workspace_bytes(3, 48) == 0
    assert g(8, FAKE, FAKE, 0, FAKE, 0, 16, 512, FAKE, need, None) == EMPTY
    assert g(10, FAKE, FAKE, 0, FAKE, 3, 16, 512, FAKE, need, None) == KIND    # Q2_K: not an integer-code kind
    assert g(12, FAKE, FAKE, 0, FAKE, 3, 16, 512, FAKE, need, None) == KIND    # Q4_K: not an integer-code kind
    assert "IQ4_NL or MXFP4" in qmm.qmm_last_error()
    assert g(8, FAKE, FAKE, 0, FAKE, 3, 16, 288, FAKE, need, None) == KALIGN
    assert g(8, FAKE, FAKE, 2, FAKE, 3, 16, 512, FAKE, need, None) == DTYPE
    assert g(8, None, FAKE, 0, FAKE, 3, 16, 512, FAKE, need, None) == ARG
    assert g(8, FAKE + 8, FAKE, 0, FAKE, 3, 16, 512, FAKE, need, None) == ARG
    assert g(8, FAKE, FAKE + 2, 0, FAKE, 3, 16, 512, FAKE, need, None) == ARG
    assert g(8, FAKE, FAKE, 0, FAKE, 9, 16, 512, FAKE, need, None) == ARG
    assert g(8, FAKE, FAKE, 0, FAKE, 8, 16, 65536, FAKE, 1 << 30, None) == ARG  # M*K > 262144
    assert g(8, FAKE, FAKE, 0, FAKE, 3, 16, 512, None, need, None) == WS
    assert g(8, FAKE, FAKE, 0, FAKE, 3, 16, 512, FAKE, need - 1, None) == WS
    assert g(8, FAKE, FAKE, 0, FAKE, 3, 16, 512, FAKE + 16, need, None) == WS


def test_moe_packed_refusals_in_order(lib):
    f = lib.qmm_moe_packed
    need = lib.qmm_moe_workspace_bytes(8, 4, 2)
    args = lambda **k: [k.get("kind", 12), k.get("P", FAKE), k.get("E", 8), k.get("ids", FAKE), k.get("topk", 2),
                        k.get("X", FAKE), k.get("dt", 1), k.get("ps", 0), k.get("Y", FAKE), k.get("M", 4),
                        k.get("N", 16), k.get("K", 256), k.get("ws", FAKE), k.get("wsb", need), None]
    assert f(*args(E=0)) == EMPTY
    assert f(*args(M=0)) == EMPTY
    assert f(*args(kind=99)) == KIND                      # not a kind
    assert f(*args(kind=2, K=288)) == KALIGN
    assert f(*args(dt=5)) == DTYPE
    assert f(*args(P=None)) == ARG
    assert f(*args(P=FAKE + 8)) == ARG
    assert f(*args(X=FAKE + 1)) == ARG
    assert f(*args(ids=FAKE + 2)) == ARG
    assert f(*args(ps=2)) == ARG
    assert f(*args(E=5000)) == ARG
    assert f(*args(M=1 << 20, topk=8, K=512, wsb=1 << 40)) == ARG     # M*topk*K >= 2^31
    assert f(*args(ws=None)) == WS
    assert f(*args(wsb=need - 1)) == WS


def test_moe_ffn_packed_refusals(lib):
    f = lib.qmm_moe_ffn_packed
    need = lib.qmm_moe_ffn_workspace_bytes(4, 2, 2, 256, 512)
    args = lambda **k: [k.get("kind", 12), k.get("Pg", FAKE), k.get("Pd", FAKE), 4, FAKE, FAKE, 2,
                        FAKE, 1, FAKE, k.get("M", 2), k.get("Nff", 256), k.get("K", 512), FAKE, need, None]
    assert f(*args(Nff=0)) == EMPTY
    assert f(*args(kind=99)) == KIND                  # not a kind
    assert f(*args(kind=2, K=288)) == KALIGN          # K not whole k-blocks
    assert f(*args(kind=2, Nff=288)) == KALIGN        # N_ff (the down matrix's K) not whole k-blocks
    assert f(*args(Pg=FAKE + 8)) == ARG
    assert f(*args(Pd=None)) == ARG


def test_moe_ffn_refusals_in_order(lib):
    g = lib.qmm_moe_ffn
    need = lib.qmm_moe_ffn_workspace_bytes(8, 4, 2, 256, 512)
    route = lib.qmm_moe_workspace_bytes(8, 4, 2)
    up = lambda b: (b + 255) // 256 * 256
    # routing words, f32 gate/up [P][2 N_ff], h [P][N_ff], down [P][K], per-pair scales [P]
    assert need == up(route) + up(8 * 512 * 4) + up(8 * 256 * 4) + up(8 * 512 * 4) + up(8 * 4)
    assert lib.qmm_moe_ffn_workspace_bytes(0, 4, 2, 256, 512) == 0
    a = dict(kind=12, Wgu=FAKE, Wd=FAKE, E=8, ids=FAKE, w=FAKE, topk=2, X=FAKE, dt=1, Y=FAKE, M=4, Nff=256,
             K=512, ws=FAKE, wsb=need, s=None)

    def call(**kw):
        b = dict(a, **kw)
        return g(b["kind"], b["Wgu"], b["Wd"], b["E"], b["ids"], b["w"], b["topk"], b["X"], b["dt"], b["Y"],
                 b["M"], b["Nff"], b["K"], b["ws"], b["wsb"], b["s"])

    assert call(E=0) == EMPTY
    assert call(Nff=0) == EMPTY
    assert call(M=0) == EMPTY
    assert call(kind=1) == KIND
    assert call(K=512 + 32) == KALIGN      # gate/up row length
    assert call(Nff=256 + 32) == KALIGN    # down row length
    assert call(dt=4) == DTYPE
    assert call(w=None) == ARG
    assert call(Wd=None) == ARG
    assert call(Y=FAKE + 4) == ARG         # Y must be 16-byte aligned
    assert call(E=5000) == ARG
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=FAKE + 16) == WS        # 256-byte aligned


def test_dequant_refusals(lib):
    assert lib.qmm_dequant(2, FAKE, FAKE, 0, None) == EMPTY
    assert lib.qmm_dequant(4, FAKE, FAKE, 32, None) == KIND
    assert lib.qmm_dequant(2, FAKE, FAKE, 33, None) == KALIGN
    assert lib.qmm_dequant(2, None, FAKE, 32, None) == ARG
    assert lib.qmm_dequant(2, FAKE, FAKE + 1, 32, None) == ARG


def test_status_strings(lib):
    for st in range(8):
        assert qmm.qmm_status_string(st)
    assert qmm.qmm_status_string(123) == "unknown status"


def test_binding_fails_loudly_without_library(tmp_path):
    saved = qmm._lib
    qmm._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            qmm.load_library(str(tmp_path / "missing.so"))
    finally:
        qmm._lib = saved


def test_binding_refuses_wrong_element_types(lib):
    """The binding checks element types before calling the library: an f16
    output of M*N elements is half the bytes the kernel writes, int64 ids
    would be read as int32 pairs.  (CPU tensors: nothing reaches the GPU.)"""
    torch = pytest.importorskip("torch")
    u8 = torch.zeros(18 * 4, dtype=torch.uint8)
    x32, x16 = torch.zeros(32), torch.zeros(32, dtype=torch.float16)
    y32, y16 = torch.zeros(4), torch.zeros(4, dtype=torch.float16)
    with pytest.raises(TypeError, match="y must be float32"):
        qmm.qmm_gemv_ex("Q4_0", u8, x32, y16, 1, 4, 32)
    with pytest.raises(TypeError, match="W must be a byte tensor"):
        qmm.qmm_gemv_ex("Q4_0", torch.zeros(18, dtype=torch.int32), x32, y32, 1, 4, 32)
    with pytest.raises(TypeError, match="x must be float32"):
        qmm.qmm_gemv("Q4_0", u8, x16, y32, 4, 32)
    with pytest.raises(TypeError, match="A must be float16"):
        qmm.qmm_gemm("Q4_0", u8, x32, y32, 1, 4, 32)
    with pytest.raises(TypeError, match="C must be float32"):
        qmm.qmm_matmul("Q4_0", u8, x16, y16, 1, 4, 32)
    ids64 = torch.zeros((1, 2), dtype=torch.int64)
    with pytest.raises(TypeError, match="ids must be int32"):
        qmm.qmm_moe("Q4_0", torch.zeros(18 * 8, dtype=torch.uint8), 2, ids64, 2, x32, 0,
                    torch.zeros(8), 1, 4, 32, None)
    ids32 = torch.zeros((1, 2), dtype=torch.int32)
    with pytest.raises(TypeError, match="topk_w must be float32"):
        qmm.qmm_moe_ffn("Q4_0", torch.zeros(18 * 8, dtype=torch.uint8), torch.zeros(18 * 8, dtype=torch.uint8),
                        2, ids32, torch.zeros((1, 2), dtype=torch.float16), 2, x32, torch.zeros(32), 1, 2, 32,
                        None)
    with pytest.raises(TypeError, match="out must be float32"):
        qmm.qmm_dequant("Q4_0", u8, torch.zeros(32, dtype=torch.float16), 32)


def test_binding_refuses_host_tensors(lib):
    """Correctly typed host tensors are refused before the library is called:
    the kernels would fault on a host address."""
    torch = pytest.importorskip("torch")
    u8 = torch.zeros(18 * 4, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device memory only"):
        qmm.qmm_gemv_ex("Q4_0", u8, torch.zeros(32), torch.zeros(4), 1, 4, 32)
    with pytest.raises(ValueError, match="device memory only"):
        qmm.qmm_repack("Q4_K", torch.zeros(144 * 16, dtype=torch.uint8), torch.zeros(144 * 16, dtype=torch.uint8),
                       16, 256)

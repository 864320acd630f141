"""The C ABI: the library loads, exports every symbol include/*.h declares, and
rejects invalid arguments with the documented status before touching a
device (CPU only: no call here reaches a kernel launch).

Every call below passes at least one invalid argument, so the fake (never
dereferenced) device addresses are safe on a machine with a GPU too.
"""

import ctypes
import glob
import os
import re

import pytest

import block_quantized_weight_qgemv_amd as q
from block_quantized_weight_qgemv_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = q.lib()

OK, NULL, SHAPE, GROUP, MIS, BATCH, DTYPE, BITS, VALUE, LARGE = range(10)

A = ctypes.c_void_p(0x100000)        # 16-byte aligned fake addresses
A2 = ctypes.c_void_p(0x200000)
A3 = ctypes.c_void_p(0x300000)
A4 = ctypes.c_void_p(0x400000)
ODD = ctypes.c_void_p(0x100008)      # 8-byte aligned only


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(q(?:g|gemv)_[A-Za-z0-9_]+)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert {"qgemv_fp4_e2m1", "qgemv_affine_u4", "qgemv_affine_u8", "qgemv_fp8_e4m3",
            "qg_quantize_fp4_e2m1", "qg_pack_u32", "qg_bytes_fp8"} <= names
    for name in sorted(names):
        assert hasattr(LIB, name), name
    # and the binding declares a signature for each of them
    assert names <= set(B.SIGNATURES), names - set(B.SIGNATURES)


def test_abi_version_and_status_strings():
    header = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    declared = int(re.search(r"#define\s+QG_ABI_VERSION\s+(\d+)", header).group(1))
    # the header, the binding's declarations and the loaded library agree
    assert q.qg_abi_version() == declared == B.ABI_VERSION
    for s in range(12):
        assert isinstance(q.qg_status_string(s), str) and q.qg_status_string(s)
    assert q.qg_status_string(999) == "unknown status"


def _fp4(codes=A, scales=A2, x=A3, y=A4, n=8, k=64, gs=32, b=1, out=0):
    return LIB.qgemv_fp4_e2m1(codes, scales, x, y, n, k, gs, b, out, None)


@pytest.mark.parametrize("kw,status", [
    ({"codes": None}, NULL), ({"scales": None}, NULL), ({"x": None}, NULL), ({"y": None}, NULL),
    ({"n": 0}, SHAPE), ({"k": 0}, SHAPE), ({"k": 48}, SHAPE), ({"n": -3}, SHAPE),
    ({"gs": 16}, GROUP), ({"gs": 96}, GROUP), ({"k": 96, "gs": 64}, GROUP),
    ({"codes": ODD}, MIS), ({"x": ODD}, MIS), ({"y": ctypes.c_void_p(0x100002)}, MIS),
    ({"b": 0}, BATCH), ({"b": 5}, BATCH), ({"out": 2}, DTYPE), ({"k": (1 << 30) + 32}, SHAPE),
])
def test_fp4_validation(kw, status):
    assert _fp4(**kw) == status


def _aff(fn, codes=A, scales=A2, biases=A2, x=A3, y=A4, n=8, k=128, gs=64, b=1, out=0):
    return fn(codes, scales, biases, x, y, n, k, gs, b, out, None)


@pytest.mark.parametrize("name", ["qgemv_affine_u4", "qgemv_affine_u8"])
@pytest.mark.parametrize("kw,status", [
    ({"biases": None}, NULL), ({"scales": None}, NULL), ({"codes": None}, NULL),
    ({"k": 24}, SHAPE), ({"gs": 0}, GROUP), ({"gs": 256}, GROUP),
    ({"biases": ctypes.c_void_p(0x200001)}, MIS), ({"b": 9}, BATCH), ({"out": -1}, DTYPE),
    ({"k": (1 << 30) + 64}, SHAPE),
])
def test_affine_validation(name, kw, status):
    assert _aff(getattr(LIB, name), **kw) == status


def test_u8_group_16_rejected_and_u4_needs_k_multiple_of_32():
    assert _aff(LIB.qgemv_affine_u8, k=128, gs=16) == GROUP
    assert _aff(LIB.qgemv_affine_u4, k=16 * 3, gs=32) == SHAPE


def _fp8(codes=A, rs=A2, x=A3, y=A4, n=8, k=64, b=1, out=0):
    return LIB.qgemv_fp8_e4m3(codes, rs, x, y, n, k, b, out, None)


@pytest.mark.parametrize("kw,status", [
    ({"rs": None}, NULL), ({"k": 8}, SHAPE), ({"rs": ctypes.c_void_p(0x200002)}, MIS),
    ({"b": 0}, BATCH), ({"out": 3}, DTYPE), ({"k": (1 << 30) + 16, "b": 1}, SHAPE),
])
def test_fp8_validation(kw, status):
    assert _fp8(**kw) == status


def test_plan_validation():
    # an out-of-range plan field is rejected before any device call
    bad = B.qg_plan(3, 0, 0)
    assert LIB.qgemv_fp4_e2m1_plan(A, A2, A3, A4, 8, 64, 32, 1, 0, ctypes.byref(bad), None) == SHAPE
    bad = B.qg_plan(0, 9, 0)
    assert LIB.qgemv_fp8_e4m3_plan(A, A2, A3, A4, 8, 64, 1, 0, ctypes.byref(bad), None) == SHAPE
    bad = B.qg_plan(0, 0, -1)
    assert LIB.qgemv_affine_u4_plan(A, A2, A2, A3, A4, 8, 128, 64, 1, 0, ctypes.byref(bad), None) == SHAPE


def test_plan_query_needs_a_device():
    """qg_plan_query never launches; without a GPU it reports QG_ERR_DEVICE."""
    import torch
    plan = B.qg_plan()
    st = q.lib().qg_plan_query(0, 64, 512, 1, ctypes.byref(plan))
    if torch.cuda.is_available():
        assert st == OK and plan.blocks >= 1 and plan.rows_per_tile in (1, 2, 4)
    else:
        assert st == 10


def test_one_hip_runtime_in_the_process():
    """PyTorch ships its own copy of the HIP runtime; the binding loads it before
    the library, so the process maps exactly one libamdhip64 (a second copy would
    not know the device pointers of the first)."""
    import torch  # noqa: F401  (what the GPU tests import after this module)
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths

def test_standalone_norm_limits():
    fn = LIB.qg_rmsnorm_bf16
    assert fn(A, A2, 1e-5, A3, (1 << 23) + 8, 1, None) == LARGE     # the row's group sums exceed 64 KiB
    assert fn(A, A2, 1e-5, A3, 12, 1, None) == SHAPE                # k % 8
    assert fn(A, A2, 1e-5, A3, 64, 5, None) == BATCH
    assert fn(A, ODD, 1e-5, A3, 64, 1, None) == MIS
    assert fn(A, A2, -1.0, A3, 64, 1, None) == VALUE
    assert fn(None, A2, 1e-5, A3, 64, 1, None) == NULL


def test_qgemm_argument_errors():
    fn = LIB.qgemm_fp4_e2m1
    assert fn(None, A2, A3, A4, 64, 256, 32, 8, 0, None) == NULL
    assert fn(A, A2, A3, A4, 0, 256, 32, 8, 0, None) == SHAPE               # n < 1
    assert fn(A, A2, A3, A4, 64, 16, 32, 8, 0, None) == SHAPE               # k < 32
    assert fn(A, A2, A3, A4, 64, 272, 32, 8, 0, None) == SHAPE              # k % 32
    assert fn(A, A2, A3, A4, 64, 256, 48, 8, 0, None) == GROUP
    assert fn(A, A2, A3, A4, 64, 320, 128, 8, 0, None) == GROUP             # k % group_size
    assert fn(A, A2, A3, A4, 64, 256, 32, 0, 0, None) == BATCH
    assert fn(A, A2, A3, A4, 64, 256, 32, 65537, 0, None) == BATCH          # above QG_GEMM_MAX_M
    assert fn(A, A2, A3, A4, 64, 256, 32, 8, 2, None) == DTYPE
    assert fn(ODD, A2, A3, A4, 64, 256, 32, 8, 0, None) == MIS              # codes 8-byte aligned only
    assert fn(A, A2, ODD, A4, 64, 256, 32, 8, 0, None) == MIS               # x
    assert fn(A, A2, A3, ctypes.c_void_p(0x400002), 64, 256, 32, 8, 0, None) == MIS   # f32 y 2-byte aligned


def test_qgemm_affine_argument_errors():
    fn = LIB.qgemm_affine_u4
    assert fn(None, A2, A2, A3, A4, 64, 256, 64, 8, 0, None) == NULL
    assert fn(A, A2, None, A3, A4, 64, 256, 64, 8, 0, None) == NULL          # biases
    assert fn(A, A2, A2, A3, A4, 0, 256, 64, 8, 0, None) == SHAPE
    assert fn(A, A2, A2, A3, A4, 64, 272, 64, 8, 0, None) == SHAPE            # k % 32
    assert fn(A, A2, A2, A3, A4, 64, 256, 16, 8, 0, None) == GROUP
    assert fn(A, A2, A2, A3, A4, 64, 320, 128, 8, 0, None) == GROUP           # k % group_size
    assert fn(A, A2, A2, A3, A4, 64, 256, 64, 0, 0, None) == BATCH
    assert fn(A, A2, A2, A3, A4, 64, 256, 64, 65537, 0, None) == BATCH
    assert fn(A, A2, A2, A3, A4, 64, 256, 64, 8, 2, None) == DTYPE
    assert fn(ODD, A2, A2, A3, A4, 64, 256, 64, 8, 0, None) == MIS
    assert fn(A, A2, ctypes.c_void_p(0x400001), A3, A4, 64, 256, 64, 8, 0, None) == MIS   # biases odd


def _q8(codes=A, scales=A2, biases=A2, xq=A3, ds=A4, y=A4, n=8, k=128, gs=64, b=1, out=0):
    return LIB.qgemv_affine_u4_q8(codes, scales, biases, xq, ds, y, n, k, gs, b, out, None)


def _q8f(codes=A, scales=A2, biases=A2, x=A3, y=A4, n=8, k=128, gs=64, b=1, out=0):
    return LIB.qgemv_affine_u4_q8_fused(codes, scales, biases, x, y, n, k, gs, b, out, None)


@pytest.mark.parametrize("kw,status", [
    ({"codes": None}, NULL), ({"biases": None}, NULL), ({"xq": None}, NULL), ({"ds": None}, NULL),
    ({"n": 0}, SHAPE), ({"k": 48}, SHAPE), ({"k": 0}, SHAPE), ({"gs": 16}, GROUP), ({"k": 96, "gs": 64}, GROUP),
    ({"codes": ODD}, MIS), ({"xq": ODD}, MIS), ({"ds": ctypes.c_void_p(0x200002)}, MIS),
    ({"b": 0}, BATCH), ({"b": 5}, BATCH), ({"out": 2}, DTYPE), ({"k": 1 << 17, "b": 1}, LARGE),
])
def test_int8_route_validation(kw, status):
    # every argument error is returned before any device call
    assert _q8(**kw) == status


@pytest.mark.parametrize("kw,status", [
    ({"x": None}, NULL), ({"x": ODD}, MIS), ({"k": 40}, SHAPE), ({"gs": 256}, GROUP), ({"b": 6}, BATCH),
    ({"k": 32768, "b": 4}, LARGE),
])
def test_int8_route_fused_validation(kw, status):
    assert _q8f(**kw) == status


def test_int8_quantize_validation():
    fn = LIB.qg_quantize_q8_1
    assert fn(None, 64, 1, A3, A4, None) == NULL
    assert fn(A3, 48, 1, A3, A4, None) == SHAPE
    assert fn(A3, 0, 1, A3, A4, None) == SHAPE
    assert fn(A3, 64, 0, A3, A4, None) == BATCH
    assert fn(A3, 64, 1, ODD, A4, None) == MIS


@pytest.mark.parametrize("name", ["qgemv_affine_u8_q8", "qgemv_affine_u8_q8_fused"])
def test_int8_route_u8_validation(name):
    fn = getattr(LIB, name)
    if name.endswith("fused"):
        call = lambda **kw: fn(kw.get("codes", A), A2, A2, kw.get("x", A3), A4, 8, kw.get("k", 128),   # noqa: E731
                               kw.get("gs", 64), kw.get("b", 1), 0, None)
    else:
        call = lambda **kw: fn(kw.get("codes", A), A2, A2, kw.get("x", A3), A4, A4, 8, kw.get("k", 128),  # noqa: E731
                               kw.get("gs", 64), kw.get("b", 1), 0, None)
    assert call(codes=None) == NULL
    assert call(x=None) == NULL
    assert call(k=48) == SHAPE
    assert call(gs=16) == GROUP
    assert call(b=5) == BATCH
    assert call(codes=ODD) == MIS
    assert call(k=1 << 17) == LARGE


# Declarations that carry no passage of the pages: the library's plumbing.
# The *_plan variants compute what their plain call computes (cited there);
# only the launch shape differs.
UNCITED_PLUMBING = {"qg_status_string", "qg_abi_version", "qg_plan_query", "qgemv_fp4_e2m1_plan",
                    "qgemv_affine_u4_plan", "qgemv_affine_u8_plan", "qgemv_fp8_e4m3_plan", "qgemv_q4k_plan"}
PAGE_TITLES = re.compile(r"Hand-Writing Gemma 4 Flash-Decoding \+ an FP4 Matvec Bonus \(Part 2\)|"
                         r"mlxcel issue #683|generalize Gemma 4 batched prefill")


def test_every_declaration_cites_its_passage():
    """Each entry point's governing comment in include/qgemv.h (the last
    comment block before its declaration) names the page it follows, with a
    section in quotes, except the plumbing listed above."""
    text = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    names = []
    for m in re.finditer(r"^(?:qg_status|int64_t|int|const char \*)\s*\*?\s*(\w+)\(", text, re.M):
        name = m.group(1)
        names.append(name)
        if name in UNCITED_PLUMBING:
            continue
        end = text.rfind("*/", 0, m.start())
        comment = re.sub(r"\s*\n\s*\*?\s*", " ", text[text.rfind("/*", 0, end):end])   # one line
        assert PAGE_TITLES.search(comment), "%s: no page cited" % name
        assert re.search(r'"[^"]+"', comment), "%s: no section named" % name
    assert UNCITED_PLUMBING <= set(names)


def _q4k(codes=A, sub=A2, sup=A2, x=A3, y=A4, n=8, k=512, b=1, out=0):
    return LIB.qgemv_q4k(codes, sub, sup, x, y, n, k, b, out, None)


@pytest.mark.parametrize("kw,status", [
    ({"codes": None}, NULL), ({"sub": None}, NULL), ({"sup": None}, NULL), ({"x": None}, NULL),
    ({"k": 384}, SHAPE), ({"k": 0}, SHAPE), ({"n": 0}, SHAPE), ({"codes": ODD}, MIS),
    ({"sup": ctypes.c_void_p(0x200002)}, MIS), ({"sub": ctypes.c_void_p(0x200001)}, MIS),
    ({"b": 0}, BATCH), ({"b": 5}, BATCH), ({"out": 2}, DTYPE),
])
def test_q4k_validation(kw, status):
    # every argument error is returned before any device call
    assert _q4k(**kw) == status

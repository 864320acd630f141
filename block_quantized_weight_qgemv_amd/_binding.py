"""ctypes declarations of libqgemv.so (the C ABI in include/qgemv.h).

Loading fails loudly: there is no fallback implementation of any entry point.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

# QG_ABI_VERSION of include/qgemv.h that these declarations follow; a
# library that reports another version is refused at load.
ABI_VERSION = 6

QG_OK = 0
QG_OUT_F32 = 0
QG_OUT_BF16 = 1
QG_FMT_FP4_E2M1 = 0
QG_FMT_AFFINE_U4 = 1
QG_FMT_AFFINE_U8 = 2
QG_FMT_FP8_E4M3 = 3
QG_FMT_Q4K = 4

STATUS_NAMES = {
    0: "QG_OK", 1: "QG_ERR_NULL_POINTER", 2: "QG_ERR_BAD_SHAPE", 3: "QG_ERR_BAD_GROUP_SIZE",
    4: "QG_ERR_MISALIGNED", 5: "QG_ERR_BAD_BATCH", 6: "QG_ERR_BAD_DTYPE", 7: "QG_ERR_BAD_BITS",
    8: "QG_ERR_BAD_VALUE", 9: "QG_ERR_TOO_LARGE", 10: "QG_ERR_DEVICE", 11: "QG_ERR_LAUNCH",
}


class qg_plan(ctypes.Structure):
    _fields_ = [("rows_per_tile", ctypes.c_int32),
                ("waves_per_block", ctypes.c_int32),
                ("blocks", ctypes.c_int32)]


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_st = ctypes.c_int

# name -> (restype, argtypes)
SIGNATURES = {
    "qgemv_fp4_e2m1": (_st, [_p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemv_fp4_e2m1_plan": (_st, [_p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p, _p]),
    "qgemv_affine_u4": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemv_affine_u4_plan": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p, _p]),
    "qgemv_affine_u8": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemv_affine_u8_plan": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p, _p]),
    "qgemv_fp8_e4m3": (_st, [_p, _p, _p, _p, _i64, _i64, _i32, _i32, _p]),
    "qgemv_fp8_e4m3_plan": (_st, [_p, _p, _p, _p, _i64, _i64, _i32, _i32, _p, _p]),
    "qgemv_fp4_e2m1_rmsnorm": (_st, [_p, _p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i32, _i32, _i32, _p, _p]),
    "qgemv_affine_u4_rmsnorm": (_st, [_p, _p, _p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i32, _i32, _i32,
                                      _p, _p]),
    "qgemv_affine_u8_rmsnorm": (_st, [_p, _p, _p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i32, _i32, _i32,
                                      _p, _p]),
    "qgemv_fp8_e4m3_rmsnorm": (_st, [_p, _p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i32, _i32, _p, _p]),
    "qgemv_q4k": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _p]),
    "qgemv_q4k_plan": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _p, _p]),
    "qgemv_q4k_rmsnorm": (_st, [_p, _p, _p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i32, _i32, _p, _p]),
    "qg_quantize_q4k": (_st, [_p, _i64, _i64, _p]),
    "qg_repack_q4k": (_st, [_p, _i64, _i64, _p, _p, _p]),
    "qg_bytes_q4k_records": (_i64, [_i64, _i64]),
    "qg_bytes_q4k": (_i64, [_i64, _i64]),
    "qg_rmsnorm_bf16": (_st, [_p, _p, ctypes.c_float, _p, _i64, _i32, _p]),
    "qgemm_fp4_e2m1": (_st, [_p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemm_affine_u4": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qg_quantize_q8_1": (_st, [_p, _i64, _i32, _p, _p, _p]),
    "qgemv_affine_u4_q8": (_st, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemv_affine_u4_q8_fused": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemv_affine_u8_q8": (_st, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qgemv_affine_u8_q8_fused": (_st, [_p, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i32, _p]),
    "qg_plan_query": (_st, [_i32, _i64, _i64, _i32, _p]),
    "qg_stream_probe": (_st, [_p, _i64, _i32, _i32, _i32, _i32, _p, _p]),
    "qg_status_string": (ctypes.c_char_p, [_st]),
    "qg_abi_version": (ctypes.c_int, []),
    "qg_quantize_fp4_e2m1": (_st, [_p, _i64, _i64, _i32, _p, _p]),
    "qg_quantize_affine": (_st, [_p, _i64, _i64, _i32, _i32, _p, _p, _p]),
    "qg_quantize_fp8_e4m3_rowwise": (_st, [_p, _i64, _i64, _p, _p]),
    "qg_pack_nibbles": (_st, [_p, _i64, _p]),
    "qg_unpack_nibbles": (_st, [_p, _i64, _p]),
    "qg_pack_u32": (_st, [_p, _i64, _i32, _p]),
    "qg_unpack_u32": (_st, [_p, _i64, _i32, _p]),
    "qg_bytes_fp4": (_i64, [_i64, _i64, _i32]),
    "qg_bytes_affine": (_i64, [_i64, _i64, _i32, _i32]),
    "qg_bytes_fp8": (_i64, [_i64, _i64]),
}


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            "libqgemv.so is not built (%s); run `python block_quantized_weight_qgemv_amd/build.py` "
            "or __graft_entry__.build()" % path)
    # PyTorch ships its own copy of the HIP runtime (same soname as ROCm's,
    # another file).  The library must share the process's one with the
    # tensors it is handed, so torch is loaded first: the library's
    # dependency on libamdhip64.so.7 then resolves to the copy already in
    # the process.  Loading the library first would put two HIP runtimes in
    # the process, and device pointers of one are unknown to the other.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.qg_abi_version() != ABI_VERSION:
        raise ImportError("%s reports ABI version %d, the binding declares %d: rebuild the library"
                          % (path, lib.qg_abi_version(), ABI_VERSION))
    return lib

"""MI355X-native block-quantized weight matvec: Python binding of libqgemv.so.

Argument marshalling only: every function forwards to the C entry point of
the same name (include/qgemv.h).  Device entry points take torch tensors that
already live on the GPU (torch is used for device memory and streams only)
and enqueue the HIP kernel on the current torch stream (or ``stream``); the
host pack module takes and returns numpy arrays.

Importing this package loads libqgemv.so and raises ImportError if it is not
built; nothing here computes a matvec on the CPU.
"""

import ctypes

import numpy as np

from . import _binding as _b

_lib = _b.load()

QG_FMT_FP4_E2M1 = _b.QG_FMT_FP4_E2M1
QG_FMT_AFFINE_U4 = _b.QG_FMT_AFFINE_U4
QG_FMT_AFFINE_U8 = _b.QG_FMT_AFFINE_U8
QG_FMT_FP8_E4M3 = _b.QG_FMT_FP8_E4M3
QG_FMT_Q4K = _b.QG_FMT_Q4K
qg_plan = _b.qg_plan

__all__ = [
    "QgError", "qgemv_fp4_e2m1", "qgemv_affine_u4", "qgemv_affine_u8", "qgemv_fp8_e4m3", "qgemm_fp4_e2m1",
    "qgemm_affine_u4",
    "qg_quantize_q8_1", "qgemv_affine_u4_q8", "qgemv_affine_u4_q8_fused", "qgemv_affine_u8_q8",
    "qgemv_affine_u8_q8_fused",
    "qg_plan", "qg_plan_query", "qg_stream_probe", "qg_status_string", "qg_abi_version",
    "qg_quantize_fp4_e2m1", "qg_quantize_affine", "qg_quantize_fp8_e4m3_rowwise",
    "qg_pack_nibbles", "qg_unpack_nibbles", "qg_pack_u32", "qg_unpack_u32",
    "qg_bytes_fp4", "qg_bytes_affine", "qg_bytes_fp8", "lib",
    "qgemv_q4k", "qg_quantize_q4k", "qg_repack_q4k", "qg_bytes_q4k", "qg_bytes_q4k_records", "QG_FMT_Q4K",
]


def lib():
    """The loaded ctypes library (for callers that marshal pointers themselves)."""
    return _lib


class QgError(RuntimeError):
    def __init__(self, status, where):
        self.status = int(status)
        self.name = _b.STATUS_NAMES.get(self.status, "unknown")
        super().__init__("%s: %s (%s)" % (where, _lib.qg_status_string(self.status).decode(), self.name))


def _check(status, where):
    if status != _b.QG_OK:
        raise QgError(status, where)


def qg_status_string(status):
    return _lib.qg_status_string(int(status)).decode()


def qg_abi_version():
    return int(_lib.qg_abi_version())


# ------------------------------------------------------------------ device entry points

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtypes, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.dim() not in ndim:
        raise ValueError("%s must have %s dimensions, has %d" % (name, ndim, t.dim()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _x_y(x, y, n):
    torch = _torch()
    xp = _dev_ptr(x, "x", (torch.bfloat16, torch.int16, torch.uint16), (1, 2))
    batch = 1 if x.dim() == 1 else x.shape[0]
    k = x.shape[-1]
    yp = _dev_ptr(y, "y", (torch.float32, torch.bfloat16), (1, 2))
    if y.numel() != batch * n or (y.dim() == 2 and tuple(y.shape) != (batch, n)):
        raise ValueError("y must be [batch=%d, n=%d], got %s" % (batch, n, tuple(y.shape)))
    out = _b.QG_OUT_F32 if y.dtype == torch.float32 else _b.QG_OUT_BF16
    if x.device != y.device:
        raise ValueError("x and y are on different devices")
    return xp, yp, batch, k, out


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _plan_ptr(plan):
    if plan is None:
        return None
    if isinstance(plan, dict):
        plan = qg_plan(**plan)
    return ctypes.byref(plan)


def _same_device(*ts):
    devs = {t.device for t in ts}
    if len(devs) != 1:
        raise ValueError("all tensors must be on one device, got %s" % devs)


def _gamma(gamma, k, x):
    torch = _torch()
    gp = _dev_ptr(gamma, "gamma", (torch.bfloat16, torch.int16, torch.uint16), (1,))
    if gamma.shape[0] != k:
        raise ValueError("gamma must have k=%d values, has %d" % (k, gamma.shape[0]))
    _same_device(gamma, x)
    return gp


def qgemv_fp4_e2m1(codes, scales, x, y, group_size, plan=None, stream=None):
    """y[b, n] = sum_k scale[n, k//gs] * E2M1(code[n, k]) * x[b, k].

    codes uint8 [n, k/2] (even column in the low nibble), scales bf16 [n, k/gs],
    x bf16 [batch, k] (or [k]), y float32 or bf16 [batch, n].
    """
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.uint8,), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] * 2 != k or tuple(scales.shape) != (n, k // group_size):
        raise ValueError("shapes: codes %s, scales %s, k=%d, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), k, group_size))
    _same_device(codes, scales, x, y)
    st = _lib.qgemv_fp4_e2m1_plan(cp, sp, xp, yp, n, k, int(group_size), batch, out,
                                  _plan_ptr(plan), _stream(stream, y.device))
    _check(st, "qgemv_fp4_e2m1")
    return y


def qgemm_fp4_e2m1(codes, scales, x, y, group_size, stream=None):
    """Y[m, n] = X[m, k] . W[n, k]^T for m activation rows (any m >= 1; the
    matvec entry points are faster for m <= 4), W as in qgemv_fp4_e2m1.

    codes uint8 [n, k/2], scales bf16 [n, k/gs], x bf16 [m, k], y float32 or bf16 [m, n].
    """
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.uint8,), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    n = codes.shape[0]
    xp, yp, m, k, out = _x_y(x, y, n)
    if codes.shape[1] * 2 != k or tuple(scales.shape) != (n, k // group_size):
        raise ValueError("shapes: codes %s, scales %s, k=%d, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), k, group_size))
    _same_device(codes, scales, x, y)
    st = _lib.qgemm_fp4_e2m1(cp, sp, xp, yp, n, k, int(group_size), m, out, _stream(stream, y.device))
    _check(st, "qgemm_fp4_e2m1")
    return y


def qgemm_affine_u4(codes, scales, biases, x, y, group_size=64, stream=None):
    """Y[m, n] = X[m, k] . W[n, k]^T for m activation rows, W affine 4-bit as
    in qgemv_affine_u4 (codes int32/uint32 [n, k/8], scales and biases bf16
    [n, k/gs]); x bf16 [m, k], y float32 or bf16 [m, n]."""
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.int32, torch.uint32), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    bp = _dev_ptr(biases, "biases", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    n = codes.shape[0]
    xp, yp, m, k, out = _x_y(x, y, n)
    if codes.shape[1] * 8 != k or tuple(scales.shape) != (n, k // group_size) \
            or tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("shapes: codes %s, scales %s, biases %s, k=%d, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), tuple(biases.shape), k, group_size))
    _same_device(codes, scales, biases, x, y)
    st = _lib.qgemm_affine_u4(cp, sp, bp, xp, yp, n, k, int(group_size), m, out, _stream(stream, y.device))
    _check(st, "qgemm_affine_u4")
    return y


def qgemv_fp4_e2m1_rmsnorm(codes, scales, x, gamma, eps, y, group_size, plan=None, stream=None):
    """y = W . RMSNorm(x) in one launch: x~ = bf16(x * gamma / sqrt(mean(x^2) + eps)) per batch row.

    As qgemv_fp4_e2m1, plus gamma bf16 [k] and eps >= 0.
    """
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.uint8,), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] * 2 != k or tuple(scales.shape) != (n, k // group_size):
        raise ValueError("shapes: codes %s, scales %s, k=%d, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), k, group_size))
    gp = _gamma(gamma, k, x)
    _same_device(codes, scales, x, y)
    st = _lib.qgemv_fp4_e2m1_rmsnorm(cp, sp, xp, gp, float(eps), yp, n, k, int(group_size), batch, out,
                                     _plan_ptr(plan), _stream(stream, y.device))
    _check(st, "qgemv_fp4_e2m1_rmsnorm")
    return y


def _affine(name, bits, codes, scales, biases, x, y, group_size, plan, stream, gamma=None, eps=0.0):
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.int32, torch.uint32), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    bp = _dev_ptr(biases, "biases", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] * (32 // bits) != k or tuple(scales.shape) != (n, k // group_size) \
            or tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("shapes: codes %s, scales %s, biases %s, k=%d, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), tuple(biases.shape), k, group_size))
    _same_device(codes, scales, biases, x, y)
    if gamma is None:
        fn = getattr(_lib, name + "_plan")
        st = fn(cp, sp, bp, xp, yp, n, k, int(group_size), batch, out, _plan_ptr(plan), _stream(stream, y.device))
        _check(st, name)
    else:
        gp = _gamma(gamma, k, x)
        fn = getattr(_lib, name + "_rmsnorm")
        st = fn(cp, sp, bp, xp, gp, float(eps), yp, n, k, int(group_size), batch, out, _plan_ptr(plan),
                _stream(stream, y.device))
        _check(st, name + "_rmsnorm")
    return y


def qgemv_q4k(codes, sub, sup, x, y, plan=None, stream=None, gamma=None, eps=0.0):
    """Two-level super-block 4-bit weights in the device layout of qg_repack_q4k:
    y[b, n] = sum_k (d*sc*q - dmin*m)[n, k] * x[b, k].

    codes uint32 [n, k/8], sub uint16 [n, k/32] (sc | m << 8), sup uint32
    [n, k/256] (fp16 d | dmin << 16), x bf16 [batch, k], y float32 or bf16.
    With gamma (bf16 [k]) the call is the fused-RMSNorm variant.
    """
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.int32, torch.uint32), (2,))
    bp = _dev_ptr(sub, "sub", (torch.int16, torch.uint16), (2,))
    sp = _dev_ptr(sup, "sup", (torch.int32, torch.uint32), (2,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] * 8 != k or tuple(sub.shape) != (n, k // 32) or tuple(sup.shape) != (n, k // 256):
        raise ValueError("shapes: codes %s, sub %s, sup %s, k=%d"
                         % (tuple(codes.shape), tuple(sub.shape), tuple(sup.shape), k))
    _same_device(codes, sub, sup, x, y)
    if gamma is None:
        st = _lib.qgemv_q4k_plan(cp, bp, sp, xp, yp, n, k, batch, out, _plan_ptr(plan), _stream(stream, y.device))
        _check(st, "qgemv_q4k")
    else:
        gp = _gamma(gamma, k, x)
        st = _lib.qgemv_q4k_rmsnorm(cp, bp, sp, xp, gp, float(eps), yp, n, k, batch, out, _plan_ptr(plan),
                                    _stream(stream, y.device))
        _check(st, "qgemv_q4k_rmsnorm")
    return y


def qgemv_affine_u4(codes, scales, biases, x, y, group_size=64, plan=None, stream=None):
    """y[b, n] = sum_k (scale[n,g] * q[n,k] + bias[n,g]) * x[b,k], 4-bit u32 low-first codes [n, k/8]."""
    return _affine("qgemv_affine_u4", 4, codes, scales, biases, x, y, group_size, plan, stream)


def qg_quantize_q8_1(x, xq=None, ds=None, stream=None):
    """bf16 x [batch, k] -> (xq int8 [batch, k], ds fp16 bits int16 [batch, k/32, 2] = {d, s}) on x's device."""
    torch = _torch()
    xp = _dev_ptr(x, "x", (torch.bfloat16, torch.int16, torch.uint16), (1, 2))
    batch = 1 if x.dim() == 1 else x.shape[0]
    k = x.shape[-1]
    if xq is None:
        xq = torch.empty((batch, k), dtype=torch.int8, device=x.device)
    if ds is None:
        ds = torch.empty((batch, k // 32, 2), dtype=torch.int16, device=x.device)
    qp = _dev_ptr(xq, "xq", (torch.int8,), (1, 2))
    dp = _dev_ptr(ds, "ds", (torch.int16, torch.uint16, torch.float16), (2, 3))
    if xq.numel() != batch * k or ds.numel() != batch * (k // 32) * 2:
        raise ValueError("xq must hold [batch=%d, k=%d], ds [batch, k/32, 2]" % (batch, k))
    _same_device(x, xq, ds)
    _check(_lib.qg_quantize_q8_1(xp, k, batch, qp, dp, _stream(stream, x.device)), "qg_quantize_q8_1")
    return xq, ds


def _affine_q8(name, bits, codes, scales, biases, xq, ds, y, group_size, stream):
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.int32, torch.uint32), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    bp = _dev_ptr(biases, "biases", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    qp = _dev_ptr(xq, "xq", (torch.int8,), (1, 2))
    dp = _dev_ptr(ds, "ds", (torch.int16, torch.uint16, torch.float16), (2, 3))
    yp = _dev_ptr(y, "y", (torch.float32, torch.bfloat16), (1, 2))
    n = codes.shape[0]
    batch = 1 if xq.dim() == 1 else xq.shape[0]
    k = xq.shape[-1]
    if codes.shape[1] * (32 // bits) != k or tuple(scales.shape) != (n, k // group_size) \
            or tuple(biases.shape) != tuple(scales.shape) or ds.numel() != batch * (k // 32) * 2:
        raise ValueError("shapes: codes %s, scales %s, biases %s, xq %s, ds %s, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), tuple(biases.shape), tuple(xq.shape),
                            tuple(ds.shape), group_size))
    if y.numel() != batch * n or (y.dim() == 2 and tuple(y.shape) != (batch, n)):
        raise ValueError("y must be [batch=%d, n=%d], got %s" % (batch, n, tuple(y.shape)))
    out = _b.QG_OUT_F32 if y.dtype == torch.float32 else _b.QG_OUT_BF16
    _same_device(codes, scales, biases, xq, ds, y)
    _check(getattr(_lib, name)(cp, sp, bp, qp, dp, yp, n, k, int(group_size), batch, out,
                               _stream(stream, y.device)), name)
    return y


def _affine_q8_fused(name, bits, codes, scales, biases, x, y, group_size, stream):
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.int32, torch.uint32), (2,))
    sp = _dev_ptr(scales, "scales", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    bp = _dev_ptr(biases, "biases", (torch.bfloat16, torch.int16, torch.uint16), (2,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] * (32 // bits) != k or tuple(scales.shape) != (n, k // group_size) \
            or tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("shapes: codes %s, scales %s, biases %s, k=%d, group_size=%d"
                         % (tuple(codes.shape), tuple(scales.shape), tuple(biases.shape), k, group_size))
    _same_device(codes, scales, biases, x, y)
    _check(getattr(_lib, name)(cp, sp, bp, xp, yp, n, k, int(group_size), batch, out,
                               _stream(stream, y.device)), name)
    return y


def qgemv_affine_u4_q8(codes, scales, biases, xq, ds, y, group_size=64, stream=None):
    """Affine u4 weights against int8 activation blocks from qg_quantize_q8_1:
    y[b, n] = sum_blk scale * d * sum(u * q) + bias * s."""
    return _affine_q8("qgemv_affine_u4_q8", 4, codes, scales, biases, xq, ds, y, group_size, stream)


def qgemv_affine_u4_q8_fused(codes, scales, biases, x, y, group_size=64, stream=None):
    """qg_quantize_q8_1 then qgemv_affine_u4_q8 in one launch (bitwise the same y)."""
    return _affine_q8_fused("qgemv_affine_u4_q8_fused", 4, codes, scales, biases, x, y, group_size, stream)


def qgemv_affine_u8_q8(codes, scales, biases, xq, ds, y, group_size=64, stream=None):
    """As qgemv_affine_u4_q8 for 8-bit codes, u32 low-first [n, k/4]."""
    return _affine_q8("qgemv_affine_u8_q8", 8, codes, scales, biases, xq, ds, y, group_size, stream)


def qgemv_affine_u8_q8_fused(codes, scales, biases, x, y, group_size=64, stream=None):
    """qg_quantize_q8_1 then qgemv_affine_u8_q8 in one launch (bitwise the same y)."""
    return _affine_q8_fused("qgemv_affine_u8_q8_fused", 8, codes, scales, biases, x, y, group_size, stream)


def qgemv_affine_u8(codes, scales, biases, x, y, group_size=64, plan=None, stream=None):
    """As qgemv_affine_u4 with 8-bit codes, u32 low-first [n, k/4]."""
    return _affine("qgemv_affine_u8", 8, codes, scales, biases, x, y, group_size, plan, stream)


def qg_rmsnorm_bf16(x, gamma, eps, out=None, stream=None):
    """out = bf16(x * gamma / sqrt(mean(x^2) + eps)) per row, exactly as the fused variants normalize x."""
    torch = _torch()
    xp = _dev_ptr(x, "x", (torch.bfloat16, torch.int16, torch.uint16), (1, 2))
    batch = 1 if x.dim() == 1 else x.shape[0]
    k = x.shape[-1]
    gp = _gamma(gamma, k, x)
    if out is None:
        out = torch.empty_like(x)
    op = _dev_ptr(out, "out", (torch.bfloat16, torch.int16, torch.uint16), (1, 2))
    if out.numel() != batch * k:
        raise ValueError("out must hold batch * k = %d values" % (batch * k))
    _same_device(x, out)
    st = _lib.qg_rmsnorm_bf16(xp, gp, float(eps), op, k, batch, _stream(stream, x.device))
    _check(st, "qg_rmsnorm_bf16")
    return out


def qgemv_affine_u4_rmsnorm(codes, scales, biases, x, gamma, eps, y, group_size=64, plan=None, stream=None):
    """y = W . RMSNorm(x) in one launch, 4-bit affine codes (see qgemv_fp4_e2m1_rmsnorm)."""
    return _affine("qgemv_affine_u4", 4, codes, scales, biases, x, y, group_size, plan, stream, gamma, eps)


def qgemv_affine_u8_rmsnorm(codes, scales, biases, x, gamma, eps, y, group_size=64, plan=None, stream=None):
    """y = W . RMSNorm(x) in one launch, 8-bit affine codes (see qgemv_fp4_e2m1_rmsnorm)."""
    return _affine("qgemv_affine_u8", 8, codes, scales, biases, x, y, group_size, plan, stream, gamma, eps)


def qgemv_fp8_e4m3(codes, row_scale, x, y, plan=None, stream=None):
    """y[b, n] = row_scale[n] * sum_k E4M3(code[n, k]) * x[b, k]; codes uint8 [n, k], row_scale f32 [n]."""
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.uint8,), (2,))
    rp = _dev_ptr(row_scale, "row_scale", (torch.float32,), (1,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] != k or row_scale.shape[0] != n:
        raise ValueError("shapes: codes %s, row_scale %s, k=%d" % (tuple(codes.shape), tuple(row_scale.shape), k))
    _same_device(codes, row_scale, x, y)
    st = _lib.qgemv_fp8_e4m3_plan(cp, rp, xp, yp, n, k, batch, out, _plan_ptr(plan), _stream(stream, y.device))
    _check(st, "qgemv_fp8_e4m3")
    return y


def qgemv_fp8_e4m3_rmsnorm(codes, row_scale, x, gamma, eps, y, plan=None, stream=None):
    """y = W . RMSNorm(x) in one launch, FP8-E4M3 codes with row scales (see qgemv_fp4_e2m1_rmsnorm)."""
    torch = _torch()
    cp = _dev_ptr(codes, "codes", (torch.uint8,), (2,))
    rp = _dev_ptr(row_scale, "row_scale", (torch.float32,), (1,))
    n = codes.shape[0]
    xp, yp, batch, k, out = _x_y(x, y, n)
    if codes.shape[1] != k or row_scale.shape[0] != n:
        raise ValueError("shapes: codes %s, row_scale %s, k=%d" % (tuple(codes.shape), tuple(row_scale.shape), k))
    gp = _gamma(gamma, k, x)
    _same_device(codes, row_scale, x, y)
    st = _lib.qgemv_fp8_e4m3_rmsnorm(cp, rp, xp, gp, float(eps), yp, n, k, batch, out, _plan_ptr(plan),
                                     _stream(stream, y.device))
    _check(st, "qgemv_fp8_e4m3_rmsnorm")
    return y


def qg_stream_probe(buf, pattern=1, unroll=8, blocks=1024, threads_per_block=256, out=None, stream=None):
    """Read every byte of the device tensor `buf` (the HBM read-bandwidth reference)."""
    torch = _torch()
    if not (isinstance(buf, torch.Tensor) and buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(blocks * threads_per_block, dtype=torch.int32, device=buf.device)
    st = _lib.qg_stream_probe(ctypes.c_void_p(buf.data_ptr()), nbytes, int(pattern), int(unroll),
                              int(blocks), int(threads_per_block), ctypes.c_void_p(out.data_ptr()),
                              _stream(stream, buf.device))
    _check(st, "qg_stream_probe")
    return out


def qg_plan_query(fmt, n, k, batch=1):
    """The launch shape the plain entry point would use on the current device."""
    p = qg_plan()
    _check(_lib.qg_plan_query(int(fmt), int(n), int(k), int(batch), ctypes.byref(p)), "qg_plan_query")
    return {"rows_per_tile": p.rows_per_tile, "waves_per_block": p.waves_per_block, "blocks": p.blocks}


# ------------------------------------------------------------------ host pack module

def _host_in(a, dtype, name):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, np.dtype(dtype), a.dtype))
    return a


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def qg_quantize_fp4_e2m1(w, group_size=32):
    """float32 [n, k] -> (codes uint8 [n, k/2], scales bf16 bits uint16 [n, k/gs])."""
    w = _host_in(w, np.float32, "w")
    n, k = w.shape
    codes = np.empty((n, k // 2), np.uint8)
    scales = np.empty((n, max(k // int(group_size), 1)), np.uint16)
    _check(_lib.qg_quantize_fp4_e2m1(_ptr(w), n, k, int(group_size), _ptr(codes), _ptr(scales)),
           "qg_quantize_fp4_e2m1")
    return codes, scales


def qg_quantize_affine(w, bits, group_size=64):
    """float32 [n, k] -> (codes uint32 [n, k*bits/32], scales, biases bf16 bits [n, k/gs])."""
    w = _host_in(w, np.float32, "w")
    n, k = w.shape
    per = 32 // int(bits) if bits in (4, 8) else 1
    codes = np.empty((n, max(k // per, 1)), np.uint32)
    scales = np.empty((n, max(k // int(group_size), 1)), np.uint16)
    biases = np.empty_like(scales)
    _check(_lib.qg_quantize_affine(_ptr(w), n, k, int(bits), int(group_size), _ptr(codes),
                                   _ptr(scales), _ptr(biases)), "qg_quantize_affine")
    return codes, scales, biases


def qg_quantize_q4k(w):
    """float32 [n, k] -> storage records uint8 [n, k/256, 144] of the two-level format."""
    w = _host_in(w, np.float32, "w")
    n, k = w.shape
    rec = np.empty((n, max(k // 256, 1), 144), np.uint8)
    _check(_lib.qg_quantize_q4k(_ptr(w), n, k, _ptr(rec)), "qg_quantize_q4k")
    return rec


def qg_repack_q4k(records):
    """Storage records [n, k/256, 144] -> the device layout (codes uint32
    [n, k/8], sub uint16 [n, k/32], sup uint32 [n, k/256])."""
    rec = _host_in(records, np.uint8, "records")
    n, nsb = rec.shape[0], rec.shape[1]
    k = nsb * 256
    codes = np.empty((n, k // 8), np.uint32)
    sub = np.empty((n, k // 32), np.uint16)
    sup = np.empty((n, nsb), np.uint32)
    _check(_lib.qg_repack_q4k(_ptr(rec), n, k, _ptr(codes), _ptr(sub), _ptr(sup)), "qg_repack_q4k")
    return codes, sub, sup


def qg_quantize_fp8_e4m3_rowwise(w):
    """float32 [n, k] -> (codes uint8 [n, k], row_scale float32 [n])."""
    w = _host_in(w, np.float32, "w")
    n, k = w.shape
    codes = np.empty((n, k), np.uint8)
    rs = np.empty(n, np.float32)
    _check(_lib.qg_quantize_fp8_e4m3_rowwise(_ptr(w), n, k, _ptr(codes), _ptr(rs)),
           "qg_quantize_fp8_e4m3_rowwise")
    return codes, rs


def qg_pack_nibbles(codes):
    c = _host_in(codes, np.uint8, "codes").ravel()
    out = np.empty(c.size // 2, np.uint8)
    _check(_lib.qg_pack_nibbles(_ptr(c), c.size, _ptr(out)), "qg_pack_nibbles")
    return out


def qg_unpack_nibbles(packed, count):
    p = _host_in(packed, np.uint8, "packed").ravel()
    if p.size * 2 < count:
        raise ValueError("packed holds %d codes, asked for %d" % (p.size * 2, count))
    out = np.empty(int(count), np.uint8)
    _check(_lib.qg_unpack_nibbles(_ptr(p), int(count), _ptr(out)), "qg_unpack_nibbles")
    return out


def qg_pack_u32(codes, bits):
    c = _host_in(codes, np.uint8, "codes").ravel()
    out = np.empty(max(c.size * int(bits) // 32, 1), np.uint32)
    _check(_lib.qg_pack_u32(_ptr(c), c.size, int(bits), _ptr(out)), "qg_pack_u32")
    return out


def qg_unpack_u32(packed, count, bits):
    p = _host_in(packed, np.uint32, "packed").ravel()
    if bits in (4, 8) and p.size * (32 // bits) < count:
        raise ValueError("packed holds %d codes, asked for %d" % (p.size * (32 // bits), count))
    out = np.empty(int(count), np.uint8)
    _check(_lib.qg_unpack_u32(_ptr(p), int(count), int(bits), _ptr(out)), "qg_unpack_u32")
    return out


def qg_bytes_fp4(n, k, group_size=32):
    return int(_lib.qg_bytes_fp4(int(n), int(k), int(group_size)))


def qg_bytes_affine(n, k, bits, group_size=64):
    return int(_lib.qg_bytes_affine(int(n), int(k), int(bits), int(group_size)))


def qg_bytes_fp8(n, k):
    return int(_lib.qg_bytes_fp8(int(n), int(k)))


def qg_bytes_q4k(n, k):
    """Bytes of the super-block format's device layout (what qgemv_q4k reads)."""
    return int(_lib.qg_bytes_q4k(int(n), int(k)))


def qg_bytes_q4k_records(n, k):
    """Bytes of the super-block format's storage records."""
    return int(_lib.qg_bytes_q4k_records(int(n), int(k)))

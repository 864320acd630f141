"""Helpers for the GPU tests: upload numpy arrays, run an entry point through
the binding (which calls the C ABI), and bring y back to the host."""

import sys

import numpy as np
import torch

import block_quantized_weight_qgemv_amd as q

DEV = "cuda:0"


def log(msg):
    """Name the case before each GPU step (a fault can end the process)."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def out_tensor(batch, n, bf16=False, fill=float("nan")):
    dt = torch.bfloat16 if bf16 else torch.float32
    return torch.full((batch, n), fill, dtype=dt, device=DEV)


def host_y(y):
    torch.cuda.synchronize()
    if y.dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


def run(fmt, arrays, x, n, bits=None, gs=None, bf16=False, plan=None):
    """arrays: host packed weights of the format; x: bf16 bits [B, K]. Returns host y."""
    x = np.atleast_2d(x)
    y = out_tensor(x.shape[0], n, bf16)
    xd = dev(x)
    if fmt == "fp4":
        codes, scales = arrays
        q.qgemv_fp4_e2m1(dev(codes), dev(scales), xd, y, gs, plan=plan)
    elif fmt == "u4":
        codes, scales, biases = arrays
        q.qgemv_affine_u4(dev(codes), dev(scales), dev(biases), xd, y, gs, plan=plan)
    elif fmt == "u8":
        codes, scales, biases = arrays
        q.qgemv_affine_u8(dev(codes), dev(scales), dev(biases), xd, y, gs, plan=plan)
    elif fmt == "fp8":
        codes, rs = arrays
        q.qgemv_fp8_e4m3(dev(codes), dev(rs), xd, y, plan=plan)
    else:
        raise ValueError(fmt)
    return host_y(y)

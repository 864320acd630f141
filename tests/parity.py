"""The parity criterion between a GPU result and the oracle (shared test helper).

A GPU result y (fp32) passes against the oracle's float64 y_ref and conditioning
mass A = sum_k |w x| when, for every element,

    |y - y_ref| / max(|y_ref|, 2**-12 * A)  <=  1e-3

The 1e-3 relative bound is the stated target; the 2**-12 * A floor only applies
to rows whose exact value nearly cancels (|y_ref| << A), where a plain relative
error is unbounded for any fp32 summation order.  Reports also carry the
unguarded maximum relative error and how many elements used the floor.
"""

import numpy as np

RTOL = 1e-3
GUARD = 2.0 ** -12


def report(y, y_ref, a_ref, rtol=RTOL, guard=GUARD):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    a_ref = np.asarray(a_ref, dtype=np.float64)
    assert y.shape == y_ref.shape == a_ref.shape, (y.shape, y_ref.shape, a_ref.shape)
    floor = guard * a_ref
    denom = np.maximum(np.abs(y_ref), floor)
    diff = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(denom > 0, diff / denom, np.where(diff == 0, 0.0, np.inf))
        plain = np.where(np.abs(y_ref) > 0, diff / np.abs(y_ref), np.where(diff == 0, 0.0, np.inf))
    worst = float(np.max(err)) if err.size else 0.0
    return {
        "ok": bool(np.all(np.isfinite(y)) and worst <= rtol),
        "max_err": worst,
        "unguarded_max_rel": float(np.max(plain)) if plain.size else 0.0,
        "guarded_elems": int(np.count_nonzero(floor > np.abs(y_ref))),
        "elems": int(y.size),
    }


def assert_parity(y, y_ref, a_ref, what=""):
    r = report(y, y_ref, a_ref)
    assert r["ok"], "parity failed %s: %r" % (what, r)
    return r

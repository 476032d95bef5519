"""Shared helpers for the GPU parity tests: device transfer and the error metrics.

Tolerances (forward and decode: max and mean |dO| over all compared elements, max |dLSE|
over all compared rows; backward: relative L2 error per tensor).
"""
import numpy as np

FWD_MAX = 2e-2
FWD_MEAN = 2e-3
LSE_MAX = 1e-3
BWD_REL_L2 = 1e-2


def to_dev(arr):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def fwd_errors(o, o_ref, lse=None, lse_ref=None):
    d = np.abs(o - o_ref)
    out = {"max": float(d.max()), "mean": float(d.mean())}
    if lse is not None:
        out["lse"] = float(np.abs(lse - lse_ref).max())
    return out


def assert_fwd_ok(err, tag=""):
    assert err["max"] <= FWD_MAX, (tag, err)
    assert err["mean"] <= FWD_MEAN, (tag, err)
    if "lse" in err:
        assert err["lse"] <= LSE_MAX, (tag, err)


def rel_l2(x, ref):
    return float(np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel()))

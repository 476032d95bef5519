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


# Guard regions: outputs and workspaces handed to the kernels sit inside a larger buffer whose
# margins hold a sentinel byte, so a write past either end of any of them (a wrong offset, a
# clamped buffer resource that reaches too far) changes a margin byte and fails the test.
GUARD_BYTES = 4096
GUARD_FILL = 0xA5


class Guarded:
    def __init__(self):
        self.bufs = []

    def empty(self, shape, dtype):
        """A contiguous tensor of `shape` and `dtype` (16-byte aligned) between two margins."""
        import torch
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((2 * GUARD_BYTES + n,), GUARD_FILL, dtype=torch.uint8, device="cuda")
        self.bufs.append(buf)
        return buf[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(*shape)

    def like(self, t):
        return self.empty(tuple(t.shape), t.dtype)

    def check(self, tag=""):
        import torch
        torch.cuda.synchronize()
        for i, buf in enumerate(self.bufs):
            lo, hi = buf[:GUARD_BYTES], buf[buf.numel() - GUARD_BYTES:]
            assert bool((lo == GUARD_FILL).all()), (tag, f"buffer {i}: write before the start")
            assert bool((hi == GUARD_FILL).all()), (tag, f"buffer {i}: write past the end")

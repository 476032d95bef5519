"""GPU parity of the Nq != Nk forward (attn_fwd_kv: chunked prefill, multi-token decode, causal
mask aligned at the bottom right) and of the packed variable-length forward (attn_fwd_varlen)
against the fp64 oracle on the same seeded inputs.

Rows that see no key must come back as exactly O = 0 and LSE = -inf; the other rows are held
to the forward tolerances.  Dense and packed calls on the same data must agree bitwise with
attn_fwd where the work per tile is the same.
"""
import numpy as np
import pytest

import oracle
from synth import default_scale, make_prefill, make_varlen
from tests._util import BWD_REL_L2, Guarded, assert_fwd_ok, fwd_errors, rel_l2, to_dev, to_host64

pytestmark = pytest.mark.gpu


def check_rows(o, lse, o_ref, lse_ref, tag):
    """Rows without keys (reference LSE = -inf) exactly; the rest within tolerance."""
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), (tag, "rows without keys differ")
    assert np.all(o[empty] == 0.0), (tag, "rows without keys must give O = 0")
    if (~empty).any():
        assert_fwd_ok(fwd_errors(o[~empty], o_ref[~empty], lse[~empty], lse_ref[~empty]), tag)


def run_kv(lib, inp, causal, scale):
    import torch
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    g = Guarded()
    o, lse = g.like(q), g.empty(q.shape[:3], torch.float32)
    lib.attn_fwd_kv(q, k, v, causal, scale, o=o, lse=lse)
    g.check("attn_fwd_kv")
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


SHAPES = [(1, 1), (1, 1000), (7, 333), (64, 64), (100, 257), (256, 4096), (300, 1000), (333, 333),
          (1000, 300), (257, 1)]


@pytest.mark.parametrize("Nq,Nk", SHAPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_kv_shapes(gpu_lib, Nq, Nk, d, causal):
    print(f"fwd_kv Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
    inp = make_prefill(1, 4, 2, Nq, d, "bf16", seed=2000 + Nq + Nk, qk_mult=2.0, L=Nk)
    scale = default_scale(d)
    o, lse = run_kv(gpu_lib, inp, causal, scale)
    o_ref, lse_ref = oracle.forward_kv(inp["q"], inp["k"], inp["v"], scale, causal)
    check_rows(o, lse, o_ref, lse_ref, f"Nq={Nq} Nk={Nk} d={d} causal={causal}")


@pytest.mark.parametrize("Nq,Nk", [(5, 200), (200, 5), (128, 128), (31, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_kv_fp32(gpu_lib, Nq, Nk, causal):
    print(f"fwd_kv fp32 Nq={Nq} Nk={Nk} causal={causal}", flush=True)
    inp = make_prefill(2, 2, 1, Nq, 64, "f32", seed=2100 + Nq, L=Nk)
    scale = default_scale(64)
    o, lse = run_kv(gpu_lib, inp, causal, scale)
    o_ref, lse_ref = oracle.forward_kv(inp["q"], inp["k"], inp["v"], scale, causal)
    check_rows(o, lse, o_ref, lse_ref, "fp32")
    empty = np.isneginf(lse_ref)
    if (~empty).any():
        assert np.abs(o[~empty] - o_ref[~empty]).max() <= 5e-5  # fp32 path keeps fp32 precision


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_kv_no_keys(gpu_lib, d):
    """An empty key sequence: every row is O = 0, LSE = -inf."""
    import torch
    q = to_dev(make_prefill(1, 2, 2, 70, d, "bf16", seed=2200)["q"])
    k = torch.empty((1, 2, 0, d), dtype=torch.bfloat16, device=q.device)
    for causal in (False, True):
        o, lse = gpu_lib.attn_fwd_kv(q, k, k, causal, default_scale(d))
        torch.cuda.synchronize()
        assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_kv_square_is_attn_fwd_bitwise(gpu_lib, d):
    """Nq == Nk runs the same tiles as attn_fwd: identical bits."""
    import torch
    inp = make_prefill(2, 4, 2, 300, d, "bf16", seed=2300 + d)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    for causal in (False, True):
        o1, l1 = gpu_lib.attn_fwd(q, k, v, causal, default_scale(d))
        o2, l2 = gpu_lib.attn_fwd_kv(q, k, v, causal, default_scale(d))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_kv_chunked_prefill_full_size(gpu_lib):
    """A 512-token chunk appended to a 16K-token causal context (B=1, Hq=32, Hkv=8, d=128):
    whole heads 0 and 31 against the oracle."""
    Nq, Nk, d = 512, 16384, 128
    print(f"fwd_kv chunk Nq={Nq} Nk={Nk}", flush=True)
    inp = make_prefill(1, 32, 8, Nq, d, "bf16", seed=2400, qk_mult=2.0, L=Nk)
    scale = default_scale(d)
    o, lse = run_kv(gpu_lib, inp, True, scale)
    for h in (0, 31):
        kv = h // 4
        o_ref, lse_ref = oracle.forward_kv(inp["q"][:, h:h + 1], inp["k"][:, kv:kv + 1], inp["v"][:, kv:kv + 1],
                                           scale, True)
        check_rows(o[:, h:h + 1], lse[:, h:h + 1], o_ref, lse_ref, f"chunk h{h}")


# ----------------------------------------------------------------------------- packed
def run_varlen(lib, x, causal, scale):
    import torch
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    cq, ck = torch.from_numpy(x["cu_q"]).cuda(), torch.from_numpy(x["cu_k"]).cuda()
    max_q = int(np.diff(x["cu_q"]).max())
    g = Guarded()
    o, lse = g.like(q), g.empty(q.shape[:2], torch.float32)
    lib.attn_fwd_varlen(q, k, v, cq, ck, max_q, causal, scale, o=o, lse=lse)
    g.check("attn_fwd_varlen")
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


LENS_Q = [0, 1, 63, 64, 65, 256, 257, 1000, 300, 2]
VARLEN_CASES = {
    "self": (LENS_Q, LENS_Q),                                        # training-style packing
    "prefix": (LENS_Q, [n + p for n, p in zip(LENS_Q, [5, 0, 700, 64, 1, 3, 256, 9, 2000, 0])]),
    "short_keys": (LENS_Q, [0, 1, 10, 64, 0, 100, 257, 999, 1, 5]),  # some Nk < Nq, some empty
}


@pytest.mark.parametrize("case", sorted(VARLEN_CASES))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_varlen(gpu_lib, case, d, causal):
    print(f"fwd_varlen {case} d={d} causal={causal}", flush=True)
    lq, lk = VARLEN_CASES[case]
    x = make_varlen(lq, lk, 4, 2, d, "bf16", seed=2500 + d, qk_mult=2.0)
    scale = default_scale(d)
    o, lse = run_varlen(gpu_lib, x, causal, scale)
    o_ref, lse_ref = oracle.forward_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], scale, causal)
    check_rows(o, lse, o_ref, lse_ref, f"{case} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_varlen_fp32(gpu_lib, causal):
    x = make_varlen([3, 130, 0, 77], [50, 130, 9, 20], 2, 1, 64, "f32", seed=2600)
    o, lse = run_varlen(gpu_lib, x, causal, default_scale(64))
    o_ref, lse_ref = oracle.forward_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], default_scale(64), causal)
    check_rows(o, lse, o_ref, lse_ref, "fp32")


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_varlen_equal_lengths_is_attn_fwd_bitwise(gpu_lib, d):
    """Equal lengths packed with the batch folded into the rows: the same tiles as the dense
    call, so the same bits."""
    import torch
    B, H, N = 3, 4, 333
    inp = make_prefill(B, H, H, N, d, "bf16", seed=2700 + d)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    fold = lambda t: t.transpose(0, 1).reshape(H, B * N, d).contiguous()
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32, device=q.device)
    for causal in (False, True):
        o1, l1 = gpu_lib.attn_fwd(q, k, v, causal, default_scale(d))
        o2, l2 = gpu_lib.attn_fwd_varlen(fold(q), fold(k), fold(v), cu, cu, N, causal, default_scale(d))
        torch.cuda.synchronize()
        assert torch.equal(fold(o1), o2)
        assert torch.equal(l1.transpose(0, 1).reshape(H, B * N), l2)


# ----------------------------------------------------------------------------- packed backward
def run_varlen_fwd_bwd(lib, x, causal, scale):
    import torch
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "dout"))
    cq, ck = torch.from_numpy(x["cu_q"]).cuda(), torch.from_numpy(x["cu_k"]).cuda()
    max_q, max_k = int(np.diff(x["cu_q"]).max()), int(np.diff(x["cu_k"]).max())
    o, lse = lib.attn_fwd_varlen(q, k, v, cq, ck, max_q, causal, scale)
    g = Guarded()
    grads = (g.like(q), g.like(k), g.like(v))
    ws = g.empty((lib.attn_bwd_varlen_workspace_bytes(len(x["cu_q"]) - 1, q.shape[0], q.shape[1]),), torch.uint8)
    lib.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, max_q, max_k, causal, scale, dq=grads[0], dk=grads[1],
                        dv=grads[2], workspace=ws)
    g.check("attn_bwd_varlen")
    return [to_host64(t) for t in grads]


@pytest.mark.parametrize("case", sorted(VARLEN_CASES))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen(gpu_lib, case, d, causal):
    print(f"bwd_varlen {case} d={d} causal={causal}", flush=True)
    lq, lk = VARLEN_CASES[case]
    x = make_varlen(lq, lk, 4, 2, d, "bf16", seed=2800 + d, with_dout=True)
    scale = default_scale(d)
    dq, dk, dv = run_varlen_fwd_bwd(gpu_lib, x, causal, scale)
    ref = oracle.backward_varlen(x["q"], x["k"], x["v"], x["dout"], x["cu_q"], x["cu_k"], scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        err = rel_l2(g, r)
        assert err <= BWD_REL_L2, (case, d, causal, name, err)
    # Rows the mask leaves without any gradient: queries that see no key (no keys, or causal
    # with i < Nq - Nk) and keys of sequences without queries must be exactly 0.
    q_dead = np.zeros(x["q"].shape[1], bool)
    k_dead = np.zeros(x["k"].shape[1], bool)
    for b, (nq, nk) in enumerate(zip(lq, lk)):
        q0, k0 = x["cu_q"][b], x["cu_k"][b]
        if nk == 0:
            q_dead[q0:q0 + nq] = True
        elif causal and nq > nk:
            q_dead[q0:q0 + nq - nk] = True
        if nq == 0:
            k_dead[k0:k0 + nk] = True
    assert np.all(dq[:, q_dead] == 0.0) and np.all(dk[:, k_dead] == 0.0) and np.all(dv[:, k_dead] == 0.0), case


def test_bwd_varlen_equal_lengths_is_attn_bwd_bitwise(gpu_lib):
    """Equal lengths packed with the batch folded into the rows: same tiles as the dense backward."""
    import torch
    B, H, N, d = 2, 4, 333, 128
    inp = make_prefill(B, H, H, N, d, "bf16", seed=2900, with_dout=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    fold = lambda t: t.transpose(0, 1).reshape(t.shape[1], B * t.shape[2], *t.shape[3:]).contiguous()
    cu = torch.arange(0, B * N + 1, N, dtype=torch.int32, device=q.device)
    for causal in (False, True):
        o, lse = gpu_lib.attn_fwd(q, k, v, causal, default_scale(d))
        g1 = gpu_lib.attn_bwd(q, k, v, o, lse, do, causal, default_scale(d))
        g2 = gpu_lib.attn_bwd_varlen(fold(q), fold(k), fold(v), fold(o), fold(lse), fold(do), cu, cu, N, N, causal,
                                     default_scale(d))
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(fold(a), b)


@pytest.fixture(scope="module")
def two_million_keys():
    return make_prefill(1, 1, 1, 8, 64, "bf16", seed=2950, L=(1 << 21) + 5)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_kv_two_million_keys(gpu_lib, two_million_keys, causal):
    """Byte offsets near the top of one head's range: 8 queries against 2^21 + 5 keys (d = 64,
    K and V 256 MiB each), every row against the oracle."""
    inp = two_million_keys
    print(f"fwd_kv Nq=8 Nk={inp['k'].shape[2]} causal={causal}", flush=True)
    scale = default_scale(64)
    o, lse = run_kv(gpu_lib, inp, causal, scale)
    o_ref, lse_ref = oracle.forward_kv(inp["q"], inp["k"], inp["v"], scale, causal)
    check_rows(o, lse, o_ref, lse_ref, f"causal={causal}")

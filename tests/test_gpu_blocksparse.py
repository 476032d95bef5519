"""GPU parity of the block-sparse forward (attn_fwd_blocksparse) against the fp64 oracle:
random per-head block masks over ragged shapes, a banded long-sequence pattern, masks that
drop whole rows of blocks, and bitwise agreement with the dense call when nothing is dropped.
"""
import numpy as np
import pytest

import oracle
from synth import default_scale, make_prefill
from tests._util import Guarded, to_dev, to_host64
from tests.test_gpu_kv_varlen import check_rows

pytestmark = pytest.mark.gpu
BLK = 128


def nblk(n):
    return -(-n // BLK)


def run_sparse(lib, inp, mask, causal, scale):
    import torch
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    g = Guarded()
    o, lse = g.like(q), g.empty(q.shape[:3], torch.float32)
    lib.attn_fwd_blocksparse(q, k, v, m, causal, scale, o=o, lse=lse)
    g.check("attn_fwd_blocksparse")
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("Nq,Nk", [(64, 64), (300, 300), (256, 1000), (1000, 333), (129, 4097)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.1, 0.5])
def test_blocksparse_random_masks(gpu_lib, Nq, Nk, d, causal, density):
    print(f"blocksparse Nq={Nq} Nk={Nk} d={d} causal={causal} density={density}", flush=True)
    B, Hq, Hkv = 1, 4, 2
    inp = make_prefill(B, Hq, Hkv, Nq, d, "bf16", seed=3000 + Nq + Nk, qk_mult=2.0, L=Nk)
    rng = np.random.default_rng(3100 + Nq + d)
    mask = (rng.random((B, Hq, nblk(Nq), nblk(Nk))) < density).astype(np.uint8)
    mask[0, 0, 0, :] = 0                       # a query block that keeps nothing
    scale = default_scale(d)
    o, lse = run_sparse(gpu_lib, inp, mask, causal, scale)
    o_ref, lse_ref = oracle.forward_blocksparse(inp["q"], inp["k"], inp["v"], mask, scale, causal)
    check_rows(o, lse, o_ref, lse_ref, f"Nq={Nq} Nk={Nk} d={d} causal={causal}")


def test_blocksparse_banded_long(gpu_lib):
    """N=8192, d=128, causal, each query block keeps its own and the three previous key blocks
    plus key block 0 (B=1, Hq=8, Hkv=2): whole heads 0 and 7 against the oracle."""
    N, d, Hq, Hkv = 8192, 128, 8, 2
    print(f"blocksparse banded N={N}", flush=True)
    inp = make_prefill(1, Hq, Hkv, N, d, "bf16", seed=3200, qk_mult=2.0)
    nb = nblk(N)
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    mask = (((i - j) >= 0) & ((i - j) < 4) | (j == 0)).astype(np.uint8)
    scale = default_scale(d)
    o, lse = run_sparse(gpu_lib, inp, mask, True, scale)
    for h in (0, 7):
        kv = h // (Hq // Hkv)
        o_ref, lse_ref = oracle.forward_blocksparse(inp["q"][:, h:h + 1], inp["k"][:, kv:kv + 1],
                                                    inp["v"][:, kv:kv + 1], mask, scale, True)
        check_rows(o[:, h:h + 1], lse[:, h:h + 1], o_ref, lse_ref, f"banded h{h}")


@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_full_mask_is_dense_and_empty_mask_is_empty(gpu_lib, d):
    import torch
    inp = make_prefill(2, 4, 2, 333, d, "bf16", seed=3300 + d, L=700)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    ones = torch.ones((nblk(333), nblk(700)), dtype=torch.uint8, device=q.device)
    for causal in (False, True):
        o1, l1 = gpu_lib.attn_fwd_kv(q, k, v, causal, default_scale(d))
        o2, l2 = gpu_lib.attn_fwd_blocksparse(q, k, v, ones, causal, default_scale(d))
        o3, l3 = gpu_lib.attn_fwd_blocksparse(q, k, v, torch.zeros_like(ones), causal, default_scale(d))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.all(o3 == 0) and torch.all(torch.isneginf(l3))


def test_blocksparse_shared_mask_equals_per_head_copy(gpu_lib):
    import torch
    inp = make_prefill(2, 4, 4, 500, 128, "bf16", seed=3400)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    rng = np.random.default_rng(3401)
    m2 = torch.from_numpy((rng.random((4, 4)) < 0.5).astype(np.uint8)).cuda()
    m4 = m2.expand(2, 4, 4, 4).contiguous()
    o1, l1 = gpu_lib.attn_fwd_blocksparse(q, k, v, m2, True, default_scale(128))
    o2, l2 = gpu_lib.attn_fwd_blocksparse(q, k, v, m4, True, default_scale(128))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------- backward
from tests._util import BWD_REL_L2, rel_l2  # noqa: E402


def run_sparse_fwd_bwd(lib, inp, mask, causal, scale):
    import torch
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    o, lse = lib.attn_fwd_blocksparse(q, k, v, m, causal, scale)
    g = Guarded()
    grads = (g.like(q), g.like(k), g.like(v))
    B, Hq, N, d = q.shape
    ws = g.empty((max(lib.attn_bwd_workspace_bytes(B, Hq, k.shape[1], N, d), 1),), torch.uint8)
    lib.attn_bwd_blocksparse(q, k, v, o, lse, do, m, causal, scale, dq=grads[0], dk=grads[1], dv=grads[2],
                             workspace=ws)
    g.check("attn_bwd_blocksparse")
    return [to_host64(t) for t in grads]


@pytest.mark.parametrize("N", [300, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.3, 0.7])
def test_bwd_blocksparse_random_masks(gpu_lib, N, d, causal, density):
    print(f"bwd blocksparse N={N} d={d} causal={causal} density={density}", flush=True)
    B, Hq, Hkv = 1, 4, 2
    inp = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=3500 + N + d, with_dout=True)
    rng = np.random.default_rng(3600 + N + d + int(causal))
    nb = nblk(N)
    mask = (rng.random((B, Hq, nb, nb)) < density).astype(np.uint8)
    mask[0, 1, 0, :] = 0       # a query block that keeps nothing
    mask[0, 2, :, nb - 1] = 0  # a key block that head 2 never keeps
    scale = default_scale(d)
    dq, dk, dv = run_sparse_fwd_bwd(gpu_lib, inp, mask, causal, scale)
    ref = oracle.backward_blocksparse(inp["q"], inp["k"], inp["v"], inp["dout"], mask, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        err = rel_l2(g, r)
        assert err <= BWD_REL_L2, (N, d, causal, density, name, err)
    assert np.all(dq[0, 1, :min(BLK, N)] == 0.0)  # rows that keep no key


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_blocksparse_full_mask_is_attn_bwd_bitwise(gpu_lib, d):
    import torch
    N = 333
    inp = make_prefill(2, 4, 2, N, d, "bf16", seed=3700 + d, with_dout=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    ones = torch.ones((nblk(N), nblk(N)), dtype=torch.uint8, device=q.device)
    for causal in (False, True):
        o, lse = gpu_lib.attn_fwd(q, k, v, causal, default_scale(d))
        g1 = gpu_lib.attn_bwd(q, k, v, o, lse, do, causal, default_scale(d))
        g2 = gpu_lib.attn_bwd_blocksparse(q, k, v, o, lse, do, ones, causal, default_scale(d))
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_per_batch_masks_fwd_bwd(gpu_lib, causal):
    """Masks that differ per batch row and per head ([B, Hq, nqb, nkb]; both strides used),
    forward and backward against the oracle."""
    B, Hq, Hkv, N, d = 2, 4, 2, 520, 128
    inp = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=3800 + int(causal), qk_mult=2.0, with_dout=True)
    rng = np.random.default_rng(3900 + int(causal))
    mask = (rng.random((B, Hq, nblk(N), nblk(N))) < 0.5).astype(np.uint8)
    mask[1, 3] = 0
    mask[1, 3, :, 0] = 1       # batch 1, head 3: only the first key block
    scale = default_scale(d)
    o, lse = run_sparse(gpu_lib, inp, mask, causal, scale)
    o_ref, lse_ref = oracle.forward_blocksparse(inp["q"], inp["k"], inp["v"], mask, scale, causal)
    check_rows(o, lse, o_ref, lse_ref, f"per-batch causal={causal}")
    grads = run_sparse_fwd_bwd(gpu_lib, inp, mask, causal, scale)
    ref = oracle.backward_blocksparse(inp["q"], inp["k"], inp["v"], inp["dout"], mask, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        assert rel_l2(g, r) <= BWD_REL_L2, (name, rel_l2(g, r))

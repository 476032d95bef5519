"""Randomised GPU parity sweep: forward, backward and the Nq != Nk forward on seeded random
shapes against the fp64 oracle, every element compared; then decode with per-sequence lengths
on seeded random batches (test_random_decode_lengths).

Shapes: N near and off the tile sizes (1 to 700), d in {64, 128}, group sizes 1 to 8, one or
two batches, causal or not, logits x1 or x2 (rows dominated by one key).  Bounds as everywhere:
forward max |dO| <= 2e-2, mean <= 2e-3, |dLSE| <= 1e-3; backward relative L2 <= 1e-2 per tensor.
"""
import numpy as np
import pytest

import oracle
from synth import default_scale, make_prefill
from tests._util import BWD_REL_L2, assert_fwd_ok, fwd_errors, rel_l2, to_dev, to_host64

pytestmark = pytest.mark.gpu

NS = [1, 2, 31, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257, 383, 511, 513, 700]


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        d = int(rng.choice([64, 128]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        hkv = int(rng.integers(1, 3))
        out.append(dict(B=int(rng.integers(1, 3)), Hq=g * hkv, Hkv=hkv, N=int(rng.choice(NS)), d=d,
                        causal=bool(rng.integers(0, 2)), qk=2.0 if rng.integers(0, 2) else 1.0, seed=9000 + c))
    return out


@pytest.mark.parametrize("case", _cases(11, 96), ids=lambda c: f"B{c['B']}-{c['Hq']}/{c['Hkv']}-N{c['N']}-d{c['d']}-"
                         f"{'c' if c['causal'] else 'f'}-x{int(c['qk'])}")
def test_random_shape(gpu_lib, case):
    import torch
    B, Hq, Hkv, N, d, causal = (case[x] for x in ("B", "Hq", "Hkv", "N", "d", "causal"))
    inp = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=case["seed"], with_dout=True, qk_mult=case["qk"])
    scale = default_scale(d)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    o, lse = gpu_lib.attn_fwd(q, k, v, causal, scale)
    dq, dk, dv = gpu_lib.attn_bwd(q, k, v, o, lse, do, causal, scale)
    nq = max(1, N // 3)
    o2, lse2 = gpu_lib.attn_fwd_kv(q[:, :, N - nq:].contiguous(), k, v, causal, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, causal)
    lse_h = lse.cpu().numpy().astype(np.float64)
    assert_fwd_ok(fwd_errors(to_host64(o), o_ref, lse_h, lse_ref), "fwd")
    # The last nq queries against every key are those rows of the square forward.
    assert_fwd_ok(fwd_errors(to_host64(o2), o_ref[:, :, N - nq:], lse2.cpu().numpy().astype(np.float64),
                             lse_ref[:, :, N - nq:]), "fwd_kv")
    refs = oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        h = to_host64(g)
        if not np.any(r):  # one visible key per row: the gradient vanishes exactly
            assert np.abs(h).max() <= 1e-3, (name, np.abs(h).max())
            continue
        assert rel_l2(h, r) <= BWD_REL_L2, (name, rel_l2(h, r))


def _decode_cases(seed, n):
    """Per-sequence-length decode: batch sizes 1 to 40, KV heads 1 to 3, groups 1 to 8 (with T
    tokens, up to 8 rows per KV head: the stream-K path), cache capacities near and off the 32-key
    blocks, lengths drawn from {0, 1, random, L} so that workgroup ranges cross sequences, KV heads
    and empty sequences; split counts 0 (automatic) to 9."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        g = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.choice([t for t in (1, 2, 4, 8) if t * g <= 8]))
        L = int(rng.choice([1, 31, 32, 33, 100, 257, 700]))
        B = int(rng.integers(1, 41))
        lens = [int(rng.choice([0, 1, int(rng.integers(0, L + 1)), L])) for _ in range(B)]
        out.append(dict(B=B, Hkv=int(rng.integers(1, 4)), g=g, T=T, L=L, d=int(rng.choice([64, 128])),
                        causal=bool(rng.integers(0, 2)), splits=int(rng.integers(0, 10)), lens=lens,
                        seed=9500 + c))
    return out


@pytest.mark.parametrize("case", _decode_cases(12, 32), ids=lambda c: f"B{c['B']}-g{c['g']}x{c['Hkv']}-T{c['T']}-"
                         f"L{c['L']}-d{c['d']}-s{c['splits']}-{'c' if c['causal'] else 'f'}")
def test_random_decode_lengths(gpu_lib, case):
    from tests.test_gpu_kv_varlen import check_rows
    from tests.test_gpu_parity import run_decode_multi
    B, Hkv, g, T, L, d = (case[x] for x in ("B", "Hkv", "g", "T", "L", "d"))
    x = make_prefill(B, g * Hkv, Hkv, T, d, "bf16", seed=case["seed"], L=L)
    scale = default_scale(d)
    o, lse = run_decode_multi(gpu_lib, x["q"], x["k"], x["v"], case["lens"], case["causal"], case["splits"], scale)
    o_ref, lse_ref = oracle.decode_multi(x["q"], x["k"], x["v"], scale, case["causal"], seqlens=case["lens"])
    check_rows(o, lse, o_ref, lse_ref, f"decode {case}")

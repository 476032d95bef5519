"""Pins for the fp64 oracle: closed forms, invariants, hand-derived fixtures, brute force.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, a transposed operand, an off-by-one in the mask) fails at least one of them.
The plant tests at the end mutate the oracle on the CPU and assert the pins notice.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_prefill, make_varlen, default_scale

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_prefix_mean(causal):
    B, H, N, d = 2, 3, 37, 8
    q = np.zeros((B, H, N, d))
    k, v = rnd(1, B, H, N, d), rnd(2, B, H, N, d)
    o, lse = oracle.forward(q, k, v, 0.3, causal)
    for i in range(N):
        upto = i + 1 if causal else N
        np.testing.assert_allclose(o[:, :, i], v[:, :, :upto].mean(axis=2), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], math.log(upto), rtol=1e-14)


def test_causal_row0_is_v0():
    B, H, N, d = 1, 2, 19, 16
    q, k, v = rnd(3, B, H, N, d), rnd(4, B, H, N, d), rnd(5, B, H, N, d)
    o, lse = oracle.forward(q, k, v, 0.25, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), rtol=1e-14)


def test_single_key_returns_v():
    q, k, v = rnd(6, 1, 1, 1, 4), rnd(7, 1, 1, 1, 4), rnd(8, 1, 1, 1, 4)
    for causal in (False, True):
        o, _ = oracle.forward(q, k, v, 1.0, causal)
        np.testing.assert_array_equal(o, v)


def test_constant_v_gives_constant_o():
    q, k = rnd(9, 1, 2, 23, 8), rnd(10, 1, 2, 23, 8)
    v = np.ones((1, 2, 23, 8))
    for causal in (False, True):
        o, _ = oracle.forward(q, k, v, 0.7, causal)
        np.testing.assert_allclose(o, 1.0, rtol=1e-14)


@pytest.mark.parametrize("alpha,beta", [(1.0, 2.0), (4.0, 0.5), (2.0, 8.0)])
def test_one_hot_queries_and_keys(alpha, beta):
    """Q_i = alpha e_{a_i}, K_j = beta e_{b_j}: S_ij = scale alpha beta [a_i == b_j]."""
    N, d, scale = 29, 6, 0.125
    rng = np.random.default_rng(11)
    a, b = rng.integers(0, d, N), rng.integers(0, d, N)
    q = np.zeros((1, 1, N, d)); q[0, 0, np.arange(N), a] = alpha
    k = np.zeros((1, 1, N, d)); k[0, 0, np.arange(N), b] = beta
    v = rnd(12, 1, 1, N, 5)
    o, lse = oracle.forward(q, k, v, scale, False)
    w = math.exp(scale * alpha * beta)
    for i in range(N):
        match = b == a[i]
        z = match.sum() * w + (N - match.sum())
        p = np.where(match, w / z, 1.0 / z)
        np.testing.assert_allclose(o[0, 0, i], p @ v[0, 0], rtol=1e-13)
        np.testing.assert_allclose(lse[0, 0, i], math.log(z), rtol=1e-14)


def _golden_rows(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            rows.setdefault(parts[0], {})[int(parts[1])] = np.array([float(x) for x in parts[2:]])
    return rows


def test_hand_derived_2x2_fixture():
    g = _golden_rows("hand_2x2.txt")
    q = np.array([[[[math.log(2), 0.0], [0.0, 0.0]]]])
    k = np.eye(2)[None, None]
    v = np.array([[[[2.0, 0.0], [1.0, 3.0]]]])
    for causal, tag in ((False, "full"), (True, "causal")):
        o, lse = oracle.forward(q, k, v, 1.0, causal)
        for i in range(2):
            np.testing.assert_allclose(o[0, 0, i], g["O_" + tag][i], rtol=1e-15, atol=1e-16)
            np.testing.assert_allclose(lse[0, 0, i], g["LSE_" + tag][i][0], rtol=1e-15)
    dout = np.array([[[[1.0, 0.0], [0.0, 0.0]]]])
    dq, dk, dv = oracle.backward(q, k, v, dout, 1.0, False)
    for name, arr in (("dQ", dq), ("dK", dk), ("dV", dv)):
        for i in range(2):
            np.testing.assert_allclose(arr[0, 0, i], g[name][i], rtol=1e-14, atol=1e-16)


def test_flop_formula_matches_printed_table():
    with open(os.path.join(GOLDEN, "flops_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            n, d, gf = line.split()
            val = oracle.attention_flops(1, 1, int(n), int(d), causal=False) / 1e9
            digits = len(gf.split(".")[1])
            assert round(val, digits) == pytest.approx(float(gf)), (n, d, val, gf)
    assert oracle.attention_flops(2, 16, 4096, 128, True) == 0.5 * 4 * 32 * 4096**2 * 128
    assert oracle.attention_flops(1, 1, 8, 4, True, backward=True) == 2.5 * 0.5 * 4 * 64 * 4


# ----------------------------------------------------------------------------- invariants
def test_probability_rows_sum_to_one_and_mask_is_exact_zero():
    q, k = rnd(13, 40, 16), rnd(14, 40, 16)
    for causal in (False, True):
        p = oracle.probabilities(q, k, 0.5, causal)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
        if causal:
            assert np.all(p[np.triu_indices(40, 1)] == 0.0)
            assert np.all(p[np.tril_indices(40)] > 0.0)


def test_key_shift_leaves_output_and_shifts_lse():
    B, H, N, d, scale = 1, 2, 31, 8, 0.4
    q, k, v = rnd(15, B, H, N, d), rnd(16, B, H, N, d), rnd(17, B, H, N, d)
    u = rnd(18, d)
    for causal in (False, True):
        o1, l1 = oracle.forward(q, k, v, scale, causal)
        o2, l2 = oracle.forward(q, k + u, v, scale, causal)
        np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, scale * (q @ u), rtol=1e-9, atol=1e-11)


def test_output_inside_convex_hull_of_values():
    q, k, v = rnd(19, 1, 1, 50, 8) * 3, rnd(20, 1, 1, 50, 8) * 3, rnd(21, 1, 1, 50, 8)
    for causal in (False, True):
        o, _ = oracle.forward(q, k, v, 1.0, causal)
        for i in range(50):
            upto = i + 1 if causal else 50
            assert np.all(o[0, 0, i] >= v[0, 0, :upto].min(axis=0) - 1e-12)
            assert np.all(o[0, 0, i] <= v[0, 0, :upto].max(axis=0) + 1e-12)


def test_joint_key_value_permutation_invariance():
    q, k, v = rnd(22, 1, 2, 33, 8), rnd(23, 1, 2, 33, 8), rnd(24, 1, 2, 33, 8)
    perm = np.random.default_rng(25).permutation(33)
    o1, l1 = oracle.forward(q, k, v, 0.3, False)
    o2, l2 = oracle.forward(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)


def test_gqa_equals_repeated_kv():
    B, Hq, Hkv, N, d = 2, 6, 2, 17, 8
    q, k, v = rnd(26, B, Hq, N, d), rnd(27, B, Hkv, N, d), rnd(28, B, Hkv, N, d)
    g = Hq // Hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    for causal in (False, True):
        o1, l1 = oracle.forward(q, k, v, 0.35, causal)
        o2, l2 = oracle.forward(q, kr, vr, 0.35, causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
    dout = rnd(29, B, Hq, N, d)
    dq1, dk1, dv1 = oracle.backward(q, k, v, dout, 0.35, True)
    dq2, dk2, dv2 = oracle.backward(q, kr, vr, dout, 0.35, True)
    np.testing.assert_allclose(dq1, dq2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2.reshape(B, Hkv, g, N, d).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(B, Hkv, g, N, d).sum(axis=2), rtol=1e-12, atol=1e-13)


def test_forward_rows_matches_full_forward():
    B, H, N, d = 1, 3, 64, 8
    q, k, v = rnd(30, B, H, N, d), rnd(31, B, H, N, d), rnd(32, B, H, N, d)
    rows = np.array([0, 1, 5, 31, 32, 63])
    for causal in (False, True):
        of, lf = oracle.forward(q, k, v, 0.3, causal)
        orow, lrow = oracle.forward_rows(q, k, v, 0.3, causal, rows)
        np.testing.assert_allclose(orow, of[:, :, rows], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lrow, lf[:, :, rows], rtol=1e-13)


# ----------------------------------------------------------------------------- brute force
def _brute_forward(q, k, v, scale, causal):
    N, d = q.shape
    L = k.shape[0]
    o = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in range(L)
             if not (causal and j > i)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        lse[i] = m + math.log(z)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(e[j] / z * v[j, c] for j in range(len(s)))
    return o, lse


@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 4), (8, 2), (7, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(N, d, causal):
    q, k, v = rnd(33 + N, N, d), rnd(44 + N, N, d), rnd(55 + N, N, d)
    o, lse = oracle.forward(q[None, None], k[None, None], v[None, None], 0.61, causal)
    ob, lb = _brute_forward(q, k, v, 0.61, causal)
    np.testing.assert_allclose(o[0, 0], ob, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lb, rtol=1e-13, atol=1e-13)


def _online_blocked(q, k, v, scale, causal, block, order):
    """Online softmax of "FlashAttention optimisation" §3.2.1 over key blocks in any order.
    A debug model of the method (fp64), used only to pin order independence (§3.2.2)."""
    N, L = q.shape[0], k.shape[0]
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    acc = np.zeros((N, v.shape[1]))
    for j0 in order:
        kb, vb = k[j0:j0 + block], v[j0:j0 + block]
        s = scale * q @ kb.T
        if causal:
            s = np.where(np.arange(j0, j0 + kb.shape[0])[None, :] > np.arange(N)[:, None], -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(m_new), m_new, 0)), 0.0)
        p = np.exp(s - np.where(np.isfinite(m_new), m_new, 0)[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ vb
        m = m_new
    return acc / l[:, None], m + np.log(l)


@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_any_block_order_equals_oracle(causal):
    N, d, blk = 48, 8, 8
    q, k, v = rnd(70, N, d) * 2, rnd(71, N, d) * 2, rnd(72, N, d)
    o, lse = oracle.forward(q[None, None], k[None, None], v[None, None], 0.5, causal)
    rng = np.random.default_rng(73)
    for _ in range(4):
        order = rng.permutation(np.arange(0, N, blk))
        ob, lb = _online_blocked(q, k, v, 0.5, causal, blk, order)
        np.testing.assert_allclose(ob, o[0, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lb, lse[0, 0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- gradients
def _loss(q, k, v, dout, scale, causal):
    o, _ = oracle.forward(q, k, v, scale, causal)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1)])
def test_backward_matches_central_differences(causal, hq, hkv):
    N, d, scale, h = 6, 3, 0.7, 1e-6
    q, k, v = rnd(80, 1, hq, N, d), rnd(81, 1, hkv, N, d), rnd(82, 1, hkv, N, d)
    dout = rnd(83, 1, hq, N, d)
    grads = oracle.backward(q, k, v, dout, scale, causal)
    for idx, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = [q, k, v]; args_p[idx] = xp
            args_m = [q, k, v]; args_m[idx] = xm
            num[pos] = (_loss(*args_p, dout, scale, causal) - _loss(*args_m, dout, scale, causal)) / (2 * h)
        err = np.linalg.norm(num - grads[idx]) / np.linalg.norm(grads[idx])
        assert err < 1e-6, (idx, err)


def test_gradient_sum_identities():
    B, H, N, d = 1, 2, 21, 8
    q, k, v, do = (rnd(90 + i, B, H, N, d) for i in range(4))
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, do, 0.3, causal)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)


def test_equal_value_rows_give_zero_query_and_key_gradients():
    B, H, N, d = 1, 1, 15, 4
    q, k, do = rnd(95, B, H, N, d), rnd(96, B, H, N, d), rnd(97, B, H, N, d)
    v = np.broadcast_to(rnd(98, d), (B, H, N, d)).copy()
    for causal in (False, True):
        dq, dk, _ = oracle.backward(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)


# ----------------------------------------------------------------------------- decode + merge
def test_decode_equals_single_row_forward_and_gqa():
    B, Hq, Hkv, L, d = 2, 8, 2, 40, 8
    q, kc, vc = rnd(100, B, Hq, d), rnd(101, B, Hkv, L, d), rnd(102, B, Hkv, L, d)
    o, lse = oracle.decode(q, kc, vc, 0.2)
    of, lf = oracle.forward(q[:, :, None, :], kc, vc, 0.2, False)
    np.testing.assert_allclose(o, of[:, :, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lf[:, :, 0], rtol=1e-13)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 40])
def test_split_kv_merge_is_independent_of_split_count(splits):
    B, Hq, Hkv, L, d = 1, 4, 1, 40, 8
    q, kc, vc = rnd(103, B, Hq, d) * 2, rnd(104, B, Hkv, L, d) * 2, rnd(105, B, Hkv, L, d)
    o, lse = oracle.decode(q, kc, vc, 0.4)
    os_, ls = oracle.split_kv_decode(q, kc, vc, 0.4, splits)
    np.testing.assert_allclose(os_, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls, lse, rtol=1e-13)


# ----------------------------------------------------------------------------- inputs
def test_bf16_rounding_matches_torch_rne():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]  # ties and a denormal
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_inputs_are_deterministic_and_upcast_exact():
    a = make_prefill(1, 2, 2, 16, 8, "bf16", seed=7, qk_mult=2.0, with_dout=True)
    b = make_prefill(1, 2, 2, 16, 8, "bf16", seed=7, qk_mult=2.0, with_dout=True)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(oracle.upcast(a["q"]), bf16_bits_to_f32(a["q"]).astype(np.float64))
    assert default_scale(128) == float(np.float32(1 / math.sqrt(128)))


# ----------------------------------------------------------------------------- planted slips
@pytest.mark.parametrize("slip", ["no_max_shift_in_lse", "mask_includes_diagonal", "transpose_v",
                                  "mask_aligned_top_left", "block_index_off_by_one"])
def test_planted_mistakes_are_caught(monkeypatch, slip):
    """Plant a plausible mistake in the oracle (CPU only) and check that a pin fails."""
    if slip == "no_max_shift_in_lse":
        orig = A._softmax_rows

        def bad(s):
            p, lse = orig(s)
            return p, lse - np.max(s, axis=1)
        monkeypatch.setattr(A, "_softmax_rows", bad)
        with pytest.raises(AssertionError):
            test_causal_row0_is_v0()
    elif slip == "mask_includes_diagonal":
        orig = A._scores

        def bad(q, k, scale, causal, row_ids=None):
            s = orig(q, k, scale, causal, row_ids)
            if causal:
                n = min(s.shape)
                s = s.copy()
                s[np.arange(1, n), np.arange(1, n)] = -np.inf
            return s
        monkeypatch.setattr(A, "_scores", bad)
        with pytest.raises(AssertionError):
            test_zero_query_gives_prefix_mean(True)
    elif slip == "block_index_off_by_one":
        orig = A.forward_blocksparse

        def bad(q, k, v, block_mask, scale, causal, block=128):   # key j read from block j//block - 1
            return orig(q, k, v, np.roll(np.asarray(block_mask), 1, axis=-1), scale, causal, block)
        monkeypatch.setattr(oracle, "forward_blocksparse", bad)
        with pytest.raises(AssertionError):
            test_blocksparse_equals_gathered_keys()
    elif slip == "mask_aligned_top_left":
        orig = A._scores

        def bad(q, k, scale, causal, row_ids=None):
            return orig(q, k, scale, causal, None)   # ignores the query positions
        monkeypatch.setattr(A, "_scores", bad)
        with pytest.raises(AssertionError):
            test_chunked_prefill_equals_rows_of_full_prefill(True)
    else:
        def bad_forward(q, k, v, scale, causal):
            q, k, v = A.upcast(q), A.upcast(k), A.upcast(v)
            o = np.empty(q.shape[:3] + (v.shape[3],))
            lse = np.empty(q.shape[:3])
            for b in range(q.shape[0]):
                for h in range(q.shape[1]):
                    p, lse[b, h] = A._softmax_rows(A._scores(q[b, h], k[b, h], scale, causal))
                    o[b, h] = p @ v[b, h].T  # square [N, d] tiles only
            return o, lse
        monkeypatch.setattr(oracle, "forward", bad_forward)
        with pytest.raises(AssertionError):
            test_hand_derived_2x2_fixture()


def test_decode_per_sequence_lengths():
    """Per-sequence cache lengths: each row equals the (independently pinned) forward over its
    first n keys, splitting a row's keys and merging by LSE gives the same, full lengths give
    plain decode, and a zero-length sequence gives O = 0, LSE = -inf."""
    B, Hq, Hkv, L, d = 4, 6, 2, 40, 8
    q, kc, vc = rnd(61, B, Hq, d), rnd(62, B, Hkv, L, d), rnd(63, B, Hkv, L, d)
    lens = np.array([0, 1, 17, 40])
    o, lse = oracle.decode(q, kc, vc, 0.4, seqlens=lens)
    for b in range(1, B):
        n = lens[b]
        of, lf = oracle.forward(q[b:b + 1, :, None, :], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], 0.4, False)
        np.testing.assert_allclose(o[b], of[0, :, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], lf[0, :, 0], rtol=1e-13)
    assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
    o1, l1 = oracle.decode(q[2:3], kc[2:3], vc[2:3], 0.4, seqlens=[7])
    o2, l2 = oracle.decode(q[2:3], kc[2:3, :, 7:], vc[2:3, :, 7:], 0.4, seqlens=[10])
    om, lm = oracle.lse_merge([o1, o2], [l1, l2])
    np.testing.assert_allclose(om[0], o[2], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lm[0], lse[2], rtol=1e-13)
    of, lf = oracle.decode(q, kc, vc, 0.4)
    ov, lv = oracle.decode(q, kc, vc, 0.4, seqlens=[L] * B)
    np.testing.assert_array_equal(of, ov)
    np.testing.assert_array_equal(lf, lv)


# ----------------------------------------------------------------------------- Nq != Nk, packed
@pytest.mark.parametrize("causal", [False, True])
def test_chunked_prefill_equals_rows_of_full_prefill(causal):
    """Prefill in chunks: chunk [a, b) of the queries against keys [0, b) gives rows a..b-1 of the
    (independently pinned) full forward; the last chunk against all keys likewise."""
    B, Hq, Hkv, N, d = 1, 4, 2, 37, 8
    q, k, v = rnd(80, B, Hq, N, d), rnd(81, B, Hkv, N, d), rnd(82, B, Hkv, N, d)
    of, lf = oracle.forward(q, k, v, 0.35, causal)
    for a, b in [(0, 1), (0, 16), (16, 17), (17, 30), (30, 37), (36, 37), (0, 37)]:
        kb = b if causal else N      # non-causal queries see every key
        oc, lc = oracle.forward_kv(q[:, :, a:b], k[:, :, :kb], v[:, :, :kb], 0.35, causal)
        np.testing.assert_allclose(oc, of[:, :, a:b], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lc, lf[:, :, a:b], rtol=1e-13)


def test_single_query_forward_kv_is_decode():
    """The last query sees every key, so one query row is decode (pinned on its own)."""
    B, Hq, Hkv, L, d = 2, 4, 1, 29, 8
    q, kc, vc = rnd(83, B, Hq, d), rnd(84, B, Hkv, L, d), rnd(85, B, Hkv, L, d)
    od, ld = oracle.decode(q, kc, vc, 0.5)
    for causal in (False, True):
        o, lse = oracle.forward_kv(q[:, :, None, :], kc, vc, 0.5, causal)
        np.testing.assert_allclose(o[:, :, 0], od, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, 0], ld, rtol=1e-13)


def test_more_queries_than_keys_and_no_keys():
    """Causal with Nk < Nq: rows i < Nq - Nk see no key (O = 0, LSE = -inf); row i >= Nq - Nk
    sees keys 0..i-(Nq-Nk), which is the square causal forward of the last Nk queries.
    Non-causal rows see all Nk keys.  Nk = 0 gives O = 0, LSE = -inf everywhere."""
    B, H, Nq, Nk, d = 1, 2, 12, 5, 4
    q, k, v = rnd(86, B, H, Nq, d), rnd(87, B, H, Nk, d), rnd(88, B, H, Nk, d)
    o, lse = oracle.forward_kv(q, k, v, 0.7, True)
    assert np.all(o[:, :, :Nq - Nk] == 0.0) and np.all(lse[:, :, :Nq - Nk] == -np.inf)
    os_, ls_ = oracle.forward(q[:, :, Nq - Nk:], k, v, 0.7, True)
    np.testing.assert_allclose(o[:, :, Nq - Nk:], os_, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, Nq - Nk:], ls_, rtol=1e-13)
    on, ln = oracle.forward_kv(q, k, v, 0.7, False)
    for i in range(Nq):
        od, ld = oracle.decode(q[:, :, i], k, v, 0.7)
        np.testing.assert_allclose(on[:, :, i], od, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ln[:, :, i], ld, rtol=1e-13)
    for causal in (False, True):
        oz, lz = oracle.forward_kv(q, k[:, :, :0], v[:, :, :0], 0.7, causal)
        assert np.all(oz == 0.0) and np.all(lz == -np.inf)


def _brute_forward_kv(q, k, v, scale, causal):
    """Scalar loops over absolute positions: query i is token Nk - Nq + i of the sequence."""
    Nq, d = q.shape
    Nk = k.shape[0]
    o = np.zeros((Nq, v.shape[1]))
    lse = np.full(Nq, -np.inf)
    for i in range(Nq):
        pos = Nk - Nq + i
        keys = [j for j in range(Nk) if not (causal and j > pos)]
        if not keys:
            continue
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = math.fsum(e)
        lse[i] = m + math.log(z)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(e[t] / z * v[j, c] for t, j in enumerate(keys))
    return o, lse


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 6), (3, 7), (6, 6), (7, 3), (4, 0)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_kv_brute_force_tiny(Nq, Nk, causal):
    q, k, v = rnd(90 + Nq, Nq, 3), rnd(91 + Nk, Nk, 3), rnd(92 + Nk, Nk, 3)
    o, lse = oracle.forward_kv(q[None, None], k[None, None], v[None, None], 0.9, causal)
    ob, lb = _brute_forward_kv(q, k, v, 0.9, causal)
    np.testing.assert_allclose(o[0, 0], ob, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lb, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_varlen_equals_per_sequence_and_dense(causal):
    """Packed sequences: each one equals forward_kv on its own rows (empty ones included), and
    a batch of equal lengths equals the dense forward with the batch folded into the rows."""
    Hq, Hkv, d = 4, 2, 8
    lens_q, lens_k = [5, 0, 9, 1, 3], [7, 4, 9, 0, 2]
    x = make_varlen(lens_q, lens_k, Hq, Hkv, d, "f32", seed=93)
    o, lse = oracle.forward_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], 0.4, causal)
    cq, ck = x["cu_q"], x["cu_k"]
    for b in range(len(lens_q)):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ob, lb = oracle.forward_kv(x["q"][None, :, sq], x["k"][None, :, sk], x["v"][None, :, sk], 0.4, causal)
        np.testing.assert_array_equal(o[:, sq], ob[0])
        np.testing.assert_array_equal(lse[:, sq], lb[0])
    assert np.all(lse[:, cq[3]:cq[4]] == -np.inf)  # sequence 3 has no keys
    B, N = 3, 11
    y = make_prefill(B, Hq, Hkv, N, d, "f32", seed=94)
    od, ld = oracle.forward(y["q"], y["k"], y["v"], 0.4, causal)
    fold = lambda t: np.ascontiguousarray(t.transpose(1, 0, 2, 3).reshape(t.shape[1], B * N, d))
    cu = np.arange(0, B * N + 1, N, dtype=np.int32)
    op, lp = oracle.forward_varlen(fold(y["q"]), fold(y["k"]), fold(y["v"]), cu, cu, 0.4, causal)
    np.testing.assert_allclose(op, fold(od), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lp, ld.transpose(1, 0, 2).reshape(Hq, B * N), rtol=1e-13)


# ----------------------------------------------------------------------------- block-sparse
def test_blocksparse_full_mask_is_forward_kv():
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 11, 19, 4
    q, k, v = rnd(100, B, Hq, Nq, d), rnd(101, B, Hkv, Nk, d), rnd(102, B, Hkv, Nk, d)
    for causal in (False, True):
        o, lse = oracle.forward_blocksparse(q, k, v, np.ones((3, 5)), 0.6, causal, block=4)
        ok, lk = oracle.forward_kv(q, k, v, 0.6, causal)
        np.testing.assert_array_equal(o, ok)
        np.testing.assert_array_equal(lse, lk)


def test_blocksparse_block_diagonal_is_separate_sequences():
    """A block-diagonal mask makes every block an independent sequence: the packed forward
    (independently pinned) over sequences of one block each."""
    Hq, Hkv, blk, nb, d = 2, 2, 5, 4, 6
    lens = [blk] * (nb - 1) + [3]                      # ragged last block
    x = make_varlen(lens, lens, Hq, Hkv, d, "f32", seed=103)
    n = sum(lens)
    for causal in (False, True):
        o, lse = oracle.forward_blocksparse(x["q"][None], x["k"][None], x["v"][None], np.eye(nb), 0.5, causal,
                                            block=blk)
        ov, lv = oracle.forward_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], 0.5, causal)
        np.testing.assert_allclose(o[0], ov, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[0], lv, rtol=1e-13)
        assert o.shape[2] == n


def test_blocksparse_lower_blocks_with_causal_is_causal_forward():
    B, H, N, d, blk = 1, 2, 23, 4, 4
    q, k, v = rnd(104, B, H, N, d), rnd(105, B, H, N, d), rnd(106, B, H, N, d)
    nb = -(-N // blk)
    lower = np.tril(np.ones((nb, nb)))
    o, lse = oracle.forward_blocksparse(q, k, v, lower, 0.5, True, block=blk)
    of, lf = oracle.forward(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, of, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lf, rtol=1e-13)


def test_blocksparse_equals_gathered_keys():
    """Without causal, query block i attends to exactly the keys of its kept blocks: the same as
    decode (pinned on its own) of each row against those keys gathered; an empty row of blocks
    gives O = 0, LSE = -inf."""
    B, Hq, Hkv, Nq, Nk, d, blk = 1, 2, 2, 10, 14, 3, 4
    q, k, v = rnd(107, B, Hq, Nq, d), rnd(108, B, Hkv, Nk, d), rnd(109, B, Hkv, Nk, d)
    mask = np.array([[1, 0, 0, 1], [0, 1, 1, 0], [0, 0, 0, 0]])   # [ceil(10/4), ceil(14/4)]
    o, lse = oracle.forward_blocksparse(q, k, v, mask, 0.7, False, block=blk)
    for i in range(Nq):
        keys = np.concatenate([np.arange(j * blk, min((j + 1) * blk, Nk)) for j in range(4) if mask[i // blk, j]]
                              + [np.zeros(0, dtype=int)]).astype(int)
        if keys.size == 0:
            assert np.all(o[:, :, i] == 0.0) and np.all(lse[:, :, i] == -np.inf)
            continue
        od, ld = oracle.decode(q[:, :, i], k[:, :, keys], v[:, :, keys], 0.7)
        np.testing.assert_allclose(o[:, :, i], od, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], ld, rtol=1e-13)


def test_blocksparse_brute_force_tiny():
    """Scalar loops over the element mask the blocks expand to, causal aligned at the bottom right."""
    Nq, Nk, d, blk = 5, 7, 2, 2
    q, k, v = rnd(110, Nq, d), rnd(111, Nk, d), rnd(112, Nk, d)
    mask = np.array([[1, 0, 1, 1], [0, 0, 1, 0], [1, 1, 0, 1]])
    for causal in (False, True):
        o, lse = oracle.forward_blocksparse(q[None, None], k[None, None], v[None, None], mask, 0.8, causal, block=blk)
        for i in range(Nq):
            keys = [j for j in range(Nk) if mask[i // blk, j // blk] and not (causal and j > i + Nk - Nq)]
            if not keys:
                assert o[0, 0, i].tolist() == [0.0, 0.0] and lse[0, 0, i] == -np.inf
                continue
            s = [0.8 * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            assert abs(lse[0, 0, i] - (m + math.log(z))) <= 1e-13
            for c in range(d):
                ref = math.fsum(math.exp(s[t] - m) / z * v[j, c] for t, j in enumerate(keys))
                assert abs(o[0, 0, i, c] - ref) <= 1e-13


# ----------------------------------------------------------------------------- packed backward
def _loss_kv(q, k, v, dout, scale, causal):
    o, _ = oracle.forward_kv(q, k, v, scale, causal)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("Nq,Nk", [(3, 7), (6, 4), (5, 5)])
def test_backward_kv_matches_central_differences(Nq, Nk):
    """Gradient of the (pinned) forward_kv, bottom-right causal mask, grouped-query heads; with
    Nk < Nq the rows that see no key must get dQ = 0."""
    rng = np.random.default_rng(120 + Nq)
    B, Hq, Hkv, d, scale, eps = 1, 2, 1, 3, 0.7, 1e-6
    q, k, v = rng.standard_normal((B, Hq, Nq, d)), rng.standard_normal((B, Hkv, Nk, d)), rng.standard_normal((B, Hkv, Nk, d))
    do = rng.standard_normal((B, Hq, Nq, d))
    dq, dk, dv = oracle.backward_kv(q, k, v, do, scale, True)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            lp = _loss_kv(**{**args, name: xp}, dout=do, scale=scale, causal=True)
            lm = _loss_kv(**{**args, name: xm}, dout=do, scale=scale, causal=True)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)
    if Nk < Nq:
        assert np.all(dq[:, :, :Nq - Nk] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_equals_per_sequence_and_dense(causal):
    Hq, Hkv, d = 4, 2, 5
    lens_q, lens_k = [4, 0, 9, 2], [6, 3, 9, 0]
    x = make_varlen(lens_q, lens_k, Hq, Hkv, d, "f32", seed=125)
    rng = np.random.default_rng(126)
    do = rng.standard_normal(x["q"].shape)
    dq, dk, dv = oracle.backward_varlen(x["q"], x["k"], x["v"], do, x["cu_q"], x["cu_k"], 0.5, causal)
    cq, ck = x["cu_q"], x["cu_k"]
    for b in range(len(lens_q)):
        sq, sk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        g = oracle.backward_kv(x["q"][None, :, sq], x["k"][None, :, sk], x["v"][None, :, sk], do[None, :, sq], 0.5,
                               causal)
        np.testing.assert_array_equal(dq[:, sq], g[0][0])
        np.testing.assert_array_equal(dk[:, sk], g[1][0])
        np.testing.assert_array_equal(dv[:, sk], g[2][0])
    B, N = 3, 7
    y = make_prefill(B, Hq, Hkv, N, d, "f32", seed=127, with_dout=True)
    gd = oracle.backward(y["q"], y["k"], y["v"], y["dout"], 0.5, causal)
    fold = lambda t: np.ascontiguousarray(t.transpose(1, 0, 2, 3).reshape(t.shape[1], B * N, d))
    cu = np.arange(0, B * N + 1, N, dtype=np.int32)
    gp = oracle.backward_varlen(fold(y["q"]), fold(y["k"]), fold(y["v"]), fold(y["dout"]), cu, cu, 0.5, causal)
    for a, b in zip(gp, gd):
        np.testing.assert_allclose(a, fold(b), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- multi-token decode
def test_decode_multi_pins():
    """T = 1 is decode (with and without lengths); T causal tokens are the last T rows of the
    causal forward over the sequence's keys; a sequence shorter than T leaves its first tokens
    without keys."""
    B, Hq, Hkv, L, d, T = 3, 4, 2, 21, 5, 3
    rng = np.random.default_rng(130)
    q, kc, vc = rng.standard_normal((B, Hq, T, d)), rng.standard_normal((B, Hkv, L, d)), rng.standard_normal((B, Hkv, L, d))
    lens = [21, 2, 9]
    o1, l1 = oracle.decode_multi(q[:, :, :1], kc, vc, 0.6, True, seqlens=lens)
    od, ld = oracle.decode(q[:, :, 0], kc, vc, 0.6, seqlens=lens)
    np.testing.assert_allclose(o1[:, :, 0], od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1[:, :, 0], ld, rtol=1e-13)
    o, lse = oracle.decode_multi(q, kc, vc, 0.6, True, seqlens=lens)
    b, n = 2, lens[2]
    qfull = np.concatenate([rng.standard_normal((1, Hq, n - T, d)), q[b:b + 1]], axis=2)
    of, lf = oracle.forward(qfull, kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], 0.6, True)
    np.testing.assert_allclose(o[b], of[0, :, n - T:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[b], lf[0, :, n - T:], rtol=1e-13)
    assert np.all(lse[1, :, 0] == -np.inf) and np.all(o[1, :, 0] == 0.0)   # len 2 < T = 3
    on, ln = oracle.decode_multi(q, kc, vc, 0.6, False, seqlens=lens)
    for t in range(T):
        od, ld = oracle.decode(q[:, :, t], kc, vc, 0.6, seqlens=lens)
        np.testing.assert_allclose(on[:, :, t], od, rtol=1e-12, atol=1e-13)


def _loss_bs(q, k, v, dout, mask, scale, causal, block):
    o, _ = oracle.forward_blocksparse(q, k, v, mask, scale, causal, block=block)
    return float(np.sum(o * dout))


def test_backward_blocksparse_pins():
    """Central differences of the (pinned) forward_blocksparse on a tiny case with an empty row
    of blocks; the full mask equals backward_kv; a block-diagonal mask equals the packed
    backward of one-block sequences."""
    rng = np.random.default_rng(140)
    B, Hq, Hkv, N, d, blk, scale, eps = 1, 2, 1, 6, 3, 2, 0.8, 1e-6
    q, k, v = rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    mask = np.array([[[1, 0, 1], [0, 0, 0], [1, 1, 0]], [[0, 1, 1], [1, 0, 1], [1, 1, 1]]])[None]
    for causal in (False, True):
        g = oracle.backward_blocksparse(q, k, v, do, mask, scale, causal, block=blk)
        for name, x, gx in (("q", q, g[0]), ("k", k, g[1]), ("v", v, g[2])):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args = {"q": q, "k": k, "v": v}
                lp = _loss_bs(**{**args, name: xp}, dout=do, mask=mask, scale=scale, causal=causal, block=blk)
                lm = _loss_bs(**{**args, name: xm}, dout=do, mask=mask, scale=scale, causal=causal, block=blk)
                num[idx] = (lp - lm) / (2 * eps)
            np.testing.assert_allclose(gx, num, rtol=1e-6, atol=1e-7, err_msg=f"{name} causal={causal}")
        assert np.all(g[0][0, 0, 2:4] == 0.0)  # head 0, query block 1 keeps nothing
    gf = oracle.backward_blocksparse(q, k, v, do, np.ones((3, 3)), scale, True, block=blk)
    gk = oracle.backward_kv(q, k, v, do, scale, True)
    for a, c in zip(gf, gk):
        np.testing.assert_allclose(a, c, rtol=1e-12, atol=1e-13)
    lens = [blk] * 3
    x = make_varlen(lens, lens, Hq, Hkv, d, "f32", seed=141)
    dox = rng.standard_normal(x["q"].shape)
    gb = oracle.backward_blocksparse(x["q"][None], x["k"][None], x["v"][None], dox[None], np.eye(3), scale, True,
                                     block=blk)
    gv = oracle.backward_varlen(x["q"], x["k"], x["v"], dox, x["cu_q"], x["cu_k"], scale, True)
    for a, c in zip(gb, gv):
        np.testing.assert_allclose(a[0], c, rtol=1e-12, atol=1e-13)


def test_bwd_bound_needs_more_than_bf16_o_on_tiny_peaky_rows():
    """A backward that forms D = rowsum(dO * O) from O as the forward stored it (bf16): on a
    tiny causal case with doubled logits (N = 2: the second row is dominated by one key, so
    dP - D nearly cancels) that rounding alone moves dQ and dK by about 2% in relative L2,
    beyond the 1e-2 bound, while the same fp64 backward with the exact O reproduces the oracle.
    Hence the dQ kernel forms D from its definition, sum_j P_ij dP_ij, wherever a query tile's
    keys fit one key tile."""
    B, Hq, Hkv, N, d = 2, 4, 2, 2, 128
    inp = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=7129, with_dout=True, qk_mult=2.0)
    scale = default_scale(d)
    q, k, v, do = (bf16_bits_to_f32(inp[x]).astype(np.float64) for x in ("q", "k", "v", "dout"))
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], scale, True)
    g = Hq // Hkv
    errs = {}
    for name in ("exact", "bf16"):
        dq = np.zeros_like(q)
        dk = np.zeros((B, Hkv, N, d))
        for b in range(B):
            for h in range(Hq):
                kv = h // g
                p = oracle.probabilities(q[b, h], k[b, kv], scale, True)
                o = p @ v[b, kv]
                if name == "bf16":
                    o = bf16_bits_to_f32(f32_to_bf16_bits(o.astype(np.float32))).astype(np.float64)
                dp = do[b, h] @ v[b, kv].T
                ds = p * (dp - np.sum(do[b, h] * o, axis=1, keepdims=True))
                dq[b, h] = scale * ds @ k[b, kv]
                dk[b, kv] += scale * ds.T @ q[b, h]
        errs[name] = (np.linalg.norm(dq - ref[0]) / np.linalg.norm(ref[0]),
                      np.linalg.norm(dk - ref[1]) / np.linalg.norm(ref[1]))
    assert max(errs["exact"]) < 1e-12
    assert min(errs["bf16"]) > 1e-2

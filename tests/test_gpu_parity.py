"""GPU parity: the HIP kernels against the fp64 oracle on the same seeded inputs.

Sizes: every workload shape at full size on the GPU, compared element by element where the
oracle finishes in seconds, else on sampled rows (exact per row: an output row depends only
on its query and all keys/values) or sampled heads; plus ragged, grouped-query and
degenerate shapes, closed forms and determinism.
"""
import math

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, default_scale, make_decode, make_prefill
from tests._util import Guarded, assert_fwd_ok, fwd_errors, rel_l2, to_dev, to_host64, BWD_REL_L2

pytestmark = pytest.mark.gpu


def run_fwd(lib, inp, causal, scale):
    """Outputs in guarded buffers: a write outside O or LSE fails the test."""
    import torch
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    g = Guarded()
    o, lse = g.like(q), g.empty(q.shape[:3], torch.float32)
    lib.attn_fwd(q, k, v, causal, scale, o=o, lse=lse)
    g.check("attn_fwd")
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


# ----------------------------------------------------------------------------- forward
def test_fwd_tiny_fp32(gpu_lib):
    w = WORKLOADS["tiny"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "f32", seed=w.seed)
    scale = default_scale(w.d)
    o, lse = run_fwd(gpu_lib, inp, w.causal, scale)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, w.causal)
    err = fwd_errors(o, o_ref, lse, lse_ref)
    assert_fwd_ok(err, "tiny")
    assert err["max"] <= 5e-5 and err["lse"] <= 5e-5, err  # fp32 path keeps fp32 precision


@pytest.mark.parametrize("seed_off", [0, 1, 2])
def test_fwd_batched_prefill(gpu_lib, seed_off):
    w = WORKLOADS["prefill"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed + seed_off)
    scale = default_scale(w.d)
    o, lse = run_fwd(gpu_lib, inp, w.causal, scale)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, w.causal)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), "prefill")


_LONG_INPUTS = {}


def long_inputs(name):
    """Seeded inputs of a long-prefill workload, drawn once per module (the N = 16384 draw
    takes seconds)."""
    if name not in _LONG_INPUTS:
        _LONG_INPUTS.clear()
        w = WORKLOADS[name]
        _LONG_INPUTS[name] = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed, qk_mult=w.qk_mult)
    return _LONG_INPUTS[name]


def sample_rows(N, seed, extra=248):
    fixed = {0, 1, 63, 64, 127, 128, N // 2, N - 1}
    rng = np.random.default_rng(seed)
    return np.array(sorted(fixed | set(rng.integers(0, N, extra).tolist())))


@pytest.mark.parametrize("name", ["long4k", "long8k", "long16k"])
@pytest.mark.parametrize("causal", [True, False])
def test_fwd_long_prefill_sampled_rows(gpu_lib, name, causal):
    w = WORKLOADS[name]
    inp = long_inputs(name)
    scale = default_scale(w.d)
    o, lse = run_fwd(gpu_lib, inp, causal, scale)
    rows = sample_rows(w.N, w.seed + int(causal))
    o_ref, lse_ref = oracle.forward_rows(inp["q"], inp["k"], inp["v"], scale, causal, rows)
    assert_fwd_ok(fwd_errors(o[:, :, rows], o_ref, lse[:, :, rows], lse_ref), name)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("h", [0, 31])
def test_fwd_long16k_full_heads(gpu_lib, causal, h):
    """Long prefill at N = 16384 (logits x2): every element of O and every LSE row of two whole
    heads, causal and not, besides the 256 sampled rows of every head above (the oracle holds
    the 16384 x 16384 score matrix of one head at a time)."""
    w = WORKLOADS["long16k"]
    print(f"long16k full head h={h} causal={causal}", flush=True)
    inp = long_inputs("long16k")
    scale = default_scale(w.d)
    o, lse = run_fwd(gpu_lib, inp, causal, scale)
    sl = {kk: inp[kk][:, h:h + 1] for kk in ("q", "k", "v")}
    o_ref, lse_ref = oracle.forward(sl["q"], sl["k"], sl["v"], scale, causal)
    assert_fwd_ok(fwd_errors(o[:, h:h + 1], o_ref, lse[:, h:h + 1], lse_ref), f"h{h} causal={causal}")


def test_fwd_long4k_every_element(gpu_lib):
    """Long prefill at N = 4096 (logits x2): every element of O and every LSE row of all 32
    heads, causal and not.  A kernel that divided O by the fp32 row sum while P V used the
    bf16 probabilities had one element of the causal case at 0.025 here."""
    w = WORKLOADS["long4k"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed, qk_mult=w.qk_mult)
    scale = default_scale(w.d)
    for causal in (True, False):
        o, lse = run_fwd(gpu_lib, inp, causal, scale)
        for h in range(w.Hq):
            sl = {kk: inp[kk][:, h:h + 1] for kk in ("q", "k", "v")}
            o_ref, lse_ref = oracle.forward(sl["q"], sl["k"], sl["v"], scale, causal)
            assert_fwd_ok(fwd_errors(o[:, h:h + 1], o_ref, lse[:, h:h + 1], lse_ref), f"h{h} causal={causal}")


def test_fwd_long8k_every_element(gpu_lib):
    """Long prefill at N = 8192 (logits x2): every element of O and every LSE row of all 32
    heads, causal and not (about 20 s of oracle time)."""
    w = WORKLOADS["long8k"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed, qk_mult=w.qk_mult)
    scale = default_scale(w.d)
    for causal in (True, False):
        o, lse = run_fwd(gpu_lib, inp, causal, scale)
        for h in range(w.Hq):
            sl = {kk: inp[kk][:, h:h + 1] for kk in ("q", "k", "v")}
            o_ref, lse_ref = oracle.forward(sl["q"], sl["k"], sl["v"], scale, causal)
            assert_fwd_ok(fwd_errors(o[:, h:h + 1], o_ref, lse[:, h:h + 1], lse_ref), f"h{h} causal={causal}")


def test_fwd_peaky_grouped_rows(gpu_lib):
    """d = 128, grouped heads, logits x2, N = 511, non-causal: a shape on which dividing O by
    the fp32 row sum put one element at 0.0225 (found by a randomised sweep)."""
    inp = make_prefill(1, 16, 2, 511, 128, "bf16", seed=7076, qk_mult=2.0)
    scale = default_scale(128)
    o, lse = run_fwd(gpu_lib, inp, False, scale)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, False)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), "peaky grouped")


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_shapes_agree(gpu_lib, causal):
    """d = 128 runs in two workgroup shapes (256 query rows with 64-key tiles, or 128 rows
    with 32-key tiles), chosen by the average key walk and by how many CUs the wide grid
    fills.  32 heads at N = 4096 take the wide shape (walk >= 2048 keys, 512 workgroups);
    two of those heads alone take the narrow one (32 wide workgroups would leave CUs idle).
    Heads are independent and both shapes take the same 32-key blocks in the same order, so
    the results must agree exactly; the narrow run, a long walk, is also checked on sampled
    rows against the oracle."""
    w = WORKLOADS["long4k"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed + 11, qk_mult=w.qk_mult)
    scale = default_scale(w.d)
    o_wide, lse_wide = run_fwd(gpu_lib, inp, causal, scale)
    sl = {kk: np.ascontiguousarray(inp[kk][:, 5:7]) for kk in ("q", "k", "v")}
    o_nar, lse_nar = run_fwd(gpu_lib, sl, causal, scale)
    assert np.array_equal(o_nar, o_wide[:, 5:7]) and np.array_equal(lse_nar, lse_wide[:, 5:7])
    rows = sample_rows(w.N, 17 + int(causal), extra=60)
    o_ref, lse_ref = oracle.forward_rows(sl["q"], sl["k"], sl["v"], scale, causal, rows)
    assert_fwd_ok(fwd_errors(o_nar[:, :, rows], o_ref, lse_nar[:, :, rows], lse_ref), "narrow long walk")


@pytest.mark.parametrize("N", [970, 1001])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_odd_key_tiles(gpu_lib, N, causal):
    """N = 970 leaves 31 32-key tiles (an odd count, padded by one fully masked tile) for every
    query tile without the causal mask and for the last one with it; N = 1001 leaves 32."""
    inp = make_prefill(1, 4, 2, N, 128, "bf16", seed=N + int(causal))
    scale = default_scale(128)
    o, lse = run_fwd(gpu_lib, inp, causal, scale)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, causal)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), f"N={N}")


@pytest.mark.parametrize("N", [1, 2, 17, 100, 257, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_ragged(gpu_lib, N, d, causal):
    inp = make_prefill(2, 3, 3, N, d, "bf16", seed=N * 7 + d)
    scale = default_scale(d)
    o, lse = run_fwd(gpu_lib, inp, causal, scale)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, causal)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), f"N={N} d={d}")


@pytest.mark.parametrize("N", [5, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_ragged_fp32(gpu_lib, N, causal):
    inp = make_prefill(1, 2, 2, N, 64, "f32", seed=N)
    o, lse = run_fwd(gpu_lib, inp, causal, 0.125)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], 0.125, causal)
    err = fwd_errors(o, o_ref, lse, lse_ref)
    assert err["max"] <= 5e-5 and err["lse"] <= 5e-5, err


@pytest.mark.parametrize("B,H,N", [(1, 2, 1000), (1, 3, 97), (2, 16, 1024)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp32_grids(gpu_lib, B, H, N, causal):
    """fp32 on both of its kernels: small grids (fewer 128-row tiles than CUs) split each
    workgroup's keys over its four waves and merge them, large ones (B=2 H=16 N=1024: 256 tiles)
    take 128-row tiles; every element of the small shapes, sampled rows of the large one."""
    print(f"fwd fp32 B={B} H={H} N={N} causal={causal}", flush=True)
    inp = make_prefill(B, H, H, N, 64, "f32", seed=7000 + N + H)
    o, lse = run_fwd(gpu_lib, inp, causal, 0.125)
    if B * H * N <= 4096:
        o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], 0.125, causal)
    else:
        rows = sample_rows(N, seed=7001, extra=56)
        o, lse = o[:, :, rows], lse[:, :, rows]
        o_ref, lse_ref = oracle.forward_rows(inp["q"], inp["k"], inp["v"], 0.125, causal, rows)
    err = fwd_errors(o, o_ref, lse, lse_ref)
    assert err["max"] <= 5e-5 and err["lse"] <= 5e-5, err  # the fp32 kernels keep fp32 precision


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_grouped_query(gpu_lib, d, causal):
    inp = make_prefill(2, 8, 2, 333, d, "bf16", seed=5 + d)
    scale = default_scale(d)
    o, lse = run_fwd(gpu_lib, inp, causal, scale)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, causal)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), "gqa")


def test_fwd_closed_forms(gpu_lib):
    """Q = 0: O_i is the (prefix) mean of V and LSE_i = ln(#keys); causal row 0 is V[0]."""
    import torch
    B, H, N, d = 1, 2, 200, 128
    inp = make_prefill(B, H, H, N, d, "bf16", seed=99)
    q0 = np.zeros_like(inp["q"])
    for causal in (False, True):
        o, lse = run_fwd(gpu_lib, {"q": q0, "k": inp["k"], "v": inp["v"]}, causal, 0.1)
        v = oracle.upcast(inp["v"])
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        ref = (np.cumsum(v, axis=2) / cnt[:, None]) if causal else np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        assert_fwd_ok(fwd_errors(o, ref, lse, np.broadcast_to(np.log(cnt), lse.shape)), f"q0 causal={causal}")
    o, _ = run_fwd(gpu_lib, inp, True, 0.1)
    np.testing.assert_array_equal(o[:, :, 0], oracle.upcast(inp["v"])[:, :, 0])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("trend", ["rising", "falling", "spike"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_moving_running_max(gpu_lib, causal, trend, d):
    """Inputs whose row maxima keep moving, so the kernels' lazily updated reference max has to
    move many times (and by large amounts, for the spike) mid-row; at d = 64 and 128."""
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    B, H, N = 1, 2, 700
    inp = make_prefill(B, H, H, N, d, "bf16", seed=41)
    k = bf16_bits_to_f32(inp["k"]).reshape(B, H, N, d)
    ramp = np.linspace(0.2, 4.0, N, dtype=np.float32)
    if trend == "falling":
        ramp = ramp[::-1].copy()
    elif trend == "spike":
        ramp = np.full(N, 0.3, np.float32)
        ramp[[37, 300, 301, 650]] = [6.0, 12.0, 20.0, 30.0]
    k = k * ramp[None, None, :, None]
    if trend == "spike":
        # Spiked keys point along the mean query, so most rows see logit jumps of tens (log2).
        q = bf16_bits_to_f32(inp["q"]).reshape(B, H, N, d)
        k[:, :, ramp > 5] = np.sign(q.mean(axis=2, keepdims=True)) * ramp[ramp > 5][None, None, :, None] * 0.5
    run = {"q": inp["q"], "k": f32_to_bf16_bits(k), "v": inp["v"]}
    scale = default_scale(d)
    o, lse = run_fwd(gpu_lib, run, causal, scale)
    o_ref, lse_ref = oracle.forward(run["q"], run["k"], run["v"], scale, causal)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), f"{trend} causal={causal}")


def test_fwd_bitwise_deterministic(gpu_lib):
    import torch
    inp = make_prefill(1, 4, 4, 1000, 128, "bf16", seed=3)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o1, l1 = gpu_lib.attn_fwd(q, k, v, True, 0.09)
    o2, l2 = gpu_lib.attn_fwd(q, k, v, True, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------- decode
@pytest.fixture(scope="module")
def decode_inputs():
    w = WORKLOADS["decode"]
    return w, make_decode(w.B, w.Hq, w.Hkv, w.L, w.d, seed=w.seed)


def test_decode_full_size_every_sequence(gpu_lib, decode_inputs):
    """The decode workload with the automatic split count: all 64 sequences against the oracle."""
    import torch
    w, inp = decode_inputs
    scale = default_scale(w.d)
    q, kc, vc = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = gpu_lib.attn_decode(q, kc, vc, scale, num_splits=0)
    torch.cuda.synchronize()
    o, lse = to_host64(o), lse.cpu().numpy().astype(np.float64)
    del q, kc, vc
    torch.cuda.empty_cache()
    o_ref, lse_ref = oracle.decode(inp["q"], inp["k"], inp["v"], scale)
    assert_fwd_ok(fwd_errors(o, o_ref, lse, lse_ref), "decode every sequence")


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_decode_full_size_sampled_batches(gpu_lib, decode_inputs, splits):
    import torch
    w, inp = decode_inputs
    scale = default_scale(w.d)
    q, kc, vc = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = gpu_lib.attn_decode(q, kc, vc, scale, num_splits=splits)
    torch.cuda.synchronize()
    o, lse = to_host64(o), lse.cpu().numpy().astype(np.float64)
    bs = [0, 17, 63]
    o_ref, lse_ref = oracle.decode(inp["q"][bs], inp["k"][bs], inp["v"][bs], scale)
    assert_fwd_ok(fwd_errors(o[bs], o_ref, lse[bs], lse_ref), f"decode splits={splits}")
    del q, kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("L", [1, 33, 1000])
@pytest.mark.parametrize("g", [1, 3, 4, 5, 16, 32, 48])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_small(gpu_lib, L, g, d):
    import torch
    g_ = g
    inp = make_decode(3, 2 * g, 2, L, d, seed=L + g + d)
    scale = default_scale(d)
    q, kc, vc = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    for splits in (0, 2, 7):
        g = Guarded()
        o, lse = g.like(q), g.empty(q.shape[:2], torch.float32)
        ws = g.empty((gpu_lib.attn_decode_workspace_bytes(3, 2 * g_, 2, L, d, splits),), torch.uint8)
        gpu_lib.attn_decode(q, kc, vc, scale, num_splits=splits, o=o, lse=lse, workspace=ws)
        g.check(f"decode L={L} g={g_} s={splits}")
        o_ref, lse_ref = oracle.decode(inp["q"], inp["k"], inp["v"], scale)
        assert_fwd_ok(fwd_errors(to_host64(o), o_ref, lse.cpu().numpy(), lse_ref), f"L={L} g={g_} s={splits}")


def test_decode_matches_forward_single_row(gpu_lib):
    """Decode equals the forward of one query row against the same keys."""
    import torch
    inp = make_decode(2, 4, 4, 300, 128, seed=8)
    o, lse = gpu_lib.attn_decode(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), 0.088)
    of, lf = oracle.forward(inp["q"][:, :, None, :], inp["k"], inp["v"], 0.088, False)
    torch.cuda.synchronize()
    assert_fwd_ok(fwd_errors(to_host64(o), of[:, :, 0], lse.cpu().numpy(), lf[:, :, 0]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_decode_per_sequence_lengths(gpu_lib, d, splits):
    """attn_decode_varlen: sequence b attends to its first seqlens[b] cached keys; lengths
    cover empty, single-key, block-boundary, ragged and full caches."""
    import torch
    L = 1000
    lens = np.array([0, 1, 31, 32, 33, 500, 999, 1000], dtype=np.int32)
    inp = make_decode(len(lens), 8, 2, L, d, seed=5 + d)
    scale = default_scale(d)
    sl = torch.from_numpy(lens).cuda()
    q = to_dev(inp["q"])
    g = Guarded()
    o, lse = g.like(q), g.empty(q.shape[:2], torch.float32)
    ws = g.empty((gpu_lib.attn_decode_workspace_bytes(len(lens), 8, 2, L, d, splits),), torch.uint8)
    gpu_lib.attn_decode_varlen(q, to_dev(inp["k"]), to_dev(inp["v"]), sl, scale, num_splits=splits, o=o, lse=lse,
                               workspace=ws)
    g.check(f"decode varlen d={d} splits={splits}")
    o_ref, lse_ref = oracle.decode(inp["q"], inp["k"], inp["v"], scale, seqlens=lens)
    o_h, lse_h = to_host64(o), lse.cpu().numpy().astype(np.float64)
    assert np.all(o_h[0] == 0.0) and np.all(lse_h[0] == -np.inf)
    assert_fwd_ok(fwd_errors(o_h[1:], o_ref[1:], lse_h[1:], lse_ref[1:]), f"varlen d={d} splits={splits}")


def run_decode_varlen(lib, inp, lens, d, splits):
    import torch
    sl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    q = to_dev(inp["q"])
    B, Hq, _ = q.shape
    Hkv, L = inp["k"].shape[1], inp["k"].shape[2]
    g = Guarded()
    o, lse = g.like(q), g.empty((B, Hq), torch.float32)
    ws = g.empty((lib.attn_decode_workspace_bytes(B, Hq, Hkv, L, d, splits),), torch.uint8)
    lib.attn_decode_varlen(q, to_dev(inp["k"]), to_dev(inp["v"]), sl, default_scale(d), num_splits=splits, o=o,
                           lse=lse, workspace=ws)
    g.check(f"decode varlen B={B} d={d} splits={splits}")
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


def check_varlen_rows(o, lse, o_ref, lse_ref, lens, tag):
    """Empty sequences give O = 0 and LSE = -inf; every other row against the oracle."""
    lens = np.asarray(lens)
    empty, full = lens <= 0, lens > 0
    assert np.all(o[empty] == 0.0) and np.all(lse[empty] == -np.inf), tag
    assert_fwd_ok(fwd_errors(o[full], o_ref[full], lse[full], lse_ref[full]), tag)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_decode_skewed_lengths(gpu_lib, d, splits):
    """attn_decode_varlen with two long sequences among many short or empty ones.  The split
    gives every workgroup the same number of 32-key blocks, so the long sequences are cut over
    many workgroups while one workgroup takes several short ones (its block range crossing
    sequence and KV-head boundaries); every row against the oracle."""
    L = 2048
    lens = np.array([L] + [0, 1, 3, 40, 0, 65, 2] * 4 + [L - 1, 0, 31, 32, 33], dtype=np.int32)
    print(f"decode skewed B={len(lens)} d={d} splits={splits}", flush=True)
    inp = make_decode(len(lens), 4, 2, L, d, seed=6000 + d + splits)
    o, lse = run_decode_varlen(gpu_lib, inp, lens, d, splits)
    o_ref, lse_ref = oracle.decode(inp["q"], inp["k"], inp["v"], default_scale(d), seqlens=lens)
    check_varlen_rows(o, lse, o_ref, lse_ref, lens, f"skewed d={d} splits={splits}")


@pytest.mark.parametrize("B", [2048, 2049])
def test_decode_lengths_many_sequences(gpu_lib, B):
    """Up to 2048 sequences the split's per-sequence block counts sit in LDS; beyond that the
    fixed key chunks take over.  Both against the oracle, lengths uniform in [0, L]."""
    L, d = 96, 64
    lens = np.random.default_rng(6100 + B).integers(0, L + 1, size=B).astype(np.int32)
    print(f"decode many B={B}", flush=True)
    inp = make_decode(B, 2, 1, L, d, seed=6200 + B)
    o, lse = run_decode_varlen(gpu_lib, inp, lens, d, 0)
    o_ref, lse_ref = oracle.decode(inp["q"], inp["k"], inp["v"], default_scale(d), seqlens=lens)
    check_varlen_rows(o, lse, o_ref, lse_ref, lens, f"many B={B}")


# ----------------------------------------------------------------------------- backward
def run_fwd_bwd(lib, inp, causal, scale):
    """Gradients and the backward workspace in guarded buffers."""
    import torch
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    o, lse = lib.attn_fwd(q, k, v, causal, scale)
    g = Guarded()
    dq, dk, dv = g.like(q), g.like(k), g.like(v)
    B, Hq, N, d = q.shape
    ws = g.empty((max(lib.attn_bwd_workspace_bytes(B, Hq, k.shape[1], N, d), 1),), torch.uint8)
    lib.attn_bwd(q, k, v, o, lse, do, causal, scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    g.check("attn_bwd")
    return [to_host64(t) for t in (dq, dk, dv)]


def check_bwd(grads, inp, scale, causal, heads=None, tag=""):
    sl = (lambda a: a) if heads is None else (lambda a: a[:, heads])
    ref = oracle.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["dout"]), scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
        if not np.any(r):
            # A single key makes the softmax constant: dQ = dK = 0 exactly, so the relative
            # error is undefined; require the GPU result to vanish up to rounding instead.
            assert np.abs(sl(g)).max() <= 1e-3, (tag, name, np.abs(sl(g)).max())
            continue
        err = rel_l2(sl(g), r)
        assert err <= BWD_REL_L2, (tag, name, err)


@pytest.fixture(scope="module")
def train_grads(gpu_lib):
    """The training-step workload (B=2, H=16, N=4096, d=128, causal): GPU forward, then GPU
    backward, once for the module."""
    w = WORKLOADS["train"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed, with_dout=True)
    return w, inp, run_fwd_bwd(gpu_lib, inp, True, default_scale(w.d))


@pytest.mark.parametrize("b", [0, 1])
def test_bwd_training_step_every_head(gpu_lib, train_grads, b):
    """Every head of the training step: dQ, dK, dV of each (b, h) against the oracle's fp64
    backward (a head's gradients depend only on its own Q, K, V and dO)."""
    w, inp, grads = train_grads
    scale = default_scale(w.d)
    for h in range(w.Hq):
        sub = {x: inp[x][b:b + 1, h:h + 1] for x in inp}
        check_bwd([g[b:b + 1, h:h + 1] for g in grads], sub, scale, True, tag=f"b{b}h{h}")


def test_bwd_training_step_other_seed(gpu_lib):
    """The training-step shape on a second seed: two heads per batch row."""
    w = WORKLOADS["train"]
    inp = make_prefill(w.B, w.Hq, w.Hkv, w.N, w.d, "bf16", seed=w.seed + 1, with_dout=True)
    scale = default_scale(w.d)
    grads = run_fwd_bwd(gpu_lib, inp, True, scale)
    for b in range(w.B):
        for h in (7, 12):
            sub = {x: inp[x][b:b + 1, h:h + 1] for x in inp}
            check_bwd([g[b:b + 1, h:h + 1] for g in grads], sub, scale, True, tag=f"b{b}h{h}")


def dominated_inputs(N, trend, qk_mult, seed, d=128):
    """Q, K, V, dO whose rows are dominated by one key over stretches longer than a key tile:
    "spike" puts a few keys along the mean query with large norms, so every later row's softmax
    is carried by the latest spike; "rising" grows the key norms along the sequence, so each
    row's largest weights sit on its most recent keys."""
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    inp = make_prefill(1, 2, 2, N, d, "bf16", seed=seed, with_dout=True, qk_mult=qk_mult)
    q = bf16_bits_to_f32(inp["q"]).reshape(1, 2, N, d)
    k = bf16_bits_to_f32(inp["k"]).reshape(1, 2, N, d)
    if trend == "rising":
        k = k * np.linspace(0.2, 3.0, N, dtype=np.float32)[None, None, :, None]
    else:
        pos = np.array(sorted({37, N // 7, N // 3, N // 3 + 1, N // 2 + 5, (5 * N) // 6}))
        k = k * 0.3
        k[:, :, pos] = (np.sign(q.mean(axis=2, keepdims=True)) * np.linspace(6.0, 16.0, len(pos),
                        dtype=np.float32)[None, None, :, None] * 0.5)
    return {"q": inp["q"], "k": f32_to_bf16_bits(k), "v": inp["v"], "dout": inp["dout"]}


@pytest.mark.parametrize("N", [1000, 4096])
@pytest.mark.parametrize("trend", ["spike", "rising"])
@pytest.mark.parametrize("qk_mult", [1.0, 2.0])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_dominated_rows_long(gpu_lib, N, trend, qk_mult, causal):
    """Backward on rows dominated by one key over many key tiles: there dP - D nearly cancels
    for the dominant key, so D must be accurate to well below the bf16 rounding of O."""
    print(f"bwd dominated N={N} {trend} x{qk_mult} causal={causal}", flush=True)
    inp = dominated_inputs(N, trend, qk_mult, seed=5100 + N + int(qk_mult))
    scale = default_scale(128)
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale)
    check_bwd(grads, inp, scale, causal, tag=f"dominated N={N} {trend} x{qk_mult} causal={causal}")


@pytest.mark.parametrize("N", [100, 1000])
@pytest.mark.parametrize("trend", ["spike", "rising"])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_dominated_rows_d64(gpu_lib, N, trend, causal):
    """d = 64 on dominated rows: query tiles whose keys fit two 64-key tiles (N = 100, and the
    first query tile of a causal sequence) form the exact D in the first dQ launch, longer ones
    in the second."""
    print(f"bwd dominated d=64 N={N} {trend} causal={causal}", flush=True)
    inp = dominated_inputs(N, trend, 2.0, seed=5300 + N, d=64)
    scale = default_scale(64)
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale)
    check_bwd(grads, inp, scale, causal, tag=f"dominated d=64 N={N} {trend} causal={causal}")


@pytest.mark.parametrize("N", [1, 17, 64, 200, 333])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged(gpu_lib, N, d, causal):
    inp = make_prefill(2, 2, 2, N, d, "bf16", seed=N + d + 11, with_dout=True)
    scale = default_scale(d)
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale)
    check_bwd(grads, inp, scale, causal, tag=f"N={N} d={d}")


@pytest.mark.parametrize("heads", [(8, 2), (4, 1)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_grouped_query(gpu_lib, heads, d, causal):
    """Grouped-query backward: dK/dV of a KV head sum the gradients of its query heads."""
    Hq, Hkv = heads
    inp = make_prefill(2, Hq, Hkv, 333, d, "bf16", seed=Hq * 10 + Hkv + d, with_dout=True)
    scale = default_scale(d)
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale)
    check_bwd(grads, inp, scale, causal, tag=f"gqa {Hq}/{Hkv} d={d}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 8, 4, 1000, 128), (1, 16, 2, 777, 64), (2, 8, 1, 640, 128),
                                         (1, 6, 2, 500, 128)])
def test_bwd_grouped_query_split(gpu_lib, B, Hq, Hkv, N, d):
    """Causal grouped-query backward on few key blocks: the group's query heads are split over
    two dK/dV workgroups whose fp32 partial sums are added in a fixed order (group sizes 2, 8 and
    4; the odd group of 3 takes the unsplit path).  Matches the oracle and repeats bit for bit."""
    inp = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=900 + Hq + Hkv + N, with_dout=True)
    scale = default_scale(d)
    grads = run_fwd_bwd(gpu_lib, inp, True, scale)
    check_bwd(grads, inp, scale, True, tag=f"split {Hq}/{Hkv} N={N} d={d}")
    again = run_fwd_bwd(gpu_lib, inp, True, scale)
    for a, b in zip(grads, again):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,causal,seed", [(2, 4, 2, 2, 128, True, 7129), (1, 3, 1, 2, 64, True, 7132),
                                                    (1, 2, 2, 2, 128, False, 7007), (2, 2, 2, 33, 64, True, 7200)])
def test_bwd_short_peaky_rows(gpu_lib, B, Hq, Hkv, N, d, causal, seed):
    """Rows whose keys fit one 64-key tile, logits x2 (rows dominated by one key): D is formed
    as sum_j P_ij dP_ij rather than from the stored bf16 O, whose rounding alone moved dQ and
    dK past the bound on these shapes."""
    inp = make_prefill(B, Hq, Hkv, N, d, "bf16", seed=seed, with_dout=True, qk_mult=2.0)
    scale = default_scale(d)
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale)
    check_bwd(grads, inp, scale, causal, tag=f"short peaky N={N} d={d}")


def uncancelled_scales(inp, scale, causal):
    """Norms of dQ and dK with |P * dP| in place of dS = P * (dP - D): the size the gradients
    would have without the cancellation in dP - D (fp64, from the inputs)."""
    Q, K, V, dO = (oracle.upcast(inp[x]) for x in ("q", "k", "v", "dout"))
    g = Q.shape[1] // K.shape[1]
    K, V = np.repeat(K, g, axis=1), np.repeat(V, g, axis=1)
    S = scale * np.einsum("bhid,bhjd->bhij", Q, K)
    if causal:
        n, m = S.shape[-2:]
        S = np.where(np.arange(m)[None, :] <= np.arange(n)[:, None] + (m - n), S, -np.inf)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    aP = np.abs(P * np.einsum("bhid,bhjd->bhij", dO, V))
    dq = scale * np.einsum("bhij,bhjd->bhid", aP, np.abs(K))
    dk = scale * np.einsum("bhij,bhid->bhjd", aP, np.abs(Q))
    return float(np.linalg.norm(dq)), float(np.linalg.norm(dk))


@pytest.mark.parametrize("N,d,causal", [(3, 128, True), (3, 64, False), (100, 128, True), (333, 64, True),
                                        (700, 128, False)])
def test_bwd_cancelling_gradients(gpu_lib, N, d, causal):
    """Logits x16 (Q and K x4): rows are one-hot to within e^-30, so dS = P (dP - D) cancels and
    the exact dQ and dK can shrink to 1e-13 of the size they would have without the cancellation
    (3-key causal rows), and a relative bound on them then measures fp32 rounding against
    nothing.  dV keeps the relative bound; dQ and dK are held to it against the larger of their
    own norm and 1e-3 of their uncancelled size (fp32 rounding of the uncancelled terms leaves a
    few 1e-7 of it)."""
    print(f"bwd cancelling N={N} d={d} causal={causal}", flush=True)
    inp = make_prefill(1, 2, 1, N, d, "bf16", seed=8800 + N + d, with_dout=True, qk_mult=4.0)
    scale = default_scale(d)
    grads = run_fwd_bwd(gpu_lib, inp, causal, scale)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], scale, causal)
    unc = uncancelled_scales(inp, scale, causal)
    for name, g, r, u in zip(("dq", "dk", "dv"), grads, ref, unc + (None,)):
        den = np.linalg.norm(r) if u is None else max(np.linalg.norm(r), 1e-3 * u)
        err = float(np.linalg.norm(g - r) / den)
        assert err <= BWD_REL_L2, (name, err)


def test_bwd_from_oracle_forward(gpu_lib):
    """Feed the oracle's O (as bf16) and LSE into attn_bwd: isolates the backward kernels."""
    import torch
    from synth import f32_to_bf16_bits
    inp = make_prefill(1, 2, 2, 500, 128, "bf16", seed=77, with_dout=True)
    scale = default_scale(128)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], scale, True)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    o = to_dev(f32_to_bf16_bits(o_ref.astype(np.float32)))
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    dq, dk, dv = gpu_lib.attn_bwd(q, k, v, o, lse, do, True, scale)
    torch.cuda.synchronize()
    check_bwd([to_host64(t) for t in (dq, dk, dv)], inp, scale, True, tag="oracle-fwd")


# ----------------------------------------------------------------------------- multi-token decode
def run_decode_multi(lib, q, kc, vc, lens, causal, splits, scale):
    import torch
    sl = None if lens is None else torch.tensor(np.asarray(lens, dtype=np.int32)).cuda()
    qd = to_dev(q)
    B, Hq, T, d = qd.shape
    Hkv, L = kc.shape[1], kc.shape[2]
    g = Guarded()
    o, lse = g.like(qd), g.empty((B, Hq, T), torch.float32)
    ws = g.empty((lib.attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, L, d, splits),), torch.uint8)
    lib.attn_decode_multi(qd, to_dev(kc), to_dev(vc), scale, causal=causal, seqlens=sl, num_splits=splits, o=o,
                          lse=lse, workspace=ws)
    g.check("decode_multi")
    return to_host64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,Hq,Hkv", [(1, 8, 2), (2, 8, 2), (4, 8, 2), (3, 10, 2), (16, 4, 4), (8, 8, 2), (32, 2, 2),
                                     (2, 32, 2), (5, 6, 2), (16, 8, 2), (40, 2, 2), (3, 32, 2)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [0, 3, 16])
def test_decode_multi(gpu_lib, T, Hq, Hkv, d, causal, splits):
    from tests.test_gpu_kv_varlen import check_rows
    print(f"decode_multi T={T} Hq={Hq} Hkv={Hkv} d={d} causal={causal} splits={splits}", flush=True)
    B, L = 6, 1000
    rng = np.random.default_rng(4000 + T + d)
    x = make_prefill(B, Hq, Hkv, T, d, "bf16", seed=4100 + T * Hq + d, qk_mult=2.0, L=L)
    lens = [1000, 0, 1, T - 1 if T > 1 else 2, 33, int(rng.integers(2, L))]
    scale = default_scale(d)
    o, lse = run_decode_multi(gpu_lib, x["q"], x["k"], x["v"], lens, causal, splits, scale)
    o_ref, lse_ref = oracle.decode_multi(x["q"], x["k"], x["v"], scale, causal, seqlens=lens)
    check_rows(o, lse, o_ref, lse_ref, f"T={T} d={d} causal={causal} splits={splits}")


def test_decode_multi_single_token_is_decode_bitwise(gpu_lib, decode_inputs):
    import torch
    _, inp = decode_inputs
    q, kc, vc = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    scale = default_scale(128)
    o1, l1 = gpu_lib.attn_decode(q, kc, vc, scale)
    o2, l2 = gpu_lib.attn_decode_multi(q[:, :, None, :].contiguous(), kc, vc, scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:, :, 0]) and torch.equal(l1, l2[:, :, 0])


def test_decode_multi_full_size_sampled_batches(gpu_lib, decode_inputs):
    """4 tokens per sequence on the decode cache (B=64, Hq=32, Hkv=8, L=8192): 16 (token, head)
    rows per KV head; sampled batches against the oracle."""
    _, inp = decode_inputs
    T = 4
    q = make_prefill(64, 32, 8, T, 128, "bf16", seed=4200)["q"]
    scale = default_scale(128)
    o, lse = run_decode_multi(gpu_lib, q, inp["k"], inp["v"], None, True, 0, scale)
    for b in (0, 37, 63):
        o_ref, lse_ref = oracle.decode_multi(q[b:b + 1], inp["k"][b:b + 1], inp["v"][b:b + 1], scale, True)
        assert_fwd_ok(fwd_errors(o[b:b + 1], o_ref, lse[b:b + 1], lse_ref), f"b{b}")


# ----------------------------------------------------------------------------- HIP graph capture
def test_hip_graph_replay_matches_eager(gpu_lib):
    """Every entry point enqueues kernels only (no allocation, no memset), so a captured graph of
    forward, backward, decode (equal and per-sequence lengths) and the packed forward replays to
    the eager results bit for bit, with eager work and synchronisation between replays."""
    import torch
    d = 128
    scale = default_scale(d)
    inp = make_prefill(1, 4, 2, 300, d, "bf16", seed=4300, with_dout=True)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "dout"))
    dec = make_decode(4, 8, 2, 1000, d, seed=4301)
    dq_, dk_, dv_ = (to_dev(dec[n]) for n in ("q", "k", "v"))
    from synth import make_varlen
    px = make_varlen([5, 0, 300, 77], [5, 9, 300, 200], 4, 2, d, "bf16", seed=4302)
    pq, pk, pv = (to_dev(px[n]) for n in ("q", "k", "v"))
    cq, ck = torch.from_numpy(px["cu_q"]).cuda(), torch.from_numpy(px["cu_k"]).cuda()

    o, lse = torch.empty_like(q), torch.empty((1, 4, 300), dtype=torch.float32, device="cuda")
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    wsb = torch.empty(gpu_lib.attn_bwd_workspace_bytes(1, 4, 2, 300, d), dtype=torch.uint8, device="cuda")
    od, ld = torch.empty_like(dq_), torch.empty((4, 8), dtype=torch.float32, device="cuda")
    wsd = torch.empty(gpu_lib.attn_decode_workspace_bytes(4, 8, 2, 1000, d, 3), dtype=torch.uint8, device="cuda")
    po, pl = torch.empty_like(pq), torch.empty((4, pq.shape[1]), dtype=torch.float32, device="cuda")
    sl = torch.tensor([1000, 0, 37, 640], dtype=torch.int32, device="cuda")  # per-sequence lengths
    ov, lv = torch.empty_like(dq_), torch.empty((4, 8), dtype=torch.float32, device="cuda")
    wsv = torch.empty_like(wsd)

    def work():
        gpu_lib.attn_fwd(q, k, v, True, scale, o=o, lse=lse)
        gpu_lib.attn_bwd(q, k, v, o, lse, do, True, scale, dq=g[0], dk=g[1], dv=g[2], workspace=wsb)
        gpu_lib.attn_decode(dq_, dk_, dv_, scale, num_splits=3, o=od, lse=ld, workspace=wsd)
        gpu_lib.attn_decode_varlen(dq_, dk_, dv_, sl, scale, num_splits=3, o=ov, lse=lv, workspace=wsv)
        gpu_lib.attn_fwd_varlen(pq, pk, pv, cq, ck, 300, True, scale, o=po, lse=pl)

    outs = (o, lse, *g, od, ld, ov, lv, po, pl)
    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(3):
        for t in outs:
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), (rep, i)
        del junk

"""Plain, slow, obviously-correct fp64 reference for exact attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline leg are
the only callers.  It shares no code with the HIP library.

Pages cited (titles as published):
  [FUND] "Attention fundamentals: the standard attention flow, complexity analysis, memory
         bottleneck and inference challenges" (FlashAttention inference tutorial, chapter 2)
  [OPT]  "FlashAttention optimisation: breaking the attention memory bottleneck"
  [NOTE] "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
         (paper note)

The method computes exactly (up to rounding order) the standard attention of [FUND] §2.1,
so the oracle is that definition written out, materialising S and P per (batch, head):
  S = scale * Q K^T, upper triangle (j > i) set to -inf when causal, P = row softmax(S)
  computed with the max-subtracted three-pass softmax of [OPT] §2.2, O = P V.
The per-row log-sum-exp LSE_i = m_i + ln(sum_j exp(S_ij - m_i)) is the statistic the
backward pass reloads ([NOTE] Method, item 3: recompute S and P instead of storing them).
The backward is the textbook softmax gradient (the pages only say that it recomputes):
  dV = P^T dO, dP = dO V^T, D_i = sum_c dO_ic O_ic, dS = P * (dP - D), dQ = scale dS K,
  dK = scale dS^T Q, with dK/dV summed over the query heads that share a KV head.
Grouped-query attention maps query head h to KV head h // (Hq / Hkv) ([OPT] §5.3).
Decode is the same definition with a single query row against a KV cache ([OPT] §4.2.2,
[FUND] §2.3.1); forward_kv takes Nq query rows against Nk keys (the causal mask aligned at
the bottom right), forward_blocksparse the same under a block keep-mask, and forward_varlen
a packed batch of sequences of different lengths.  Every function is pinned by tests against closed forms, invariants,
brute-force scalar loops and hand-derived fixtures; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = ["upcast", "probabilities", "forward", "forward_kv", "forward_blocksparse", "forward_varlen", "forward_rows",
           "backward", "backward_kv", "backward_blocksparse", "backward_varlen", "decode_multi",
           "decode", "split_kv_decode", "lse_merge", "attention_flops"]


def upcast(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 values -> float64, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, row_ids=None) -> np.ndarray:
    """S = scale * q k^T with the causal mask of [FUND] §2.1 (j > i set to -inf).

    q: [n, d] rows whose absolute query positions are row_ids (default 0..n-1); k: [L, d].
    The mask keeps the diagonal (a query attends to itself).
    """
    s = scale * (q @ k.T)
    if causal:
        rows = np.arange(q.shape[0]) if row_ids is None else np.asarray(row_ids)
        cols = np.arange(k.shape[0])
        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
    return s


def _softmax_rows(s: np.ndarray):
    """Safe softmax of [OPT] §2.2: pass 1 row max, pass 2 exp and sum, pass 3 normalise.

    Returns (P, LSE).  A row with every entry masked would give P = 0 and LSE = -inf; the
    square causal mask never produces one.
    """
    m = np.max(s, axis=1, keepdims=True)                         # pass 1
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)                                       # pass 2
    l = np.sum(e, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l > 0, e / l, 0.0)                          # pass 3
        lse = np.where(l > 0, m_safe + np.log(l), -np.inf)
    return p, lse[:, 0]


def probabilities(q, k, scale: float, causal: bool):
    """P for one head: q [N, d], k [L, d] (float64).  Returned for pin tests."""
    p, _ = _softmax_rows(_scores(q, k, scale, causal))
    return p


def _kv_head(h: int, hq: int, hkv: int) -> int:
    assert hq % hkv == 0
    return h // (hq // hkv)


def forward(q, k, v, scale: float, causal: bool):
    """O [B,Hq,N,d] and LSE [B,Hq,N] in float64.

    q: [B,Hq,N,d]; k, v: [B,Hkv,L,d] (float64, or bf16 bits / float32 to be upcast).
    Causal requires L == N (the square mask of [FUND] §2.1).
    """
    q, k, v = upcast(q), upcast(k), upcast(v)
    B, Hq, N, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    if causal:
        assert L == N, "causal mask is defined here for square attention only"
    o = np.empty((B, Hq, N, v.shape[3]))
    lse = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            p, lse[b, h] = _softmax_rows(_scores(q[b, h], k[b, kv], scale, causal))
            o[b, h] = p @ v[b, kv]
    return o, lse


def forward_kv(q, k, v, scale: float, causal: bool):
    """Nq queries against Nk keys: q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] -> O [B,Hq,Nq,d], LSE [B,Hq,Nq].

    Chunked prefill onto a KV cache and multi-token decode sit between the full prefill and
    the single-token decode of [OPT] §4.2.  Reading for the causal mask: the queries are the
    last Nq positions of a sequence whose Nk keys include them, so query i sits at absolute
    position i + Nk - Nq and the square mask of [FUND] §2.1 on absolute positions keeps keys
    j <= i + Nk - Nq (aligned at the bottom right).  A row that keeps no key (Nk = 0, or
    causal with i + Nk - Nq < 0) gets O = 0 and LSE = -inf, the log of an empty sum.
    """
    q, k, v = upcast(q), upcast(k), upcast(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    o = np.zeros((B, Hq, Nq, dv))
    lse = np.full((B, Hq, Nq), -np.inf)
    if Nk == 0:
        return o, lse
    pos = np.arange(Nq) + (Nk - Nq)
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            p, lse[b, h] = _softmax_rows(_scores(q[b, h], k[b, kv], scale, causal, row_ids=pos))
            o[b, h] = p @ v[b, kv]
    return o, lse


def forward_blocksparse(q, k, v, block_mask, scale: float, causal: bool, block: int = 128):
    """forward_kv restricted to the (query block, key block) pairs a mask keeps.

    [OPT] §7.2 names block sparsity.  Reading: with a given block pattern the result is exact
    attention under the element mask that pattern expands to; score (i, j) takes part iff
    block_mask[.., i // block, j // block] is non-zero (and j <= i + Nk - Nq when causal).
    block_mask broadcasts against [B, Hq, ceil(Nq/block), ceil(Nk/block)].  Rows that keep no
    key get O = 0 and LSE = -inf.
    """
    q, k, v = upcast(q), upcast(k), upcast(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    nqb, nkb = -(-Nq // block), -(-Nk // block)
    mask = np.broadcast_to(np.asarray(block_mask) != 0, (B, Hq, nqb, nkb))
    o = np.zeros((B, Hq, Nq, dv))
    lse = np.full((B, Hq, Nq), -np.inf)
    if Nk == 0:
        return o, lse
    pos = np.arange(Nq) + (Nk - Nq)
    qi, kj = np.arange(Nq) // block, np.arange(Nk) // block
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            s = _scores(q[b, h], k[b, kv], scale, causal, row_ids=pos)
            s = np.where(mask[b, h][qi[:, None], kj[None, :]], s, -np.inf)
            p, lse[b, h] = _softmax_rows(s)
            o[b, h] = p @ v[b, kv]
    return o, lse


def forward_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool):
    """A batch of sequences of different lengths, packed without padding ([NOTE] Method,
    implementation details: each sequence at its true length).

    Reading of the packed layout: the batch is folded into the row axis of every head, so
    q [Hq, total_q, d], k/v [Hkv, total_k, d]; sequence b owns query rows cu_q[b]..cu_q[b+1]-1
    and key rows cu_k[b]..cu_k[b+1]-1.  Each sequence is forward_kv on its own rows (causal
    masks aligned with its own lengths).  Returns O [Hq, total_q, d], LSE [Hq, total_q].
    """
    q, k, v = upcast(q), upcast(k), upcast(v)
    Hq, total_q, _ = q.shape
    o = np.zeros((Hq, total_q, v.shape[2]))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        ob, lb = forward_kv(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], scale, causal)
        o[:, q0:q1], lse[:, q0:q1] = ob[0], lb[0]
    return o, lse


def forward_rows(q, k, v, scale: float, causal: bool, rows):
    """O and LSE for selected query rows only: O_i depends on q_i and all of K, V alone
    ([FUND] §2.1: each output row is a weighted average of the rows of V), so a row
    sample is exact per row.  q [B,Hq,N,d]; returns O [B,Hq,R,d], LSE [B,Hq,R].
    """
    rows = np.asarray(rows)
    q = upcast(np.asarray(q)[:, :, rows, :])
    k, v = upcast(k), upcast(v)
    B, Hq, R, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, Hq, R, v.shape[3]))
    lse = np.empty((B, Hq, R))
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            p, lse[b, h] = _softmax_rows(_scores(q[b, h], k[b, kv], scale, causal, row_ids=rows))
            o[b, h] = p @ v[b, kv]
    return o, lse


def backward(q, k, v, dout, scale: float, causal: bool):
    """dQ, dK, dV (float64) of L = sum(O * dO), by recomputing S and P per head.

    D_i = sum_c dO_ic O_ic uses the oracle's own fp64 O.  With grouped-query heads the
    key/value gradients of the query heads sharing a KV head are summed.
    """
    q, k, v, dout = upcast(q), upcast(k), upcast(v), upcast(dout)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            p, _ = _softmax_rows(_scores(q[b, h], k[b, kv], scale, causal))
            o = p @ v[b, kv]
            do = dout[b, h]
            dv[b, kv] += p.T @ do
            dp = do @ v[b, kv].T
            dd = np.sum(do * o, axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, h] = scale * (ds @ k[b, kv])
            dk[b, kv] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_kv(q, k, v, dout, scale: float, causal: bool):
    """backward for Nq queries against Nk keys, the gradient of forward_kv (causal mask aligned
    at the bottom right: query i sees keys j <= i + Nk - Nq).  Rows that see no key have P = 0
    and contribute nothing; their dQ is 0."""
    q, k, v, dout = upcast(q), upcast(k), upcast(v), upcast(dout)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Nk == 0 or Nq == 0:
        return dq, dk, dv
    pos = np.arange(Nq) + (Nk - Nq)
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            p, _ = _softmax_rows(_scores(q[b, h], k[b, kv], scale, causal, row_ids=pos))
            o = p @ v[b, kv]
            do = dout[b, h]
            dv[b, kv] += p.T @ do
            dp = do @ v[b, kv].T
            dd = np.sum(do * o, axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, h] = scale * (ds @ k[b, kv])
            dk[b, kv] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_blocksparse(q, k, v, dout, block_mask, scale: float, causal: bool, block: int = 128):
    """Gradient of forward_blocksparse (the textbook softmax chain rule under the element mask
    the blocks expand to; causal aligned at the bottom right).  Rows that keep no key have P = 0
    and contribute nothing."""
    q, k, v, dout = upcast(q), upcast(k), upcast(v), upcast(dout)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    nqb, nkb = -(-Nq // block), -(-Nk // block)
    mask = np.broadcast_to(np.asarray(block_mask) != 0, (B, Hq, nqb, nkb))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if Nk == 0 or Nq == 0:
        return dq, dk, dv
    pos = np.arange(Nq) + (Nk - Nq)
    qi, kj = np.arange(Nq) // block, np.arange(Nk) // block
    for b in range(B):
        for h in range(Hq):
            kv = _kv_head(h, Hq, Hkv)
            s = _scores(q[b, h], k[b, kv], scale, causal, row_ids=pos)
            s = np.where(mask[b, h][qi[:, None], kj[None, :]], s, -np.inf)
            p, _ = _softmax_rows(s)
            o = p @ v[b, kv]
            do = dout[b, h]
            dv[b, kv] += p.T @ do
            dp = do @ v[b, kv].T
            dd = np.sum(do * o, axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[b, h] = scale * (ds @ k[b, kv])
            dk[b, kv] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_varlen(q, k, v, dout, cu_q, cu_k, scale: float, causal: bool):
    """Gradient of forward_varlen: each packed sequence is backward_kv on its own rows.
    q/dout [Hq, total_q, d], k/v [Hkv, total_k, d]; returns dQ, dK, dV in the same layouts."""
    q, k, v, dout = upcast(q), upcast(k), upcast(v), upcast(dout)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        g = backward_kv(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], dout[None, :, q0:q1], scale, causal)
        dq[:, q0:q1], dk[:, k0:k1], dv[:, k0:k1] = g[0][0], g[1][0], g[2][0]
    return dq, dk, dv


def decode(q, k_cache, v_cache, scale: float, seqlens=None):
    """Single-token decode: q [B,Hq,d] against caches [B,Hkv,L,d]; no mask.

    With seqlens, sequence b attends to the first seqlens[b] keys of its cache (clamped to
    [0, L]); a sequence with no key gets O = 0 and LSE = -inf, the log of an empty sum.
    Returns O [B,Hq,d] and LSE [B,Hq] (float64).  Works one (b, KV head) at a time so
    a large bf16 cache is widened to fp64 slice by slice.
    """
    B, Hq, d = np.asarray(q).shape
    Hkv, L = np.asarray(k_cache).shape[1], np.asarray(k_cache).shape[2]
    g = Hq // Hkv
    o = np.empty((B, Hq, np.asarray(v_cache).shape[3]))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = L if seqlens is None else min(max(int(seqlens[b]), 0), L)
        for kv in range(Hkv):
            rows = slice(kv * g, (kv + 1) * g)
            if n == 0:
                o[b, rows] = 0.0
                lse[b, rows] = -np.inf
                continue
            qg = upcast(q[b, rows])
            kk, vv = upcast(k_cache[b, kv, :n]), upcast(v_cache[b, kv, :n])
            p, lse[b, rows] = _softmax_rows(_scores(qg, kk, scale, False))
            o[b, rows] = p @ vv
    return o, lse


def decode_multi(q, k_cache, v_cache, scale: float, causal: bool, seqlens=None):
    """T query tokens per sequence against its cache: q [B,Hq,T,d], caches [B,Hkv,L,d].

    Sequence b holds seqlens[b] keys (clamped to [0, L]; all L without seqlens) and its T
    tokens are the last T of them, so this is forward_kv of the T queries against those keys
    (causal aligned at the bottom right: token t sees keys j <= len - T + t).  T = 1 is
    decode ([OPT] §4.2.2).  Returns O [B,Hq,T,d], LSE [B,Hq,T].
    """
    B, Hq, T, d = np.asarray(q).shape
    L = np.asarray(k_cache).shape[2]
    o = np.zeros((B, Hq, T, np.asarray(v_cache).shape[3]))
    lse = np.full((B, Hq, T), -np.inf)
    for b in range(B):
        n = L if seqlens is None else min(max(int(seqlens[b]), 0), L)
        ob, lb = forward_kv(q[b:b + 1], k_cache[b:b + 1, :, :n], v_cache[b:b + 1, :, :n], scale, causal)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Merge attention partials computed over disjoint key ranges.

    Each part s holds O_s = softmax over its keys applied to V and lse_s = its log-sum-exp.
    By the order independence of [OPT] §3.2.2 the exact result over the union of keys is
    O = sum_s w_s O_s / sum_s w_s with w_s = exp(lse_s - M), M = max_s lse_s, and
    lse = M + ln(sum_s w_s).  o_parts [S, ..., d], lse_parts [S, ...].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m)
    z = np.sum(w, axis=0)
    o = np.sum(w[..., None] * o_parts, axis=0) / z[..., None]
    return o, m + np.log(z)


def split_kv_decode(q, k_cache, v_cache, scale: float, splits: int):
    """Decode computed as `splits` independent key chunks merged by lse_merge.

    Chunk s covers keys [s*L//splits, (s+1)*L//splits).  Equal to decode() in exact
    arithmetic; the tests use it to pin the merge formula.
    """
    L = np.asarray(k_cache).shape[2]
    bounds = [s * L // splits for s in range(splits + 1)]
    parts = [decode(q, k_cache[:, :, a:b], v_cache[:, :, a:b], scale)
             for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    return lse_merge([p[0] for p in parts], [p[1] for p in parts])


def attention_flops(B, H, N, d, causal: bool, backward: bool = False) -> float:
    """Algorithmic FLOPs: 4 N^2 d per head for the two products of [FUND] §2.2.1
    (QK^T and PV, 2 N^2 d each), exactly halved when causal; the backward counts five
    N^2 d products (S recompute, dV, dP, dQ, dK), i.e. 2.5x the forward.
    """
    f = 4.0 * B * H * N * N * d
    if causal:
        f *= 0.5
    return f * 2.5 if backward else f

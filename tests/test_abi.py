"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/attn.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from exact_io_aware_71_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# Fake, 256-byte-aligned addresses: validation rejects every call below before any
# HIP call could touch them.
P = 0x10000
lib = None


def setup_module(module):
    global lib
    lib = binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "attn_fwd" in names and "attn_bwd" in names and "attn_decode" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding.EXPORTS)


def test_version_and_status_strings():
    assert lib.attn_abi_version() == 2
    assert lib.attn_status_str(0) == b"ok"
    assert lib.attn_status_str(3) == b"workspace too small"


def fwd(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=2, N=64, d=128, dt=1, causal=1, scale=0.1):
    return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, dt, causal, ctypes.c_float(scale), None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(B=0), 1), (dict(N=-3), 1), (dict(Hq=3, Hkv=2), 1),
    (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(scale=-1.0), 1), (dict(k=P + 8), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(dt=0, d=128), 2), (dict(dt=7), 1),
    (dict(B=1 << 16, Hq=1 << 10, Hkv=1 << 10, N=1 << 10), 2),
])
def test_fwd_validation(kwargs, status):
    assert fwd(**kwargs) == status
    assert lib.attn_last_error() != b""


def test_fwd_kv_and_varlen_validation():
    def kv(Nq=64, Nk=128, k=P, d=128, dt=1):
        return lib.attn_fwd_kv(P, k, P, P, P, 1, 2, 2, Nq, Nk, d, dt, 1, ctypes.c_float(0.1), None)
    assert kv(Nq=0) == 1
    assert kv(Nk=-1) == 1
    assert kv(d=96) == 2
    assert kv(Nk=1 << 23) == 2          # a head's N*d above 2^29
    assert kv(k=None) == 1              # keys present but no pointer

    def vl(cu_q=P, cu_k=P, B=4, total_q=100, total_k=300, max_q=40, q=P, k=P, dt=1):
        return lib.attn_fwd_varlen(q, k, P, P, P, cu_q, cu_k, B, 2, 1, total_q, total_k, max_q, 64, dt, 1,
                                   ctypes.c_float(0.1), None)
    assert vl(cu_q=None) == 1
    assert vl(cu_k=P + 2) == 1          # int32 offsets must be 4-byte aligned
    assert vl(max_q=101) == 1           # longer than the packed total
    assert vl(max_q=-1) == 1
    assert vl(total_k=-5) == 1
    assert vl(B=0) == 1
    assert vl(q=None) == 1
    assert lib.attn_last_error() != b""


def test_fwd_blocksparse_validation():
    def bs(mask=P, sb=0, sh=0, Nq=256, Nk=256, dt=1, d=128):
        return lib.attn_fwd_blocksparse(P, P, P, P, P, mask, sb, sh, 1, 2, 2, Nq, Nk, d, dt, 1, ctypes.c_float(0.1),
                                        None)
    assert bs(mask=None) == 1
    assert bs(sb=-1) == 1
    assert bs(sh=-4) == 1
    assert bs(Nq=0) == 1
    assert bs(dt=0, d=64) == 2           # fp32 is dense only
    assert bs(Nk=524224 + 1) == 2        # beyond the tile list
    assert bs(d=96) == 2


def test_bwd_blocksparse_validation():
    def bb(mask=P, sb=0, sh=0, N=1024, Hq=4, Hkv=2, dt=1, ws_bytes=1 << 30):
        return lib.attn_bwd_blocksparse(P, P, P, P, P, P, P, P, P, mask, sb, sh, 1, Hq, Hkv, N, 128, dt, 1,
                                        ctypes.c_float(0.1), P, ws_bytes, None)
    assert bb(mask=None) == 1
    assert bb(sh=-1) == 1
    assert bb(N=0) == 1
    assert bb(N=131072 + 64) == 2            # tiles beyond 2047
    assert bb(N=65536, Hq=16, Hkv=2) == 2    # 8 heads x 1024 tiles > 8191 pairs
    assert bb(dt=0) == 2
    assert bb(ws_bytes=16) == 3


def bwd(ws=P, ws_bytes=1 << 30, Hq=2, Hkv=2, d=128, dt=1, scale=0.1, dq=P):
    return lib.attn_bwd(P, P, P, P, P, P, dq, P, P, 1, Hq, Hkv, 64, d, dt, 1, ctypes.c_float(scale),
                        ws, ws_bytes, None)


def r256(x):
    return (x + 255) // 256 * 256


def flags(B, Hq, N):
    """One 4-byte flag per wave (four per 128-query dQ workgroup), rounded up to 256 bytes."""
    return r256(B * Hq * ((N + 127) // 128) * 4 * 4)


def test_bwd_workspace_split():
    """Causal grouped-query backward with few key blocks splits each group's query heads over two
    dK/dV workgroups; their fp32 partial sums follow the statistics and the dQ flags."""
    stats = 2 * 1 * 32 * 4096 * 4
    part = 4 * 1 * 8 * 4096 * 128 * 4            # [dV, dK] x [two halves] x B*Hkv*N x d, fp32
    assert lib.attn_bwd_workspace_bytes(1, 32, 8, 4096, 128) == stats + flags(1, 32, 4096) + part
    assert lib.attn_bwd_workspace_bytes(1, 32, 32, 4096, 128) == stats + flags(1, 32, 4096)  # no groups
    assert lib.attn_bwd_workspace_bytes(1, 6, 2, 4096, 128) == 2 * 6 * 4096 * 4 + flags(1, 6, 4096)  # odd group
    assert lib.attn_bwd_workspace_bytes(4, 32, 8, 4096, 128) == 2 * 4 * 32 * 4096 * 4 + flags(4, 32, 4096)


def test_bwd_validation():
    need = lib.attn_bwd_workspace_bytes(1, 2, 2, 64, 128)
    assert need == 1024 + 256                # LSE2 and D rows padded to 64 queries; dQ flags
    assert lib.attn_bwd_workspace_bytes(1, 2, 2, 65, 128) == 2 * 2 * 128 * 4 + flags(1, 2, 65)
    assert bwd(dq=None) == 1
    assert bwd(Hq=3, Hkv=2) == 1           # Hq must be a multiple of Hkv
    assert bwd(dt=0) == 2
    assert bwd(d=80) == 2
    assert bwd(ws=None) == 3
    assert bwd(ws_bytes=need - 1) == 3
    assert bwd(ws=P + 16) == 1               # workspace must be 256-byte aligned


def test_bwd_varlen_validation():
    need = lib.attn_bwd_varlen_workspace_bytes(3, 4, 100)
    assert need == r256(2 * 4 * (100 + 64 * 3) * 4) + flags(3, 4, 100)

    def bv(cu_q=P, cu_k=P, ws=P, ws_bytes=need, max_q=40, max_k=50, total_k=200, dt=1):
        return lib.attn_bwd_varlen(P, P, P, P, P, P, P, P, P, cu_q, cu_k, 3, 4, 2, 100, total_k, max_q, max_k, 128, dt,
                                   1, ctypes.c_float(0.1), ws, ws_bytes, None)
    assert bv(cu_q=None) == 1
    assert bv(cu_k=P + 1) == 1
    assert bv(max_q=101) == 1
    assert bv(max_k=201) == 1
    assert bv(ws_bytes=need - 1) == 3
    assert bv(ws=None) == 3
    assert bv(dt=0) == 2


def test_decode_plan_and_validation():
    s = lib.attn_decode_auto_splits(64, 32, 8, 8192, 128)
    assert 1 <= s <= 64
    need = lib.attn_decode_workspace_bytes(64, 32, 8, 8192, 128, 0)
    assert need >= s * 64 * 32 * (128 + 1) * 4
    # Requests beyond the number of 32-key blocks are clamped.
    assert lib.attn_decode_workspace_bytes(1, 4, 1, 40, 64, 1000) == \
        lib.attn_decode_workspace_bytes(1, 4, 1, 40, 64, 2)

    def dec(Hq=32, Hkv=8, d=128, dt=1, splits=0, ws=P, ws_bytes=need, scale=0.1):
        return lib.attn_decode(P, P, P, P, P, 64, Hq, Hkv, 8192, d, dt, ctypes.c_float(scale), splits, ws,
                               ws_bytes, None)
    assert lib.attn_decode(P, P, P, P, P, 1, 8194, 2, 64, 128, 1, ctypes.c_float(0.1), 0, P, 1 << 30, None) == 2
    assert b"rows per KV head" in lib.attn_last_error()  # 4097 heads per group
    assert dec(d=32) == 2
    assert dec(dt=0) == 2
    assert dec(splits=-1) == 1
    assert dec(ws=None) == 3
    assert dec(ws_bytes=need - 4) == 3
    assert dec(scale=float("inf")) == 1

    def decm(T=4, Hq=32, Hkv=8, seqlens=P):
        return lib.attn_decode_multi(P, P, P, seqlens, P, P, 64, Hq, Hkv, T, 8192, 128, 1, 1, ctypes.c_float(0.1), 0, P,
                                     1 << 30, None)
    assert decm(T=0) == 1
    assert decm(T=1025) == 2         # 1025 tokens x 4 heads > 4096 rows per KV head
    assert decm(seqlens=P + 4) == 1  # misaligned
    assert lib.attn_decode_multi_workspace_bytes(64, 32, 8, 4, 8192, 128, 0) >= 4 * need - 1024

    def decv(seqlens=P, d=128):
        return lib.attn_decode_varlen(P, P, P, seqlens, P, P, 64, 32, 8, 8192, d, 1, ctypes.c_float(0.1), 0, P,
                                      need, None)
    assert decv(seqlens=None) == 1
    assert decv(seqlens=P + 4) == 1  # misaligned
    assert decv(d=32) == 2


def test_decode_workspace_layout():
    """Decode partials are B*Hq*T rows of d fp32 values plus one fp32 LSE each, each array
    256-byte aligned: (splits + 1) sets on the vector-ALU path (up to 8 (token, head) rows per KV
    head; the stream-K split of per-sequence lengths writes up to one set more than the split
    count) and 4 * splits sets on the matrix-core path (one partial per wave)."""
    def size(rows, d):
        up = lambda x: (x + 255) // 256 * 256
        return up(rows * d * 4) + up(rows * 4)
    B, Hq, Hkv, L = 3, 8, 2, 1000
    for d in (64, 128):
        for s in (1, 3, 16):  # 1000 keys in chunks of 1000, 352 and 64 keys: exactly s chunks
            assert lib.attn_decode_workspace_bytes(B, Hq, Hkv, L, d, s) == size((s + 1) * B * Hq, d)
            assert lib.attn_decode_multi_workspace_bytes(B, Hq, Hkv, 2, L, d, s) == size((s + 1) * B * Hq * 2, d)
            # 4 tokens x 4 heads = 16 rows per KV head: the matrix-core path.
            assert lib.attn_decode_multi_workspace_bytes(B, Hq, Hkv, 4, L, d, s) == size(4 * s * B * Hq * 4, d)


def test_decode_noalloc_validation():
    """attn_decode_noalloc: argument errors as attn_decode, and shapes whose partials exceed the
    library's fixed 16 MiB scratch are refused before any HIP call."""
    def decn(B=64, Hq=32, Hkv=8, L=8192, d=128, dt=1, splits=0, q=P, scale=0.1):
        return lib.attn_decode_noalloc(q, P, P, P, P, B, Hq, Hkv, L, d, dt, ctypes.c_float(scale), splits, None)
    assert binding.DECODE_NOALLOC_SCRATCH_BYTES == 16 << 20
    # The decode workload fits (about 3.2 MB of partials).
    assert lib.attn_decode_workspace_bytes(64, 32, 8, 8192, 128, 0) <= binding.DECODE_NOALLOC_SCRATCH_BYTES
    big = lib.attn_decode_workspace_bytes(4096, 32, 8, 8192, 128, 0)
    assert big > binding.DECODE_NOALLOC_SCRATCH_BYTES
    assert decn(B=4096) == 2
    assert b"scratch" in lib.attn_last_error()
    assert decn(splits=64) == 2      # 64 splits of the decode workload: 67 MB of partials
    assert decn(q=None) == 1
    assert decn(q=P + 8) == 1        # misaligned
    assert decn(d=32) == 2
    assert decn(dt=0) == 2
    assert decn(splits=-1) == 1
    assert decn(scale=float("nan")) == 1
    assert decn(Hq=30) == 1          # Hq not a multiple of Hkv


def test_binding_raises_typed_error():
    with pytest.raises(binding.AttnError) as ei:
        binding._check(fwd(d=96))
    assert ei.value.status == 2


def test_calibration_library_loads_and_validates():
    """The benchmark's calibration library (streaming read, MFMA loop, atomic adds) loads,
    exports its entry points and rejects bad arguments before launching anything."""
    from exact_io_aware_71_amd import build
    calib = ctypes.CDLL(build.CALIB_LIB)
    calib.calib_stream_read.restype = ctypes.c_int
    calib.calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    calib.calib_mfma.restype = ctypes.c_int
    calib.calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    invalid = 1  # hipErrorInvalidValue
    assert calib.calib_stream_read(None, 1024, P, 4, None) == invalid
    assert calib.calib_stream_read(P, 1000, P, 4, None) == invalid
    assert calib.calib_stream_read(P, 1024, P, 0, None) == invalid
    assert calib.calib_mfma(4, 8, None, P, None) == invalid
    assert calib.calib_mfma(4, 7, P, P, None) == invalid
    assert calib.calib_mfma(0, 8, P, P, None) == invalid
    calib.calib_atomic_add.restype = ctypes.c_int
    calib.calib_atomic_add.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    assert calib.calib_atomic_add(None, 32, 4096, 16, 1024, None) == invalid
    assert calib.calib_atomic_add(P, 32, 100, 16, 1024, None) == invalid  # N not a multiple of 64
    assert calib.calib_atomic_add(P, 0, 4096, 16, 1024, None) == invalid
    assert calib.calib_atomic_add(P, 32, 4096, 16, 0, None) == invalid

// C-ABI entry points of libexact_attn.so (declared in include/attn.h).
//
// Every argument is validated on the host before any HIP call, so the validation paths are
// exercised without a GPU.  The library allocates nothing: scratch space comes from the
// caller's workspace, which keeps every call capturable in a HIP graph.  The one exception,
// attn_decode_noalloc, takes its scratch from a fixed device array of the library instead.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

namespace {

constexpr int kAbiVersion = 2;
thread_local char g_err[512] = "";

attn_status_t fail(attn_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

attn_status_t ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

attn_status_t check_scale(float scale) {
  if (!(isfinite(scale) && scale > 0.f)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", (double)scale);
  return ATTN_OK;
}

// Element offsets of a head are formed in 64-bit, row indices and byte offsets within a head
// in 32-bit: keep B*H*N in int range and a head's bytes (N*d elements of up to 4 bytes) below
// 2^31.
attn_status_t check_rows(int B, int Hq, int Hkv, int N, int d) {
  if ((long long)B * Hq * N > 0x7fffffffLL || (long long)B * Hkv * N > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "B*H*N exceeds 2^31-1");
  if ((long long)N * d > (1LL << 29)) return fail(ATTN_ERR_UNSUPPORTED, "N*d exceeds 2^29 per head");
  return ATTN_OK;
}

attn_status_t check_heads(int B, int Hq, int Hkv, int N, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d N=%d d=%d)", B, Hq, Hkv, N, d);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  return check_rows(B, Hq, Hkv, N, d);
}

#define RETURN_IF(expr)                 \
  do {                                  \
    attn_status_t _s = (expr);          \
    if (_s != ATTN_OK) return _s;       \
  } while (0)

attn_status_t from_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Split choice for decode (chunks of whole 32-key blocks): about 1024 workgroups, but chunks of
// at least 2048 keys where that still leaves 256 workgroups (one per CU), and never chunks
// under 256 keys.  Measured on the 2 GiB cache and on longer caches of fewer sequences (B=4,
// L=32768; B=1, L=65536): 512-1024 workgroups of long chunks stream fastest, and chunks of
// 1024 keys or fewer cost 7-25% there in partial results and their merge.
int auto_splits(int B, int Hkv, int L) {
  const long long groups = (long long)B * Hkv;
  long long s = (1024 + groups - 1) / groups;
  const long long long_chunks = (L + 2047) / 2048;
  if (s > long_chunks) s = long_chunks;
  const long long fill = (256 + groups - 1) / groups;
  if (s < fill) s = fill;
  const long long max_by_len = (L + 255) / 256;
  if (s > max_by_len) s = max_by_len;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

// Effective (splits, keys per split) for a requested count.
void decode_plan(int L, int requested, int* splits, int* kps) {
  const int blocks = (L + 31) / 32;
  int s = requested;
  if (s > blocks) s = blocks;
  if (s < 1) s = 1;
  const int per = (blocks + s - 1) / s;  // 32-key blocks per split
  *kps = per * 32;
  *splits = (L + *kps - 1) / *kps;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return kAbiVersion; }

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_err; }

// Shared by the three forward entry points: dense (cu_q == nullptr) with Nq query and Nk key
// rows per head, or packed variable-length with totals Nq, Nk and longest query run max_q.
static attn_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_q,
                              const int* cu_k, int B, int Hq, int Hkv, int Nq, int Nk, int max_q, int d,
                              attn_dtype_t dtype, int causal, float scale, void* stream,
                              const unsigned char* block_mask = nullptr, long long mask_sb = 0,
                              long long mask_sh = 0) {
  if ((Nq > 0 && (!q || !o)) || (Nk > 0 && (!k || !v)))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-null (k and v may be null when there are no keys)");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d)", B, Hq, Hkv, d);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Nq < 0 || Nk < 0 || max_q < 0 || max_q > Nq)
    return fail(ATTN_ERR_INVALID_ARG, "bad row counts (Nq=%d Nk=%d max_q=%d)", Nq, Nk, max_q);
  const int Bd = cu_q ? 1 : B;  // packed tensors hold the batch inside the row count
  RETURN_IF(check_rows(Bd, Hq, Hq, Nq, d));
  RETURN_IF(check_rows(Bd, Hkv, Hkv, Nk, d));
  if ((long long)B * Hq * ((max_q + 31) / 32) > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
  RETURN_IF(check_scale(scale));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (dtype == ATTN_BF16) {
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "bf16 forward supports d in {64, 128} (got %d)", d);
  } else if (dtype == ATTN_F32) {
    if (d != 64) return fail(ATTN_ERR_UNSUPPORTED, "fp32 forward supports d == 64 only (got %d)", d);
  } else {
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  }
  xattn::FwdArgs a{q, k, v, o, lse, cu_q, cu_k, B, Hq, Hkv, Nq, Nk, max_q, d, dtype == ATTN_BF16 ? 1 : 0,
                   causal ? 1 : 0, scale, (hipStream_t)stream, block_mask, mask_sb, mask_sh};
  return from_hip(xattn::launch_fwd(a), "attn_fwd launch");
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                       int Hkv, int N, int d, attn_dtype_t dtype, int causal, float scale, void* stream) {
  if (N <= 0) return fail(ATTN_ERR_INVALID_ARG, "N must be positive (got %d)", N);
  return fwd_impl(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, N, N, N, d, dtype, causal, scale, stream);
}

attn_status_t attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int Nq, int Nk, int d, attn_dtype_t dtype, int causal, float scale,
                          void* stream) {
  if (Nq <= 0 || Nk < 0) return fail(ATTN_ERR_INVALID_ARG, "need Nq > 0 and Nk >= 0 (got Nq=%d Nk=%d)", Nq, Nk);
  return fwd_impl(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, Nq, d, dtype, causal, scale, stream);
}

attn_status_t attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const unsigned char* block_mask, long long mask_stride_b,
                                   long long mask_stride_h, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                   attn_dtype_t dtype, int causal, float scale, void* stream) {
  if (!block_mask) return fail(ATTN_ERR_INVALID_ARG, "block_mask must be non-null");
  if (mask_stride_b < 0 || mask_stride_h < 0)
    return fail(ATTN_ERR_INVALID_ARG, "mask strides must be >= 0 (got %lld, %lld)", mask_stride_b, mask_stride_h);
  if (Nq <= 0 || Nk < 0) return fail(ATTN_ERR_INVALID_ARG, "need Nq > 0 and Nk >= 0 (got Nq=%d Nk=%d)", Nq, Nk);
  if (dtype == ATTN_F32) return fail(ATTN_ERR_UNSUPPORTED, "block-sparse forward supports bf16 only");
  if (Nk > xattn::kMaxSparseKeys)
    return fail(ATTN_ERR_UNSUPPORTED, "block-sparse forward supports Nk <= %d (got %d)", xattn::kMaxSparseKeys, Nk);
  return fwd_impl(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Nq, Nk, Nq, d, dtype, causal, scale, stream,
                  block_mask, mask_stride_b, mask_stride_h);
}

attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                              int total_q, int total_k, int max_seqlen_q, int d, attn_dtype_t dtype, int causal,
                              float scale, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be non-null");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens arrays must be 4-byte aligned");
  return fwd_impl(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k, max_seqlen_q, d,
                  dtype, causal, scale, stream);
}

// Rows of the backward's per-row statistics are padded to whole 64-query tiles: per head in the
// dense layout, per sequence (64 spare rows each) in the packed one.
int bwd_npad(int N) { return (N + 63) / 64 * 64; }

static size_t bwd_stats_bytes(int B, int Hq, int N) {
  return align_up(2 * (size_t)B * Hq * bwd_npad(N) * sizeof(float), 256);
}
static size_t bwd_varlen_stats_bytes(int B, int Hq, int total_q) {
  return align_up(2 * (size_t)Hq * ((size_t)total_q + 64 * (size_t)B) * sizeof(float), 256);
}
// One word per wave of each dQ workgroup of 128 queries (its "walk again with the exact D"
// flag), after the statistics; the packed layout bounds the longest sequence by the total.
static size_t bwd_flag_bytes(int B, int Hq, int max_q) {
  return align_up((size_t)B * Hq * (size_t)((max_q + 127) / 128) * 4 * sizeof(unsigned), 256);
}
// fp32 partial dK/dV of the split grouped-query backward (see kBwdSplitGrid), after the flags.
static size_t bwd_part_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (!xattn::bwd_split_possible(B, Hq, Hkv, N) || d <= 0) return 0;
  return align_up(4 * (size_t)B * Hkv * N * d * sizeof(float), 256);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return bwd_stats_bytes(B, Hq, N) + bwd_flag_bytes(B, Hq, N) + bwd_part_bytes(B, Hq, Hkv, N, d);
}

size_t attn_bwd_varlen_workspace_bytes(int B, int Hq, int total_q) {
  if (B <= 0 || Hq <= 0 || total_q < 0) return 0;
  return bwd_varlen_stats_bytes(B, Hq, total_q) + bwd_flag_bytes(B, Hq, total_q);
}

// Shared by attn_bwd (dense, cu_q == nullptr) and attn_bwd_varlen (packed).
static attn_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, const int* cu_q, const int* cu_k, int B,
                              int Hq, int Hkv, int Nq, int Nk, int max_q, int max_k, int d, attn_dtype_t dtype,
                              int causal, float scale, void* workspace, size_t workspace_bytes, void* stream,
                              const unsigned char* block_mask = nullptr, long long mask_sb = 0, long long mask_sh = 0) {
  if ((Nq > 0 && (!q || !o || !lse || !dout || !dq)) || (Nk > 0 && (!k || !v || !dk || !dv)))
    return fail(ATTN_ERR_INVALID_ARG, "all tensor pointers of attn_bwd must be non-null");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d)", B, Hq, Hkv, d);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Nq < 0 || Nk < 0 || max_q < 0 || max_q > Nq || max_k < 0 || max_k > Nk)
    return fail(ATTN_ERR_INVALID_ARG, "bad row counts (Nq=%d Nk=%d max_q=%d max_k=%d)", Nq, Nk, max_q, max_k);
  const int Bd = cu_q ? 1 : B;
  RETURN_IF(check_rows(Bd, Hq, Hq, Nq, d));
  RETURN_IF(check_rows(Bd, Hkv, Hkv, Nk, d));
  if ((long long)B * Hq * ((max_q + 63) / 64) > 0x7fffffffLL || (long long)B * Hkv * ((max_k + 127) / 128) > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
  RETURN_IF(check_scale(scale));
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (dtype != ATTN_BF16) return fail(dtype == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID_ARG,
                                      "backward supports bf16 only");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "backward supports d in {64, 128} (got %d)", d);
  const size_t need = cu_q ? attn_bwd_varlen_workspace_bytes(B, Hq, Nq) : attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, d);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "attn_bwd needs %zu workspace bytes (got %zu)", need, workspace ? workspace_bytes : 0);
  if (!aligned256(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const long long stride = cu_q ? (long long)Nq + 64LL * B : bwd_npad(Nq);
  const long long half = cu_q ? (long long)Hq * stride : (long long)B * Hq * stride;
  const size_t stats_bytes = cu_q ? bwd_varlen_stats_bytes(B, Hq, Nq) : bwd_stats_bytes(B, Hq, Nq);
  unsigned* flags = (unsigned*)((char*)workspace + stats_bytes);
  float* part = nullptr;  // dense causal grouped-query backward with few key blocks: split dK/dV
  if (!cu_q && causal && bwd_part_bytes(B, Hq, Hkv, Nq, d) > 0)
    part = (float*)((char*)workspace + stats_bytes + bwd_flag_bytes(B, Hq, Nq));
  xattn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, cu_q, cu_k, B, Hq, Hkv, Nq, Nk, max_q, max_k, d,
                   causal ? 1 : 0, scale, (float*)workspace, stride, half, (hipStream_t)stream, block_mask, mask_sb,
                   mask_sh, part, flags};
  return from_hip(xattn::launch_bwd(a), "attn_bwd launch");
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                       attn_dtype_t dtype, int causal, float scale, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (N <= 0) return fail(ATTN_ERR_INVALID_ARG, "N must be positive (got %d)", N);
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, B, Hq, Hkv, N, N, N, N, d, dtype, causal,
                  scale, workspace, workspace_bytes, stream);
}

attn_status_t attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                   const void* dout, void* dq, void* dk, void* dv, const unsigned char* block_mask,
                                   long long mask_stride_b, long long mask_stride_h, int B, int Hq, int Hkv, int N,
                                   int d, attn_dtype_t dtype, int causal, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!block_mask) return fail(ATTN_ERR_INVALID_ARG, "block_mask must be non-null");
  if (mask_stride_b < 0 || mask_stride_h < 0)
    return fail(ATTN_ERR_INVALID_ARG, "mask strides must be >= 0 (got %lld, %lld)", mask_stride_b, mask_stride_h);
  if (N <= 0) return fail(ATTN_ERR_INVALID_ARG, "N must be positive (got %d)", N);
  // The dK/dV workgroup lists its group's kept (head, 64-row tile) pairs: at most 8191 of them,
  // tiles below 2048 and at most 32 heads per group.
  if (Hkv > 0 && Hq % Hkv == 0 &&
      ((long long)(Hq / Hkv) * ((N + 63) / 64) > xattn::kMaxSparseKeys / 64 || N > 2048 * 64 || Hq / Hkv > 32))
    return fail(ATTN_ERR_UNSUPPORTED, "block-sparse backward supports (Hq/Hkv) * ceil(N/64) <= 8191, N <= 131072");
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, B, Hq, Hkv, N, N, N, N, d, dtype, causal, scale,
                  workspace, workspace_bytes, stream, block_mask, mask_stride_b, mask_stride_h);
}

attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                              const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k,
                              int max_seqlen_q, int max_seqlen_k, int d, attn_dtype_t dtype, int causal, float scale,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be non-null");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens arrays must be 4-byte aligned");
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, d, dtype, causal, scale, workspace, workspace_bytes, stream);
}

int attn_decode_auto_splits(int B, int Hq, int Hkv, int L, int d) {
  (void)Hq;
  (void)d;
  if (B <= 0 || Hkv <= 0 || L <= 0) return 0;
  return auto_splits(B, Hkv, L);
}

size_t attn_decode_multi_workspace_bytes(int B, int Hq, int Hkv, int T, int L, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || L <= 0 || d <= 0 || num_splits < 0) return 0;
  int splits, kps;
  decode_plan(L, num_splits == 0 ? auto_splits(B, Hkv, L) : num_splits, &splits, &kps);
  const size_t rows = xattn::decode_partial_rows(splits, T, Hq / Hkv, (size_t)B * Hq * T);
  return align_up(rows * d * sizeof(float), 256) + align_up(rows * sizeof(float), 256);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int num_splits) {
  return attn_decode_multi_workspace_bytes(B, Hq, Hkv, 1, L, d, num_splits);
}

// ------------------------------------------------------------ scratch of attn_decode_noalloc
// The split partials of attn_decode_noalloc live in this array instead of a caller workspace.
// Each GPU the library runs on holds its own copy until the process ends; host code reaches
// it only through the device address hipGetSymbolAddress returns on that device (the array's
// name on the host is a stand-in, not a device address), looked up once per device.
constexpr size_t kNoallocScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
static attn_status_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

// use_scratch: take the partials from the library's scratch array (attn_decode_noalloc); the
// workspace arguments are then ignored.
static attn_status_t decode_impl(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                                 void* o, float* lse, int B, int Hq, int Hkv, int L, int d, attn_dtype_t dtype,
                                 float scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream,
                                 int T = 1, int causal = 0, bool use_scratch = false) {
  if (!q || !k_cache || !v_cache || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be non-null");
  if (T <= 0) return fail(ATTN_ERR_INVALID_ARG, "T must be positive (got %d)", T);
  RETURN_IF(check_heads(B, Hq, Hkv, L, d));
  if ((long long)B * Hq * T > 0x7fffffffLL) return fail(ATTN_ERR_UNSUPPORTED, "B*Hq*T exceeds 2^31-1");
  RETURN_IF(check_scale(scale));
  if (num_splits < 0) return fail(ATTN_ERR_INVALID_ARG, "num_splits must be >= 0 (got %d)", num_splits);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (dtype != ATTN_BF16) return fail(dtype == ATTN_F32 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID_ARG,
                                      "decode supports bf16 only");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "decode supports d in {64, 128} (got %d)", d);
  if ((long long)T * (Hq / Hkv) > xattn::kDecMaxRows)
    return fail(ATTN_ERR_UNSUPPORTED, "decode supports at most %d (token, head) rows per KV head (T=%d, group %d)",
                xattn::kDecMaxRows, T, Hq / Hkv);
  const size_t need = attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, L, d, num_splits);
  if (use_scratch) {
    if (need > kNoallocScratchBytes)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "attn_decode_noalloc needs %zu scratch bytes for this shape, above the %zu the library holds "
                  "(use attn_decode with a workspace)", need, kNoallocScratchBytes);
    RETURN_IF(noalloc_scratch(&workspace));
    workspace_bytes = kNoallocScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "attn_decode needs %zu workspace bytes (got %zu)", need, workspace ? workspace_bytes : 0);
  if (!aligned256(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int splits, kps;
  decode_plan(L, num_splits == 0 ? auto_splits(B, Hkv, L) : num_splits, &splits, &kps);
  if ((long long)B * Hkv * ((T * (Hq / Hkv) + 31) / 32) * splits > 0x7fffffffLL)
    return fail(ATTN_ERR_UNSUPPORTED, "decode grid too large");
  const size_t rows = xattn::decode_partial_rows(splits, T, Hq / Hkv, (size_t)B * Hq * T);
  float* part_o = (float*)workspace;
  float* part_lse = (float*)((char*)workspace + align_up(rows * d * sizeof(float), 256));
  xattn::DecodeArgs a{q, k_cache, v_cache, o, lse, B, Hq, Hkv, L, d, scale, splits, kps, part_o, part_lse,
                      (hipStream_t)stream, seqlens, T, causal ? 1 : 0};
  return from_hip(xattn::launch_decode(a), "attn_decode launch");
}

attn_status_t attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B,
                          int Hq, int Hkv, int L, int d, attn_dtype_t dtype, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, nullptr, o, lse, B, Hq, Hkv, L, d, dtype, scale, num_splits, workspace,
                     workspace_bytes, stream);
}

attn_status_t attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                  int B, int Hq, int Hkv, int L, int d, attn_dtype_t dtype, float scale,
                                  int num_splits, void* stream) {
  return decode_impl(q, k_cache, v_cache, nullptr, o, lse, B, Hq, Hkv, L, d, dtype, scale, num_splits, nullptr, 0,
                     stream, 1, 0, true);
}

attn_status_t attn_decode_multi(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                                void* o, float* lse, int B, int Hq, int Hkv, int T, int L, int d, attn_dtype_t dtype,
                                int causal, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (seqlens && !aligned16(seqlens)) return fail(ATTN_ERR_INVALID_ARG, "seqlens must be 16-byte aligned");
  return decode_impl(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, L, d, dtype, scale, num_splits, workspace,
                     workspace_bytes, stream, T, causal);
}

attn_status_t attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                                 void* o, float* lse, int B, int Hq, int Hkv, int L, int d, attn_dtype_t dtype,
                                 float scale, int num_splits, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!seqlens) return fail(ATTN_ERR_INVALID_ARG, "seqlens must be non-null");
  if (!aligned16(seqlens)) return fail(ATTN_ERR_INVALID_ARG, "seqlens must be 16-byte aligned");
  return decode_impl(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, L, d, dtype, scale, num_splits, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

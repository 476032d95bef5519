/*
 * exact_attn — exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libexact_attn.so.  Plain pointers and sizes only.
 *
 * Pages cited by title:
 *   [FUND] "Attention fundamentals: the standard attention flow, complexity analysis,
 *          memory bottleneck and inference challenges" (FlashAttention inference tutorial,
 *          chapter 2)
 *   [OPT]  "FlashAttention optimisation: breaking the attention memory bottleneck"
 *   [NOTE] "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 *          (paper note)
 *
 * What is computed ([FUND] §2.1): per (batch b, query head h) with KV head
 * kv = h / (Hq / Hkv) ([OPT] §5.3, consecutive query heads share a KV head):
 *     S = scale * Q K^T,   S_ij = -inf for j > i when causal (the diagonal is kept),
 *     P = row-softmax(S),  O = P V,   LSE_i = ln(sum_j exp(S_ij))  (natural log).
 * The kernels never write S or P to memory: Q, K and V are processed in tiles with the
 * running max / running sum of [OPT] §3.1-§3.2 and [NOTE] Method items 1-2; the backward
 * recomputes S and P from Q, K, V and the saved LSE ([NOTE] Method item 3).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library allocates
 *     nothing and keeps no device state, so every call may be captured in a HIP graph.
 *   - Layouts are dense, row-major: Q/O/dQ/dO [B, Hq, N, d]; K/V/dK/dV [B, Hkv, N, d];
 *     LSE and D are fp32 [B, Hq, N]; decode Q/O are [B, Hq, d] (one token each), the KV
 *     cache [B, Hkv, L, d].  Element type is given by `dtype` for Q/K/V/O/dO/dQ/dK/dV.
 *   - Pointers must be 16-byte aligned.  `scale` must be finite and > 0.
 *   - Sizes: B*H*N below 2^31 and N*d at most 2^29 per head (offsets within a head are 32-bit);
 *     larger requests return ATTN_ERR_UNSUPPORTED.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls only
 *     enqueue work and return; kernel faults surface at the caller's synchronisation.
 *   - Arguments are validated before any HIP call.  On a non-OK return nothing has been
 *     enqueued and attn_last_error() (thread-local) describes the problem.
 *   - Calls are thread-safe.  Calls that write the same buffers must be ordered by the
 *     caller (same stream or events).
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, Hq % Hkv != 0, bad scale */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement (see each call) */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the matching *_workspace_bytes() */
  ATTN_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} attn_status_t;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* ABI revision of this header; bumped on any incompatible change. */
int attn_abi_version(void);

/* Static description of a status code. */
const char* attn_status_str(attn_status_t status);

/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* attn_last_error(void);

/*
 * Forward attention ([FUND] §2.1; tiled online softmax of [OPT] §3.1-§3.2, deferred
 * normalisation of [OPT] §7.1).
 *   q [B,Hq,N,d], k/v [B,Hkv,N,d]  inputs (read only)
 *   o [B,Hq,N,d]                   output, same dtype as q
 *   lse [B,Hq,N] fp32              optional output (NULL to skip); needed by attn_bwd
 *   causal != 0                    mask j > i (square attention, query i vs key j)
 * Supported: dtype BF16 with d in {64, 128}; dtype F32 with d == 64.  Other d or dtype
 * combinations return ATTN_ERR_UNSUPPORTED.  No workspace.  Bitwise deterministic.
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, attn_dtype_t dtype, int causal,
                       float scale, void* stream);

/*
 * Forward attention of Nq queries against Nk keys per (batch, head): chunked prefill of Nq new
 * tokens onto a cache of Nk keys, or multi-token decode, the cases between the full prefill
 * and the single-token decode of [OPT] §4.2.1-§4.2.2.  Reading: the queries are the last Nq
 * positions of a sequence whose keys are the Nk cached ones (the new tokens included).
 *   q/o [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], lse [B,Hq,Nq] (optional)
 *   causal != 0        query i sees keys j <= i + (Nk - Nq): the mask is aligned at the bottom
 *                      right, so the last query sees every key and Nq == Nk is attn_fwd's mask
 * A query row that sees no key (Nk == 0, or causal with i + Nk - Nq < 0) gets o = 0 and
 * lse = -inf (the log of an empty sum).  Nq >= 1, Nk >= 0.  Supported d and dtype as attn_fwd;
 * no workspace; bitwise deterministic.
 */
attn_status_t attn_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, attn_dtype_t dtype,
                          int causal, float scale, void* stream);

/*
 * Block-sparse forward: attn_fwd_kv restricted to the (query block, key block) pairs a mask
 * keeps, exact for that pattern ([OPT] §7.2 names block sparsity; here no weight is dropped
 * that the mask keeps).  Blocks are 128 query rows by 128 keys:
 *   block_mask  uint8 device array; byte (b, h, i, j) at
 *               block_mask[b*mask_stride_b + h*mask_stride_h + i*ceil(Nk/128) + j]
 *               keeps (non-zero) or drops (zero) the scores of query rows 128i .. 128i+127
 *               against keys 128j .. 128j+127, for i < ceil(Nq/128), j < ceil(Nk/128);
 *               strides in bytes, >= 0 (0 shares one [ceil(Nq/128), ceil(Nk/128)] mask)
 *   causal      applied on top of the mask, aligned at the bottom right as in attn_fwd_kv
 * Score (i, j) enters the softmax iff its block is kept (and j <= i + Nk - Nq when causal); a
 * row that keeps no key gets o = 0 and lse = -inf.  Dropped blocks are neither loaded nor
 * multiplied where a whole workgroup (256 query rows at d = 128, 128 at d = 64) drops them.
 * Supported: BF16, d in {64, 128}, Nk <= 524224 (8191 tiles of 64).  Other arguments as
 * attn_fwd_kv.
 */
attn_status_t attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const unsigned char* block_mask, long long mask_stride_b,
                                   long long mask_stride_h, int B, int Hq, int Hkv, int Nq, int Nk,
                                   int d, attn_dtype_t dtype, int causal, float scale, void* stream);

/*
 * Forward attention over a batch of sequences of different lengths with no padding ([NOTE]
 * Method, implementation details: each sequence is processed at its true length).  The tensors are packed: the batch
 * is folded into the row axis of each head.
 *   q/o [Hq,total_q,d], k/v [Hkv,total_k,d], lse [Hq,total_q] fp32 (optional)
 *   cu_seqlens_q/k [B+1] int32 device arrays, 4-byte aligned, non-decreasing from 0 to
 *                  total_q/total_k: sequence b owns query rows cu_seqlens_q[b] ..
 *                  cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *   max_seqlen_q   the longest query sequence (sizes the grid; rows of a sequence at positions
 *                  >= max_seqlen_q are not computed), 0 <= max_seqlen_q <= total_q
 *   causal         per sequence as in attn_fwd_kv (bottom-right aligned with its own lengths)
 * Sequences may be empty; a query row that sees no key gets o = 0 and lse = -inf.  The
 * kernels clamp the offsets into [0, total] and make them non-decreasing, so malformed arrays
 * give wrong rows but no out-of-bounds access.  Supported d and dtype as attn_fwd.
 */
attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                              int Hkv, int total_q, int total_k, int max_seqlen_q, int d,
                              attn_dtype_t dtype, int causal, float scale, void* stream);

/* Bytes of device workspace attn_bwd needs:
 *   - fp32 per-row statistics (LSE * log2(e) and -D, see attn_bwd) for every query row padded
 *     to a multiple of 64: 2 * B * Hq * roundup(N, 64) * 4 bytes, rounded up to 256;
 *   - one 4-byte flag per wave of 32 query rows, B * Hq * ceil(N/128) * 4 * 4 bytes rounded up
 *     to 256 (a wave that meets a probability above 1/2 asks for D from its definition);
 *   - when Hq/Hkv is even and above 1 and B * Hkv * ceil(N/128) < 512, 4 * B * Hkv * N * d * 4
 *     bytes (rounded up to 256) of fp32 partial dK/dV: a causal backward of such a shape splits
 *     each group's query heads over two dK/dV workgroups (the causal work of the key blocks
 *     differs too much for one round of workgroups) and adds their two partial sums in a fixed
 *     order. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/*
 * Backward attention by recomputation ([NOTE] Method item 3): S and P are rebuilt per tile
 * from q, k, v and the forward's lse; nothing of size N x N is stored.
 *   q, k, v, o, lse                 exactly what attn_fwd consumed and produced
 *   dout [B,Hq,N,d]                 upstream gradient dL/dO
 *   dq [B,Hq,N,d], dk/dv [B,Hkv,N,d] outputs (overwritten, same dtype as q)
 *   workspace                        >= attn_bwd_workspace_bytes(...) device bytes, 256-byte
 *                                    aligned; contents on entry are ignored
 * Supported: BF16, d in {64, 128}.  Grouped-query heads ([OPT] §5.3, kv = h / (Hq/Hkv)): dk and
 * dv of a KV head are the sums of the gradients of the Hq/Hkv query heads sharing it.
 * D_i = sum_j P_ij dP_ij enters dS = P (dP - D).  It is taken as rowsum(dO * O) from the stored
 * O, except where the bf16 rounding of O could dominate the nearly cancelling dP - D of a key
 * that carries most of a row: 128-query blocks whose keys fit two 64-key tiles form D from its
 * definition in the first dQ launch, and blocks that hold a row whose largest probability
 * exceeds 1/2 get it from a second dQ launch, which also computes their dQ again (dK and dV use
 * that D too).
 * Deterministic (no atomics).
 */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int Hq, int Hkv, int N, int d, attn_dtype_t dtype, int causal,
                       float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of attn_fwd_blocksparse for square attention (Nq = Nk = N): the gradient of exact
 * attention under the block keep-mask (same layout and strides as attn_fwd_blocksparse, 128 x
 * 128 blocks), by recomputation.  Both backward kernels walk only kept tiles: the dQ workgroup
 * of 128 queries (one mask row of blocks) its kept 64-key tiles, the dK/dV workgroup of 128
 * keys (one mask column) its kept (query head, 64-query tile) pairs.  Rows that keep no key get
 * dq = 0, keys that no query keeps get dk = dv = 0.
 *   q, k, v, o, lse, dout   as attn_bwd, with o and lse from attn_fwd_blocksparse (same mask)
 *   workspace               >= attn_bwd_workspace_bytes(B, Hq, Hkv, N, d)
 * Supported: BF16, d in {64, 128}, (Hq/Hkv) * ceil(N/64) <= 8191, N <= 131072.
 */
attn_status_t attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                   const unsigned char* block_mask, long long mask_stride_b,
                                   long long mask_stride_h, int B, int Hq, int Hkv, int N, int d,
                                   attn_dtype_t dtype, int causal, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_bwd_varlen needs: the same two fp32 statistics per query
 * row, each sequence padded by up to 64 rows, i.e. 2 * Hq * (total_q + 64 * B) * 4 bytes,
 * rounded up to 256, then the flags of attn_bwd for B * Hq * ceil(total_q/128) workgroups
 * (B * Hq * ceil(total_q/128) * 16 bytes, rounded up to 256). */
size_t attn_bwd_varlen_workspace_bytes(int B, int Hq, int total_q);

/*
 * attn_bwd for the packed variable-length layout of attn_fwd_varlen ([NOTE] Method: no
 * padding; item 3: recomputation): q/o/dout/dq [Hq,total_q,d], k/v/dk/dv [Hkv,total_k,d],
 * lse [Hq,total_q] as attn_fwd_varlen wrote it, offsets cu_seqlens_q/k [B+1] (int32, device,
 * 4-byte aligned), max_seqlen_q/k the longest query and key sequences (they size the grids).
 * Causal masks per sequence are aligned at the bottom right (as attn_fwd_varlen).  Query rows
 * that see no key get dq = 0; keys that no query sees get dk = dv = 0.
 *   workspace  >= attn_bwd_varlen_workspace_bytes(B, Hq, total_q), 256-byte aligned
 * Supported: BF16, d in {64, 128}, Hq a multiple of Hkv.  Deterministic (no atomics).
 */
attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                              int Hkv, int total_q, int total_k, int max_seqlen_q,
                              int max_seqlen_k, int d, attn_dtype_t dtype, int causal, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split count attn_decode uses for num_splits == 0 (the automatic choice), so callers can
 * size the workspace and reproduce the split.
 */
int attn_decode_auto_splits(int B, int Hq, int Hkv, int L, int d);

/* Bytes of workspace attn_decode needs for the given split count (0 = automatic). */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int num_splits);

/*
 * Single-token decode against a KV cache ([OPT] §4.2.2 and §5.3; [FUND] §2.3.1), no mask.
 * The key axis is split into `num_splits` contiguous chunks processed in parallel; each
 * chunk yields a partial (O_s, lse_s) and a second pass merges them by log-sum-exp, which
 * is exact by the order independence of the online softmax ([OPT] §3.2.2).
 *   q [B,Hq,d]                 one query token per sequence and head
 *   k_cache/v_cache [B,Hkv,L,d] caches (read only)
 *   o [B,Hq,d]                 output, same dtype as q
 *   lse [B,Hq] fp32            optional output (NULL to skip)
 *   num_splits                 0 = attn_decode_auto_splits(), else 1..L (clamped to
 *                              ceil(L/32) chunks of whole 32-key blocks)
 *   workspace                  >= attn_decode_workspace_bytes(...) bytes, 256-byte aligned
 * Supported: BF16, d in {64, 128}, 1 <= Hq/Hkv <= 4096.  Bitwise deterministic for a fixed
 * split count.
 */
attn_status_t attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                          float* lse, int B, int Hq, int Hkv, int L, int d, attn_dtype_t dtype,
                          float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * attn_decode without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and results as attn_decode with the same num_splits (bit for bit); the split
 * partials go to a fixed scratch array inside the library instead of a caller workspace.
 *   - The scratch holds ATTN_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, set aside on
 *     every GPU the library runs on until the process ends.  A shape whose
 *     attn_decode_workspace_bytes(...) exceeds it returns ATTN_ERR_UNSUPPORTED (nothing is
 *     enqueued); the decode workload (B=64, Hq=32, Hkv=8, L=8192, d=128, automatic splits)
 *     needs about 3.2 MB.
 *   - The call allocates nothing: no hipMalloc, no hipFree, no library routine that
 *     allocates.  Its first call on a device looks up the scratch's device address there once.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (other
 *     streams, other threads, a graph replayed while another call runs) race and must be
 *     ordered by the caller.  No state carries over between calls: every partial is written
 *     before the merge reads it.
 * Errors: as attn_decode (minus the workspace errors), plus ATTN_ERR_UNSUPPORTED above.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
attn_status_t attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                                  float* lse, int B, int Hq, int Hkv, int L, int d,
                                  attn_dtype_t dtype, float scale, int num_splits, void* stream);

/*
 * attn_decode for a batch whose sequences hold different numbers of cached keys (caches of
 * one capacity L, each sequence b filled to its own length).  Sequence b attends to keys
 * [0, seqlens[b]) of its cache rows; everything else is as in attn_decode (same workspace
 * size for the same L and num_splits).  Up to 2048 sequences (and 2^31 32-key blocks over all
 * B*Hkv groups) the num_splits*B*Hkv workgroups each take an equal share of the 32-key blocks
 * of all groups, so a long sequence is cut over many of them and short ones share one: the
 * time follows the total length, not the longest.  Beyond that, fixed key chunks of L as in
 * attn_decode.
 *   seqlens [B] int32          device array, 16-byte aligned, read by the kernels; values are
 *                              clamped to [0, L]; a sequence of length 0 gets o = 0 and
 *                              lse = -inf (the log of an empty sum)
 * Errors: as attn_decode, plus ATTN_ERR_INVALID_ARG for a null or misaligned seqlens.
 */
attn_status_t attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                                 int L, int d, attn_dtype_t dtype, float scale, int num_splits,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace attn_decode_multi needs for T tokens per sequence (0 splits = automatic,
 * the same split choice as attn_decode). */
size_t attn_decode_multi_workspace_bytes(int B, int Hq, int Hkv, int T, int L, int d, int num_splits);

/*
 * Multi-token decode: T new tokens per sequence against its cache ([OPT] §4.2.2 for one token;
 * T > 1 is the verification step of speculative decoding, between decode and the chunked
 * prefill of attn_fwd_kv).  Same split-KV + LSE merge as attn_decode; the T tokens of all
 * g = Hq/Hkv heads of a KV head are processed together, so the cache is read once per group.
 *   q [B,Hq,T,d], o [B,Hq,T,d], lse [B,Hq,T] fp32 (optional)
 *   k_cache/v_cache [B,Hkv,L,d]; seqlens [B] int32 device (16-byte aligned) or NULL for L
 *   causal != 0   token t sees keys j <= len - T + t (the tokens are the last T cached
 *                 positions of their sequence); causal == 0: every token sees all len keys
 * A token that sees no key gets o = 0 and lse = -inf.  T = 1 computes what attn_decode (or,
 * with seqlens, attn_decode_varlen) computes.
 * Supported: BF16, d in {64, 128}, T * Hq/Hkv <= 4096 (beyond 32 rows per KV head the cache is
 * read once per 32 rows).  Workspace as attn_decode_multi_workspace_bytes().  Bitwise
 * deterministic for a fixed split count.
 */
attn_status_t attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                                const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                                int T, int L, int d, attn_dtype_t dtype, int causal, float scale,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */

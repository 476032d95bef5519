// Internal launcher interface between the C-ABI layer (api.hip) and the kernel files.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace xattn {

// Forward: dense Q/O [B,Hq,Nq,d], K/V [B,Hkv,Nk,d] (cu_q == nullptr), or packed
// variable-length Q/O [Hq,Nq,d], K/V [Hkv,Nk,d] with per-sequence offsets cu_q/cu_k [B+1]
// (Nq, Nk are then the totals and max_q the longest query sequence).  Causal masks are
// aligned at the bottom right of each (query, key) block.
struct FwdArgs {
  const void* q; const void* k; const void* v; void* o; float* lse;
  const int* cu_q; const int* cu_k;
  int B, Hq, Hkv, Nq, Nk, max_q, d, dtype, causal;
  float scale;
  hipStream_t stream;
  const unsigned char* block_mask;  // optional [B, Hq, ceil(Nq/128), ceil(Nk/128)] keep bytes (dense layout only)
  long long mask_sb, mask_sh;       // batch and head strides of block_mask in bytes
};

// Backward: dense [B,H,N,d] tensors (cu_q == nullptr, Nq == Nk == N) or packed
// variable-length [H,total,d] tensors with offsets cu_q/cu_k [B+1] (Nq, Nk the totals, max_q,
// max_k the longest sequences).  The workspace holds two fp32 halves (LSE*log2(e), then -D,
// D = sum_j P_ij dP_ij = rowsum(dO*O)) of `stat_half` floats; the rows of (b, h) start at (b*Hq + h)*stat_stride
// (dense, stat_stride = roundup(N, 64)) or at h*stat_stride + cu_q[b] + 64b (packed,
// stat_stride = total_q + 64B), so every sequence owns roundup(len, 64) rows.
struct BwdArgs {
  const void* q; const void* k; const void* v; const void* o; const float* lse; const void* dout;
  void* dq; void* dk; void* dv;
  const int* cu_q; const int* cu_k;
  int B, Hq, Hkv, Nq, Nk, max_q, max_k, d, causal;
  float scale;
  float* stats;
  long long stat_stride, stat_half;
  hipStream_t stream;
  const unsigned char* block_mask;  // optional [B, Hq, ceil(N/128), ceil(N/128)] keep bytes (dense layout only)
  long long mask_sb, mask_sh;       // batch and head strides of block_mask in bytes
  float* part;                      // fp32 [2 (dV, dK)][2 halves][B*Hkv*N][d] for the split dK/dV, or null
  unsigned* flags;                  // [ceil(max_q/128) * B * Hq][4]: per dQ wave, walk again with the exact D
};

// Causal grouped-query backward with few key blocks: when the dK/dV grid has fewer workgroups
// than this, the query heads of each group are split over two workgroups per key block (their
// causal work differs by up to the number of key blocks, and one round of workgroups would run
// as long as the heaviest); each writes fp32 partial sums that a second pass adds in a fixed
// order.  Dense layout (with or without a block mask), even group size.
constexpr int kBwdSplitGrid = 512;
inline bool bwd_split_possible(int B, int Hq, int Hkv, int N) {
  if (B <= 0 || Hkv <= 0 || N <= 0 || Hq % Hkv != 0) return false;
  const int g = Hq / Hkv;
  return g >= 2 && g % 2 == 0 && (long long)B * Hkv * ((N + 127) / 128) < kBwdSplitGrid;
}

struct DecodeArgs {
  const void* q; const void* k; const void* v; void* o; float* lse;
  int B, Hq, Hkv, L, d;
  float scale;
  int splits;           // effective number of key chunks (>= 1, every chunk non-empty)
  int keys_per_split;   // multiple of 32
  float* part_o;        // [splits * partials per split, B, Hq, T, d] fp32
  float* part_lse;      // [splits * partials per split, B, Hq, T] fp32 (base-2 log-sum-exp)
  hipStream_t stream;
  const int* seqlens;   // [B] keys per sequence (device), clamped to [0, L]; null = L for all
  int T;                // query tokens per sequence (T * Hq/Hkv <= kDecMaxRows); q/o [B,Hq,T,d]
  int causal;           // token t sees keys j <= len - T + t
};

// Longest key sequence the block-sparse forward walks (its tile list holds 8191 tiles of 64).
constexpr int kMaxSparseKeys = 8191 * 64;

// Decode path: rows = T * (Hq/Hkv) (token, head) pairs per KV head.  Up to kDecValuRows
// rows the vector-ALU kernel (one partial per workgroup), above it the matrix-core kernel
// (one partial per wave: four per workgroup; 32 rows per workgroup) up to kDecMaxRows.  Measured on the 2 GiB decode
// cache: at 4 and 8 rows the vector-ALU kernel is 3-6% faster, at 16 rows the matrix-core one
// 1.7x (its P V no longer scales with the row count).
constexpr int kDecValuRows = 8;
constexpr int kDecMaxRows = 4096;
inline bool decode_uses_mma(int T, int g) { return T * g > kDecValuRows; }
inline int decode_partials_per_split(int T, int g) { return decode_uses_mma(T, g) ? 4 : 1; }
// Per-sequence lengths on the vector-ALU kernel take the stream-K split (equal block ranges per
// workgroup) up to kDecSkMaxB sequences and 2^31 blocks in all.
constexpr int kDecSkMaxB = 2048;
inline bool decode_stream_k(bool has_seqlens, int B, int Hkv, int L) {
  return has_seqlens && B <= kDecSkMaxB && (long long)B * Hkv * ((L + 31) / 32) < (1LL << 31);
}
// Partial rows of a decode with `splits` key chunks: the stream-K split writes up to
// splits*B*Hkv + B*Hkv group partials, so the vector-ALU path reserves one set more.
inline size_t decode_partial_rows(int splits, int T, int g, size_t BHqT) {
  return decode_uses_mma(T, g) ? (size_t)splits * 4 * BHqT : (size_t)(splits + 1) * BHqT;
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

}  // namespace xattn

// Shared device helpers for the gfx950 (CDNA4) attention kernels.
//
// Register layouts used throughout (wave64, verified on gfx950):
//   v_mfma_f32_32x32x16_bf16  A[32 x 16]: lane l holds row l%32, k-group l/32 (8 values)
//                             B[16 x 32]: lane l holds col l%32, k-group l/32 (8 values)
//                             C[32 x 32]: lane l, register r holds
//                                         row 8*(r/4) + 4*(l/32) + r%4, col l%32
//   v_mfma_f32_16x16x32_bf16  A: row l%16, k-group l/16; B: col l%16, k-group l/16;
//                             C: lane l, register r holds row 4*(l/16) + r, col l%16
//   v_mfma_f32_32x32x2_f32    A: row l%32, k = l/32; B: col l%32, k = l/32; C as above
// The hardware pairs A's k-slot (group, element) with B's same slot, so any consistent
// assignment of contraction indices to slots gives the exact product.
//
// ds_read_b64_tr_b16 (transposing LDS read): within each 16-lane group, lane j supplies an
// address of 4 contiguous 16-bit values; output lane i receives, as element e, value (i%4)
// of source lane 4*e + i/4.  With source lanes reading rows r0 + j/4 at columns
// c0 + 4*(j%4), output lane i gets the column c0 + i over rows r0..r0+3: a row-major LDS
// tile read as a column, which is what an MFMA operand needs when its contraction index
// is the tile's row index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace xattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 2^x on the hardware exp unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value held by lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Broadcast lane `src` of each 16-lane row to the whole row (DPP row_newbcast).
template <int src>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + src, 0xf, 0xf, false));
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {lo, hi};
  const bf16x2 v = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ s16x4 ds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, lds_addr));
}
__device__ __forceinline__ bf16x8 join_tr(const s16x4& a, const s16x4& b) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// LDS tiles of 64 rows x D bf16 columns are stored unpadded with the 16-byte chunks of each
// row XOR-permuted by a function of the row index, chosen so that
//   (i)  a 16-byte read of one chunk from 16 consecutive rows (an MFMA operand whose rows
//        are the tile rows), and
//   (ii) a ds_read_b64_tr_b16 over a 4-row x 4-chunk block starting at a row multiple of 4
// each touch 16 distinct 4-bank groups of the 64-bank LDS, i.e. run without bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  static_assert(D == 64 || D == 128, "tile width");
  if constexpr (D == 128) return row * 256 + 16 * (chunk ^ (4 * (row & 3) + ((row >> 2) & 3)));
  else return row * 128 + 16 * (chunk ^ (4 * ((row >> 1) & 1) + ((row >> 2) & 3)));
}
// Byte offset of element (row, col) in the swizzled tile (col multiple of 4 for 8-byte reads).
template <int D>
__device__ __forceinline__ int swz_elem(int row, int col) {
  return swz<D>(row, col >> 3) + (col & 7) * 2;
}

// Transposed MFMA operand from a swizzled 64 x D LDS tile: lane gets column col0 + lane%32
// over rows row0 + {8t + 4*(lane/32) + i : t in 0..1, i in 0..3}, the contraction slots that
// pair with C-layout registers 8*sh .. 8*sh+7 of a 32x32 MFMA output (row0 = 16*sh + ...).
template <int D>
__device__ __forceinline__ bf16x8 ld_tr_operand(const char* tile, int row0, int col0, int lane) {
  const int G = lane >> 4, j = lane & 15;
  const int row = row0 + 4 * (G >> 1) + (j >> 2);
  const int col = col0 + 16 * (G & 1) + 4 * (j & 3);
  return join_tr(ds_read_tr16(tile + swz_elem<D>(row, col)), ds_read_tr16(tile + swz_elem<D>(row + 8, col)));
}

// Lane-dependent LDS byte offsets of the MFMA operands inside a swizzled 64 x D tile: k[c] for
// row-major operands (row lane%32, chunk 2c + lane/32: K or V rows as the A operand of a
// 32x32x16 product), v[db][e] for the transposed reads of columns db*32 .. (rows rl, rl + 8
// of ld_tr_operand's pattern).  The swizzle depends on the row modulo 16 only, so for row
// blocks starting at multiples of 16 the block's row offset is a constant added to these.
template <int D>
struct TileOffsets {
  uint32_t k[D / 16];
  uint32_t v[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, h32 = lane >> 5;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) k[c] = swz<D>(l32, 2 * c + h32);
    const int G = lane >> 4, j = lane & 15;
    const int rl = 4 * (G >> 1) + (j >> 2), cl = 16 * (G & 1) + 4 * (j & 3);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) v[db][e] = swz_elem<D>(rl + 8 * e, db * 32 + cl);
  }
  // Switch between two LDS stages (stage size a power of two larger than every offset).
  __device__ __forceinline__ void toggle(uint32_t stage_bytes) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) k[c] ^= stage_bytes;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      v[db][0] ^= stage_bytes;
      v[db][1] ^= stage_bytes;
    }
  }
};

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// As ld_global16 for data read once (a decode's KV cache): the nontemporal hint streams it past
// the caches (a plain read of 4 GiB: 6.3 TB/s with the hint's loads at 7.1).
template <typename T>
__device__ __forceinline__ T ld_global_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4, SGPR base + 32-bit
// VGPR byte offset): lane i's bytes land at lds + 16 * i.  `base` and `lds` must be the same
// for every lane of the wave.  Issued from inline assembly so that the compiler does not tie
// later LDS reads of other buffers to its completion; the caller waits explicitly with
// wait_vmem*() before a barrier that publishes the data.  M0 holds the LDS destination;
// nothing else in these kernels keeps a value in M0.
__device__ __forceinline__ const void* wave_uniform(const void* p) {
  const uintptr_t u = (uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uintptr_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const void* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(wave_uniform(base)), "s"(m0v)
               : "memory");
}

// As dma16 with a wave-uniform base already in scalar registers and the LDS byte address given
// directly (a wave-uniform value).
__device__ __forceinline__ void dma16_m0(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory");
}

// Raw buffer resource (stride 0) over `bytes` bytes at the wave-uniform address `base`: a
// load through it at a byte offset at or past `bytes` returns zeros, dword by dword (no memory
// access), so a copy of rows past the end of a tensor needs no clamping.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes) {
  const uintptr_t u = (uintptr_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)u;
  r[1] = (int)((uint32_t)(u >> 32) & 0xffffu);  // address bits 47:32; stride 0
  r[2] = bytes > 0 ? bytes : 0;
  r[3] = 0x00020000;  // 32-bit data format, no swizzle
  return r;
}

// As dma16_m0 through a buffer resource: lane i's 16 bytes at byte offset voff of the buffer
// (zeros where out of range) land at lds_addr + 16 * i.
__device__ __forceinline__ void bdma16_m0(const i32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "s"(lds_addr)
               : "memory");
}

// As dma16_m0 with 4 bytes per lane.
__device__ __forceinline__ void dma4_m0(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds_addr) : "memory");
}

// As dma16 with 4 bytes per lane (global_load_lds_dword): lane i's word lands at lds + 4 * i.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, const void* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(wave_uniform(base)), "s"(m0v)
               : "memory");
}

// s_waitcnt vmcnt(0): every global load (register or LDS destination) of this wave has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(n): all but the n most recent global loads of this wave have landed (loads
// complete in order).
template <int n>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// Workgroup barrier that waits only for this wave's LDS operations (lgkmcnt(0)), not for
// outstanding global loads, so prefetches may stay in flight across it.  The wavefront-scope
// fences keep the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Rows of one (batch, head) slice of the forward's tensors.  Dense tensors are [B, H, N, d]
// (cu == nullptr): slice (b, h) starts at row (b*H + h)*N and holds N rows.  Packed
// variable-length tensors are [H, total, d], the batch folded into the sequence axis:
// sequence b of head h starts at row h*total + cu[b] and holds cu[b+1] - cu[b] rows.  The
// offsets are clamped into [0, total] and made non-decreasing, so a malformed offset array
// yields wrong rows but never an access outside the tensors.
struct SeqGeo {
  const int* cu_q;  // [B+1] query offsets, or nullptr (dense)
  const int* cu_k;  // [B+1] key offsets (used when cu_q is not null)
  int nq, nk;       // dense: rows per head; packed: total rows
};
struct SeqRows {
  size_t q, k;      // first row of the slice in Q/O/LSE and in K/V
  int lq, lk;       // query and key rows of the slice
};
__device__ __forceinline__ SeqRows seq_rows(const SeqGeo& g, int b, int hq, int Hq, int hk, int Hkv) {
  SeqRows r;
  if (g.cu_q == nullptr) {
    r.lq = g.nq;
    r.lk = g.nk;
    r.q = ((size_t)b * Hq + hq) * g.nq;
    r.k = ((size_t)b * Hkv + hk) * g.nk;
  } else {
    const int q0 = min(max(g.cu_q[b], 0), g.nq), q1 = min(max(g.cu_q[b + 1], q0), g.nq);
    const int k0 = min(max(g.cu_k[b], 0), g.nk), k1 = min(max(g.cu_k[b + 1], k0), g.nk);
    r.lq = q1 - q0;
    r.lk = k1 - k0;
    r.q = (size_t)hq * g.nq + q0;
    r.k = (size_t)hk * g.nk + k0;
  }
  return r;
}

// Block-sparse mask: byte (b, h, i, j) at mask[b*sb + h*sh + i*nkb + j] keeps (non-zero) or
// drops (zero) every score of query block i (rows 128i .. 128i+127) against key block j
// (keys 128j .. 128j+127).  Strides of 0 share one mask across batches or heads.
constexpr int kSparseBlock = 128;
// A tile list is an LDS array of kMaxSparseTiles uint16 entries whose last entry holds the
// count, so at most kMaxSparseTiles - 1 tiles (16 KB in all: two dQ workgroups still fit a CU).
constexpr int kMaxSparseTiles = 8192;
struct BlockMask {
  const unsigned char* mask;  // nullptr: dense
  long long sb, sh;
  int nqb, nkb;
};

// Lists, in key order, the 64-key tiles t < T that some query block of a workgroup's QB
// blocks (starting at block qb0) keeps: entry = t | (keep bits of the QB blocks) << 14.
// Wave 0 compacts 64 tiles per ballot; returns the count to every thread (one barrier).
template <int QB>
__device__ __forceinline__ int build_tile_list(const BlockMask& bm, int b, int h, int qb0, int T, uint16_t* list) {
  static_assert(QB >= 1 && QB <= 2, "two keep bits per entry");
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    const unsigned char* rows = bm.mask + b * bm.sb + h * bm.sh;
    int n = 0;
    for (int t0 = 0; t0 < T; t0 += 64) {
      const int t = t0 + lane;
      uint32_t keep = 0;
      if (t < T) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
          if (qb0 + i < bm.nqb && rows[(size_t)(qb0 + i) * bm.nkb + (t >> 1)] != 0) keep |= 1u << i;
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep != 0);
      const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (keep != 0) list[pos] = (uint16_t)(t | (keep << 14));
      n += __builtin_popcountll(bal);
    }
    if (lane == 0) list[kMaxSparseTiles - 1] = (uint16_t)n;
  }
  __syncthreads();
  return list[kMaxSparseTiles - 1];
}

// Initial running max of the forward kernels: the most negative finite float rather than
// -inf, so that 2^(s - m) of a masked score (s = -inf) is 0 even for a row that has seen
// no key yet, and a row without any key ends with l = 0 (O = 0, LSE = -inf).
constexpr float kMaxInit = -3.402823466e38f;

// Pins the instruction order: the scheduler moves nothing across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

}  // namespace xattn

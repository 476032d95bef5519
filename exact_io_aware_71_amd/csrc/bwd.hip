// Backward attention kernels for gfx950: recompute S and P per tile from Q, K, V and the
// forward's log-sum-exp instead of storing them.
//
// Pages cited by title:
//   [NOTE] "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
//   [OPT]  "FlashAttention optimisation: breaking the attention memory bottleneck"
//
// [NOTE] Method item 3: the backward rebuilds S and P from Q/K/V blocks, trading about one
// extra forward's FLOPs for O(N) instead of O(N^2) activation memory.  The gradient of
// O = softmax(scale Q K^T) V (the pages only state that it recomputes; this is the
// textbook chain rule):
//   P = exp(scale S - LSE), dV = P^T dO, dP = dO V^T, D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three launches (four for a causal grouped-query shape with few key blocks), deterministic
// (no atomics):
//   1. bwd_dq_kernel: one workgroup per 128 queries; S^T = K Q^T and dP^T = V dO^T with
//      Q and dO resident in registers, K/V tiles streamed through LDS; dS^T in the C layout
//      is the A operand of dQ = dS K, K entering through the transposing read.  It also
//      writes D = rowsum(dO * O) (sum_j P_ij dP_ij where the rows' keys fit two tiles) and
//      LSE * log2(e) of its rows into row-padded arrays of the caller's workspace (padding
//      rows get LSE = +inf, so their probabilities vanish), and flags each wave that met a
//      probability above 1/2.
//   2. bwd_dq_kernel again (REDO): workgroups with a flagged wave form D = sum_j P_ij dP_ij
//      from its definition, write it, and compute their dQ again with it; the others exit.
//   3. bwd_dkdv_lag_kernel: one workgroup per 128 keys of a KV head; each wave keeps its 32
//      keys' K (or V) rows in registers as the B operand of S = Q K^T (or dP = dO V^T) and
//      its dV (or dK) accumulator in registers, while [Q | dO | LSE | D] tiles of 64 queries
//      stream through a three-stage LDS ring.  In the C layout of S each lane owns one key,
//      so P and dS are already the A operand of dV = P^T dO and dK = dS^T Q; dO and Q enter
//      those products through the transposing ds_read_b64_tr_b16.  Causal: query tiles
//      before the diagonal are never visited.  With few key blocks and an even group size the
//      group's query heads split over two workgroups whose fp32 partial sums
//      bwd_dkdv_sum_kernel adds (the fourth launch).
// Every kernel takes the per-sequence row map of the forward (dense [B,H,N,d], or packed
// variable-length [H,total,d] with offsets), and causal masks aligned at the bottom right:
// query i of Nq sees keys j <= i + Nk - Nq.
#include "common.h"
#include "launch.h"

namespace xattn {

// MFMA operands read from LDS run this many MFMA slots ahead of their use (dK/dV and dQ).
constexpr int kDkdvLookahead = 4;
constexpr int kDqLookahead = 4;

// ------------------------------------------------------------------ D = rowsum(dO * O), LSE2
// First statistics row of (b, h) in each half of the workspace (see BwdArgs).
__device__ __forceinline__ size_t stat_row(const SeqGeo& g, long long stride, int b, int h, int Hq) {
  if (g.cu_q == nullptr) return ((size_t)b * Hq + h) * stride;
  return (size_t)h * stride + min(max(g.cu_q[b], 0), g.nq) + 64 * (size_t)b;
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int sh) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(x[8 * sh + 2 * e], x[8 * sh + 2 * e + 1]);
  return as_bf16x8(u);
}

// ------------------------------------------------------------------ dK, dV
constexpr int kBwdBQ = 64;   // queries per streamed tile (dK/dV kernel)
constexpr int kBwdBK = 64;   // keys per streamed tile (dQ kernel)

template <int D>
struct BwdTile {
  static constexpr int BYTES = 64 * D * 2;   // one swizzled 64-row tile
};

// Block-sparse dK/dV: lists the (query head, query tile) pairs of a workgroup that the mask
// keeps, in the order the virtual tile sequence visits them: heads h0 .. h0+g-1 of the group,
// 64-row tiles qt_begin .. qt_begin+nt-1 each, against key block kb; entry = tile | (head
// offset << 11).  Wave 0 compacts 64 pairs per ballot; the count lands in the list's last
// entry and is returned to every thread (one barrier).
__device__ __forceinline__ int build_qtile_list(const BlockMask& bm, int b, int h0, int g, int kb, int qt_begin, int nt,
                                                uint16_t* list) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    int n = 0;
    const int total = g * nt;
    for (int i0 = 0; i0 < total; i0 += 64) {
      const int i = i0 + lane;
      bool keep = false;
      int e = 0;
      if (i < total) {
        const int hh = i / nt, t = qt_begin + (i - hh * nt);
        keep = bm.mask[b * bm.sb + (h0 + hh) * bm.sh + (size_t)(t >> 1) * bm.nkb + kb] != 0;
        e = t | (hh << 11);
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (keep) list[pos] = (uint16_t)e;
      n += __builtin_popcountll(bal);
    }
    if (lane == 0) list[kMaxSparseTiles - 1] = (uint16_t)n;
  }
  __syncthreads();
  return list[kMaxSparseTiles - 1];
}

// dK, dV with a lagged dK wave.  Waves g and g + 4 share a SIMD and the same 32 keys, the
// first accumulating dV, the second dK, and P crosses from the first to the second through
// LDS (as bf16, the precision the dS product rounds to anyway).  The dK
// wave works one query tile behind: in iteration t the dV wave forms S, P and P^T dO for
// tile t while the dK wave forms dP, dS and dS^T Q for tile t-1 from the P written in
// iteration t-1.  One barrier per tile instead of two, and each SIMD always holds one wave
// in each kind of phase.  LDS: a three-stage ring of [Q | dO | LSE2 | D] tiles (t-1, t and
// the copy of t+1) and two P buffers.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_lag_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ stats, const uint16_t* __restrict__ dout, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, SeqGeo geo, BlockMask bm, long long stat_stride, long long stat_half, float scale,
    float scale_log2, int BHkv, int Hq, int Hkv, float* __restrict__ part, int nsplit) {
  constexpr int NW = 8, NG = 4, BK = NG * 32, BQ = kBwdBQ, DC = D / 16, DB = D / 32, NQB = BQ / 32;
  using T = BwdTile<D>;
  constexpr int STAGE = (2 * T::BYTES + 2 * BQ * 4 + 1023) / 1024 * 1024;  // Q, dO, LSE2, D
  constexpr int NS = 3;
  constexpr int PGRP = NQB * 2 * 1024;  // one group's P of a tile: [qb][sh][lane] x 16 B
  constexpr int PBYTES = NG * PGRP;
  constexpr int RPC = 1024 / (2 * D), CPTT = T::BYTES / 1024, CPW = 2 * CPTT / NW;
  static_assert(CPTT % NW == 0 || (2 * CPTT) % NW == 0, "tile pieces split over the waves");
  static_assert(NW % (16 / RPC) == 0, "pieces of a wave share their swizzle");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE + 2 * PBYTES];
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseTiles : 1];  // kept (head, query tile) pairs
  static_assert(!SPARSE || BK == kSparseBlock, "a workgroup's keys form one mask block");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  const int grp = wave & (NG - 1), role = wave / NG;
  // MFMA operands from the swizzled LDS tiles of the ring stage this wave reads: per-lane
  // offsets of row block 0 of that stage (the swizzle repeats every 16 rows), other row blocks
  // and the dO tile by constants.  Row-major operand: rows row0 + lane%32, chunk 2c + lane/32;
  // transposed operand: as ld_tr_operand at column db*32.  The offsets move one stage per
  // iteration (loop-carried, so the compiler keeps 16 registers instead of one per operand).
  TileOffsets<D> ofs;
  ofs.init(lane);
  // One workgroup per (batch, KV head, 128 keys).  With grouped-query heads the g query heads
  // sharing the KV head are visited one after the other ([OPT] §5.3 mapping kv = h / g), so
  // dK and dV accumulate the whole group's gradient without atomics.  Split (nsplit = 2, part
  // non-null): two workgroups per key block take half of the group's heads each and write fp32
  // partial sums, which bwd_dkdv_sum_kernel adds.
  const int bkv = blockIdx.x % BHkv, b = bkv / Hkv, hk = bkv - b * Hkv;
  const int kbs = blockIdx.x / BHkv, kblk = kbs / nsplit, half_ = kbs - kblk * nsplit;
  const int g = Hq / Hkv / nsplit, h0 = hk * (Hq / Hkv) + half_ * g;  // this workgroup's first query head
  const SeqRows sr = seq_rows(geo, b, h0, Hq, hk, Hkv);
  const int Nq = sr.lq, Nk = sr.lk, doff = Nk - Nq;  // query i sees keys j <= i + doff (causal)
  // Causal: early key blocks see the most queries and are dispatched first.
  const int k0 = kblk * BK;
  if (k0 >= Nk) return;  // key block past the end of a shorter sequence
  const int kw0 = k0 + grp * 32;
  // Query head h0 + i of the group: rows + i * geo.nq (the head stride of both layouts).
  const uint16_t* qp = q + sr.q * D;
  const uint16_t* kp = k + sr.k * D;
  const uint16_t* vp = v + sr.k * D;
  const uint16_t* dop = dout + sr.q * D;
  // stats = [LSE2 | -D]; LSE2 is the log-sum-exp times log2(e).  Head i of the group: + i*stride.
  const float* lse_b = stats + stat_row(geo, stat_stride, b, h0, Hq);
  const float* dl_b = lse_b + stat_half;
  const int npad = (Nq + BQ - 1) / BQ * BQ;  // statistics rows of one head of this sequence
  const int qt_begin = CAUSAL ? max(k0 - doff, 0) / BQ : 0;
  const int qt_end = (Nq + BQ - 1) / BQ;
  // Virtual tiles vt = 0 .. g*nt - 1: query head vt / nt of the group, tile qt_begin + vt % nt
  // (block-sparse: the kept pairs of the list, in the same order).  The LDS ring slot and the
  // P slot follow vt.
  const int nt = qt_end - qt_begin;
  int nvt = g * nt;
  if constexpr (SPARSE) nvt = nt > 0 ? build_qtile_list(bm, b, h0, g, k0 / kSparseBlock, qt_begin, nt, tlist) : 0;
  auto entry = [&](int i) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane((int)tlist[min(i, nvt - 1)]);
  };
  uint16_t* outp = (role == 0 ? dv : dk) + sr.k * D;
  // Split: fp32 partial of (role, half) at the key's row of [B*Hkv*Nk, D].
  float* partp = part ? part + ((size_t)(role * nsplit + half_) * BHkv * geo.nk + sr.k) * D : nullptr;
  if (nvt <= 0) {  // no query sees these keys: dK = dV = 0
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        if (kr < Nk) {
          if (partp) partp[(size_t)kr * D + db * 32 + l32] = 0.f;
          else outp[(size_t)kr * D + db * 32 + l32] = 0;
        }
      }
    return;
  }

  // Tile copies: wave w copies 1 KB pieces j = w, w + NW, ... of [Q tile | dO tile]; piece j
  // covers tile rows RPC*(j % CPTT) ...; lane l fills physical chunk l, i.e. logical chunk
  // (l%(D/8)) ^ swizzle(row), the same swizzle for all pieces of a wave.  Rows past the last
  // query read the last query (their LSE2 is +inf, so they contribute nothing); waves 0 and 1
  // copy the tile's 64 LSE2 and 64 D values (the padded rows hold +inf and 0).
  const int lrow = lane / (D / 8);
  const uint32_t loff0 =
      lrow * (2 * D) + 16 * ((lane % (D / 8)) ^ ((swz<D>(RPC * wave + lrow, 0) >> 4) & (D / 8 - 1)));
  auto copy_tile = [&](int vt, int h, int t) __attribute__((always_inline)) {
    char* dst = smem + (vt % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int j = wave + NW * i;
      const bool is_q = j < CPTT;
      const int jt = is_q ? j : j - CPTT;
      const int row0 = t * BQ + RPC * jt;
      const uint16_t* base = (is_q ? qp : dop) + (size_t)h * geo.nq * D;
      char* d = dst + (is_q ? 0 : T::BYTES) + 1024 * jt;
      if (row0 + RPC <= Nq) {
        dma16(base, (uint32_t)row0 * (2 * D) + loff0, d);
      } else {
        const int row = min(row0 + lrow, Nq - 1);
        dma16(base, (uint32_t)row * (2 * D) + (loff0 - lrow * (2 * D)), d);
      }
    }
    if (wave < 2)
      dma4((wave == 0 ? lse_b : dl_b) + (size_t)h * stat_stride, 4 * min(t * BQ + lane, npad - 1),
           dst + 2 * T::BYTES + wave * BQ * 4);
  };

  // Branch-free single pieces, for issue between the MFMAs of the interleaved tiles: piece i
  // of this wave, and the statistics (even waves copy LSE2, odd waves D; the copies of one
  // kind write the same bytes).
  const void* qbase = wave_uniform(qp);
  const void* dobase = wave_uniform(dop);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // The piece goes through a buffer resource that starts at its first row, so the per-lane
  // offset is the constant loff0 and rows past the last query arrive as zeros (their LSE2 is
  // +inf and D is 0, so they contribute nothing); the address work is scalar.
  auto copy_piece = [&](int vt, int h, int t, int i) __attribute__((always_inline)) {
    const int j = wv + NW * i;
    const bool is_q = j < CPTT;
    const int jt = is_q ? j : j - CPTT;
    const int first = t * BQ + RPC * jt;
    const uint32_t m0v = lds0 + (vt % NS) * STAGE + (is_q ? 0 : T::BYTES) + 1024 * jt;
    const char* base = reinterpret_cast<const char*>(is_q ? qbase : dobase) + ((size_t)h * geo.nq + first) * (2 * D);
    bdma16_m0(buffer_rsrc(base, (Nq - first) * (2 * D)), loff0, m0v);
  };
  auto copy_stats = [&](int vt, int h, int t) __attribute__((always_inline)) {
    const uint32_t m0v = lds0 + (vt % NS) * STAGE + 2 * T::BYTES + (wv & 1) * BQ * 4;
    const float* base = ((wv & 1) ? dl_b : lse_b) + (size_t)h * stat_stride;
    dma4_m0(wave_uniform(base), 4 * min(t * BQ + lane, npad - 1), m0v);
  };

  int h_cur = 0, t_cur = qt_begin;  // (head, tile) of vt
  if constexpr (SPARSE) {
    const int e = entry(0);
    h_cur = e >> 11;
    t_cur = e & 2047;
  }
  copy_tile(0, h_cur, t_cur);
  // K^T (dV wave) or V^T (dK wave), the B operand of S = Q K^T or dP = dO V^T: lane owns key
  // kw0 + l32.
  const int kj = kw0 + l32;
  const uint16_t* kvp = role == 0 ? kp : vp;
  bf16x8 kreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    u32x4 a = {0u, 0u, 0u, 0u};
    if (kj < Nk) a = ld_global16(kvp + (size_t)kj * D + 16 * c + 8 * h32);
    kreg[c] = as_bf16x8(a);
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  wait_vmem();
  lds_barrier();

  char* pbase = smem + NS * STAGE + grp * PGRP;
  auto rowop = [&](int tofs, int row0, int c) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + ofs.k[c] + (tofs + row0 * (2 * D)));
  };
  auto trop = [&](int tofs, int row0, int db) __attribute__((always_inline)) -> bf16x8 {
    const int o = tofs + row0 * (2 * D);
    return join_tr(ds_read_tr16(smem + ofs.v[db][0] + o), ds_read_tr16(smem + ofs.v[db][1] + o));
  };
  // The dV wave reads the stage of tile vt, the dK wave the stage of tile vt - 1.
  auto ofs_add = [&](int delta) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < DC; ++c) ofs.k[c] += delta;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      ofs.v[db][0] += delta;
      ofs.v[db][1] += delta;
    }
  };
  if (role == 1) ofs_add((NS - 1) * STAGE);
  auto dv_tile_plain = [&](int vt, int t) __attribute__((always_inline)) {
    // dV wave, virtual tile vt (query tile t): S = Q K^T, P = 2^(S scale log2 e - LSE2)
    // (masked), P to LDS, dV += P^T dO.
    const char* qs = smem + (vt % NS) * STAGE;
    const char* dos = qs + T::BYTES;
    const float* ls = reinterpret_cast<const float*>(qs + 2 * T::BYTES);
    char* pw = pbase + (vt & 1) * PBYTES;
    const int q0 = t * BQ;
    f32x16 sv[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[qb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c)
        sv[qb] = mfma32(rowop(0, qb * 32, c), kreg[c], sv[qb]);
    }
    bf16x8 pa[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // Lane owns key kj; register r holds query q0 + 32 qb + 8(r/4) + 4*h32 + r%4.
      // Queries that do not see the key (causal: kj > i + doff) get P = 0.
      const int qb0 = q0 + qb * 32 + doff;
      const bool need_mask = CAUSAL && (qb0 < kw0 + 31);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qb * 32 + 8 * r4 + 4 * h32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * r4 + i;
          float pv = fast_exp2(fmaf(sv[qb][r], scale_log2, -l4[i]));
          if (need_mask && kj > qb0 + 8 * r4 + 4 * h32 + i) pv = 0.f;
          sv[qb][r] = pv;
        }
      }
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        pa[qb][sh] = pack8(sv[qb], sh);
        *reinterpret_cast<bf16x8*>(pw + (qb * 2 + sh) * 1024 + 16 * lane) = pa[qb][sh];
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(pa[qb][sh], trop(T::BYTES, qb * 32 + 16 * sh, db), acc[db]);
  };
  // -D of the 32 queries of block qb in the C layout of dP (register r: query 32 qb + 8(r/4) +
  // 4 h32 + r%4): the dP products accumulate onto it, so dP - D comes out of the matrix core.
  auto neg_d = [&](const float* dls, int qb) __attribute__((always_inline)) -> f32x16 {
    f32x16 x;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dls + qb * 32 + 8 * r4 + 4 * h32);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * r4 + e] = d4[e];
    }
    return x;
  };
  auto dk_tile_plain = [&](int tt) __attribute__((always_inline)) {
    // dK wave, tile t-1: dP = dO V^T, dS = P (dP - D) with P from LDS, dK += dS^T Q.
    const char* qs = smem + (tt % NS) * STAGE;
    const char* dos = qs + T::BYTES;
    const float* dls = reinterpret_cast<const float*>(qs + 2 * T::BYTES) + BQ;
    const char* pr = pbase + (tt & 1) * PBYTES;
    f32x16 dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      dp[qb] = neg_d(dls, qb);
#pragma unroll
      for (int c = 0; c < DC; ++c)
        dp[qb] = mfma32(rowop(T::BYTES, qb * 32, c), kreg[c], dp[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const u32x4 pw = *reinterpret_cast<const u32x4*>(pr + (qb * 2 + sh) * 1024 + 16 * lane);
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
          const int r = 8 * sh + 4 * r4;
          dp[qb][r + 0] = bf16_lo(pw[2 * r4]) * dp[qb][r + 0];
          dp[qb][r + 1] = bf16_hi(pw[2 * r4]) * dp[qb][r + 1];
          dp[qb][r + 2] = bf16_lo(pw[2 * r4 + 1]) * dp[qb][r + 2];
          dp[qb][r + 3] = bf16_hi(pw[2 * r4 + 1]) * dp[qb][r + 3];
        }
      }
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const bf16x8 dsa = pack8(dp[qb], sh);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = mfma32(dsa, trop(0, qb * 32 + 16 * sh, db), acc[db]);
      }
    }
  };
  // Interleaved versions: 32 MFMA slots per tile.  dV wave: S of block 0, then S of block 1
  // while the vector ALU forms P of block 0, then dV of block 0 while it forms P of block 1,
  // then dV of block 1.  The dK wave does the same with dP, dS and dK.  On a diagonal tile the
  // dV wave zeroes the probabilities of queries that do not see its key (causal), so the dK
  // wave, whose dS = P * (dP - D) then vanishes there, needs no mask.
  constexpr int LA = kDkdvLookahead;
  constexpr bool kIlv = D == 128;  // the interleaved slot plan assumes 8 chunks, 4 blocks
  auto dv_tile_ilv = [&](int vt, int t, int cvt, int ch, int ct) __attribute__((always_inline)) {
   if constexpr (kIlv) {  // only instantiated where the slot plan applies
    const int q0 = t * BQ;
    const char* qs = smem + (vt % NS) * STAGE;
    const char* dos = qs + T::BYTES;
    const float* ls = reinterpret_cast<const float*>(qs + 2 * T::BYTES);
    char* pw = pbase + (vt & 1) * PBYTES;
    // Operand j: j < 16: Q rows of block j/8, chunk j%8 (A of S); else dO^T of block
    // (j-16)/8, half ((j-16)/4)%2, features ((j-16)%4)*32 (B of dV).
    auto opnd = [&](auto jc) __attribute__((always_inline)) -> bf16x8 {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 16) {
        return rowop(0, (j / 8) * 32, j % 8);
      } else {
        constexpr int jj = j - 16, qb = jj / 8, sh = (jj / 4) % 2, db = jj % 4;
        return trop(T::BYTES, qb * 32 + 16 * sh, db);
      }
    };
    f32x16 sv[NQB];
    bf16x8 pa[NQB][2];
    bf16x8 buf[LA];
    static_for<LA>([&](auto jc) { buf[decltype(jc)::value] = opnd(jc); });
    sched_fence();
    static_for<32>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < 16) {
        constexpr int qb = i / 8, c = i % 8;
        if constexpr (c == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          sv[qb] = mfma32(buf[i % LA], kreg[0], z);
        } else {
          sv[qb] = mfma32(buf[i % LA], kreg[c], sv[qb]);
        }
      } else {
        constexpr int jj = i - 16, qb = jj / 8, sh = (jj / 4) % 2, db = jj % 4;
        acc[db] = mfma32(pa[qb][sh], buf[i % LA], acc[db]);
      }
      if constexpr (i + LA < 32) buf[i % LA] = opnd(std::integral_constant<int, i + LA>{});
      // P of block (i-8)/8 over slots 8..23, two r4 groups every other slot.
      if constexpr (i >= 8 && i < 24 && i % 2 == 0) {
        constexpr int qb = (i - 8) / 8, r4 = ((i - 8) % 8) / 2;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qb * 32 + 8 * r4 + 4 * h32);
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = fast_exp2(fmaf(sv[qb][4 * r4 + e], scale_log2, -l4[e]));
        // Causal, on a diagonal tile: register 4 r4 + e holds query qb0 + 8 r4 + 4 h32 + e,
        // which sees key kj only if kj <= that query + doff.
        const int qb0 = q0 + qb * 32 + doff;
        if (CAUSAL && qb0 < kw0 + 31) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kj > qb0 + 8 * r4 + 4 * h32 + e) pv[e] = 0.f;
        }
        u32x2 w;
        w[0] = pack_bf16x2(pv[0], pv[1]);
        w[1] = pack_bf16x2(pv[2], pv[3]);
        asm volatile("" : "+v"(w));  // keeps this slot's vector work in place
        u32x4 u = __builtin_bit_cast(u32x4, pa[qb][r4 / 2]);
        u[2 * (r4 % 2)] = w[0];
        u[2 * (r4 % 2) + 1] = w[1];
        pa[qb][r4 / 2] = as_bf16x8(u);
        if constexpr (r4 % 2 == 1) *reinterpret_cast<bf16x8*>(pw + (qb * 2 + r4 / 2) * 1024 + 16 * lane) = pa[qb][r4 / 2];
      }
      if constexpr (i % 3 == 1 && i / 3 < CPW) copy_piece(cvt, ch, ct, i / 3);
      if constexpr (i == 3 * CPW + 1) copy_stats(cvt, ch, ct);
      sched_fence();
    });
   }
  };

  auto dk_tile_ilv = [&](int tt, int cvt, int ch, int ct) __attribute__((always_inline)) {
   if constexpr (kIlv) {  // only instantiated where the slot plan applies
    const char* qs = smem + (tt % NS) * STAGE;
    const char* dos = qs + T::BYTES;
    const float* dls = reinterpret_cast<const float*>(qs + 2 * T::BYTES) + BQ;
    const char* pr = pbase + (tt & 1) * PBYTES;
    auto opnd = [&](auto jc) __attribute__((always_inline)) -> bf16x8 {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 16) {
        return rowop(T::BYTES, (j / 8) * 32, j % 8);
      } else {
        constexpr int jj = j - 16, qb = jj / 8, sh = (jj / 4) % 2, db = jj % 4;
        return trop(0, qb * 32 + 16 * sh, db);
      }
    };
    f32x16 dp[NQB];
    bf16x8 dsa[NQB][2];
    bf16x8 buf[LA];
    dp[0] = neg_d(dls, 0);
    static_for<LA>([&](auto jc) { buf[decltype(jc)::value] = opnd(jc); });
    sched_fence();
    static_for<32>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i == 3) dp[1] = neg_d(dls, 1);  // read ahead of its first product (slot 8)
      if constexpr (i < 16) {
        constexpr int qb = i / 8, c = i % 8;
        dp[qb] = mfma32(buf[i % LA], kreg[c], dp[qb]);
      } else {
        constexpr int jj = i - 16, qb = jj / 8, sh = (jj / 4) % 2, db = jj % 4;
        acc[db] = mfma32(dsa[qb][sh], buf[i % LA], acc[db]);
      }
      if constexpr (i + LA < 32) buf[i % LA] = opnd(std::integral_constant<int, i + LA>{});
      // dS of block (i-8)/8 over slots 8..23: half sh every fourth slot.
      if constexpr (i >= 8 && i < 24 && i % 4 == 0) {
        constexpr int qb = (i - 8) / 8, sh = ((i - 8) % 8) / 4;
        const u32x4 pw = *reinterpret_cast<const u32x4*>(pr + (qb * 2 + sh) * 1024 + 16 * lane);
        u32x4 u;
#pragma unroll
        for (int r4 = 0; r4 < 2; ++r4) {
          const int r = 8 * sh + 4 * r4;
          const float e0 = bf16_lo(pw[2 * r4]) * dp[qb][r + 0];
          const float e1 = bf16_hi(pw[2 * r4]) * dp[qb][r + 1];
          const float e2 = bf16_lo(pw[2 * r4 + 1]) * dp[qb][r + 2];
          const float e3 = bf16_hi(pw[2 * r4 + 1]) * dp[qb][r + 3];
          u[2 * r4] = pack_bf16x2(e0, e1);
          u[2 * r4 + 1] = pack_bf16x2(e2, e3);
        }
        asm volatile("" : "+v"(u));  // keeps this slot's vector work in place
        dsa[qb][sh] = as_bf16x8(u);
      }
      if constexpr (i % 3 == 1 && i / 3 < CPW) copy_piece(cvt, ch, ct, i / 3);
      if constexpr (i == 3 * CPW + 1) copy_stats(cvt, ch, ct);
      sched_fence();
    });
   }
  };

  // Virtual tile vt+1 is copied during iteration vt: one piece every third MFMA of the first
  // half of an interleaved tile, else up front.  Past the end the last
  // head's tile qt_end is copied, its rows and statistics clamped to the last ones, into the
  // stage nobody reads in this iteration.
  int h_nxt = nt == 1 ? 1 : 0, t_nxt = nt == 1 ? qt_begin : qt_begin + 1;  // of vt + 1
  int h_end = g - 1, t_end = qt_end;  // copied past the end (clamped rows, an idle stage)
  if constexpr (SPARSE) {
    const int e = entry(1), l = entry(nvt - 1);
    h_nxt = e >> 11;
    t_nxt = e & 2047;
    h_end = l >> 11;
    t_end = l & 2047;
  }
  for (int vt = 0; vt <= nvt; ++vt) {
    const bool more = vt + 1 < nvt;
    const int ch = more ? h_nxt : h_end, ct = more ? t_nxt : t_end;
    const bool ilv_dv = kIlv && role == 0 && vt < nvt;
    const bool ilv_dk = kIlv && role == 1 && vt > 0;
    if (!(ilv_dv || ilv_dk) && more) copy_tile(vt + 1, h_nxt, t_nxt);
    if (role == 0) {
      if (vt < nvt) {
        if (ilv_dv) dv_tile_ilv(vt, t_cur, vt + 1, ch, ct);
        else dv_tile_plain(vt, t_cur);
      }
    } else if (vt > 0) {
      if (ilv_dk) dk_tile_ilv(vt - 1, vt + 1, ch, ct);
      else dk_tile_plain(vt - 1);
    }
    if (more) wait_vmem();  // virtual tile vt+1 has landed
    lds_barrier();
    ofs_add(((role == 0 ? vt : vt + NS - 1) % NS) == NS - 1 ? -(NS - 1) * STAGE : STAGE);
    h_cur = h_nxt;
    t_cur = t_nxt;
    if constexpr (SPARSE) {
      const int e = entry(vt + 2);
      h_nxt = e >> 11;
      t_nxt = e & 2047;
    } else if (++t_nxt == qt_end) {
      t_nxt = qt_begin;
      ++h_nxt;
    }
  }

  // C layout: lane holds feature db*32 + l32 of keys kw0 + 8(r/4) + 4*h32 + r%4.
  const float oscale = role == 0 ? 1.f : scale;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      if (kr < Nk) {
        if (partp) partp[(size_t)kr * D + db * 32 + l32] = acc[db][r] * oscale;
        else outp[(size_t)kr * D + db * 32 + l32] = (uint16_t)(pack_bf16x2(acc[db][r] * oscale, 0.f) & 0xffffu);
      }
    }
}

// Split dK/dV: out = bf16(partial of the first half + partial of the second half), four
// elements per thread; n4 = B*Hkv*N*d/4 per tensor, grid over both tensors (dV, then dK).
__global__ __launch_bounds__(256) void bwd_dkdv_sum_kernel(const float* __restrict__ part, uint16_t* __restrict__ dv,
                                                           uint16_t* __restrict__ dk, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const int role = i >= n4;
  const long long j = i - role * n4;
  const f32x4 a = reinterpret_cast<const f32x4*>(part + (size_t)(2 * role) * n4 * 4)[j];
  const f32x4 c = reinterpret_cast<const f32x4*>(part + (size_t)(2 * role + 1) * n4 * 4)[j];
  u32x2 w;
  w[0] = pack_bf16x2(a[0] + c[0], a[1] + c[1]);
  w[1] = pack_bf16x2(a[2] + c[2], a[3] + c[3]);
  reinterpret_cast<u32x2*>(role ? dk : dv)[j] = w;
}

// ------------------------------------------------------------------ dQ
// Slot of vector group g (0..3) within an interleaved phase of L MFMA slots.
constexpr int dq_vslot(int L, int g) { return 1 + g * (L - 2) / 3; }

// Also forms the per-row statistics the dK/dV kernel reads (it runs first): LSE2 = LSE*log2(e)
// and -D for its 128 rows (negated: the dK/dV kernel starts its dP accumulators from it, so that
// the products give dP - D directly), padding rows up to the sequence's multiple of 64 getting
// +inf and 0.
//
// D.  dS = P (dP - D) takes D = rowsum(dO * O), known before the key walk, but O is stored in
// bf16 and that D carries O's rounding, up to 2^-9 relative.  On the key that dominates a row
// dP - D nearly cancels, and there the rounding moves dQ_i by about scale * dD_i * sum_j P_ij K_j,
// as large as dQ_i itself once the row's largest probability nears 1 (relative error about
// 2^-9 / sqrt(1 - P_max)).  Each wave therefore notes the largest probability it meets (one
// v_max3 per two) and flags itself when that exceeds 1/2.  A second launch (REDO) exits at once
// in workgroups without a flagged wave; in the others it forms D from its definition,
// sum_j P_ij dP_ij (fp32), in a walk that computes only S and dP, writes it for the dK/dV kernel
// (launched after both), and walks the key tiles once more, last first (the last two are still
// in LDS), for dQ with that D.  On N(0,1) inputs only the first rows of a causal sequence (few
// keys) trigger it; rows whose keys all fit one or two tiles get the exact D in the first
// launch.  The redo launch takes light (early) query tiles first, where that work sits.
template <int D, bool CAUSAL, bool SPARSE, bool REDO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o, const float* __restrict__ lse, float* __restrict__ stats,
    const uint16_t* __restrict__ dout, uint16_t* __restrict__ dq, SeqGeo geo, BlockMask bm, long long stat_stride,
    long long stat_half, float scale, float scale_log2, int n_qtiles, int BH, int Hq, int Hkv,
    unsigned* __restrict__ flags) {
  constexpr int NW = 4, BM = NW * 32, BN = kBwdBK, KB = BN / 32, DC = D / 16, DB = D / 32;
  static_assert(!SPARSE || BM == kSparseBlock, "a workgroup's queries form one mask block");
  using T = BwdTile<D>;
  constexpr int STAGE = 2 * T::BYTES;  // K, V
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseTiles : 1];  // kept key tiles (block-sparse)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  const int bh = blockIdx.x % BH;
  const int t_ = blockIdx.x / BH;
  // Causal: the first launch takes heavy (late) query tiles first; the redo launch, whose work
  // sits in the first query tiles of a sequence, takes them first.
  const int qt = (CAUSAL && !REDO) ? (n_qtiles - 1 - t_) : t_;
  const size_t fl = 4 * ((size_t)qt * BH + bh);  // this workgroup's flag words (one per wave)
  const int q0 = qt * BM, qw0 = q0 + wave * 32, qi = qw0 + l32;
  // K/V of the query head's KV head (grouped-query: kv = h / (Hq/Hkv)).
  const int b = bh / Hq, hq = bh - b * Hq, hk = hq / (Hq / Hkv);
  const SeqRows sr = seq_rows(geo, b, hq, Hq, hk, Hkv);
  const int Nq = sr.lq, Nk = sr.lk;
  if (q0 >= Nq) return;  // query tile past the end of a shorter sequence
  if constexpr (REDO) {  // one flag word per wave of the first launch
    const u32x4 f = *reinterpret_cast<const u32x4*>(flags + fl);
    if (__builtin_amdgcn_readfirstlane(f[0] | f[1] | f[2] | f[3]) == 0) return;
  }
  const int qd0 = qw0 + (Nk - Nq), kmax = qi + (Nk - Nq);  // causal: query i sees keys <= i + Nk - Nq
  const uint16_t* qp = q + sr.q * D;
  const uint16_t* kp = k + sr.k * D;
  const uint16_t* vp = v + sr.k * D;
  const uint16_t* dop = dout + sr.q * D;

  bf16x8 qreg[DC], doreg[DC];
  float dsum = 0.f;  // this lane's half of rowsum(dO * O)
  const uint16_t* op = o + sr.q * D;
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u}, w = {0u, 0u, 0u, 0u};
    if (qi < Nq) {
      a = ld_global16(qp + (size_t)qi * D + 16 * c + 8 * h32);
      g = ld_global16(dop + (size_t)qi * D + 16 * c + 8 * h32);
      if constexpr (!REDO) w = ld_global16(op + (size_t)qi * D + 16 * c + 8 * h32);
    }
    qreg[c] = as_bf16x8(a);
    doreg[c] = as_bf16x8(g);
#pragma unroll
    for (int e = 0; e < 4; ++e) dsum += bf16_lo(g[e]) * bf16_lo(w[e]) + bf16_hi(g[e]) * bf16_hi(w[e]);
  }
  // Statistics of row qi: LSE2 = LSE*log2(e) and D = rowsum(dO * O) (the other half of the
  // row's features sits in lane qi + 32).  Rows past the sequence up to its multiple of 64 are
  // padding (+inf, 0) so that the dK/dV kernel's 64-row tile copies need no bounds check.
  const float dtot = sum_xor32(dsum);
  float* st = stats + stat_row(geo, stat_stride, b, hq, Hq);
  float dl = qi < Nq ? dtot : 0.f;  // D_O = rowsum(dO * O); the redo launch forms the exact D
  const float lse2 = qi < Nq ? lse[sr.q + qi] * kLog2e : INFINITY;
  if (!REDO && h32 == 0 && qi < (Nq + 63) / 64 * 64) {
    st[qi] = lse2;
    st[stat_half + qi] = -dl;
  }

  f32x16 dq_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.f;

  const int kv_end = CAUSAL ? min(Nk, q0 + BM + (Nk - Nq)) : Nk;
  int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // Block-sparse: walk only the key tiles the workgroup's query block keeps (position t holds
  // key tile kt(t)); dropped blocks hold no score, so no further masking is needed.
  if constexpr (SPARSE) ntiles = build_tile_list<1>(bm, b, hq, q0 / kSparseBlock, ntiles, tlist);
  auto kt = [&](int t) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return __builtin_amdgcn_readfirstlane((int)tlist[min(t, ntiles - 1)]) & 0x3fff;
    else return t;
  };
  // K/V tiles arrive by direct global -> LDS copies (no staging registers, which lets two
  // workgroups share a CU).  Wave w copies 1 KB pieces j = w, w + NW, ... of [K tile | V
  // tile]; piece j covers tile rows RPC*(j % CPTT) ...; lane l fills physical chunk l, i.e.
  // logical chunk (l%(D/8)) ^ swizzle(row).  The swizzle depends on the row modulo 16 only,
  // which is the same for all pieces of a wave.  Rows past the last key read the last key
  // (masked below).
  constexpr int RPC = 1024 / (2 * D), CPTT = T::BYTES / 1024, CPW = 2 * CPTT / NW;
  static_assert(CPTT % NW == 0 && NW % (16 / RPC) == 0, "pieces of a wave share their swizzle");
  const int lrow = lane / (D / 8);
  const uint32_t loff0 =
      lrow * (2 * D) + 16 * ((lane % (D / 8)) ^ ((swz<D>(RPC * wave + lrow, 0) >> 4) & (D / 8 - 1)));
  auto copy_tile = [&](int t, int stage) __attribute__((always_inline)) {
    char* dst = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int j = wave + NW * i;
      const bool is_k = j < CPTT;
      const int jt = is_k ? j : j - CPTT;
      const int row0 = t * BN + RPC * jt;
      const uint16_t* base = is_k ? kp : vp;
      char* d = dst + (is_k ? 0 : T::BYTES) + 1024 * jt;
      if (row0 + RPC <= Nk) {
        dma16(base, (uint32_t)row0 * (2 * D) + loff0, d);
      } else {
        const int row = min(row0 + lrow, Nk - 1);
        dma16(base, (uint32_t)row * (2 * D) + (loff0 - lrow * (2 * D)), d);
      }
    }
  };

  // Branch-free single pieces of tile t, issued between the MFMAs of the first key blocks so
  // that the workgroups' copies do not all queue at the tile start.
  const void* kbase = wave_uniform(kp);
  const void* vbase = wave_uniform(vp);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // Through a buffer resource that starts at the piece's first row: constant per-lane offset
  // loff0, rows past the last key read as zeros (masked), scalar address work.
  auto copy_piece = [&](int t, int ktile, int i) __attribute__((always_inline)) {
    const int j = wv + NW * i;
    const bool is_k = j < CPTT;
    const int jt = is_k ? j : j - CPTT;
    const int first = ktile * BN + RPC * jt;
    const uint32_t m0v = lds0 + (t & 1) * STAGE + (is_k ? 0 : T::BYTES) + 1024 * jt;
    const char* base = reinterpret_cast<const char*>(is_k ? kbase : vbase) + (size_t)first * (2 * D);
    bdma16_m0(buffer_rsrc(base, (Nk - first) * (2 * D)), loff0, m0v);
  };

  uint16_t* dqp = dq + sr.q * D;
  // Workgroups whose rows' keys fit two tiles form the exact D in this launch, so the redo
  // launch skips them: at d = 64 through the two-walk path below, at d = 128 through a walk for D
  // ahead of the main walk (the two-walk path in this launch cost the d = 128 main walk two
  // register reloads per tile).
  const bool two_walk = REDO || (D == 64 && ntiles == 2);
  if (!REDO && lane == 0 && ntiles <= 2) flags[fl + wave] = 0u;
  if (ntiles == 0) {  // no key for any row of the tile: dQ = 0
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = qw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        if (qq < Nq) dqp[(size_t)qq * D + db * 32 + l32] = 0;
      }
    return;
  }
  copy_tile(kt(0), 0);
  wait_vmem();  // also covers the Q/dO loads
  lds_barrier();
  // Tile t+1 is copied during tile t (past the end: rows clamped, into the idle stage).
  // Interleaved tile: the MFMAs of one 64-key tile run in fixed slots and the vector work of
  // each key block sits between the MFMAs that do not depend on it.  Slot phases (one MFMA
  // per slot, DC = D/16 slots for a score block, 2*DB for a dQ block):
  //   A: S_0 = K_0 Q^T          B: dP_0 = V_0 dO^T    || P_0 = 2^(S_0 scale log2 e - LSE2)
  //   C: S_1                    || dS_0 = P_0 (dP_0 - D), packed to bf16
  //   D: dP_1                   || P_1
  //   E: dQ += dS_0 K_0         || dS_1
  //   F: dQ += dS_1 K_1
  // Masked keys (causal, or past the last key) get P = 0 in a uniform branch taken only by
  // blocks that hold such a key.  Per accumulator the products are summed in the same order
  // as block by block, so the result does not depend on this schedule.  The next tile's copy
  // pieces go out on the odd slots of phases A and B; LDS operands are read LA slots ahead.
  constexpr int LA = kDqLookahead;
  constexpr int PA = 0, PB = DC, PC = 2 * DC, PD = 3 * DC, PE = 4 * DC, PF = 4 * DC + 2 * DB, NSLOT = 4 * DC + 4 * DB;
  static_assert(CPW <= DC, "copy pieces fit the odd slots of phases A and B");
  static_assert((STAGE & (STAGE - 1)) == 0 && STAGE >= 2 * T::BYTES, "stage toggled by XOR");
  TileOffsets<D> ofs;  // operand offsets of the current stage (toggled per tile)
  ofs.init(lane);
  // Operand j of a tile: [A | B | C | D] row-major K or V chunks, [E | F] K^T of block 0 / 1.
  auto opnd = [&](auto jc) __attribute__((always_inline)) -> bf16x8 {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < PE) {
      constexpr int ph = j / DC, c = j % DC, kb = ph / 2, isv = ph % 2;
      return *reinterpret_cast<const bf16x8*>(smem + ofs.k[c] + (isv * T::BYTES + kb * 32 * 2 * D));
    } else {
      constexpr int jj = j - PE, kb = jj / (2 * DB), sh = (jj % (2 * DB)) / DB, db = jj % DB;
      constexpr int roff = (kb * 32 + 16 * sh) * 2 * D;
      return join_tr(ds_read_tr16(smem + ofs.v[db][0] + roff), ds_read_tr16(smem + ofs.v[db][1] + roff));
    }
  };
  // S (as P, masked) and dP of key block kb of the tile at key t0, from the current stage.
  auto tile_sdp = [&](auto kc, int t0, f32x16& sv, f32x16& dpv) __attribute__((always_inline)) {
    constexpr int kb = decltype(kc)::value;
    static_for<DC>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      const bf16x8 ak = opnd(std::integral_constant<int, (2 * kb) * DC + c>{});
      const bf16x8 av = opnd(std::integral_constant<int, (2 * kb + 1) * DC + c>{});
      if constexpr (c == 0) {
        sv = mfma32(ak, qreg[0], f32x16{});
        dpv = mfma32(av, doreg[0], f32x16{});
      } else {
        sv = mfma32(ak, qreg[c], sv);
        dpv = mfma32(av, doreg[c], dpv);
      }
    });
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kj = t0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      const float pr = fast_exp2(fmaf(sv[r], scale_log2, -lse2));
      sv[r] = (kj >= Nk || (CAUSAL && kj > kmax)) ? 0.f : pr;
    }
  };
  // d = 128, rows whose keys fit two tiles: D from its definition in a walk over the two tiles
  // (S and dP only) before the main walk, which then takes that D; both tiles stay in the two
  // stages, so the main walk starts on tile 0 as usual.
  bool exact_d = false;
  if constexpr (!REDO && D == 128) {
    if (ntiles == 2) {
      float dpart = 0.f;
      for (int t = 0; t < 2; ++t) {
        const int t0 = kt(t) * BN;
        if (t == 0) copy_tile(kt(1), 1);
        if (!(CAUSAL && t0 > qd0 + 31)) {
          static_for<2>([&](auto kc) {
            f32x16 sv, dpv;
            tile_sdp(kc, t0, sv, dpv);
#pragma unroll
            for (int r = 0; r < 16; ++r) dpart = fmaf(sv[r], dpv[r], dpart);
          });
        }
        wait_vmem();
        lds_barrier();
        ofs.toggle(STAGE);
      }
      dl = qi < Nq ? sum_xor32(dpart) : 0.f;
      if (h32 == 0 && qi < Nq) st[stat_half + qi] = -dl;
      exact_d = true;
    }
  }
  if (two_walk) {
    // D_i = sum_j P_ij dP_ij over the rows' keys, from S and dP alone (tile t+1 copied during
    // tile t), then dQ with it, walking the tiles last first: the last two are still in the two
    // stages, and tile t-2 is copied into the stage of tile t during tile t-1.
    float dpart = 0.f;
    for (int t = 0; t < ntiles; ++t) {
      const int t0 = kt(t) * BN;
      if (t + 1 < ntiles) copy_tile(kt(t + 1), (t + 1) & 1);
      if (!(CAUSAL && t0 > qd0 + 31)) {
        static_for<2>([&](auto kc) {
          f32x16 sv, dpv;
          tile_sdp(kc, t0, sv, dpv);
#pragma unroll
          for (int r = 0; r < 16; ++r) dpart = fmaf(sv[r], dpv[r], dpart);
        });
      }
      wait_vmem();
      lds_barrier();
      if (t + 1 < ntiles) ofs.toggle(STAGE);
    }
    dl = qi < Nq ? sum_xor32(dpart) : 0.f;
    if (h32 == 0 && qi < Nq) st[stat_half + qi] = -dl;
    // ofs is on the stage of tile ntiles-1 and tile ntiles-2 is still in the other stage.  At
    // tile t <= ntiles-2 the stage of tile t+1 is free again and takes tile t-1.
    for (int t = ntiles - 1; t >= 0; --t) {
      const int t0 = kt(t) * BN;
      if (t <= ntiles - 2 && t >= 1) copy_tile(kt(t - 1), (t - 1) & 1);
      if (!(CAUSAL && t0 > qd0 + 31)) {
        bf16x8 dsv[2][2];
        static_for<2>([&](auto kc) {
          constexpr int kb = decltype(kc)::value;
          f32x16 sv, dpv;
          tile_sdp(kc, t0, sv, dpv);
#pragma unroll
          for (int r = 0; r < 16; ++r) dpv[r] = sv[r] * (dpv[r] - dl);
          dsv[kb][0] = pack8(dpv, 0);
          dsv[kb][1] = pack8(dpv, 1);
        });
        static_for<4 * DB>([&](auto jc) {
          constexpr int jj = decltype(jc)::value, kb = jj / (2 * DB), sh = (jj % (2 * DB)) / DB, db = jj % DB;
          dq_acc[db] = mfma32(dsv[kb][sh], opnd(std::integral_constant<int, PE + jj>{}), dq_acc[db]);
        });
      }
      wait_vmem();  // tile t-1 has landed
      lds_barrier();
      ofs.toggle(STAGE);
    }
  } else
  if (ntiles == 1) {
    // The tile's keys are all the keys of these rows: D = sum_j P_ij dP_ij, its definition,
    // replaces rowsum(dO * O) here and in the statistics the dK/dV kernel reads.  O is stored in
    // bf16 and D inherits its rounding; on rows dominated by one key dP - D nearly cancels, and
    // on such short rows that rounding alone moved dQ and dK by up to a few percent.
    const int t0 = kt(0) * BN;
    f32x16 sv[2], dpv[2];
    static_for<2>([&](auto kc) {
      constexpr int kb = decltype(kc)::value;
      static_for<DC>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const bf16x8 ak = opnd(std::integral_constant<int, (2 * kb) * DC + c>{});
        const bf16x8 av = opnd(std::integral_constant<int, (2 * kb + 1) * DC + c>{});
        if constexpr (c == 0) {
          sv[kb] = mfma32(ak, qreg[0], f32x16{});
          dpv[kb] = mfma32(av, doreg[0], f32x16{});
        } else {
          sv[kb] = mfma32(ak, qreg[c], sv[kb]);
          dpv[kb] = mfma32(av, doreg[c], dpv[kb]);
        }
      });
    });
    float dpart = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = t0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        float pr = fast_exp2(fmaf(sv[kb][r], scale_log2, -lse2));
        if (kj >= Nk || (CAUSAL && kj > kmax)) pr = 0.f;
        sv[kb][r] = pr;
        dpart += pr * dpv[kb][r];
      }
    const float dex = sum_xor32(dpart);
    if (h32 == 0 && qi < Nq) st[stat_half + qi] = -dex;
    bf16x8 dsv[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dpv[kb][r] = sv[kb][r] * (dpv[kb][r] - dex);
      dsv[kb][0] = pack8(dpv[kb], 0);
      dsv[kb][1] = pack8(dpv[kb], 1);
    }
    static_for<4 * DB>([&](auto jc) {
      constexpr int jj = decltype(jc)::value, kb = jj / (2 * DB), sh = (jj % (2 * DB)) / DB, db = jj % DB;
      dq_acc[db] = mfma32(dsv[kb][sh], opnd(std::integral_constant<int, PE + jj>{}), dq_acc[db]);
    });
  } else {
  float pmx = 0.f;  // largest probability this lane meets (first launch)
  // The dP accumulators start from -D (every element of a lane belongs to its query row), so
  // the matrix cores return dP - D and dS = P (dP - D) is one multiply per element: 32 vector
  // subtractions fewer per tile for 16 registers held across the walk (1.3% off the kernel).
  f32x16 ndl;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndl[r] = -dl;
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = kt(t) * BN, kn = kt(t + 1);
    if (CAUSAL && t0 > qd0 + 31) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) copy_piece(t + 1, kn, i);
    } else {
      f32x16 s0, dp0, s1, dp1;
      bf16x8 ds0[2], ds1[2];
      bf16x8 buf[LA];
      static_for<LA>([&](auto jc) { buf[decltype(jc)::value] = opnd(jc); });
      // Keys of block kb for this lane: t0 + 32 kb + 8(r/4) + 4*h32 + r%4.
      auto mask_block = [&](f32x16& p, int kb) __attribute__((always_inline)) {
        const int kb0 = t0 + kb * 32;
        if ((kb0 + 32 > Nk) || (CAUSAL && kb0 + 31 > qd0)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = kb0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            if (kj >= Nk || (CAUSAL && kj > kmax)) p[r] = 0.f;
          }
        }
      };
      auto exp_group = [&](f32x16& x, int g) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * g + e] = fast_exp2(fmaf(x[4 * g + e], scale_log2, -lse2));
        asm volatile("" : "+v"(x[4 * g]), "+v"(x[4 * g + 1]), "+v"(x[4 * g + 2]), "+v"(x[4 * g + 3]));
      };
      auto ds_group = [&](const f32x16& p, f32x16& dp, bf16x8 (&ds)[2], int g) __attribute__((always_inline)) {
        if constexpr (!REDO) pmx = fmaxf(fmaxf(pmx, p[4 * g]), fmaxf(fmaxf(p[4 * g + 1], p[4 * g + 2]), p[4 * g + 3]));
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * g + e] = p[4 * g + e] * dp[4 * g + e];  // dp holds dP - D
        if (g % 2 == 1) {
          ds[g / 2] = pack8(dp, g / 2);
          asm volatile("" : "+v"(ds[g / 2]));
        }
      };
      sched_fence();
      static_for<NSLOT>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        // Uniform mask branches before the first vector work that reads P of a block.
        if constexpr (i == PC) { sched_fence(); mask_block(s0, 0); sched_fence(); }
        if constexpr (i == PE) { sched_fence(); mask_block(s1, 1); sched_fence(); }
        if constexpr (i < PB) {
          if constexpr (i == PA) { s0 = mfma32(buf[i % LA], qreg[0], f32x16{}); }
          else s0 = mfma32(buf[i % LA], qreg[i - PA], s0);
        } else if constexpr (i < PC) {
          if constexpr (i == PB) dp0 = mfma32(buf[i % LA], doreg[0], ndl);
          else dp0 = mfma32(buf[i % LA], doreg[i - PB], dp0);
        } else if constexpr (i < PD) {
          if constexpr (i == PC) s1 = mfma32(buf[i % LA], qreg[0], f32x16{});
          else s1 = mfma32(buf[i % LA], qreg[i - PC], s1);
        } else if constexpr (i < PE) {
          if constexpr (i == PD) dp1 = mfma32(buf[i % LA], doreg[0], ndl);
          else dp1 = mfma32(buf[i % LA], doreg[i - PD], dp1);
        } else if constexpr (i < PF) {
          constexpr int jj = i - PE, sh = jj / DB, db = jj % DB;
          dq_acc[db] = mfma32(ds0[sh], buf[i % LA], dq_acc[db]);
        } else {
          constexpr int jj = i - PF, sh = jj / DB, db = jj % DB;
          dq_acc[db] = mfma32(ds1[sh], buf[i % LA], dq_acc[db]);
        }
        if constexpr (i + LA < NSLOT) buf[i % LA] = opnd(std::integral_constant<int, i + LA>{});
        static_for<4>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          if constexpr (i == PB + dq_vslot(DC, g)) exp_group(s0, g);
          if constexpr (i == PC + dq_vslot(DC, g)) ds_group(s0, dp0, ds0, g);
          if constexpr (i == PD + dq_vslot(DC, g)) exp_group(s1, g);
          if constexpr (i == PE + dq_vslot(2 * DB, g)) ds_group(s1, dp1, ds1, g);
        });
        if constexpr (i % 2 == 1 && i / 2 < CPW) copy_piece(t + 1, kn, i / 2);
        sched_fence();
      });
    }
    ofs.toggle(STAGE);
    wait_vmem();  // tile t+1 has landed
    lds_barrier();
  }
  if constexpr (!REDO) {
    // The wave's flag for the redo launch (rows past the sequence have P = 0, so a flagged
    // lane holds a real row).
    const bool dom = __builtin_amdgcn_ballot_w64(pmx > 0.5f) != 0;
    if (lane == 0 && !exact_d) flags[fl + wave] = dom ? 1u : 0u;
  }
  }
  // C layout: lane holds feature db*32 + l32 of queries qw0 + 8(r/4) + 4*h32 + r%4.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = qw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      if (qq < Nq) dqp[(size_t)qq * D + db * 32 + l32] = (uint16_t)(pack_bf16x2(dq_acc[db][r] * scale, 0.f) & 0xffffu);
    }
}

// ------------------------------------------------------------------ host launcher
template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  const int BH = a.B * a.Hq, BHkv = a.B * a.Hkv;
  const float sl2 = a.scale * kLog2e;
  const SeqGeo geo{a.cu_q, a.cu_k, a.Nq, a.Nk};
  const BlockMask bm{a.block_mask, a.mask_sb, a.mask_sh, (a.Nq + kSparseBlock - 1) / kSparseBlock,
                     (a.Nk + kSparseBlock - 1) / kSparseBlock};
  // dQ first: it also writes the row statistics the dK/dV kernel reads.
  const int n_qt = (a.max_q + 127) / 128;
  if (n_qt > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, SPARSE, false>), dim3(n_qt * BH), dim3(256), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.o, a.lse,
                       a.stats, (const uint16_t*)a.dout, (uint16_t*)a.dq, geo, bm, a.stat_stride, a.stat_half, a.scale,
                       sl2, n_qt, BH, a.Hq, a.Hkv, a.flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Workgroups that met a probability above 1/2 walk again for dQ with the exact D; the
    // others exit at once.
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, SPARSE, true>), dim3(n_qt * BH), dim3(256), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.o, a.lse,
                       a.stats, (const uint16_t*)a.dout, (uint16_t*)a.dq, geo, bm, a.stat_stride, a.stat_half, a.scale,
                       sl2, n_qt, BH, a.Hq, a.Hkv, a.flags);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_kt = (a.max_k + 127) / 128;
  if (n_kt > 0) {
    // The caller hands over the partial buffer only where the split applies (dense causal
    // grouped-query heads, even group size, fewer than kBwdSplitGrid workgroups).
    const bool split = CAUSAL && a.part != nullptr && a.cu_q == nullptr && bwd_split_possible(a.B, a.Hq, a.Hkv, a.Nk) &&
                       a.Nq == a.Nk;
    const int nsplit = split ? 2 : 1;
    hipLaunchKernelGGL((bwd_dkdv_lag_kernel<D, CAUSAL, SPARSE>), dim3(n_kt * nsplit * BHkv), dim3(512), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const float*)a.stats,
                       (const uint16_t*)a.dout, (uint16_t*)a.dk, (uint16_t*)a.dv, geo, bm, a.stat_stride,
                       a.stat_half, a.scale, sl2, BHkv, a.Hq, a.Hkv, split ? a.part : nullptr, nsplit);
    if (split) {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const long long n4 = (long long)BHkv * a.Nk * D / 4;
      hipLaunchKernelGGL(bwd_dkdv_sum_kernel, dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0, a.stream,
                         (const float*)a.part, (uint16_t*)a.dv, (uint16_t*)a.dk, n4);
    }
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  if (a.block_mask) return a.causal ? launch_bwd_t<D, true, true>(a) : launch_bwd_t<D, false, true>(a);
  return a.causal ? launch_bwd_t<D, true, false>(a) : launch_bwd_t<D, false, false>(a);
}

hipError_t launch_bwd(const BwdArgs& a) { return a.d == 128 ? launch_bwd_d<128>(a) : launch_bwd_d<64>(a); }

}  // namespace xattn

// Single-token grouped-query decode for gfx950: split-KV partials, then an LSE merge.
//
// Pages cited by title:
//   [OPT]  "FlashAttention optimisation: breaking the attention memory bottleneck"
//   [FUND] "Attention fundamentals: the standard attention flow, complexity analysis,
//          memory bottleneck and inference challenges"
//
// Decode reads the whole KV cache once per token and does O(L d) work ([OPT] §4.2.2,
// [FUND] §2.3.1), so the kernel is bound by HBM bandwidth, not by arithmetic.  Design:
//   * One workgroup per (batch, KV head, key chunk).  All g = Hq/Hkv query heads that share
//     the KV head ([OPT] §5.3) are processed together, so every K/V byte is read from HBM
//     exactly once and used g times.
//   * Scores: v_mfma_f32_16x16x32_bf16 with the K rows as the A operand straight from
//     global memory (16-byte loads) and the g query vectors as the B operand (columns
//     g..15 zero).  In the C layout lane (16*j + h) holds head h's scores for keys 4j..4j+3
//     of the 16-key block.
//   * P V on the vector ALU: lane (16*j + c) owns features [c*D/16, (c+1)*D/16) of keys
//     4j + r; the probability p[h][key] sits in lane 16*j + h of the same 16-lane row and
//     is broadcast with a DPP row_newbcast move.  V rows are read with coalesced 16-byte
//     loads (D = 128) and no LDS staging.  K and V loads carry the nontemporal hint: the cache
//     is read once per token, and streaming it past the caches reads HBM faster.
//   * Online softmax per 32-key chunk ([OPT] §3.2.1); the four row groups of a wave and the
//     four waves of a workgroup share one running max per head, so only the final
//     cross-wave combine needs LDS.
//   * Each chunk writes (O_s normalised, lse_s); the merge kernel combines the chunks with
//     weights 2^(lse_s - max) — exact by the order independence of [OPT] §3.2.2.
//   * Sequences of their own lengths: the workgroups share the 32-key blocks of all groups
//     equally (stream-K), so long and short sequences load the chip evenly; a workgroup may
//     write partials of several groups, and decode_merge_sk_kernel gathers them.
//   * Multi-token decode: T new tokens per sequence; the MFMA rows are the T x g (token,
//     head) pairs of the group, so the cache is still read once per group.  With the causal
//     mask aligned at the bottom right, token t sees keys j <= len - T + t.  Up to 8 rows the
//     kernel below runs (P V on the vector ALU); from 9 to 32 rows decode_mma_kernel, whose
//     P V runs on the matrix cores.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace xattn {

constexpr int kDecWaves = 4;
constexpr float kDecLazy = 8.f;
// 32-key blocks of a sequence of len keys (clamped to [0, L]).
__device__ __forceinline__ int dec_blocks(int len, int L) { return (min(max(len, 0), L) + 31) >> 5; }

template <int D, int GP, bool SK>
__global__ __launch_bounds__(kDecWaves * 64) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    float* __restrict__ part_o, float* __restrict__ part_lse, int B, int Hq, int Hkv, int L,
    int splits, int keys_per_split, float scale_log2, const int* __restrict__ seqlens, int T, int causal) {
  constexpr int EPL = D / 16;  // features per lane in the P V product
  constexpr int DC = D / 32;   // 32-wide feature chunks of the score MFMA
  __shared__ float s_m[kDecWaves][GP];
  __shared__ float s_l[kDecWaves][GP];
  __shared__ float s_acc[kDecWaves][GP][D];
  __shared__ int s_pre[SK ? kDecSkMaxB + 1 : 1];  // stream-K: 32-key blocks of sequences < b
  __shared__ int s_scan[SK ? kDecWaves * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = Hq / Hkv, R = T * g;  // MFMA row r < R: token r / g of head kvh*g + r % g
  // One key range [kbeg, kend) of group (b, kv head kvh): the rows' partial (O normalised,
  // base-2 LSE) goes to partial row prow(h, tok) of MFMA row h.
  auto chunk = [&](int b, int kvh, int len, int kbeg, int kend, auto prow) __attribute__((always_inline)) {
    const size_t bk = (size_t)b * Hkv + kvh;
    const uint16_t* kp = kc + bk * L * D;
    const uint16_t* vp = vc + bk * L * D;

    // Causal: the last key row col's token sees (rows past R see every key; they are never
    // written).
    const int ctok = col / g;
    const int klast = (causal && col < R) ? len - T + ctok : L;
    bf16x8 qB[DC];
  #pragma unroll
    for (int c = 0; c < DC; ++c) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (col < R)
        u = ld_global16(q + ((size_t)(b * Hq + kvh * g + col - ctok * g) * T + ctok) * D + 32 * c + 8 * grp);
      qB[c] = as_bf16x8(u);
    }

    // The running max starts finite (kMaxInit), so rows whose keys a chunk masks entirely get
    // probability 0 there, and a row without any key ends with l = 0.
    float m_run = kMaxInit, l_run = 0.f;
    float acc[GP][EPL];
  #pragma unroll
    for (int h = 0; h < GP; ++h)
  #pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

    const int nchunks = (kend - kbeg + 31) / 32;
    for (int ci = wave; ci < nchunks; ci += kDecWaves) {
      const int k0 = kbeg + ci * 32;
      // Issue this chunk's K and V loads together (V is consumed after the softmax), so each
      // wave keeps 2 x 8 KB in flight.
      u32x4 kraw[2][DC];
      using VRaw = typename std::conditional<EPL == 8, u32x4, u32x2>::type;
      VRaw vraw[2][4];
  #pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int key = k0 + blk * 16 + col;
  #pragma unroll
        for (int c = 0; c < DC; ++c) {
          u32x4 u = {0u, 0u, 0u, 0u};
          if (key < kend) u = ld_global_nt<u32x4>(kp + (size_t)key * D + 32 * c + 8 * grp);
          kraw[blk][c] = u;
        }
      }
  #pragma unroll
      for (int blk = 0; blk < 2; ++blk)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + blk * 16 + 4 * grp + r;
          VRaw u = {};
          if (key < kend) u = ld_global_nt<VRaw>(vp + (size_t)key * D + EPL * col);
          vraw[blk][r] = u;
        }
      f32x4 sc[2];
  #pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int c = 0; c < DC; ++c) sc[blk] = mfma16(as_bf16x8(kraw[blk][c]), qB[c], sc[blk]);
      }
      // Lane (16*grp + col): head col, keys k0 + 16*blk + 4*grp + r.
      float mx = -INFINITY;
  #pragma unroll
      for (int blk = 0; blk < 2; ++blk)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + blk * 16 + 4 * grp + r;
          if (key >= kend || key > klast) sc[blk][r] = -INFINITY;
          mx = fmaxf(mx, sc[blk][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx *= scale_log2;
      // Lazy reference max (as in the forward kernel): move m_run and rescale only when some
      // head's chunk max exceeds it by more than 2^kDecLazy; the result is unchanged.
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kDecLazy) != 0) {
        const float m_new = fmaxf(m_run, mx);  // finite: m_run starts at kMaxInit
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        static_for<GP>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const float a_h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
  #pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= a_h;
        });
      }
      float rs = 0.f;
  #pragma unroll
      for (int blk = 0; blk < 2; ++blk)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(sc[blk][r], scale_log2, -m_run));
          sc[blk][r] = p;
          rs += p;
        }
      l_run += rs;
  #pragma unroll
      for (int blk = 0; blk < 2; ++blk)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          float vf[EPL];
  #pragma unroll
          for (int e = 0; e < EPL / 2; ++e) { vf[2 * e] = bf16_lo(vraw[blk][r][e]); vf[2 * e + 1] = bf16_hi(vraw[blk][r][e]); }
          const float pr = sc[blk][r];
          static_for<GP>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const float p_h = row_bcast<h>(pr);
  #pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p_h, vf[e], acc[h][e]);
          });
        }
    }

    // Combine the four row groups of the wave (they share m_run), then the four waves.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
  #pragma unroll
    for (int h = 0; h < GP; ++h)
  #pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = acc[h][e] + __shfl_xor(acc[h][e], 16);
        acc[h][e] = x + __shfl_xor(x, 32);
      }
    if (grp == 0) {
  #pragma unroll
      for (int h = 0; h < GP; ++h)
  #pragma unroll
        for (int e = 0; e < EPL; ++e) s_acc[wave][h][EPL * col + e] = acc[h][e];
    }
    if (lane < GP) {
      s_m[wave][lane] = m_run;
      s_l[wave][lane] = l_tot;
    }
    __syncthreads();
    for (int i = tid; i < R * D; i += kDecWaves * 64) {
      const int h = i / D, d = i - h * D;  // MFMA row h: token h / g, head kvh*g + h % g
      float M = kMaxInit;
  #pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, s_m[w][h]);
      float num = 0.f, den = 0.f;
  #pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float wt = fast_exp2(s_m[w][h] - M);  // a wave that saw no key has l = 0
        num = fmaf(wt, s_acc[w][h][d], num);
        den = fmaf(wt, s_l[w][h], den);
      }
      const int tok = h / g;
      const size_t row = prow(h, tok);
      // A chunk holding no key of this row: partial O = 0, lse = -inf (weight 0 in the merge).
      const bool empty = !(den > 0.f);
      part_o[row * D + d] = empty ? 0.f : num / den;
      if (d == 0) part_lse[row] = empty ? -INFINITY : M + fast_log2(den);
    }
  };

  if constexpr (!SK) {
    // Workgroup (b*Hkv + kv head, key chunk split), the group fastest: workgroups go to the
    // XCDs in turn, so each XCD gets every split of its groups, short and long alike when the
    // sequences have their own lengths (with the split fastest and two splits, four XCDs got
    // every full first chunk and the other four only the partial second ones; 4-7% faster on
    // lengths uniform in [L/2, L], no change with equal lengths).
    const int BK = B * Hkv;
    const int split = blockIdx.x / BK;
    const int bk = blockIdx.x - split * BK;  // b * Hkv + kv head
    const int b = bk / Hkv, kvh = bk - b * Hkv;
    // Sequence b attends to the first len keys of its cache (all L without seqlens).
    const int len = seqlens != nullptr ? min(max(seqlens[b], 0), L) : L;
    const int kbeg = split * keys_per_split;
    const int kend = max(kbeg, min(len, kbeg + keys_per_split));
    chunk(b, kvh, len, kbeg, kend, [&](int h, int tok) {
      return ((size_t)(split * B + b) * Hq + kvh * g + h - tok * g) * T + tok;
    });
  } else {
    // Stream-K split for sequences of their own lengths: the 32-key blocks of all groups, in
    // (b, kv head) order, are cut into gridDim.x equal ranges, so every workgroup reads the
    // same number of blocks whatever the lengths.  Workgroup w takes blocks
    // [w NB / G, (w+1) NB / G) and writes one partial per group it meets, to slot w + k
    // (k = b*Hkv + kv head; unique, since along the blocks neither w nor k decreases), rows
    // slot * R + h.  decode_merge_sk_kernel finds a group's workgroups from the same sums.
    static_assert(kDecWaves * 64 == 256, "four values per lane in the scan of wave 0");
    constexpr int NT = kDecWaves * 64;
    const int per = (B + NT - 1) / NT;  // sequences per thread (B <= kDecSkMaxB)
    int loc = 0;
    for (int i = 0; i < per; ++i) {
      const int bb = tid * per + i;
      if (bb < B) loc += dec_blocks(seqlens[bb], L);
    }
    s_scan[tid] = loc;
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of the 256 per-thread counts
      const int v0 = s_scan[4 * lane], v1 = s_scan[4 * lane + 1], v2 = s_scan[4 * lane + 2], v3 = s_scan[4 * lane + 3];
      const int sum = v0 + v1 + v2 + v3;
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int ex = incl - sum;
      s_scan[4 * lane] = ex;
      s_scan[4 * lane + 1] = ex + v0;
      s_scan[4 * lane + 2] = ex + v0 + v1;
      s_scan[4 * lane + 3] = ex + v0 + v1 + v2;
    }
    __syncthreads();
    int run = s_scan[tid];
    for (int i = 0; i < per; ++i) {
      const int bb = tid * per + i;
      if (bb < B) {
        s_pre[bb] = run;
        run += dec_blocks(seqlens[bb], L);
      }
    }
    if (tid == NT - 1) s_pre[B] = run;  // the total (the last thread's range ends at or past B)
    __syncthreads();
    const long long NB = (long long)Hkv * s_pre[B], G = gridDim.x, w = blockIdx.x;
    const long long lo = w * NB / G, hi = (w + 1) * NB / G;
    if (lo < hi) {
      // The sequence holding block lo: the largest b with Hkv * s_pre[b] <= lo (it has blocks).
      int b = 0;
      for (int top = B - 1; b < top;) {
        const int m = (b + top + 1) >> 1;
        if ((long long)Hkv * s_pre[m] <= lo) b = m;
        else top = m - 1;
      }
      int nb = s_pre[b + 1] - s_pre[b];
      int kvh = (int)((lo - (long long)Hkv * s_pre[b]) / nb);
      long long S = (long long)Hkv * s_pre[b] + (long long)kvh * nb;  // first block of the group
      while (S < hi) {
        const long long x0 = S > lo ? S : lo, x1 = S + nb < hi ? S + nb : hi;
        const int len = min(max(seqlens[b], 0), L);
        const int kbeg = (int)(x0 - S) * 32, kend = min(len, (int)(x1 - S) * 32);
        const size_t slot = (size_t)w + (size_t)b * Hkv + kvh;
        chunk(b, kvh, len, kbeg, kend, [&](int h, int) { return slot * R + h; });
        __syncthreads();  // the next group's combine reuses s_m, s_l and s_acc
        if (++kvh == Hkv) {
          kvh = 0;
          do { ++b; } while (b < B && s_pre[b + 1] == s_pre[b]);
          if (b >= B) break;
          nb = s_pre[b + 1] - s_pre[b];
        }
        S = (long long)Hkv * s_pre[b] + (long long)kvh * nb;
      }
    }
  }
}

// Decode with (token, head) rows of a KV head on the matrix cores, 32 per workgroup, as the
// forward computes a 32-row block: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K rows straight from
// global memory as the A operand, the rows' Q^T resident as the B operand), so that in the C
// layout each lane owns one row and 16 keys; the probabilities are then already the B operand
// of O^T += V^T P^T, whose V^T operand is read with the transposing ds_read_b64_tr_b16 from a
// per-wave double-buffered LDS copy of the 32-key V block (direct global -> LDS, swizzled as
// the forward's tiles).  Each of the four waves walks every fourth 32-key block of the
// workgroup's chunk and writes its own partial (O_w, lse_w): the merge kernel combines
// 4 x splits partials, exactly as it combines chunks.  More than 32 rows take several
// workgroups, each reading the cache once.
template <int D>
__global__ __launch_bounds__(kDecWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    float* __restrict__ part_o, float* __restrict__ part_lse, int B, int Hq, int Hkv, int L,
    int splits, int keys_per_split, float scale_log2, const int* __restrict__ seqlens, int T, int causal) {
  constexpr int DC = D / 16, DB = D / 32;
  constexpr int VBYTES = 32 * D * 2;      // one 32-key V block
  constexpr int NCP = VBYTES / 1024;      // 1 KB copies per block
  constexpr int RPC = 1024 / (2 * D);     // rows per 1 KB copy
  __shared__ __attribute__((aligned(1024))) char vbuf[kDecWaves * 2 * VBYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  const int g = Hq / Hkv, R = T * g, nrc = (R + 31) / 32;
  // Workgroup (b*Hkv + kv head, 32-row chunk rc of the group's R rows, key chunk split); the
  // split fastest (the group-fastest order of decode_split_kernel measured 3% slower on the
  // multi-token workload with equal lengths).
  const int split = blockIdx.x % splits;
  const int rc = (blockIdx.x / splits) % nrc;
  const int bk = blockIdx.x / (splits * nrc);  // b * Hkv + kv head
  const int b = bk / Hkv, kvh = bk - b * Hkv;
  const int len = seqlens != nullptr ? min(max(seqlens[b], 0), L) : L;
  const int kbeg = split * keys_per_split;
  const int kend = max(kbeg, min(len, kbeg + keys_per_split));
  const uint16_t* kp = kc + (size_t)bk * L * D;
  const uint16_t* vp = vc + (size_t)bk * L * D;

  // Row r = 32 rc + l32: token r / g of head kvh*g + r % g.  Q^T operand: features 16c +
  // 8*h32 .. +7.
  const int row_r = 32 * rc + l32;
  const int tok = row_r / g, hh = row_r - tok * g;
  const bool row_ok = row_r < R;
  const int klast = (causal && row_ok) ? len - T + tok : 0x7fffffff;  // last key of the row
  bf16x8 qreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (row_ok) u = ld_global16(q + ((size_t)(b * Hq + kvh * g + hh) * T + tok) * D + 16 * c + 8 * h32);
    qreg[c] = as_bf16x8(u);
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = kMaxInit, l_run = 0.f;

  // V copies: 1 KB piece j of a block covers rows RPC*j ..; lane l fills physical chunk l,
  // i.e. it reads logical chunk (l%(D/8)) ^ swizzle(row).  Rows past kend read row kend-1
  // (finite data; their probabilities are 0).
  const int lrow = lane / (D / 8);
  const void* vbase = wave_uniform(vp);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)vbuf;
  const uint32_t wdst = lds0 + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * (2 * VBYTES);
  const int nblk = (kend - kbeg + 31) / 32;
  auto issue = [&](int blk, int stage, bf16x8 (&kop)[DC]) __attribute__((always_inline)) {
    const int k0 = kbeg + 32 * blk;
    const int key = min(k0 + l32, kend - 1);
#pragma unroll
    for (int c = 0; c < DC; ++c) kop[c] = as_bf16x8(ld_global16(kp + (size_t)key * D + 16 * c + 8 * h32));
#pragma unroll
    for (int j = 0; j < NCP; ++j) {
      const int r = RPC * j + lrow;
      const int row = min(k0 + r, kend - 1);
      const uint32_t off = (uint32_t)row * (2 * D) + 16 * ((lane % (D / 8)) ^ ((swz<D>(r, 0) >> 4) & (D / 8 - 1)));
      dma16_m0(vbase, off, wdst + stage * VBYTES + 1024 * j);
    }
  };
  // Block blk uses stage st and K operands kcur; the next block of this wave (blk + 4) is
  // issued into the other stage and knxt first.  Two calls per loop trip keep the register
  // sets static.
  auto step = [&](int blk, int st, bf16x8 (&kcur)[DC], bf16x8 (&knxt)[DC]) __attribute__((always_inline)) {
    if (blk + kDecWaves < nblk) {
      issue(blk + kDecWaves, st ^ 1, knxt);
      wait_vmem_n<DC + NCP>();
    } else {
      wait_vmem();
    }
    const int k0 = kbeg + 32 * blk;
    f32x16 sv;
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = 0.f;
#pragma unroll
    for (int c = 0; c < DC; ++c) sv = mfma32(kcur[c], qreg[c], sv);
    // Lane owns row l32; register r holds key k0 + 8(r/4) + 4*h32 + r%4.
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      if (key >= kend || key > klast) sv[r] = -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = max_xor32(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kDecLazy) != 0) {  // lazy reference max
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = fast_exp2(fmaf(sv[r], scale_log2, -m_run));
      rs += sv[r];
    }
    l_run += rs;
    const char* vs = vbuf + (wave * 2 + st) * VBYTES;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      u32x4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(sv[8 * sh + 2 * e], sv[8 * sh + 2 * e + 1]);
      const bf16x8 pb = as_bf16x8(u);
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32(ld_tr_operand<D>(vs, 16 * sh, db * 32, lane), pb, acc[db]);
    }
  };
  bf16x8 kA[DC], kB[DC];
  if (wave < nblk) issue(wave, 0, kA);
  for (int blk = wave; blk < nblk; blk += 2 * kDecWaves) {
    step(blk, 0, kA, kB);
    if (blk + kDecWaves < nblk) step(blk + kDecWaves, 1, kB, kA);
  }

  // Partial of this wave: rows r < R, O^T C layout (lane l32 = row, register r = feature
  // db*32 + 8(r/4) + 4*h32 + r%4).  A row that saw no key writes O = 0, lse = -inf.
  const float lt = sum_xor32(l_run);
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.f / lt;
  if (row_ok) {
    const size_t row = ((size_t)((split * kDecWaves + wave) * B + b) * Hq + kvh * g + hh) * T + tok;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) part_o[row * D + db * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3)] = acc[db][r] * inv;
    if (h32 == 0) part_lse[row] = empty ? -INFINITY : m_run + fast_log2(lt);
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, uint16_t* __restrict__ o,
    float* __restrict__ lse, int BHq, int splits) {
  const int row = blockIdx.x, d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_lse[(size_t)s * BHq + row]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float ls = part_lse[(size_t)s * BHq + row];
    const float w = ls == -INFINITY ? 0.f : fast_exp2(ls - M);
    num = fmaf(w, part_o[((size_t)s * BHq + row) * D + d], num);
    den += w;
  }
  // No key at all (a zero-length sequence): O = 0 and LSE = -inf, the empty sum's log.
  const bool empty = M == -INFINITY;
  const float val = empty ? 0.f : num / den;
  const uint32_t packed = pack_bf16x2(val, 0.f);
  o[(size_t)row * D + d] = (uint16_t)(packed & 0xffffu);
  if (lse != nullptr && d == 0) lse[row] = empty ? -INFINITY : (M + fast_log2(den)) * kLn2;
}

// Merge of the stream-K partials (decode_split_kernel with SK): row (b, head, token) of group
// k = b*Hkv + kv head gathers the partials of the workgroups whose block range meets the
// group's blocks [S, E), from slot w + k, with the prefix sums the split kernel used.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_sk_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, uint16_t* __restrict__ o,
    float* __restrict__ lse, const int* __restrict__ seqlens, int B, int Hq, int Hkv, int T, int L, int G) {
  __shared__ int s_red[2][D / 64];
  const int row = blockIdx.x, d = threadIdx.x, lane = d & 63, wv = d >> 6;
  const int tok = row % T, bh = row / T, b = bh / Hq, head = bh - b * Hq;
  const int g = Hq / Hkv, kvh = head / g, R = T * g, h = tok * g + head - kvh * g;
  int before = 0, total = 0;
  for (int i = d; i < B; i += D) {
    const int n = dec_blocks(seqlens[i], L);
    total += n;
    if (i < b) before += n;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off);
    total += __shfl_xor(total, off);
  }
  if (lane == 0) {
    s_red[0][wv] = before;
    s_red[1][wv] = total;
  }
  __syncthreads();
  before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    before += s_red[0][i];
    total += s_red[1][i];
  }
  const int nb = dec_blocks(seqlens[b], L);
  const long long NB = (long long)Hkv * total, S = (long long)Hkv * before + (long long)kvh * nb, E = S + nb;
  const long long k = (long long)b * Hkv + kvh;
  // Workgroup holding block x: the largest w with w NB / G <= x, i.e. ((x + 1) G - 1) / NB.
  const long long wf = nb > 0 ? ((S + 1) * G - 1) / NB : 0, wl = nb > 0 ? (E * G - 1) / NB : -1;
  auto meets = [&](long long w) {  // workgroup w's range meets [S, E) (an empty range meets nothing)
    const long long lo = w * NB / G, hi = (w + 1) * NB / G;
    return (lo > S ? lo : S) < (hi < E ? hi : E);
  };
  float M = -INFINITY;
  for (long long w = wf; w <= wl; ++w)
    if (meets(w)) M = fmaxf(M, part_lse[(size_t)(w + k) * R + h]);
  float num = 0.f, den = 0.f;
  for (long long w = wf; w <= wl; ++w) {
    if (!meets(w)) continue;
    const size_t pr = (size_t)(w + k) * R + h;
    const float ls = part_lse[pr];
    const float wt = ls == -INFINITY ? 0.f : fast_exp2(ls - M);
    num = fmaf(wt, part_o[pr * D + d], num);
    den += wt;
  }
  const bool empty = M == -INFINITY;
  const float val = empty ? 0.f : num / den;
  const uint32_t packed = pack_bf16x2(val, 0.f);
  o[(size_t)row * D + d] = (uint16_t)(packed & 0xffffu);
  if (lse != nullptr && d == 0) lse[row] = empty ? -INFINITY : (M + fast_log2(den)) * kLn2;
}

template <int D, int GP>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const float sl2 = a.scale * kLog2e;
  const int G = a.B * a.Hkv * a.splits;
  if (decode_stream_k(a.seqlens != nullptr, a.B, a.Hkv, a.L)) {
    hipLaunchKernelGGL((decode_split_kernel<D, GP, true>), dim3(G), dim3(kDecWaves * 64), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.part_o, a.part_lse, a.B,
                       a.Hq, a.Hkv, a.L, a.splits, a.keys_per_split, sl2, a.seqlens, a.T, a.causal);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_sk_kernel<D>), dim3(a.B * a.Hq * a.T), dim3(D), 0, a.stream, a.part_o,
                       a.part_lse, (uint16_t*)a.o, a.lse, a.seqlens, a.B, a.Hq, a.Hkv, a.T, a.L, G);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_split_kernel<D, GP, false>), dim3(G), dim3(kDecWaves * 64), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.part_o,
                     a.part_lse, a.B, a.Hq, a.Hkv, a.L, a.splits, a.keys_per_split, sl2, a.seqlens, a.T, a.causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.B * a.Hq * a.T), dim3(D), 0, a.stream, a.part_o, a.part_lse,
                     (uint16_t*)a.o, a.lse, a.B * a.Hq * a.T, a.splits);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_mma(const DecodeArgs& a) {
  const float sl2 = a.scale * kLog2e;
  const int nrc = (a.T * (a.Hq / a.Hkv) + 31) / 32;  // 32-row chunks per KV head
  hipLaunchKernelGGL((decode_mma_kernel<D>), dim3(a.B * a.Hkv * nrc * a.splits), dim3(kDecWaves * 64), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.part_o, a.part_lse, a.B,
                     a.Hq, a.Hkv, a.L, a.splits, a.keys_per_split, sl2, a.seqlens, a.T, a.causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.B * a.Hq * a.T), dim3(D), 0, a.stream, a.part_o, a.part_lse,
                     (uint16_t*)a.o, a.lse, a.B * a.Hq * a.T, a.splits * kDecWaves);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  const int g = a.T * (a.Hq / a.Hkv);  // MFMA rows per group
  if (decode_uses_mma(a.T, a.Hq / a.Hkv)) return launch_decode_mma<D>(a);
  if (g <= 1) return launch_decode_t<D, 1>(a);
  if (g <= 2) return launch_decode_t<D, 2>(a);
  if (g <= 4) return launch_decode_t<D, 4>(a);
  if (g <= 8) return launch_decode_t<D, 8>(a);
  return launch_decode_t<D, 16>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.d == 128 ? launch_decode_d<128>(a) : launch_decode_d<64>(a);
}

}  // namespace xattn

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
//     loads (D = 128) and no LDS staging.
//   * Online softmax per 32-key chunk ([OPT] §3.2.1); the four row groups of a wave and the
//     four waves of a workgroup share one running max per head, so only the final
//     cross-wave combine needs LDS.
//   * Each chunk writes (O_s normalised, lse_s); the merge kernel combines the chunks with
//     weights 2^(lse_s - max) — exact by the order independence of [OPT] §3.2.2.
//   * Multi-token decode: T new tokens per sequence; the MFMA rows are the T x g (token,
//     head) pairs of the group (at most 16), so the cache is still read once per group.  With
//     the causal mask aligned at the bottom right, token t sees keys j <= len - T + t.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace xattn {

constexpr int kDecWaves = 4;
constexpr float kDecLazy = 8.f;

template <int D, int GP>
__global__ __launch_bounds__(kDecWaves * 64) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    float* __restrict__ part_o, float* __restrict__ part_lse, int B, int Hq, int Hkv, int L,
    int splits, int keys_per_split, float scale_log2, const int* __restrict__ seqlens, int T, int causal) {
  constexpr int EPL = D / 16;  // features per lane in the P V product
  constexpr int DC = D / 32;   // 32-wide feature chunks of the score MFMA
  __shared__ float s_m[kDecWaves][GP];
  __shared__ float s_l[kDecWaves][GP];
  __shared__ float s_acc[kDecWaves][GP][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int g = Hq / Hkv, R = T * g;  // MFMA row r < R: token r / g of head kvh*g + r % g
  const int split = blockIdx.x % splits;
  const int bk = blockIdx.x / splits;  // b * Hkv + kv head
  const int b = bk / Hkv, kvh = bk - b * Hkv;
  // Sequence b attends to the first len keys of its cache (all L without seqlens).
  const int len = seqlens != nullptr ? min(max(seqlens[b], 0), L) : L;
  const int kbeg = split * keys_per_split;
  const int kend = max(kbeg, min(len, kbeg + keys_per_split));
  const uint16_t* kp = kc + (size_t)bk * L * D;
  const uint16_t* vp = vc + (size_t)bk * L * D;

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
        if (key < kend) u = ld_global16(kp + (size_t)key * D + 32 * c + 8 * grp);
        kraw[blk][c] = u;
      }
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + blk * 16 + 4 * grp + r;
        VRaw u = {};
        if (key < kend) u = *reinterpret_cast<const VRaw*>(vp + (size_t)key * D + EPL * col);
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
    const size_t row = ((size_t)(split * B + b) * Hq + kvh * g + h - tok * g) * T + tok;
    // A chunk holding no key of this row: partial O = 0, lse = -inf (weight 0 in the merge).
    const bool empty = !(den > 0.f);
    part_o[row * D + d] = empty ? 0.f : num / den;
    if (d == 0) part_lse[row] = empty ? -INFINITY : M + fast_log2(den);
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

template <int D, int GP>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((decode_split_kernel<D, GP>), dim3(a.B * a.Hkv * a.splits), dim3(kDecWaves * 64), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.part_o,
                     a.part_lse, a.B, a.Hq, a.Hkv, a.L, a.splits, a.keys_per_split, sl2, a.seqlens, a.T, a.causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.B * a.Hq * a.T), dim3(D), 0, a.stream, a.part_o, a.part_lse,
                     (uint16_t*)a.o, a.lse, a.B * a.Hq * a.T, a.splits);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  const int g = a.T * (a.Hq / a.Hkv);  // MFMA rows per group
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

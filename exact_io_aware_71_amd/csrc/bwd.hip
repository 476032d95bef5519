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
// Three launches, deterministic (no atomics):
//   1. bwd_delta_kernel: D = rowsum(dO * O) (HBM-bound streaming pass).
//   2. bwd_dkdv_kernel: one workgroup per 128 keys; each wave keeps its 32 keys' K and V
//      rows in registers (B operands of S = Q K^T and dP = dO V^T) and the dK, dV
//      accumulators in registers while Q/dO tiles of 64 queries stream through a double-
//      buffered LDS.  In the C layout of S each lane owns one key, so P and dS are already
//      the A operand of dV = P^T dO and dK = dS^T Q; dO and Q enter those products through
//      the transposing ds_read_b64_tr_b16.  Causal: query tiles before the diagonal are
//      never visited.
//   3. bwd_dq_kernel: one workgroup per 128 queries; S^T = K Q^T and dP^T = V dO^T with
//      Q and dO resident in registers, K/V tiles streamed through LDS; dS^T in the C layout
//      is the A operand of dQ = dS K, K entering through the transposing read.
#include "common.h"
#include "launch.h"

namespace xattn {

// ------------------------------------------------------------------ D = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, int rows) {
  constexpr int LPR = D / 8;             // lanes per row, 8 features each
  constexpr int RPB = 256 / LPR;         // rows per block
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / LPR;
  const int c = tid % LPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = ld_global16(o + (size_t)row * D + 8 * c);
    const u32x4 g = ld_global16(dout + (size_t)row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf16_lo(a[e]) * bf16_lo(g[e]) + bf16_hi(a[e]) * bf16_hi(g[e]);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && c == 0) delta[row] = s;
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ delta, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, float scale, float scale_log2,
    int n_ktiles, int BH) {
  constexpr int NW = 4, BK = NW * 32, BQ = kBwdBQ, DC = D / 16, DB = D / 32;
  constexpr int CPT = BQ * D / 8 / (NW * 64);
  using T = BwdTile<D>;
  constexpr int STAGE = 2 * T::BYTES + 2 * BQ * 4;  // Q, dO, lse2, delta
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  const int bh = blockIdx.x % BH;
  // Causal: early key tiles see the most queries and are dispatched first.
  const int ktile = blockIdx.x / BH;
  const int k0 = ktile * BK;
  const int kw0 = k0 + wave * 32;
  const uint16_t* qp = q + (size_t)bh * N * D;
  const uint16_t* kp = k + (size_t)bh * N * D;
  const uint16_t* vp = v + (size_t)bh * N * D;
  const uint16_t* dop = dout + (size_t)bh * N * D;
  const float* lsep = lse + (size_t)bh * N;
  const float* dlp = delta + (size_t)bh * N;

  // K^T and V^T operands (B of S = Q K^T, dP = dO V^T): lane owns key kw0 + l32.
  bf16x8 kreg[DC], vreg[DC];
  {
    const int kj = kw0 + l32;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      u32x4 a = {0u, 0u, 0u, 0u}, bb = {0u, 0u, 0u, 0u};
      if (kj < N) {
        a = ld_global16(kp + (size_t)kj * D + 16 * c + 8 * h32);
        bb = ld_global16(vp + (size_t)kj * D + 16 * c + 8 * h32);
      }
      kreg[c] = as_bf16x8(a);
      vreg[c] = as_bf16x8(bb);
    }
  }
  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk_acc[db][r] = 0.f; dv_acc[db][r] = 0.f; }

  const int qt_begin = CAUSAL ? (k0 / BQ) : 0;
  const int qt_end = (N + BQ - 1) / BQ;

  u32x4 pq[CPT], pdo[CPT];
  float plse = 0.f, pdl = 0.f;
  auto load_tile = [&](int t) {
    const int q0 = t * BQ;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NW * 64;
      const int row = c / (D / 8), col = c % (D / 8), qi = q0 + row;
      u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
      if (qi < N) {
        a = ld_global16(qp + (size_t)qi * D + col * 8);
        g = ld_global16(dop + (size_t)qi * D + col * 8);
      }
      pq[i] = a;
      pdo[i] = g;
    }
    if (tid < BQ) {
      const int qi = q0 + tid;
      // Rows past N get lse = +inf so that their probabilities vanish.
      plse = qi < N ? lsep[qi] * kLog2e : INFINITY;
      pdl = qi < N ? dlp[qi] : 0.f;
    }
  };
  auto store_tile = [&](int stage) {
    char* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NW * 64;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<u32x4*>(base + swz<D>(row, col)) = pq[i];
      *reinterpret_cast<u32x4*>(base + T::BYTES + swz<D>(row, col)) = pdo[i];
    }
    if (tid < BQ) {
      reinterpret_cast<float*>(base + 2 * T::BYTES)[tid] = plse;
      reinterpret_cast<float*>(base + 2 * T::BYTES + BQ * 4)[tid] = pdl;
    }
  };

  if (qt_begin < qt_end) {
    load_tile(qt_begin);
    store_tile(0);
  }
  __syncthreads();
  for (int t = qt_begin; t < qt_end; ++t) {
    const int st = (t - qt_begin) & 1;
    if (t + 1 < qt_end) load_tile(t + 1);
    const char* qs = smem + st * STAGE;
    const char* dos = qs + T::BYTES;
    const float* ls = reinterpret_cast<const float*>(qs + 2 * T::BYTES);
    const float* dls = ls + BQ;
    const int q0 = t * BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qb0 = q0 + qb * 32;
      // Causal: a query block entirely before this wave's keys contributes nothing.
      if (CAUSAL && qb0 + 31 < kw0) continue;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const int off = swz<D>(qb * 32 + l32, 2 * c + h32);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qs + off);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dos + off);
        s = mfma32(aq, kreg[c], s);
        dp = mfma32(ad, vreg[c], dp);
      }
      // Lane owns key kw0 + l32; register r holds query qb0 + 8(r/4) + 4*h32 + r%4.
      const int kj = kw0 + l32;
      const bool need_mask = CAUSAL && (qb0 < kw0 + 31);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qoff = qb * 32 + 8 * r4 + 4 * h32;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qoff);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dls + qoff);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * r4 + i;
          float p = fast_exp2(fmaf(s[r], scale_log2, -l4[i]));
          if (need_mask && kj > qb0 + 8 * r4 + 4 * h32 + i) p = 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - d4[i]);
        }
      }
      // dV += P^T dO ; dK += dS^T Q  (contraction over the 32 queries, 16 per MFMA).
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const bf16x8 pa = pack8(s, sh);
        const bf16x8 dsa = pack8(dp, sh);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 bdo = ld_tr_operand<D>(dos, qb * 32 + 16 * sh, db * 32, lane);
          const bf16x8 bq = ld_tr_operand<D>(qs, qb * 32 + 16 * sh, db * 32, lane);
          dv_acc[db] = mfma32(pa, bdo, dv_acc[db]);
          dk_acc[db] = mfma32(dsa, bq, dk_acc[db]);
        }
      }
    }
    if (t + 1 < qt_end) store_tile(st ^ 1);
    __syncthreads();
  }

  // C layout: lane holds feature db*32 + l32 of keys kw0 + 8(r/4) + 4*h32 + r%4.
  uint16_t* dkp = dk + (size_t)bh * N * D;
  uint16_t* dvp = dv + (size_t)bh * N * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kj = kw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      if (kj < N) {
        const size_t off = (size_t)kj * D + db * 32 + l32;
        dkp[off] = (uint16_t)(pack_bf16x2(dk_acc[db][r] * scale, 0.f) & 0xffffu);
        dvp[off] = (uint16_t)(pack_bf16x2(dv_acc[db][r], 0.f) & 0xffffu);
      }
    }
}

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ delta, const uint16_t* __restrict__ dout,
    uint16_t* __restrict__ dq, int N, float scale, float scale_log2, int n_qtiles, int BH) {
  constexpr int NW = 4, BM = NW * 32, BN = kBwdBK, KB = BN / 32, DC = D / 16, DB = D / 32;
  constexpr int CPT = BN * D / 8 / (NW * 64);
  using T = BwdTile<D>;
  constexpr int STAGE = 2 * T::BYTES;  // K, V
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  const int bh = blockIdx.x % BH;
  const int t_ = blockIdx.x / BH;
  const int qt = CAUSAL ? (n_qtiles - 1 - t_) : t_;
  const int q0 = qt * BM, qw0 = q0 + wave * 32, qi = qw0 + l32;
  const uint16_t* qp = q + (size_t)bh * N * D;
  const uint16_t* kp = k + (size_t)bh * N * D;
  const uint16_t* vp = v + (size_t)bh * N * D;
  const uint16_t* dop = dout + (size_t)bh * N * D;

  bf16x8 qreg[DC], doreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    u32x4 a = {0u, 0u, 0u, 0u}, g = {0u, 0u, 0u, 0u};
    if (qi < N) {
      a = ld_global16(qp + (size_t)qi * D + 16 * c + 8 * h32);
      g = ld_global16(dop + (size_t)qi * D + 16 * c + 8 * h32);
    }
    qreg[c] = as_bf16x8(a);
    doreg[c] = as_bf16x8(g);
  }
  const float lse2 = qi < N ? lse[(size_t)bh * N + qi] * kLog2e : INFINITY;
  const float dl = qi < N ? delta[(size_t)bh * N + qi] : 0.f;

  f32x16 dq_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  u32x4 pk[CPT], pv[CPT];
  auto load_tile = [&](int t) {
    const int t0 = t * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NW * 64;
      const int row = c / (D / 8), col = c % (D / 8), key = t0 + row;
      u32x4 a = {0u, 0u, 0u, 0u}, bb = {0u, 0u, 0u, 0u};
      if (key < N) {
        a = ld_global16(kp + (size_t)key * D + col * 8);
        bb = ld_global16(vp + (size_t)key * D + col * 8);
      }
      pk[i] = a;
      pv[i] = bb;
    }
  };
  auto store_tile = [&](int stage) {
    char* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * NW * 64;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<u32x4*>(base + swz<D>(row, col)) = pk[i];
      *reinterpret_cast<u32x4*>(base + T::BYTES + swz<D>(row, col)) = pv[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1);
    const int t0 = t * BN;
    const char* ks = smem + (t & 1) * STAGE;
    const char* vs = ks + T::BYTES;
    if (!CAUSAL || t0 <= qw0 + 31) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int off = swz<D>(kb * 32 + l32, 2 * c + h32);
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(ks + off);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(vs + off);
          s = mfma32(ak, qreg[c], s);
          dp = mfma32(av, doreg[c], dp);
        }
        // Lane owns query qi; register r holds key t0 + kb*32 + 8(r/4) + 4*h32 + r%4.
        const int kb0 = t0 + kb * 32;
        const bool need_mask = (kb0 + 32 > N) || (CAUSAL && kb0 + 31 > qw0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[r], scale_log2, -lse2));
          if (need_mask) {
            const int kj = kb0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            if (kj >= N || (CAUSAL && kj > qi)) p = 0.f;
          }
          dp[r] = p * (dp[r] - dl);
        }
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const bf16x8 dsa = pack8(dp, sh);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 bk = ld_tr_operand<D>(ks, kb * 32 + 16 * sh, db * 32, lane);
            dq_acc[db] = mfma32(dsa, bk, dq_acc[db]);
          }
        }
      }
    }
    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }
  // C layout: lane holds feature db*32 + l32 of queries qw0 + 8(r/4) + 4*h32 + r%4.
  uint16_t* dqp = dq + (size_t)bh * N * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = qw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      if (qq < N) dqp[(size_t)qq * D + db * 32 + l32] = (uint16_t)(pack_bf16x2(dq_acc[db][r] * scale, 0.f) & 0xffffu);
    }
}

// ------------------------------------------------------------------ host launcher
template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  const int BH = a.B * a.Hq;
  const int rows = BH * a.N;
  const float sl2 = a.scale * kLog2e;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((rows + 256 / (D / 8) - 1) / (256 / (D / 8))), dim3(256), 0,
                     a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_kt = (a.N + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(n_kt * BH), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.lse, a.delta,
                     (const uint16_t*)a.dout, (uint16_t*)a.dk, (uint16_t*)a.dv, a.N, a.scale, sl2, n_kt, BH);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qt = (a.N + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(n_qt * BH), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.lse, a.delta,
                     (const uint16_t*)a.dout, (uint16_t*)a.dq, a.N, a.scale, sl2, n_qt, BH);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
  return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
}

}  // namespace xattn

// Forward attention kernels for gfx950.
//
// Pages cited by title:
//   [FUND] "Attention fundamentals: the standard attention flow, complexity analysis,
//          memory bottleneck and inference challenges"
//   [OPT]  "FlashAttention optimisation: breaking the attention memory bottleneck"
//   [NOTE] "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
//
// One workgroup owns BM query rows of one (batch, head) and streams the key/value rows of
// that head through LDS in tiles of BN keys ([OPT] §3.1, [NOTE] Method item 1).  Per tile
// each wave computes its score block, updates the running row max m and running sum l and
// rescales its output accumulator by 2^(m_old - m_new) ([OPT] §3.2.1, [NOTE] Method item
// 2), then adds P V.  Normalisation by l happens once at the end ([OPT] §7.1).  Only O and
// the per-row log-sum-exp reach HBM ([OPT] §3.1).
//
// MI355X mapping:
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K is the
//     A operand read from LDS, Q^T the B operand held in registers for the whole kernel.
//     In the C layout each lane then owns one query column and 16 keys, so the row max and
//     row sum are 16 in-lane operations plus one v_permlane32_swap, and the probabilities
//     are already in the B-operand layout of the P V product (O^T = V^T P^T): no LDS round
//     trip for P.
//   * V^T, the A operand of that product, is read from the row-major V tile with the
//     transposing ds_read_b64_tr_b16, so the tile is stored exactly as it arrives.
//   * K/V tiles arrive ahead of use, so HBM/L2 latency hides behind compute ([OPT] §5.2):
//     fwd_ilv_kernel (bf16, d = 64 and 128) copies them straight into LDS rings of four
//     stages (buffer_load ... lds, no registers), K three tiles and V two tiles ahead, one
//     barrier per tile; fwd_f32_kernel (fp32 inputs) is single-buffered, and
//     fwd_f32_split_kernel (fp32, grids too small to fill the CUs) splits each workgroup's keys
//     over its waves, which load their next tile into registers during the current one.
//   * fwd_ilv_kernel software-pipelines each wave: the MFMAs of P_{u-1} V_{u-1} and of S_{u+1}
//     interleave with the vector work of the softmax of S_u in fixed slots.
//   * Causal: tiles past the diagonal are never loaded, waves whose rows all precede a tile
//     skip its MFMA work, and only diagonal tiles evaluate the mask.  Heavy (late) query
//     tiles are dispatched first; all query tiles of one head land on one XCD when the
//     head count is a multiple of 8, so the head's K/V stay in that XCD's L2.
//   * The exponentials use the base-2 hardware exp with scale*log2(e) folded into one FMA.
#include "common.h"
#include "launch.h"

namespace xattn {

constexpr int kFwdBN = 64;  // keys per tile
static_assert((kMaxSparseTiles - 1) * kFwdBN == kMaxSparseKeys, "block-sparse tile list size");

// Work-item -> (head, query tile): heavy-first for causal, head index fastest.
__device__ __forceinline__ void fwd_tile_of(int id, int BH, int n_qtiles, bool causal, int& bh, int& qt) {
  bh = id % BH;
  int t = id / BH;
  qt = causal ? (n_qtiles - 1 - t) : t;
}

// Interleaved forward (bf16, d = 64 and 128).  Each wave owns 32 query rows of the
// workgroup's block and software-pipelines its own work over 32-key blocks u: in step u it
// issues
//   O^T += V_{u-1}^T P_{u-1}^T  and  S_{u+1}^T = K_{u+1} Q^T        (MFMAs)
// and, between those MFMAs, the online softmax of S_u into P_u       (vector ALU),
// which are independent of each other, so the matrix core and the vector ALU of the SIMD
// work at the same time within one wave; two waves share each SIMD.  The S and P register
// sets alternate roles between even and odd steps.  K and V arrive in 64-key tiles through
// direct global -> LDS copies into two rings of four stages; the two steps of tile t read
// K_t, K_{t+1}, V_{t-1}, V_t, copy K_{t+3} and V_{t+2}, and end with one barrier.  With
// 32-key tiles each step is a tile of its own: step t reads K_{t+1} and V_{t-1}, copies
// K_{t+3} and V_{t+2}, and ends with the barrier.  A rescale of O forced by a moved running
// max is applied after the step's MFMAs, before P_u is added.
//
// LDS operands of the MFMAs are read this many MFMA slots ahead of their use.
constexpr int kIlvLookahead = 4;
// MFMA slot (modulo the copy spacing) at which a step issues each of its copies.
constexpr int kIlvCopySlot = 6;
// Dense and packed d = 128 inputs come in two shapes.  Wide: 8 waves (256 query rows) with
// 64-key tiles, one workgroup per CU (128 KB of LDS).  Narrow: 4 waves (128 rows) with 32-key
// tiles (64 KB), two workgroups per CU, so that one's prologue (Q loads, first copies) and
// epilogue (O stores) overlap the other's steps; it pays twice the copies and barriers per
// key.  Measured per workgroup, prologue plus epilogue cost about as much as 4-5 64-key tiles,
// so the narrow shape wins when a query tile walks few keys (+8% at N = 2048 causal, +18% at
// N = 512, +10% on packed batches of 256-4096 tokens), ties at 2048 keys (N = 4096 causal)
// and loses 2-5% on long walks (non-causal N = 4096, causal N = 16384, a 1024-query chunk
// onto 8192 keys).  Both give bit-identical results (same 32-key block order and arithmetic).
// The narrow shape is taken below this many average keys per query tile, or when the wide
// grid would leave CUs idle.
constexpr double kFwd128NarrowKeys = 2048.0;
// Largest lane-partial row sum of one 32-key step accepted without moving the reference max
// (so every probability stays below it).  Probabilities up to 2^16 keep the bf16 P and the fp32
// sums and products far from overflow; against 2^8 the larger bound moves the max, and redoes a
// step, less often on peaky rows (3-5% faster on the causal long prefill with doubled logits,
// unchanged on N(0,1) inputs).
constexpr float kSumMax = 65536.f;
// fp32: below this many 128-row workgroups (one per CU), the split-key kernel runs instead.
constexpr long long kFwdF32SplitGrid = 256;

template <int D, int NW_, int BN_>
struct IlvShape {
  static constexpr int BN = BN_, DC = D / 16, DB = D / 32;
  static constexpr int SPT = BN / 32;              // 32-key steps per tile
  static constexpr int NW = NW_, BM = NW * 32;     // waves, query rows per workgroup
  static constexpr int TILE = BN * D * 2;          // bytes of one K or V tile
  static constexpr int NS = 4;                     // stages per ring
  static constexpr int RPC = 1024 / (2 * D);       // tile rows per 1 KB wave copy
  static constexpr int CPW = TILE / 1024 / NW;     // copies per wave and tile of one tensor
  static constexpr int CPS = SPT == 2 ? CPW : 2 * CPW;  // copies per wave and step
  static_assert(SPT == 1 || SPT == 2, "32- or 64-key tiles");
  static constexpr int NPV = 2 * DB;               // V^T operands per 32-key block
  static constexpr int NQK = DC;                   // K operands per 32-key block
};

template <int D, int NW_, int BN_, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(64 * NW_) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_ilv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, SeqGeo geo, BlockMask bm,
    float scale_log2, int n_qtiles, int BH) {
  using S = IlvShape<D, NW_, BN_>;
  constexpr int BN = S::BN, SPT = S::SPT, DC = S::DC, DB = S::DB, NS = S::NS, NW = S::NW;
  constexpr int TILE = S::TILE, CPW = S::CPW, CPS = S::CPS, RPC = S::RPC, NPV = S::NPV, NQK = S::NQK;
  constexpr int NMF = NPV + NQK, L = kIlvLookahead;
  static_assert(NS == 4 && CPS <= 4, "copy schedule");
  static_assert(!SPARSE || BN == 64, "the block-sparse tile list counts 64-key tiles");
  constexpr int CSP = NMF / CPS;  // MFMA slots per copy
  static_assert(NMF % CPS == 0, "copies spread evenly over the step");
  __shared__ __attribute__((aligned(1024))) char smem[2 * NS * TILE];  // [K ring | V ring]
  __shared__ uint16_t tlist[SPARSE ? kMaxSparseTiles : 1];             // kept key tiles

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;

  int bh, qt;
  fwd_tile_of(blockIdx.x, BH, n_qtiles, CAUSAL, bh, qt);
  const int b = bh / Hq;
  const int hq = bh - b * Hq;
  const int hk = hq / (Hq / Hkv);
  const SeqRows sr = seq_rows(geo, b, hq, Hq, hk, Hkv);
  const int Nq = sr.lq, Nk = sr.lk;
  const int q0 = qt * S::BM;
  if (q0 >= Nq) return;  // query tile past the end of a shorter sequence
  const uint16_t* qp = q + sr.q * D;
  const uint16_t* kp = k + sr.k * D;
  const uint16_t* vp = v + sr.k * D;
  const int qw0 = q0 + wave * 32;  // rows qw0 + l32
  // Causal masks align the last query with the last key: query i sees keys j <= i + Nk - Nq.
  // A wave without query rows (past the end of a shorter sequence) skips all its MFMA work:
  // under the causal test its limit lies before every key.
  const bool has_rows = qw0 < Nq;
  const int qd0 = has_rows ? qw0 + (Nk - Nq) : -(1 << 29);  // last key visible to the wave's first row

  // Q^T operands: lane holds query qw0 + l32, features 16c + 8*h32 .. +7.
  bf16x8 qreg[DC];
  {
    const int qi = qw0 + l32;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (qi < Nq) u = ld_global16(qp + (size_t)qi * D + 16 * c + 8 * h32);
      qreg[c] = as_bf16x8(u);
    }
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  // O is divided by the sum of the same bf16 probabilities its P V product used, so that a row
  // dominated by one key gets that key's V row exactly; the fp32 sum l_run still gives the LSE.
  // Dividing by the fp32 sum instead leaves the bf16 rounding of the dominant probability (up
  // to 2^-9 relative: under the lazy reference max it lies in (1, 2^16], not at 1) in O, which
  // with the final rounding of O can exceed the 2e-2 error bound on peaky rows.  The sum comes
  // from the matrix cores at half the cost of one 32x32x16 product per 32 keys: one
  // v_mfma_f32_16x16x32_bf16 per 16 keys reads the P^T operand as its B (32 k x 16 n; column n,
  // k-groups 0..3 = query n keys 0-7, query n+16 keys 0-7, query n keys 8-15, query n+16 keys
  // 8-15) against a 0/1 selector A (row 0 picks groups 0 and 2, row 1 groups 1 and 3), so that
  // C row 0 accumulates the sum of query n and row 1 that of query n+16, in lanes 0-15.
  // (Measured against eight v_dot2_f32_bf16 per step, and two 32x32x16 products against ones:
  // 2.5-5% faster at d = 128, 3-13% at d = 64.)
  f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  const bool sel_on = ((lane & 15) == 0 && ((lane >> 4) & 1) == 0) || ((lane & 15) == 1 && ((lane >> 4) & 1) == 1);
  const bf16x8 sel16 = sel_on ? as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u})
                              : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  // Rescale of lsum by the per-row factor a: row 1 of lanes 0-15 belongs to query lane + 16.
  auto lsum_scale = [&](float a) __attribute__((always_inline)) {
    const float a_hi = __shfl(a, (lane & 15) + 16);
    lsum[0] *= a;
    lsum[1] *= a_hi;
  };
  float m_run = kMaxInit, l_run = 0.f;

  // Epilogue: O = acc / l, LSE = ln2 * (m + log2 l); a row without keys (l = 0) gets O = 0
  // and LSE = -inf.
  auto epilogue = [&]() __attribute__((always_inline)) {
    uint16_t* op = o + sr.q * D;
    const float lt = sum_xor32(l_run);
    // A row with keys has a bf16 sum >= 1: its largest probability is at least 1 against the
    // reference max, which never exceeds the row's running max.
    const float r0 = __shfl(lsum[0], l32 & 15), r1 = __shfl(lsum[1], l32 & 15);
    const float inv = lt > 0.f ? 1.f / (l32 < 16 ? r0 : r1) : 0.f;
    const int qi = qw0 + l32;
    if (qi < Nq) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = db * 32 + 8 * jj + 4 * h32;
          u32x2 w;
          w[0] = pack_bf16x2(acc[db][4 * jj + 0] * inv, acc[db][4 * jj + 1] * inv);
          w[1] = pack_bf16x2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
          *reinterpret_cast<u32x2*>(op + (size_t)qi * D + d) = w;
        }
      if (lse != nullptr && h32 == 0) lse[sr.q + qi] = (m_run + fast_log2(lt)) * kLn2;
    }
  };

  const int kv_end = CAUSAL ? min(Nk, q0 + S::BM + (Nk - Nq)) : Nk;
  int T = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  // Block-sparse: the workgroup walks only the tiles that one of its query blocks keeps; tile
  // position i of the walk holds key tile kt(i).  Dense: kt(i) = i.
  if constexpr (SPARSE) T = build_tile_list<S::BM / kSparseBlock>(bm, b, hq, q0 / kSparseBlock, T, tlist);
  if (T == 0) {  // no key for any row of the tile (empty key sequence, causal with Nk < Nq, or
    epilogue();  // every block dropped)
    return;
  }
  // 32-key tiles go two per pass: an odd count gets one more tile past the last key (clamped
  // copies, every score masked: probabilities 0), whose step does the last P V product.
  if constexpr (SPT == 1) T += T & 1;
  auto entry = [&](int i) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_readfirstlane((int)tlist[min(i, T - 1)]);
  };
  const int wblk = (qw0 - q0) / kSparseBlock;  // the wave's query block within the workgroup
  TileOffsets<D> ofs;
  ofs.init(lane);
  // The V ring sits above the K ring; its base goes into the per-lane V offsets so that the
  // constant part of every V address fits the 16-bit offset field of the LDS reads.
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    ofs.v[db][0] += NS * TILE;
    ofs.v[db][1] += NS * TILE;
  }

  // Copies: tile i of K (V) lives in stage i % 4 of the K (V) ring.  Wave copy j covers tile
  // rows RPC*j .. RPC*j + RPC-1; lane l fills physical chunk l of that 1 KB block (row
  // RPC*j + l/(D/8), chunk l%(D/8)), so it reads logical chunk (l%(D/8)) ^ swizzle(row).
  // Each copy goes through a buffer resource over the key rows from the tile's first row on,
  // so the per-lane byte offset within the tile is a constant and rows past the last key
  // arrive as zeros (finite data whose probabilities are zero); the resource and the LDS
  // destination are scalar work.  Byte counts stay below 2^31: the API bounds the key rows
  // times 2d under that.
  const int lrow = lane / (D / 8);
  uint32_t loff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = RPC * (wave * CPW + i) + lrow;
    loff[i] = r * (2 * D) + 16 * ((lane % (D / 8)) ^ ((swz<D>(r, 0) >> 4) & (D / 8 - 1)));
  }
  const char* kbase = reinterpret_cast<const char*>(wave_uniform(kp));
  const char* vbase = reinterpret_cast<const char*>(wave_uniform(vp));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;
  const uint32_t wdst = lds0 + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * (CPW * 1024);
  auto copy = [&](int tile, int ktile, bool is_k, int i) __attribute__((always_inline)) {
    const int first = ktile * BN;  // first key row of the tile
    const i32x4 rsrc = buffer_rsrc((is_k ? kbase : vbase) + (size_t)first * (2 * D), (Nk - first) * (2 * D));
    const uint32_t m0v = wdst + (is_k ? 0 : NS * TILE) + (tile & (NS - 1)) * TILE + 1024 * i;
    bdma16_m0(rsrc, loff[i], m0v);
  };
  // LDS base of 32-key block u of V (relative to the V ring, see ofs.v): tile u/SPT, rows
  // 32*(u%SPT) ..
  constexpr int SPT_SH = SPT == 2 ? 1 : 0;
  auto vblk = [&](int u) __attribute__((always_inline)) {
    return smem + ((u >> SPT_SH) & (NS - 1)) * TILE + (u & (SPT - 1)) * 32 * (2 * D);
  };
  // Operand j of a step: j < NPV are V^T operands (sh, db), db fastest; then the K operands c.
  auto operand = [&](const char* ks, const char* vs, auto jc) __attribute__((always_inline)) -> bf16x8 {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < NPV) {
      constexpr int db = j % DB, sh = j / DB;
      const char* base = vs + 16 * sh * (2 * D);
      return join_tr(ds_read_tr16(base + ofs.v[db][0]), ds_read_tr16(base + ofs.v[db][1]));
    } else {
      return *reinterpret_cast<const bf16x8*>(ks + ofs.k[j - NPV]);
    }
  };
  // A wave has work in step u if it holds a query row and key block u-1 still holds keys at
  // or before its last row (block-sparse: every step; dropped and masked blocks give
  // probability 0).
  auto active = [&](int u) __attribute__((always_inline)) {
    if constexpr (SPARSE || !CAUSAL) return has_rows;
    else return (u - 1) * 32 <= qd0 + 31;
  };
  auto kt = [&](int i) __attribute__((always_inline)) -> int {
    if constexpr (SPARSE) return entry(i) & 0x3fff;
    else return i;
  };
  // Copy ci (< CPS) of step phase ph (0 .. SPT-1) of the steps of tile t: with 64-key tiles
  // the first step copies K_{t+3}, the second V_{t+2}; with 32-key tiles the one step copies
  // both.
  auto step_copy = [&](int t, auto phc, int ci) __attribute__((always_inline)) {
    constexpr int ph = decltype(phc)::value;
    if constexpr (SPT == 2) {
      if constexpr (ph == 0) copy(t + 3, kt(t + 3), true, ci);
      else copy(t + 2, kt(t + 2), false, ci);
    } else {
      if (ci < CPW) copy(t + 3, kt(t + 3), true, ci);
      else copy(t + 2, kt(t + 2), false, ci - CPW);
    }
  };

  // Prologue: K_0, K_1, K_2, V_0, V_1; V stage 3 (read as block -1, with P_{-1} = 0) is zeroed.
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    copy(0, kt(0), true, i);
    if (1 < T) copy(1, kt(1), true, i);
    if (2 < T) copy(2, kt(2), true, i);
    copy(0, kt(0), false, i);
    if (1 < T) copy(1, kt(1), false, i);
  }
  for (int i = tid; i < TILE / 16; i += NW * 64)
    *reinterpret_cast<u32x4*>(smem + NS * TILE + (NS - 1) * TILE + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  f32x16 sA, sB;
  u32x4 pA[2], pB[2];
  pA[0] = u32x4{0u, 0u, 0u, 0u};
  pA[1] = u32x4{0u, 0u, 0u, 0u};
  wait_vmem();  // also covers the Q loads
  lds_barrier();
  // S_0.
  {
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + ofs.k[c]);
      if (c == 0) {
        f32x16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.f;
        sA = mfma32(a, qreg[0], z);
      } else {
        sA = mfma32(a, qreg[c], sA);
      }
    }
  }

  // Operands in flight (read L products ahead of their use, across step boundaries).  Step 0's
  // first ones are V block -1 (stage NS-1, zeroed; its second half with 64-key tiles).
  static_assert(L <= NPV, "the operands read across a step boundary are V^T operands");
  bf16x8 buf[L];
  {
    const char* vs0 = smem + ((NS - 1) * TILE + (SPT - 1) * 32 * (2 * D));
    static_for<L>([&](auto jc) { buf[decltype(jc)::value] = operand(vs0, vs0, jc); });
  }

  // Step u (phase ph of tile t = u / SPT): sc = S_u (complete), sn <- S_{u+1}, pp = P_{u-1},
  // pc <- P_u; the step's share of the tile's copy list (step_copy).  Tiles past the end are
  // copied too, clamped to the last key, into stages nobody reads any more, so every step
  // issues the same copies and the wait counts stay fixed.  kcur is the key tile of S_u and
  // keep whether the wave's query block keeps it (block-sparse).
  auto step = [&](int u, auto phc, auto stc, f32x16& sc, f32x16& sn, u32x4(&pp)[2], u32x4(&pc)[2], int t, int kcur,
                  bool keep) __attribute__((always_inline)) {
    if (active(u)) {
      const int u0 = kcur * BN + (u & (SPT - 1)) * 32;  // first key of S_u
      const bool drop = SPARSE && !keep;
      if (drop || (u0 + 32 > Nk) || (CAUSAL && u0 + 31 > qd0)) {
        const int kmax = qd0 + l32;  // last key of this lane's row
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = u0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
          if (drop || kj >= Nk || (CAUSAL && kj > kmax)) sc[r] = -INFINITY;
        }
      }
      // K block u+1 and V block u-1 at offsets known at compile time from the ring stage of
      // tile t (the tile loop is unrolled over the four stages).
      constexpr int st = decltype(stc)::value, ph = decltype(phc)::value;
      constexpr int kst = SPT == 2 ? (st + ph) % NS : (st + 1) % NS, khalf = SPT == 2 ? 1 - ph : 0;
      constexpr int vst = SPT == 2 ? (st + NS - 1 + ph) % NS : (st + NS - 1) % NS, vhalf = SPT == 2 ? 1 - ph : 0;
      const char* ks = smem + (kst * TILE + khalf * 32 * (2 * D));
      const char* vs = smem + (vst * TILE + vhalf * 32 * (2 * D));  // V ring base is in ofs.v
      // The next step's V block is V_u: stage st, half ph.  It has landed (it is read in this
      // tile or the next one) and no copy overwrites its stage before the next tile's barrier.
      const char* nvs = smem + (st * TILE + ph * 32 * (2 * D));
      float rs0 = 0.f, rs1 = 0.f;
      sched_fence();
      static_for<NMF>([&](auto ic) {
        constexpr int j = decltype(ic)::value;
        if constexpr (j < NPV) {
          constexpr int db = j % DB, sh = j / DB;
          acc[db] = mfma32(buf[j % L], as_bf16x8(pp[sh]), acc[db]);
          if constexpr (db == 0) lsum = mfma16(sel16, as_bf16x8(pp[sh]), lsum);
        } else {
          constexpr int c = j - NPV;
          if constexpr (c == 0) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.f;
            sn = mfma32(buf[j % L], qreg[0], z);
          } else {
            sn = mfma32(buf[j % L], qreg[c], sn);
          }
        }
        // Operand reads L slots ahead; the last L slots read the next step's first operands.
        if constexpr (j + L < NMF) buf[j % L] = operand(ks, vs, std::integral_constant<int, j + L>{});
        else buf[j % L] = operand(ks, nvs, std::integral_constant<int, j + L - NMF>{});
        // Vector work: the exponentials of S_u, four per group.  d = 128 (16 slots): spread
        // evenly over slots 1 .. 14 (1, 4, 7, 10).  d = 64 (8 slots): every other slot from 0
        // on, so that the chain of S_{u+1} products in the second half of the step also runs
        // beside vector work (2-5% faster than slots 1-4 on the d = 64 prefill shapes; for
        // d = 128 the placement measured within 1%).
        constexpr int E0 = 1, NE = 4, ESPAN = NMF - 2 - E0;
        static_for<NE>([&](auto ec) {
          constexpr int jq = decltype(ec)::value;
          if constexpr ((NMF == 8 ? 2 * jq : E0 + jq * ESPAN / NE) == j) {
            float p[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) p[w] = fast_exp2(fmaf(sc[4 * jq + w], scale_log2, -m_run));
            uint32_t w0 = pack_bf16x2(p[0], p[1]), w1 = pack_bf16x2(p[2], p[3]);
            // fp32 row sums (summing the bf16-rounded values would cost the LSE up to 2^-9).  The
            // first group assigns: adding it to 0.f is not an identity for the compiler (signed
            // zeros), so it would cost two adds per step.
            if constexpr (jq == 0) {
              rs0 = p[0] + p[2];
              rs1 = p[1] + p[3];
            } else {
              rs0 += p[0] + p[2];
              rs1 += p[1] + p[3];
            }
            // Keeps this step's vector work in its slot (the compiler would otherwise sink it).
            asm volatile("" : "+v"(w0), "+v"(w1), "+v"(rs0), "+v"(rs1));
            pc[jq / 2][2 * (jq % 2)] = w0;
            pc[jq / 2][2 * (jq % 2) + 1] = w1;
          }
        });
        // The step's CPS copies, one every CSP slots (slots 6 and 14 with 64-key tiles at d = 128).
        if constexpr (j % CSP == kIlvCopySlot % CSP && j / CSP < CPS) step_copy(t, phc, j / CSP);
        sched_fence();
      });
      // Reference max check ([OPT] §3.2.1, lazily): the step's probabilities were formed
      // against the current reference m.  If every lane-partial row sum stays at or below
      // kSumMax (so does every probability; the first visible key of a row overflows against
      // the initial m = kMaxInit, and +inf fails the test) they are kept.  Otherwise the wave
      // redoes the step with m moved to the running max (at least kMaxInit, so finite) and
      // rescales O and l by 2^(m_old - m_new); the P V products already issued this step used
      // the old m, as O did.  Masked scores (-inf) give probability 0 against any finite m.
      if (__builtin_amdgcn_ballot_w64(!(rs0 + rs1 <= kSumMax)) != 0) {
        sched_fence();
        float mx = sc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
        mx = max_xor32(mx) * scale_log2;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          float pv[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) pv[w] = fast_exp2(fmaf(sc[4 * jq + w], scale_log2, -m_new));
          const uint32_t w0 = pack_bf16x2(pv[0], pv[1]), w1 = pack_bf16x2(pv[2], pv[3]);
          const float a0 = pv[0] + pv[2], a1 = pv[1] + pv[3];
          rs0 = jq == 0 ? a0 : rs0 + a0;
          rs1 = jq == 0 ? a1 : rs1 + a1;
          pc[jq / 2][2 * (jq % 2)] = w0;
          pc[jq / 2][2 * (jq % 2) + 1] = w1;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        lsum_scale(alpha);
        sched_fence();
      }
      // One branch only: a second one on the same condition costs the allocator ~40 registers.
      l_run += rs0 + rs1;
    } else {
#pragma unroll
      for (int i = 0; i < CPS; ++i) step_copy(t, phc, i);
    }
  };

  // Four tiles per pass, one per ring stage, so that every LDS operand address is a per-lane
  // offset plus a constant; the pass stops after the last tile.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  for (int t = 0; t < T;) {
    static_for<NS>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      if (t < T) {
        if constexpr (SPT == 2) {
          int kc = t, keep = 1;
          if constexpr (SPARSE) {
            const int e = entry(t);
            kc = e & 0x3fff;
            keep = (e >> (14 + wblk)) & 1;
          }
          step(2 * t, I0{}, stc, sA, sB, pA, pB, t, kc, keep != 0);
          step(2 * t + 1, I1{}, stc, sB, sA, pB, pA, t, kc, keep != 0);
        } else if constexpr (st % 2 == 0) {  // 32-key tiles: S/P register roles alternate per tile
          step(t, I0{}, stc, sA, sB, pA, pB, t, t, true);
        } else {
          step(t, I0{}, stc, sB, sA, pB, pA, t, t, true);
        }
        // Everything copied before this tile's steps must have landed (64-key tiles: K_{t+2}
        // and V_{t+1}; 32-key tiles: K_{t+2} and V_t); this tile's copies may stay in flight.
        wait_vmem_n<2 * CPW>();
        lds_barrier();
        ++t;
      }
    });
  }
  wait_vmem();

  // P_{last} V_{last} (the last step is odd, so P is in pA).
  if (active(SPT * T)) {
    const char* vs = vblk(SPT * T - 1);
    static_for<NPV>([&](auto jc) {
      constexpr int j = decltype(jc)::value, db = j % DB, sh = j / DB;
      const bf16x8 a = operand(vs, vs, jc);
      acc[db] = mfma32(a, as_bf16x8(pA[sh]), acc[db]);
      if constexpr (db == 0) lsum = mfma16(sel16, as_bf16x8(pA[sh]), lsum);
    });
  }

  epilogue();
}

// fp32 inputs (d = 64): the same tiled online softmax with v_mfma_f32_32x32x2_f32, one
// wave per 32 queries and 32-key tiles, single-buffered.  Keeps full fp32 precision.
template <bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, SeqGeo geo, BlockMask /*dense only*/,
    float scale_log2, int n_qtiles, int BH) {
  constexpr int D = 64, BM = 128, BN = 32, P = D + 1;  // P: padded pitch in floats
  __shared__ float ks[BN * P];
  __shared__ float vs[BN * P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  int bh, qt;
  fwd_tile_of(blockIdx.x, BH, n_qtiles, CAUSAL, bh, qt);
  const int b = bh / Hq, hq = bh - b * Hq, hk = hq / (Hq / Hkv);
  const SeqRows sr = seq_rows(geo, b, hq, Hq, hk, Hkv);
  const int Nq = sr.lq, Nk = sr.lk;
  const int q0 = qt * BM, qw0 = q0 + wave * 32, qi = qw0 + l32;
  if (q0 >= Nq) return;  // query tile past the end of a shorter sequence
  const float* qp = q + sr.q * D;
  const float* kp = k + sr.k * D;
  const float* vp = v + sr.k * D;
  const int qd0 = qw0 + (Nk - Nq), kmax = qi + (Nk - Nq);  // causal: query i sees keys <= i + Nk - Nq

  float qr[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qr[c] = (qi < Nq) ? qp[(size_t)qi * D + 2 * c + h32] : 0.f;
  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { acc[0][r] = 0.f; acc[1][r] = 0.f; }
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = CAUSAL ? min(Nk, q0 + BM + (Nk - Nq)) : Nk;
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * BN;
    for (int i = tid; i < BN * D; i += 256) {
      const int row = i / D, col = i % D, key = t0 + row;
      ks[row * P + col] = key < Nk ? kp[(size_t)key * D + col] : 0.f;
      vs[row * P + col] = key < Nk ? vp[(size_t)key * D + col] : 0.f;
    }
    __syncthreads();
    if (!CAUSAL || t0 <= qd0 + 31) {
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 2; ++c) s = mfma32_f32(ks[l32 * P + 2 * c + h32], qr[c], s);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = t0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        if (kj >= Nk || (CAUSAL && kj > kmax)) s[r] = -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = fast_exp2(fmaf(s[r], scale_log2, -m_use)); rs += s[r]; }
      l_run = fmaf(l_run, alpha, rs);
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[0][r] *= alpha; acc[1][r] *= alpha; }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * h32 + (r & 3);
        acc[0] = mfma32_f32(vs[key * P + l32], s[r], acc[0]);
        acc[1] = mfma32_f32(vs[key * P + 32 + l32], s[r], acc[1]);
      }
    }
    __syncthreads();
  }
  // A row without keys (l = 0, m = -inf) gets O = 0 and LSE = -inf.
  const float lt = sum_xor32(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < Nq) {
    float* op = o + (sr.q + qi) * D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) op[db * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3)] = acc[db][r] * inv;
    if (lse != nullptr && h32 == 0) lse[sr.q + qi] = lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

// fp32 inputs with few query rows (a grid of 128-row tiles that would leave CUs idle, such as
// one head of 256 queries): a workgroup takes 32 query rows and its four waves split the keys,
// wave w walking the 32-key tiles w, w+4, w+8, ... with its own running max, sum and output.
// The four partial results are merged through LDS at the end: with m = max_w m_w and
// e_w = 2^(m_w - m), O = sum_w e_w O_w / sum_w e_w l_w, the same combination as for blocks of one
// row ([OPT] §3.2.2), exact in real arithmetic.  Each wave keeps its own K/V tile in LDS (no
// workgroup barrier in the walk) and loads its next tile into registers while it computes the
// current one.
template <bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_split_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, SeqGeo geo, BlockMask /*dense only*/,
    float scale_log2, int n_qtiles, int BH) {
  constexpr int D = 64, BM = 32, BN = 32, P = D + 1, NW = 4;  // P: padded pitch in floats
  constexpr int MP = 33;                                      // merge: [d][query] pitch
  static_assert(NW * (D * MP + 2 * BM) <= NW * 2 * BN * P, "merge area fits the tiles");
  __shared__ float smem[NW * 2 * BN * P];  // per wave: K tile, V tile; then the merge area
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h32 = lane >> 5;
  int bh, qt;
  fwd_tile_of(blockIdx.x, BH, n_qtiles, CAUSAL, bh, qt);
  const int b = bh / Hq, hq = bh - b * Hq, hk = hq / (Hq / Hkv);
  const SeqRows sr = seq_rows(geo, b, hq, Hq, hk, Hkv);
  const int Nq = sr.lq, Nk = sr.lk;
  const int q0 = qt * BM, qi = q0 + l32;
  if (q0 >= Nq) return;  // query tile past the end of a shorter sequence
  const float* qp = q + sr.q * D;
  const float* kp = k + sr.k * D;
  const float* vp = v + sr.k * D;
  const int qd0 = q0 + (Nk - Nq), kmax = qi + (Nk - Nq);  // causal: query i sees keys <= i + Nk - Nq

  float qr[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qr[c] = (qi < Nq) ? qp[(size_t)qi * D + 2 * c + h32] : 0.f;
  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { acc[0][r] = 0.f; acc[1][r] = 0.f; }
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = CAUSAL ? min(Nk, q0 + BM + (Nk - Nq)) : Nk;
  const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  float* ks = smem + wave * (2 * BN * P);
  float* vs = ks + BN * P;
  // Tile rows 4j + lane/16 (j = 0..7), 16-byte chunk lane%16; rows past the last key read the
  // last key (their scores are masked, so they get probability 0).
  f32x4 pk[8], pv[8];
  auto fetch = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = min(t * BN + 4 * j + (lane >> 4), Nk - 1);
      pk[j] = *reinterpret_cast<const f32x4*>(kp + (size_t)row * D + 4 * (lane & 15));
      pv[j] = *reinterpret_cast<const f32x4*>(vp + (size_t)row * D + 4 * (lane & 15));
    }
  };
  if (wave < ntiles) fetch(wave);
  for (int t = wave; t < ntiles; t += NW) {
    const int t0 = t * BN;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ks[(4 * j + (lane >> 4)) * P + 4 * (lane & 15) + e] = pk[j][e];
        vs[(4 * j + (lane >> 4)) * P + 4 * (lane & 15) + e] = pv[j][e];
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done before its reads
    __builtin_amdgcn_wave_barrier();
    if (t + NW < ntiles) fetch(t + NW);  // in flight during this tile
    if (!CAUSAL || t0 <= qd0 + 31) {
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 2; ++c) s = mfma32_f32(ks[l32 * P + 2 * c + h32], qr[c], s);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = t0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        if (kj >= Nk || (CAUSAL && kj > kmax)) s[r] = -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = fast_exp2(fmaf(s[r], scale_log2, -m_use)); rs += s[r]; }
      l_run = fmaf(l_run, alpha, rs);
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[0][r] *= alpha; acc[1][r] *= alpha; }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * h32 + (r & 3);
        acc[0] = mfma32_f32(vs[key * P + l32], s[r], acc[0]);
        acc[1] = mfma32_f32(vs[key * P + 32 + l32], s[r], acc[1]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this tile's LDS reads are done before the next writes
    __builtin_amdgcn_wave_barrier();
  }

  // Merge.  Wave w's partial: mo[w][d * MP + query] (unnormalised O), then m_w and l_w per query.
  const float lt = sum_xor32(l_run);
  __syncthreads();  // every wave is done with its tiles
  float* mo = smem + wave * (D * MP + 2 * BM);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) mo[(db * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3)) * MP + l32] = acc[db][r];
  if (h32 == 0) {
    mo[D * MP + l32] = m_run;
    mo[D * MP + BM + l32] = lt;
  }
  __syncthreads();
  // Wave w finishes features 16w + 8 h32 .. +7 of query q0 + l32.
  float mw[NW], ew[NW];
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = smem[w * (D * MP + 2 * BM) + D * MP + l32];
    m = fmaxf(m, mw[w]);
  }
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    ew[w] = (m == -INFINITY) ? 0.f : fast_exp2(mw[w] - m);  // a row without keys: every e_w = 0
    L = fmaf(ew[w], smem[w * (D * MP + 2 * BM) + D * MP + BM + l32], L);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (qi < Nq) {
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 16 * wave + 8 * h32 + e;
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) x = fmaf(ew[w], smem[w * (D * MP + 2 * BM) + d * MP + l32], x);
      out[e] = x * inv;
    }
    float* op = o + (sr.q + qi) * D + 16 * wave + 8 * h32;
    *reinterpret_cast<f32x4*>(op) = f32x4{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<f32x4*>(op + 4) = f32x4{out[4], out[5], out[6], out[7]};
    if (lse != nullptr && wave == 0 && h32 == 0) lse[sr.q + qi] = L > 0.f ? (m + fast_log2(L)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------------- host launchers
// Grid: one workgroup per (query tile, batch, head); query tiles cover the longest query
// sequence and those past a shorter sequence's end exit at once.
template <typename T>
using FwdKernel = void (*)(const T*, const T*, const T*, T*, float*, int, int, SeqGeo, BlockMask, float, int, int);

template <typename T>
static hipError_t launch_fwd_grid(FwdKernel<T> kern, int BM, int threads, const FwdArgs& a) {
  const int n_qtiles = (a.max_q + BM - 1) / BM;
  const int BH = a.B * a.Hq;
  if (n_qtiles == 0) return hipSuccess;  // every query sequence is empty
  const SeqGeo geo{a.cu_q, a.cu_k, a.Nq, a.Nk};
  const BlockMask bm{a.block_mask, a.mask_sb, a.mask_sh, (a.Nq + kSparseBlock - 1) / kSparseBlock,
                     (a.Nk + kSparseBlock - 1) / kSparseBlock};
  hipLaunchKernelGGL(kern, dim3(n_qtiles * BH), dim3(threads), 0, a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.o, a.lse, a.Hq, a.Hkv, geo, bm, a.scale * kLog2e, n_qtiles, BH);
  return hipGetLastError();
}

// Picks the <causal, sparse> instantiation of a kernel template.
#define XATTN_PICK(K, ...)                                                                           \
  (a.block_mask ? (a.causal ? K<__VA_ARGS__, true, true> : K<__VA_ARGS__, false, true>)              \
                : (a.causal ? K<__VA_ARGS__, true, false> : K<__VA_ARGS__, false, false>))

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == 0) {  // fp32, d = 64 (dense only)
    // A grid of 128-row tiles that leaves CUs idle takes 32-row tiles whose waves split the keys.
    if ((long long)((a.max_q + 127) / 128) * a.B * a.Hq < kFwdF32SplitGrid)
      return launch_fwd_grid<float>(a.causal ? fwd_f32_split_kernel<true> : fwd_f32_split_kernel<false>, 32, 256, a);
    return launch_fwd_grid<float>(a.causal ? fwd_f32_kernel<true> : fwd_f32_kernel<false>, 128, 256, a);
  }
  if (a.d == 64) {  // four waves, 128-row tiles, 64-key tiles: two workgroups per CU
    using S = IlvShape<64, 4, 64>;
    return launch_fwd_grid<uint16_t>(XATTN_PICK(fwd_ilv_kernel, 64, S::NW, S::BN), S::BM, S::NW * 64, a);
  }
  using W = IlvShape<128, 8, 64>;
  using N = IlvShape<128, 4, 32>;
  if (a.block_mask)  // the block-sparse tile list counts 64-key tiles
    return launch_fwd_grid<uint16_t>(XATTN_PICK(fwd_ilv_kernel, 128, W::NW, W::BN), W::BM, W::NW * 64, a);
  // Average keys walked by one query tile (packed: per-sequence averages).
  const double nq = a.cu_q ? (double)a.Nq / a.B : (double)a.Nq;
  const double nk = a.cu_q ? (double)a.Nk / a.B : (double)a.Nk;
  const double walk = a.causal ? (nk > nq ? nk - nq : 0.0) + 0.5 * (nq < nk ? nq : nk) : nk;
  const long long wide_grid = (long long)((a.max_q + W::BM - 1) / W::BM) * a.B * a.Hq;
  if (walk < kFwd128NarrowKeys || wide_grid < 256)
    return launch_fwd_grid<uint16_t>(a.causal ? fwd_ilv_kernel<128, N::NW, N::BN, true, false>
                                              : fwd_ilv_kernel<128, N::NW, N::BN, false, false>,
                                     N::BM, N::NW * 64, a);
  return launch_fwd_grid<uint16_t>(a.causal ? fwd_ilv_kernel<128, W::NW, W::BN, true, false>
                                            : fwd_ilv_kernel<128, W::NW, W::BN, false, false>,
                                   W::BM, W::NW * 64, a);
}
#undef XATTN_PICK

}  // namespace xattn

// fa2_fwd.hip -- exact attention forward for gfx950: O and the per-row logsumexp.
//
// Method (FlashAttention-2 pages: "Flash Attention spiegata: una guida completa", datacamp,
// sections "Tiling" and "Flash Attention 2"; wiki article "FlashAttention-2", section on
// technical architecture): Q is split into row blocks, K/V are streamed through on-chip
// memory tile by tile, and the softmax is applied incrementally -- a running row max m and
// row sum l, with the output accumulator rescaled whenever m grows -- so the N x N matrix is
// never stored. Only O and LSE = m + ln l reach HBM.
//
// gfx950 mapping (one workgroup per (batch, query head, query block of 256 or 128 rows)):
//  * 8 waves for long sequences on large grids, else 4 (several workgroups per CU); two waves
//    per SIMD (three at d = 64 with 4-wave workgroups, one at d = 256 with a sliding window).
//    Each wave owns 32 query rows for the whole pass, so the online-softmax state and all row
//    reductions stay in that wave's registers. Head dim 256 without a window runs the
//    split-role kernel at the end of this file instead: the two waves of a SIMD share 32 rows,
//    one holding O's first 128 columns and the softmax, the other O's last 128 columns.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: each lane then
//    holds one query row and 16 keys, the row max/sum are in-register reductions plus one
//    v_permlane32_swap, and S^T's accumulator is directly the B operand of O^T += V^T P^T.
//  * K and V tiles (64 keys) arrive by buffer_load ... lds (no staging registers), double
//    buffered. K is read as 16-byte A-operand rows; V^T is read with ds_read_b64_tr_b16.
//    Both tiles are XOR-swizzled so these reads hit distinct LDS banks. Each tile is one
//    unrolled MFMA stream (S slots, then P V slots) whose LDS operands are read a few slots
//    ahead; the exponentials of one tile run between the S MFMAs of the next.
//  * Causal: K/V tiles above a wave's last row are skipped; only tiles that straddle the
//    diagonal (or the ragged end of the sequence) are masked. Query blocks are scheduled
//    heaviest first, and blocks of one head stay on one XCD so their K/V reads share an L2.
//    8-wave d = 128 workgroups take four query blocks one after the other, one from each
//    quarter of the blocks sorted by length (snake order), so every workgroup carries the
//    same causal work and the workgroups of a head stay close together on the key tiles.
//  * Sliding window (causal, keys i - W .. i): the workgroup starts at its first visible tile,
//    and the leading tiles that cross the window's lower edge are masked too.
//  * Scale folded into the exponent: p = 2^(s*c - m) with c = |scale|*log2(e); a negative
//    scale flips the sign of the Q operand instead. The reference m is raised -- and O and l
//    rescaled -- only when some row's tile max exceeds it by more than 8 (log2 units), so p
//    stays below 2^8.
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, N;
  int causal;
  float c;        // |scale| * log2(e)
  unsigned qneg;  // 0x80008000 flips both bf16 signs of a packed pair when scale < 0
  int nqb;        // query blocks per head
  int xcd_remap;  // B*Hq divisible by 8: keep each head's blocks on one XCD
  int window;     // causal window: query i sees keys i - window .. i (>= N: no window)
  float vmul;     // factor on O: 1, or the FP8 value scale of V
};

// NW waves per workgroup (8 or 4; 4 at d = 256).
template <int D, int NW>
struct FwdCfg {
  static constexpr int BN = 64;               // keys per tile
  // Waves per SIMD: three for 4-wave workgroups at d = 64 (the kernel fits 168 registers; three
  // workgroups share a CU), two otherwise up to d = 128. At d = 256 a 32-row block's O
  // accumulators alone take 128 registers, so one wave per SIMD with them in AGPRs.
  static constexpr int WAVES = NW;
  static constexpr int WPE = D <= 64 && NW == 4 ? 3 : D <= 128 ? 2 : 1;
  static constexpr int QPW = 32;              // query rows per wave
  static constexpr int NQB = QPW / 32;        // 32-row MFMA blocks per wave
  static constexpr int BM = WAVES * QPW;      // query rows per workgroup
  static constexpr int KS = D / 16;           // k-steps of the Q.K contraction
  static constexpr int DB = D / 32;           // 32-wide blocks of the head dim
  static constexpr int CH = D / 8;            // 16-byte chunks per bf16 row
  static constexpr int ROWB = D * 2;          // bytes per bf16 row
  static constexpr int TILE = BN * ROWB;      // bytes of one K or V tile
  static constexpr int LPW = TILE / 1024 / WAVES;  // 1 KB direct-to-LDS loads per wave per tile
  static constexpr int LA = 3;  // LDS operand reads run this many MFMA slots ahead
  static_assert(TILE % (1024 * WAVES) == 0, "a tile splits evenly into the waves' copies");
};

// Copy keys [j0, j0+64) of one head into a swizzled LDS tile. Rows past N read as zero.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, lds_char* tile, int j0,
                                          int wave, int lane) {
  using C = FwdCfg<D, NW>;
#pragma unroll
  for (int t = 0; t < C::LPW; ++t) {
    const int blk = wave * C::LPW + t;
    const int pos = blk * 1024 + lane * 16;  // where this lane's 16 bytes land
    const int r = pos / C::ROWB;
    const int cp = (pos % C::ROWB) / 16;
    const int c = cp ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
    buffer_load16_lds(rs, tile + blk * 1024, (uint32_t)(j0 + r) * C::ROWB + c * 16);
  }
}

// Workgroups per head. With 8-wave workgroups at d = 128 (one workgroup per CU, nothing else
// to hide its start-up behind) each takes 2 kp query blocks, which divides the workgroups'
// start-up (Q, first K/V tiles) and wind-down (O stores) costs by four. Measured against one
// block per workgroup at causal B2 H32 N8192: two blocks 6 % faster, four 9 %, eight slower
// again (too few workgroups to balance). The other configurations keep one block per
// workgroup (a second block's live ranges push them into register spills).
// kp: pairs of query blocks per workgroup; 0: one block per workgroup.
__host__ __device__ constexpr int fwd_pairs_per_wg(int d, int nw) { return d == 128 && nw == 8 ? 2 : 0; }
__host__ __device__ inline int fwd_work_items(int nqb, int kp) {
  return kp == 0 ? nqb : ((nqb + 1) / 2 + kp - 1) / kp;
}

// Block id -> (head slice, work item j). Workgroups are dealt round-robin to the 8 XCDs
// (bid & 7 is the XCD); when the slice count divides by 8, each XCD gets a contiguous range of
// heads and walks their work items in order.
__device__ __forceinline__ void map_block(int bid, const FwdParams& p, int kp, int& bh, int& j) {
  const int nw = fwd_work_items(p.nqb, kp);
  if (p.xcd_remap) {
    const int x = bid & 7, s = bid >> 3;
    const int heads_per_xcd = (p.B * p.Hq) >> 3;
    bh = x * heads_per_xcd + s / nw;
    j = s % nw;
  } else {
    bh = bid / nw;
    j = bid % nw;
  }
}

// Online softmax with a reference that is raised only when needed. The exponentials of a
// tile are taken against the row's reference m (log2 domain), p = 2^(s c - m). All terms of
// a row share the reference, so any m gives the same softmax; m only has to keep p small.
// Before a tile's exponentials are formed, m is raised to that tile's row max -- rescaling O
// and l -- if the max exceeds m by more than kRescaleSlack; so p <= 2^kRescaleSlack and the
// 64 accumulator registers of a row block are rescaled only when a max really moves.
constexpr float kRescaleSlack = 8.0f;

// __builtin_amdgcn_sched_barrier mask that lets VALU, SALU, transcendental, VMEM and LDS-write
// instructions be scheduled across, but neither LDS reads nor MFMAs (the all-ALU bit 0x1 would
// let MFMAs pass too, so it stays clear).
constexpr int kPinDsReadMfma = 0x0002 | 0x0004 | 0x0010 | 0x0020 | 0x0040 | 0x0200 | 0x0400;

// FP8: Q and K are FP8 E4M3FN rows of D bytes and S^T = K Q^T runs on the FP8 MFMA (64-deep
// k-steps); V arrives as bf16 (widened exactly from FP8 by fa2_fp8_widen_kernel), so P V and
// everything after S are the bf16 path's. The K tile is stored like a bf16 tile of D/2
// elements (same bytes per row, same swizzle).
template <int D, int NW, bool FP8>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D, NW>::WPE, FwdCfg<D, NW>::WPE)))
void fa2_fwd_kernel(FwdParams p) {
  using C = FwdCfg<D, NW>;
  static_assert(!FP8 || D == 128, "the FP8 forward is built for head dim 128");
  constexpr int KROWB = FP8 ? D : 2 * D;      // bytes per Q / K row
  constexpr int KSS = FP8 ? D / 64 : C::KS;   // k-steps of S^T = K Q^T
  constexpr int KDE = FP8 ? D / 2 : D;        // K tile as a bf16 tile of KDE elements per row
  using kop_t = std::conditional_t<FP8, u32x8, u32x4>;
  // Two K and two V stages in separate arrays: a DMA into one array and LDS reads of another
  // are then provably independent, so reads never wait on an unrelated in-flight DMA.
  __shared__ __attribute__((aligned(1024))) char k_st0[C::BN * KROWB];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::BN * KROWB];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const int l32 = lane & 31;
  if constexpr (D == 256) agpr_accumulators_hint();  // O in AGPRs: one wave per SIMD

  constexpr int KP = fwd_pairs_per_wg(D, NW);
  int bh, j;
  map_block(blockIdx.x, p, KP, bh, j);
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const int N = p.N;
  auto block = [&](int qblk) __attribute__((always_inline)) {
  const int q0 = qblk * C::BM;
  const int qlo = q0 + wave * C::QPW;

  const uint32_t head_bytes = (uint32_t)N * C::ROWB;
  const uint32_t qk_head_bytes = (uint32_t)N * KROWB;
  const size_t qoff = (size_t)bh * N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + hkv) * (size_t)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.q + qoff * (KROWB / D), qk_head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)p.k + kvoff * (KROWB / D), qk_head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + kvoff, head_bytes);

  // Tiles are numbered from the workgroup's first visible tile tbase (a window hides the keys
  // before q0 - window). Counted from there: the workgroup's tiles, the tiles this wave
  // computes (causal: up to its last row), the leading tiles that cross the window's lower
  // edge for some row of this wave (masked), and the tiles wholly below its diagonal.
  const int W = p.window;
  const int tbase = q0 > W ? (q0 - W) / C::BN : 0;
  const int qend = min(q0 + C::BM, N);
  const int ntiles_abs = p.causal ? (qend + C::BN - 1) / C::BN : (N + C::BN - 1) / C::BN;
  const int nmine_abs = p.causal ? min(ntiles_abs, (qlo + C::QPW - 1) / C::BN + 1) : ntiles_abs;
  const int nfree_abs = min(nmine_abs, p.causal ? (qlo + 1) / C::BN : N / C::BN);
  const int ntiles = ntiles_abs - tbase;
  const int nmine = nmine_abs - tbase;
  const int nfree = max(0, nfree_abs - tbase);
  const int edge = qlo + C::QPW - 1 - W;  // keys below this fall outside some row's window
  const int nlead = edge > 0 ? max(0, (edge + C::BN - 1) / C::BN - tbase) : 0;

  // Tile t goes to stage t % 2: K two tiles ahead of its use, V one tile ahead. At d = 128,
  // tiles at and past ntiles (beyond the end of the head, where rows read as zero, or past the
  // causal range) are fetched anyway into stages nobody reads any more: without a branch
  // around the loads the step body stays one basic block the scheduler can interleave (3 %
  // faster). At d = 64 and 256 the branch stays: there the freed schedule spills registers.
  constexpr bool kFetchAlways = D == 128;
  auto fetch_k = [&](int t) {
    if (kFetchAlways || t < ntiles)
      load_tile<KDE, NW, false>(rk, (t & 1) ? (lds_char*)k_st1 : (lds_char*)k_st0, (tbase + t) * C::BN, wave, lane);
  };
  auto fetch_v = [&](int t) {
    if (kFetchAlways || t < ntiles)
      load_tile<D, NW, true>(rv, (t & 1) ? (lds_char*)v_st1 : (lds_char*)v_st0, (tbase + t) * C::BN, wave, lane);
  };

  // Q as the B operand of S^T = K Q^T: lane holds query l32 and, per k-step, the bytes of
  // head dims [16 ks + 8 hf, +8) (bf16) or [64 ks + 32 hf, +32) (FP8).
  kop_t qf[C::NQB][KSS];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const uint32_t row = (uint32_t)(qlo + qb * 32 + l32);
#pragma unroll
    for (int ks = 0; ks < KSS; ++ks) {
      if constexpr (FP8) {
        const u32x4 lo = buffer_load16(rq, row * KROWB + 64 * ks + 32 * hf) ^ p.qneg;
        const u32x4 hi = buffer_load16(rq, row * KROWB + 64 * ks + 32 * hf + 16) ^ p.qneg;
        qf[qb][ks] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        qf[qb][ks] = buffer_load16(rq, row * C::ROWB + (16 * ks + 8 * hf) * 2) ^ p.qneg;
      }
    }
  }
  fetch_k(0);
  fetch_v(0);
  fetch_k(1);

  // K A-operand: row l32 (+32 per key block), 16-byte chunks 2*ks + hf (bf16) or
  // 4*ks + 2*hf and the next one (FP8).
  constexpr int NKO = FP8 ? 2 * KSS : KSS;
  int koff[NKO];
#pragma unroll
  for (int i = 0; i < NKO; ++i) {
    const int chunk = FP8 ? 4 * (i >> 1) + 2 * hf + (i & 1) : 2 * i + hf;
    koff[i] = l32 * KROWB + ((chunk ^ swz_k<KDE>(l32)) << 4);
  }
  int voff[C::DB];  // V^T A-operand: transposing read base per 32-wide head-dim block
  {
    const int r = 4 * hf + ((lane & 15) >> 2);  // + 32*kb + 16*h (+8) leaves swz_v unchanged
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db] = r * C::ROWB + (((d >> 3) ^ swz_v<D>(r)) << 4) + (d & 7) * 2;
    }
  }

  f32x16 acc[C::NQB][C::DB];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[qb][db] = f32x16{};
  // Row sums relative to m, this lane's part: [0] of the fp32 p (for LSE), [1] of the bf16 P
  // that P V consumed (for normalising O). Normalising by the sum of the very weights applied
  // keeps O a convex combination of V rows: with the lazy reference the dominant p can be up
  // to 2^8, and its bf16 rounding would otherwise shift a nearly one-hot row by up to 2^-9 |O|.
  typedef float Sums[C::NQB][2];
  float m[C::NQB];        // reference (log2 domain) per query row, -inf before tile 0
  Sums l;
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    l[qb][0] = l[qb][1] = 0.f;
    m[qb] = -INFINITY;
  }
  const float c = p.c;

  // Scores of one tile: S^T blocks [qb][kb] of 32 keys x 32 queries.
  typedef f32x16 STile[C::NQB][2];
  // P^T of a tile as MFMA B operands [qb][kb][h] (16 keys x 32 queries, packed bf16), built in
  // place so the MFMAs read them without register copies.
  typedef u32x4 PTile[C::NQB][2][2];
  constexpr int NPV = 4 * C::DB;  // PV MFMA steps per tile (per query block)
  constexpr int MAX_SLICE = 32 / NPV;    // score elements max-reduced per PV step
  constexpr int EXP_PAIRS = 16 / KSS;    // exponential pairs formed per S k-step

  auto kread = [&](const lds_char* kt, int ks, int kb) -> kop_t {
    if constexpr (FP8) {
      const u32x4 lo = lds_read16(kt + koff[2 * ks] + kb * 32 * KROWB);
      const u32x4 hi = lds_read16(kt + koff[2 * ks + 1] + kb * 32 * KROWB);
      return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return lds_read16(kt + koff[ks] + kb * 32 * C::ROWB);
    }
  };
  auto mfma_s = [](kop_t a, kop_t b, f32x16 c) {
    if constexpr (FP8) return mfma32x32x64_fp8(a, b, c);
    else return mfma32x32x16(a, b, c);
  };
  // P V step i covers (kb, h, db) with db fastest, so consecutive MFMAs update different
  // accumulators.
  auto vread = [&](const lds_char* vt, int i) {
    const int db = i % C::DB, kb = i / (2 * C::DB), h = (i / C::DB) & 1;
    const lds_char* base = vt + voff[db] + (32 * kb + 16 * h) * C::ROWB;
    const u32x2 lo = lds_read8_tr(base);
    const u32x2 hi = lds_read8_tr(base + 8 * C::ROWB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // Pairs j0 .. j1-1: elements 2j, 2j+1 of a lane's 32 scores per query block (element
  // e = 16*kb + r). A row that has not met a visible key yet (possible under a window) still
  // has m = -inf; its masked scores then use reference 0 and give p = 0.
  auto exp_pairs = [&](STile& sc, PTile& pf, Sums& sum, int j0, int j1) {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        const int kb = j >> 3, r = (2 * j) & 15;
        const float mref = m[qb] == -INFINITY ? 0.f : m[qb];
        const float p0 = fast_exp2(__builtin_fmaf(sc[qb][kb][r], c, -mref));
        const float p1 = fast_exp2(__builtin_fmaf(sc[qb][kb][r + 1], c, -mref));
        const unsigned pk = pack_bf16(p0, p1);
        sum[qb][0] += p0 + p1;
        sum[qb][1] = add_bf16_pair(pk, sum[qb][1]);
        pf[qb][kb][r >> 3][(r >> 1) & 3] = pk;
      }
  };
  auto max_slice = [&](STile& sn, float (&mx)[C::NQB], int e0, bool mask, int j0) {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const int qi = qlo + qb * 32 + l32;
      const int lim = p.causal ? min(qi, N - 1) : N - 1;  // last visible key
      const int lo = qi - W;                              // first visible key
#pragma unroll
      for (int e = e0; e < e0 + MAX_SLICE; ++e) {
        const int kb = e >> 4, r = e & 15;
        if (mask) {
          const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          sn[qb][kb][r] = (key > lim || key < lo) ? -INFINITY : sn[qb][kb][r];
        }
        mx[qb] = fmaxf(mx[qb], sn[qb][kb][r]);
      }
    }
  };
  // One tile's MFMA stream: the S^T = K Q^T slots (k-step ks, key block kb; kb fastest) if
  // HAS_S, then the O^T += V^T P^T slots if HAS_PV. Every LDS operand is read LA slots ahead
  // of its MFMA from a ring of LA + 1 operands, so the reads of the P V phase start during the
  // last S slots. also_s(ks) and also_pv(i) are VALU work placed after the MFMAs of S k-step
  // ks and P V step i. Up to d = 128 the compiler's scheduler interleaves them (fences around
  // each slot measured 1-2 % slower); at d = 256 (one wave per SIMD) fences keep the slot
  // order, which measured 9 % faster there.
  auto mfma_stream = [&](auto has_s, auto has_pv, const lds_char* kt, STile& sn, const lds_char* vt,
                         PTile& pf, auto&& also_s, auto&& also_pv) __attribute__((always_inline)) {
    constexpr bool HAS_S = decltype(has_s)::value, HAS_PV = decltype(has_pv)::value;
    constexpr int LA = C::LA;
    constexpr int NSS = HAS_S ? 2 * KSS : 0;
    constexpr int NOP = NSS + (HAS_PV ? NPV : 0);
    kop_t kring[LA + 1];
    u32x4 vring[LA + 1];
    auto load = [&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j < NSS) kring[j % (LA + 1)] = kread(kt, j >> 1, j & 1);
      else vring[j % (LA + 1)] = vread(vt, j - NSS);
    };
    if constexpr (HAS_S) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sn[qb][kb] = f32x16{};
    }
    static_for<0, (LA < NOP ? LA : NOP)>(load);
    static_for<0, NOP>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j + LA < NOP) load(std::integral_constant<int, j + LA>{});
      // Keep this slot's LDS read ahead of the MFMAs that follow: left alone, the scheduler
      // sinks each read next to its MFMA (one slot ahead instead of LA), and every S MFMA then
      // waits out the LDS latency. VALU work may still move across.
      if constexpr (D == 128) __builtin_amdgcn_sched_barrier(kPinDsReadMfma);
      if constexpr (D == 256) __builtin_amdgcn_sched_barrier(0);
      if constexpr (j < NSS) {
        constexpr int ks = j >> 1, kb = j & 1;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) sn[qb][kb] = mfma_s(kring[j % (LA + 1)], qf[qb][ks], sn[qb][kb]);
        if constexpr (kb == 1) also_s(ks);
      } else {
        constexpr int i = j - NSS;
        constexpr int db = i % C::DB, kb = i / (2 * C::DB), h = (i / C::DB) & 1;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) acc[qb][db] = mfma32x32x16(vring[j % (LA + 1)], pf[qb][kb][h], acc[qb][db]);
        also_pv(i);
      }
      if constexpr (D == 256) __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto rescale_if_needed = [&](const float (&mx)[C::NQB]) {
    float mt[C::NQB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      mt[qb] = max_halves(mx[qb]) * c;
      grow |= mt[qb] > m[qb] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        const float mnew = fmaxf(m[qb], mt[qb]);
        // 0 when the row had no visible key before (m = -inf); 1 when its reference does not
        // move -- also for a row that still has none (m = mnew = -inf), which another row of
        // the wave brought into this branch.
        const float alpha = m[qb] == mnew ? 1.f : fast_exp2(m[qb] - mnew);
        m[qb] = mnew;
        l[qb][0] *= alpha;
        l[qb][1] *= alpha;
        // Scaled through a zero-operand MFMA: every definition of an accumulator is then an
        // MFMA result, and the allocator keeps one register home for it around this branch.
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          acc[qb][db] = mfma32x32x16(u32x4{}, u32x4{}, acc[qb][db] * alpha);
      }
    }
  };
  auto sync_stage = [&]() {
    wait_vmem_all();
    __syncthreads();
  };

  // Software pipeline over tiles with two score buffers. Step t (PAR = t % 2): fetch K(t+2)
  // and V(t+1); S(t+1) on the MFMA pipe while the VALU forms P(t) from S(t); PV(t) on the MFMA
  // pipe while the VALU masks and max-reduces S(t+1); raise the reference before P(t+1) if
  // the new max moved past the slack; one barrier.
  STile sbuf[2];
  auto step = [&](auto par_tag, auto mask_tag, int t) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr bool MASK_NEXT = decltype(mask_tag)::value;
    const lds_char* k_next = (const lds_char*)(PAR ? k_st0 : k_st1);
    const lds_char* v_cur = (const lds_char*)(PAR ? v_st1 : v_st0);
    // 4-wave workgroups at d = 128 (two per CU, so two workgroups' waves share each SIMD): waves
    // 2 and 3 take precedence in the instruction arbitration during the S phase of each step,
    // the half that carries the exponentials. Measured 1-4.5 % faster at B4 H16 N1024-4096 and
    // under sliding windows, outputs bitwise identical; with 8-wave workgroups it measured
    // neutral, so those keep the default order (the older wave first).
    if (D == 128 && NW == 4 && wave >= NW / 2) __builtin_amdgcn_s_setprio(1);
    fetch_k(t + 2);
    fetch_v(t + 1);
    PTile pf;
    Sums sum;
    float mx[C::NQB];
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      sum[qb][0] = sum[qb][1] = 0.f;
      mx[qb] = -INFINITY;
    }
    mfma_stream(std::true_type{}, std::true_type{}, k_next, sbuf[PAR ^ 1], v_cur, pf,
                [&](int ks) { exp_pairs(sbuf[PAR], pf, sum, ks * EXP_PAIRS, (ks + 1) * EXP_PAIRS); },
                [&](int i) {
                  if (D == 128 && NW == 4 && i == 0) __builtin_amdgcn_s_setprio(0);
                  max_slice(sbuf[PAR ^ 1], mx, i * MAX_SLICE, MASK_NEXT, (tbase + t + 1) * C::BN);
                });
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      l[qb][0] += sum[qb][0];
      l[qb][1] += sum[qb][1];
    }
    rescale_if_needed(mx);
    sync_stage();
  };
  auto last_step = [&](auto par_tag, int t) {  // t = nmine - 1: no next tile to prepare
    constexpr int PAR = decltype(par_tag)::value;
    const lds_char* v_cur = (const lds_char*)(PAR ? v_st1 : v_st0);
    fetch_k(t + 2);
    fetch_v(t + 1);
    PTile pf;
    Sums sum;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) sum[qb][0] = sum[qb][1] = 0.f;
    exp_pairs(sbuf[PAR], pf, sum, 0, 16);
    mfma_stream(std::false_type{}, std::true_type{}, nullptr, sbuf[PAR], v_cur, pf, [](int) {}, [](int) {});
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      l[qb][0] += sum[qb][0];
      l[qb][1] += sum[qb][1];
    }
    sync_stage();
  };

  sync_stage();  // Q, K(0), V(0), K(1) have landed
  {
    float mx[C::NQB];
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) mx[qb] = -INFINITY;
    PTile unused;
    mfma_stream(std::true_type{}, std::false_type{}, (const lds_char*)k_st0, sbuf[0], nullptr, unused,
                [](int) {}, [](int) {});
    for (int i = 0; i < NPV; ++i) max_slice(sbuf[0], mx, i * MAX_SLICE, nfree == 0 || nlead > 0, tbase * C::BN);
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) m[qb] = -INFINITY;
    rescale_if_needed(mx);  // sets the first reference; O and l are still zero
  }
  // Step 0 refills K(0)'s stage with K(2): every wave must be done reading K(0) first.
  __syncthreads();
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // Steps run in pairs (stage 0, then stage 1) so each step names its arrays statically and no
  // branch merges the accumulators. Step t masks tile t+1: unmasked steps are those with
  // nlead <= t + 1 < nfree; masking an unmasked tile is merely slower, so the counts are
  // rounded to pairs (the window's leading masked steps up, the unmasked ones down).
  int t = 0;
  const int lead_steps = nlead & ~1;
  for (; t < lead_steps && t + 2 < nmine; t += 2) {
    step(P0{}, std::true_type{}, t);
    step(P1{}, std::true_type{}, t + 1);
  }
  const int nfree_steps = nfree > 0 ? ((nfree - 1) & ~1) : 0;
  for (; t < nfree_steps; t += 2) {
    step(P0{}, std::false_type{}, t);
    step(P1{}, std::false_type{}, t + 1);
  }
  for (; t + 2 < nmine; t += 2) {
    step(P0{}, std::true_type{}, t);
    step(P1{}, std::true_type{}, t + 1);
  }
  // One or two steps remain (t even): t = nmine - 1, or t = nmine - 2 then t = nmine - 1.
  if (t + 1 < nmine) {
    step(P0{}, std::true_type{}, t);
    last_step(P1{}, t + 1);
  } else {
    last_step(P0{}, t);
  }
  t = nmine;
  for (; t < ntiles; ++t) {  // tiles above this wave's rows: keep the shared fetch cadence
    fetch_k(t + 2);
    fetch_v(t + 1);
    sync_stage();
  }

  // ---- epilogue: O = acc / (sum of the bf16 P), LSE = (m + log2 l) ln 2 ----
  // A lane holds O for one row (l32) in 16-byte pieces 32 bytes apart, so storing it directly
  // writes 32 bytes per row per instruction. Instead each wave passes its 32 x D tile through
  // its own part of the K/V stages (idle after the last barrier; each wave touches only its
  // part, so no barrier is needed) in column chunks, and stores whole 128-byte lines: the
  // epilogue measured 3x shorter with line-sized stores.
  static_assert(C::NQB == 1, "one 32-row block per wave");
  constexpr int SUB = NW / 4;                         // waves sharing one stage array
  constexpr int REG = C::BN * KROWB / SUB;            // bytes of LDS per wave
  constexpr int CW = REG / 128 < D ? REG / 128 : D;   // columns per chunk (32 rows x CW fp32)
  constexpr int UPR = CW / 4;                         // 16-byte units per chunk row
  static_assert(CW % 32 == 0 && D % CW == 0 && (UPR & (UPR - 1)) == 0, "chunk shape");
  {
    // From d = 128 up the lane index is made opaque here so that the chunk addresses below are
    // computed in the epilogue, not hoisted to the kernel start where they would stay live
    // across the tile loop (which then spilled 30 registers and ran 9 % slower). At d = 64
    // the hoisted form fits and measured faster.
    int el = lane;
    if constexpr (D >= 128) asm volatile("" : "+v"(el));
    const int e32 = el & 31, ehf = el >> 5;
    const float lt = sum_halves(l[0][0]);
    const float inv = p.vmul / sum_halves(l[0][1]);
    const int arr = wave / SUB;
    lds_char* reg = (arr == 0 ? (lds_char*)k_st0 : arr == 1 ? (lds_char*)k_st1
                    : arr == 2 ? (lds_char*)v_st0 : (lds_char*)v_st1) + (wave % SUB) * REG;
    float* obase = p.o + qoff + (size_t)qlo * D;
#pragma unroll
    for (int c = 0; c < D / CW; ++c) {
#pragma unroll
      for (int dbc = 0; dbc < CW / 32; ++dbc)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int db = c * (CW / 32) + dbc;
          const f32x4 val = {acc[0][db][4 * rq] * inv, acc[0][db][4 * rq + 1] * inv,
                             acc[0][db][4 * rq + 2] * inv, acc[0][db][4 * rq + 3] * inv};
          const int cu = 8 * dbc + 2 * rq + ehf;
          *(FA2_LDS f32x4*)(reg + e32 * (UPR * 16) + ((cu ^ (e32 & (UPR - 1))) << 4)) = val;
        }
#pragma unroll
      for (int k = 0; k < UPR / 2; ++k) {
        const int u = 64 * k + el, r = u / UPR, cu = u % UPR;
        const f32x4 val = *(const FA2_LDS f32x4*)(reg + r * (UPR * 16) + ((cu ^ (r & (UPR - 1))) << 4));
        if (qlo + r < N) *(f32x4*)(obase + (size_t)r * D + c * CW + 4 * cu) = val;
      }
    }
    const int row = qlo + l32;
    if (row < N && hf == 0) p.lse[(size_t)bh * N + row] = (m[0] + __log2f(lt)) * kLn2;
  }
  };
  if constexpr (KP == 0) {
    block(p.causal ? p.nqb - 1 - j : j);  // causal: longest rows first
  } else {
    // Rank the blocks of the head by length (causal: longest first) and cut the ranking into
    // 2 KP runs of nw. Block i of workgroup j is number j of run i, counted from the front in
    // even runs and from the back in odd ones, so the lengths of each workgroup's blocks add up
    // to the same total. All workgroups of a head start their even-run blocks together, and
    // every block starts on the head's first key tile, so they read the same K/V tiles at
    // nearly the same time and share them through L2: against mirrored pairs (block p, then
    // nqb - 1 - p), 32 % less HBM fetch at causal B2 H32 N8192 (1.21 against 1.79 GB).
    const int nw = fwd_work_items(p.nqb, KP);
    for (int i = 0; i < 2 * KP; ++i) {
      const int rank = i * nw + (i & 1 ? nw - 1 - j : j);
      if (rank >= p.nqb) continue;
      const int qblk = p.causal ? p.nqb - 1 - rank : rank;
      if (i) __syncthreads();  // every wave is past its last reads of the previous block's tiles
      block(qblk);
    }
  }
}

// Forward at head dim 256 without a sliding window: split roles on each SIMD. A 32-row block's O
// (128 fp32 registers) does not fit beside Q and two score tiles in one of two waves per SIMD, so
// the general kernel runs one wave per SIMD at d = 256. Here the two waves of a SIMD share 32 rows
// instead: A waves (0-3) keep Q and do S^T = K Q^T, the online softmax, P, and O^T over head-dim
// columns [0, D/2); B waves (4-7; B wave 4 + k shares A wave k's SIMD) take P from LDS one tile
// later, accumulate O^T over [D/2, D), apply the rescale factors A leaves beside P whenever its
// reference moves, and issue every K/V tile load. 32-key tiles: K in two stages, V in three (the
// B wave reads V(t - 1) while A reads V(t) and V(t + 1) lands), P and the factors in two
// buffers, one barrier per tile. (Built for any head dim; at d = 128, where the general kernel
// already runs two symmetric waves per SIMD, it measured slower, so only d = 256 uses it.)
template <int D_>
struct SplitCfg {
  static constexpr int D = D_, BN = D == 256 ? 32 : 64, KB = BN / 32, BM = 128, ROWB = 2 * D;
  static constexpr int TILE = BN * ROWB;
  static constexpr int KS = D / 16, DB = D / 32;
  static constexpr int DBA = DB / 2, DBB = DB - DBA;  // head-dim blocks of A and of B
  static constexpr int PBW = KB * 2048;  // one A wave's P of a tile
};

// Keys [j0, j0 + BN) of one head into a swizzled LDS tile, split over the four B waves (w = 0-3).
template <int D, bool IS_V>
__device__ __forceinline__ void split_load_tile(__amdgpu_buffer_rsrc_t rs, lds_char* tile, int j0, int w,
                                                int lane) {
  using S_ = SplitCfg<D>;
  constexpr int LPW = S_::TILE / 1024 / 4;
#pragma unroll
  for (int t = 0; t < LPW; ++t) {
    const int blk = w * LPW + t;
    const int pos = blk * 1024 + lane * 16;
    const int r = pos / S_::ROWB;
    const int cp = (pos % S_::ROWB) / 16;
    const int c = cp ^ (IS_V ? swz_v<D>(r) : swz_k<D>(r));
    buffer_load16_lds(rs, tile + blk * 1024, (uint32_t)(j0 + r) * S_::ROWB + c * 16);
  }
}

template <int D_>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_split_kernel(FwdParams p) {
  using S_ = SplitCfg<D_>;
  constexpr int D = D_, KS = S_::KS, DBA = S_::DBA, DBB = S_::DBB, KB = S_::KB;
  __shared__ __attribute__((aligned(1024))) char k_st0[S_::TILE];
  __shared__ __attribute__((aligned(1024))) char k_st1[S_::TILE];
  __shared__ __attribute__((aligned(1024))) char v_st0[S_::TILE];
  __shared__ __attribute__((aligned(1024))) char v_st1[S_::TILE];
  __shared__ __attribute__((aligned(1024))) char v_st2[S_::TILE];
  __shared__ __attribute__((aligned(1024))) char p_buf0[4 * S_::PBW];
  __shared__ __attribute__((aligned(1024))) char p_buf1[4 * S_::PBW];
  __shared__ __attribute__((aligned(1024))) char ctl0[4 * 256];  // per A wave: alpha[32] (+128: flag)
  __shared__ __attribute__((aligned(1024))) char ctl1[4 * 256];
  __shared__ __attribute__((aligned(1024))) char inv_buf[4 * 128];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool awave = wave < 4;
  const int aw = wave & 3;  // the A wave whose rows this wave serves
  const int hf = lane >> 5, l32 = lane & 31;
  int bh, j;
  map_block(blockIdx.x, p, 0, bh, j);
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  const int N = p.N;
  const int qblk = p.causal ? p.nqb - 1 - j : j;
  const int q0 = qblk * S_::BM;
  const int qlo = q0 + aw * 32;
  const uint32_t head_bytes = (uint32_t)N * S_::ROWB;
  const size_t qoff = (size_t)bh * N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + hkv) * (size_t)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qoff, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + kvoff, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + kvoff, head_bytes);

  // Tiles: the workgroup's, and those this wave pair computes (causal: up to its last row).
  const int qend = min(q0 + S_::BM, N);
  const int ntiles = p.causal ? (qend + S_::BN - 1) / S_::BN : (N + S_::BN - 1) / S_::BN;
  const int nmine = p.causal ? min(ntiles, (qlo + 31) / S_::BN + 1) : ntiles;
  const int nfree = min(nmine, p.causal ? (qlo + 1) / S_::BN : N / S_::BN);

  auto kst = [&](int t) { return (lds_char*)((t & 1) ? k_st1 : k_st0); };
  auto vst_rt = [&](int t) { const int s = t % 3; return (lds_char*)(s == 0 ? v_st0 : s == 1 ? v_st1 : v_st2); };
  auto fetch_k = [&](int t) { split_load_tile<D, false>(rk, kst(t), t * S_::BN, wave - 4, lane); };
  auto fetch_v = [&](int t) { split_load_tile<D, true>(rv, vst_rt(t), t * S_::BN, wave - 4, lane); };

  int voff[S_::DB];
  {
    const int r = 4 * hf + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < S_::DB; ++db) {
      const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db] = r * S_::ROWB + (((d >> 3) ^ swz_v<D>(r)) << 4) + (d & 7) * 2;
    }
  }
  // P V operand i of a tile over nb head-dim blocks from dbase (A: blocks [0, DBA), B: [DBA, DB)):
  // 2 KB nb MFMA steps, i = (kb, h, block) with the block fastest.
  auto vread = [&](const lds_char* vt, int i, int dbase, int nb) {
    const int db = dbase + i % nb, kb = i / (2 * nb), h = (i / nb) & 1;
    const lds_char* base = vt + voff[db] + (32 * kb + 16 * h) * S_::ROWB;
    const u32x2 lo = lds_read8_tr(base);
    const u32x2 hi = lds_read8_tr(base + 8 * S_::ROWB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  typedef u32x4 PTile[KB][2];  // [kb][h]

  // Epilogue: this wave's 32 rows x (32 nb) columns of O (from head-dim block db0), staged in its
  // own 8 KB of the K/V stages (every load has landed and every wave is past its last read).
  auto store_o = [&](auto& acc, int db0) __attribute__((always_inline)) {
    constexpr int NB = sizeof(acc) / sizeof(acc[0]);
    int el = lane;
    asm volatile("" : "+v"(el));
    const int e32 = el & 31, ehf = el >> 5;
    const float inv = *(const FA2_LDS float*)((lds_char*)inv_buf + aw * 128 + e32 * 4);
    constexpr int CW = 64, UPR = CW / 4;
    lds_char* reg = (lds_char*)(wave < 2 ? k_st0 : wave < 4 ? k_st1 : wave < 6 ? v_st0 : v_st1) + (wave & 1) * 8192;
    static_assert(S_::TILE >= 16384, "two 8 KB regions per stage");
    const int dbase = 32 * db0;
    float* obase = p.o + qoff + (size_t)qlo * D + dbase;
#pragma unroll
    for (int c = 0; c < NB / 2; ++c) {
#pragma unroll
      for (int dbc = 0; dbc < 2; ++dbc)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int db = 2 * c + dbc;
          const f32x4 val = {acc[db][4 * rq] * inv, acc[db][4 * rq + 1] * inv, acc[db][4 * rq + 2] * inv,
                             acc[db][4 * rq + 3] * inv};
          const int cu = 8 * dbc + 2 * rq + ehf;
          *(FA2_LDS f32x4*)(reg + e32 * (UPR * 16) + ((cu ^ (e32 & (UPR - 1))) << 4)) = val;
        }
#pragma unroll
      for (int k = 0; k < UPR / 2; ++k) {
        const int u = 64 * k + el, r = u / UPR, cu = u % UPR;
        const f32x4 val = *(const FA2_LDS f32x4*)(reg + r * (UPR * 16) + ((cu ^ (r & (UPR - 1))) << 4));
        if (qlo + r < N) *(f32x4*)(obase + (size_t)r * D + c * CW + 4 * cu) = val;
      }
    }
  };

  if (!awave) {
    // ---------------- B wave ----------------
    f32x16 acc[DBB];
#pragma unroll
    for (int i = 0; i < DBB; ++i) acc[i] = f32x16{};
    fetch_k(0);
    fetch_v(0);
    fetch_k(1);
    wait_vmem_all();
    __syncthreads();  // prologue: Q, K(0), V(0), K(1) landed
    __syncthreads();  // A waves' first S done; K(0)'s stage may be refilled
    for (int t = 0; t <= ntiles; ++t) {
      fetch_k(t + 2);
      fetch_v(t + 1);
      const int u = t - 1;  // tile whose P this step consumes
      if (u >= 0 && u < nmine) {
        const lds_char* pb = (const lds_char*)((u & 1) ? p_buf1 : p_buf0);
        PTile pf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) pf[kb][h] = lds_read16(pb + aw * S_::PBW + (2 * kb + h) * 1024 + lane * 16);
        const lds_char* vt = vst_rt(u);
        constexpr int NPV = 2 * KB * DBB;
        u32x4 vr[NPV];
#pragma unroll
        for (int i = 0; i < NPV; ++i) vr[i] = vread(vt, i, DBA, DBB);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int kb = i / (2 * DBB), h = (i / DBB) & 1;
          acc[i % DBB] = mfma32x32x16(vr[i], pf[kb][h], acc[i % DBB]);
        }
        const lds_char* cb = (const lds_char*)((u & 1) ? ctl1 : ctl0);
        const unsigned flag = *(const FA2_LDS unsigned*)(cb + aw * 256 + 128);
        if (__builtin_amdgcn_readfirstlane(flag)) {
          const float alpha = *(const FA2_LDS float*)(cb + aw * 256 + l32 * 4);
#pragma unroll
          for (int i = 0; i < DBB; ++i) acc[i] = mfma32x32x16(u32x4{}, u32x4{}, acc[i] * alpha);
        }
      }
      wait_vmem_all();
      __syncthreads();
    }
    store_o(acc, DBA);
  } else {
    // ---------------- A wave ----------------
    f32x16 acc[DBA];
#pragma unroll
    for (int i = 0; i < DBA; ++i) acc[i] = f32x16{};
    u32x4 qf[KS];
    {
      const uint32_t row = (uint32_t)(qlo + l32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = buffer_load16(rq, row * S_::ROWB + (16 * ks + 8 * hf) * 2) ^ p.qneg;
    }
    constexpr int NKO = KS < 8 ? KS : 8;  // chunks 16 and up: the same offsets + 256 bytes
    int koff[NKO];
#pragma unroll
    for (int i = 0; i < NKO; ++i) koff[i] = l32 * S_::ROWB + (((2 * i + hf) ^ swz_k<D>(l32)) << 4);
    float m = -INFINITY, l0 = 0.f, l1 = 0.f;
    const float c = p.c;
    typedef f32x16 STile[KB];
    auto exp_pairs = [&](STile& sc, PTile& pf, float& s0, float& s1, int j0, int j1) {
#pragma unroll
      for (int jj = j0; jj < j1; ++jj) {
        const int kb = jj >> 3, r = (2 * jj) & 15;
        const float mref = m == -INFINITY ? 0.f : m;
        const float p0 = fast_exp2(__builtin_fmaf(sc[kb][r], c, -mref));
        const float p1 = fast_exp2(__builtin_fmaf(sc[kb][r + 1], c, -mref));
        const unsigned pk = pack_bf16(p0, p1);
        s0 += p0 + p1;
        s1 = add_bf16_pair(pk, s1);
        pf[kb][r >> 3][(r >> 1) & 3] = pk;
      }
    };
    auto max_slice = [&](STile& sn, float& mx, int e0, int ne, bool mask, int j0) {
      const int qi = qlo + l32;
      const int lim = p.causal ? min(qi, N - 1) : N - 1;
#pragma unroll
      for (int e = e0; e < e0 + ne; ++e) {
        const int kb = e >> 4, r = e & 15;
        if (mask) {
          const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * hf + (r & 3);
          sn[kb][r] = key > lim ? -INFINITY : sn[kb][r];
        }
        mx = fmaxf(mx, sn[kb][r]);
      }
    };
    // One tile's stream: S^T = K Q^T slots (16) if HAS_S, then P V slots (8) if HAS_PV.
    auto stream = [&](auto has_s, auto has_pv, const lds_char* kt, STile& sn, const lds_char* vt,
                      PTile& pf, auto&& also_s, auto&& also_pv) __attribute__((always_inline)) {
      constexpr bool HS = decltype(has_s)::value, HP = decltype(has_pv)::value;
      constexpr int LA = 3, NSS = HS ? KB * KS : 0, NOP = NSS + (HP ? 2 * KB * DBA : 0);
      u32x4 ring[LA + 1];
      auto load = [&](auto J) __attribute__((always_inline)) {
        constexpr int jj = decltype(J)::value;
        if constexpr (jj < NSS) {
          constexpr int ks = jj / KB, kb = jj % KB;
          ring[jj % (LA + 1)] = lds_read16(kt + koff[ks % NKO] + (ks / NKO) * 256 + kb * 32 * S_::ROWB);
        }
        else ring[jj % (LA + 1)] = vread(vt, jj - NSS, 0, DBA);
      };
      if constexpr (HS) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sn[kb] = f32x16{};
      }
      static_for<0, (LA < NOP ? LA : NOP)>(load);
      static_for<0, NOP>([&](auto J) __attribute__((always_inline)) {
        constexpr int jj = decltype(J)::value;
        if constexpr (jj + LA < NOP) load(std::integral_constant<int, jj + LA>{});
        __builtin_amdgcn_sched_barrier(kPinDsReadMfma);
        if constexpr (jj < NSS) {
          constexpr int ks = jj / KB, kb = jj % KB;
          sn[kb] = mfma32x32x16(ring[jj % (LA + 1)], qf[ks], sn[kb]);
          if constexpr (kb == KB - 1) also_s(ks);
        } else {
          constexpr int i = jj - NSS, kb = i / (2 * DBA), h = (i / DBA) & 1;
          acc[i % DBA] = mfma32x32x16(ring[jj % (LA + 1)], pf[kb][h], acc[i % DBA]);
          also_pv(i);
        }
      });
    };
    auto rescale = [&](float mx, lds_char* cb) {
      const float mt = max_halves(mx) * c;
      const bool grow = mt > m + kRescaleSlack;
      const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
      if (any) {
        const float mnew = fmaxf(m, mt);
        const float alpha = m == mnew ? 1.f : fast_exp2(m - mnew);
        m = mnew;
        l0 *= alpha;
        l1 *= alpha;
#pragma unroll
        for (int i = 0; i < DBA; ++i) acc[i] = mfma32x32x16(u32x4{}, u32x4{}, acc[i] * alpha);
        if (hf == 0) *(FA2_LDS float*)(cb + aw * 256 + l32 * 4) = alpha;
      }
      if (lane == 0) *(FA2_LDS unsigned*)(cb + aw * 256 + 128) = any ? 1u : 0u;
    };
    auto store_p = [&](const PTile& pf, lds_char* pb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) *(FA2_LDS u32x4*)(pb + aw * S_::PBW + (2 * kb + h) * 1024 + lane * 16) = pf[kb][h];
    };
    STile sbuf[2];
    auto step = [&](auto par, auto mask_tag, int t) {
      constexpr int PAR = decltype(par)::value;
      constexpr bool MASK_NEXT = decltype(mask_tag)::value;
      PTile pf;
      float s0 = 0.f, s1 = 0.f, mx = -INFINITY;
      stream(std::true_type{}, std::true_type{}, (const lds_char*)kst(t + 1), sbuf[PAR ^ 1], (const lds_char*)vst_rt(t), pf,
             [&](int ks) {
               // 8 KB exponential pairs over the KS k-steps: EPN pairs every EPD steps
               constexpr int EPN = 8 * KB >= KS ? 8 * KB / KS : 1, EPD = 8 * KB >= KS ? 1 : KS / (8 * KB);
               if (ks % EPD == 0) exp_pairs(sbuf[PAR], pf, s0, s1, (ks / EPD) * EPN, (ks / EPD) * EPN + EPN);
               if (ks == KS - 1) store_p(pf, (lds_char*)(PAR ? p_buf1 : p_buf0));
             },
             [&](int i) {
               constexpr int MS = 16 * KB / (2 * KB * DBA);  // score elements max-reduced per P V step
               max_slice(sbuf[PAR ^ 1], mx, MS * i, MS, MASK_NEXT, (t + 1) * S_::BN);
             });
      l0 += s0;
      l1 += s1;
      rescale(mx, (lds_char*)(PAR ? ctl1 : ctl0));
      wait_vmem_all();
      __syncthreads();
    };
    auto last_step = [&](auto par, int t) {
      constexpr int PAR = decltype(par)::value;
      PTile pf;
      float s0 = 0.f, s1 = 0.f;
      exp_pairs(sbuf[PAR], pf, s0, s1, 0, 8 * KB);
      store_p(pf, (lds_char*)(PAR ? p_buf1 : p_buf0));
      if (lane == 0) *(FA2_LDS unsigned*)((lds_char*)(PAR ? ctl1 : ctl0) + aw * 256 + 128) = 0u;
      stream(std::false_type{}, std::true_type{}, nullptr, sbuf[PAR], (const lds_char*)vst_rt(t), pf, [](int) {}, [](int) {});
      l0 += s0;
      l1 += s1;
      wait_vmem_all();
      __syncthreads();
    };
    wait_vmem_all();
    __syncthreads();  // prologue loads landed
    {
      float mx = -INFINITY;
      PTile unused;
      stream(std::true_type{}, std::false_type{}, (const lds_char*)k_st0, sbuf[0], nullptr, unused, [](int) {}, [](int) {});
      max_slice(sbuf[0], mx, 0, 16 * KB, nfree == 0, 0);
      const float mt = max_halves(mx) * c;
      m = mt;  // first reference (O, l still zero)
    }
    __syncthreads();
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int t = 0;
    const int nfree_steps = nfree > 0 ? ((nfree - 1) & ~1) : 0;
    for (; t < nfree_steps; t += 2) {
      step(P0{}, std::false_type{}, t);
      step(P1{}, std::false_type{}, t + 1);
    }
    for (; t + 2 < nmine; t += 2) {
      step(P0{}, std::true_type{}, t);
      step(P1{}, std::true_type{}, t + 1);
    }
    if (t + 1 < nmine) {
      step(P0{}, std::true_type{}, t);
      last_step(P1{}, t + 1);
    } else {
      last_step(P0{}, t);
    }
    // 1 / (sum of the bf16 P) for the B wave, and this wave's LSE.
    const float lt = sum_halves(l0);
    const float inv = p.vmul / sum_halves(l1);
    if (hf == 0) *(FA2_LDS float*)((lds_char*)inv_buf + aw * 128 + l32 * 4) = inv;
    const int row = qlo + l32;
    if (row < N && hf == 0) p.lse[(size_t)bh * N + row] = (m + __log2f(lt)) * kLn2;
    for (t = nmine; t <= ntiles; ++t) {  // keep the barrier cadence of the B waves
      wait_vmem_all();
      __syncthreads();
    }
    store_o(acc, 0);
  }
}

// Waves per workgroup: 4 (128 query rows, several workgroups per CU, so that one's start-up --
// Q and the first K/V tiles -- and O stores overlap the others' tiles), or, at d = 128 only, 8
// (256 rows, fewer K/V tile copies per row, four blocks per workgroup) where that measured
// faster: causal with N >= 2048 on grids of at least four 256-row blocks per CU (one full round
// of 8-wave workgroups; 6-9 % faster at B4 H16 N4096, B4 H32 N2048 and B1 Hq64 Hkv8 N4096,
// slower below either bound), non-causal with N > 4096 on grids of at least six per CU, and
// never under a window of 4096 keys or fewer, which makes each row's work as short as a short
// sequence's. d = 64 runs three 4-wave workgroups per CU and d = 256 one.
constexpr int kComputeUnits = 256;
static int forward_waves(const AttnShape& s) {
  if (s.d != 128 || (s.window >= 0 && s.window <= 4096)) return 4;
  const long wg8 = (long)s.B * s.Hq * ((s.N + 255) / 256);
  if (s.causal) return s.N >= 2048 && wg8 >= 4L * kComputeUnits ? 8 : 4;
  return s.N > 4096 && wg8 >= 6L * kComputeUnits ? 8 : 4;
}

static FwdParams forward_params(const void* q, const void* k, const void* v, float* o, float* lse,
                                const AttnShape& s, int nw) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.N = s.N;
  p.causal = s.causal;
  p.c = fabsf(s.scale) * kLog2e;
  p.qneg = s.scale < 0.f ? 0x80008000u : 0u;
  const int BM = 32 * nw;  // FwdCfg<D, nw>::BM
  p.nqb = (s.N + BM - 1) / BM;
  p.xcd_remap = ((s.B * s.Hq) % 8) == 0;
  p.window = kernel_window(s);
  p.vmul = 1.0f;
  return p;
}

template <int D, int NW, bool FP8>
static void launch_fwd_kernel(const FwdParams& p, const AttnShape& s, hipStream_t stream) {
  static_assert(32 * NW == FwdCfg<D, NW>::BM, "rows per workgroup");
  const dim3 grid((unsigned)(s.B * s.Hq * fwd_work_items(p.nqb, fwd_pairs_per_wg(D, NW))));
  hipLaunchKernelGGL((fa2_fwd_kernel<D, NW, FP8>), grid, dim3(NW * 64), 0, stream, p);
}

hipError_t launch_forward(const void* q, const void* k, const void* v, float* o, float* lse,
                          const AttnShape& s, hipStream_t stream) {
  if (s.d == 256 && kernel_window(s) == kNoWindow) {
    // 6-10 % faster than the one-wave-per-SIMD d = 256 configuration (same box, causal
    // B2 H16 N8192, B1 Hq32 Hkv8 N16384, B4 H16 N4096); that one stays for sliding windows.
    const FwdParams p = forward_params(q, k, v, o, lse, s, 4);  // 128-row blocks
    hipLaunchKernelGGL(fa2_fwd_split_kernel<256>, dim3((unsigned)(s.B * s.Hq * p.nqb)), dim3(512), 0,
                       stream, p);
    return hipGetLastError();
  }
  const int nw = forward_waves(s);
  const FwdParams p = forward_params(q, k, v, o, lse, s, nw);
  if (s.d == 256)
    launch_fwd_kernel<256, 4, false>(p, s, stream);
  else if (s.d == 128)
    nw == 8 ? launch_fwd_kernel<128, 8, false>(p, s, stream) : launch_fwd_kernel<128, 4, false>(p, s, stream);
  else
    launch_fwd_kernel<64, 4, false>(p, s, stream);
  return hipGetLastError();
}

// FP8 E4M3FN codes -> bf16, exactly (every E4M3FN value is a bf16 value): 16 codes per thread.
__global__ __launch_bounds__(256) void fa2_fp8_widen_kernel(const uint8_t* __restrict__ src,
                                                            uint16_t* __restrict__ dst, long n16) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 w = *(const u32x4*)(src + i * 16);
  u32x4 out[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);  // codes 0, 1 of the word
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);   // codes 2, 3
    out[j >> 1][2 * (j & 1)] = pack_bf16(lo[0], lo[1]);
    out[j >> 1][2 * (j & 1) + 1] = pack_bf16(hi[0], hi[1]);
  }
  *(u32x4*)(dst + i * 16) = out[0];
  *(u32x4*)(dst + i * 16 + 8) = out[1];
}

size_t forward_fp8_workspace_bytes(const AttnShape& s) {
  const size_t bytes = (size_t)s.B * s.Hkv * s.N * s.d * 2;
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_forward_fp8(const void* q8, const void* k8, const void* v8, float q_scale,
                              float k_scale, float v_scale, float* o, float* lse,
                              const AttnShape& s, void* ws, hipStream_t stream) {
  const long n16 = (long)s.B * s.Hkv * s.N * s.d / 16;
  hipLaunchKernelGGL(fa2_fp8_widen_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(v8), static_cast<uint16_t*>(ws), n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nw = forward_waves(s);
  FwdParams p = forward_params(q8, k8, ws, o, lse, s, nw);
  p.c = fabsf(s.scale) * q_scale * k_scale * kLog2e;
  p.qneg = s.scale < 0.f ? 0x80808080u : 0u;
  p.vmul = v_scale;
  nw == 8 ? launch_fwd_kernel<128, 8, true>(p, s, stream) : launch_fwd_kernel<128, 4, true>(p, s, stream);
  return hipGetLastError();
}

}  // namespace fa2

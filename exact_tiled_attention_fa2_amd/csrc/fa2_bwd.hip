// fa2_bwd.hip -- exact attention backward for gfx950: dQ, dK, dV from Q, K, V, O, LSE, dO.
//
// Method (FlashAttention-2 pages: "Flash Attention spiegata: una guida completa", datacamp,
// section "Ricomputazione"): the probabilities are recomputed tile by tile from the saved
// per-row logsumexp, P_ij = exp(scale <q_i,k_j> - LSE_i), instead of being read back from
// a stored N x N matrix. The gradients are the chain rule of the standard definition:
//   dV_j = sum_i P_ij dO_i,  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  D_i = <dO_i, O_i>.
// Three kernels, none with atomics (the result is deterministic, as the wiki article
// "FlashAttention-2" stresses in its performance section); the full backward runs dQ in the
// form that does step 1 for its own rows, then dK/dV:
//   1. preprocess   D_i = sum_c dO_ic O_ic                   (one value per query row)
//   2. dK/dV        per (batch, KV head) 128-key blocks, each walking every query tile of
//                   every query head sharing the KV head: four pairs of waves, one pair per
//                   32 keys; the first keeps K and makes P and dV, the second keeps V and
//                   makes dS and dK from the P its partner leaves in LDS. A workgroup takes
//                   one block, or four blocks (one from each quarter of the blocks sorted by
//                   length) without grouped-query heads. Head dim 256: 64-key blocks, a quad
//                   of waves per 32 keys (S and dP computed once, dV and dK split by head-dim
//                   half, P and dS handed over through LDS).
//   3. dQ           per (batch, query head) query blocks; each wave keeps its 32 queries' Q,
//                   dO and fp32 dQ^T in registers and walks the key tiles (eight waves, two
//                   per SIMD; four at head dim 256). A workgroup takes a mirrored pair of
//                   blocks (two pairs at head dim 256).
// Q/dO (dK/dV kernels) and K/V (dQ kernel) tiles stream into LDS by buffer_load ... lds, in
// two or three stages, in a layout that serves both 16-byte row reads and the transposing
// ds_read_b64_tr_b16 reads without bank conflicts.
#include <type_traits>

#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // -D, [B,Hq,N]
  float* lse2;   // LSE * log2(e), [B,Hq,N]
  const float* o;    // forward output and logsumexp: read by the dQ kernel that also does the
  const float* lse;  // preprocess (else unused)
  int B, Hq, Hkv, N;
  int causal;
  float c;        // |scale| * log2(e)
  float scale;    // signed scale, applied to dQ and dK
  unsigned kneg;  // sign flip applied to the register-resident score operand when scale < 0
  int nblk;       // key blocks (dK/dV) or query blocks (dQ) per head
  int window;     // causal window: query i sees keys i - window .. i (>= N: no window)
};

// Shared by the dK/dV and dQ kernels: 64-row tiles of bf16 rows, read as 16-byte rows and by
// transposing reads.
template <int D>
struct BwdCfg {
  static constexpr int WAVES = 4;           // waves the tile loader splits a tile over by default
  static constexpr int BR = 128;            // keys per dK/dV workgroup
  static constexpr int BT = 64;             // rows per streamed tile
  static constexpr int KS = D / 16;         // k-steps of a contraction over the head dim
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = BT * ROWB;
  static constexpr int RO = KS < 8 ? KS : 8;  // distinct row-read offsets (chunks 16+ add 256 B)
};

// One swizzle for tiles read both as 16-byte rows (16 consecutive rows, one chunk) and by
// transposing reads (4 consecutive rows x 4 consecutive chunks per half-wave): chunk c of
// row r sits at c ^ swz(r); both access patterns then cover all 16 LDS bank groups. It only
// permutes the low four bits of the chunk index.
template <int D>
__device__ __forceinline__ int swz_dual(int r) {
  using S = SwzCfg<D>;
  constexpr int Q4 = S::SWZ_SPAN / 4;
  const int i = r / S::SWZ_ROWS;
  return ((i % Q4) << 2) | ((i / Q4) & 3);
}

template <int D, int NW = BwdCfg<D>::WAVES>
__device__ __forceinline__ void load_tile_dual(__amdgpu_buffer_rsrc_t rs, lds_char* tile, int row0,
                                               int wave, int lane) {
  using C = BwdCfg<D>;
  constexpr int LPW = C::TILE / 1024 / NW;  // 1 KB loads per wave
  static_assert(LPW * NW * 1024 == C::TILE, "tile not divisible among the waves");
#pragma unroll
  for (int t = 0; t < LPW; ++t) {
    const int blk = wave * LPW + t;
    const int pos = blk * 1024 + lane * 16;
    const int r = pos / C::ROWB;
    const int cp = (pos % C::ROWB) / 16;
    buffer_load16_lds(rs, tile + blk * 1024, (uint32_t)(row0 + r) * C::ROWB + ((cp ^ swz_dual<D>(r)) << 4));
  }
}

// 16-byte row read (A operand, rows 32*blk + l%32, head-dim chunk 2*ks + half).
template <int D>
__device__ __forceinline__ int row_read_off(int lane, int ks) {
  using C = BwdCfg<D>;
  const int r = lane & 31;  // + 32*blk leaves the swizzle unchanged
  return r * C::ROWB + (((2 * ks + (lane >> 5)) ^ swz_dual<D>(r)) << 4);
}

// Transposing read base (A operand = tile^T, head-dim block db) for tile rows
// 8*upper + 4*(l/32) + (l%16)/4; adding 32*blk + 16*h leaves the swizzle unchanged, adding 8
// does not, so the two reads of a fragment (rows +0 and +8) have separate bases.
template <int D>
__device__ __forceinline__ int tr_read_off(int lane, int db, int upper) {
  using C = BwdCfg<D>;
  const int r = 8 * upper + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return r * C::ROWB + (((d >> 3) ^ swz_dual<D>(r)) << 4) + (d & 7) * 2;
}

__device__ __forceinline__ u32x4 tr_pair(const lds_char* lo_base, const lds_char* hi_base) {
  const u32x2 lo = lds_read8_tr(lo_base);
  const u32x2 hi = lds_read8_tr(hi_base);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Block id -> (head slice, block within head). Workgroups are dealt round-robin to the 8 XCDs
// (bid & 7 is the XCD); when the slice count divides by 8, each XCD gets a contiguous range of
// slices and walks their blocks in order, so the blocks of one slice share that XCD's L2.
__device__ __forceinline__ void map_slice_block(int bid, int nslices, int nblk, int& slice, int& blk) {
  if ((nslices & 7) == 0) {
    const int x = bid & 7, s = bid >> 3;
    slice = x * (nslices >> 3) + s / nblk;
    blk = s % nblk;
  } else {
    slice = bid / nblk;
    blk = bid % nblk;
  }
}

// ------------------------------------------------------------------ 1. preprocess

// delta[i] = -D_i = -sum_c dO_ic O_ic, and lse2[i] = LSE_i * log2(e): the kernels below form
// P = 2^(s c - lse2) with one FMA and one exp2 per score, and start the dP accumulators from
// -D, so that an MFMA chain ends at dP - D.
template <int D>
__global__ __launch_bounds__(256) void fa2_bwd_pre_kernel(const float* __restrict__ o,
                                                          const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ delta,
                                                          float* __restrict__ lse2, long rows) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 g = *(const u32x4*)(dO + row * D + part * 8);
    const f32x4 a = *(const f32x4*)(o + row * D + part * 8);
    const f32x4 b = *(const f32x4*)(o + row * D + part * 8 + 4);
    acc = __uint_as_float(g[0] << 16) * a[0] + __uint_as_float(g[0] & 0xffff0000u) * a[1] +
          __uint_as_float(g[1] << 16) * a[2] + __uint_as_float(g[1] & 0xffff0000u) * a[3] +
          __uint_as_float(g[2] << 16) * b[0] + __uint_as_float(g[2] & 0xffff0000u) * b[1] +
          __uint_as_float(g[3] << 16) * b[2] + __uint_as_float(g[3] & 0xffff0000u) * b[3];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && part == 0) {
    delta[row] = -acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ------------------------------------------------------------------ 2. dK / dV, paired waves

// Work items (workgroups per slice) of the paired dK/dV kernel (head dims 64 and 128). Without
// grouped-query heads a workgroup takes 2 kDkdvPairs key blocks, which spreads its fixed
// start-up and wind-down over four blocks (2-4% faster than two on causal d=64 and d=128
// shapes); otherwise one key block each.
constexpr int kDkdvPairs = 2;
__host__ __device__ inline int dkdv_work_items(int nblk, int G) {
  return G == 1 ? ((nblk + 1) / 2 + kDkdvPairs - 1) / kDkdvPairs : nblk;
}
// Pairs of query blocks per dQ workgroup: two at head dim 256 (3% faster than one), one below,
// where a second pair measured no faster.
__host__ __device__ constexpr int dq_pairs(int d) { return d == 256 ? 2 : 1; }
__host__ __device__ inline int dq_work_items(int nblk, int d) {
  return ((nblk + 1) / 2 + dq_pairs(d) - 1) / dq_pairs(d);
}

// Eight waves, two per SIMD, in four pairs that each own 32 keys. Wave w
// (w < 4) keeps the keys' K and computes S = Q K^T, P = 2^(S c - lse2) and dV^T += dO^T P; it
// leaves P in LDS as packed bf16, in the MFMA operand layout. Its partner w + 4, on the same
// SIMD, keeps V and works one query tile behind: dP = dO V^T, dS = P (dP - D) from the P it
// reads back, dK^T += Q^T dS. The two halves are one MFMA sequence on one register set (K or
// V, dV^T or dK^T, S or dP, P or dS) with the row-read and transposed-read tiles swapped, so
// a wave holds half the state of a wave doing all four products: everything stays in VGPRs,
// and a SIMD runs the MFMAs of one wave beside the exponentials or dS arithmetic of the other.
// P enters dS rounded to bf16, the value the dV product consumed. Q/dO tiles (and -D, lse2)
// stream into LDS by buffer_load ... lds; rows past the end of the sequence need no mask:
// their Q, dO, -D and LSE read as zero, so P = 1 there but dO = 0 and dS = 1 * (0 + 0) = 0,
// and they add nothing to dV or dK.
template <int D>
struct PairCfg {
  static_assert(D <= 128, "head dim 256 runs the quad kernel below");
  static constexpr int WAVES = 8;
  static constexpr int PAIRS = 4;
  static constexpr int RPW = 32;             // keys per pair
  static constexpr int BR = PAIRS * RPW;     // keys per workgroup
  static constexpr int BT = 64;              // query rows per tile (two 32-row blocks)
  static constexpr int NMB = BT / 32;
  static constexpr int TILE = BT * 2 * D;
  static constexpr int DBP = D / 32;         // dK/dV head-dim blocks of a wave: all of them
  static constexpr int PBUF = PAIRS * NMB * 2048;  // one tile's P: [pair][row block][half][lane] x 16 B
  // The LDS statistics arrays come after the tiles and P buffers: reads reach them through a
  // base lowered by this much.
  static constexpr int STAT_BIAS = D == 128 ? 131072 : 65536;
  static_assert(BR == BwdCfg<D>::BR, "the key blocks of the launcher's grid");
};

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa2_bwd_dkdv_pair_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  using PC = PairCfg<D>;
  // Three stages (the P waves read tile s while their partners read tile s - 1 and tile s + 1
  // lands), each in separate arrays, and two P buffers. The compiler lays the 16 KB arrays out
  // as q0 q1 q2 do0 do1 do2 pbuf0 pbuf1, then the statistics: an LDS read reaches the tiles
  // below 64 KB through its immediate offset; the others get lane offsets raised by 64 KB
  // once per tile (tile below), the statistics a base lowered by 128 KB.
  __shared__ __attribute__((aligned(1024))) char t0_do0[PC::TILE];
  __shared__ __attribute__((aligned(1024))) char t1_do1[PC::TILE];
  __shared__ __attribute__((aligned(1024))) char t2_do2[PC::TILE];
  __shared__ __attribute__((aligned(1024))) char t3_q0[PC::TILE];
  __shared__ __attribute__((aligned(1024))) char t4_q1[PC::TILE];
  __shared__ __attribute__((aligned(1024))) char t5_q2[PC::TILE];
  __shared__ __attribute__((aligned(1024))) char t6_pbuf0[PC::PBUF];
  __shared__ __attribute__((aligned(1024))) char t7_pbuf1[PC::PBUF];
  __shared__ __attribute__((aligned(1024))) char stat_st0[2048];
  __shared__ __attribute__((aligned(1024))) char stat_st1[2048];
  __shared__ __attribute__((aligned(1024))) char stat_st2[2048];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave & 3;
  const bool pwave = wave < 4;  // keeps K and produces P (else keeps V and produces dS)
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = p.N;
  // Without grouped-query heads each workgroup takes four key blocks of one slice, one block
  // after the other (order below), which spreads the workgroups' start-up and wind-down costs
  // over four blocks (two blocks against one: 3 % at B2 H32 N8192, 8 % at B4 H16 N4096; four
  // another 1-3 %). With a group of query heads per block the work per block is long
  // already, and one block per workgroup keeps the blocks of a head walking the same query
  // tiles in step (two blocks measured 1-2 % slower).
  const int G = p.Hq / p.Hkv;
  const int nwork = dkdv_work_items(p.nblk, G);
  int bg, j;
  map_slice_block(blockIdx.x, p.B * p.Hkv, nwork, bg, j);
  const bool paired = G == 1;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  auto block = [&](int kblk) __attribute__((always_inline)) {
  const int k0 = kblk * PC::BR;
  const int kw = k0 + pair * PC::RPW;  // the pair's first key

  const uint32_t head_bytes = (uint32_t)N * C::ROWB;
  const size_t kvoff = ((size_t)b * p.Hkv + g) * (size_t)N * D;

  // Query tiles: every query head of the group, tiles from the one holding key k0 up to the
  // last one that sees a key of the block (the end, unless a window stops earlier), walked
  // from the TOP tile down, so all key blocks of a head start on the same tiles and read them
  // at about the same time (shared through L2 instead of each block from HBM).
  const int W = p.window;
  constexpr int BT = PC::BT, NMB = PC::NMB;
  const int nqt_all = (N + BT - 1) / BT;
  const int qt0 = p.causal ? k0 / BT : 0;
  const int qt_top = min(nqt_all - 1, (k0 + PC::BR - 1 + W) / BT);
  const int nqt = qt_top - qt0 + 1;
  const int iters = G * nqt;

  auto q_st = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    return (lds_char*)(s == 0 ? t3_q0 : s == 1 ? t4_q1 : t5_q2);
  };
  auto do_st = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    return (lds_char*)(s == 0 ? t0_do0 : s == 1 ? t1_do1 : t2_do2);
  };
  auto stat_st = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    return (lds_char*)(s == 0 ? stat_st0 : s == 1 ? stat_st1 : stat_st2);
  };
  // Tiles are numbered it = h nqt + u (query head g G + h, tile row (qt_top - u) BT); the
  // loops below step a (head, tile) cursor instead of dividing.
  struct Cursor {
    int h, u;
  };
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.u == nqt) {
      c.u = 0;
      ++c.h;
    }
  };
  // Lane part of the DMA offsets (row within the tile, swizzled chunk), fixed for the kernel:
  // [0] for this wave's 1 KB blocks of a tile, [1] for those of wave + 4.
  constexpr int LPW = PC::TILE / 1024 / PC::WAVES;
  uint32_t dma_off[2][LPW];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int pos = ((wave + 4 * h) * LPW + t) * 1024 + lane * 16;
      const int r = pos / C::ROWB;
      dma_off[h][t] = (uint32_t)(r * C::ROWB + ((((pos % C::ROWB) / 16) ^ swz_dual<D>(r)) << 4));
    }
  // Q/dO tile `it` and its statistics into stage S: this wave's blocks, and with BOTH also those
  // of wave + 4. Past the last tile (it >= iters) the loads read beyond the head's end (zeros)
  // into a stage no wave reads again, so no branch splits the step around them.
  auto fetch = [&](auto S, auto both, int it, const Cursor& cur) __attribute__((always_inline)) {
    constexpr int NH = decltype(both)::value ? 2 : 1;
    const bool live = it < iters;
    const int hq = g * G + (live ? cur.h : 0);
    const int qrow0 = live ? (qt_top - cur.u) * BT : N;
    const size_t qoff = ((size_t)b * p.Hq + hq) * (size_t)N * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dO + qoff, head_bytes);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int t = 0; t < LPW; ++t) {
        const uint32_t off = (uint32_t)qrow0 * C::ROWB + dma_off[h][t];
        buffer_load16_lds(rq, q_st(S) + ((wave + 4 * h) * LPW + t) * 1024, off);
        buffer_load16_lds(rd, do_st(S) + ((wave + 4 * h) * LPW + t) * 1024, off);
      }
    if (wave == 1 || wave == 2) {
      // -D (wave 1) or lse2 (wave 2) of the tile's BT rows; lanes past BT/4 - 1 read past the
      // end (zeros).
      const size_t roff = ((size_t)b * p.Hq + hq) * (size_t)N;
      const uint32_t off = lane < BT / 4 ? (uint32_t)(qrow0 + 4 * lane) * 4 : (uint32_t)N * 4;
      const float* src = wave == 1 ? p.delta : p.lse2;
      buffer_load16_lds(make_rsrc(src + roff, (uint32_t)N * 4), stat_st(S) + (wave - 1) * 1024, off);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  fetch(I0{}, std::false_type{}, 0, Cursor{0, 0});

  constexpr int KS = C::KS, DB = PC::DBP;
  int roff[C::RO], toff[DB], toff8[DB];
#pragma unroll
  for (int ks = 0; ks < C::RO; ++ks) roff[ks] = row_read_off<D>(lane, ks);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    toff[db] = tr_read_off<D>(lane, db, 0);
    toff8[db] = tr_read_off<D>(lane, db, 1);
  }

  const float c = p.c;
  const int key = kw + l32;

  // One query tile: NS MFMA steps, S or dP of the NMB row blocks (KS steps each), then
  // dV^T or dK^T over (row block, half, head-dim block). Operand reads run PF steps ahead.
  // The steps are placed in this order with no scheduling fences: the compiler interleaves
  // them as well (fences around each step measured the same within about 1 %; in the dQ
  // kernel they measured 1-3 % faster and stay).
  // The P or dS values of row block mb become readable DL steps after its last S or dP step
  // (ready) and are consumed from step use(mb, h) on: the first half's eight values are made
  // in [ready, use(mb, 0)), the second half's in [use(mb, 0), use(mb, 1)).
  constexpr int NS = NMB * KS + NMB * 2 * DB;
  constexpr int PF = 3;
  constexpr int DL = 2;
  auto use = [](int mb, int h) { return NMB * KS + (2 * mb + h) * DB; };
  auto first = [](int mb, int h) {  // first step forming values of (mb, h)
    const int ready = KS * (mb + 1) + DL, use0 = NMB * KS + 2 * mb * DB;
    return h == 0 ? (ready < use0 ? ready : use0 - 1) : use0;
  };
  // RH / TH: the row-read / transposed-read tile lies above the reach of a read's immediate
  // offset; its reads then use lane offsets raised by 64 KB once per tile (an opaque add, so
  // the compiler does not fold it back into one add per read).
  auto tile = [&](auto PW, auto RH, auto TH, const u32x4 (&kv)[KS], f32x16 (&acc)[DB],
                  const lds_char* rsrc, const lds_char* tsrc, const lds_char* stat, lds_char* pb,
                  int qrow0, bool fix) __attribute__((always_inline)) {
    constexpr bool PWAVE = decltype(PW)::value;
    constexpr int RB = decltype(RH)::value ? 65536 : 0, TB = decltype(TH)::value ? 65536 : 0;
    int ro[C::RO], to[DB], to8[DB];
#pragma unroll
    for (int k = 0; k < C::RO; ++k) ro[k] = RB ? opaque_add<RB>(roff[k]) : roff[k];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      to[db] = TB ? opaque_add<TB>(toff[db]) : toff[db];
      to8[db] = TB ? opaque_add<TB>(toff8[db]) : toff8[db];
    }
    const lds_char* rlo = rsrc - RB;
    const lds_char* tlo = tsrc - TB;
    f32x16 sd[NMB];        // S (P waves) or dP
    u32x4 op[NMB][2];      // [mb][h]: P or dS, 16 queries x 32 keys, packed bf16
    float pf[NMB][16];     // P in fp32 until packed (P waves)
    f32x4 st4[NMB][4];     // lse2 (P waves) or -D of the lane's rows
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) sd[mb] = f32x16{};
    constexpr int SB = PC::STAT_BIAS;
    const FA2_LDS float* sbase = (const FA2_LDS float*)(stat - SB + opaque_add<SB>(16 * hf));
    auto load_stats = [&](int mb) __attribute__((always_inline)) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) st4[mb][rq] = *(const FA2_LDS f32x4*)(sbase + 32 * mb + 8 * rq);
    };
    lds_char* pfrag = pb + pair * (NMB * 2048) + lane * 16;  // + (2 mb + h) KB
    // Zero P outside key <= query <= key + window for the eight rows of half h. Registers hold
    // query rows 32 mb + 8 (r / 4) + 4 hf + r % 4 of the tile; the row sees this lane's key iff
    // lo <= 32 mb + 8 (r / 4) + r % 4 <= lo + window, lo = key - qrow0 - 4 hf.
    auto causal_fixup = [&](int mb, int h) __attribute__((always_inline)) {
      const int lo = key - qrow0 - 4 * hf;
      const int hi = lo + W;
#pragma unroll
      for (int r = 8 * h; r < 8 * h + 8; r += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int x = 32 * mb + 8 * ((r + u) >> 2) + ((r + u) & 3);
          pf[mb][r + u] = (x >= lo && x <= hi) ? pf[mb][r + u] : 0.f;
        }
        op[mb][h][(r >> 1) & 3] = pack_bf16(pf[mb][r], pf[mb][r + 1]);
      }
    };
    auto values = [&](int mb, int h, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
      for (int e = e0; e < e1; e += 2) {
        const int r = 8 * h + e;
        if constexpr (PWAVE) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            pf[mb][r + u] = fast_exp2(__builtin_fmaf(sd[mb][r + u], c, -st4[mb][(r + u) >> 2][(r + u) & 3]));
          op[mb][h][(r >> 1) & 3] = pack_bf16(pf[mb][r], pf[mb][r + 1]);
        } else {
          // sd holds dP - D (its chain started from -D).
          const unsigned w = op[mb][h][(r >> 1) & 3];
          const float p0 = __uint_as_float(w << 16), p1 = __uint_as_float(w & 0xffff0000u);
          op[mb][h][(r >> 1) & 3] = pack_bf16(p0 * sd[mb][r], p1 * sd[mb][r + 1]);
        }
      }
    };
    auto read_op = [&](auto J) __attribute__((always_inline)) -> u32x4 {
      constexpr int j = decltype(J)::value;
      if constexpr (j < NMB * KS) {
        constexpr int ks = j % KS;
        return lds_read16(rlo + ro[ks % C::RO] + (ks / C::RO) * 256 + (j / KS) * 32 * C::ROWB);
      } else {
        constexpr int i = j - NMB * KS, db = i % DB, mb = i / (2 * DB), h = (i / DB) & 1;
        const int rowsel = (32 * mb + 16 * h) * C::ROWB;
        return tr_pair(tlo + to[db] + rowsel, tlo + to8[db] + rowsel);
      }
    };
    auto mfma_step = [&](auto J, u32x4 a) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j < NMB * KS) {
        constexpr int mb = j / KS;
        if constexpr (!PWAVE && j % KS == 0) {
          // dP chain of row block mb starts from -D (register r holds row 8 (r/4) + 4 hf + r%4).
          const f32x16 init = {st4[mb][0][0], st4[mb][0][1], st4[mb][0][2], st4[mb][0][3],
                               st4[mb][1][0], st4[mb][1][1], st4[mb][1][2], st4[mb][1][3],
                               st4[mb][2][0], st4[mb][2][1], st4[mb][2][2], st4[mb][2][3],
                               st4[mb][3][0], st4[mb][3][1], st4[mb][3][2], st4[mb][3][3]};
          sd[mb] = mfma32x32x16(a, kv[0], init);
        } else {
          sd[mb] = mfma32x32x16(a, kv[j % KS], sd[mb]);
        }
      } else {
        constexpr int i = j - NMB * KS, db = i % DB, mb = i / (2 * DB), h = (i / DB) & 1;
        acc[db] = mfma32x32x16(a, op[mb][h], acc[db]);
      }
    };
    auto valu_step = [&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j == 0) {
        if constexpr (PWAVE) {
          load_stats(0);
        } else {
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int h = 0; h < 2; ++h) op[mb][h] = lds_read16(pfrag + (2 * mb + h) * 1024);
        }
      }
      if constexpr (PWAVE && NMB > 1 && j == KS) load_stats(1);
      static_for<0, 2 * NMB>([&](auto MH) __attribute__((always_inline)) {
        constexpr int mb = decltype(MH)::value / 2, h = decltype(MH)::value % 2;
        constexpr int lo = first(mb, h), hi = use(mb, h), n = hi - lo;
        if constexpr (j >= lo && j < hi) {
          constexpr int e0 = 2 * ((4 * (j - lo)) / n), e1 = 2 * ((4 * (j - lo + 1)) / n);
          values(mb, h, e0, e1);
          if constexpr (PWAVE && j == hi - 1) {
            if (fix) causal_fixup(mb, h);
            *(FA2_LDS u32x4*)(pfrag + (2 * mb + h) * 1024) = op[mb][h];
          }
        }
      });
    };
    if constexpr (!PWAVE) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) load_stats(mb);  // -D initialises the dP chains
    }
    u32x4 ring[PF + 1];
    static_for<0, PF>([&](auto J) __attribute__((always_inline)) { ring[decltype(J)::value] = read_op(J); });
    static_for<0, NS>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j + PF < NS) ring[(j + PF) % (PF + 1)] = read_op(std::integral_constant<int, j + PF>{});
      mfma_step(J, ring[j % (PF + 1)]);
      valu_step(J);
    });
  };

  // Each role runs its own copy of the loop (the barriers match one to one: both run
  // iters + 1 steps), so the two register sets never meet at a branch merge.
  auto run = [&](auto PW) __attribute__((always_inline)) {
    constexpr bool PWAVE = decltype(PW)::value;
    // K (sign-flipped when scale < 0) or V of the pair's 32 keys as B operands.
    u32x4 kv[KS];
    {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc((PWAVE ? p.k : p.v) + kvoff, head_bytes);
      const unsigned flip = PWAVE ? p.kneg : 0u;
      const uint32_t row = (uint32_t)(kw + l32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[ks] = buffer_load16(rs, row * C::ROWB + (16 * ks + 8 * hf) * 2) ^ flip;
    }
    f32x16 acc[DB];  // dV^T or dK^T: rows = head dim, columns = keys (lanes)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

    // Step s: the P waves take tile s, their partners tile s - 1; tile s + 1 is fetched into
    // the third stage. The barrier at the end orders P(s) before its reads and frees stage
    // s - 1 for the next fetch.
    Cursor fc{0, 0}, tc{0, 0};  // the tile fetched next (s + 1) and the one this wave takes
    advance(fc);
    auto step = [&](auto S, int s) __attribute__((always_inline)) {
      constexpr int st = decltype(S)::value;
      using SN = std::integral_constant<int, (st + 1) % 3>;
      using SP = std::integral_constant<int, (st + 2) % 3>;
      // Only the P waves load the next tile, their blocks and their partners': a wave cannot
      // issue while the CU's vector-memory queue is full, and with all eight waves issuing their
      // loads at the start of a step each lost 300-450 cycles before its first MFMA. The P
      // waves finish their tile several hundred cycles before their partners and absorb it.
      if constexpr (PWAVE) fetch(SN{}, std::true_type{}, s + 1, fc);
      advance(fc);
      const int t = PWAVE ? s : s - 1;
      if (t >= 0 && t < iters) {
        const int qrow0 = (qt_top - tc.u) * BT;
        advance(tc);
        // Causal: skip tiles wholly above the pair's keys or past their window.
        const bool skip = (p.causal && qrow0 + BT - 1 < kw) || qrow0 > kw + PC::RPW - 1 + W;
        lds_char* pb = (lds_char*)((t & 1) ? t7_pbuf1 : t6_pbuf0);
        if (!skip) {
          // With 16 KB tiles, dO stages 1 and 2 lie at 64 KB and above.
          constexpr bool HI = PC::TILE == 16384;
          if constexpr (PWAVE) {
            const bool fix = (p.causal && qrow0 < kw + PC::RPW - 1) || qrow0 + BT - 1 > kw + W;
            tile(PW, std::false_type{}, std::bool_constant<HI && st != 0>{}, kv, acc, q_st(S),
                 do_st(S), stat_st(S) + 1024, pb, qrow0, fix);
          } else {
            tile(PW, std::bool_constant<HI && SP::value != 0>{}, std::false_type{}, kv, acc,
                 do_st(SP{}), q_st(SP{}), stat_st(SP{}), pb, qrow0, false);
          }
        }
      }
      wait_vmem_all();
      __syncthreads();
    };

    int s = 0;
    for (; s + 3 <= iters + 1; s += 3) {
      step(I0{}, s);
      step(I1{}, s + 1);
      step(I2{}, s + 2);
    }
    if (s <= iters) step(I0{}, s);
    if (s + 1 <= iters) step(I1{}, s + 1);

    // Store dV, or dK = scale dK^T^T: lane = key, registers = head dim (this pass's columns),
    // 16-byte pieces 32 bytes apart. After the last barrier every LDS array is idle: each wave
    // passes its 32 keys through its own array in column chunks and stores whole 128-byte lines
    // (no barrier needed; the next block's loads wait for one). The lane index is made opaque so
    // that the chunk addresses are formed here, not hoisted across the tile loop.
    {
      int el = lane;
      asm volatile("" : "+v"(el));
      const int e32 = el & 31, ehf = el >> 5;
      constexpr int REG = PC::TILE < PC::PBUF ? PC::TILE : PC::PBUF;  // bytes per wave
      constexpr int CW = REG / 128 < DB * 32 ? REG / 128 : DB * 32;      // columns per chunk
      constexpr int UPR = CW / 4;                                        // 16-byte units per row
      static_assert(CW % 32 == 0 && (DB * 32) % CW == 0 && (UPR & (UPR - 1)) == 0, "chunk shape");
      lds_char* reg = (lds_char*)(wave == 0 ? t0_do0 : wave == 1 ? t1_do1 : wave == 2 ? t2_do2
                                  : wave == 3 ? t3_q0 : wave == 4 ? t4_q1 : wave == 5 ? t5_q2
                                  : wave == 6 ? t6_pbuf0 : t7_pbuf1);
      float* base = (PWAVE ? p.dv : p.dk) + kvoff + (size_t)kw * D;
      const float f = PWAVE ? 1.f : p.scale;
#pragma unroll
      for (int c = 0; c < DB * 32 / CW; ++c) {
#pragma unroll
        for (int dbc = 0; dbc < CW / 32; ++dbc)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int db = c * (CW / 32) + dbc, cu = 8 * dbc + 2 * rq + ehf;
            *(FA2_LDS f32x4*)(reg + e32 * (UPR * 16) + ((cu ^ (e32 & (UPR - 1))) << 4)) =
                f32x4{acc[db][4 * rq], acc[db][4 * rq + 1], acc[db][4 * rq + 2], acc[db][4 * rq + 3]} * f;
          }
#pragma unroll
        for (int k = 0; k < UPR / 2; ++k) {
          const int u = 64 * k + el, r = u / UPR, cu = u % UPR;
          const f32x4 val = *(const FA2_LDS f32x4*)(reg + r * (UPR * 16) + ((cu ^ (r & (UPR - 1))) << 4));
          if (kw + r < N) *(f32x4*)(base + (size_t)r * D + c * CW + 4 * cu) = val;
        }
      }
    }
  };

  wait_vmem_all();
  __syncthreads();
  if (pwave)
    run(std::true_type{});
  else
    run(std::false_type{});
  };
  if (!paired) {
    block(j);
  } else {
    // Block i of workgroup j is number j of the i-th run of nwork blocks in length order
    // (causal: the longest key walks, the lowest blocks, first), counted from the back in odd
    // runs, so every workgroup carries the same total. Every block walks down from the head's
    // top query tile, and the workgroups of a slice start their even-run blocks together, so
    // they read the same Q/dO tiles at nearly the same time: against mirrored pairs (blocks j,
    // nblk - 1 - j), 32 % less HBM fetch at causal B2 H32 N8192 (0.95 against 1.40 GB).
    bool first = true;
    for (int i = 0; i < 2 * kDkdvPairs; ++i) {
      const int rank = i * nwork + (i & 1 ? nwork - 1 - j : j);
      if (rank >= p.nblk) continue;
      if (!first) __syncthreads();  // every wave is done with its stores' LDS staging
      first = false;
      block(rank);
    }
  }
}

// ------------------------------------------------------------------ 2b. dK/dV at head dim 256

// At head dim 256 a wave cannot hold both its keys' K (or V) and their whole dV (or dK) beside
// the rest, so the work of each 32 keys is split over a quad of waves by role and by half of the
// head dim, and S and dP are computed once:
//   A_P  (waves 0, 2): K; S = Q K^T, P = 2^(S c - lse2) -> LDS; dV^T[0:128) += dO^T P
//   A_DP (waves 1, 3): V; dP = dO V^T (from -D), dS = P (dP - D) with P from LDS -> LDS;
//                      dK^T[0:128) += Q^T dS
//   B_DV (waves 5, 7): dV^T[128:256) += dO^T P, P from LDS
//   B_DK (waves 4, 6): dK^T[128:256) += Q^T dS, dS from LDS
// Waves w and w + 4 share a SIMD, so each SIMD pairs an A role (24 MFMAs per 32-row query
// tile) with a B role (8), and a quad's four waves sit on two SIMDs. A_P takes tile s at step
// s, A_DP and B_DV tile s - 1, B_DK tile s - 2; Q/dO tiles stream through four stages
// (tile s + 1 lands while s, s - 1, s - 2 are read), P and dS through two buffers each; the
// B waves, with the least MFMA work, issue every load. One barrier per step.
struct QuadCfg {
  static constexpr int D = 256;
  static constexpr int WAVES = 8;
  static constexpr int RPW = 32;           // keys per quad
  static constexpr int BR = 2 * RPW;       // keys per workgroup
  static constexpr int BT = 32;            // query rows per tile
  static constexpr int ROWB = 2 * D;
  static constexpr int TILE = BT * ROWB;   // 16 KB of Q or dO
  static constexpr int KS = D / 16;        // k-steps of S or dP
  static constexpr int DB = 4;             // 32-wide head-dim blocks of a wave's dV or dK
  static constexpr int QBUF = 2 * 2048;    // one tile's P (or dS) of both quads
  static constexpr int LPW = TILE / 1024 / WAVES;  // 1 KB loads per slot of eight
};

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa2_bwd_dkdv_quad_kernel(BwdParams p) {
  using Q = QuadCfg;
  constexpr int D = Q::D, KS = Q::KS, DB = Q::DB, BT = Q::BT;
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char q_st0[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char q_st1[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char q_st2[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char q_st3[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char do_st0[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char do_st1[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char do_st2[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char do_st3[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char p_buf0[Q::QBUF];
  __shared__ __attribute__((aligned(1024))) char p_buf1[Q::QBUF];
  __shared__ __attribute__((aligned(1024))) char ds_buf0[Q::QBUF];
  __shared__ __attribute__((aligned(1024))) char ds_buf1[Q::QBUF];
  __shared__ __attribute__((aligned(1024))) char st_st0[2048];
  __shared__ __attribute__((aligned(1024))) char st_st1[2048];
  __shared__ __attribute__((aligned(1024))) char st_st2[2048];
  __shared__ __attribute__((aligned(1024))) char st_st3[2048];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int simd = wave & 3, quad = simd >> 1;
  const bool awave = wave < 4, odd = simd & 1;
  const int hf = lane >> 5, l32 = lane & 31;
  const int N = p.N;
  const int G = p.Hq / p.Hkv;
  int bg, kblk;
  map_slice_block(blockIdx.x, p.B * p.Hkv, p.nblk, bg, kblk);
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int k0 = kblk * Q::BR;
  const int kw = k0 + quad * Q::RPW;  // the quad's first key
  const uint32_t head_bytes = (uint32_t)N * Q::ROWB;
  const size_t kvoff = ((size_t)b * p.Hkv + g) * (size_t)N * D;

  // Query tiles as in the paired kernel: every query head of the group, from the top tile that
  // sees a key of the block down to the one holding key k0.
  const int W = p.window;
  const int nqt_all = (N + BT - 1) / BT;
  const int qt0 = p.causal ? k0 / BT : 0;
  const int qt_top = min(nqt_all - 1, (k0 + Q::BR - 1 + W) / BT);
  const int nqt = qt_top - qt0 + 1;
  const int iters = G * nqt;

  auto q_st = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value & 3;
    return (lds_char*)(s == 0 ? q_st0 : s == 1 ? q_st1 : s == 2 ? q_st2 : q_st3);
  };
  auto do_st = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value & 3;
    return (lds_char*)(s == 0 ? do_st0 : s == 1 ? do_st1 : s == 2 ? do_st2 : do_st3);
  };
  auto st_st = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value & 3;
    return (lds_char*)(s == 0 ? st_st0 : s == 1 ? st_st1 : s == 2 ? st_st2 : st_st3);
  };
  auto p_buf = [&](auto S) __attribute__((always_inline)) {
    return (lds_char*)((decltype(S)::value & 1) ? p_buf1 : p_buf0);
  };
  auto ds_buf = [&](auto S) __attribute__((always_inline)) {
    return (lds_char*)((decltype(S)::value & 1) ? ds_buf1 : ds_buf0);
  };
  struct Cursor {
    int h, u;
  };
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    if (++c.u == nqt) {
      c.u = 0;
      ++c.h;
    }
  };
  // DMA offsets of load slots `wave & 3` and `(wave & 3) + 4` (the slots this wave fills when it
  // loads a whole tile with another wave), and slot `wave` (the first tile, loaded by all).
  uint32_t dma_off[3][Q::LPW];
#pragma unroll
  for (int h = 0; h < 3; ++h)
#pragma unroll
    for (int t = 0; t < Q::LPW; ++t) {
      const int slot = h == 2 ? wave : (wave & 3) + 4 * h;
      const int pos = (slot * Q::LPW + t) * 1024 + lane * 16;
      const int r = pos / Q::ROWB;
      dma_off[h][t] = (uint32_t)(r * Q::ROWB + ((((pos % Q::ROWB) / 16) ^ swz_dual<D>(r)) << 4));
    }
  // Tile `it` into stage S: slots h in [H0, H1) of dma_off; -D by wave 5, lse2 by wave 6.
  auto fetch = [&](auto S, auto H0, auto H1, int it, const Cursor& cur) __attribute__((always_inline)) {
    const bool live = it < iters;
    const int hq = g * G + (live ? cur.h : 0);
    const int qrow0 = live ? (qt_top - cur.u) * BT : N;
    const size_t qoff = ((size_t)b * p.Hq + hq) * (size_t)N * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dO + qoff, head_bytes);
    static_for<decltype(H0)::value, decltype(H1)::value>([&](auto HH) __attribute__((always_inline)) {
      constexpr int h = decltype(HH)::value;
      const int slot = h == 2 ? wave : (wave & 3) + 4 * h;
#pragma unroll
      for (int t = 0; t < Q::LPW; ++t) {
        const uint32_t off = (uint32_t)qrow0 * Q::ROWB + dma_off[h][t];
        buffer_load16_lds(rq, q_st(S) + (slot * Q::LPW + t) * 1024, off);
        buffer_load16_lds(rd, do_st(S) + (slot * Q::LPW + t) * 1024, off);
      }
    });
    if (wave == 5 || wave == 6) {
      const size_t roff = ((size_t)b * p.Hq + hq) * (size_t)N;
      const uint32_t off = lane < BT / 4 ? (uint32_t)(qrow0 + 4 * lane) * 4 : (uint32_t)N * 4;
      const float* src = wave == 5 ? p.delta : p.lse2;
      buffer_load16_lds(make_rsrc(src + roff, (uint32_t)N * 4), st_st(S) + (wave - 5) * 1024, off);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  fetch(I0{}, I2{}, I3{}, 0, Cursor{0, 0});

  // A roles accumulate head-dim blocks 0-3, B roles 4-7.
  const int dh = awave ? 0 : 1;
  int roff[C::RO], toff[DB], toff8[DB];
#pragma unroll
  for (int ks = 0; ks < C::RO; ++ks) roff[ks] = row_read_off<D>(lane, ks);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    toff[db] = tr_read_off<D>(lane, dh * DB + db, 0);
    toff8[db] = tr_read_off<D>(lane, dh * DB + db, 1);
  }
  const float c = p.c;
  const int key = kw + l32;
  const int qslot = quad * 2048 + lane * 16;  // this lane's 16 bytes of a quad's P or dS (+ h KB)

  // A roles, one query tile: KS steps of S (or dP), then 2 DB steps of dV^T (or dK^T); P (or dS)
  // of half h is formed just before its first use, waiting on the last S or dP MFMA while the
  // B wave on the same SIMD keeps it busy.
  constexpr int NS = KS + 2 * DB;
  constexpr int PF = 3;
  auto tile_a = [&](auto PW, const u32x4 (&kv)[KS], f32x16 (&acc)[DB], const lds_char* rsrc,
                    const lds_char* tsrc, const lds_char* stat, lds_char* pin, lds_char* pout,
                    int qrow0, bool fix) __attribute__((always_inline)) {
    constexpr bool PWAVE = decltype(PW)::value;
    f32x16 sd = f32x16{};
    u32x4 op[2];
    float pf[16];
    f32x4 st4[4];
    const FA2_LDS float* sbase = (const FA2_LDS float*)(stat + 16 * hf);
    auto load_stats = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) st4[rq] = *(const FA2_LDS f32x4*)(sbase + 8 * rq);
    };
    auto causal_fixup = [&](int h) __attribute__((always_inline)) {
      const int lo = key - qrow0 - 4 * hf;
      const int hi = lo + W;
#pragma unroll
      for (int r = 8 * h; r < 8 * h + 8; r += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int x = 8 * ((r + u) >> 2) + ((r + u) & 3);
          pf[r + u] = (x >= lo && x <= hi) ? pf[r + u] : 0.f;
        }
        op[h][(r >> 1) & 3] = pack_bf16(pf[r], pf[r + 1]);
      }
    };
    auto values = [&](int h) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int r = 8 * h + e;
        if constexpr (PWAVE) {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            pf[r + u] = fast_exp2(__builtin_fmaf(sd[r + u], c, -st4[(r + u) >> 2][(r + u) & 3]));
          op[h][(r >> 1) & 3] = pack_bf16(pf[r], pf[r + 1]);
        } else {
          const unsigned w = op[h][(r >> 1) & 3];
          const float p0 = __uint_as_float(w << 16), p1 = __uint_as_float(w & 0xffff0000u);
          op[h][(r >> 1) & 3] = pack_bf16(p0 * sd[r], p1 * sd[r + 1]);
        }
      }
    };
    auto read_op = [&](auto J) __attribute__((always_inline)) -> u32x4 {
      constexpr int j = decltype(J)::value;
      if constexpr (j < KS) {
        return lds_read16(rsrc + roff[j % C::RO] + (j / C::RO) * 256);
      } else {
        constexpr int i = j - KS, db = i % DB, h = i / DB;
        return tr_pair(tsrc + toff[db] + 16 * h * Q::ROWB, tsrc + toff8[db] + 16 * h * Q::ROWB);
      }
    };
    load_stats();
    if constexpr (!PWAVE) {
#pragma unroll
      for (int h = 0; h < 2; ++h) op[h] = lds_read16(pin + qslot + h * 1024);
    }
    u32x4 ring[PF + 1];
    static_for<0, PF>([&](auto J) __attribute__((always_inline)) { ring[decltype(J)::value] = read_op(J); });
    static_for<0, NS>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j + PF < NS) ring[(j + PF) % (PF + 1)] = read_op(std::integral_constant<int, j + PF>{});
      if constexpr (j < KS) {
        if constexpr (!PWAVE && j == 0) {
          // The dP chain starts from -D (register r holds row 8 (r/4) + 4 hf + r%4).
          const f32x16 init = {st4[0][0], st4[0][1], st4[0][2], st4[0][3], st4[1][0], st4[1][1],
                               st4[1][2], st4[1][3], st4[2][0], st4[2][1], st4[2][2], st4[2][3],
                               st4[3][0], st4[3][1], st4[3][2], st4[3][3]};
          sd = mfma32x32x16(ring[j % (PF + 1)], kv[0], init);
        } else {
          sd = mfma32x32x16(ring[j % (PF + 1)], kv[j], sd);
        }
        if constexpr (j == KS - 1) {
          values(0);
          if constexpr (PWAVE) {
            if (fix) causal_fixup(0);
          }
          *(FA2_LDS u32x4*)(pout + qslot) = op[0];
        }
      } else {
        constexpr int i = j - KS, db = i % DB, h = i / DB;
        acc[db] = mfma32x32x16(ring[j % (PF + 1)], op[h], acc[db]);
        if constexpr (i < DB) {  // the second half's values beside the first half's MFMAs
          if constexpr (i == 0) values(1);
          if constexpr (i == DB - 1) {
            if constexpr (PWAVE) {
              if (fix) causal_fixup(1);
            }
            *(FA2_LDS u32x4*)(pout + qslot + 1024) = op[1];
          }
        }
      }
    });
  };
  // B roles, one query tile: 2 DB steps of dV^T (or dK^T) with P (or dS) from LDS.
  auto tile_b = [&](f32x16 (&acc)[DB], const lds_char* tsrc, const lds_char* pin) __attribute__((always_inline)) {
    u32x4 op[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) op[h] = lds_read16(pin + qslot + h * 1024);
    u32x4 ring[2 * DB];
    static_for<0, 2 * DB>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value, db = i % DB, h = i / DB;
      ring[i] = tr_pair(tsrc + toff[db] + 16 * h * Q::ROWB, tsrc + toff8[db] + 16 * h * Q::ROWB);
    });
    static_for<0, 2 * DB>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value, db = i % DB, h = i / DB;
      acc[db] = mfma32x32x16(ring[i], op[h], acc[db]);
    });
  };

  // ROLE: 0 A_P, 1 A_DP, 2 B_DV, 3 B_DK; each runs its own copy of the step loop, with the same
  // number of steps and barriers.
  auto run = [&](auto RL) __attribute__((always_inline)) {
    constexpr int ROLE = decltype(RL)::value;
    constexpr bool AROLE = ROLE < 2;
    constexpr int LAG = ROLE == 0 ? 0 : ROLE == 3 ? 2 : 1;
    u32x4 kv[AROLE ? KS : 1];
    if constexpr (AROLE) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc((ROLE == 0 ? p.k : p.v) + kvoff, head_bytes);
      const unsigned flip = ROLE == 0 ? p.kneg : 0u;
      const uint32_t row = (uint32_t)(kw + l32);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[ks] = buffer_load16(rs, row * Q::ROWB + (16 * ks + 8 * hf) * 2) ^ flip;
    }
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    Cursor fc{0, 0}, tc{0, 0};
    advance(fc);
    auto step = [&](auto S, int s) __attribute__((always_inline)) {
      constexpr int st = decltype(S)::value;
      using SN = std::integral_constant<int, (st + 1) & 3>;
      using ST = std::integral_constant<int, (st + 4 - LAG) & 3>;  // stage of this wave's tile
      if constexpr (!AROLE) fetch(SN{}, I0{}, I2{}, s + 1, fc);
      advance(fc);
      const int t = s - LAG;
      if (t >= 0 && t < iters) {
        const int qrow0 = (qt_top - tc.u) * BT;
        advance(tc);
        const bool skip = (p.causal && qrow0 + BT - 1 < kw) || qrow0 > kw + Q::RPW - 1 + W;
        if (!skip) {
          if constexpr (ROLE == 0) {
            const bool fix = (p.causal && qrow0 < kw + Q::RPW - 1) || qrow0 + BT - 1 > kw + W;
            tile_a(std::true_type{}, kv, acc, q_st(ST{}), do_st(ST{}), st_st(ST{}) + 1024, nullptr,
                   p_buf(ST{}), qrow0, fix);
          } else if constexpr (ROLE == 1) {
            tile_a(std::false_type{}, kv, acc, do_st(ST{}), q_st(ST{}), st_st(ST{}), p_buf(ST{}),
                   ds_buf(ST{}), qrow0, false);
          } else if constexpr (ROLE == 2) {
            tile_b(acc, do_st(ST{}), p_buf(ST{}));
          } else {
            tile_b(acc, q_st(ST{}), ds_buf(ST{}));
          }
        }
      }
      wait_vmem_all();
      __syncthreads();
    };
    const int nsteps = iters + 2;
    int s = 0;
    for (; s + 4 <= nsteps; s += 4) {
      step(I0{}, s);
      step(I1{}, s + 1);
      step(I2{}, s + 2);
      step(I3{}, s + 3);
    }
    if (s < nsteps) step(I0{}, s);
    if (s + 1 < nsteps) step(I1{}, s + 1);
    if (s + 2 < nsteps) step(I2{}, s + 2);

    // dV or dK = scale (dK^T)^T of this wave's 32 keys and 128 head-dim columns, staged through
    // its own 16 KB of the (now idle) Q/dO stages and stored in whole 128-byte lines.
    {
      int el = lane;
      asm volatile("" : "+v"(el));
      const int e32 = el & 31, ehf = el >> 5;
      constexpr int CW = DB * 32, UPR = CW / 4;
      lds_char* reg = (lds_char*)(wave == 0 ? q_st0 : wave == 1 ? q_st1 : wave == 2 ? q_st2
                                  : wave == 3 ? q_st3 : wave == 4 ? do_st0 : wave == 5 ? do_st1
                                  : wave == 6 ? do_st2 : do_st3);
      constexpr bool DV = ROLE == 0 || ROLE == 2;
      float* base = (DV ? p.dv : p.dk) + kvoff + (size_t)kw * D + dh * CW;
      const float f = DV ? 1.f : p.scale;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int cu = 8 * db + 2 * rq + ehf;
          *(FA2_LDS f32x4*)(reg + e32 * (UPR * 16) + ((cu ^ (e32 & (UPR - 1))) << 4)) =
              f32x4{acc[db][4 * rq], acc[db][4 * rq + 1], acc[db][4 * rq + 2], acc[db][4 * rq + 3]} * f;
        }
#pragma unroll
      for (int k = 0; k < UPR / 2; ++k) {
        const int u = 64 * k + el, r = u / UPR, cu = u % UPR;
        const f32x4 val = *(const FA2_LDS f32x4*)(reg + r * (UPR * 16) + ((cu ^ (r & (UPR - 1))) << 4));
        if (kw + r < N) *(f32x4*)(base + (size_t)r * D + 4 * cu) = val;
      }
    }
  };

  wait_vmem_all();
  __syncthreads();
  if (awave) {
    if (!odd) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    if (odd) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
  }
}

// ------------------------------------------------------------------ 3. dQ

template <int D, int NW = 4>
struct DqCfg {
  static constexpr int WAVES = NW;          // one (4) or two (8) waves per SIMD
  static constexpr int WPE = NW / 4;
  // Query rows per wave. Two waves per SIMD (head dims 64, 128): one 32-row block each, every
  // accumulator in VGPRs, and one wave's exponentials run beside the other's MFMAs. One wave
  // per SIMD: two blocks up to d = 128 (each K/V fragment read feeds two MFMAs); at d = 256
  // the Q and dO operands of one block already take 128 registers.
  static constexpr int NQB = D <= 128 && NW == 4 ? 2 : 1;
  static constexpr int RPW = 32 * NQB;
  static constexpr int BR = WAVES * RPW;    // query rows per workgroup
  static constexpr int BT = 64;             // keys per streamed tile: two 32-key halves
  static constexpr int TILE = BT * D * 2;
  static constexpr int DB = D / 32;         // dQ accumulator blocks (the whole head dim)
  // K/V ring: three stages (one barrier per tile) when three fit in LDS, else two stages
  // with a second barrier per tile before a stage is refilled.
  static constexpr int STAGES = D <= 128 ? 3 : 2;
};

// PRE: the kernel also does the preprocess step for its rows (-D and LSE log2(e) from o, dO and
// lse) and leaves both in the workspace for a dK/dV kernel that runs after it; else it reads
// them from the workspace.
template <int D, int NW, bool PRE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DqCfg<D, NW>::WPE, DqCfg<D, NW>::WPE)))
void fa2_bwd_dq_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  using Q = DqCfg<D, NW>;
  static_assert(Q::BT == C::BT, "tiles are loaded by load_tile_dual");
  constexpr int KS = C::KS, DB = Q::DB, NQB = Q::NQB;
  // K and V stages in separate arrays (a DMA into one never aliases reads of another).
  constexpr int TILE3 = Q::STAGES == 3 ? Q::TILE : 1024;
  __shared__ __attribute__((aligned(1024))) char k_st0[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char k_st1[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char k_st2[TILE3];
  __shared__ __attribute__((aligned(1024))) char v_st0[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char v_st1[Q::TILE];
  __shared__ __attribute__((aligned(1024))) char v_st2[TILE3];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  if constexpr (NW == 4) agpr_accumulators_hint();
  const int N = p.N;
  // Each workgroup takes dq_pairs(D) pairs of query blocks of one head, one block after the
  // other: a block and its mirror nblk - 1 - block (causal: the longest rows with the shortest,
  // so every workgroup carries about the same work), which spreads the workgroups' start-up and
  // wind-down costs.
  int bh, j;
  map_slice_block(blockIdx.x, p.B * p.Hq, dq_work_items(p.nblk, D), bh, j);
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int hkv = hq / (p.Hq / p.Hkv);
  auto block = [&](int qblk) __attribute__((always_inline)) {
  const int q0 = qblk * Q::BR;
  const int qw = q0 + wave * Q::RPW;  // this wave's first query

  const uint32_t head_bytes = (uint32_t)N * C::ROWB;
  const size_t qoff = (size_t)bh * N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + hkv) * (size_t)N * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + kvoff, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + kvoff, head_bytes);

  // Key tiles of the workgroup, numbered from its first visible tile tbase (a window hides
  // the keys before q0 - window) up to its last row (causal); halves u = 0 .. 2 ntiles - 1.
  const int W = p.window;
  const int tbase = q0 > W ? (q0 - W) / Q::BT : 0;
  const int qend = min(q0 + Q::BR, N);
  const int ntiles = (p.causal ? (qend + Q::BT - 1) / Q::BT : (N + Q::BT - 1) / Q::BT) - tbase;
  // Last half this wave computes (causal: the one holding its last row); -1 if it has no rows.
  const int my_last = qw >= N ? -1
                              : (p.causal ? min(2 * ntiles - 1, (qw + Q::RPW - 1) / 32 - 2 * tbase)
                                          : 2 * ntiles - 1);

  auto kst = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    return (lds_char*)(s == 0 ? k_st0 : s == 1 ? k_st1 : k_st2);
  };
  auto vst = [&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    return (lds_char*)(s == 0 ? v_st0 : s == 1 ? v_st1 : v_st2);
  };
  // Tile t <= ntiles (tile ntiles only feeds the look-ahead half of the last step; rows past
  // the end read as zero).
  auto fetch = [&](auto S, int t) __attribute__((always_inline)) {
    if (t > ntiles) return;
    load_tile_dual<D, NW>(rk, kst(S), (tbase + t) * Q::BT, wave, lane);
    load_tile_dual<D, NW>(rv, vst(S), (tbase + t) * Q::BT, wave, lane);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  fetch(I0{}, 0);
  fetch(I1{}, 1);

  // Q and dO of this wave's queries as B operands (lane = query, k = head dim).
  u32x4 qf[NQB][KS], df[NQB][KS];
  float lse2v[NQB];
  f32x16 negd[NQB];  // -D of the lane's query in every register: the start of each dP chain
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dO + qoff, head_bytes);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qi = qw + 32 * qb + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = (uint32_t)qi * C::ROWB + (16 * ks + 8 * hf) * 2;
        qf[qb][ks] = buffer_load16(rq, off) ^ p.kneg;
        df[qb][ks] = buffer_load16(rd, off);
      }
      float nd;
      if constexpr (PRE) {
        // D = sum_c dO_c O_c of the lane's query: the lane holds dO at head dims
        // 16 ks + 8 hf .. + 7 (df), multiplies them with O there, and the two half-waves
        // (hf = 0, 1) add their parts. Rows past the end read O = 0, so D = 0 there.
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + qoff, (uint32_t)N * D * 4);
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t off = (uint32_t)qi * (D * 4) + (16 * ks + 8 * hf) * 4;
          const u32x4 a = buffer_load16(ro, off), b = buffer_load16(ro, off + 16);
          const u32x4 g = df[qb][ks];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const u32x4& x = w < 2 ? a : b;
            part += __uint_as_float(g[w] << 16) * __uint_as_float(x[2 * (w & 1)]) +
                    __uint_as_float(g[w] & 0xffff0000u) * __uint_as_float(x[2 * (w & 1) + 1]);
          }
        }
        nd = -(part + __shfl_xor(part, 32));
        lse2v[qb] = qi < N ? p.lse[(size_t)bh * N + qi] * kLog2e : 0.f;
        if (hf == 0 && qi < N) {
          p.delta[(size_t)bh * N + qi] = nd;
          p.lse2[(size_t)bh * N + qi] = lse2v[qb];
        }
      } else {
        lse2v[qb] = qi < N ? p.lse2[(size_t)bh * N + qi] : 0.f;
        nd = qi < N ? p.delta[(size_t)bh * N + qi] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) negd[qb][r] = nd;
    }
  }

  int roff[C::RO], toff[DB], toff8[DB];
#pragma unroll
  for (int ks = 0; ks < C::RO; ++ks) roff[ks] = row_read_off<D>(lane, ks);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    toff[db] = tr_read_off<D>(lane, db, 0);
    toff8[db] = tr_read_off<D>(lane, db, 1);
  }
  // Row-read offset of k-step ks (k-steps 8.. repeat 0.. shifted by 16 chunks).
  auto rowoff = [&](int ks) { return roff[ks % C::RO] + (ks / C::RO) * 256; };

  f32x16 adq[NQB][DB];  // dQ^T per row block: rows = head dim, columns = queries (lanes)
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) adq[qb][db] = f32x16{};
  const float c = p.c;

  // Per 32-key half u: S^T = K Q^T and dP^T = V dO^T (32 keys x 32 queries per row block;
  // register r holds key 8 (r / 4) + 4 hf + r % 4 of the half, lane = query),
  // P^T = 2^(S^T c - lse2), dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
  // The work is software-pipelined across halves. Step u runs S(u+1) MFMAs beside dS(u),
  // then dQ(u) MFMAs beside P(u+1), then dP(u+1) MFMAs beside the rest of P(u+1).
  // Each step reads one A operand (shared by both row blocks) PF steps ahead.
  f32x16 s[NQB], dp[NQB];
  float pf[NQB][16];      // P^T of the half in flight, fp32
  u32x4 pd[NQB][2];       // dS^T as B operands [qb][h]: 16 keys x 32 queries, packed bf16
  constexpr int NST = 2 * KS + 2 * DB;  // steps per half
  constexpr int PF = 3;
  constexpr int DL = 2;                 // steps between an accumulator's last MFMA and its use
  constexpr int NEL = 16 * NQB;         // P elements per lane and half
  constexpr int EXP0 = KS + DL, EXPN = NST - EXP0;  // steps carrying P(u+1)
  constexpr int DS_STEPS = KS < NEL / 2 ? KS : NEL / 2;  // steps carrying dS(u)
  constexpr int DS_RATE = NEL / 2 / DS_STEPS;            // dS element pairs per step

  auto exp_el = [&](int e) __attribute__((always_inline)) {
    const int qb = e >> 4, rr = e & 15;
    pf[qb][rr] = fast_exp2(__builtin_fmaf(s[qb][rr], c, -lse2v[qb]));
  };
  // dS element pairs q in h-major order, so pd[.][0] is complete before pd[.][1].
  auto ds_pair = [&](int q) __attribute__((always_inline)) {
    const int h = q / (4 * NQB), qb = (q / 4) % NQB, rr = 8 * h + 2 * (q % 4);
    const float a = pf[qb][rr] * dp[qb][rr];  // dp holds dP - D
    const float bb = pf[qb][rr + 1] * dp[qb][rr + 1];
    pd[qb][h][(rr >> 1) & 3] = pack_bf16(a, bb);
  };
  // Causal: zero P^T outside query - window <= key <= query, for a half (first key 32 ua)
  // crossing this wave's diagonal or its window's start.
  auto causal_fixup = [&](int ua) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int lim = qw + 32 * qb + l32 - 32 * ua - 4 * hf;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int x = 8 * (rr >> 2) + (rr & 3);
        pf[qb][rr] = (x > lim || x < lim - W) ? 0.f : pf[qb][rr];
      }
    }
  };

  auto half = [&](auto SC, auto KBC, auto SN, auto KBN, int u) __attribute__((always_inline)) {
    constexpr int kbc = decltype(KBC)::value, kbn = decltype(KBN)::value;
    const lds_char* kc = kst(SC) + kbc * 32 * C::ROWB;
    const lds_char* kn = kst(SN) + kbn * 32 * C::ROWB;
    const lds_char* vn = vst(SN) + kbn * 32 * C::ROWB;
    const int ua = u + 2 * tbase;  // the half's index from key 0
    const bool fix = p.causal && (32 * ua + 31 > qw || 32 * ua < qw + Q::RPW - 1 - W);
    auto read_op = [&](auto J) __attribute__((always_inline)) -> u32x4 {
      constexpr int j = decltype(J)::value;
      if constexpr (j < KS) {
        return lds_read16(kn + rowoff(j));
      } else if constexpr (j < KS + 2 * DB) {
        constexpr int i = j - KS, db = i % DB, h = i / DB;
        return tr_pair(kc + toff[db] + 16 * h * C::ROWB, kc + toff8[db] + 16 * h * C::ROWB);
      } else {
        return lds_read16(vn + rowoff(j - KS - 2 * DB));
      }
    };
    auto mfma_step = [&](auto J, u32x4 a) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        // S(u+1) starts from zero and dP(u+1) from -D; dP(u) stays live until dS(u) is done.
        if constexpr (j < KS) {
          s[qb] = mfma32x32x16(a, qf[qb][j], j == 0 ? f32x16{} : s[qb]);
        } else if constexpr (j < KS + 2 * DB) {
          constexpr int i = j - KS, db = i % DB, h = i / DB;
          adq[qb][db] = mfma32x32x16(a, pd[qb][h], adq[qb][db]);
        } else {
          constexpr int ks = j - KS - 2 * DB;
          dp[qb] = mfma32x32x16(a, df[qb][ks], ks == 0 ? negd[qb] : dp[qb]);
        }
      }
    };
    auto valu_step = [&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j == 0) {
        if (fix) causal_fixup(ua);
      }
      if constexpr (j >= DL && j < DL + DS_STEPS) {
#pragma unroll
        for (int q = (j - DL) * DS_RATE; q < (j - DL + 1) * DS_RATE; ++q) ds_pair(q);
      }
      if constexpr (j >= EXP0) {
        constexpr int e0 = (NEL * (j - EXP0)) / EXPN, e1 = (NEL * (j - EXP0 + 1)) / EXPN;
#pragma unroll
        for (int e = e0; e < e1; ++e) exp_el(e);
      }
    };
    u32x4 ring[PF + 1];
    static_for<0, PF>([&](auto J) __attribute__((always_inline)) { ring[decltype(J)::value] = read_op(J); });
    static_for<0, NST>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      if constexpr (j + PF < NST) ring[(j + PF) % (PF + 1)] = read_op(std::integral_constant<int, j + PF>{});
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(J, ring[j % (PF + 1)]);
      valu_step(J);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  wait_vmem_all();
  __syncthreads();
  // Prologue: S(0), dP(0) and P(0) from the first half of tile 0.
  if (my_last >= 0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = negd[qb];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 ka = lds_read16((const lds_char*)k_st0 + rowoff(ks));
      const u32x4 va = lds_read16((const lds_char*)v_st0 + rowoff(ks));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = mfma32x32x16(ka, qf[qb][ks], s[qb]);
        dp[qb] = mfma32x32x16(va, df[qb][ks], dp[qb]);
      }
    }
#pragma unroll
    for (int e = 0; e < NEL; ++e) exp_el(e);
  }

  // Tile T: half 2T, then (all waves past their reads of tile T-1, tile T+1 landed) the DMA of
  // tile T+2 into T-1's stage, then half 2T+1, which looks ahead into tile T+1.
  auto tile_iter = [&](auto S, int T) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    using SN = std::integral_constant<int, (st + 1) % 3>;
    using SN2 = std::integral_constant<int, (st + 2) % 3>;
    if (2 * T <= my_last) half(S, I0{}, S, I1{}, 2 * T);
    wait_vmem_all();
    __syncthreads();
    // Waves 4-7 load their part of tile T+2 after half 2T+1, not beside waves 0-3 right after
    // the barrier: a wave cannot issue while the CU's vector-memory queue is full, and half as
    // many loads at once halves that stall. The tile is first read after the next barrier.
    if (wave < 4) fetch(SN2{}, T + 2);
    if (2 * T + 1 <= my_last) half(S, I1{}, SN{}, I0{}, 2 * T + 1);
    if (wave >= 4) fetch(SN2{}, T + 2);
  };
  // Two stages: tile T in stage T % 2 and T+1 in the other; half 2T+1 reads both, so the DMA
  // of tile T+2 into T's stage waits for a barrier after it.
  auto tile_iter2 = [&](auto S, int T) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    using SN = std::integral_constant<int, st ^ 1>;
    if (2 * T <= my_last) half(S, I0{}, S, I1{}, 2 * T);
    wait_vmem_all();
    __syncthreads();
    if (2 * T + 1 <= my_last) half(S, I1{}, SN{}, I0{}, 2 * T + 1);
    __syncthreads();
    fetch(S, T + 2);
  };
  int T = 0;
  if constexpr (Q::STAGES == 3) {
    for (; T + 3 <= ntiles; T += 3) {
      tile_iter(I0{}, T);
      tile_iter(I1{}, T + 1);
      tile_iter(I2{}, T + 2);
    }
    if (T < ntiles) tile_iter(I0{}, T);
    if (T + 1 < ntiles) tile_iter(I1{}, T + 1);
  } else {
    for (; T + 2 <= ntiles; T += 2) {
      tile_iter2(I0{}, T);
      tile_iter2(I1{}, T + 1);
    }
    if (T < ntiles) tile_iter2(I0{}, T);
  }

  // Store dQ = scale dQ^T^T: lane = query, registers = head dim, 16-byte pieces 32 bytes apart.
  // Once every wave is past its last reads (and the last look-ahead load has landed), each wave
  // passes its 32 rows through half of one K/V stage array in column chunks and stores whole
  // 128-byte lines. The lane index is made opaque so that the chunk addresses are formed here,
  // not hoisted across the tile loop.
  static_assert(NQB == 1, "one 32-row block per wave");
  wait_vmem_all();
  __syncthreads();
  {
    int el = lane;
    asm volatile("" : "+v"(el));
    const int e32 = el & 31, ehf = el >> 5;
    constexpr int REG = Q::TILE / 2;                             // bytes per wave
    constexpr int CW = REG / 128 < DB * 32 ? REG / 128 : DB * 32;  // columns per chunk
    constexpr int UPR = CW / 4;                                  // 16-byte units per row
    static_assert(CW % 32 == 0 && (DB * 32) % CW == 0 && (UPR & (UPR - 1)) == 0, "chunk shape");
    // Waves 2a and 2a+1 share array a of k_st0, k_st1, k_st2, v_st0 (four waves at d = 256 use
    // only the first two, full-size arrays).
    static_assert(NW == 8 ? Q::STAGES == 3 : NW == 4, "the arrays the waves use");
    const int arr = wave >> 1;
    lds_char* reg = (lds_char*)(arr == 0 ? k_st0 : arr == 1 ? k_st1 : arr == 2 ? k_st2 : v_st0) + (wave & 1) * REG;
    float* base = p.dq + qoff + (size_t)qw * D;
#pragma unroll
    for (int c = 0; c < DB * 32 / CW; ++c) {
#pragma unroll
      for (int dbc = 0; dbc < CW / 32; ++dbc)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int db = c * (CW / 32) + dbc, cu = 8 * dbc + 2 * rq + ehf;
          *(FA2_LDS f32x4*)(reg + e32 * (UPR * 16) + ((cu ^ (e32 & (UPR - 1))) << 4)) =
              f32x4{adq[0][db][4 * rq], adq[0][db][4 * rq + 1], adq[0][db][4 * rq + 2],
                    adq[0][db][4 * rq + 3]} * p.scale;
        }
#pragma unroll
      for (int k = 0; k < UPR / 2; ++k) {
        const int u = 64 * k + el, r = u / UPR, cu = u % UPR;
        const f32x4 val = *(const FA2_LDS f32x4*)(reg + r * (UPR * 16) + ((cu ^ (r & (UPR - 1))) << 4));
        if (qw + r < N) *(f32x4*)(base + (size_t)r * D + c * CW + 4 * cu) = val;
      }
    }
  }
  };
  const int npair = (p.nblk + 1) / 2;
  constexpr int KP = dq_pairs(D);
  for (int i = 0; i < 2 * KP; ++i) {
    const int pi = j * KP + i / 2;
    const int first = p.causal ? p.nblk - 1 - pi : pi;  // causal: longest rows first
    const int qb = i & 1 ? p.nblk - 1 - first : first;
    if (pi >= npair || (i & 1 && qb == first)) continue;
    if (i) __syncthreads();  // every wave is past its last reads of the previous block's tiles
    block(qb);
  }
}

// ------------------------------------------------------------------ launchers

// Workspace layout: D at [0, R) and lse2 at [R, 2R) floats, R = B*Hq*N.
static BwdParams make_params(const void* q, const void* k, const void* v, const void* dO,
                             float* ws, const AttnShape& s) {
  BwdParams p = {};
  const size_t R = (size_t)s.B * s.Hq * s.N;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dO = static_cast<const uint16_t*>(dO);
  p.delta = ws;
  p.lse2 = ws + R;
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.N = s.N;
  p.causal = s.causal;
  p.c = fabsf(s.scale) * kLog2e;
  p.scale = s.scale;
  p.kneg = s.scale < 0.f ? 0x80008000u : 0u;
  p.window = kernel_window(s);
  return p;
}

hipError_t launch_bwd_preprocess(const float* o, const void* dO, const float* lse, float* ws,
                                 const AttnShape& s, hipStream_t stream) {
  const long rows = (long)s.B * s.Hq * s.N;
  const long threads = rows * (s.d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  float* lse2 = ws + rows;
  if (s.d == 128)
    hipLaunchKernelGGL(fa2_bwd_pre_kernel<128>, grid, block, 0, stream, o, (const uint16_t*)dO, lse, ws, lse2, rows);
  else if (s.d == 256)
    hipLaunchKernelGGL(fa2_bwd_pre_kernel<256>, grid, block, 0, stream, o, (const uint16_t*)dO, lse, ws, lse2, rows);
  else
    hipLaunchKernelGGL(fa2_bwd_pre_kernel<64>, grid, block, 0, stream, o, (const uint16_t*)dO, lse, ws, lse2, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* ws, float* dk, float* dv, const AttnShape& s,
                           hipStream_t stream) {
  BwdParams p = make_params(q, k, v, dO, const_cast<float*>(ws), s);
  p.dk = dk;
  p.dv = dv;
  if (s.d == 256) {
    p.nblk = (s.N + QuadCfg::BR - 1) / QuadCfg::BR;
    hipLaunchKernelGGL(fa2_bwd_dkdv_quad_kernel, dim3((unsigned)(s.B * s.Hkv * p.nblk)),
                       dim3(QuadCfg::WAVES * 64), 0, stream, p);
    return hipGetLastError();
  }
  p.nblk = (s.N + BwdCfg<128>::BR - 1) / BwdCfg<128>::BR;
  const dim3 grid((unsigned)(s.B * s.Hkv * dkdv_work_items(p.nblk, s.Hq / s.Hkv)));
  const dim3 block(PairCfg<128>::WAVES * 64);
  if (s.d == 128)
    hipLaunchKernelGGL(fa2_bwd_dkdv_pair_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fa2_bwd_dkdv_pair_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

template <bool PRE>
static hipError_t launch_dq(BwdParams p, const AttnShape& s, hipStream_t stream) {
  constexpr int NW = 8;  // head dims 64 and 128: two waves per SIMD (measured 5-20 % faster)
  const int BR = s.d == 256 ? DqCfg<256>::BR : DqCfg<128, NW>::BR;
  p.nblk = (s.N + BR - 1) / BR;
  const dim3 grid((unsigned)(s.B * s.Hq * dq_work_items(p.nblk, s.d)));
  if (s.d == 128)
    hipLaunchKernelGGL((fa2_bwd_dq_kernel<128, NW, PRE>), grid, dim3(NW * 64), 0, stream, p);
  else if (s.d == 256)
    hipLaunchKernelGGL((fa2_bwd_dq_kernel<256, 4, PRE>), grid, dim3(4 * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((fa2_bwd_dq_kernel<64, NW, PRE>), grid, dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* ws, float* dq, const AttnShape& s, hipStream_t stream) {
  BwdParams p = make_params(q, k, v, dO, const_cast<float*>(ws), s);
  p.dq = dq;
  return launch_dq<false>(p, s, stream);
}

hipError_t launch_bwd_dq_pre(const void* q, const void* k, const void* v, const void* dO,
                             const float* o, const float* lse, float* ws, float* dq,
                             const AttnShape& s, hipStream_t stream) {
  BwdParams p = make_params(q, k, v, dO, ws, s);
  p.dq = dq;
  p.o = o;
  p.lse = lse;
  return launch_dq<true>(p, s, stream);
}

}  // namespace fa2

// fa2_decode.hip -- decode-shaped attention for gfx950: Nq query rows against an Nk-row KV
// cache (Nq << Nk), the inference shape of the pages (the qualellm.it guide "Flash Attention
// 2: attivarla (llama.cpp, Ollama, vLLM)", sections "Perché Flash Attention 2" and
// "Guadagno misurato in base alla dimensione del contesto"; FlashDecoding++ in the wiki
// article's literature list). The result is the same exact attention as the forward, with the
// causal mask aligned to the end of the cache (query i sees keys j <= Nk - Nq + i).
//
// The work per query row is tiny and every row of a KV group reads the same cache, so the pass
// is bound by streaming K/V from HBM once. Mapping:
//  * The G = Hq/Hkv heads sharing a KV head contribute their Nq rows each; those G*Nq rows are
//    contiguous in q and o ([B,Hq,Nq,d] with the group's heads adjacent), so they form one
//    query block of R = G*Nq rows, split into 32-row MFMA blocks.
//  * The cache is split into chunks; one wave per (batch, KV head, row block, chunk) runs an
//    online softmax over its chunk (the forward's tile loop, with no barriers: waves share
//    nothing) and writes a partial (O, LSE). A second kernel merges the chunks of each row:
//    LSE = ln sum_s e^LSE_s, O = sum_s e^(LSE_s - LSE) O_s. With one chunk the first kernel
//    writes O and LSE directly.
//  * Per 64-key tile a wave loads its K rows straight into MFMA A-operand registers and copies
//    the V tile into its own LDS slot (buffer_load ... lds, swizzled for the transposing
//    reads), one tile ahead of the tile it computes (two register sets, two LDS slots), so
//    each wave keeps about 32 KB of the cache in flight.
#include "fa2_device.h"
#include "fa2_launch.h"

namespace fa2 {

struct DecParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;      // [B,Hq,Nq,d]  (nsplit == 1)
  float* lse;    // [B,Hq,Nq]    (nsplit == 1)
  float* po;     // partial O    [B*Hkv, nsplit, R, d]  (nsplit > 1)
  float* plse;   // partial LSE  [B*Hkv, nsplit, R]     (nsplit > 1), natural log
  int B, Hq, Hkv, Nq, Nk;
  int causal;
  float c;        // |scale| * log2(e)
  unsigned qneg;  // sign flip of the Q operand when scale < 0
  int R;          // query rows per KV group: (Hq / Hkv) * Nq
  int nrb;        // 32-row blocks per group
  int nsplit;     // cache chunks
  int chunk;      // keys per chunk, a multiple of 64
  int nwaves;     // B * Hkv * nrb * nsplit
};

template <int D>
struct DecCfg {
  static constexpr int WAVES = 4;          // waves per workgroup (independent)
  static constexpr int BN = 64;            // keys per tile
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = BN * ROWB;   // one V tile in LDS
  static constexpr int LPT = TILE / 1024;  // 1 KB direct-to-LDS loads per tile
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa2_decode_kernel(DecParams p) {
  using C = DecCfg<D>;
  // Two V slots per wave, in separate arrays, for the two tiles in flight.
  __shared__ __attribute__((aligned(1024))) char v_slot_a[C::WAVES][C::TILE];
  __shared__ __attribute__((aligned(1024))) char v_slot_b[C::WAVES][C::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int wid = blockIdx.x * C::WAVES + wave;
  if (wid >= p.nwaves) return;
  // wid = ((vh * nsplit) + s) * nrb + rb: the row blocks of one chunk run side by side.
  const int rb = wid % p.nrb;
  const int s = (wid / p.nrb) % p.nsplit;
  const int vh = wid / (p.nrb * p.nsplit);  // b * Hkv + g
  const int b = vh / p.Hkv, g = vh % p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int Nk = p.Nk;

  const size_t qrow0 = ((size_t)b * p.Hq + (size_t)g * G) * p.Nq;  // the group's first q/o row
  const size_t kvoff = (size_t)vh * Nk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + qrow0 * D, (uint32_t)p.R * C::ROWB);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + kvoff, (uint32_t)Nk * C::ROWB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + kvoff, (uint32_t)Nk * C::ROWB);

  // This lane's query row r of the group (the S^T column it holds); rows past R read zeros
  // and are never stored. Causal: row r = (head h, query i = r % Nq) sees keys <= Nk - Nq + i.
  const int r = rb * 32 + l32;
  const int lim = p.causal ? Nk - p.Nq + r % p.Nq : Nk - 1;

  u32x4 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) qf[ks] = buffer_load16(rq, (uint32_t)r * C::ROWB + (16 * ks + 8 * hf) * 2) ^ p.qneg;

  // This chunk's keys [k0, k1) (the last row of the group sees every key of the cache).
  const int k0 = s * p.chunk;
  const int k1 = min(Nk, k0 + p.chunk);
  const int ntiles = (k1 - k0 + C::BN - 1) / C::BN;
  // Tiles from this index on may hold keys that some row must not see (causal edge, end of
  // the cache, end of the chunk) and are masked.
  const int mask_from = p.causal ? (Nk - p.Nq + 1 - k0) / C::BN : (k1 - k0) / C::BN;

  int voff[C::DB];  // V^T A-operand: transposing read base per 32-wide head-dim block
  {
    const int rr = 4 * hf + ((lane & 15) >> 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int dd = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      voff[db] = rr * C::ROWB + (((dd >> 3) ^ swz_v<D>(rr)) << 4) + (dd & 7) * 2;
    }
  }
  lds_char* va = (lds_char*)v_slot_a[wave];
  lds_char* vb = (lds_char*)v_slot_b[wave];

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  float m = -INFINITY;  // row reference, log2 domain
  float l = 0.f;        // this lane's partial row sum
  const float c = p.c;

  // Software pipeline, two tiles deep: tile t+1's K rows (registers) and V tile (the other LDS
  // array) are requested before tile t is computed; V(t) is waited for just before its reads.
  // VMEM requests complete in order, so "V(t) landed" is "at most the requests of tile t+1 are
  // still outstanding".
  constexpr int KLOADS = 2 * C::KS;  // K loads per tile
  constexpr int VLOADS = C::LPT;     // V copies per tile
  auto issue = [&](int t, lds_char* vdst, u32x4 (&kdst)[2][C::KS]) __attribute__((always_inline)) {
    const int j0 = k0 + t * C::BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        kdst[kb][ks] = buffer_load16(rk, (uint32_t)(j0 + 32 * kb + l32) * C::ROWB + (16 * ks + 8 * hf) * 2);
#pragma unroll
    for (int blk = 0; blk < C::LPT; ++blk) {
      const int pos = blk * 1024 + lane * 16;
      const int row = pos / C::ROWB;
      const int cp = (pos % C::ROWB) / 16;
      buffer_load16_lds(rv, vdst + blk * 1024, (uint32_t)(j0 + row) * C::ROWB + ((cp ^ swz_v<D>(row)) << 4));
    }
  };
  auto compute = [&](int t, const lds_char* vt, const u32x4 (&kf)[2][C::KS], bool next_in_flight)
      __attribute__((always_inline)) {
    const int j0 = k0 + t * C::BN;
    // S^T = K Q^T: two 32-key blocks; register e of block kb holds key 8(e/4) + 4hf + e%4.
    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) st[kb] = mfma32x32x16(kf[kb][ks], qf[ks], st[kb]);
    }
    float mx = -INFINITY;
    const bool mask = t >= mask_from;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (mask) {
          const int key = j0 + 32 * kb + 8 * (e >> 2) + 4 * hf + (e & 3);
          st[kb][e] = (key > lim || key >= k1) ? -INFINITY : st[kb][e];
        }
        mx = fmaxf(mx, st[kb][e]);
      }
    // Online softmax: raise the reference to the tile max, rescale O and l.
    const float mnew = fmaxf(m, max_halves(mx) * c);
    const float alpha = m == mnew ? 1.f : fast_exp2(m - mnew);  // m = mnew = -inf: no key yet
    m = mnew;
    const float mref = m == -INFINITY ? 0.f : m;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
    u32x4 pf[2][2];  // P^T as B operands [kb][h]: 16 keys x 32 rows, packed bf16
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(st[kb][e], c, -mref));
        const float p1 = fast_exp2(__builtin_fmaf(st[kb][e + 1], c, -mref));
        l += p0 + p1;
        pf[kb][e >> 3][(e >> 1) & 3] = pack_bf16(p0, p1);
      }
    // V(t) must have landed: only tile t+1's requests may still be outstanding.
    if (next_in_flight) {
      static_assert(KLOADS + VLOADS <= 63, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KLOADS + VLOADS) : "memory");
    } else {
      wait_vmem_all();
    }
    // O^T += V^T P^T, V^T fragments by transposing LDS reads.
#pragma unroll
    for (int i = 0; i < 4 * C::DB; ++i) {
      const int db = i % C::DB, kb = i / (2 * C::DB), h = (i / C::DB) & 1;
      const lds_char* base = vt + voff[db] + (32 * kb + 16 * h) * C::ROWB;
      const u32x2 lo = lds_read8_tr(base);
      const u32x2 hi = lds_read8_tr(base + 8 * C::ROWB);
      acc[db] = mfma32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kb][h], acc[db]);
    }
  };
  // Tiles alternate between (va, kfa) and (vb, kfb). A slot is refilled only after the tile
  // that used it is computed (its LDS reads are consumed by then).
  u32x4 kfa[2][C::KS], kfb[2][C::KS];
  if (ntiles > 0) issue(0, va, kfa);
  for (int t = 0; t < ntiles; t += 2) {
    const bool n1 = t + 1 < ntiles;
    if (n1) issue(t + 1, vb, kfb);
    compute(t, va, kfa, n1);
    if (!n1) break;
    const bool n2 = t + 2 < ntiles;
    if (n2) issue(t + 2, va, kfa);
    compute(t + 1, vb, kfb, n2);
  }

  // ---- epilogue: this chunk's O and LSE for row r (a row that met no visible key in the
  // chunk contributes O = 0 with LSE = -inf) ----
  const float lt = sum_halves(l);
  if (r >= p.R) return;
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  const float lse_r = empty ? -INFINITY : (m + __log2f(lt)) * kLn2;
  float* orow;
  float* lrow;
  if (p.nsplit == 1) {
    orow = p.o + (qrow0 + r) * D;
    lrow = p.lse + qrow0 + r;
  } else {
    const size_t prow = ((size_t)vh * p.nsplit + s) * p.R + r;
    orow = p.po + prow * D;
    lrow = p.plse + prow;
  }
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *(f32x4*)(orow + 32 * db + 8 * rq + 4 * hf) = f32x4{acc[db][4 * rq] * inv, acc[db][4 * rq + 1] * inv,
                                                          acc[db][4 * rq + 2] * inv, acc[db][4 * rq + 3] * inv};
  if (hf == 0) *lrow = lse_r;
}

// Merge of the chunks of each row: one workgroup per row. The workgroup first finds the row's
// largest chunk LSE M (finite: some chunk sees a key for every row); thread (slice sl, column
// c4) then sums w_s = e^(LSE_s - M) and w_s O_s over chunks sl, sl + NSL, ... for 4
// consecutive head-dim values (a chunk with LSE = -inf gets w = 0), and the slices are added
// in LDS: LSE = M + ln sum_s w_s, O = sum_s w_s O_s / sum_s w_s.
template <int D>
__global__ __launch_bounds__(256) void fa2_decode_merge_kernel(DecParams p) {
  constexpr int NC = D / 4;       // column threads per row
  constexpr int NSL = 256 / NC;   // chunk slices
  __shared__ f32x4 so[NSL][NC];
  __shared__ float ss[NSL];
  __shared__ float smax[4];
  const long row = blockIdx.x;    // (b * Hkv + g) * R + r
  const int tid = threadIdx.x;
  const int c = tid % NC, sl = tid / NC;
  const long vh = row / p.R;
  const int r = (int)(row % p.R);
  const float* pl = p.plse + (size_t)vh * p.nsplit * p.R + r;
  const float* po = p.po + ((size_t)vh * p.nsplit * p.R + r) * D + 4 * c;
  const size_t sstride = (size_t)p.R * D;

  float mx = -INFINITY;
  for (int s = tid; s < p.nsplit; s += 256) mx = fmaxf(mx, pl[(size_t)s * p.R]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) smax[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));

  float sum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = sl; s < p.nsplit; s += NSL) {
    const float w = __expf(pl[(size_t)s * p.R] - M);  // e^-inf = 0
    sum += w;
    o += w * *(const f32x4*)(po + s * sstride);
  }
  so[sl][c] = o;
  if (c == 0) ss[sl] = sum;
  __syncthreads();
  if (sl != 0) return;
#pragma unroll
  for (int t = 1; t < NSL; ++t) {
    o += so[t][c];
    sum += ss[t];
  }
  const int b = (int)(vh / p.Hkv), g = (int)(vh % p.Hkv);
  const size_t orow = ((size_t)b * p.Hq + (size_t)g * (p.Hq / p.Hkv)) * p.Nq + r;
  *(f32x4*)(p.o + orow * D + 4 * c) = o * (1.0f / sum);  // sum >= 1 (the chunk holding M)
  if (c == 0) p.lse[orow] = M + __logf(sum);
}

// Chunking: about two rounds of resident waves (one wave per SIMD and workgroup-per-CU
// residency give 1024 at a time), chunks a multiple of the 64-key tile and at least 256 keys;
// chunks are lengthened to 1024 or 512 keys when that still leaves a full round of waves,
// since a longer chunk spends less of its time filling the pipeline.
static void decode_split(const AttnShape& s, int Nq, int Nk, int* nsplit, int* chunk) {
  const long groups = (long)s.B * s.Hkv * ((s.Hq / s.Hkv * Nq + 31) / 32);
  const long want = (2048 + groups - 1) / groups;
  int ch = (int)((Nk + want - 1) / want);
  ch = (ch + 63) / 64 * 64;
  for (int longer : {1024, 512, 256})
    if (ch < longer && (longer == 256 || groups * ((Nk + longer - 1) / longer) >= 1024)) {
      ch = longer;
      break;
    }
  *chunk = ch;
  *nsplit = (Nk + ch - 1) / ch;
}

size_t decode_workspace_bytes(const AttnShape& s, int Nq, int Nk) {
  int nsplit, chunk;
  decode_split(s, Nq, Nk, &nsplit, &chunk);
  if (nsplit == 1) return 0;
  const size_t R = (size_t)(s.Hq / s.Hkv) * Nq;
  const size_t rows = (size_t)s.B * s.Hkv * nsplit * R;
  const size_t bytes = rows * ((size_t)s.d + 1) * 4;
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, float* o, float* lse,
                         const AttnShape& s, int Nq, int Nk, float* ws, hipStream_t stream) {
  DecParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.causal = s.causal;
  p.c = fabsf(s.scale) * kLog2e;
  p.qneg = s.scale < 0.f ? 0x80008000u : 0u;
  p.R = (s.Hq / s.Hkv) * Nq;
  p.nrb = (p.R + 31) / 32;
  decode_split(s, Nq, Nk, &p.nsplit, &p.chunk);
  p.nwaves = s.B * s.Hkv * p.nrb * p.nsplit;
  if (p.nsplit > 1) {
    const size_t rows = (size_t)s.B * s.Hkv * p.nsplit * p.R;
    p.po = ws;
    p.plse = ws + rows * s.d;
  }
  const dim3 grid((unsigned)((p.nwaves + 3) / 4)), block(256);
  if (s.d == 128)
    hipLaunchKernelGGL(fa2_decode_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fa2_decode_kernel<64>, grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const dim3 mgrid((unsigned)((long)s.B * s.Hkv * p.R));
  if (s.d == 128)
    hipLaunchKernelGGL(fa2_decode_merge_kernel<128>, mgrid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fa2_decode_merge_kernel<64>, mgrid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa2

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
//    reads). Two waves per SIMD overlap one wave's loads with the other's MFMAs.
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa2_decode_kernel(DecParams p) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(1024))) char v_slot[C::WAVES][C::TILE];

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
  lds_char* vt = (lds_char*)v_slot[wave];

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};
  float m = -INFINITY;  // row reference, log2 domain
  float l = 0.f;        // this lane's partial row sum
  const float c = p.c;

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = k0 + t * C::BN;
    // V tile -> this wave's LDS slot (swizzled rows), K rows -> A-operand registers.
#pragma unroll
    for (int blk = 0; blk < C::LPT; ++blk) {
      const int pos = blk * 1024 + lane * 16;
      const int row = pos / C::ROWB;
      const int cp = (pos % C::ROWB) / 16;
      buffer_load16_lds(rv, vt + blk * 1024, (uint32_t)(j0 + row) * C::ROWB + ((cp ^ swz_v<D>(row)) << 4));
    }
    u32x4 kf[2][C::KS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        kf[kb][ks] = buffer_load16(rk, (uint32_t)(j0 + 32 * kb + l32) * C::ROWB + (16 * ks + 8 * hf) * 2);
    wait_vmem_all();

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
    // O^T += V^T P^T, V^T fragments by transposing LDS reads.
#pragma unroll
    for (int i = 0; i < 4 * C::DB; ++i) {
      const int db = i % C::DB, kb = i / (2 * C::DB), h = (i / C::DB) & 1;
      const lds_char* base = vt + voff[db] + (32 * kb + 16 * h) * C::ROWB;
      const u32x2 lo = lds_read8_tr(base);
      const u32x2 hi = lds_read8_tr(base + 8 * C::ROWB);
      acc[db] = mfma32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kb][h], acc[db]);
    }
    // The next tile's V overwrites this slot: every read above has been consumed by now.
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

// Merge of the chunks of each row: one thread per 4 consecutive head-dim values of a row.
template <int D>
__global__ __launch_bounds__(256) void fa2_decode_merge_kernel(DecParams p) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long rows = (long)p.B * p.Hkv * p.R;
  const long row = gid / (D / 4);
  const int c4 = (int)(gid % (D / 4)) * 4;
  if (row >= rows) return;
  const long vh = row / p.R;
  const int r = (int)(row % p.R);
  const float* pl = p.plse + (size_t)vh * p.nsplit * p.R + r;
  float mx = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) mx = fmaxf(mx, pl[(size_t)s * p.R]);
  float sum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.nsplit; ++s) {
    const float ls = pl[(size_t)s * p.R];
    const float w = ls == -INFINITY ? 0.f : __expf(ls - mx);  // mx is finite: some chunk sees a key
    sum += w;
    o += w * *(const f32x4*)(p.po + (((size_t)vh * p.nsplit + s) * p.R + r) * D + c4);
  }
  const int b = (int)(vh / p.Hkv), g = (int)(vh % p.Hkv);
  const size_t orow = ((size_t)b * p.Hq + (size_t)g * (p.Hq / p.Hkv)) * p.Nq + r;
  *(f32x4*)(p.o + orow * D + c4) = o * (1.0f / sum);
  if (c4 == 0) p.lse[orow] = mx + __logf(sum);
}

// Chunking: at least ~4096 waves in flight across the chip (two per SIMD, two rounds), chunks
// of at least 256 keys, a multiple of the 64-key tile.
static void decode_split(const AttnShape& s, int Nq, int Nk, int* nsplit, int* chunk) {
  const long groups = (long)s.B * s.Hkv * ((s.Hq / s.Hkv * Nq + 31) / 32);
  long want = (4096 + groups - 1) / groups;
  const long most = (Nk + 255) / 256;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int ch = (int)((Nk + want - 1) / want);
  ch = (ch + 63) / 64 * 64;
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
  const long threads = (long)s.B * s.Hkv * p.R * (s.d / 4);
  const dim3 mgrid((unsigned)((threads + 255) / 256));
  if (s.d == 128)
    hipLaunchKernelGGL(fa2_decode_merge_kernel<128>, mgrid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fa2_decode_merge_kernel<64>, mgrid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa2

/*
 * fa2.h -- exact tiled attention (FlashAttention-2 style) for AMD MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention
 *     O = softmax(scale * Q K^T) V
 * without ever storing the N x N score matrix. The forward streams K/V tiles through on-chip
 * memory and applies the softmax incrementally, saving only O and the per-row logsumexp;
 * the backward recomputes the probabilities from that logsumexp instead of reading a stored
 * matrix. Source: the FlashAttention-2 pages ("Flash Attention spiegata: una guida completa",
 * datacamp, sections "Attention standard vs Flash attention", "Tiling", "Ricomputazione";
 * wiki article "FlashAttention-2", section on technical architecture). The result is exact:
 * it equals standard attention up to floating-point rounding.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller. The library allocates, frees and
 *     retains nothing, and keeps no state between calls; calls are re-entrant.
 *   - Layouts are contiguous row-major: q, dO, o, dq        [B, Hq,  N, d]
 *                                        k, v, dk, dv       [B, Hkv, N, d]
 *                                        lse                [B, Hq,  N]
 *   - Dtypes: q, k, v, dO are bfloat16 (raw 16-bit patterns); o, lse, dq, dk, dv are float32.
 *     lse is the natural-log logsumexp of the scaled scores of each query row.
 *   - Grouped-query attention: query head hq reads key/value head hq / (Hq / Hkv).
 *   - causal != 0: query row i attends to key rows j <= i (square, top-left aligned).
 *   - d must be 64, 128 or 256 (fa2_decode: 64 or 128); FlashAttention-2 handles head dims up
 *     to 256 ("Flash Attention spiegata: una guida completa", section "Supporto per dimensioni di
 *     testa maggiori").
 *     Other head dims (96, 192, ...) are rejected with FA2_ERR_UNSUPPORTED_HEAD_DIM: the pages
 *     treat an unsupported head dimension as a reported error, not a silent fallback ("Flash
 *     Attention 2: attivarla (llama.cpp, Ollama, vLLM)", qualellm.it, section "Risoluzione dei
 *     problemi", item "Errore unsupported head dimension").
 *   - scale must be finite and non-zero (negative values are accepted).
 *   - Every pointer must be 16-byte aligned; outputs must not overlap inputs or each other.
 *   - B == 0 or N == 0 is an empty problem: nothing is enqueued and FA2_OK is returned
 *     (pointers may then be NULL). Negative sizes, Hq or Hkv < 1, Hq % Hkv != 0 and sizes
 *     whose element offsets would not fit the kernels' index arithmetic are errors.
 *   - All validation happens before anything is enqueued: on error nothing is launched and
 *     no output is written. FA2_OK means the work is ENQUEUED on `stream` (NULL = the null
 *     stream); results are valid once the stream has been synchronised.
 *   - FA2_ERR_HIP reports a failed launch (hipGetLastError after the launch); an error left
 *     pending on the device by earlier, unrelated work may surface here as well.
 *   - Bitwise deterministic: identical inputs, sizes and build give identical outputs (no
 *     floating-point atomics; each output element is reduced in a fixed order).
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA2_OK = 0,
  FA2_ERR_NULL_POINTER = 1,         /* a required pointer is NULL (non-empty problem)      */
  FA2_ERR_BAD_SHAPE = 2,            /* negative size, or offsets overflow index arithmetic */
  FA2_ERR_UNSUPPORTED_HEAD_DIM = 3, /* d not in {64, 128, 256} ({64, 128} for fa2_decode)   */
  FA2_ERR_BAD_GQA = 4,              /* Hq < 1, Hkv < 1 or Hq % Hkv != 0                    */
  FA2_ERR_BAD_SCALE = 5,            /* scale is NaN, infinite or zero                      */
  FA2_ERR_MISALIGNED = 6,           /* a pointer is not 16-byte aligned                    */
  FA2_ERR_ALIASING = 7,             /* an output overlaps an input or another output       */
  FA2_ERR_WORKSPACE = 8,            /* workspace NULL or smaller than required             */
  FA2_ERR_HIP = 9,                  /* a kernel launch failed                              */
  FA2_ERR_BAD_WINDOW = 10,          /* sliding window < 0                                  */
  FA2_ERR_SCRATCH_LIMIT = 11        /* fa2_backward_noalloc: problem exceeds its fixed buffer */
} fa2_status;

/*
 * Forward pass: O and LSE from Q, K, V.
 *   q      bf16 [B,Hq,N,d]   (read only)
 *   k, v   bf16 [B,Hkv,N,d]  (read only)
 *   o      f32  [B,Hq,N,d]   (written)   O_i = sum_j P_ij v_j, P = softmax over visible keys
 *   lse    f32  [B,Hq,N]     (written)   LSE_i = ln sum_j exp(scale <q_i, k_j>)
 * Tiles Q into row blocks, streams K/V tiles through LDS with an online softmax (running
 * row max and sum, accumulator rescaled when the max grows), skips K/V tiles that the causal
 * mask hides entirely and masks only tiles that straddle the diagonal.
 */
int fa2_forward(const void* q, const void* k, const void* v, float* o, float* lse,
                int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                hipStream_t stream);

/* Bytes of device workspace fa2_backward needs: two floats per query row (-D, with
   D = rowsum(dO*O), and LSE*log2(e)), rounded up to 256 bytes. 0 for an empty problem or
   negative sizes. Layout, with R = B*Hq*N: -D at floats [0, R), LSE*log2(e) at floats [R, 2R)
   (the kernels start their dP accumulators from -D). */
size_t fa2_backward_workspace_size(int B, int Hq, int N);

/*
 * Backward pass: dQ, dK, dV of L = sum(O * dO), recomputing P from the saved LSE.
 *   q, k, v      as in fa2_forward (read only)
 *   o, lse       the outputs of fa2_forward for the same q, k, v, sizes, causal, scale
 *   dO           bf16 [B,Hq,N,d]  (read only)
 *   dq           f32  [B,Hq,N,d]  (written)  scale * sum_j dS_ij k_j
 *   dk, dv       f32  [B,Hkv,N,d] (written)  sums over the Hq/Hkv query heads of a group
 *   workspace    device scratch of at least fa2_backward_workspace_size(B,Hq,N) bytes,
 *                owned by the caller; its contents on entry do not matter and are
 *                overwritten. Must not overlap any other argument.
 * Two launches in stream order: a dQ kernel (one workgroup per query block, looping over key
 * blocks) that first does the preprocess for its rows (D_i = sum_c dO_ic O_ic, written to the
 * workspace with LSE*log2(e)), then a dK/dV kernel (one workgroup per key block, looping over
 * query blocks and the group's query heads) that reads them. No atomics.
 */
int fa2_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 const void* dO, float* dq, float* dk, float* dv,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The steps of fa2_backward as separate calls. Each validates its own arguments like
 * fa2_backward (same codes) and enqueues one kernel; `workspace` must be at least
 * fa2_backward_workspace_size(B,Hq,N) bytes. fa2_backward_dq_preprocess then
 * fa2_backward_dkdv, on one stream with one workspace, is what fa2_backward runs and gives
 * bitwise its results. fa2_backward_preprocess, then fa2_backward_dkdv and fa2_backward_dq in
 * either order, computes the same (the preprocess step on its own, as the method's backward
 * states it: "Flash Attention spiegata: una guida completa", section "Ricomputazione"); its D
 * is summed in another order, so results agree with fa2_backward to rounding, not bitwise.
 *
 * fa2_backward_preprocess: fills the workspace from o f32 [B,Hq,N,d], dO bf16 [B,Hq,N,d] and
 *   lse f32 [B,Hq,N] (all read only): -D_i = -sum_c dO_ic o_ic and LSE_i * log2(e).
 */
int fa2_backward_preprocess(const float* o, const void* dO, const float* lse, void* workspace,
                            size_t workspace_bytes, int B, int Hq, int N, int d,
                            hipStream_t stream);

/* fa2_backward_dkdv: dK, dV (f32 [B,Hkv,N,d], written) from q, k, v, dO and a workspace filled
   by fa2_backward_preprocess or fa2_backward_dq_preprocess (read only); recomputes P from the
   logsumexp, no atomics. */
int fa2_backward_dkdv(const void* q, const void* k, const void* v, const void* dO,
                      const void* workspace, size_t workspace_bytes, float* dk, float* dv,
                      int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                      hipStream_t stream);

/* fa2_backward_dq: dQ (f32 [B,Hq,N,d], written) from the same inputs as fa2_backward_dkdv. */
int fa2_backward_dq(const void* q, const void* k, const void* v, const void* dO,
                    const void* workspace, size_t workspace_bytes, float* dq, int B, int Hq,
                    int Hkv, int N, int d, int causal, float scale, hipStream_t stream);

/* fa2_backward_dq_preprocess: dQ (written) from q, k, v, o, lse, dO (read only), and the
   workspace filled as fa2_backward_preprocess fills it (written: -D and LSE*log2(e) of every
   query row), ready for fa2_backward_dkdv. The workspace counts as an output here: it must not
   overlap any other argument. */
int fa2_backward_dq_preprocess(const void* q, const void* k, const void* v, const float* o,
                               const float* lse, const void* dO, void* workspace,
                               size_t workspace_bytes, float* dq, int B, int Hq, int Hkv, int N,
                               int d, int causal, float scale, hipStream_t stream);

/*
 * Sliding-window (local) causal attention: query row i attends to key rows j with
 * max(0, i - window) <= j <= i, i.e. itself and the `window` keys before it. The pages name
 * sliding-window models (Mistral variants, Gemma's local layers) as the case where FA2
 * runtimes may fall back to another path ("Flash Attention 2: attivarla (llama.cpp, Ollama,
 * vLLM)", section "Casi in cui non aiuta (o peggiora la situazione)"); they give no formula,
 * and this is the plain reading of a window of `window` previous tokens.
 *   window >= 0 (FA2_ERR_BAD_WINDOW otherwise, checked first); window >= N - 1 is exactly
 *   fa2_forward / fa2_backward with causal = 1. All other arguments, layouts, checks and
 *   guarantees are those of fa2_forward / fa2_backward (causal is implied). K/V tiles that lie
 *   wholly outside every row's window are neither loaded nor computed, so the work is about
 *   N * (window + 1) key visits per head instead of N^2 / 2.
 * fa2_backward_window takes the o and lse written by fa2_forward_window with the same window.
 */
int fa2_forward_window(const void* q, const void* k, const void* v, float* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, int window, float scale,
                       hipStream_t stream);

int fa2_backward_window(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dO, float* dq, float* dk, float* dv,
                        int B, int Hq, int Hkv, int N, int d, int window, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode-shaped attention: Nq query rows against a cache of Nk key/value rows (Nq << Nk), the
 * long-context inference shape the pages centre on ("Flash Attention 2: attivarla (llama.cpp,
 * Ollama, vLLM)", sections "Perché Flash Attention 2" and "Guadagno misurato in base alla
 * dimensione del contesto"; FlashDecoding++ in the literature of the wiki article
 * "FlashAttention-2"). Exact attention, as fa2_forward, over rectangular shapes:
 *   q      bf16 [B,Hq,Nq,d]   k, v  bf16 [B,Hkv,Nk,d]      (read only)
 *   o      f32  [B,Hq,Nq,d]   lse   f32  [B,Hq,Nq]         (written; natural log)
 *   causal != 0: the rows are the newest tokens -- query i stands at cache position
 *   Nk - Nq + i and sees keys j <= Nk - Nq + i (requires Nq <= Nk). causal == 0: all keys.
 * The cache is split into chunks processed in parallel; each chunk yields a partial (O, LSE)
 * and a second kernel merges them: LSE = ln sum_s e^LSE_s, O = sum_s e^(LSE_s - LSE) O_s.
 * workspace: device scratch for the partial results, at least
 * fa2_decode_workspace_size(B,Hq,Hkv,Nq,Nk,d) bytes (0 when a single chunk suffices; then
 * workspace may be NULL); owned by the caller, contents on entry irrelevant; must not overlap
 * any other argument. Checks as fa2_forward; additionally Nk == 0 with Nq > 0, and causal with
 * Nq > Nk, are FA2_ERR_BAD_SHAPE. B == 0 or Nq == 0 is an empty problem (FA2_OK).
 */
size_t fa2_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d);

int fa2_decode(const void* q, const void* k, const void* v, float* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 forward (FlashAttention-3 adds FP8 arithmetic: wiki article "FlashAttention-2 (IT)",
 * section "FlashAttention-3"; "Flash Attention spiegata: una guida completa", section
 * "Precisione FP8 nativa"). q, k, v hold OCP FP8 E4M3FN codes (1 byte: sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; largest finite 448; 0x7F / 0xFF are NaN) in the layouts
 * of fa2_forward, standing for
 *     Q = code(q) * q_scale,  K = code(k) * k_scale,  V = code(v) * v_scale
 * (per-tensor scales, finite and > 0; quantising is the caller's business). The result is exact
 * attention over those values: o, lse as in fa2_forward. S = Q K^T runs on the FP8 matrix
 * cores (each product of two E4M3 values is exact in fp32); V is widened exactly to bf16 into
 * the workspace and P V runs as in the bf16 path. d must be 128.
 * workspace: at least fa2_forward_fp8_workspace_size(B,Hkv,N,d) bytes (2 bytes per element of
 * v), caller-owned, contents irrelevant, no overlap with other arguments. Other checks as
 * fa2_forward; a non-positive or non-finite q/k/v scale is FA2_ERR_BAD_SCALE.
 */
size_t fa2_forward_fp8_workspace_size(int B, int Hkv, int N, int d);

int fa2_forward_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                    float v_scale, float* o, float* lse, int B, int Hq, int Hkv, int N, int d,
                    int causal, float scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * fa2_backward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Arguments, layouts, checks, results
 * and guarantees are those of fa2_backward (bitwise the same outputs), without the workspace
 * arguments: the workspace is a fixed array of FA2_NOALLOC_SCRATCH_BYTES bytes of device memory
 * inside the library, one per GPU, which lives until the process ends. No call allocates or
 * frees anything; the first call on a device looks up that device's array (with that device
 * current) and keeps its address.
 *   Limit: fa2_backward_workspace_size(B, Hq, N) <= FA2_NOALLOC_SCRATCH_BYTES, i.e.
 *   B*Hq*N <= 2^21 query rows; larger problems return FA2_ERR_SCRATCH_LIMIT (checked before
 *   anything else) and launch nothing.
 *   Every call on one GPU uses that GPU's one array: calls whose work overlaps in time on the
 *   same GPU (other streams, other host threads) race on it and corrupt each other's results;
 *   the caller must order them (one stream, or events). Nothing in the array needs to be
 *   zero on entry: each call overwrites the part it reads.
 */
#define FA2_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int fa2_backward_noalloc(const void* q, const void* k, const void* v, const float* o,
                         const float* lse, const void* dO, float* dq, float* dk, float* dv,
                         int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         hipStream_t stream);

/* Static, human-readable name of a status code ("FA2_OK", ...); "FA2_UNKNOWN" otherwise. */
const char* fa2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */

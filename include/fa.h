/*
 * fa.h - exact IO-aware attention for AMD MI355X (gfx950): the C ABI of libfa.so.
 *
 * Computes exact scaled-dot-product attention, O = softmax(scale * Q K^T + mask) V,
 * tile by tile with an online softmax, so the N x N score and probability matrices
 * never reach device memory. The forward pass writes only O and the per-row
 * logsumexp; the backward pass recomputes P block by block from it.
 *
 * Sources (web pages on FlashAttention), cited by title and section:
 *  - "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness",
 *    AI Atlas summary: "En pocas palabras" (same result as standard attention),
 *    "Ideas clave" -> "Pensar en la E/S", "Tiling", "Softmax en línea",
 *    "Recalcular en vez de guardar".
 *  - "FlashAttention-2 (PT)", Systems analysis wiki: "Arquitetura técnica e
 *    princípios de funcionamento" (fewer non-matmul FLOPs; parallelism across blocks
 *    of one head; work split inside a block).
 *  - "FlashAttention", aiunderstanding.org: "Plongée profonde", "Aperçu technique".
 *  - "Flash Attention", docs.monostate.ai: "Con Sequence Packing" (packed batches).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except where noted is a DEVICE pointer owned by the caller.
 *    The library never allocates, frees, or synchronises, and keeps no state between
 *    calls. All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and is asynchronous: a device-side fault surfaces on the caller's next
 *    synchronising call, not here. The calls enqueue kernel launches only (no memset,
 *    copy or host synchronisation), so they may be captured in a HIP graph; a
 *    captured call keeps the pointers and sizes it was captured with.
 *  - Layout: q, k, v, o, dout, dq, dk, dv are contiguous (batch, seqlen, heads,
 *    head_dim), head_dim innermost. With cu_seqlens != NULL (a packed batch) they are
 *    (total_tokens, heads, head_dim) and sequence b owns tokens
 *    [cu_seqlens[b], cu_seqlens[b+1]); `seqlen` is then the longest sequence
 *    (host-known; sizes the launch grid) and `batch` the number of sequences.
 *  - lse: fp32 natural-log logsumexp of the scaled, masked scores of each query row,
 *    (batch, heads, seqlen), or (heads, total_tokens) for a packed batch.
 *  - dtype: FA_DTYPE_BF16 (tensors bf16, arithmetic fp32 with bf16 MFMA operands) or
 *    FA_DTYPE_FP32 (tensors and all arithmetic fp32).
 *  - head_dim in {64, 128}; seqlen >= 1; batch >= 1; heads >= 1; every tensor pointer
 *    16-byte aligned. Queries and keys share one length (self-attention).
 *  - causal != 0: query i sees key j iff j <= i, within its own sequence.
 *  - softmax_scale must be finite and > 0 (every entry point returns
 *    FA_ERR_INVALID_ARG otherwise): the kernels keep the running maximum of the raw
 *    scores q.k, which is the maximum of the scaled scores only for a positive scale.
 *  - stream is a hipStream_t passed as void* (the same pointer value), so that this
 *    header compiles without the HIP headers.
 *  - Argument checks run on the host before any HIP call and return
 *    FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED / FA_ERR_WORKSPACE without touching the
 *    device. A failed launch returns FA_ERR_HIP.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, bad alignment, overflow */
  FA_ERR_UNSUPPORTED = 2,  /* head_dim or dtype outside what the kernels are built for */
  FA_ERR_WORKSPACE = 3,    /* workspace pointer NULL or smaller than required        */
  FA_ERR_HIP = 4,          /* a kernel launch failed (hipGetLastError != success)      */
  FA_ERR_SCRATCH = 5       /* fa_bwd_noalloc: problem larger than its fixed scratch     */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP32 = 1 } fa_dtype;

/*
 * Forward pass. Writes o (same dtype and layout as q) and lse (fp32).
 * One workgroup per (sequence, head, query tile): parallel over the sequence, as in
 * "FlashAttention-2 (PT)", "2. Paralelismo aprimorado". Each workgroup keeps its query
 * tile in registers, streams key/value tiles through LDS, and carries the running row
 * maximum and sum ("Softmax en línea"). Bitwise deterministic from run to run.
 *
 * total_tokens is read only when cu_seqlens != NULL; cu_seqlens is a device int32
 * array of batch+1 non-decreasing prefix sums with cu_seqlens[0] = 0 and
 * cu_seqlens[batch] = total_tokens, and no sequence longer than seqlen (the kernels
 * do not check this: a violation is undefined behaviour).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int batch, int heads, int seqlen, int head_dim,
           float softmax_scale, int causal,
           const int32_t* cu_seqlens, int total_tokens,
           int dtype, void* stream);

/*
 * (A reading: the pages fix what the backward computes, not how a library hands it
 * scratch memory; a caller-owned workspace keeps the library free of allocations.)
 * Bytes of device workspace fa_bwd needs: two fp32 row statistics per (head, query
 * row), D_i = sum_k dO_ik * O_ik and -LSE_i / softmax_scale, each array rounded up to
 * 256 bytes, then 256 bytes of work counters that the dK/dV stage hands its key tiles out
 * with (written by the statistics stage, back to zero when the dK/dV stage ends). For a
 * packed batch (varlen != 0) pass total_tokens; otherwise it is ignored. Returns 0 for
 * invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int batch, int heads, int seqlen, int head_dim,
                              int varlen, int total_tokens);

/*
 * Backward pass for the loss gradient dout = dL/dO. Reads q, k, v, o, dout (as written
 * by fa_fwd and the caller) and lse (from fa_fwd); writes dq, dk, dv in the dtype and
 * layout of q. P is recomputed tile by tile from lse, never stored ("Recalcular en vez
 * de guardar"). Two stages run on `stream`, in order (see below):
 *   1. fa_bwd_dq_stats: the dQ accumulation pass, one workgroup per (sequence, head,
 *      query tile) accumulating dQ on chip while it walks the key tiles; it also forms
 *      D_i = rowsum(dO * O) and -LSE_i / softmax_scale of its query rows into the
 *      workspace (bf16: one kernel; fp32: fa_bwd_preprocess, then fa_bwd_dq);
 *   2. fa_bwd_dkdv: one workgroup per (sequence, head, key tile) accumulating dK and dV
 *      on chip while it walks the query tiles, reading those statistics.
 * No atomics: the result is bitwise deterministic from run to run.
 * workspace: device buffer of at least fa_bwd_workspace_bytes(...) bytes, 256-byte
 * aligned, owned by the caller; its contents on entry do not matter.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse,
           void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           int batch, int heads, int seqlen, int head_dim,
           float softmax_scale, int causal,
           const int32_t* cu_seqlens, int total_tokens,
           int dtype, void* stream);

/*
 * The backward in one pass over the key tiles (head_dim 128, FA_DTYPE_BF16): the same
 * arguments, outputs and tolerances as fa_bwd, with dQ accumulated by fp32 atomics from
 * the dK/dV kernel instead of a separate dQ pass. Recomputing P by blocks ("Recalcular
 * en vez de guardar", AI Atlas summary) then costs five matrix products per tile instead
 * of seven. Three kernels run on `stream`, in order: the row statistics (which also clear
 * the accumulator), the fused dK/dV/dQ kernel, and the conversion of the accumulator to
 * dq. dk and dv are bitwise reproducible; dq depends on the order in which the atomics
 * land, so it may differ from run to run in its last bits (the pages' "exact and
 * deterministic", "Desempenho e eficiência": fa_bwd keeps that; this entry point trades
 * the last bits of dq for speed).
 * workspace: at least fa_bwd_atomic_workspace_bytes(...) bytes (fa_bwd's statistics, then
 * an fp32 accumulator of (heads * tokens + 64) x head_dim), 256-byte aligned, owned by
 * the caller; its contents on entry do not matter. Other head_dim or dtype values return
 * FA_ERR_UNSUPPORTED; fa_bwd covers them.
 */
size_t fa_bwd_atomic_workspace_bytes(int batch, int heads, int seqlen, int head_dim,
                                     int varlen, int total_tokens);
int fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse,
                  void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes,
                  int batch, int heads, int seqlen, int head_dim,
                  float softmax_scale, int causal,
                  const int32_t* cu_seqlens, int total_tokens,
                  int dtype, void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and results. The row statistics go to a fixed device array
 * inside the library instead, FA_BWD_NOALLOC_MAX_SCRATCH bytes per GPU, held from the
 * library's first use on that GPU until the process ends; problems needing more than that
 * (8 * heads * tokens + 256 bytes, tokens = batch * seqlen or total_tokens: up to 2^21
 * (head, token) pairs, e.g. 32 heads x 65536 tokens) return FA_ERR_SCRATCH without
 * launching. No call allocates (no hipMalloc, no allocating library routine); the first
 * call on a device looks up the array's device address once (hipGetSymbolAddress), on
 * the calling thread's current device, which must be the device of the tensors and the
 * stream. Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (two streams, two threads) race and give wrong results; calls in stream order
 * are safe.
 */
#define FA_BWD_NOALLOC_MAX_SCRATCH ((16u << 20) + 256u)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse,
                   void* dq, void* dk, void* dv,
                   int batch, int heads, int seqlen, int head_dim,
                   float softmax_scale, int causal,
                   const int32_t* cu_seqlens, int total_tokens,
                   int dtype, void* stream);

/*
 * The stages of the backward, callable on their own (same arguments, conventions and
 * workspace as fa_bwd). The workspace statistics are written either by
 * fa_bwd_preprocess or by fa_bwd_dq_stats, which must complete before fa_bwd_dkdv (and
 * fa_bwd_dq) start; fa_bwd_dq only reads the workspace and may run concurrently with
 * fa_bwd_dkdv on a different stream. fa_bwd_dkdv also uses the workspace's work counters
 * (it leaves them as it found them, zero), so two fa_bwd_dkdv calls must not share a
 * workspace at the same time. Each enqueues exactly one kernel, except
 * fa_bwd_dq_stats with FA_DTYPE_FP32 (two).
 *
 *  fa_bwd_preprocess: workspace <- D_i = sum_k dO_ik * O_ik and -LSE_i / softmax_scale
 *    (fp32, lse layout each). D is the row sum of P * dP, the term the softmax backward
 *    subtracts; computing it from the stored O avoids touching P ("Recalcular en vez
 *    de guardar"). The second array is the starting value of the S = Q K^T
 *    accumulation in fa_bwd_dkdv, so that P = exp2(scale * log2(e) * (S - LSE / scale))
 *    needs no per-row term afterwards.
 *  fa_bwd_dkdv: dk, dv. Each (sequence, head, key tile) is taken by one workgroup, which
 *    accumulates dK and dV on chip while walking the query tiles, recomputing P from lse
 *    (at head_dim 128 one persistent workgroup per compute unit takes tile after tile).
 *  fa_bwd_dq: dq. One workgroup per (sequence, head, query tile) accumulates dQ on chip
 *    while walking the key tiles, recomputing P from lse.
 */
/*
 *  fa_bwd_dq_stats: dq, and the workspace statistics of fa_bwd_preprocess (the same
 *    values up to the order of the fp32 additions in D), in one pass: the dQ pass loads
 *    the dO row of each of its queries anyway, and with the O row beside it forms D.
 *    Every query row belongs to exactly one of its tiles. It is what fa_bwd runs first.
 */
int fa_bwd_dq_stats(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse,
                    void* workspace, size_t workspace_bytes, void* dq,
                    int batch, int heads, int seqlen, int head_dim,
                    float softmax_scale, int causal,
                    const int32_t* cu_seqlens, int total_tokens, int dtype, void* stream);

int fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                      void* workspace, size_t workspace_bytes,
                      int batch, int heads, int seqlen, int head_dim, float softmax_scale,
                      const int32_t* cu_seqlens, int total_tokens, int dtype, void* stream);

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                int batch, int heads, int seqlen, int head_dim,
                float softmax_scale, int causal,
                const int32_t* cu_seqlens, int total_tokens, int dtype, void* stream);

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
              const void* workspace, size_t workspace_bytes, void* dq,
              int batch, int heads, int seqlen, int head_dim,
              float softmax_scale, int causal,
              const int32_t* cu_seqlens, int total_tokens, int dtype, void* stream);

/*
 * Decoding: seqlen_q new queries (1..32) attend to a cache of seqlen_k keys and values
 * of which they are the last seqlen_q positions (the pages cite faster inference; the
 * semantics are the forward's with two lengths). q and o are (batch, seqlen_q, heads,
 * head_dim), k and v (batch, seqlen_k, heads, head_dim); lse (batch, heads, seqlen_q).
 * causal != 0: query i sees key j iff j <= seqlen_k - seqlen_q + i (bottom-right
 * alignment; requires seqlen_q <= seqlen_k). bf16 only.
 *
 * The key range is cut into num_splits splits (0 = chosen by the library; otherwise at
 * most ceil(seqlen_k / 64), and fewer may be used since a split is a whole number of
 * 64-key tiles); each is processed independently into the workspace (its O
 * normalised by its own softmax sum, and its logsumexp), then the splits are merged
 * exactly by logsumexp weights ("Softmax en línea": softmax blocks combine through their
 * maxima and sums). Two kernels run on `stream`.
 *
 * fa_fwd_decode_workspace_bytes returns the workspace size for these arguments (the same
 * split choice fa_fwd_decode makes), or 0 if they are invalid. The workspace must be
 * 256-byte aligned and at least that large; its contents on entry do not matter.
 */
size_t fa_fwd_decode_workspace_bytes(int batch, int heads, int seqlen_q, int seqlen_k,
                                     int head_dim, int num_splits);

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  int batch, int heads, int seqlen_q, int seqlen_k, int head_dim,
                  float softmax_scale, int causal, int num_splits,
                  void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * Forward pass on 8-bit inputs ([SA] "FlashAttention-2 (PT)", "Comparação com versões
 * subsequentes": the later FlashAttention-3 adds 8-bit floating point). q, k, v are
 * (batch, seqlen, heads, head_dim) arrays of OCP FP8 E4M3 codes (one byte each: sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN) and
 * the real inputs are descale_q * q, descale_k * k, descale_v * v. Writes o (bf16, same
 * layout, head_dim 64 or 128) and lse (fp32, (batch, heads, seqlen), natural log of the
 * scaled scores' row sums, as fa_fwd). causal: query i sees key j iff j <= i.
 * Both products run on 8-bit MFMAs: the scores S = Q K^T accumulate in fp32, and the
 * probabilities are rounded to E4M3 (round to nearest even, relative error <= 2^-4)
 * before P V; the row sums use the unrounded fp32 P. O therefore differs from the exact
 * attention of the real inputs by about 2^-4 / sqrt(3) of its size in relative L2 (the
 * tests allow 5e-2). Padded batches only (no cu_seqlens). All pointers 16-byte aligned. descale_q and
 * descale_k must be finite and > 0, and so must softmax_scale * descale_q * descale_k
 * (the scale the kernel applies to the raw 8-bit scores); descale_v must be finite.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int batch, int heads, int seqlen, int head_dim,
               float softmax_scale, float descale_q, float descale_k, float descale_v,
               int causal, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). Not from the pages
 * (whose interface is a switch in a training library): the ABI reports errors as status
 * codes instead of exceptions, and this names them. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

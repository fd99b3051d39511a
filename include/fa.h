/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * What is computed.  For each batch b and query head h, with KV head
 * g = h / (Hq / Hkv):
 *     S = (Q[b,h] K[b,g]^T) * scale,   P = row-softmax(S),   O[b,h] = P V[b,g]
 * and per query row LSE = ln(sum_j exp(S_ij)) over the visible keys.
 * This is the standard self-attention of the "flash attention v3 paper"
 * search-result page (standard self-attention snippet: S = QK^T, row softmax,
 * O = PV), with the scale placed after the product as in the "Flash Attention
 * 2 algorithm" pseudocode of "Flash Attention on the 5090 in CUDA C++".
 * It is computed exactly, tile by tile, with the online softmax of that page's
 * "v1 -- basic version" (running max, running denominator, rescaled O), so the
 * Nq x Nk score matrix is never written to memory ("Flash Attention",
 * aiunderstanding.org: deep dive).
 *
 * Readings where the pages say nothing (fixed here):
 *   - layout: every tensor is contiguous row-major, d innermost:
 *       q, o : [B, Hq, Nq, d]     k, v : [B, Hkv, Nk, d]     lse : [B, Hq, Nq]
 *   - causal: key j is visible to query i iff j <= i + (Nk - Nq)
 *     (lower-triangular when Nq == Nk; aligned to the last key otherwise);
 *   - a query row with no visible key gets O = 0 and LSE = -inf;
 *   - LSE is the natural log of the sum of exp of the *scaled* scores.
 *
 * Conventions shared by every entry point.
 *   - All tensor pointers are device pointers owned by the caller.  The
 *     library allocates nothing and frees nothing.  Its only global state is
 *     the fixed scratch array of fa_fwd_splitkv_noalloc (below) and that
 *     array's per-device address, looked up once.
 *   - bf16 tensors are IEEE bfloat16 bit patterns (uint16); fp32 are float.
 *   - Tensor pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; the library never synchronizes.
 *   - Arguments are checked on the host before anything is enqueued.  On any
 *     error nothing is enqueued and a non-zero fa_status is returned.
 *   - A failed kernel launch returns FA_ERR_LAUNCH.  The check reads (and so
 *     clears) the calling thread's pending HIP error.
 *   - B, Nq, Nk may be 0 (nothing to compute, or every row without keys).
 *     Hq, Hkv >= 1 and Hq % Hkv == 0.  d must be 64 or 128 (fa_fwd also
 *     takes 192 and 256; the others return FA_ERR_UNSUPPORTED for them).
 *     scale must be finite and > 0.  causal must be 0 or 1.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* negative size, Hq % Hkv != 0, or sizes overflow */
  FA_ERR_UNSUPPORTED = 3, /* head size or mode not implemented */
  FA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  FA_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch */
  FA_ERR_ARG = 7          /* scale not finite and > 0, causal not 0/1, bad split count */
} fa_status;

/*
 * fa_fwd -- bf16 attention forward (prefill).
 * q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] bf16 in; o [B,Hq,Nq,d] bf16 out (round to
 * nearest even), lse [B,Hq,Nq] fp32 out.  Products run in bf16 with fp32
 * accumulation; the softmax runs in fp32; probabilities are rounded to bf16
 * before the P.V product while the row sums use the unrounded values.
 * d = 64, 128, 192 or 256 (head sizes above 128, the 5090 page's "What next"
 * item, run on their own kernel: 4 waves per 128 query rows, 32-key tiles).
 * o and lse must not overlap the inputs.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, void* stream);

/* Work layouts of fa_fwd, as reported by fa_fwd_layout. */
#define FA_LAYOUT_KV_PARITY 0        /* 128 query rows per workgroup, KV tiles alternate between two wave groups */
#define FA_LAYOUT_KV_PARITY_PAIRED 1 /* the same, causal: query blocks n-1-p and p per workgroup */
#define FA_LAYOUT_ROWS 2             /* 256 query rows per workgroup, both wave groups over every KV tile */
#define FA_LAYOUT_ROWS_PAIRED 3      /* the same, causal pairs */
#define FA_LAYOUT_WIDE_ONE_GROUP 4   /* d = 192/256: 4 waves per 128 rows, two workgroups per CU */
#define FA_LAYOUT_WIDE_TWO_GROUPS 5  /* d = 192/256: 8 waves per 128 rows, KV-parity groups */

/*
 * fa_fwd_layout -- the FA_LAYOUT_* value fa_fwd uses for this shape (the
 * choice depends on the grid size only), or -1 for a head size fa_fwd does
 * not take. Introspection for tests and benchmarks: no argument checks, no
 * GPU work.
 */
int fa_fwd_layout(int B, int Hq, int Nq, int d, int causal);

/*
 * fa_fwd_fp32 -- the same operation in fp32 throughout (debug / reference
 * path; plain FMA arithmetic, no matrix cores).  It computes the standard
 * self-attention defined at the top of this file with the online softmax of
 * the "v1 -- basic version" bullets of "Flash Attention on the 5090 in CUDA
 * C++" taken one key at a time (running max m, running denominator l, O
 * rescaled by exp(m_old - m_new) whenever m rises), with exact expf/logf.
 * Same layout and rules as fa_fwd with float tensors; d = 64 or 128.
 */
fa_status fa_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      float scale, int causal, void* stream);

/*
 * fa_fwd_fp8 -- attention forward over 8-bit inputs.  The pages name MXFP8
 * matrix instructions as the reason to write the kernel by hand ("Flash
 * Attention on the 5090 in CUDA C++", the goal at the top and "What next")
 * and low-precision paths as FlashAttention-3's direction ("Flash Attention",
 * aiunderstanding.org, FAQ), without fixing a format.  Reading taken here:
 * q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] are OCP E4M3 bytes (bias 7, no
 * infinities, 0x7F/0xFF NaN) with one descale factor per tensor; element x
 * stands for e4m3(x) * descale.  The operation is exactly the one above on
 * those values: S = (Q K^T) * scale, O = softmax(S) V, LSE as for fa_fwd.
 * o [B,Hq,Nq,d] bf16 out, lse [B,Hq,Nq] fp32 out.
 * Arithmetic: both products on fp8 matrix cores with fp32 accumulation; the
 * softmax in fp32; probabilities rounded to E4M3 (nearest even) for P.V, the
 * row sums taken before that rounding.  So LSE is as accurate as for bf16,
 * and each O element is within about 2^-4 * sum_j P_ij |V_j| of the exact
 * value (E4M3 keeps 3 mantissa bits).
 * d must be 128 (64 returns FA_ERR_UNSUPPORTED).  Descales must be finite
 * and > 0, and scale * q_descale * k_descale * log2(e) a normal fp32 value,
 * else FA_ERR_ARG.  Other rules as fa_fwd (16-byte alignment of every
 * pointer, 128-byte rows).  NaN inputs are out of contract.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v,
                     float q_descale, float k_descale, float v_descale,
                     void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, void* stream);

/*
 * fa_bwd_workspace_bytes -- bytes of workspace fa_bwd needs: the fp32 row
 * sums D [B,Hq,Nq], rounded up to a multiple of 256.  Returns 0 for invalid
 * sizes (and for Nq = 0).
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq, int d);

/*
 * fa_bwd -- gradients of the bf16 forward.  The pages name the backward pass
 * and training use ("Flash Attention", aiunderstanding.org) but print no
 * algorithm for it; what is computed is the chain rule through the forward
 * definition above.  With dO = dout the gradient of a loss with respect to
 * O, P = exp(S - LSE) recomputed from the forward's lse, and
 * D_i = sum_c dO_ic O_ic:
 *     dV = P^T dO,   dS = P * (dO V^T - D),   dQ = dS K * scale,
 *     dK = dS^T Q * scale,
 * with dK, dV of a KV head summed over its query heads (GQA) and masked
 * entries contributing nothing (a query row without keys gets dQ = 0).
 * q, o, dout, dq [B,Hq,Nq,d] bf16; k, v, dk, dv [B,Hkv,Nk,d] bf16; lse
 * [B,Hq,Nq] fp32 as written by fa_fwd with the same q, k, v, scale, causal.
 * Products run on bf16 matrix cores with fp32 accumulation; P and dS are
 * rounded to bf16 as MFMA operands, D and the softmax are fp32.  dQ is
 * accumulated in registers over all keys (S and dP are computed a second
 * time for it) and rounded to bf16 once; no atomics are used, so the result
 * does not depend on scheduling.
 * d must be 64 or 128.  workspace (device, caller-owned, 256-byte aligned)
 * of at least fa_bwd_workspace_bytes(B,Hq,Nq,d) bytes; its contents are
 * overwritten.  Other rules as fa_fwd; outputs must not overlap the inputs.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_splitkv_workspace_bytes -- bytes of workspace fa_fwd_splitkv needs for
 * its per-chunk partial results (the split of the keys into chunks whose
 * partial softmax results are merged afterwards is the decode scheme the
 * FlashDecoding++ snippet of the "flash attention v3 paper" search-result
 * page refers to): partial outputs O_s [B,Hq,S,Nq,d] fp32 followed (at the
 * next 256-byte boundary) by partial LSE_s [B,Hq,S,Nq] fp32.  Returns 0 for
 * invalid sizes.
 */
size_t fa_splitkv_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits);

/*
 * fa_fwd_splitkv -- split-KV forward (decode): the keys are cut into
 * num_splits contiguous chunks, chunk s = [s*C, min(Nk, (s+1)*C)) with
 * C = ceil(Nk / num_splits).  A first kernel writes, per chunk, the exact
 * attention of every query row over that chunk alone (normalised O_s in fp32
 * and LSE_s) into the workspace; a second kernel (the same as fa_combine)
 * merges them with LSE weights into o (bf16) and lse (fp32).  A chunk with no
 * key has LSE_s = -inf and weight 0.  Split partial results and their merge
 * follow the online-softmax rescale of the "v1 -- basic version" bullets
 * applied to whole chunks; partial-softmax merging is the step the
 * FlashDecoding++ snippet of the "flash attention v3 paper" page names as costly.
 * Requires 1 <= num_splits <= 1024, (Hq/Hkv)*Nq <= 256 query rows per KV head,
 * and workspace_bytes >= fa_splitkv_workspace_bytes(B,Hq,Nq,d,num_splits).
 * The workspace (device memory, caller-owned, 256-byte aligned) holds the
 * partial results after the call and may be inspected by the caller.
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d,
                         float scale, int causal, int num_splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results (bit for bit: the same kernels run) and rules as fa_fwd_splitkv,
 * minus the workspace.  The split partials go to a fixed scratch array of
 * FA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; a call whose partials would not fit, i.e.
 * fa_splitkv_workspace_bytes(B,Hq,Nq,d,num_splits) > FA_NOALLOC_SCRATCH_BYTES,
 * returns FA_ERR_WORKSPACE and enqueues nothing.  The first call on a device
 * looks the scratch up (hipGetSymbolAddress); no call allocates or frees.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialized by the caller.  Nothing in the scratch needs
 * clearing: each call writes every partial it reads.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                 float scale, int causal, int num_splits, void* stream);

/*
 * fa_fwd_splitkv_paged -- fa_fwd_splitkv over a paged K/V cache, one key
 * count per sequence.  PagedAttention appears on the "flash attention v3
 * paper" search-result page only as a name; the cache layout, table and
 * length conventions below are this library's.
 *   k_cache, v_cache : [num_pages, Hkv, page_size, d] bf16 (each page holds
 *                      page_size consecutive keys of one KV head);
 *   block_table      : int32 [B, max_pages]; logical page j of sequence b
 *                      (keys j*page_size .. (j+1)*page_size-1) is physical
 *                      page block_table[b*max_pages + j];
 *   seq_lens         : int32 [B], the number of keys of each sequence
 *                      (0 <= seq_lens[b] <= max_pages * page_size);
 *   q, o, lse        : as fa_fwd_splitkv ([B,Hq,Nq,d], [B,Hq,Nq]).
 * Sequence b is attended as fa_fwd_splitkv attends Nk = seq_lens[b] keys
 * (causal: key j visible to query i iff j <= i + seq_lens[b] - Nq), cut into
 * num_splits chunks of ceil(seq_lens[b] / num_splits) keys, then merged.
 * page_size must be a power of two in [16, 65536].  Table entries outside
 * [0, num_pages) and lengths outside [0, max_pages*page_size] are clamped into
 * range on the device (memory stays in bounds; such results are unspecified).
 * block_table and seq_lens are device pointers, 4-byte aligned; the
 * workspace is the same as fa_fwd_splitkv's (fa_splitkv_workspace_bytes).
 */
fa_status fa_fwd_splitkv_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seq_lens, void* o, float* lse,
                               int B, int Hq, int Hkv, int Nq, int d,
                               int num_pages, int page_size, int max_pages,
                               float scale, int causal, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_combine -- LSE-weighted merge of per-chunk results.  Each chunk's
 * (O_s, LSE_s) is a finished online-softmax state over its keys; merging the
 * states is the rescale step of the "v1 -- basic version" bullets of "Flash
 * Attention on the 5090 in CUDA C++" (scale the older sums by exp(m_old -
 * m_new) when the running max rises, then add) applied to whole chunks.
 * o_part [B,Hq,S,Nq,d] fp32, lse_part [B,Hq,S,Nq] fp32 in; o [B,Hq,Nq,d] bf16
 * and lse [B,Hq,Nq] fp32 out.  With M = max_s LSE_s, w_s = exp(LSE_s - M):
 * O = sum_s w_s O_s / sum_s w_s, LSE = M + ln(sum_s w_s); rows whose chunks
 * are all empty get O = 0, LSE = -inf.  1 <= num_splits <= 1024.
 */
fa_status fa_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                     int B, int Hq, int Nq, int d, int num_splits, void* stream);

/* fa_status_str -- static, human-readable name of a status code. */
const char* fa_status_str(fa_status s);

/*
 * fa_default_scale -- the score scale the "Flash Attention 2 algorithm"
 * pseudocode of "Flash Attention on the 5090 in CUDA C++" uses, DIM**-0.5,
 * for head size d, rounded to fp32 (0 for d < 1).  Callers that have no scale
 * of their own pass this value as `scale`.
 */
float fa_default_scale(int d);

/*
 * fa_build_hash -- static string: the hash of the sources the library was
 * built from (16 hex digits of SHA-256 over csrc/ and include/, as computed by
 * the package's srchash module).  The Python binding refuses a library whose
 * hash differs from its source tree.
 */
const char* fa_build_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

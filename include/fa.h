/*
 * fa.h — C ABI of the MI355X (gfx950) FlashAttention forward library.
 *
 * The library computes exact attention O = softmax(scale * Q K^T) V tile by
 * tile, with the online-softmax update, never writing the score matrix S or
 * the probability matrix P to device memory.  Sources (cited by section):
 *
 *   [FA-notes]   "flash-attn" notes, minjae-portfolio.vercel.app/notes/flash-attn
 *                §3 tiling and fusion, §4 online softmax, §5.2 forward kernel sketch
 *                (per Q tile: loop over K/V tiles, keep row max m and row sum l,
 *                rescale the output accumulator, store the statistics).
 *   [FA-evo]     "Attention is All You Need부터 FlashAttention-3까지: Transformer
 *                Attention 메커니즘의 진화와 O(1) 메모리 최적화 실전 구현", tildalice.io,
 *                section "실전 구현": [batch, seq, heads, head_dim] tensors, causal
 *                masking, bf16/fp16 inputs.
 *   [LLM-basics] "LLM 기초 — Attention부터 FlashAttention까지", gylee815.github.io/llmso/w1,
 *                ①-2 scaled dot-product attention, ①-7 causal mask, ②-3/②-4 KV cache
 *                and decode, ②-7 GQA, ③-1 safe softmax, ③-2 online softmax,
 *                ③-5 FlashAttention's tile loop.
 *   [FA3-entry]  "FlashAttention-3 (FA-3)", itpe.jackerlab.com, §2 (MQA/GQA support)
 *                and §4 (FlashDecoding, an inference-time attention kernel).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, contiguous, row-major, 16-byte
 *     aligned (the decode LSE output and seqlens_k need only 4-byte alignment).  The
 *     caller owns every buffer; the library allocates nothing and never synchronises.
 *     Its only state is a fixed device scratch array (one per GPU, held until the
 *     process ends) used by fa_decode_splitkv_noalloc.  Work is enqueued on `stream`
 *     (NULL = the default stream) and the call returns right after the launch.
 *   - Arguments are validated on the host before any HIP call; a negative
 *     fa_status is returned and nothing is launched.  A launch failure reported
 *     by hipGetLastError returns FA_ERR_HIP.  Device-side faults surface at the
 *     caller's next synchronisation.
 *   - Layouts: Q and O are [B, Nq, Hq, d]; K and V are [B, Nk, Hkv, d]; the
 *     log-sum-exp LSE is [B, Hq, Nq] in natural-log units of the scaled score,
 *     LSE_i = m_i + ln l_i with m_i = max_j S_ij and l_i = sum_j exp(S_ij - m_i).
 *     (The [FA-notes] §5.2 sketch stores l and m separately; LSE carries the same
 *     information: P_ij = exp(S_ij - LSE_i).)
 *   - GQA ([LLM-basics] ②-7): Hq must be a multiple of Hkv; query head h reads
 *     K/V head h / (Hq / Hkv) (consecutive query heads share a K/V head).
 *   - Causal ([LLM-basics] ①-7): key j is visible from query row i iff
 *     j <= i + (Nk - Nq) (rows aligned to the end of the key sequence; for
 *     Nq == Nk this is "token i sees tokens 0..i").  causal with Nq > Nk is
 *     rejected because some rows would see no key at all.
 *   - d (head dimension) must be 64 or 128.
 *   - Sizes: one batch's rows are addressed with 32-bit byte offsets, sized for the
 *     fp32 tensors of the same shape: (Nq + 256) * Hq * d * 4 and (Nk + 256) * Hkv * d * 4
 *     must stay below 2^31 (FA_ERR_SHAPE otherwise; e.g. Nq <= 65279 at Hq = 64,
 *     d = 128), and the grid is one-dimensional.
 *   - Thread safety: every function may be called concurrently from several
 *     host threads; calls on one stream execute in stream order.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* B, H, N or d <= 0; Hq % Hkv != 0; causal with Nq > Nk;
                              sizes whose element counts overflow 32-bit row indexing */
  FA_ERR_UNSUPPORTED = -3, /* d not in {64, 128}; decode chunk or page size not a positive
                              multiple of 64 */
  FA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned (or a packed row
                              stride is not a multiple of 8 elements) */
  FA_ERR_WORKSPACE = -5,   /* decode or backward workspace missing or smaller than required */
  FA_ERR_HIP = -6,         /* the kernel launch failed (hipGetLastError) */
  FA_ERR_SCRATCH = -7      /* fa_decode_splitkv_noalloc: the request needs more than the
                              library's fixed device scratch */
} fa_status;

/*
 * fa_forward — prefill / full-sequence forward, bf16 inputs.
 *
 * [FA-notes] §3-§5.2, [LLM-basics] ③-5: for every (batch, query head, block of
 * query rows) the kernel keeps the Q block on chip, streams the K/V blocks of
 * the matching K/V head through on-chip memory, and for each block updates the
 * running row max m, the running row sum l and the output accumulator
 * (m_new = max(m, block max); acc and l rescaled by exp(m - m_new)).  At the
 * end O = acc / l and LSE = m + ln l are written.  Causal runs skip key blocks
 * that lie wholly in the future of a query block and mask only the blocks that
 * cross the diagonal.
 *
 *   q      bf16  [B, Nq, Hq, d]   (read)
 *   k, v   bf16  [B, Nk, Hkv, d]  (read)
 *   o      fp32  [B, Nq, Hq, d]   (written; every element)
 *   lse    fp32  [B, Hq, Nq]      (written; every element)
 *   scale  multiplier of Q K^T (1/sqrt(d) for standard attention)
 *   causal 0 or 1
 * Scores and the softmax are computed in fp32; QK^T and P V are bf16 x bf16
 * products accumulated in fp32 (P is rounded to bf16 for the second product).
 * Returns FA_OK or a negative fa_status.
 */
int fa_forward(const void* q, const void* k, const void* v, float* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
               hipStream_t stream);

/*
 * fa_forward_f32 — the same contract with fp32 Q, K, V: the attention of [LLM-basics]
 * ①-2 (scores, 1/sqrt(d_k) scaling, row softmax, weighted sum of V) computed with the
 * tile loop of [FA-notes] §5.2.  Everything, including the probabilities multiplied
 * into V, stays in fp32 (nothing is rounded to a 16-bit type).
 */
int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   hipStream_t stream);

/*
 * fa_forward_fp8 — fa_forward with FP8 Q, K, V ([FA3-entry] §3 names FP8 low precision
 * for the forward pass).
 *
 *   q            OCP FP8 E4M3 codes [B, Nq, Hq, d]      (read; value = code * q_descale)
 *   k, v         OCP FP8 E4M3 codes [B, Nk, Hkv, d]     (read; value = code * k/v_descale)
 *   o, lse       fp32 as in fa_forward                  (written)
 *   q_descale, k_descale, v_descale   per-tensor positive finite factors
 * Both products take E4M3 operands with fp32 accumulation: S = scale * q_descale *
 * k_descale * (codes product); the weights P = exp(S - m) are rounded to E4M3 (round to
 * nearest even; every weight is <= 2^8 by construction) for P V, O is normalised by the
 * sum of those rounded weights and scaled by v_descale, and the LSE uses the fp32 sum of
 * the unrounded weights.  Same sizes, alignment and causal rule as fa_forward;
 * FA_ERR_SHAPE also for a descale that is not a positive finite number.
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   float q_descale, float k_descale, float v_descale, hipStream_t stream);

/*
 * fa_forward_varlen — fa_forward over a batch of variable-length sequences packed
 * along the token axis, bf16 inputs.
 *
 * [FA3-entry] §2 lists variable-length inputs among the supported attention forms.
 * Sequence b owns query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key/value
 * tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1 and attends only within itself; each
 * sequence is computed exactly as fa_forward computes one batch entry (the same
 * kernel, causal alignment to the end of that sequence's keys).  No padding is read
 * or computed.
 *
 *   q              bf16, token t, head h at q[t * q_row_stride + h * d + i]   (read)
 *   k, v           bf16, token t, head h at k[t * k_row_stride + h * d + i]   (read)
 *                  (a stride larger than H*d lets q, k, v be views of one packed
 *                  [total, Hq + 2 Hkv, d] QKV tensor)
 *   cu_seqlens_q   int32 [B + 1] on the device, non-decreasing, 0 .. total_q
 *   cu_seqlens_k   int32 [B + 1] on the device, non-decreasing, 0 .. total_k
 *                  (the kernel clamps both into range for memory safety)
 *   o              fp32 [total_q, Hq, d]   (written for every token of every sequence)
 *   lse            fp32 [Hq, total_q]      (written likewise)
 *   max_seqlen_q   longest query sequence, >= 1 (sizes the grid)
 *   max_seqlen_k   longest key sequence, >= 0.  Both are the caller's bound: a sequence
 *                  longer than either is cut to it (only its first max_seqlen_q queries
 *                  are written and its first max_seqlen_k keys read), never read past.
 *                  Byte offsets inside one sequence are 32-bit, so (max_seqlen + 256) *
 *                  row_stride * 2 must stay below 2^31 (FA_ERR_SHAPE); the pack as a whole
 *                  may be larger.
 *   total_q        rows of q, o and lse; total_k: rows of k and v (0 allowed)
 *   q_row_stride   elements between consecutive tokens of q: >= Hq * d, a multiple of 8
 *   k_row_stride   likewise for k, >= Hkv * d; v_row_stride must equal it
 *   causal         0 or 1; key j of a sequence is visible from its query i iff
 *                  j <= i + (Nk_b - Nq_b)
 * A query that sees no key (a sequence with no keys, or under causal masking a query
 * ahead of all keys when Nq_b > Nk_b) gets O = 0 and LSE = -inf.  The cu_seqlens
 * arrays need 4-byte alignment.  Returns FA_OK or a negative fa_status.
 */
int fa_forward_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                      int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                      float scale, int causal, int q_row_stride, int k_row_stride,
                      int v_row_stride, hipStream_t stream);

/*
 * fa_backward_workspace_bytes — helper (no computation): bytes of device workspace
 * fa_backward needs for the two per-row statistics of the backward pass that
 * [FA-notes] §5.2 recomputes from the forward's outputs: two fp32 vectors of
 * B * Hq * Nq entries (D_i and LSE_i log2 e), each padded to 256 bytes.
 * Returns 0 for non-positive sizes.
 */
size_t fa_backward_workspace_bytes(int B, int Hq, int Nq);

/*
 * fa_backward — gradients of the bf16 forward (fa_forward) for an upstream gradient dO.
 *
 * [FA-notes] §5.2 sketches the backward pass: the probabilities are rebuilt on chip from
 * Q, K and the statistics the forward stored, instead of being kept, and dV = P^T dO,
 * dP = dO V^T ([LLM-basics] ③-5 names the same recomputation for training).  The steps
 * the sketch leaves out are the derivative of the row softmax: D_i = sum_j P_ij dP_ij
 * (computed as sum_c dO_ic O_ic), dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * P = exp(scale Q K^T - LSE) uses the forward's LSE directly.  GQA: the dK and dV of a
 * K/V head add up its Hq / Hkv query heads.  Deterministic (no atomics): one kernel
 * forms dK and dV per block of 256 keys, another dQ per block of 128 query rows, each
 * recomputing the S and dP blocks it needs.
 *
 *   q, k, v     as in fa_forward (bf16)                          (read)
 *   o, lse      fp32 O [B, Nq, Hq, d] and LSE [B, Hq, Nq] of the forward on the same
 *               q, k, v, scale and causal flag                    (read)
 *   dout        bf16 dO [B, Nq, Hq, d]                            (read)
 *   dq          fp32 [B, Nq, Hq, d]                               (written; every element)
 *   dk, dv      fp32 [B, Nk, Hkv, d]                              (written; every element)
 *   workspace   at least fa_backward_workspace_bytes(B, Hq, Nq) bytes, 16-byte aligned,
 *               caller-owned; contents on entry do not matter
 * Sizes, alignment and the causal rule are those of fa_forward.  The three kernels run in
 * order on `stream`.  Products are bf16 x bf16 with fp32 accumulation: P and dS are
 * rounded to bf16 for the products that take them.  Returns FA_OK or a negative
 * fa_status.
 */
int fa_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int Nq,
                int Nk, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * fa_decode_splitkv_workspace_bytes — helper (no computation): bytes of device
 * workspace that fa_decode_splitkv needs for these sizes, i.e. the per-piece partial
 * results (O_p, lse_p) that the two-block merge of [FA-notes] §4 combines: fp32, with
 * room for ceil(ceil(Nk_max / 64) / (chunk / 64)) + 1 pieces per (b, query head).
 * Returns 0 for invalid sizes.
 */
size_t fa_decode_splitkv_workspace_bytes(int B, int Hq, int Nk_max, int d, int chunk);

/*
 * fa_decode_splitkv — one decode step over a padded KV cache, split over keys.
 *
 * [LLM-basics] ②-3/②-4: a single new query token per sequence attends to all
 * of that sequence's cached keys and values; [FA3-entry] §4 names a dedicated
 * decode kernel.  The keys of every (b, K/V head) are cut into pieces; kernel 1
 * computes, for every piece, the attention of all Hq/Hkv query heads of that
 * group to the piece's keys: the piece-normalised output O_p and lse_p.  The
 * pieces come from splitting all (b, K/V head) key ranges, laid end to end, into
 * equal runs, one per wave of the GPU, so every wave streams the same number of
 * bytes whatever the length mix; a run is at least `chunk` keys.  Kernel 2
 * merges the pieces of each (b, query head) with the two-block online-softmax
 * merge of [FA-notes] §4 applied across all pieces:
 * LSE = M + ln sum_p exp(lse_p - M), O = sum_p exp(lse_p - LSE) O_p.
 *
 *   q          bf16  [B, Hq, d]             (read)
 *   k_cache    bf16  [B, Nk_max, Hkv, d]    (read; rows >= seqlens_k[b] are never read)
 *   v_cache    bf16  [B, Nk_max, Hkv, d]    (read; rows >= seqlens_k[b] are never read)
 *   seqlens_k  int32 [B] on the device; 1 <= seqlens_k[b] <= Nk_max is the caller's
 *              contract.  The kernels clamp it to [0, Nk_max] for memory safety;
 *              a sequence with 0 keys gets O = 0 and LSE = -inf.
 *   o          fp32  [B, Hq, d]             (written)
 *   lse        fp32  [B, Hq]                (written)
 *   chunk      smallest run of keys one wave takes, a positive multiple of 64 (256 for
 *              the standard setup); it bounds the number of pieces and so the workspace
 *   workspace  device buffer of at least fa_decode_splitkv_workspace_bytes(...)
 *              bytes, 16-byte aligned, owned by the caller; its contents on entry
 *              do not matter and are overwritten.
 * One sequence's K or V rows are addressed with 32-bit byte offsets:
 * (Nk_max + 64) * Hkv * d * 2 must stay below 2^31 (FA_ERR_SHAPE otherwise; a larger
 * cache goes through fa_decode_paged, which addresses page by page).
 * Placement (performance only): the split kernel reads the K row and the V row of one
 * token and head at the same time, and they are v_cache - k_cache bytes apart.  When
 * that distance is a multiple of 1 KiB (two separately allocated, 2 MiB-aligned caches)
 * those reads fall in the same 256-byte address class and the kernel streams about 5%
 * slower on MI355X; any other distance modulo 1 KiB avoids it (the Python helper
 * kv_cache_empty puts V 256 bytes past that class).  The same holds for the page pools
 * of fa_decode_paged.
 * The two kernels run in order on `stream`; stream order is the only
 * synchronisation between them.  Returns FA_OK or a negative fa_status.
 */
int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int* seqlens_k, float* o, float* lse,
                      int B, int Hq, int Hkv, int Nk_max, int d, float scale, int chunk,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode_splitkv_noalloc — fa_decode_splitkv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, computation, results (bit for bit) and errors as
 * fa_decode_splitkv, without the workspace: the split kernel's partial results go to a
 * device scratch array of the library, 80 MiB per GPU (a file-scope device array, so
 * every GPU the library runs on holds its own copy until the process ends).  The call
 * allocates nothing (no hipMalloc / hipFree or allocating library routine).
 *   - A request whose partial results need more than 80 MiB, i.e. more than
 *     fa_decode_splitkv_workspace_bytes(B, Hq, Nk_max, d, chunk) reports, returns
 *     FA_ERR_SCRATCH before any HIP call (the 16-sequence, 64-query-head, d = 128,
 *     Nk_max = 32768, chunk = 256 decode needs 68.2 MB).
 *   - Every call on one GPU uses that GPU's one scratch array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that overlap in
 *     time on one GPU (two streams, two host threads without ordering) race on it and
 *     give undefined results; calls ordered on one stream are safe.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress) with that device current; FA_ERR_HIP if that fails.
 */
int fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seqlens_k, float* o, float* lse, int B, int Hq, int Hkv,
                              int Nk_max, int d, float scale, int chunk, hipStream_t stream);

/*
 * fa_decode_paged — fa_decode_splitkv over a paged KV cache.
 *
 * [LLM-basics] ②-8 (PagedAttention): the cache is a pool of fixed-size pages and each
 * sequence has a block table that maps its logical page j (keys j*page_size ..
 * (j+1)*page_size - 1) to a physical page; sequences may share pages.  The step, the
 * work split and the merge are those of fa_decode_splitkv, with every 64-key step
 * read from the page the table names.
 *
 *   q            bf16  [B, Hq, d]                          (read)
 *   k_pages      bf16  [num_pages, page_size, Hkv, d]      (read; only rows of the pages
 *   v_pages      bf16  [num_pages, page_size, Hkv, d]       a sequence uses, below its length)
 *   block_table  int32 [B, max_pages] on the device; entries 0 <= e < num_pages for the
 *                ceil(seqlens_k[b] / page_size) pages in use (later entries are never
 *                read); the kernel clamps entries into [0, num_pages) for memory safety
 *   seqlens_k    int32 [B] on the device, 1 <= seqlens_k[b] <= max_pages * page_size
 *                (clamped as in fa_decode_splitkv; 0 keys gives O = 0, LSE = -inf)
 *   o, lse       fp32 [B, Hq, d], [B, Hq]                  (written)
 *   page_size    keys per page, a positive multiple of 64
 *   chunk        as in fa_decode_splitkv
 *   workspace    at least fa_decode_splitkv_workspace_bytes(B, Hq, max_pages * page_size,
 *                d, chunk) bytes, 16-byte aligned
 * block_table needs 4-byte alignment.  Returns FA_OK or a negative fa_status.
 */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                    const int* block_table, const int* seqlens_k, float* o, float* lse,
                    int B, int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                    float scale, int chunk, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* fa_status_str — helper (no computation, no page passage): a static, human-readable
 * string for a status code; unknown codes give "unknown fa_status". */
const char* fa_status_str(int status);

/*
 * fa_probe_mfma_bf16 — measurement helper (not an operation of the method, no page
 * passage): the sustained rate of the bf16 matrix cores, for comparing a kernel's rate
 * with what the hardware delivers under the same power limit.  Launches `blocks`
 * workgroups of 256 threads; every thread loads 8 x 16 bytes of `operands` (its four A
 * and four B fragments, bf16) and runs `iters` iterations of four independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) with no other memory traffic, then writes
 * the sum of its accumulators to out[thread].  Work per launch: blocks * 4 * iters * 4 *
 * 32768 FLOP.  operands: device buffer of at least fa_probe_mfma_bf16_operand_bytes(blocks)
 * bytes (operand_bytes gives its size); out: device float[blocks * 256]; both 16-byte
 * aligned and caller-owned.  Errors: FA_ERR_NULL, FA_ERR_SHAPE (blocks or iters not
 * positive, blocks > 2^20, operands too small), FA_ERR_ALIGN, FA_ERR_HIP.
 */
size_t fa_probe_mfma_bf16_operand_bytes(int blocks);
int fa_probe_mfma_bf16(const void* operands, size_t operand_bytes, float* out, int blocks,
                       int iters, hipStream_t stream);

/*
 * fa_probe_stream_read — measurement helper (not an operation of the method, no page
 * passage): the HBM streaming-read rate, for comparing the decode's K/V stream with what
 * plain reads of the same size reach on the same board.  Launches `blocks` workgroups of
 * 256 threads that read every byte of `buf` once, 16 bytes per lane per load with the
 * non-temporal cache policy of the decode's K/V loads, each workgroup taking 32 KB chunks
 * `blocks` chunks apart; thread t of workgroup w writes the XOR of the 32-bit words it read
 * to out[w * 256 + t] (the XOR over all of out equals the XOR of all words of buf).
 * buf: device buffer of `bytes` bytes, 16-byte aligned, bytes a positive multiple of 16 and
 * at most 2^31; out: device uint32[blocks * 256], 4-byte aligned; both caller-owned.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (blocks outside 1..65536, bytes out of range),
 * FA_ERR_ALIGN, FA_ERR_HIP.
 */
int fa_probe_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

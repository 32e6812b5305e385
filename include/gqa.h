/*
 * libgqa -- causal grouped-query attention for AMD Instinct MI355X (gfx950).
 *
 * One operation, with entry points for dense, E4M3, varlen and paged
 * block-sparse causal prefill and for an FP8-cache verifier tail:
 *
 *   O = softmax(scale * Q K^T + mask) V
 *
 * with Hq query heads sharing Hkv K/V heads (query head h reads K/V head
 * h / (Hq/Hkv)), head dimension D, fp16 Q/K/V/O and fp32 accumulation.  A
 * query at position p sees the keys at positions 0..p ("causal").  The shape
 * family is the one of the long-prefill page ("[Kernel][SM70] Default
 * long-prefill GQA architecture", Purpose): Hq = 6, Hkv = 1, D = 256,
 * scale 1/16; this version supports exactly Hkv = 1, Hq = 6 and D = 256 and
 * returns GQA_ERR_UNSUPPORTED for anything else (the page routes other shapes
 * elsewhere, Safety section).
 *
 * Conventions shared by all entry points
 * --------------------------------------
 *  - Every tensor pointer is a DEVICE pointer (memory of the current HIP
 *    device), contiguous, row-major, with the layout stated per argument.
 *    Q and O are [nq][Hq][D] fp16 (IEEE binary16); the caller owns every buffer.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous: they enqueue kernels on `stream` and return; they
 *    never synchronise, never allocate device memory, and keep no state
 *    between calls, so concurrent calls on different streams are safe when
 *    their workspaces differ.  (gqa_verify_fp8kv_noalloc instead uses a fixed
 *    per-device scratch array that the library holds; see there.)
 *  - `workspace` is caller-provided device scratch of at least the size the
 *    matching *_workspace_size() query returns for the same arguments
 *    (NULL is allowed when that size is 0).  Its contents on entry do not
 *    matter and on exit are unspecified.  It must not be shared by calls that
 *    may run at the same time.
 *  - Arguments are validated on the host before anything is enqueued:
 *      GQA_ERR_INVALID      null pointer, non-positive size, positions out of range
 *      GQA_ERR_UNSUPPORTED  a shape outside the supported family
 *      GQA_ERR_WORKSPACE    workspace smaller than the size query demands
 *                           (the typed workspace failure of the long-prefill
 *                           page, Purpose and Safety: the caller can fall back)
 *      GQA_ERR_HIP          a HIP launch failed; gqa_last_hip_error() gives
 *                           the hipError_t of the failing call on this thread
 *    Nothing is enqueued when a call returns anything but GQA_OK.  No C++
 *    exception crosses this interface.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 1

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID = 1,
  GQA_ERR_UNSUPPORTED = 2,
  GQA_ERR_WORKSPACE = 3,
  GQA_ERR_HIP = 4
} gqa_status;

/* ------------------------------------------------------------------------ *
 * Dense causal prefill.
 *
 * Defined by the long-prefill page (Purpose): causal FP16 prefill of
 * Q = 8000 rows against KV = 40000..128000 keys, Hq = 6 heads sharing one K/V
 * head of D = 256, scale 1/16, with the six heads packed together and
 * per-tile online-softmax (max, sum, accumulator) states merged exactly.
 *
 *   q   [nq][hq][d]    fp16, query row r sits at position q_pos0 + r
 *   k,v [n_kv][hkv][d] fp16, key j at position j
 *   o   [nq][hq][d]    fp16 output (round to nearest even of the fp32 result)
 *   requires nq >= 1, q_pos0 >= 0, q_pos0 + nq <= n_kv; scale finite and > 0.
 *   Row r attends to keys 0 .. q_pos0 + r.
 * ------------------------------------------------------------------------ */
gqa_status gqa_prefill_causal_workspace_size(int32_t nq, int32_t n_kv, int32_t q_pos0, int32_t hq, int32_t hkv,
                                             int32_t d, size_t* bytes);

gqa_status gqa_prefill_causal(const void* q, const void* k, const void* v, void* o, int32_t nq, int32_t n_kv,
                              int32_t q_pos0, int32_t hq, int32_t hkv, int32_t d, float scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Causal prefill over E4M3 inputs.
 *
 * The long-context page ("[Perf] Ship the qualified SM70 long-context layout
 * and drop its context fences", What) runs its grouped operator over a K/V
 * cache kept as E4M3 codes with FP32 arithmetic.  Here Q is quantised the same
 * way so that the Q K^T products run on the FP8 matrix cores: the operation is
 * the causal prefill of gqa_prefill_causal applied to the decoded values
 *     Q = decode(q_e4m3) * q_scale,  K = decode(k_e4m3) * k_scale,
 *     V = decode(v_e4m3) * v_scale,
 * with decode the OCP E4M3 ("E4M3FN") format and one fp32 scale per tensor.
 *
 *   q_e4m3 [nq][hq][d] uint8, k_e4m3 / v_e4m3 [n_kv][hkv][d] uint8 (device)
 *   o      [nq][hq][d] fp16 (device), query row r at position q_pos0 + r
 *   scales finite and > 0; the workspace is the one gqa_prefill_causal needs
 *   (same query, gqa_prefill_causal_workspace_size), same shape family and
 *   errors.  Every E4M3 product is exact in fp32; P is rounded to fp16 and
 *   P V accumulates in fp32, as in gqa_prefill_causal.
 * ------------------------------------------------------------------------ */
gqa_status gqa_prefill_causal_e4m3(const uint8_t* q_e4m3, float q_scale, const uint8_t* k_e4m3, float k_scale,
                                   const uint8_t* v_e4m3, float v_scale, void* o, int32_t nq, int32_t n_kv,
                                   int32_t q_pos0, int32_t hq, int32_t hkv, int32_t d, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Varlen causal prefill: a batch of independent sequences packed end to end.
 *
 * The dense causal prefill above, applied to each sequence of a batch the
 * way a serving engine packs requests (the long-prefill page measures the
 * operator under serving, Test Result), with the per-row log-sum-exp
 * returned so that a caller can merge the result with other attention
 * pieces (the exact online-softmax merge of the same page, Purpose).
 *
 *   q, o   [total_q][hq][d] fp16;  k, v [total_kv][hkv][d] fp16
 *   cu_q, cu_kv [batch + 1] int32 in device memory: sequence i owns query
 *          tokens cu_q[i] .. cu_q[i+1]-1 and keys cu_kv[i] .. cu_kv[i+1]-1;
 *          its nq_i queries sit at its last nq_i positions (query j of the
 *          sequence sees its keys 0 .. nkv_i - nq_i + j).  Requires
 *          0 <= cu_q[i] <= cu_q[i+1] <= total_q, the same for cu_kv with
 *          total_kv, and nq_i <= nkv_i; a sequence that breaks this is
 *          skipped (its rows of o and lse are not written) and counted,
 *          see gqa_prefill_causal_varlen_skipped().  Sequences may be empty.
 *   lse    [total_q][hq] fp32 or NULL: natural-log log-sum-exp of each row's
 *          scaled scores, log sum_j exp(scale * q . k_j).
 *   The workspace holds the per-block schedule the device builds from the
 *   offsets and the split-KV partials; its size depends on batch and total_q
 *   only.  Same shape family and errors as gqa_prefill_causal; batch must be
 *   in [1, 2^20].
 * ------------------------------------------------------------------------ */
gqa_status gqa_prefill_causal_varlen_workspace_size(int32_t batch, int32_t total_q, int32_t hq, int32_t hkv,
                                                    int32_t d, size_t* bytes);

gqa_status gqa_prefill_causal_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                     const int32_t* cu_q, const int32_t* cu_kv, int32_t batch, int32_t total_q,
                                     int32_t total_kv, int32_t hq, int32_t hkv, int32_t d, float scale,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Number of sequences the last varlen call on `workspace` skipped as
 * invalid (synchronises `stream`). */
gqa_status gqa_prefill_causal_varlen_skipped(const void* workspace, int32_t* count, void* stream);

/* ------------------------------------------------------------------------ *
 * Paged block-sparse causal prefill.
 *
 * Defined by the block-sparse page ("[Kernel][SM70] Repair #378 on latest
 * main", Changes): selected four-token blocks of a paged page-16 cache are
 * fetched in locality order for the Hq6/Hkv1/D256 prefill, positions are
 * clamped to the live request length and a partial tail block is admitted
 * only for the tokens that exist.  Selecting every block up to the diagonal
 * gives the paged dense causal prefill of the same page (Test Result: the
 * page-16 and page-784 smokes), so any page size that is a multiple of the
 * 4-token block is accepted.
 *
 *   q        [nq][hq][d] fp16, query row r at position q_pos0 + r
 *   k_cache, v_cache [n_pages][page_size][hkv][d] fp16
 *   page_table [n_table] int32: logical page i of the request lives in
 *            physical page page_table[i]; logical token j is in page
 *            j / page_size, slot j % page_size
 *   qblock_offsets [ceil(nq / qblock_rows) + 1] int32 (CSR row pointer) and
 *   kv_block_ids [n_block_ids] int32: query block b (rows b*qblock_rows ..
 *            b*qblock_rows + qblock_rows - 1) selects the logical blocks
 *            kv_block_ids[qblock_offsets[b] .. qblock_offsets[b+1]-1]; block
 *            id x covers tokens x*kv_block_tokens .. x*kv_block_tokens +
 *            kv_block_tokens - 1.  A query block's selection is a set: its
 *            order does not change the result, and a repeated id is dropped
 *            and counted (see below).  The blocks are gathered in logical
 *            order, which keeps the blocks of a page together.  For requests
 *            of more than 262144 blocks (1M tokens) repeats are found only in
 *            selections of up to 2048 ids; a longer selection there is used in
 *            the given order and a repeated id in it counts twice.
 *   Row r of block b sees token j iff j lies in a selected block of b,
 *   j <= q_pos0 + r and j < live_len.  A row that sees nothing outputs 0.
 *   requires q_pos0 >= 0, q_pos0 + nq <= live_len <= n_table * page_size;
 *   this version requires page_size to be a multiple of 4 up to 4096
 *   (16 and 784 in the page's geometries), kv_block_tokens = 4 and
 *   qblock_rows = 64 (GQA_ERR_UNSUPPORTED otherwise).
 *
 *   The index arrays live in device memory and are checked on the device,
 *   not on the host: a block id outside [0, n_table*page_size/kv_block_tokens),
 *   a physical page outside [0, n_pages) or a decreasing/out-of-range offset
 *   is dropped (it contributes nothing, no memory outside the arrays is
 *   touched) and counted, as is each repeated id; gqa_prefill_paged_sparse_dropped()
 *   reads the count.
 * ------------------------------------------------------------------------ */
gqa_status gqa_prefill_paged_sparse_workspace_size(int32_t nq, int32_t n_block_ids, int32_t qblock_rows,
                                                   int32_t kv_block_tokens, int32_t hq, int32_t hkv, int32_t d,
                                                   size_t* bytes);

gqa_status gqa_prefill_paged_sparse(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, int32_t n_table, int32_t n_pages, int32_t page_size,
                                    const int32_t* qblock_offsets, const int32_t* kv_block_ids, int32_t n_block_ids,
                                    int32_t qblock_rows, int32_t kv_block_tokens, int32_t nq, int32_t q_pos0,
                                    int32_t live_len, int32_t hq, int32_t hkv, int32_t d, float scale, void* o,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Number of index entries the last paged call that used `workspace` dropped
 * as invalid or repeated (see above).  Synchronises `stream`; host pointer `count`. */
gqa_status gqa_prefill_paged_sparse_dropped(const void* workspace, int32_t* count, void* stream);

/* ------------------------------------------------------------------------ *
 * FP8 (E4M3) KV verifier tail.
 *
 * Defined by the long-context page ("[Perf] Ship the qualified SM70
 * long-context layout...", What and Changes): a grouped attention operator over
 * an E4M3 K/V cache with fp32 accumulation, used for a speculative-decoding
 * verifier tail of query_rows 2..8 at contexts up to the operator capability
 * of 262144 tokens, and (nq = 1) for the single-row tail the same page routes
 * to its compact operator.
 *
 *   q        [nq][hq][d] fp16: the last nq positions n_kv-nq .. n_kv-1
 *   k_e4m3, v_e4m3 [n_kv][hkv][d] uint8 OCP E4M3 ("E4M3FN") codes; the cached
 *            value is decode(code) * k_scale (resp. v_scale), one fp32 scale
 *            per tensor.  Codes 0x7F / 0xFF (NaN) must not occur.
 *   o        [nq][hq][d] fp16
 *   Row r attends to keys 0 .. n_kv - nq + r (causal among the query rows).
 *   requires 1 <= nq <= 8, nq <= n_kv <= 262144, scales finite and > 0.
 * ------------------------------------------------------------------------ */
gqa_status gqa_verify_fp8kv_workspace_size(int32_t nq, int32_t n_kv, int32_t hq, int32_t hkv, int32_t d,
                                           size_t* bytes);

gqa_status gqa_verify_fp8kv(const void* q, const uint8_t* k_e4m3, const uint8_t* v_e4m3, float k_scale,
                            float v_scale, void* o, int32_t nq, int32_t n_kv, int32_t hq, int32_t hkv, int32_t d,
                            float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * FP8 verifier tail without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).
 *
 * Same operation, arguments, requirements and errors as gqa_verify_fp8kv,
 * without the workspace: the split-KV partials go to a fixed scratch array
 * of 33,816,576 bytes (512 partial slots of 64 rows) that the library holds
 * in device memory, one copy per device, from the library's load until the
 * process ends.  Every valid call fits it (nq <= 8, n_kv <= 262144; anything
 * larger is GQA_ERR_UNSUPPORTED as above).  The call allocates and frees
 * nothing; on its first call on a device it looks up that device's copy of
 * the array (a failure there is GQA_ERR_HIP).
 *
 * All calls on one device share that device's array and it keeps the last
 * call's contents: calls that may run at the same time on one device (other
 * streams, other threads) race on it and must be serialised by the caller.
 * ------------------------------------------------------------------------ */
gqa_status gqa_verify_fp8kv_noalloc(const void* q, const uint8_t* k_e4m3, const uint8_t* v_e4m3, float k_scale,
                                    float v_scale, void* o, int32_t nq, int32_t n_kv, int32_t hq, int32_t hkv,
                                    int32_t d, float scale, void* stream);

/* ------------------------------------------------------------------------ *
 * Kernel timing (observability).
 *
 * Between gqa_profile_start() and gqa_profile_stop() on one host thread, every
 * successful call made by that thread records a pair of HIP events on its
 * stream around its main attention kernel (the one that reads K/V; merge and
 * index kernels are excluded).  The events are timing-only
 * (hipEventDisableSystemFence: recording them writes back no cache).
 * gqa_profile_stop() waits for those events and
 * returns the summed kernel time in milliseconds and the number of kernels
 * timed; it returns GQA_ERR_INVALID when profiling was not started.  This is
 * the only state the library keeps between calls; it is per thread and holds
 * HIP events plus one 16-byte device buffer, allocated by the first
 * gqa_profile_start() on a device and kept until the process ends.
 *
 * While profiling is on, the dense causal prefill kernels (fp16 and E4M3)
 * also add the lifetime of each of their workgroups in shader clock cycles
 * (s_memtime) and in constant-rate wall-clock ticks (s_memrealtime) to that
 * buffer.
 * gqa_profile_clock_mhz() then returns the average shader clock those
 * kernels ran at in the last stopped session, in MHz (0 if none ran or the
 * buffer could not be allocated): the clock against which the matrix-core
 * peak can be rescaled.
 * ------------------------------------------------------------------------ */
gqa_status gqa_profile_start(void);
gqa_status gqa_profile_stop(double* total_ms, int32_t* count);
gqa_status gqa_profile_clock_mhz(double* mhz);

/* ------------------------------------------------------------------------ *
 * Utilities.
 * ------------------------------------------------------------------------ */
/* Static, NUL-terminated description of a status code (never NULL). */
const char* gqa_status_string(gqa_status status);
/* hipError_t (as int) of the last failed HIP call made by this thread, 0 if none. */
int gqa_last_hip_error(void);
/* GQA_ABI_VERSION of the loaded library. */
int gqa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */

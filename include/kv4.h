/*
 * kv4.h -- C ABI of libkv4: single-token decode attention over a paged,
 * calibration-free INT4 KV cache with a bounded INT8 side cache for the
 * attention-sink and recent positions, on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [NEWS] news summary "Async RL squeezes context into fewer decode steps;
 *          INT4 KV cache speeds rollouts but loses accuracy, bounded INT8
 *          protection recovers it": Synopsis; Interpretation paragraphs 1-4.
 *   [ABS]  paper page "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR
 *          with INT4 KV Cache Quantization": The abstract; The Brief.
 *   [ART]  news article on the same paper, section "INT4 as the base, INT8
 *          insurance for critical positions".
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  Structs passed by
 *     pointer are host structs.
 *   - Every call is asynchronous on `stream` and returns a kv4_status.  Host
 *     argument checks happen before anything is launched; on an error nothing
 *     is launched and nothing is written.  KV4_ERR_LAUNCH reports a failed
 *     launch; faults inside a kernel surface at the caller's next stream sync.
 *   - The caller allocates and owns every buffer (pools, side cache, page
 *     table, lengths, q, out, lse, workspace).  The library allocates no
 *     device memory and keeps no mutable global state, except the fixed
 *     per-GPU scratch array of kv4_decode_attention_noalloc; calls on
 *     different streams are independent as long as they do not write the same
 *     pages, side blocks, outputs or workspace (or both use that scratch).
 *   - bf16 / fp16 values are passed as their raw 16-bit patterns (uint16_t).
 *   - Page pools and side caches must be zero-filled when first allocated.
 *     Decode reads whole pages and tiles; rows outside a sequence's context
 *     get weight 0, which is exact only if their bytes are finite numbers --
 *     true for zero fill and for anything append ever wrote.
 *
 * Cache layout (readings: the pages say only "paged INT4" plus an INT8 side
 * cache of at most 144 positions, [NEWS] Interpretation para 3, [ART]):
 *   pages: [num_pages][num_kv_heads][block_bytes]; a page holds 16
 *          consecutive positions of one sequence (page_size = 16).
 *   side:  [num_slots][num_kv_heads][side_bytes]; one side block per
 *          sequence slot holds the INT8 copies of that sequence's protected
 *          positions: sink position p < S in row p, later positions p >= S in
 *          ring row S + ((p - S) mod R).
 *   Quantization (calibration-free, [NEWS] Synopsis; [ABS] The abstract):
 *   symmetric, scale = fp16(min(amax / qmax, 65504)) rounded to nearest even,
 *   code = clamp(rint(x / scale), -qmax, qmax) with fp32 divides; INT4 per
 *   (token, kv head, 32-channel group) with qmax 7, INT8 per (token, kv head)
 *   with qmax 127.  The byte layout inside a block is documented next to
 *   kv4_block_bytes below.
 */
#ifndef KV4_H
#define KV4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV4_ABI_VERSION 5

typedef enum {
  KV4_OK = 0,
  KV4_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad shape        */
  KV4_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim, page...) */
  KV4_ERR_WORKSPACE = -3,   /* workspace smaller than *_workspace_size       */
  KV4_ERR_LAUNCH = -4       /* the HIP runtime rejected a launch             */
} kv4_status;

/* Shapes (host).  Supported: head_dim 64 or 128, page_size 16, group_size 32,
 * num_q_heads a multiple of num_kv_heads, n_sink >= 0, n_recent >= 0 and
 * n_sink + n_recent <= 144 (the bound on the protected set, [NEWS]
 * Interpretation para 3).  n_sink = n_recent = 0 is plain INT4 KV.  The kv8_
 * and kvbf16_ entry points ignore n_sink / n_recent.
 * flags (bit mask; other bits: KV4_ERR_INVALID_ARG):
 *   KV4_LAYOUT_WIDE_PROTECTION lifts the bound to n_sink + n_recent <= 4096,
 *     for studies of wider protection than the method's; same kernels.
 *   KV4_LAYOUT_INT8_QUERY makes kv4_decode_attention / kv4_decode_phases use
 *     the integer query-key path of the "integer attention path" ([NEWS]
 *     Interpretation para 3): each query head's row of q is quantized by the
 *     INT8 row rule (symmetric, fp16 scale from the head's largest |q|,
 *     qmax 127) and multiplied with the INT4 / INT8 key codes in exact integer
 *     arithmetic; probabilities and values are as without the flag.  The
 *     pages do not say how the query enters the integer path: a reading.
 *     kv8_ / kvbf16_ decodes return KV4_ERR_UNSUPPORTED with it; appends
 *     ignore it. */
#define KV4_LAYOUT_WIDE_PROTECTION 1u
#define KV4_LAYOUT_INT8_QUERY 2u
#define KV4_WIDE_PROTECTION_MAX 4096
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t group_size;
  int32_t n_sink;
  int32_t n_recent;
  uint32_t flags;
} kv4_layout;

/* Cache storage (host struct of device pointers). */
typedef struct {
  void* pages;       /* [num_pages][num_kv_heads][block_bytes]          */
  int64_t num_pages;
  void* side;        /* [num_slots][num_kv_heads][kv4_side_bytes]; may be
                        NULL when n_sink + n_recent == 0 or for kv8/kvbf16 */
  int32_t num_slots;
} kv4_cache;

/* One batch of sequences (host struct of device pointers). */
typedef struct {
  const int32_t* page_table; /* [batch][max_pages] physical page ids       */
  int32_t max_pages;         /* row stride of page_table; every sequence
                                must satisfy seq_lens[b] <= 16 * max_pages */
  const int32_t* seq_lens;   /* [batch] context length, counting the tokens
                                appended by kv4_append in this step       */
  const int32_t* slot_ids;   /* [batch] side-cache slot; NULL = slot b     */
  int32_t batch;
} kv4_batch;

/* ---- versioning and status ------------------------------------------------ */
int32_t kv4_abi_version(void);
/* Text of a status code; any other integer gives "unknown status".  Static
 * string, never NULL. */
const char* kv4_status_string(int32_t status);

/* ---- sizes (host) ---------------------------------------------------------- */
/* INT4 page block per (page, kv head), 18 * head_dim bytes (D = head_dim,
 * r = position mod 16, c = channel, q4 = r/4, rr = r%4, t = c/16, n = c%16):
 *   K codes  [0, 8D)    byte r*(D/2) + c/2, low nibble = even channel
 *   V codes  [8D, 16D)  byte (q4*16 + n)*(D/8) + 4*((rr/2)*(D/64) + t/4)
 *                       + 2*(rr%2) + (t%4)/2, low nibble = even t
 *   K scales [16D, 17D) fp16 at byte (grp*16 + r)*2, grp = c/32
 *   V scales [17D, 18D) fp16 likewise
 * Nibbles are two's complement.  Returns 0 for an unsupported layout. */
size_t kv4_block_bytes(const kv4_layout* layout);
/* Side block per (slot, kv head): ceil((S+R)/16) INT8 tiles of 32*D + 64
 * bytes; side row rho is row rho%16 of tile rho/16.  INT8 tile:
 *   K codes  [0, 16D)      byte r*D + c
 *   V codes  [16D, 32D)    byte (q4*16 + n)*(D/4) + t*4 + rr
 *   K scales [32D, 32D+32) fp16 at 2r;  V scales [32D+32, 32D+64) fp16 at 2r */
size_t kv4_side_bytes(const kv4_layout* layout);
/* kv8 pages are single INT8 tiles (32*D + 64 bytes).  kvbf16 pages are 64*D
 * bytes: K bf16 at element r*D + c; V at byte 32D + (q4*16 + n)*(D/2) +
 * t*8 + rr*2. */
size_t kv8_block_bytes(const kv4_layout* layout);
size_t kvbf16_block_bytes(const kv4_layout* layout);

/* ---- append ------------------------------------------------------------------
 * Quantize and store new K/V tokens ([NEWS] Interpretation para 3: the whole
 * context is kept in paged INT4; INT8 copies only for sinks and recent
 * positions).  Sequence b receives n_b = cu_new[b+1] - cu_new[b] tokens at
 * positions seq_lens[b] - n_b ... seq_lens[b] - 1; the caller has already
 * added n_b to seq_lens[b] and mapped the pages of those positions in
 * page_table.  Every new position is written to its INT4 page; a position
 * p < S is also written to sink row p and a position p >= S (when R > 0) to
 * ring row S + ((p - S) mod R) of side block slot_ids[b].
 *   k_new, v_new  bf16 [total_new][num_kv_heads][head_dim]
 *   cu_new        int32 [batch + 1], cu_new[0] = 0, non-decreasing,
 *                 cu_new[batch] = total_new (device)
 *   total_new     number of new tokens (host); 0 is a no-op
 * Inputs must be finite.  Two positions of one call never share a byte, so
 * any number of tokens per sequence may be appended in one call. */
kv4_status kv4_append(const kv4_layout* layout, const kv4_cache* cache,
                      const kv4_batch* batch, const uint16_t* k_new,
                      const uint16_t* v_new, const int32_t* cu_new,
                      int32_t total_new, hipStream_t stream);
/* Same contract; INT8 pages (kv8) or bf16 pages (kvbf16); no side cache. */
kv4_status kv8_append(const kv4_layout* layout, const kv4_cache* cache,
                      const kv4_batch* batch, const uint16_t* k_new,
                      const uint16_t* v_new, const int32_t* cu_new,
                      int32_t total_new, hipStream_t stream);
kv4_status kvbf16_append(const kv4_layout* layout, const kv4_cache* cache,
                         const kv4_batch* batch, const uint16_t* k_new,
                         const uint16_t* v_new, const int32_t* cu_new,
                         int32_t total_new, hipStream_t stream);

/* ---- decode ------------------------------------------------------------------
 * Workspace needed by *_decode_attention for `batch` sequences with page
 * tables of `max_pages` columns (host out-parameter). */
kv4_status kv4_decode_workspace_size(const kv4_layout* layout, int32_t batch,
                                     int32_t max_pages, size_t* bytes);

/* Single-token GQA decode attention.  For sequence b and query head hq
 * (kv head hq / (num_q_heads / num_kv_heads)) over the L = seq_lens[b]
 * positions: sinks [0, min(S, L)) and recent [max(S, L-R), L) are read from
 * the INT8 side cache, which replaces INT4 there; the middle [S, L-R) from the
 * INT4 pages ([NEWS] Interpretation para 3; [ART]).  Scores are
 * softmax_scale * q . k; the regions are combined by an exact log-sum-exp
 * merge ([NEWS] Interpretation para 3), so the result equals one softmax over
 * all positions of the dequantized keys.
 *   q      bf16 [batch][num_q_heads][head_dim]
 *   out    bf16 [batch][num_q_heads][head_dim] (rounded to nearest even)
 *   lse    fp32 [batch][num_q_heads] natural-log sum of exp, or NULL
 * softmax_scale must be positive and finite (KV4_ERR_INVALID_ARG otherwise).
 * KV4_ERR_UNSUPPORTED if batch x ceil(max_pages / 32) x num_kv_heads x
 * ceil(num_q_heads / num_kv_heads / (2048 / head_dim)) reaches 2^31 (the
 * work units are numbered in 32 bits).
 * L = 0 gives out = 0 and lse = -inf.  Arithmetic: exact dequantized
 * products, fp32 accumulation.  The workspace is scratch for this call
 * (PLAN + ATTEND + MERGE of kv4_decode_phases). */
kv4_status kv4_decode_attention(const kv4_layout* layout, const kv4_cache* cache,
                                const kv4_batch* batch, const uint16_t* q,
                                float softmax_scale, uint16_t* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
/* Reference variants at the same shapes: every position from INT8 pages
 * (kv8) or bf16 pages (kvbf16) -- the KV8 and BF16 rollouts the pages compare
 * against ([NEWS] Interpretation para 1). */
kv4_status kv8_decode_attention(const kv4_layout* layout, const kv4_cache* cache,
                                const kv4_batch* batch, const uint16_t* q,
                                float softmax_scale, uint16_t* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);
kv4_status kvbf16_decode_attention(const kv4_layout* layout, const kv4_cache* cache,
                                   const kv4_batch* batch, const uint16_t* q,
                                   float softmax_scale, uint16_t* out, float* lse,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ---- decode in phases -------------------------------------------------------
 * A decode call is three kernels in stream order; *_decode_attention runs all
 * three.  The phased form runs the ones selected by `phases` (bit mask):
 *   KV4_PHASE_PLAN    work list of the batch (reads seq_lens; writes the
 *                     workspace's plan).  The plan depends only on the format,
 *                     the layout, batch, max_pages, seq_lens and slot_ids.
 *   KV4_PHASE_ATTEND  attention over the planned work items: sequences held
 *                     by one item get out / lse, split ones leave fp32
 *                     partials in the workspace.
 *   KV4_PHASE_MERGE   exact log-sum-exp merge of those partials into out / lse
 *                     ([NEWS] Interpretation para 3).
 * The caller orders the phases on streams.  After one PLAN, any number of
 * ATTEND+MERGE pairs may use the plan while the inputs it depends on are
 * unchanged -- e.g. every layer of a decode step, whose layers share the page
 * table and seq_lens but have their own cache and q.  A plan is only valid
 * for the function (format) that made it.  ATTEND+MERGE pairs that share a
 * workspace must not overlap: the partials live there, and so do the counters
 * from which an ATTEND launch's waves draw the end of the work list (the
 * launch leaves them as it found them).  Arguments and
 * errors as for *_decode_attention; `phases` outside 1..7 is
 * KV4_ERR_INVALID_ARG; q/out/cache are not read by PLAN alone (may be NULL). */
#define KV4_PHASE_PLAN 1u
#define KV4_PHASE_ATTEND 2u
#define KV4_PHASE_MERGE 4u
kv4_status kv4_decode_phases(const kv4_layout* layout, const kv4_cache* cache,
                             const kv4_batch* batch, const uint16_t* q,
                             float softmax_scale, uint16_t* out, float* lse,
                             void* workspace, size_t workspace_bytes,
                             uint32_t phases, hipStream_t stream);
kv4_status kv8_decode_phases(const kv4_layout* layout, const kv4_cache* cache,
                             const kv4_batch* batch, const uint16_t* q,
                             float softmax_scale, uint16_t* out, float* lse,
                             void* workspace, size_t workspace_bytes,
                             uint32_t phases, hipStream_t stream);
kv4_status kvbf16_decode_phases(const kv4_layout* layout, const kv4_cache* cache,
                                const kv4_batch* batch, const uint16_t* q,
                                float softmax_scale, uint16_t* out, float* lse,
                                void* workspace, size_t workspace_bytes,
                                uint32_t phases, hipStream_t stream);

/* ---- append + decode in one call ------------------------------------------------
 * One layer's decode step: kv4_append(k_new, v_new, cu_new, total_new) and
 * then kv4_decode_phases(..., phases) on the same batch, with the same results
 * bit for bit.  When `phases` holds KV4_PHASE_PLAN, the plan is made in the
 * launch that stores the new tokens (one extra workgroup): the plan reads
 * only seq_lens, the page table and slot_ids, which the append does not
 * write, so the two latency-bound pieces overlap.  The pages describe the
 * decode step as appending the new token to the paged cache and attending
 * over it ([NEWS] Interpretation para 3); putting both in one call is this
 * library's.  Arguments, errors and contracts are those of the two calls
 * (the cache is required even for phases = KV4_PHASE_PLAN); every argument
 * is checked before anything is launched.  total_new = 0 runs the decode
 * phases alone. */
kv4_status kv4_append_decode_phases(const kv4_layout* layout, const kv4_cache* cache,
                                    const kv4_batch* batch, const uint16_t* k_new,
                                    const uint16_t* v_new, const int32_t* cu_new,
                                    int32_t total_new, const uint16_t* q,
                                    float softmax_scale, uint16_t* out, float* lse,
                                    void* workspace, size_t workspace_bytes,
                                    uint32_t phases, hipStream_t stream);
kv4_status kv8_append_decode_phases(const kv4_layout* layout, const kv4_cache* cache,
                                    const kv4_batch* batch, const uint16_t* k_new,
                                    const uint16_t* v_new, const int32_t* cu_new,
                                    int32_t total_new, const uint16_t* q,
                                    float softmax_scale, uint16_t* out, float* lse,
                                    void* workspace, size_t workspace_bytes,
                                    uint32_t phases, hipStream_t stream);
kv4_status kvbf16_append_decode_phases(const kv4_layout* layout, const kv4_cache* cache,
                                       const kv4_batch* batch, const uint16_t* k_new,
                                       const uint16_t* v_new, const int32_t* cu_new,
                                       int32_t total_new, const uint16_t* q,
                                       float softmax_scale, uint16_t* out, float* lse,
                                       void* workspace, size_t workspace_bytes,
                                       uint32_t phases, hipStream_t stream);

/* ---- multi-query decode ------------------------------------------------------
 * T = num_queries query tokens per sequence (1 <= T <= KV4_MAX_QUERIES): the
 * last T positions of each context, already appended.  Query t of sequence b
 * sits at position N - T + t (N = seq_lens[b]) and attends causally to the
 * n = N - T + t + 1 positions [0, n) of the cache as it stands after the
 * append: sinks [0, min(S, n)) and the positions the ring holds,
 * [max(S, N - R), N) within [0, n), from the INT8 side cache; the rest of
 * [S, n) from the INT4 pages.  Regions are merged exactly as in
 * kv4_decode_attention, which this is for T = 1.  The pages describe the
 * single-token decode step; running several query tokens over one cache
 * state (speculative verification, chunked prefill over the cache) is a
 * reading of this library.
 *   q      bf16 [batch][T][num_q_heads][head_dim]
 *   out    bf16 [batch][T][num_q_heads][head_dim]
 *   lse    fp32 [batch][T][num_q_heads], or NULL
 * Queries with n <= 0 (T > N) give out = 0 and lse = -inf.  The workspace
 * is kv4_decode_workspace_size(layout, batch * T, max_pages); the 2^31-unit
 * bound of kv4_decode_attention applies to batch * T sequences.  With INT4
 * pages at head_dim 128 one work unit serves 16 / G queries of a kv head
 * (G = num_q_heads / num_kv_heads; the MFMA columns are (query, head) pairs),
 * so a block of queries reads and converts its K/V once; otherwise (kv8,
 * kvbf16, head_dim 64, KV4_LAYOUT_INT8_QUERY) each query reads the cache on
 * its own, next to the other queries of its sequence so that the repeats are
 * served from the caches. */
#define KV4_MAX_QUERIES 64
kv4_status kv4_decode_attention_mq(const kv4_layout* layout, const kv4_cache* cache,
                                   const kv4_batch* batch, const uint16_t* q,
                                   int32_t num_queries, float softmax_scale,
                                   uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);
kv4_status kv8_decode_attention_mq(const kv4_layout* layout, const kv4_cache* cache,
                                   const kv4_batch* batch, const uint16_t* q,
                                   int32_t num_queries, float softmax_scale,
                                   uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);
kv4_status kvbf16_decode_attention_mq(const kv4_layout* layout, const kv4_cache* cache,
                                      const kv4_batch* batch, const uint16_t* q,
                                      int32_t num_queries, float softmax_scale,
                                      uint16_t* out, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* ---- decode without a caller workspace ------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and arguments as kv4_decode_attention, without the workspace.
 * The library keeps one scratch array of KV4_NOALLOC_SCRATCH_BYTES per GPU in
 * its code object (each GPU the library runs on holds it until the process
 * ends) and uses the current device's.  It allocates nothing, neither device
 * nor host memory.  A batch whose kv4_decode_workspace_size exceeds
 * KV4_NOALLOC_SCRATCH_BYTES is rejected with KV4_ERR_WORKSPACE before
 * anything is launched (about 3,900 work items at 32 query heads and
 * head_dim 128, e.g. 120 sequences with page tables of 1,040 columns).
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (other streams, other host threads) race and must be ordered by the
 * caller.  The array's contents are never read before a call writes them, so
 * nothing needs clearing between calls.  KV4_ERR_LAUNCH also reports a failed
 * lookup of the array's device address (once per device, on first use). */
#define KV4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kv4_status kv4_decode_attention_noalloc(const kv4_layout* layout, const kv4_cache* cache,
                                        const kv4_batch* batch, const uint16_t* q,
                                        float softmax_scale, uint16_t* out, float* lse,
                                        hipStream_t stream);

/* ---- capacity model (host) ---------------------------------------------------
 * The pages credit part of the end-to-end gain to the higher concurrency a
 * smaller cache allows, and note that a fixed page budget limits it ([NEWS]
 * Perspective paragraphs 1 and 2).  For `num_layers` layers of this layout in
 * `format` (KV4_FORMAT_*), sequence i of `seq_lens` (host array of n lengths,
 * each >= 0) holds ceil(seq_lens[i] / page_size) pages per layer, each of
 * num_kv_heads blocks of *_block_bytes; with KV4_FORMAT_KV4 and
 * n_sink + n_recent > 0 it also holds one side block of kv4_side_bytes per kv
 * head and layer.  Writes *total_bytes, the bytes of all n sequences, and
 * *fit, the largest k such that sequences 0 .. k-1 fit in budget_bytes.
 * Host arithmetic only (no device call); KV4_ERR_INVALID_ARG for a negative
 * length, n < 0, num_layers < 1 or an unknown format. */
#define KV4_FORMAT_KV4 0
#define KV4_FORMAT_KV8 1
#define KV4_FORMAT_BF16 2
kv4_status kv4_cache_capacity(const kv4_layout* layout, int32_t format, int32_t num_layers,
                              const int32_t* seq_lens, int32_t n, uint64_t budget_bytes,
                              uint64_t* total_bytes, int32_t* fit);

/* ---- measurement aid ----------------------------------------------------------
 * Streams `bytes` (a multiple of 16) of `buf` through 128-bit nontemporal
 * loads, each wave reading its own contiguous share in whole-KiB pieces, and
 * stores one XOR-folded word per workgroup into `sink` (device,
 * [kv4_probe_blocks] uint32) so the loads are not removed.  Used to measure
 * the achievable HBM read bandwidth; not part of the decode path. */
int32_t kv4_probe_blocks(void);
kv4_status kv4_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KV4_H */

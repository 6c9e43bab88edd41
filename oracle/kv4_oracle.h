/*
 * kv4_oracle.h -- plain, slow CPU oracle for KV4-RL decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle exists to check the GPU library.
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load it.  It shares no code, header, table or constant with the HIP
 * library under int4_kv_cache_amd/csrc, and it includes nothing from there.
 *
 * Sources (web pages; cited by title and section, never by line):
 *   [NEWS]  news summary "Async RL squeezes context into fewer decode steps;
 *           INT4 KV cache speeds rollouts but loses accuracy, bounded INT8
 *           protection recovers it" -- sections Synopsis, Interpretation
 *           (paragraphs 1-4), Perspective.
 *   [ABS]   paper page "KV4-RL: Unlocking Faster Asynchronous Rollouts for
 *           RLVR with INT4 KV Cache Quantization" -- The abstract; The Brief.
 *   [ART]   news article on the same paper, section "INT4 as the base, INT8
 *           insurance for critical positions".
 *
 * What the pages fix: the whole context is stored in paged INT4 ([NEWS]
 * Interpretation para 3; [ART]); the INT4 quantization needs no calibration
 * ([NEWS] Synopsis; [ABS] The abstract); INT8 copies are kept only for
 * attention-sink and recent positions, at most 144 of them ([NEWS]
 * Interpretation para 3); attention is evaluated region by region and the
 * regions are combined by an exact softmax merge ([NEWS] Interpretation
 * para 3).  Everything else (group size, scale format, rounding, nibble and
 * block layout, the sink/recent split) is a reading of this implementation;
 * each reading is stated where it is used.
 *
 * Arithmetic: quantizer decisions are taken in IEEE fp32 exactly as the GPU
 * takes them (fp32 divide, round-half-even); everything after dequantization
 * is fp64.  Build with -O2 -ffp-contract=off and no fast-math.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py
 * (hand-worked quantizer cases, numpy float16 for the fp16 rounding, closed
 * forms, brute force, torch scaled_dot_product_attention in float64).
 */
#ifndef KV4_ORACLE_H
#define KV4_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache formats. */
#define ORC_FMT_KV4 0  /* INT4 pages for every position + INT8 sink/recent side cache */
#define ORC_FMT_KV8 1  /* INT8 pages for every position (reference variant)          */
#define ORC_FMT_BF16 2 /* bf16 pages for every position (reference variant)          */

typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;   /* 64 or 128 */
  int32_t page_size;  /* 16 */
  int32_t group_size; /* 32 */
  int32_t n_sink;     /* S */
  int32_t n_recent;   /* R */
} orc_layout;

/* ---- scalar conversions -------------------------------------------------- */
float orc_bf16_to_f32(uint16_t b);
double orc_f16_to_f64(uint16_t h);
uint16_t orc_f32_to_f16_rne(float x);

/* ---- quantizer ----------------------------------------------------------- */
/* Symmetric quantization of n bf16 values with one fp16 scale; qmax = 7
 * (INT4 group) or 127 (INT8 row).  Writes n codes and the scale's fp16 bits. */
void orc_quant_sym(const uint16_t* x_bf16, int n, int qmax, int8_t* codes,
                   uint16_t* scale_bits);

/* ---- layout -------------------------------------------------------------- */
size_t orc_block_bytes(int fmt, const orc_layout* L); /* per (page, kv head) */
size_t orc_side_bytes(const orc_layout* L);           /* per (slot, kv head) */
/* Regions of a context of length n: sink [0,*se), middle [*mb,*me),
 * recent [*rb, n).  Empty ranges have begin == end. */
void orc_regions(int n, int S, int R, int* se, int* mb, int* me, int* rb);
/* Side-cache row of protected position p, or -1 if p is never stored there. */
int orc_side_row(int p, int S, int R);

/* ---- append (quantize + pack + place) ------------------------------------ */
int orc_append(int fmt, const orc_layout* L, uint8_t* pages, int64_t num_pages,
               uint8_t* side, int32_t num_slots, const int32_t* page_table,
               int32_t max_pages, const int32_t* seq_lens,
               const int32_t* slot_ids, int32_t batch, const uint16_t* k_new,
               const uint16_t* v_new, const int32_t* cu_new);

/* ---- gather: the dequantized K/V rows the attention reads ---------------- */
/* For sequence b and kv head h writes K[n][D], V[n][D] (fp64) and the region
 * of every position (0 sink, 1 middle, 2 recent).  Returns n or < 0. */
int orc_gather(int fmt, const orc_layout* L, const uint8_t* pages,
               int64_t num_pages, const uint8_t* side, int32_t num_slots,
               const int32_t* page_table, int32_t max_pages,
               const int32_t* seq_lens, const int32_t* slot_ids, int32_t b,
               int32_t h, double* K, double* V, uint8_t* region);

/* ---- attention over explicit rows ---------------------------------------- */
/* Region partials + exact merge, and independently one softmax over all rows.
 * out[D], *lse (natural log), *gap = max |merged - concatenated| / max|concat|. */
void orc_attend(int n, int D, const double* q, const double* K,
                const double* V, const uint8_t* region, double sm_scale,
                double* out, double* lse, double* gap);

/* Softmax distribution over the n positions, in position order. */
void orc_probs(int n, int D, const double* q, const double* K, double sm_scale,
               double* probs);

/* ---- decode -------------------------------------------------------------- */
/* For every sequence in subset (or all when subset == NULL) and every query
 * head: out[i][Hq][D], lse[i][Hq]; *max_gap = largest merge gap seen.
 * q_int8 != 0 selects the integer-query variant of the "integer attention
 * path" ([NEWS] Interpretation para 3): each query head's row of q is first
 * quantized by the same symmetric rule as an INT8 cache row (orc_quant_sym,
 * qmax 127, fp16 scale) and attention uses code x scale in place of q.  The
 * pages do not say how the query enters the integer path; this is a reading. */
int orc_decode(int fmt, const orc_layout* L, const uint8_t* pages,
               int64_t num_pages, const uint8_t* side, int32_t num_slots,
               const int32_t* page_table, int32_t max_pages,
               const int32_t* seq_lens, const int32_t* slot_ids, int32_t batch,
               const uint16_t* q, double sm_scale, const int32_t* subset,
               int32_t n_subset, double* out, double* lse, double* max_gap,
               int32_t nthreads, int32_t q_int8);

/* Multi-query decode: T query tokens per sequence (q [batch][T][Hq][D]);
 * query t of sequence b sees the first N - T + t + 1 positions of the cache
 * as it stands (N = seq_lens[b]), each read from where the cache holds it.
 * out[i][T][Hq][D], lse[i][T][Hq]; queries that see no position give 0 and
 * -inf.  q_int8 as in orc_decode.  T = 1 is orc_decode. */
int orc_decode_mq(int fmt, const orc_layout* L, const uint8_t* pages,
                  int64_t num_pages, const uint8_t* side, int32_t num_slots,
                  const int32_t* page_table, int32_t max_pages,
                  const int32_t* seq_lens, const int32_t* slot_ids, int32_t batch,
                  const uint16_t* q, int32_t T, double sm_scale,
                  const int32_t* subset, int32_t n_subset, double* out,
                  double* lse, double* max_gap, int32_t nthreads, int32_t q_int8);
/* ---- capacity model -------------------------------------------------------- */
/* Bytes of all n sequences (num_layers layers) and the largest k such that
 * sequences 0 .. k-1 fit in budget bytes.  Returns 0, or < 0 on bad input. */
int orc_cache_capacity(int fmt, const orc_layout* L, int32_t num_layers,
                       const int32_t* seq_lens, int32_t n, uint64_t budget,
                       uint64_t* total, int32_t* fit);
#ifdef __cplusplus
}
#endif
#endif

/*
 * kv4_oracle.c -- plain, slow CPU oracle for KV4-RL decode attention.
 *
 * TEST INFRASTRUCTURE ONLY (see kv4_oracle.h for the sources, their tags and
 * the rules).  Written for clarity, not speed: one loop per definition, no
 * blocking, no fusion.
 */
#include "kv4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================== */
/* Scalar conversions                                                        */
/* ======================================================================== */

/* bf16 is the upper half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* Round a binary32 to the nearest binary16, ties to even (IEEE default). */
uint16_t orc_f32_to_f16_rne(float xf) {
  double x = (double)xf; /* exact */
  uint16_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return 0x7E00;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  int E = e - 1; /* a = (1.f) * 2^E */
  if (E < -14) {
    /* subnormal range: a = k * 2^-24; rint rounds half to even */
    double k = rint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)k); /* k == 1024 is the smallest normal */
  }
  double frac = (ldexp(a, -E) - 1.0) * 1024.0; /* exact in fp64 */
  double k = rint(frac);
  if (k == 1024.0) {
    k = 0.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7C00); /* overflow to infinity */
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)k);
}

/* ======================================================================== */
/* Quantizer                                                                 */
/* ======================================================================== */

/*
 * Calibration-free symmetric quantization ([NEWS] Synopsis; [ABS] The
 * abstract): the scale depends only on the values being quantized.
 * Readings (the pages fix none of this): the scale is amax / qmax computed
 * as an fp32 divide, saturated at 65504 and rounded to fp16 (nearest, ties
 * to even); codes are x / scale16 as an fp32 divide, rounded half to even,
 * clamped to [-qmax, qmax].  A zero scale gives all-zero codes.
 */
void orc_quant_sym(const uint16_t* x_bf16, int n, int qmax, int8_t* codes,
                   uint16_t* scale_bits) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float v = fabsf(orc_bf16_to_f32(x_bf16[i]));
    if (v > amax) amax = v;
  }
  float s32 = amax / (float)qmax;
  if (s32 > 65504.0f) s32 = 65504.0f;
  uint16_t h = orc_f32_to_f16_rne(s32);
  *scale_bits = h;
  if (h == 0) {
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return;
  }
  float s16 = (float)orc_f16_to_f64(h); /* exact */
  for (int i = 0; i < n; ++i) {
    float r = orc_bf16_to_f32(x_bf16[i]) / s16;
    float c = rintf(r);
    if (c > (float)qmax) c = (float)qmax;
    if (c < (float)-qmax) c = (float)-qmax;
    codes[i] = (int8_t)c;
  }
}

/* ======================================================================== */
/* Layout                                                                    */
/* ======================================================================== */
/*
 * The pages say "paged INT4" and nothing more ([NEWS] Interpretation para 3;
 * [ART]).  Readings: a page holds 16 consecutive positions of one sequence;
 * the pool is [page][kv head][block]; a side block per (slot, kv head)
 * holds the INT8 copies of the protected positions.  Inside a block, K and
 * V are laid out as below (D = head_dim, r = row = position mod 16,
 * c = channel, q4 = r / 4, rr = r % 4, t = c / 16, n = c % 16).
 *
 *   INT4 page block, 18*D bytes:
 *     K codes   [0, 8D)    byte r*(D/2) + c/2; low nibble = even channel
 *     V codes   [8D, 16D)  byte (q4*16 + n)*(D/8) + 4*((rr/2)*(D/64) + t/4)
 *                          + 2*(rr%2) + (t%4)/2; low nibble = even t
 *                          (a 32-bit word holds 4 channels of positions
 *                          rr and rr+1 of a row quad, one 16-bit half each)
 *     K scales  [16D, 17D) fp16 at (grp*16 + r)*2, grp = c / 32
 *     V scales  [17D, 18D) fp16 likewise
 *   Nibbles hold the code in two's complement.
 *
 *   INT8 tile (16 rows), 32*D + 64 bytes -- side-cache tiles and INT8 pages:
 *     K codes   [0, 16D)    byte r*D + c
 *     V codes   [16D, 32D)  byte (q4*16 + n)*(D/4) + t*4 + rr
 *     K scales  [32D, 32D+32)     fp16 at 2r
 *     V scales  [32D+32, 32D+64)  fp16 at 2r
 *
 *   bf16 tile (16 rows), 64*D bytes -- bf16 pages:
 *     K         [0, 32D)    element r*D + c
 *     V         [32D, 64D)  byte (q4*16 + n)*(D/2) + t*8 + rr*2
 *
 * Side block: ceil((S+R)/16) INT8 tiles; side row rho lives in tile rho/16
 * at row rho%16.
 */

#define PAGE 16

static size_t int4_block(int D) { return (size_t)18 * D; }
static size_t int8_tile(int D) { return (size_t)32 * D + 64; }
static size_t bf16_tile(int D) { return (size_t)64 * D; }

size_t orc_block_bytes(int fmt, const orc_layout* L) {
  int D = L->head_dim;
  if (fmt == ORC_FMT_KV4) return int4_block(D);
  if (fmt == ORC_FMT_KV8) return int8_tile(D);
  return bf16_tile(D);
}

size_t orc_side_bytes(const orc_layout* L) {
  int rows = L->n_sink + L->n_recent;
  int tiles = (rows + PAGE - 1) / PAGE;
  return (size_t)tiles * int8_tile(L->head_dim);
}

/* byte offsets inside the blocks (see the table above) */
static size_t k4_byte(int D, int r, int c) { return (size_t)r * (D / 2) + c / 2; }
static int k4_high(int c) { return c & 1; }
static size_t v4_byte(int D, int r, int c) {
  int q4 = r / 4, rr = r % 4, t = c / 16, n = c % 16;
  int word = (rr / 2) * (D / 64) + t / 4;
  return (size_t)8 * D + (size_t)(q4 * 16 + n) * (D / 8) + 4 * word + 2 * (rr % 2) + (t % 4) / 2;
}
static int v4_high(int c) { return (c / 16) & 1; }
static size_t k4_scale(int D, int r, int c) { return (size_t)16 * D + ((c / 32) * 16 + r) * 2; }
static size_t v4_scale(int D, int r, int c) { return (size_t)17 * D + ((c / 32) * 16 + r) * 2; }

static size_t k8_byte(int D, int r, int c) { return (size_t)r * D + c; }
static size_t v8_byte(int D, int r, int c) {
  int q4 = r / 4, rr = r % 4, t = c / 16, n = c % 16;
  return (size_t)16 * D + (size_t)(q4 * 16 + n) * (D / 4) + t * 4 + rr;
}
static size_t k8_scale(int D, int r) { return (size_t)32 * D + 2 * r; }
static size_t v8_scale(int D, int r) { return (size_t)32 * D + 32 + 2 * r; }

static size_t kb_elem(int D, int r, int c) { return (size_t)2 * (r * D + c); }
static size_t vb_byte(int D, int r, int c) {
  int q4 = r / 4, rr = r % 4, t = c / 16, n = c % 16;
  return (size_t)32 * D + (size_t)(q4 * 16 + n) * (D / 2) + t * 8 + rr * 2;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xFF);
  p[1] = (uint8_t)(v >> 8);
}
static void put_nibble(uint8_t* byte, int high, int8_t code) {
  uint8_t nib = (uint8_t)(code & 0xF);
  if (high)
    *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
  else
    *byte = (uint8_t)((*byte & 0xF0) | nib);
}
static int8_t get_nibble(uint8_t byte, int high) {
  int nib = high ? (byte >> 4) : (byte & 0xF);
  return (int8_t)(nib >= 8 ? nib - 16 : nib); /* two's complement */
}

/* ======================================================================== */
/* Regions and side rows                                                     */
/* ======================================================================== */
/*
 * The protected set is the attention sinks plus the recent context, at most
 * 144 positions ([NEWS] Interpretation para 3; [ABS] The Brief).  Readings:
 * sinks are positions [0, S); recent are the last R positions that are not
 * sinks, [max(S, n-R), n); the middle [S, n-R) is everything else.  Every
 * position is in exactly one region; with n <= S+R nothing is middle.
 */
void orc_regions(int n, int S, int R, int* se, int* mb, int* me, int* rb) {
  *se = n < S ? n : S;
  int r0 = n - R > S ? n - R : S;
  if (r0 > n) r0 = n;
  *rb = r0;
  if (n - R > S) {
    *mb = S;
    *me = n - R;
  } else {
    *mb = *me = *se;
  }
}

/*
 * Side rows.  Reading: a sink position p < S has row p and is written once;
 * a later position p >= S goes to the ring row S + ((p - S) mod R), so the
 * ring always holds the latest R non-sink positions.
 */
int orc_side_row(int p, int S, int R) {
  if (p < S) return p;
  if (R <= 0) return -1;
  return S + (p - S) % R;
}

/* ======================================================================== */
/* Append                                                                    */
/* ======================================================================== */

static void write_int8_row(uint8_t* tile, int D, int r, const uint16_t* k,
                           const uint16_t* v) {
  int8_t codes[128];
  uint16_t s;
  orc_quant_sym(k, D, 127, codes, &s);
  for (int c = 0; c < D; ++c) tile[k8_byte(D, r, c)] = (uint8_t)codes[c];
  wr16(tile + k8_scale(D, r), s);
  orc_quant_sym(v, D, 127, codes, &s);
  for (int c = 0; c < D; ++c) tile[v8_byte(D, r, c)] = (uint8_t)codes[c];
  wr16(tile + v8_scale(D, r), s);
}

static void write_int4_row(uint8_t* blk, int D, int r, const uint16_t* k,
                           const uint16_t* v) {
  int G = 32;
  for (int g0 = 0; g0 < D; g0 += G) {
    int8_t codes[32];
    uint16_t s;
    orc_quant_sym(k + g0, G, 7, codes, &s);
    for (int i = 0; i < G; ++i) put_nibble(blk + k4_byte(D, r, g0 + i), k4_high(g0 + i), codes[i]);
    wr16(blk + k4_scale(D, r, g0), s);
    orc_quant_sym(v + g0, G, 7, codes, &s);
    for (int i = 0; i < G; ++i) put_nibble(blk + v4_byte(D, r, g0 + i), v4_high(g0 + i), codes[i]);
    wr16(blk + v4_scale(D, r, g0), s);
  }
}

static void write_bf16_row(uint8_t* tile, int D, int r, const uint16_t* k,
                           const uint16_t* v) {
  for (int c = 0; c < D; ++c) {
    wr16(tile + kb_elem(D, r, c), k[c]);
    wr16(tile + vb_byte(D, r, c), v[c]);
  }
}

static int layout_ok(const orc_layout* L) {
  if (L->num_kv_heads <= 0 || L->num_q_heads <= 0) return 0;
  if (L->num_q_heads % L->num_kv_heads) return 0;
  if (L->head_dim != 64 && L->head_dim != 128) return 0;
  if (L->page_size != 16 || L->group_size != 32) return 0;
  if (L->n_sink < 0 || L->n_recent < 0) return 0;
  return 1;
}

/*
 * Sequence b receives n_b = cu_new[b+1] - cu_new[b] tokens at positions
 * seq_lens[b] - n_b ... seq_lens[b] - 1 (seq_lens already counts them).
 * KV4: every position is written to its INT4 page ([NEWS] Interpretation
 * para 3: the whole context is in INT4) and, if it is a sink or enters the
 * recent ring, its INT8 copy to the side cache.
 */
int orc_append(int fmt, const orc_layout* L, uint8_t* pages, int64_t num_pages,
               uint8_t* side, int32_t num_slots, const int32_t* page_table,
               int32_t max_pages, const int32_t* seq_lens,
               const int32_t* slot_ids, int32_t batch, const uint16_t* k_new,
               const uint16_t* v_new, const int32_t* cu_new) {
  if (!layout_ok(L)) return -1;
  int D = L->head_dim, H = L->num_kv_heads, S = L->n_sink, R = L->n_recent;
  size_t bb = orc_block_bytes(fmt, L), sb = orc_side_bytes(L);
  for (int b = 0; b < batch; ++b) {
    int nb = cu_new[b + 1] - cu_new[b];
    int len = seq_lens[b];
    int slot = slot_ids ? slot_ids[b] : b;
    for (int i = 0; i < nb; ++i) {
      int p = len - nb + i;
      int t = cu_new[b] + i;
      if (p < 0 || p / PAGE >= max_pages) return -2;
      int64_t pid = page_table[(int64_t)b * max_pages + p / PAGE];
      if (pid < 0 || pid >= num_pages) return -3;
      int r = p % PAGE;
      for (int h = 0; h < H; ++h) {
        const uint16_t* k = k_new + ((size_t)t * H + h) * D;
        const uint16_t* v = v_new + ((size_t)t * H + h) * D;
        uint8_t* blk = pages + ((size_t)pid * H + h) * bb;
        if (fmt == ORC_FMT_KV4) {
          write_int4_row(blk, D, r, k, v);
          int row = orc_side_row(p, S, R);
          if (row >= 0) {
            if (slot < 0 || slot >= num_slots) return -4;
            uint8_t* sblk = side + ((size_t)slot * H + h) * sb;
            write_int8_row(sblk + (size_t)(row / PAGE) * int8_tile(D), D, row % PAGE, k, v);
          }
        } else if (fmt == ORC_FMT_KV8) {
          write_int8_row(blk, D, r, k, v);
        } else {
          write_bf16_row(blk, D, r, k, v);
        }
      }
    }
  }
  return 0;
}

/* ======================================================================== */
/* Gather                                                                    */
/* ======================================================================== */

static void read_int8_row(const uint8_t* tile, int D, int r, double* k, double* v) {
  double sk = orc_f16_to_f64(rd16(tile + k8_scale(D, r)));
  double sv = orc_f16_to_f64(rd16(tile + v8_scale(D, r)));
  for (int c = 0; c < D; ++c) {
    k[c] = (double)(int8_t)tile[k8_byte(D, r, c)] * sk;
    v[c] = (double)(int8_t)tile[v8_byte(D, r, c)] * sv;
  }
}

static void read_int4_row(const uint8_t* blk, int D, int r, double* k, double* v) {
  for (int c = 0; c < D; ++c) {
    double sk = orc_f16_to_f64(rd16(blk + k4_scale(D, r, c)));
    double sv = orc_f16_to_f64(rd16(blk + v4_scale(D, r, c)));
    k[c] = (double)get_nibble(blk[k4_byte(D, r, c)], k4_high(c)) * sk;
    v[c] = (double)get_nibble(blk[v4_byte(D, r, c)], v4_high(c)) * sv;
  }
}

static void read_bf16_row(const uint8_t* tile, int D, int r, double* k, double* v) {
  for (int c = 0; c < D; ++c) {
    k[c] = (double)orc_bf16_to_f32(rd16(tile + kb_elem(D, r, c)));
    v[c] = (double)orc_bf16_to_f32(rd16(tile + vb_byte(D, r, c)));
  }
}

/*
 * KV4: protected positions are read from the INT8 side cache and replace
 * their INT4 copies; the middle is read from the INT4 pages ([NEWS]
 * Interpretation para 3; [ART]).  KV8 and BF16 read every position from
 * their pages (one region).
 */
int orc_gather(int fmt, const orc_layout* L, const uint8_t* pages,
               int64_t num_pages, const uint8_t* side, int32_t num_slots,
               const int32_t* page_table, int32_t max_pages,
               const int32_t* seq_lens, const int32_t* slot_ids, int32_t b,
               int32_t h, double* K, double* V, uint8_t* region) {
  if (!layout_ok(L)) return -1;
  int D = L->head_dim, H = L->num_kv_heads;
  int S = fmt == ORC_FMT_KV4 ? L->n_sink : 0;
  int R = fmt == ORC_FMT_KV4 ? L->n_recent : 0;
  int n = seq_lens[b];
  if (n < 0 || (n + PAGE - 1) / PAGE > max_pages) return -2;
  size_t bb = orc_block_bytes(fmt, L), sb = orc_side_bytes(L);
  int slot = slot_ids ? slot_ids[b] : b;
  int se, mb, me, rb;
  orc_regions(n, S, R, &se, &mb, &me, &rb);
  for (int p = 0; p < n; ++p) {
    int reg = p < se ? 0 : (p >= rb ? 2 : 1);
    region[p] = (uint8_t)reg;
    double* k = K + (size_t)p * D;
    double* v = V + (size_t)p * D;
    if (reg != 1) {
      /* protected: INT8 copy from the side cache */
      if (slot < 0 || slot >= num_slots) return -4;
      int row = orc_side_row(p, S, R);
      const uint8_t* sblk = side + ((size_t)slot * H + h) * sb;
      read_int8_row(sblk + (size_t)(row / PAGE) * int8_tile(D), D, row % PAGE, k, v);
    } else {
      int64_t pid = page_table[(int64_t)b * max_pages + p / PAGE];
      if (pid < 0 || pid >= num_pages) return -3;
      const uint8_t* blk = pages + ((size_t)pid * H + h) * bb;
      if (fmt == ORC_FMT_KV4)
        read_int4_row(blk, D, p % PAGE, k, v);
      else if (fmt == ORC_FMT_KV8)
        read_int8_row(blk, D, p % PAGE, k, v);
      else
        read_bf16_row(blk, D, p % PAGE, k, v);
    }
  }
  return n;
}

/* ======================================================================== */
/* Attention                                                                 */
/* ======================================================================== */

static double score(int D, const double* q, const double* k, double sm) {
  double s = 0.0;
  for (int c = 0; c < D; ++c) s += q[c] * k[c];
  return sm * s;
}

/*
 * Exact regional softmax merge ([NEWS] Interpretation para 3).  Each region
 * r gives m_r = max s_j, l_r = sum exp(s_j - m_r), o_r = sum exp(s_j - m_r) V_j.
 * With M = max_r m_r:  o = sum_r e^(m_r-M) o_r / sum_r e^(m_r-M) l_r and
 * lse = M + ln sum_r e^(m_r-M) l_r.  This is algebraically one softmax over
 * all positions; that single softmax is also computed and the largest
 * relative difference reported as *gap.
 */
void orc_attend(int n, int D, const double* q, const double* K,
                const double* V, const uint8_t* region, double sm,
                double* out, double* lse, double* gap) {
  for (int c = 0; c < D; ++c) out[c] = 0.0;
  *gap = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  for (int j = 0; j < n; ++j) s[j] = score(D, q, K + (size_t)j * D, sm);

  /* region partials */
  double m[3] = {-INFINITY, -INFINITY, -INFINITY}, l[3] = {0, 0, 0};
  double* o = (double*)calloc((size_t)3 * D, sizeof(double));
  int nonempty[3] = {0, 0, 0};
  for (int j = 0; j < n; ++j) {
    int r = region ? region[j] : 1;
    nonempty[r] = 1;
    if (s[j] > m[r]) m[r] = s[j];
  }
  for (int j = 0; j < n; ++j) {
    int r = region ? region[j] : 1;
    double e = exp(s[j] - m[r]);
    l[r] += e;
    for (int c = 0; c < D; ++c) o[r * D + c] += e * V[(size_t)j * D + c];
  }
  /* merge */
  double M = -INFINITY;
  for (int r = 0; r < 3; ++r)
    if (nonempty[r] && m[r] > M) M = m[r];
  double ltot = 0.0;
  for (int r = 0; r < 3; ++r)
    if (nonempty[r]) ltot += exp(m[r] - M) * l[r];
  for (int c = 0; c < D; ++c) {
    double acc = 0.0;
    for (int r = 0; r < 3; ++r)
      if (nonempty[r]) acc += exp(m[r] - M) * o[r * D + c];
    out[c] = acc / ltot;
  }
  *lse = M + log(ltot);

  /* independent check: one softmax over the concatenated rows */
  double mc = -INFINITY, lc = 0.0, omax = 0.0, dmax = 0.0;
  for (int j = 0; j < n; ++j)
    if (s[j] > mc) mc = s[j];
  for (int j = 0; j < n; ++j) lc += exp(s[j] - mc);
  for (int c = 0; c < D; ++c) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j) acc += exp(s[j] - mc) * V[(size_t)j * D + c];
    acc /= lc;
    if (fabs(acc) > omax) omax = fabs(acc);
    if (fabs(acc - out[c]) > dmax) dmax = fabs(acc - out[c]);
  }
  *gap = omax > 0 ? dmax / omax : dmax;
  free(o);
  free(s);
}

void orc_probs(int n, int D, const double* q, const double* K, double sm,
               double* probs) {
  if (n <= 0) return;
  double mx = -INFINITY, tot = 0.0;
  for (int j = 0; j < n; ++j) {
    probs[j] = score(D, q, K + (size_t)j * D, sm);
    if (probs[j] > mx) mx = probs[j];
  }
  for (int j = 0; j < n; ++j) {
    probs[j] = exp(probs[j] - mx);
    tot += probs[j];
  }
  for (int j = 0; j < n; ++j) probs[j] /= tot;
}

/* ======================================================================== */
/* Decode                                                                    */
/* ======================================================================== */
/*
 * Single-token GQA decode: query head hq attends with kv head hq / g,
 * g = Hq / Hkv (reading: contiguous head groups).  q is bf16, used exactly.
 */
int orc_decode(int fmt, const orc_layout* L, const uint8_t* pages,
               int64_t num_pages, const uint8_t* side, int32_t num_slots,
               const int32_t* page_table, int32_t max_pages,
               const int32_t* seq_lens, const int32_t* slot_ids, int32_t batch,
               const uint16_t* q, double sm, const int32_t* subset,
               int32_t n_subset, double* out, double* lse, double* max_gap,
               int32_t nthreads, int32_t q_int8) {
  if (!layout_ok(L)) return -1;
  int D = L->head_dim, H = L->num_kv_heads, Hq = L->num_q_heads, g = Hq / H;
  int nseq = subset ? n_subset : batch;
  int nwork = nseq * H;
  int status = 0;
  double gap_all = 0.0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(max : gap_all) reduction(min : status)
#endif
  for (int w = 0; w < nwork; ++w) {
    int i = w / H, h = w % H;
    int b = subset ? subset[i] : i;
    if (b < 0 || b >= batch) {
      status = -5;
      continue;
    }
    int n = seq_lens[b];
    size_t rows = n > 0 ? (size_t)n : 1;
    double* K = (double*)malloc(sizeof(double) * rows * D);
    double* V = (double*)malloc(sizeof(double) * rows * D);
    uint8_t* reg = (uint8_t*)malloc(rows);
    int rc = orc_gather(fmt, L, pages, num_pages, side, num_slots, page_table,
                        max_pages, seq_lens, slot_ids, b, h, K, V, reg);
    if (rc < 0) {
      status = rc;
    } else {
      for (int j = 0; j < g; ++j) {
        int hq = h * g + j;
        double qv[128];
        const uint16_t* qrow = q + ((size_t)b * Hq + hq) * D;
        if (q_int8) {
          /* integer query: the INT8 row quantizer, then code x scale */
          int8_t qc[128];
          uint16_t qs;
          orc_quant_sym(qrow, D, 127, qc, &qs);
          for (int c = 0; c < D; ++c) qv[c] = (double)qc[c] * orc_f16_to_f64(qs);
        } else {
          for (int c = 0; c < D; ++c) qv[c] = (double)orc_bf16_to_f32(qrow[c]);
        }
        double gap;
        orc_attend(n, D, qv, K, V, reg, sm, out + ((size_t)i * Hq + hq) * D,
                   lse + (size_t)i * Hq + hq, &gap);
        if (gap > gap_all) gap_all = gap;
      }
    }
    free(K);
    free(V);
    free(reg);
  }
  *max_gap = gap_all;
  return status;
}

/* Multi-query decode (a reading of this library: the pages describe the
 * single-token step).  Query t of sequence b sits at position N - T + t of a
 * cache holding N = seq_lens[b] positions and sees the first
 * n_t = N - T + t + 1 of them, each read from where the cache holds it after
 * the append: the side cache for sinks and for the positions the ring still
 * holds, the INT4 pages for the rest ([NEWS] Interpretation para 3).  That is
 * exactly a prefix of the rows orc_gather returns for the whole cache, so
 * every query attends over the first n_t gathered rows. */
int orc_decode_mq(int fmt, const orc_layout* L, const uint8_t* pages,
                  int64_t num_pages, const uint8_t* side, int32_t num_slots,
                  const int32_t* page_table, int32_t max_pages,
                  const int32_t* seq_lens, const int32_t* slot_ids, int32_t batch,
                  const uint16_t* q, int32_t T, double sm, const int32_t* subset,
                  int32_t n_subset, double* out, double* lse, double* max_gap,
                  int32_t nthreads, int32_t q_int8) {
  if (!layout_ok(L) || T < 1) return -1;
  int D = L->head_dim, H = L->num_kv_heads, Hq = L->num_q_heads, g = Hq / H;
  int nseq = subset ? n_subset : batch;
  int nwork = nseq * H;
  int status = 0;
  double gap_all = 0.0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(max : gap_all) reduction(min : status)
#endif
  for (int w = 0; w < nwork; ++w) {
    int i = w / H, h = w % H;
    int b = subset ? subset[i] : i;
    if (b < 0 || b >= batch) {
      status = -5;
      continue;
    }
    int N = seq_lens[b];
    size_t rows = N > 0 ? (size_t)N : 1;
    double* K = (double*)malloc(sizeof(double) * rows * D);
    double* V = (double*)malloc(sizeof(double) * rows * D);
    uint8_t* reg = (uint8_t*)malloc(rows);
    int rc = orc_gather(fmt, L, pages, num_pages, side, num_slots, page_table,
                        max_pages, seq_lens, slot_ids, b, h, K, V, reg);
    if (rc < 0) {
      status = rc;
    } else {
      for (int t = 0; t < T; ++t) {
        int n = N - T + t + 1;
        if (n < 0) n = 0;
        for (int j = 0; j < g; ++j) {
          int hq = h * g + j;
          double qv[128];
          const uint16_t* qrow = q + (((size_t)b * T + t) * Hq + hq) * D;
          if (q_int8) {
            /* the integer-query variant, as in orc_decode */
            int8_t qc[128];
            uint16_t qs;
            orc_quant_sym(qrow, D, 127, qc, &qs);
            for (int c = 0; c < D; ++c) qv[c] = (double)qc[c] * orc_f16_to_f64(qs);
          } else {
            for (int c = 0; c < D; ++c) qv[c] = (double)orc_bf16_to_f32(qrow[c]);
          }
          double gap;
          size_t o = ((size_t)i * T + t) * Hq + hq;
          orc_attend(n, D, qv, K, V, reg, sm, out + o * D, lse + o, &gap);
          if (gap > gap_all) gap_all = gap;
        }
      }
    }
    free(K);
    free(V);
    free(reg);
  }
  *max_gap = gap_all;
  return status;
}

/* Cache bytes of a batch and how many of its sequences fit in a budget
 * ([NEWS] Perspective paragraphs 1 and 2: a smaller cache allows higher
 * concurrency, and a fixed page budget limits it).  A sequence of length L
 * holds ceil(L / page_size) pages per layer, each of num_kv_heads blocks;
 * KV4 with protection adds one side block per kv head and layer. */
int orc_cache_capacity(int fmt, const orc_layout* L, int32_t num_layers,
                       const int32_t* seq_lens, int32_t n, uint64_t budget,
                       uint64_t* total, int32_t* fit) {
  if (!layout_ok(L) || num_layers < 1 || n < 0) return -1;
  uint64_t page = (uint64_t)orc_block_bytes(fmt, L) * (uint64_t)L->num_kv_heads;
  uint64_t side = 0;
  if (fmt == ORC_FMT_KV4 && L->n_sink + L->n_recent > 0)
    side = (uint64_t)orc_side_bytes(L) * (uint64_t)L->num_kv_heads;
  uint64_t sum = 0;
  int32_t k = 0;
  int over = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (seq_lens[i] < 0) return -2;
    uint64_t pages = ((uint64_t)seq_lens[i] + (uint64_t)L->page_size - 1) / (uint64_t)L->page_size;
    sum += (pages * page + side) * (uint64_t)num_layers;
    if (!over && sum <= budget) k = i + 1;
    else over = 1;
  }
  *total = sum;
  *fit = k;
  return 0;
}

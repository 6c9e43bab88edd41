// kv4_common.h -- device helpers and the cache byte layout shared by the
// libkv4 kernels (gfx950, wave64).  The layout is the one documented in
// include/kv4.h; every offset below is a byte offset inside one block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4.h"

namespace kv4 {

constexpr int kPage = 16;   // positions per page
constexpr int kGroup = 32;  // channels per INT4 scale group
constexpr int kWave = 64;
constexpr int kMaxProtected = 144;  // sinks + recent, the pages' bound

// kFmtKV4Q8: the KV4 cache read with an INT8-quantized query (the integer
// query-key products of the "integer attention path" variant).
enum Format : int { kFmtKV4 = 0, kFmtKV8 = 1, kFmtBF16 = 2, kFmtKV4Q8 = 3 };

// ---- block sizes ------------------------------------------------------------
__host__ __device__ constexpr size_t int4_block_bytes(int D) { return size_t(18) * D; }
__host__ __device__ constexpr size_t int8_tile_bytes(int D) { return size_t(32) * D + 64; }
__host__ __device__ constexpr size_t bf16_tile_bytes(int D) { return size_t(64) * D; }
__host__ __device__ constexpr int side_tiles(int S, int R) { return (S + R + kPage - 1) / kPage; }

// ---- INT4 page block (r = row, c = channel) ----------------------------------
// K codes: row-major nibbles, even channel in the low nibble.
__host__ __device__ constexpr size_t k4_byte(int D, int r, int c) { return size_t(r) * (D / 2) + c / 2; }
// V codes: tiled so that the 4 positions of a row quad and the D/16 channels
// n, n+16, ... sit in one contiguous D/8-byte run.  A 32-bit word holds 4 of
// those channels for positions rr (low half) and rr+1 (high half); a byte
// holds channels c and c+16 (c/16 even in the low nibble) of one position.
__host__ __device__ constexpr size_t v4_byte(int D, int r, int c) {
  return size_t(8) * D + size_t((r / 4) * 16 + c % 16) * (D / 8) +
         4 * (((r % 4) / 2) * (D / 64) + (c / 16) / 4) + 2 * ((r % 4) % 2) + ((c / 16) % 4) / 2;
}
__host__ __device__ constexpr size_t k4_scale(int D, int r, int grp) { return size_t(16) * D + (grp * 16 + r) * 2; }
__host__ __device__ constexpr size_t v4_scale(int D, int r, int grp) { return size_t(17) * D + (grp * 16 + r) * 2; }

// ---- INT8 tile (side cache rows and kv8 pages) -------------------------------
__host__ __device__ constexpr size_t k8_byte(int D, int r, int c) { return size_t(r) * D + c; }
__host__ __device__ constexpr size_t v8_byte(int D, int r, int c) {
  return size_t(16) * D + size_t((r / 4) * 16 + c % 16) * (D / 4) + (c / 16) * 4 + (r % 4);
}
__host__ __device__ constexpr size_t k8_scale(int D, int r) { return size_t(32) * D + 2 * r; }
__host__ __device__ constexpr size_t v8_scale(int D, int r) { return size_t(32) * D + 32 + 2 * r; }

// ---- bf16 tile (kvbf16 pages) ------------------------------------------------
__host__ __device__ constexpr size_t kb_byte(int D, int r, int c) { return size_t(2) * (r * D + c); }
__host__ __device__ constexpr size_t vb_byte(int D, int r, int c) {
  return size_t(32) * D + size_t((r / 4) * 16 + c % 16) * (D / 2) + (c / 16) * 8 + (r % 4) * 2;
}

// ---- regions -----------------------------------------------------------------
// sink [0, se), middle [mb, me), recent [rb, n).
struct Regions {
  int se, mb, me, rb;
};
// Regions of a query that sees positions [0, n) of a cache holding N >= n
// positions: sinks [0, se), middle [mb, me) from the INT4 pages, recent
// [rb, n) from the ring, which holds positions [max(S, N - R), N).
__host__ __device__ inline Regions regions_in(int n, int N, int S, int R) {
  Regions g;
  g.se = n < S ? n : S;
  const int ring0 = N - R > S ? N - R : S;
  const int cut = n < ring0 ? n : ring0;  // end of the INT4 region
  if (n > S) {
    g.mb = S;
    g.me = cut;
    g.rb = cut;
  } else {
    g.mb = g.me = g.rb = g.se;
  }
  return g;
}
// Regions of a context of length n (its last position is the query).
__host__ __device__ inline Regions regions(int n, int S, int R) { return regions_in(n, n, S, R); }
// Side row of protected position p (p < S: sink row; else ring row).
__host__ __device__ inline int side_row(int p, int S, int R) { return p < S ? p : S + (p - S) % R; }

// ---- scalar conversions ------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ inline float f16_to_f32(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
// Round to nearest even (the hardware default rounding mode).
__device__ inline uint16_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, _Float16(x)); }
__device__ inline uint16_t f32_to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, __bf16(x)); }

// ---- the symmetric quantizer (append and the integer query) -------------------
// scale = fp16_rne(min(amax / qmax, 65504)), fp32 divide; returns its bits.
__device__ inline uint16_t quant_scale_bits(float amax, float qmax) {
  return f32_to_f16_bits(fminf(amax / qmax, 65504.0f));
}
// code = clamp(rint(x / scale), -qmax, qmax) (fp32 divide, ties to even); 0 if scale is 0.
__device__ inline int quant_code(float x, float scale, float qmax) {
  if (scale == 0.0f) return 0;
  return int(fminf(fmaxf(rintf(x / scale), -qmax), qmax));
}

// ---- wave reductions ---------------------------------------------------------
template <int WIDTH>
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
template <int WIDTH>
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace kv4

// decode.hip -- single-token GQA decode attention over the paged caches,
// with QK^T and PV on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Three kernels on the caller's stream:
//   1. worklist  (1 workgroup): per sequence, the number of work items.  The
//      middle region is cut into chunks of kChunkPages pages; item 0 also
//      carries the protected rows (INT8 sinks + recent ring).
//   2. attention (persistent grid; one wave per unit = item x kv head x head
//      block): online softmax over the item's 16-row tiles, two tiles (32
//      positions) per step.  A sequence with one item writes the bf16 output
//      and lse directly, otherwise an fp32 partial (o, m, l).
//   3. merge: exact log-sum-exp merge of the partials of split sequences.
// Processing sinks, middle and recent rows in one online softmax, or in
// partials merged by log-sum-exp, both equal one softmax over all positions:
// the exact regional merge of the news summary "Async RL squeezes context
// into fewer decode steps; ...", Interpretation paragraph 3.
//
// Matrix-core mapping (rows m = (head, 32-channel group): 4 heads x 4 groups
// at head_dim 128, 8 x 2 at 64):
//   QK  A = 16 positions x 32 channels of K codes, B = q with row m holding
//       only its own group's channels, so D[pos][m] is the per-group partial
//       dot product; the per-(position, group) INT4 scale is applied after.
//   PV  A = p * v_scale for row m (its group's scale), K = 32 positions,
//       B = V codes of 16 channels; row m is used only for channels of its
//       group.  p is split into bf16 hi + lo so the product keeps ~16 bits.
// INT4 codes enter the MFMA as the exact bf16 value 1 + (code + 8)/128: the
// nibble becomes the low four mantissa bits, one bit operation per pair of
// codes plus a shift for all but the lowest nibble pair of a word.  The
// constant part is removed through the accumulator input (-(1 + 8/128) times
// the sum of the other operand), which leaves sum(x * code) / 128 exactly up
// to fp32 rounding.
#include "kv4_common.h"
#include "kv4_launch.h"
#include "append_body.h"

#include <mutex>

namespace kv4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef float f32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));

// Tuning constants (each value measured against its neighbours on MI355X).
constexpr int kChunkPages = 32;        // smallest chunk of middle pages per work item
constexpr int kWavesPerEU = 2;         // attention waves per SIMD (215 of 256 registers)
constexpr int kStages4 = 2;            // register pipeline depth of the INT4 page loop (3 and 4: 1% slower)
constexpr int kStages8 = 2;            // pipeline depth of the INT8 tile loops; bf16 tiles use 1
constexpr int kUnitsPerWave = 4;       // work-list granularity: chunk size from the total work
constexpr int kMergeK = 4;             // partial rows a merge task loads per round (8: 104 registers, slower)
constexpr int kMaxChunkPages = 128;    // largest chunk of the single-query kernel (two page ids per lane)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.0f;  // re-reference the running max when it grows by 2^8
constexpr int kAttnThreads = 512;  // single-query attention workgroup: two waves per SIMD of one CU
// fp32 partial of one (item, query head): o[D], m, l, two words of padding so
// that rows start on 16-byte boundaries
__host__ __device__ constexpr int part_stride(int D) { return D + 4; }

enum Kind : int { kInt4Page = 0, kInt8Tile = 1, kBf16Page = 2 };

__device__ inline bf16x8_t bf8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ inline f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef int i32x4_t __attribute__((__vector_size__(16)));
// int8 x int8 -> int32, 16 x 16 x 64: A lane L byte e = (row L%16, k 16(L/16)+e),
// B lane L byte e = (k 16(L/16)+e, column L%16), D as for the bf16 MFMA.
__device__ inline i32x4_t mfma_i8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, const uint32_t (&b)[4],
                                  i32x4_t c) {
  const i32x4_t va = {int(a0), int(a1), int(a2), int(a3)}, vb = {int(b[0]), int(b[1]), int(b[2]), int(b[3])};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(va, vb, c, 0, 0, 0);
}
// two fp32 -> packed bf16 pair, round to nearest even
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((__vector_size__(4)));
  bf16x2_t v;
  v[0] = __bf16(lo);
  v[1] = __bf16(hi);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// two small exact integers in fp32 -> bf16 pair (the low halves are zero)
__device__ inline uint32_t pack_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ inline float h2f_lo(uint32_t w) { return f16_to_f32(uint16_t(w & 0xFFFF)); }
__device__ inline float h2f_hi(uint32_t w) { return f16_to_f32(uint16_t(w >> 16)); }
// x * (fp16 half of w) as one mixed-precision FMA.  The +0 addend keeps the
// FMA from being folded into a multiply (and then into a neighbouring add);
// the sign of a zero product is irrelevant to every use here.
__device__ inline float mul_h_lo(float x, uint32_t w) { return fmaf(x, h2f_lo(w), 0.0f); }
__device__ inline float mul_h_hi(float x, uint32_t w) { return fmaf(x, h2f_hi(w), 0.0f); }
// max of three finite-or-infinite floats in one instruction (fmaxf would first
// quiet signalling NaNs of operands the compiler cannot prove canonical; no
// NaN reaches this point)
__device__ inline float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float sbyte(uint32_t w, int k) { return float(int32_t(w << (24 - 8 * k)) >> 24); }

// INT4 encoding: code c -> bf16 1 + (c + 8)/128, the nibble (sign bit flipped)
// in the low four mantissa bits.
constexpr float kEnc = 128.0f;
constexpr float kEncConst = 1.0f + 8.0f / kEnc;              // 1.0625
constexpr uint32_t kEncMask = 0x000F000Fu;
constexpr uint32_t kEncBits = 0x3F883F88u;                   // 1.0 with the sign bit of the code flipped

// INT4: nibbles k and k+4 of d -> bf16 pair 1 + (code+8)/128.
template <int K>
__device__ inline uint32_t nib_pair(uint32_t d) {
  return ((d >> (4 * K)) & kEncMask) ^ kEncBits;
}
__device__ inline uint32_t nib_pair_at(uint32_t d, int k) {  // k in 0..3 (unrolled)
  switch (k) {
    case 0: return nib_pair<0>(d);
    case 1: return nib_pair<1>(d);
    case 2: return nib_pair<2>(d);
    default: return nib_pair<3>(d);
  }
}

// x >> S for a register pair in one instruction (the compiler splits a
// 64-bit shift into two 32-bit ones).
template <int S>
__device__ inline uint64_t shr64(uint64_t x) {
  uint64_t y;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(y) : "I"(S), "v"(x));
  return y;
}
// Nibble pairs K of words a and b (b the next register), K = 1..3 from one
// shift of the pair: the high word's nibbles that enter the top of the low
// word land in bits the mask drops.
template <int K>
__device__ inline void nib_pairs2(uint32_t a, uint32_t b, uint32_t& oa, uint32_t& ob) {
  if constexpr (K == 0) {
    oa = nib_pair<0>(a);
    ob = nib_pair<0>(b);
  } else {
    const uint64_t y = shr64<4 * K>((uint64_t(b) << 32) | a);
    oa = (uint32_t(y) & kEncMask) ^ kEncBits;
    ob = (uint32_t(y >> 32) & kEncMask) ^ kEncBits;
  }
}

// Cross-lane moves inside groups of 4 lanes (DPP quad permutations).
__device__ inline float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ inline float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// value of lane E of this lane's group of 4
template <int E>
__device__ inline float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), E * 0x55, 0xF, 0xF, true));
}
// Reduce-scatter over groups of 4 lanes: lane g of a group gets the sum over
// the group of element x[g].  Two exchange levels (partner g ^ 2, then g ^ 1);
// at each, a lane keeps the half of its elements that its own index selects
// and adds the partner's copy of the same half.
__device__ inline float quad_reduce_scatter(const float (&x)[4], int lane) {
  const bool b2 = (lane & 2) != 0, b1 = (lane & 1) != 0;
  const float y0 = (b2 ? x[2] : x[0]) + quad_xor2(b2 ? x[0] : x[2]);
  const float y1 = (b2 ? x[3] : x[1]) + quad_xor2(b2 ? x[1] : x[3]);
  return (b1 ? y1 : y0) + quad_xor1(b1 ? y0 : y1);
}

// ------------------------------------------------------------ tile loads --
// Every load is (uniform block base) + (per-lane 32-bit offset, fixed for the
// kernel), which maps to global_load with a scalar base and costs no vector
// address arithmetic per tile.
template <int KIND, int D>
struct LaneOff {
  uint32_t k, v, ks, vs;
  uint32_t sc;      // INT4, D = 128: this lane's dword of the scale area
  int put, get;     // INT4, D = 128: where it goes in the wave's LDS slot, where the lane's four are
  __device__ inline LaneOff(int ln, int kg) : sc(0), put(0), get(0) {
    constexpr int NG = D / 32;
    if constexpr (KIND == kInt4Page) {
      k = ln * (D / 2) + kg * (D / 8);
      v = 8 * D + (kg * 16 + ln) * (D / 8);
      ks = 16 * D + ((ln % NG) * 16 + kg * 4) * 2;
      vs = ks + D;
      // At D = 128 the four lanes kg * 16 + g + 4j (j = 0..3, one query head
      // each) need the same scales: group g of positions 4kg..4kg+3, two K
      // dwords and two V dwords.  Lane j of them loads dword j only (every
      // lane one distinct dword of the 256-byte scale area) and each lane
      // gathers the four from its group (ds_bpermute addresses in src).
      const int j = ln >> 2;
      sc = (j < 2 ? ks : vs) + 4 * (j & 1);
      // LDS slot positions: the group's four dwords next to each other
      put = kg * 16 + (ln % NG) * 4 + j;
      get = kg * 16 + (ln % NG) * 4;
    } else if constexpr (KIND == kInt8Tile) {
      k = ln * D + kg * (D / 4);
      v = 16 * D + (kg * 16 + ln) * (D / 4);
      ks = 32 * D + kg * 8;
      vs = ks + 32;
    } else {
      k = (ln * D + kg * (D / 4)) * 2;
      v = 32 * D + (kg * 16 + ln) * (D / 2);
      ks = vs = 0;
    }
  }
};

// Tile reads go through a buffer resource whose range is the tile, so a load
// issued for a step past the end of a run (the pipeline issues every load
// unconditionally) gets an empty range and returns zeros without reading
// memory.  INT4 pages that no other sequence of the batch shares are read
// with the nontemporal hint: every load instruction covers whole 128-byte
// lines and each byte is read once per decode step, and on gfx950 the hint
// raises the sustained streaming read rate.  Shared prompt pages, INT8 and
// bf16 tiles keep the default policy: the first are read again by the other
// sequences of the group, the others are read in half-line pieces, and both
// need their lines to stay in the caches in between.
struct TileSrc {
  __amdgpu_buffer_rsrc_t r;
  __device__ inline TileSrc(const uint8_t* base, int bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), short(0), bytes, 0x00020000)) {}
};

typedef uint32_t ldv4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ldv2_t __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ inline uint4 ld16(const TileSrc& t, uint32_t off) {
  const ldv4_t r = __builtin_amdgcn_raw_buffer_load_b128(t.r, off, 0, NT ? 2 : 0);
  return make_uint4(r.x, r.y, r.z, r.w);
}

template <bool NT>
__device__ inline uint2 ld8(const TileSrc& t, uint32_t off) {
  const ldv2_t r = __builtin_amdgcn_raw_buffer_load_b64(t.r, off, 0, NT ? 2 : 0);
  return make_uint2(r.x, r.y);
}

template <bool NT>
__device__ inline uint32_t ld4(const TileSrc& t, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(t.r, off, 0, NT ? 2 : 0);
}

template <int KIND, int D>
struct Tile;

template <int D>
struct Tile<kInt4Page, D> {
  static constexpr int KW = D / 32;  // dwords of K codes per lane (D/8 bytes)
  uint32_t k[KW];
  uint32_t v[KW];
  uint32_t ks[2], vs[2];  // fp16 scales of positions 4kg..4kg+3, group = ln % NG
  uint32_t sc;            // D = 128: this lane's dword of the scales, until `gather`
  static constexpr int kBytes = int(int4_block_bytes(D));
  template <bool NT>
  __device__ inline void load(const TileSrc& blk, const LaneOff<kInt4Page, D>& o) {
    if constexpr (KW == 4) {
      const uint4 a = ld16<NT>(blk, o.k);
      const uint4 b = ld16<NT>(blk, o.v);
      k[0] = a.x; k[1] = a.y; k[2] = a.z; k[3] = a.w;
      v[0] = b.x; v[1] = b.y; v[2] = b.z; v[3] = b.w;
      // one dword per lane: the texture path moves every lane's bytes, and
      // the 8-byte scale loads of the four lanes sharing them cost a third of
      // a tile's load time
      sc = ld4<NT>(blk, o.sc);
    } else {
      const uint2 a = ld8<NT>(blk, o.k);
      const uint2 b = ld8<NT>(blk, o.v);
      k[0] = a.x; k[1] = a.y;
      v[0] = b.x; v[1] = b.y;
      const uint2 s = ld8<NT>(blk, o.ks);
      const uint2 t = ld8<NT>(blk, o.vs);
      ks[0] = s.x; ks[1] = s.y;
      vs[0] = t.x; vs[1] = t.y;
    }
  }
  // After the loads have arrived: each lane's scales from the lanes that
  // loaded them, through the wave's own 256-byte LDS slot (the exchange stays
  // within the wave, whose LDS operations complete in order).
  __device__ inline void gather(const LaneOff<kInt4Page, D>& o, uint32_t* slot) {
    if constexpr (KW == 4) {
      slot[o.put] = sc;
      __builtin_amdgcn_wave_barrier();
      const uint4 x = *reinterpret_cast<const uint4*>(slot + o.get);
      __builtin_amdgcn_wave_barrier();
      ks[0] = x.x; ks[1] = x.y;
      vs[0] = x.z; vs[1] = x.w;
    }
  }
};

template <int D>
struct Tile<kInt8Tile, D> {
  static constexpr int KW = D / 16;  // D/4 bytes per lane
  uint32_t k[KW];
  uint32_t v[KW];
  uint32_t ks[2], vs[2];
  static constexpr int kBytes = int(int8_tile_bytes(D));
  template <bool NT>
  __device__ inline void load(const TileSrc& tile, const LaneOff<kInt8Tile, D>& o) {
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const uint4 a = ld16<NT>(tile, o.k + 16 * i);
      const uint4 b = ld16<NT>(tile, o.v + 16 * i);
      k[4 * i] = a.x; k[4 * i + 1] = a.y; k[4 * i + 2] = a.z; k[4 * i + 3] = a.w;
      v[4 * i] = b.x; v[4 * i + 1] = b.y; v[4 * i + 2] = b.z; v[4 * i + 3] = b.w;
    }
    const uint2 s = ld8<NT>(tile, o.ks);
    const uint2 t = ld8<NT>(tile, o.vs);
    ks[0] = s.x; ks[1] = s.y;
    vs[0] = t.x; vs[1] = t.y;
  }
  __device__ inline void gather(const LaneOff<kInt8Tile, D>&, uint32_t*) {}
};

template <int D>
struct Tile<kBf16Page, D> {
  static constexpr int KW = D / 8;  // D/2 bytes per lane
  uint32_t k[KW];
  uint32_t v[KW];
  static constexpr int kBytes = int(bf16_tile_bytes(D));
  template <bool NT>
  __device__ inline void load(const TileSrc& tile, const LaneOff<kBf16Page, D>& o) {
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const uint4 a = ld16<NT>(tile, o.k + 16 * i);
      const uint4 b = ld16<NT>(tile, o.v + 16 * i);
      k[4 * i] = a.x; k[4 * i + 1] = a.y; k[4 * i + 2] = a.z; k[4 * i + 3] = a.w;
      v[4 * i] = b.x; v[4 * i + 1] = b.y; v[4 * i + 2] = b.z; v[4 * i + 3] = b.w;
    }
  }
  __device__ inline void gather(const LaneOff<kBf16Page, D>&, uint32_t*) {}
};

// ----------------------------------------------------------- unit state --
template <int D>
struct Unit {
  static constexpr int NG = D / 32;  // scale groups per head
  static constexpr int NT = D / 16;  // PV N-tiles
  bf16x8_t bq[NG];                   // q operand per QK MFMA
  float qsum;                        // sum of this lane's row (head, group) of q
  uint32_t q8[(D / 64) > 0 ? D / 64 : 1][4];  // integer query: INT8 codes per i8 MFMA
  int cin8;                          // integer query: -8 x the row group's code sum
  f32x4_t o[NT];                     // PV accumulators (D layout)
  f32x4_t corr;                      // INT4 V-encoding correction per row (D layout)
  float m;                           // running max (log2 units) of head ln / NG
  float l;                           // this lane's share of the softmax denominator
  float qk_scale;                    // softmax_scale * log2(e)
};

// QK for one tile -> x[e] = per-group partial score of position 4kg+e, before
// the softmax scale (and, for INT4, before the factor kEnc of the encoding).
template <int KIND, int D, bool Q8>
__device__ inline void qk_tile(const Unit<D>& u, const Tile<KIND, D>& T, float (&x)[4]) {
  constexpr int NG = D / 32;
  f32x4_t acc;
  if constexpr (Q8 && KIND != kBf16Page) {
    // Integer query: i8 MFMAs over 64 channels (16 per lane, taken in the
    // order even channels then odd channels of each 8-channel half, which is
    // how the nibbles unpack; the query codes are stored in the same order).
    constexpr int MQ = D / 64;
    i32x4_t ai;
    if constexpr (KIND == kInt4Page) {
      // nibble -> byte (code + 8); the offset is removed through cin8
      ai = i32x4_t{u.cin8, u.cin8, u.cin8, u.cin8};
#pragma unroll
      for (int t = 0; t < MQ; ++t) {
        const uint32_t d0 = T.k[2 * t], d1 = T.k[2 * t + 1];
        ai = mfma_i8((d0 & 0x0F0F0F0Fu) ^ 0x08080808u, ((d0 >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u,
                     (d1 & 0x0F0F0F0Fu) ^ 0x08080808u, ((d1 >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u, u.q8[t], ai);
      }
    } else {
      ai = i32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < MQ; ++t) {
        const uint32_t w0 = T.k[4 * t], w1 = T.k[4 * t + 1], w2 = T.k[4 * t + 2], w3 = T.k[4 * t + 3];
        ai = mfma_i8(__builtin_amdgcn_perm(w1, w0, 0x06040200u), __builtin_amdgcn_perm(w1, w0, 0x07050301u),
                     __builtin_amdgcn_perm(w3, w2, 0x06040200u), __builtin_amdgcn_perm(w3, w2, 0x07050301u), u.q8[t],
                     ai);
      }
    }
    acc = f32x4_t{float(ai[0]), float(ai[1]), float(ai[2]), float(ai[3])};
  } else if constexpr (KIND == kInt4Page) {
    const float c = -kEncConst * u.qsum;
    acc = f32x4_t{c, c, c, c};
#pragma unroll
    for (int t = 0; t < NG; t += 2) {
      uint32_t a[4], b[4];
      nib_pairs2<0>(T.k[t], T.k[t + 1], a[0], b[0]);
      nib_pairs2<1>(T.k[t], T.k[t + 1], a[1], b[1]);
      nib_pairs2<2>(T.k[t], T.k[t + 1], a[2], b[2]);
      nib_pairs2<3>(T.k[t], T.k[t + 1], a[3], b[3]);
      acc = mfma(bf8(a[0], a[1], a[2], a[3]), u.bq[t], acc);
      acc = mfma(bf8(b[0], b[1], b[2], b[3]), u.bq[t + 1], acc);
    }
  } else if constexpr (KIND == kInt8Tile) {
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      const uint32_t w0 = T.k[2 * t], w1 = T.k[2 * t + 1];
      acc = mfma(bf8(pack_exact(sbyte(w0, 0), sbyte(w1, 0)), pack_exact(sbyte(w0, 1), sbyte(w1, 1)),
                     pack_exact(sbyte(w0, 2), sbyte(w1, 2)), pack_exact(sbyte(w0, 3), sbyte(w1, 3))),
                 u.bq[t], acc);
    }
  } else {
    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NG; ++t)
      acc = mfma(bf8(T.k[4 * t], T.k[4 * t + 1], T.k[4 * t + 2], T.k[4 * t + 3]), u.bq[t], acc);
  }
  if constexpr (KIND == kBf16Page) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = acc[e];
  } else {
    x[0] = mul_h_lo(acc[0], T.ks[0]);
    x[1] = mul_h_hi(acc[1], T.ks[0]);
    x[2] = mul_h_lo(acc[2], T.ks[1]);
    x[3] = mul_h_hi(acc[3], T.ks[1]);
  }
}

// V operand of PV N-tile t from two tiles: positions 4kg..4kg+3 of T0 then of
// T1, channel 16t + ln.  Rows outside the context get p = 0; their bytes are
// finite (written by append, or the zero fill the pools start from), so they
// contribute exactly 0.
template <int KIND, int D>
__device__ inline bf16x8_t v_operand(const Tile<KIND, D>& T0, const Tile<KIND, D>& T1, int t) {
  if constexpr (KIND == kInt4Page) {
    // word (pair*(D/64) + t/4) holds channel 16t+n of positions (2 pair,
    // 2 pair + 1) as nibble t%4 of its low and high half.
    constexpr int QW = D / 64;
    const int j = t & 3, w = t >> 2;
    return bf8(nib_pair_at(T0.v[w], j), nib_pair_at(T0.v[QW + w], j), nib_pair_at(T1.v[w], j),
               nib_pair_at(T1.v[QW + w], j));
  } else if constexpr (KIND == kInt8Tile) {
    const uint32_t a = T0.v[t], b = T1.v[t];
    return bf8(pack_exact(sbyte(a, 0), sbyte(a, 1)), pack_exact(sbyte(a, 2), sbyte(a, 3)),
               pack_exact(sbyte(b, 0), sbyte(b, 1)), pack_exact(sbyte(b, 2), sbyte(b, 3)));
  } else {
    return bf8(T0.v[2 * t], T0.v[2 * t + 1], T1.v[2 * t], T1.v[2 * t + 1]);
  }
}

// Per-head value (held by score-layout lane head*NG) for the PV-layout
// accumulator element e of this lane.
template <int D>
__device__ inline float head_value_for_acc(float v, int lane, int e) {
  constexpr int NG = D / 32;
  if constexpr (NG == 4) {
    return __shfl(v, (lane >> 4) * 4, kWave);
  } else {
    return __shfl(v, ((lane >> 4) * 2 + (e >> 1)) * 2, kWave);
  }
}

template <int KIND, int D>
__device__ inline void pv_step(Unit<D>& u, const Tile<KIND, D>& T0, const Tile<KIND, D>& T1, const float (&pr)[8]);

// One step: two 16-row tiles (32 positions).  mask0/mask1: 16-bit row masks.
template <int KIND, int D, bool MASKED, bool Q8>
__device__ inline void step(Unit<D>& u, const Tile<KIND, D>& T0, const Tile<KIND, D>& T1, uint32_t mask0,
                            uint32_t mask1, int lane) {
  constexpr int NG = D / 32;
  constexpr int NT = D / 16;
  const int kg = lane >> 4;
  const uint32_t va0 = (mask0 >> (4 * kg)) & 15u, va1 = (mask1 >> (4 * kg)) & 15u;

  float x0[4], x1[4];
  qk_tile<KIND, D, Q8>(u, T0, x0);
  qk_tile<KIND, D, Q8>(u, T1, x1);
  // score (log2 units) = sc * x; INT4 partials carry the encoding's 1/kEnc
  const float sc = (KIND == kInt4Page && !Q8) ? kEnc * u.qk_scale : u.qk_scale;
  if constexpr (NG == 4) {
    // Lanes 4h..4h+3 hold the four group partials of head h for positions
    // 4kg..4kg+3.  Lane 4h+g sums position 4kg+g only and takes its
    // exponential; the PV operand then gathers the four probabilities of the
    // group of lanes.  One exponential per position instead of four.
    float z0 = quad_reduce_scatter(x0, lane), z1 = quad_reduce_scatter(x1, lane);
    if ((mask0 & mask1) != 0xFFFFu) {  // wave-uniform: only partial steps are masked
      const int g = lane & 3;
      z0 = ((va0 >> g) & 1u) ? z0 : -INFINITY;
      z1 = ((va1 >> g) & 1u) ? z1 : -INFINITY;
    }
    float mx = fmaxf(z0, z1);
    if (__any(mx * sc > u.m + kRescale)) {  // wave-uniform, rare
      mx = fmaxf(mx, quad_xor1(mx));
      mx = fmaxf(mx, quad_xor2(mx));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mn = fmaxf(u.m, mx * sc);
      const float alpha = (mn == u.m) ? 1.0f : __builtin_amdgcn_exp2f(u.m - mn);
      u.l *= alpha;
      u.m = mn;
      // only the accumulator element of each N-tile that holds the head's
      // own group is used (the others are discarded at the end)
      const float r = head_value_for_acc<D>(alpha, lane, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) u.corr[e] *= r;
#pragma unroll
      for (int t = 0; t < NT; ++t) u.o[t][t / 2] *= r;
    }
    const float mneg = u.m == -INFINITY ? 0.0f : -u.m;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(z0, sc, mneg));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(z1, sc, mneg));
    u.l += p0 + p1;
    float pr[8];
    pr[0] = quad_bcast<0>(p0);
    pr[1] = quad_bcast<1>(p0);
    pr[2] = quad_bcast<2>(p0);
    pr[3] = quad_bcast<3>(p0);
    pr[4] = quad_bcast<0>(p1);
    pr[5] = quad_bcast<1>(p1);
    pr[6] = quad_bcast<2>(p1);
    pr[7] = quad_bcast<3>(p1);
    pv_step<KIND, D>(u, T0, T1, pr);
    return;
  }
  // head_dim 64: sum the two group partials of a head (lanes 2h, 2h+1)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x0[e] += quad_xor1(x0[e]);
    x1[e] += quad_xor1(x1[e]);
    if constexpr (NG == 4) {
      x0[e] += quad_xor2(x0[e]);
      x1[e] += quad_xor2(x1[e]);
    }
  }
  if ((mask0 & mask1) != 0xFFFFu) {  // wave-uniform: only partial steps are masked
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] = ((va0 >> e) & 1u) ? x0[e] : -INFINITY;
      x1[e] = ((va1 >> e) & 1u) ? x1[e] : -INFINITY;
    }
  }
  float mx = max3(max3(x0[0], x0[1], x0[2]), max3(x0[3], x1[0], x1[1]), max3(x1[2], x1[3], -INFINITY));

  // The running max of a head is only re-referenced when a score exceeds it
  // by 2^kRescale (then to the head's exact maximum so far), so p <= 2^8 and
  // the accumulators are rescaled rarely; the result does not depend on it.
  // The accumulators are multiplied on every step (by 1 when the reference
  // stays): a multiply only inside the branch makes the compiler copy every
  // accumulator on the path that skips it.
  float r01 = 1.0f, r23 = 1.0f;  // factor for accumulator elements 0-1 / 2-3
  if (__any(mx * sc > u.m + kRescale)) {
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mn = fmaxf(u.m, mx * sc);
    const float alpha = (mn == u.m) ? 1.0f : __builtin_amdgcn_exp2f(u.m - mn);
    u.l *= alpha;
    u.m = mn;
    r01 = head_value_for_acc<D>(alpha, lane, 0);
    r23 = NG == 2 ? head_value_for_acc<D>(alpha, lane, 2) : r01;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) u.corr[e] *= e < 2 ? r01 : r23;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int e0 = t / 2;
    u.o[t][e0] *= e0 < 2 ? r01 : r23;
    if constexpr (NG == 2) u.o[t][e0 + 2] *= r23;
  }

  // p = 2^(sc*x - m); masked rows have x = -inf -> p = 0
  const float mneg = u.m == -INFINITY ? 0.0f : -u.m;
  float pr[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pr[e] = __builtin_amdgcn_exp2f(fmaf(x0[e], sc, mneg));
    pr[e + 4] = __builtin_amdgcn_exp2f(fmaf(x1[e], sc, mneg));
  }
  u.l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  pv_step<KIND, D>(u, T0, T1, pr);
}

// PV of one step from the probabilities pr[e] of this lane's head at the
// positions of its A operand (4kg + e of T0, then of T1).
template <int KIND, int D>
__device__ inline void pv_step(Unit<D>& u, const Tile<KIND, D>& T0, const Tile<KIND, D>& T1, const float (&pr)[8]) {
  constexpr int NT = D / 16;
  // A operand of PV: p * v_scale of (position, this row's group), split into
  // bf16 hi + lo.  INT8 and bf16 rows carry the 1/kEnc of the INT4 encoding.
  float ap[8];
  if constexpr (KIND == kBf16Page) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ap[e] = pr[e] * (1.0f / kEnc);
  } else {
    ap[0] = mul_h_lo(pr[0], T0.vs[0]);
    ap[1] = mul_h_hi(pr[1], T0.vs[0]);
    ap[2] = mul_h_lo(pr[2], T0.vs[1]);
    ap[3] = mul_h_hi(pr[3], T0.vs[1]);
    ap[4] = mul_h_lo(pr[4], T1.vs[0]);
    ap[5] = mul_h_hi(pr[5], T1.vs[0]);
    ap[6] = mul_h_lo(pr[6], T1.vs[1]);
    ap[7] = mul_h_hi(pr[7], T1.vs[1]);
    if constexpr (KIND != kInt4Page) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ap[e] *= (1.0f / kEnc);
    }
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[j] = pack_bf16(ap[2 * j], ap[2 * j + 1]);
    // low half moved up with a byte permute (0x0c selects a zero byte)
    const float h0 = __uint_as_float(__builtin_amdgcn_perm(0u, hi[j], 0x01000c0cu));
    lo[j] = pack_bf16(ap[2 * j] - h0, ap[2 * j + 1] - bf16_hi(hi[j]));
  }
  const bf16x8_t a_hi = bf8(hi[0], hi[1], hi[2], hi[3]);
  const bf16x8_t a_lo = bf8(lo[0], lo[1], lo[2], lo[3]);

  if constexpr (KIND == kInt4Page) {
    // -(1 + 8/kEnc) * sum over the positions of this row's A: the constant
    // part of the V codes' encoding, added to the output at the end.
    constexpr uint32_t kNeg = 0xBF88BF88u;  // -(1 + 8/128) in both halves
    const bf16x8_t ones = bf8(kNeg, kNeg, kNeg, kNeg);
    u.corr = mfma(a_hi, ones, u.corr);
    u.corr = mfma(a_lo, ones, u.corr);
  }
  if constexpr (KIND == kInt4Page) {
    // N-tiles j and j + 4 (head_dim 128) from one shift of each word pair:
    // words (pair, w) and (pair, w + 1) are adjacent, holding tiles 4w + j.
    // Head_dim 64: the two words of a tile are the two position pairs.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t a0, b0, a1, b1, a2, b2, a3, b3;
      if (j == 0) {
        nib_pairs2<0>(T0.v[0], T0.v[1], a0, b0);
        nib_pairs2<0>(T1.v[0], T1.v[1], a1, b1);
      } else if (j == 1) {
        nib_pairs2<1>(T0.v[0], T0.v[1], a0, b0);
        nib_pairs2<1>(T1.v[0], T1.v[1], a1, b1);
      } else if (j == 2) {
        nib_pairs2<2>(T0.v[0], T0.v[1], a0, b0);
        nib_pairs2<2>(T1.v[0], T1.v[1], a1, b1);
      } else {
        nib_pairs2<3>(T0.v[0], T0.v[1], a0, b0);
        nib_pairs2<3>(T1.v[0], T1.v[1], a1, b1);
      }
      if constexpr (D == 128) {
        if (j == 0) {
          nib_pairs2<0>(T0.v[2], T0.v[3], a2, b2);
          nib_pairs2<0>(T1.v[2], T1.v[3], a3, b3);
        } else if (j == 1) {
          nib_pairs2<1>(T0.v[2], T0.v[3], a2, b2);
          nib_pairs2<1>(T1.v[2], T1.v[3], a3, b3);
        } else if (j == 2) {
          nib_pairs2<2>(T0.v[2], T0.v[3], a2, b2);
          nib_pairs2<2>(T1.v[2], T1.v[3], a3, b3);
        } else {
          nib_pairs2<3>(T0.v[2], T0.v[3], a2, b2);
          nib_pairs2<3>(T1.v[2], T1.v[3], a3, b3);
        }
        // tile j: words (pair 0, w 0), (pair 1, w 0) of both tiles; tile j + 4: w 1
        const bf16x8_t bv0 = bf8(a0, a2, a1, a3), bv1 = bf8(b0, b2, b1, b3);
        f32x4_t c = u.o[j];
        c = mfma(a_hi, bv0, c);
        c = mfma(a_lo, bv0, c);
        u.o[j] = c;
        c = u.o[j + 4];
        c = mfma(a_hi, bv1, c);
        c = mfma(a_lo, bv1, c);
        u.o[j + 4] = c;
      } else {
        const bf16x8_t bv = bf8(a0, b0, a1, b1);
        f32x4_t c = u.o[j];
        c = mfma(a_hi, bv, c);
        c = mfma(a_lo, bv, c);
        u.o[j] = c;
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const bf16x8_t bv = v_operand<KIND, D>(T0, T1, t);
    f32x4_t c = u.o[t];
    c = mfma(a_hi, bv, c);
    c = mfma(a_lo, bv, c);
    u.o[t] = c;
  }
}

// Runs n tiles (ptr(i), mask(i)) two at a time (a step).  STAGES = 1: load
// then compute (bf16 tiles, whose registers leave no room for more); 2: the
// next step's loads are in flight while a step is computed.  Every load is
// issued unconditionally (past the end with an empty range) so the loop body
// has one fixed load sequence and each wait covers exactly the step it
// needs.  Tile n (odd n) reads as zeros and is masked.  setup(0) is called
// once the first step's loads are in flight, setup(1) after the first step
// and setup(2) after the second (and again on later steps; the caller acts on
// the first call of each).
template <int KIND, int D, int STAGES, bool Q8, bool NT, class PtrFn, class MaskFn, class SetupFn>
__device__ inline void run_tiles(Unit<D>& u, int n, PtrFn ptr, MaskFn mask, int lane, SetupFn setup) {
  if (n <= 0) return;
  const LaneOff<KIND, D> off(lane & 15, lane >> 4);
  const int nsteps = (n + 1) >> 1;
  const int last = nsteps - 1;
  constexpr int kBytes = Tile<KIND, D>::kBytes;
  // steps past the last and the tile after an odd last one get an empty
  // range: their loads return zeros and read no memory
  auto load = [&](Tile<KIND, D>& t0, Tile<KIND, D>& t1, int s) {
    const bool live = s <= last;
    s = s < last ? s : last;
    const int i = 2 * s;
    t0.template load<NT>(TileSrc(ptr(i), live ? kBytes : 0), off);
    t1.template load<NT>(TileSrc(ptr(i + 1 < n ? i + 1 : i), live && i + 1 < n ? kBytes : 0), off);
  };
  // per-wave LDS slots of the scale exchange, one per tile of a step
  __shared__ uint32_t sq_slots[kAttnThreads / kWave][2][kWave];
  uint32_t* slot0 = sq_slots[threadIdx.x / kWave][0];
  uint32_t* slot1 = sq_slots[threadIdx.x / kWave][1];
  auto run = [&](Tile<KIND, D>& t0, Tile<KIND, D>& t1, int s) {
    const int i = 2 * s;
    t0.gather(off, slot0);
    t1.gather(off, slot1);
    step<KIND, D, true, Q8>(u, t0, t1, mask(i), i + 1 < n ? mask(i + 1) : 0u, lane);
  };
  if constexpr (STAGES == 1) {
    for (int s = 0; s < nsteps; ++s) {
      Tile<KIND, D> a0, a1;
      load(a0, a1, s);
      setup(0);
      run(a0, a1, s);
      setup(s + 1 < 2 ? s + 1 : 2);
    }
  } else {
    static_assert(STAGES == 2, "one or two pipeline stages");
    Tile<KIND, D> a0, a1, b0, b1;
    load(a0, a1, 0);
    setup(0);
    for (int s = 0;; s += 2) {
      load(b0, b1, s + 1);
      run(a0, a1, s);
      setup(1);
      if (s + 1 >= nsteps) break;
      load(a0, a1, s + 2);
      run(b0, b1, s + 1);
      setup(2);
      if (s + 2 >= nsteps) break;
    }
  }
}

__device__ inline uint32_t range_mask(int lo, int hi) {  // bits [lo, hi) of 0..15
  lo = lo < 0 ? 0 : lo;
  hi = hi > 16 ? 16 : hi;
  if (hi <= lo) return 0u;
  return ((1u << hi) - 1u) & ~((1u << lo) - 1u);
}

// ---------------------------------------------------------------- worklist --
constexpr int kMaxChunkPagesMc = 64;           // one page id per lane in the multi-column kernel
static_assert(kMaxChunkPages == 128, "the single-query kernel holds two page ids per lane");
constexpr int kProtectedCost = 2;    // an INT8 tile costs about two INT4 pages

struct SeqWork {
  int L;           // positions the query sees: [0, L)
  int N;           // positions in the cache (clamped to the page table)
  int mid_first;   // first / last page holding middle rows (last < first: none)
  int mid_last;
  int prot_tiles;  // INT8 side tiles holding protected rows
};

// Side rows a query reads: the sinks it sees, and when it sees any ring
// position the whole written ring (its other rows are masked).
__device__ inline int side_rows(int L, int N, int S, int R) {
  const Regions g = regions_in(L, N, S, R);
  const int nring = N > S ? (N - S < R ? N - S : R) : 0;
  return L > g.rb ? S + nring : g.se;
}

// Work blocks: query t of sequence b sits at position N - nq + t and sees
// positions [0, N - nq + t + 1).  Block u = b * nqb + j holds the queries
// [j * tq, min((j + 1) * tq, nq)) of sequence b and covers what its last
// query sees.
__device__ inline int n_blocks(const DecodeParams& p) { return (p.nq + p.tq - 1) / p.tq; }
__device__ inline int block_queries(const DecodeParams& p, int u) {
  const int t0 = (u % n_blocks(p)) * p.tq;
  return p.nq - t0 < p.tq ? p.nq - t0 : p.tq;
}

__device__ inline SeqWork seq_work(const DecodeParams& p, int u) {
  SeqWork w;
  const int nqb = n_blocks(p);
  const int b = u / nqb, t_last = (u % nqb) * p.tq + block_queries(p, u) - 1;
  int N = p.seq_lens[b];
  N = N < 0 ? 0 : (N > p.max_pages * kPage ? p.max_pages * kPage : N);
  int L = N - p.nq + 1 + t_last;
  L = L < 0 ? 0 : L;
  w.L = L;
  w.N = N;
  const Regions g = regions_in(L, N, p.n_sink, p.n_recent);
  w.mid_first = g.mb / kPage;
  w.mid_last = g.me > g.mb ? (g.me - 1) / kPage : w.mid_first - 1;
  w.prot_tiles = (side_rows(L, N, p.n_sink, p.n_recent) + kPage - 1) / kPage;
  return w;
}

__device__ inline int mid_pages(const SeqWork& w) { return w.mid_last - w.mid_first + 1; }
__device__ inline int n_items(const SeqWork& w, int chunk) {
  const int n = (mid_pages(w) + chunk - 1) / chunk;
  return n < 1 ? 1 : n;
}
__device__ inline int item_pages(const SeqWork& w, int chunk, int k) {
  const int r = mid_pages(w) - k * chunk;
  return r > chunk ? chunk : (r < 0 ? 0 : r);
}

// Order key of an item that is not a full chunk: its pages plus the cost of
// the side tiles its unit reads (the first item of a sequence), so that the
// list ends on the cheapest units.
__device__ inline int item_key(const SeqWork& w, int chunk, int k) {
  const int c = item_pages(w, chunk, k) + (k == 0 ? kProtectedCost * w.prot_tiles : 0);
  return c < kMaxChunkPages ? c : kMaxChunkPages;
}

// Work-item descriptor, two int4:
//   [0] = {u, L, first middle page of the item, (chunk index << 8) | pages}
//   [1] = {items of u, first partial slot of u, side slot, N}
// Query j of a split block u keeps its partial of item k in slot
// pbase + j * items + k.
__device__ inline void write_item(const DecodeParams& p, uint32_t pos, int v, const SeqWork& w, int chunk, int k,
                                  int n, int pbase) {
  const int b = v / n_blocks(p);
  const int slot = p.slot_ids ? p.slot_ids[b] : b;
  p.ws.items[2 * pos] = make_int4(v, w.L, w.mid_first + k * chunk, (k << 8) | item_pages(w, chunk, k));
  p.ws.items[2 * pos + 1] = make_int4(n, pbase, slot, w.N);
}

// Block-wide helpers of the work-list kernel (1024 threads = 16 waves).
// Inclusive scan of a 64-bit value within a wave.
__device__ inline unsigned long long wave_scan_u64(unsigned long long v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t lo = __shfl_up(uint32_t(v), o, kWave), hi = __shfl_up(uint32_t(v >> 32), o, kWave);
    if (lane >= o) v += (unsigned long long)lo | ((unsigned long long)hi << 32);
  }
  return v;
}
// Exclusive prefix of v over the block's threads and the block total (every
// thread gets both).  `part` is a 16-entry LDS array; the call ends with a
// barrier, so `part` may be reused right after.
__device__ inline unsigned long long block_exclusive_scan(unsigned long long v, unsigned long long* part,
                                                          unsigned long long& total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const unsigned long long inc = wave_scan_u64(v, lane);
  if (lane == kWave - 1) part[wid] = inc;
  __syncthreads();
  unsigned long long before = 0ull, all = 0ull;
  for (int i = 0; i < 16; ++i) {
    const unsigned long long t = part[i];
    if (i < wid) before += t;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + inc - v;
}

__device__ inline void pool_reset(const DecodeParams& p, int tid, int nthreads);

// One workgroup: chooses the chunk size from the total work, numbers the
// partial slots of split sequences and writes the item descriptors: all full
// chunks first, then the remaining (shorter) items in decreasing cost (pages
// plus side tiles), so the units handed out last are the cheapest.  Each
// thread handles sequences tid, tid + 1024, ...; the first one's lengths
// are read once and kept.
__device__ inline void plan_body(const DecodeParams& p, int units_per_item) {
  __shared__ unsigned long long part[16];
  __shared__ uint32_t bucket[kMaxChunkPages + 2];
  __shared__ uint32_t nmerge;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int nv = p.batch * n_blocks(p);  // work blocks
  pool_reset(p, tid, 1024);
  for (int i = tid; i < kMaxChunkPages + 2; i += 1024) bucket[i] = 0u;
  if (tid == 0) nmerge = 0u;
  SeqWork w0{};
  if (tid < nv) w0 = seq_work(p, tid);
  unsigned long long mine = 0ull;
  for (int b = tid; b < nv; b += 1024) {
    const SeqWork w = b == tid ? w0 : seq_work(p, b);
    mine += unsigned(mid_pages(w)) + unsigned(kProtectedCost * w.prot_tiles);
  }
  unsigned long long total_pages = 0ull;
  (void)block_exclusive_scan(mine, part, total_pages);
  // about kUnitsPerWave units per resident wave
  const unsigned long long denom = unsigned(kUnitsPerWave) * unsigned(p.resident_waves > 0 ? p.resident_waves : 1);
  unsigned long long cl = (total_pages * unsigned(units_per_item) + denom - 1) / denom;
  const unsigned cmax = p.tq > 1 ? unsigned(kMaxChunkPagesMc) : unsigned(kMaxChunkPages);
  cl = cl < unsigned(kChunkPages) ? unsigned(kChunkPages) : (cl > cmax ? cmax : cl);
  const int chunk = int(cl);

  // pass 1: full items (scan) and the histogram of the other items' sizes;
  // the first sequence's partial slot and first full-item position are also
  // kept in registers for pass 2
  int run_full = 0, run_split = 0, pbase0 = 0, fpos0 = 0;
  for (int base = 0; base < nv; base += 1024) {
    const int b = base + tid;
    int full = 0, split = 0;
    if (b < nv) {
      const SeqWork w = base == 0 ? w0 : seq_work(p, b);
      const int n = n_items(w, chunk);
      for (int k = 0; k < n; ++k) {
        const int pg = item_pages(w, chunk, k);
        if (pg == chunk) ++full;
        else atomicAdd(&bucket[kMaxChunkPages - item_key(w, chunk, k)], 1u);
      }
      split = n > 1 ? n * block_queries(p, b) : 0;
    }
    unsigned long long tile = 0ull;
    const unsigned long long ex =
        block_exclusive_scan((unsigned long long)full | ((unsigned long long)split << 32), part, tile);
    if (b < nv) {
      p.ws.item_base[b] = run_split + int(ex >> 32);
      p.ws.merge_list[b].x = run_full + int(ex & 0xFFFFFFFFull);  // scratch: first full-item position
      if (base == 0) {
        pbase0 = run_split + int(ex >> 32);
        fpos0 = run_full + int(ex & 0xFFFFFFFFull);
      }
    }
    run_full += int(tile & 0xFFFFFFFFull);
    run_split += int(tile >> 32);
  }
  // positions of the shorter items, costliest first (bucket i holds key
  // kMaxChunkPages - i): an exclusive scan of the bucket counts by wave 0
  if (wid == 0) {
    constexpr int BPL = (kMaxChunkPages + kWave) / kWave;  // buckets per lane (kMaxChunkPages + 1 of them)
    uint32_t c[BPL], sum = 0u;
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      const int i = BPL * lane + k;
      c[k] = i <= kMaxChunkPages ? bucket[i] : 0u;
      sum += c[k];
    }
    const unsigned long long inc = wave_scan_u64((unsigned long long)sum, lane);
    uint32_t start = uint32_t(run_full) + uint32_t(inc) - sum;
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      const int i = BPL * lane + k;
      if (i <= kMaxChunkPages) bucket[i] = start;
      start += c[k];
    }
    if (lane == kWave - 1) {
      p.ws.header[0] = 0u;
      p.ws.header[1] = uint32_t(run_full) + uint32_t(inc);
      p.ws.header[2] = uint32_t(chunk);
    }
  }
  __syncthreads();
  // pass 2: descriptors
  for (int b = tid; b < nv; b += 1024) {
    const SeqWork w = b == tid ? w0 : seq_work(p, b);
    const int n = n_items(w, chunk);
    const int pbase = b == tid ? pbase0 : p.ws.item_base[b];
    uint32_t fpos = uint32_t(b == tid ? fpos0 : p.ws.merge_list[b].x);
    for (int k = 0; k < n; ++k) {
      const int pg = item_pages(w, chunk, k);
      const uint32_t pos = pg == chunk ? fpos++ : atomicAdd(&bucket[kMaxChunkPages - item_key(w, chunk, k)], 1u);
      write_item(p, pos, b, w, chunk, k, n, pbase);
    }
  }
  __syncthreads();
  // records of the split sequences for the merge (overwrite the scratch use
  // above): the merge loads one record instead of the list entry and then
  // the sequence's slot and item count
  for (int b = tid; b < nv; b += 1024) {
    const SeqWork w = b == tid ? w0 : seq_work(p, b);
    const int n = n_items(w, chunk);
    if (n > 1) p.ws.merge_list[atomicAdd(&nmerge, 1u)] = make_int4(b, b == tid ? pbase0 : p.ws.item_base[b], n, 0);
  }
  __syncthreads();
  if (tid == 0) p.ws.header[3] = nmerge;
}

__global__ __launch_bounds__(1024) void worklist_kernel(DecodeParams p, int units_per_item) {
  plan_body(p, units_per_item);
}

// Append and plan in one launch: workgroup 0 writes the work list (it reads
// only seq_lens, the page table and slot ids, none of which the append
// writes), the others append one (token, kv head) per wave, so the two
// latency-bound pieces overlap instead of running one after the other.
template <int AFMT, int E>
__global__ __launch_bounds__(1024) void append_plan_kernel(AppendParams a, DecodeParams p, int units_per_item) {
  if (blockIdx.x == 0) {
    plan_body(p, units_per_item);
    return;
  }
  append_row<AFMT, E>(a, int64_t(blockIdx.x - 1) * (1024 / kWave) + threadIdx.x / kWave);
}

// ------------------------------------------------------------- attention --
struct ItemDesc {
  int b, L, first, ck, npg, nitems, pbase, slot, N;  // b: work index b * nq + t
};

// A work-item descriptor as loaded (two int4, identical in every lane) and its
// decoded form.  Decoding makes the fields explicitly wave-uniform so that the
// loop control and the page addresses derived from them live in scalar
// registers; it waits for the load, so it is done one unit after the load was
// issued.
struct RawItem {
  int4 a, c;
};

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline RawItem load_item(const DecodeParams& p, uint32_t item) {
  return RawItem{p.ws.items[2 * item], p.ws.items[2 * item + 1]};
}

__device__ inline ItemDesc decode_item(const RawItem& r) {
  ItemDesc d;
  d.b = uniform(r.a.x);
  d.L = uniform(r.a.y);
  d.first = uniform(r.a.z);
  const int w = uniform(r.a.w);
  d.ck = w >> 8;
  d.npg = w & 0xFF;
  d.nitems = uniform(r.c.x);
  d.pbase = uniform(r.c.y);
  d.slot = uniform(r.c.z);
  d.N = uniform(r.c.w);
  return d;
}

// Work distribution.  One workgroup per CU holds both waves of every SIMD.
// The list (full chunks first, then the other items in decreasing cost) is
// cut in two.  The head -- about three quarters of the items, a whole number
// of rounds of C items (C workgroups) -- is shared out: workgroup c owns one
// item of every round, in serpentine order (c, 2C - 1 - c, 2C + c, ...), so
// the shares hold equal amounts of every cost, and its waves take the units
// of those items (upi per item, next to each other) in ticket order from a
// counter in LDS, so a faster wave takes more of them.  The tail, the
// cheapest items, is one queue for the whole GPU: a wave whose workgroup's
// share is used up takes its next unit there, from a device counter.  CUs and
// XCDs do not run at the same speed and the plan's cost estimate is not
// exact; the tail absorbs both, and it ends on the smallest units.
//
// The device counters sit on 128-byte lines of the workspace: line 0 counts
// the waves that have finished, line 1 is the tail's ticket counter.  The plan
// zeroes them, and the last wave of an attention launch to finish zeroes them
// again, so one plan serves any number of attention launches.
constexpr int kCtrStride = 32;  // uint32 words per counter line
constexpr int kSc1 = 16;        // buffer cache-policy bit of device-coherent stores

// items in the shared-out head of a list of nitems items, for C workgroups
__device__ inline uint32_t head_items(uint32_t nitems, uint32_t C) { return (nitems - nitems / 4u) / C * C; }

// LDS ticket of the workgroup's share
__device__ inline uint32_t pool_ticket(uint32_t* counter, int lane) {
  uint32_t t = 0u;
  if (lane == 0) t = atomicAdd(counter, 1u);
  return uint32_t(uniform(int(t)));
}
// the unit of ticket t of this workgroup's share, or `units` past its end
__device__ inline uint32_t pool_unit(uint32_t t, uint32_t upi, uint32_t nhead, uint32_t units) {
  const uint32_t round = t / upi, C = gridDim.x;
  const uint32_t item = round * C + ((round & 1u) ? C - 1u - blockIdx.x : blockIdx.x);
  return item < nhead ? item * upi + t % upi : units;
}

// Atomic add of 1 by lane 0 of the wave when `enable` (wave-uniform),
// returned in lane 0; otherwise no memory access.  The buffer range is the
// 4-byte counter (or empty), and the other lanes' offsets lie past it:
// buffer accesses outside the range are dropped (an atomic returns 0), so the
// wave makes at most one increment with no branch around the atomic.  (A
// global atomic under `if (lane == 0)` inside the unit loop makes the
// compiler keep the page loads' buffer descriptors in vector registers, with
// a readfirstlane loop around every page load.)
__device__ inline uint32_t lane0_atomic_add(uint32_t* ctr, bool enable, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(ctr, short(0), enable ? 4 : 0, 0x00020000);
  return uint32_t(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, r, lane == 0 ? 0 : 64, 0, 0));
}

// A drawn unit: from the workgroup's share (`local` < units), or a pending
// tail ticket (`raw`, lane 0) to be read once its atomic has returned.
struct Ticket {
  uint32_t local, raw;
};
__device__ inline Ticket pool_issue(const DecodeParams& p, uint32_t* counter, uint32_t upi, uint32_t nhead,
                                    uint32_t units, int lane) {
  const uint32_t u = pool_unit(pool_ticket(counter, lane), upi, nhead, units);
  return Ticket{u, lane0_atomic_add(p.ws.ctr + kCtrStride, u >= units, lane)};
}
// The unit of a drawn ticket, or `units` when the list is used up.
// Wave-uniform.
__device__ inline uint32_t pool_finish(const Ticket& k, uint32_t upi, uint32_t nhead, uint32_t units) {
  if (k.local < units) return k.local;
  const uint32_t g = uint32_t(uniform(int(k.raw))), tail = units - nhead * upi;
  return g < tail ? nhead * upi + g : units;
}

// A wave that has drawn its last ticket: after every memory operation it
// issued has completed (so its ticket atomics have been made), it counts
// itself finished; the last wave of the launch zeroes the device counters.
__device__ inline void pool_leave(const DecodeParams& p, int lane) {
  __builtin_amdgcn_s_waitcnt(0);
  const uint32_t waves = gridDim.x * (blockDim.x / kWave);
  const uint32_t n = uint32_t(uniform(int(lane0_atomic_add(p.ws.ctr, true, lane))));
  if (n + 1u == waves) {
    const __amdgpu_buffer_rsrc_t all =
        __builtin_amdgcn_make_buffer_rsrc(p.ws.ctr, short(0), int(2 * kCtrStride * sizeof(uint32_t)), 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(0u, all, uint32_t(lane) * uint32_t(kCtrStride * sizeof(uint32_t)), 0, kSc1);
  }
}

// Zeroes the device counters (the plan; nthreads threads of one workgroup).
__device__ inline void pool_reset(const DecodeParams& p, int tid, int nthreads) {
  for (int v = tid; v < 2; v += nthreads)
    __hip_atomic_store(p.ws.ctr + v * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int D>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, 8))) void attention_kernel(
    DecodeParams p) {
  constexpr int NG = D / 32, HB = 16 / NG, NT = D / 16;
  constexpr bool KV4 = FMT == kFmtKV4 || FMT == kFmtKV4Q8;
  constexpr bool Q8 = FMT == kFmtKV4Q8;
  constexpr int MAIN = KV4 ? kInt4Page : (FMT == kFmtKV8 ? kInt8Tile : kBf16Page);
  const int lane = threadIdx.x & (kWave - 1);
  const int ln = lane & 15, kg = lane >> 4;
  const int H = p.num_kv_heads, Hq = p.num_q_heads, G = Hq / H;
  const int NHB = (G + HB - 1) / HB;
  const int UPI = H * NHB;  // units per item
  const int S = KV4 ? p.n_sink : 0;
  const int R = KV4 ? p.n_recent : 0;
  // unit indices fit 32 bits: the host bounds the work list (items x units per item < 2^31)
  const uint32_t nitems = p.ws.header[1];
  const uint32_t units = nitems * uint32_t(UPI);
  if (units == 0) return;

  // Units come from the pool (see pool_issue).  A wave works on one unit
  // and prepares the next one: its ticket is drawn when the unit starts, and
  // resolved after the unit's first step (by then the atomic has returned),
  // which also issues the next descriptor's load; after the second step the
  // descriptor is decoded and the next unit's page ids are loaded.  So a wave
  // holds one unit beyond the one it works on, and when the pool runs dry the
  // waves finish within about one unit of each other.
  const uint32_t nhead = head_items(nitems, gridDim.x);
  __shared__ uint32_t next_ticket;
  if (threadIdx.x == 0) next_ticket = 0u;
  __syncthreads();
  auto issue = [&]() -> Ticket { return pool_issue(p, &next_ticket, UPI, nhead, units, lane); };
  auto finish = [&](const Ticket& k) -> uint32_t { return pool_finish(k, UPI, nhead, units); };
  auto item_of = [&](uint32_t t) -> uint32_t { return (t < units ? t : units - 1) / uint32_t(UPI); };
  // Page ids of an item, one per lane, loaded one unit ahead as raw page-table
  // words: this lane's page and the pages at the same index of the work
  // indices before and after it (other queries of the sequence, or the
  // neighbouring sequences).  The loads are unconditional (clamped indices)
  // and every check is made when the unit starts, so nothing waits for them
  // early.  A page is shared when a neighbour holds the same physical page at
  // the same index: a shared prompt.
  // With 128-page chunks a lane holds pages lane and lane + 64 of the item.
  constexpr int NH = kMaxChunkPages / kWave;  // page ids per lane
  struct Pids {
    int x[NH], xp[NH], xn[NH];
  };
  auto fetch_pids = [&](const ItemDesc& d) -> Pids {
    const int nv = p.batch * p.nq;
    const int bp = d.b > 0 ? d.b - 1 : 0, bn = d.b + 1 < nv ? d.b + 1 : d.b;
    Pids r;
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const int c = d.first + lane + k * kWave;
      const int col = c < p.max_pages ? c : p.max_pages - 1;
      r.x[k] = p.page_table[int64_t(d.b / p.nq) * p.max_pages + col];  // tq = 1: u = b * nq + t
      r.xp[k] = r.xn[k] = -1;
      if constexpr (KV4) {
        r.xp[k] = p.page_table[int64_t(bp / p.nq) * p.max_pages + col];
        r.xn[k] = p.page_table[int64_t(bn / p.nq) * p.max_pages + col];
      }
    }
    return r;
  };
  // this lane's page ids (-1 past the item or out of range) and the lane
  // masks of shared pages, one per half
  auto resolve_pids = [&](const Pids& r, const ItemDesc& d, int (&pid)[NH], uint64_t (&shared)[NH]) {
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const bool ok = lane + k * kWave < d.npg && r.x[k] >= 0 && int64_t(r.x[k]) < p.num_pages;
      pid[k] = ok ? r.x[k] : -1;
      const bool sh =
          ok && ((d.b > 0 && r.xp[k] == r.x[k]) || (d.b + 1 < p.batch * p.nq && r.xn[k] == r.x[k]));
      shared[k] = __ballot(KV4 && sh);
    }
  };
  uint32_t t0 = finish(issue());
  ItemDesc d0 = decode_item(load_item(p, item_of(t0)));
  Pids pid0 = fetch_pids(d0);

  while (t0 < units) {
    // this unit's page ids (loaded during the previous unit)
    int pid0v[NH];
    uint64_t shared0[NH];
    resolve_pids(pid0, d0, pid0v, shared0);
    // ---- the next unit: ticket now, the rest in `advance` (from setup(1)
    // and setup(2), and after the unit for what a short unit left undone)
    const Ticket k1 = issue();
    uint32_t t1 = units;
    RawItem r1;
    ItemDesc d1;
    Pids pid1;
    int next_stage = 0;
    auto advance = [&](int upto) {
      if (next_stage < 1 && upto >= 1) {
        next_stage = 1;
        t1 = finish(k1);
        r1 = load_item(p, item_of(t1));
      }
      if (next_stage < 2 && upto >= 2) {
        next_stage = 2;
        d1 = decode_item(r1);
        pid1 = fetch_pids(d1);
      }
    };

    const int rem = int(t0 % uint32_t(UPI));
    const int h = rem / NHB, hb = rem % NHB;
    const ItemDesc d = d0;
    const int b = d.b, L = d.L;
    const Regions g = regions_in(L, d.N, S, R);

    // ---- unit set-up.  The q loads are issued here, but the q operand is
    // built only after the unit's first tile loads are in flight (run_tiles
    // calls `setup` after its prologue), so the q latency overlaps them.
    Unit<D> u;
    uint4 qraw[NG];
    bool pending = true;
    {
      const int hl = ln / NG, grp = ln % NG;
      const int j = hb * HB + hl;
      const bool valid = j < G;
      // lanes whose k-slice is the row's group hold q (all of the group's
      // channels between them); the others hold zeros
      const bool take = valid && ((NG == 4 ? kg : (kg >> 1)) == grp);
      const uint16_t* qrow = p.q + (int64_t(b) * Hq + h * G + (valid ? j : 0)) * D;
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        qraw[t] = make_uint4(0u, 0u, 0u, 0u);
        if (take) qraw[t] = *reinterpret_cast<const uint4*>(qrow + kg * (D / 4) + 8 * t);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) u.o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u.corr = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u.m = -INFINITY;
      u.l = 0.f;
      u.qk_scale = p.softmax_scale * kLog2e;
    }
    auto setup = [&](int stage) {
      if (stage > 0) {
        advance(stage);
        return;
      }
      if (!pending) return;
      pending = false;
      if constexpr (Q8) {
        // Integer query: the head's row of q is quantized by the INT8 row rule
        // (scale from the head's largest |q|).  The lanes holding a row's
        // group quantize it; the head maximum gathers the head's rows.
        float am = 0.f;
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          const uint32_t w[4] = {qraw[t].x, qraw[t].y, qraw[t].z, qraw[t].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) am = max3(am, fabsf(bf16_lo(w[k])), fabsf(bf16_hi(w[k])));
        }
        am = fmaxf(am, __shfl_xor(am, 16, kWave));
        am = fmaxf(am, __shfl_xor(am, 32, kWave));
        am = fmaxf(am, quad_xor1(am));
        if constexpr (NG == 4) am = fmaxf(am, quad_xor2(am));
        const float qs16 = f16_to_f32(quant_scale_bits(am, 127.0f));
        int isum = 0;
#pragma unroll
        for (int t = 0; t < D / 64; ++t) {
          // 16 channels: qraw[2t] holds 0..7, qraw[2t+1] holds 8..15; bytes in
          // the order 0 2 4 6 | 1 3 5 7 | 8 10 12 14 | 9 11 13 15
          const uint32_t a[4] = {qraw[2 * t].x, qraw[2 * t].y, qraw[2 * t].z, qraw[2 * t].w};
          const uint32_t c[4] = {qraw[2 * t + 1].x, qraw[2 * t + 1].y, qraw[2 * t + 1].z, qraw[2 * t + 1].w};
          int ev[8], od[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            ev[k] = quant_code(bf16_lo(a[k]), qs16, 127.0f);
            od[k] = quant_code(bf16_hi(a[k]), qs16, 127.0f);
            ev[4 + k] = quant_code(bf16_lo(c[k]), qs16, 127.0f);
            od[4 + k] = quant_code(bf16_hi(c[k]), qs16, 127.0f);
          }
          auto pack = [](const int* v) {
            return (uint32_t(v[0]) & 0xFFu) | ((uint32_t(v[1]) & 0xFFu) << 8) | ((uint32_t(v[2]) & 0xFFu) << 16) |
                   ((uint32_t(v[3]) & 0xFFu) << 24);
          };
          u.q8[t][0] = pack(ev);
          u.q8[t][1] = pack(od);
          u.q8[t][2] = pack(ev + 4);
          u.q8[t][3] = pack(od + 4);
#pragma unroll
          for (int k = 0; k < 8; ++k) isum += ev[k] + od[k];
        }
        // the row group's code sum: the other lanes of the row hold zeros
        isum += __shfl_xor(isum, 16, kWave);
        isum += __shfl_xor(isum, 32, kWave);
        u.cin8 = -8 * isum;
        u.qk_scale = p.softmax_scale * kLog2e * qs16;
        return;
      }
      float qs = 0.f;
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        const uint32_t w0 = qraw[t].x, w1 = qraw[t].y, w2 = qraw[t].z, w3 = qraw[t].w;
        if constexpr (MAIN == kBf16Page) {
          u.bq[t] = bf8(w0, w1, w2, w3);  // channels in natural order
        } else {
          // element pairs (c, c+4): the order the code conversions produce
          u.bq[t] = bf8(__builtin_amdgcn_perm(w2, w0, 0x05040100u), __builtin_amdgcn_perm(w2, w0, 0x07060302u),
                        __builtin_amdgcn_perm(w3, w1, 0x05040100u), __builtin_amdgcn_perm(w3, w1, 0x07060302u));
          qs += ((bf16_lo(w0) + bf16_hi(w0)) + (bf16_lo(w1) + bf16_hi(w1))) +
                ((bf16_lo(w2) + bf16_hi(w2)) + (bf16_lo(w3) + bf16_hi(w3)));
        }
      }
      // the row's sum of q over its group: the other lanes of the row hold 0
      qs += __shfl_xor(qs, 16, kWave);
      qs += __shfl_xor(qs, 32, kWave);
      u.qsum = qs;
    };

    // ---- protected rows: INT8 side-cache tiles (sinks, then the ring)
    if (KV4 && d.ck == 0 && L > 0 && S + R > 0 && d.slot >= 0 && d.slot < p.num_slots) {
      const int ntiles = (side_rows(L, d.N, S, R) + kPage - 1) / kPage;
      // the ring rows of the recent positions [g.rb, L): a cyclic run of
      // L - g.rb rows from row S + (g.rb - S) mod R
      const int cnt = L - g.rb;
      const int rs = cnt > 0 ? (g.rb - S) % R : 0;
      const int r1 = rs + cnt < R ? rs + cnt : R;  // first run [rs, r1)
      const int r2 = rs + cnt - r1;                // wrapped run [0, r2)
      const uint8_t* sblk = p.side + (int64_t(d.slot) * H + h) * p.side_bytes;
      auto ptr = [&](int i) { return sblk + int64_t(i) * int8_tile_bytes(D); };
      auto mask = [&](int i) {
        const int r0 = i * kPage;
        return range_mask(0 - r0, g.se - r0) | range_mask(S + rs - r0, S + r1 - r0) |
               range_mask(S - r0, S + r2 - r0);
      };
      run_tiles<kInt8Tile, D, kStages8, Q8, false>(u, ntiles, ptr, mask, lane, setup);
    }

    // ---- middle pages of this item (at most kMaxChunkPages: NH page ids per lane)
    if (d.npg > 0) {
      constexpr int ST = MAIN == kInt4Page ? kStages4 : (MAIN == kInt8Tile ? kStages8 : 1);
      // pages [0, ns) of the item are shared with a neighbouring sequence
      int ns = ~shared0[0] == 0ull ? kWave : int(__builtin_ctzll(~shared0[0]));
      if constexpr (NH == 2) {
        if (ns == kWave) ns += ~shared0[1] == 0ull ? kWave : int(__builtin_ctzll(~shared0[1]));
      }
      auto ptr = [&](int i) {
        int pid = __builtin_amdgcn_readlane(pid0v[0], i & (kWave - 1));
        if constexpr (NH == 2) {
          if (i >= kWave) pid = __builtin_amdgcn_readlane(pid0v[1], i & (kWave - 1));
        }
        return p.pages + (int64_t(pid < 0 ? 0 : pid) * H + h) * p.block_bytes;
      };
      // Row masks: the region [mb, me) can cut only the item's first and last
      // pages; a page whose id is out of range contributes nothing.
      uint64_t okmv[NH];
#pragma unroll
      for (int k = 0; k < NH; ++k) okmv[k] = __ballot(pid0v[k] >= 0);
      const int pf = d.first * kPage, il = d.npg - 1;
      const uint32_t m_first = range_mask(g.mb - pf, g.me - pf);
      const uint32_t m_last = range_mask(g.mb - pf - il * kPage, g.me - pf - il * kPage);
      auto mask = [&](int i) {
        const uint32_t m = i == 0 ? m_first : (i == il ? m_last : 0xFFFFu);
        const uint64_t okm = (NH == 2 && i >= kWave) ? okmv[NH - 1] : okmv[0];
        return ((okm >> (i & (kWave - 1))) & 1ull) ? m : 0u;
      };
      if constexpr (MAIN == kInt4Page) {
        run_tiles<MAIN, D, ST, Q8, false>(u, ns, ptr, mask, lane, setup);
        run_tiles<MAIN, D, ST, Q8, true>(
            u, d.npg - ns, [&](int i) { return ptr(ns + i); }, [&](int i) { return mask(ns + i); }, lane, setup);
      } else {
        run_tiles<MAIN, D, ST, Q8, false>(u, d.npg, ptr, mask, lane, setup);
      }
    }

    // ---- finish: per-head denominators, then output or partial
    float lt = u.l;
    if constexpr (NG == 4) {  // each lane of a head's group of 4 summed its own positions
      lt += quad_xor1(lt);
      lt += quad_xor2(lt);
    }
    lt += __shfl_xor(lt, 16, kWave);
    lt += __shfl_xor(lt, 32, kWave);
    const int64_t pslot = int64_t(d.pbase) + d.ck;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int k = 0; k < (NG == 4 ? 1 : 2); ++k) {
        const int e = t / 2 + 2 * k;
        const float lh = head_value_for_acc<D>(lt, lane, e);
        const int hl = NG == 4 ? (lane >> 4) : ((lane >> 4) * 2 + k);
        const int j = hb * HB + hl;
        if (j < G) {
          const int hq = h * G + j;
          const int c = 16 * t + ln;
          const float o = u.o[t][e] + u.corr[e];
          if (d.nitems == 1) {
            const float v = lh > 0.f ? kEnc * o / lh : 0.f;
            p.out[(int64_t(b) * Hq + hq) * D + c] = f32_to_bf16_bits(v);
          } else {
            p.ws.partials[(pslot * Hq + hq) * part_stride(D) + c] = kEnc * o;
          }
        }
      }
    }
    if (kg == 0 && (ln % NG) == 0) {
      const int j = hb * HB + ln / NG;
      if (j < G) {
        const int hq = h * G + j;
        if (d.nitems == 1) {
          if (p.lse) p.lse[int64_t(b) * Hq + hq] = lt > 0.f ? (u.m + log2f(lt)) * kLn2 : -INFINITY;
        } else {
          float* part = p.ws.partials + (pslot * Hq + hq) * part_stride(D);
          part[D] = u.m;
          part[D + 1] = lt;
        }
      }
    }
    // ---- rotate the run-ahead state
    advance(2);  // what a unit with fewer than two steps left undone
    t0 = t1;
    d0 = d1;
    pid0 = pid1;
  }
  pool_leave(p, lane);
}

// ------------------------------------------------ multi-query attention --
// Several query tokens of one sequence read the same K/V.  A unit is
// (item, kv head) and its 16 MFMA columns are (query, q head) pairs: 16 / G
// queries of the G = Hq / Hkv heads of the kv head.  QK rows are positions and
// every column uses every channel, so no MFMA work is wasted; the INT4 scales
// are per (position, 32-channel group), so each group has its own QK
// accumulator and its own P x V-scale operand.  INT4 pages and the INT8 side
// tiles at head_dim 128.  Queries see different position ranges (query t of
// T sees [0, N - T + t + 1)), so masks are per lane (column).


// Per-lane byte offsets inside a block, D = 128, lane (ln = L % 16, kg = L / 16).
struct McOff {
  uint32_t k4, v4, s4, sc4, k8, v8, s8;
  __device__ inline McOff(int ln, int kg) {
    k4 = ln * 64 + kg * 4;               // INT4 K: + 16g -> channels 32g + 8kg .. +7 of row ln
    v4 = 8 * 128 + (kg * 16 + ln) * 16;  // INT4 V: as the single-query tile
    s4 = 16 * 128 + kg * 8;              // INT4 K scales of rows 4kg..4kg+3: + 32g; V scales + 128
    // the 16 lanes kg * 16 + n use the same 16 scale dwords (K and V of
    // rows 4kg..4kg+3, every group); lane n loads dword n: group n / 4,
    // K (n % 4 < 2) or V, half n % 2
    sc4 = s4 + 32 * (ln >> 2) + 128 * ((ln >> 1) & 1) + 4 * (ln & 1);
    k8 = ln * 128 + kg * 8;              // INT8 K: + 32g -> channels 32g + 8kg .. +7 of row ln
    v8 = 16 * 128 + (kg * 16 + ln) * 32; // INT8 V: as the single-query tile
    s8 = 32 * 128 + kg * 8;              // INT8 K scales of rows 4kg..4kg+3; V scales + 32
  }
};

template <int KIND>
struct McTile;

template <>
struct McTile<kInt4Page> {
  static constexpr int kBytes = int(int4_block_bytes(128));
  uint32_t k[4];      // group g: channels 32g + 8kg .. +7 of row ln (8 nibbles)
  uint32_t v[4];      // V codes, the single-query tile's layout
  uint32_t ks[4][2];  // group g: fp16 K scales of rows 4kg..4kg+3 (after `gather`)
  uint32_t vs[4][2];
  uint32_t sc;        // this lane's dword of the scale area, until `gather`
  __device__ inline void load(const TileSrc& s, const McOff& o) {
#pragma unroll
    for (int g = 0; g < 4; ++g) k[g] = ld4<false>(s, o.k4 + 16 * g);
    const uint4 a = ld16<false>(s, o.v4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    // one distinct dword per lane: with each lane loading its 64 bytes of
    // scales itself, two thirds of the bytes a tile moves through the
    // texture path were scale loads repeated by the 16 lanes of a row
    sc = ld4<false>(s, o.sc4);
  }
  // After the loads have arrived: the wave's 64 scale dwords pass through its
  // own 256-byte LDS slot, and each lane reads its row's 16 (group g: K
  // halves at 4g, 4g + 1, V halves at 4g + 2, 4g + 3).  The exchange stays
  // within the wave, whose LDS operations complete in order.
  __device__ inline void gather(uint32_t* slot, int lane) {
    slot[lane] = sc;
    __builtin_amdgcn_wave_barrier();
    const uint32_t* row = slot + (lane >> 4) * 16;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 x = *reinterpret_cast<const uint4*>(row + 4 * g);
      ks[g][0] = x.x; ks[g][1] = x.y;
      vs[g][0] = x.z; vs[g][1] = x.w;
    }
    __builtin_amdgcn_wave_barrier();
  }
};

template <>
struct McTile<kInt8Tile> {
  static constexpr int kBytes = int(int8_tile_bytes(128));
  uint32_t k[8];  // group g: dwords 2g, 2g+1 = channels 32g + 8kg .. +7 of row ln
  uint32_t v[8];
  uint32_t ks[2], vs[2];  // one fp16 scale per row, rows 4kg..4kg+3
  __device__ inline void load(const TileSrc& s, const McOff& o) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 a = ld8<false>(s, o.k8 + 32 * g);
      k[2 * g] = a.x; k[2 * g + 1] = a.y;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 b = ld16<false>(s, o.v8 + 16 * i);
      v[4 * i] = b.x; v[4 * i + 1] = b.y; v[4 * i + 2] = b.z; v[4 * i + 3] = b.w;
    }
    const uint2 x = ld8<false>(s, o.s8), y = ld8<false>(s, o.s8 + 32);
    ks[0] = x.x; ks[1] = x.y;
    vs[0] = y.x; vs[1] = y.y;
  }
  __device__ inline void gather(uint32_t*, int) {}
};

struct McUnit {
  bf16x8_t bq[4];  // group g: q of this lane's column, channels 32g + 8kg + (0 4 1 5 2 6 3 7)
  float qs[4];     // group g: sum of the column's q over the group's 32 channels
  f32x4_t o[8];    // PV accumulators: N-tile t, rows (columns) 4kg'..4kg'+3 of lane (n, kg')
  f32x4_t corr[4]; // INT4 V-encoding correction per group, same layout
  float m;         // running max (log2 units) of this lane's column
  float l;         // this lane's share of the column's softmax denominator
  float qk_scale;
};

// x times fp16 half e % 2 of word w[e / 2], as one mixed-precision FMA
__device__ inline float mul_h_at(float x, const uint32_t (&w)[2], int e) {
  return (e & 1) ? mul_h_hi(x, w[e >> 1]) : mul_h_lo(x, w[e >> 1]);
}
__device__ inline float h2f_at(const uint32_t (&w)[2], int e) { return (e & 1) ? h2f_hi(w[e >> 1]) : h2f_lo(w[e >> 1]); }

template <int KIND>
__device__ inline void qk_mc(const McUnit& u, const McTile<KIND>& T, float (&x)[4]) {
  if constexpr (KIND == kInt4Page) {
    f32x4_t acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float c = -kEncConst * u.qs[g];
      const uint32_t d = T.k[g];
      acc[g] = mfma(bf8(nib_pair<0>(d), nib_pair<1>(d), nib_pair<2>(d), nib_pair<3>(d)), u.bq[g],
                    f32x4_t{c, c, c, c});
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = mul_h_at(acc[0][e], T.ks[0], e);
      s = fmaf(acc[1][e], h2f_at(T.ks[1], e), s);
      s = fmaf(acc[2][e], h2f_at(T.ks[2], e), s);
      x[e] = fmaf(acc[3][e], h2f_at(T.ks[3], e), s);
    }
  } else {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t w0 = T.k[2 * g], w1 = T.k[2 * g + 1];
      acc = mfma(bf8(pack_exact(sbyte(w0, 0), sbyte(w1, 0)), pack_exact(sbyte(w0, 1), sbyte(w1, 1)),
                     pack_exact(sbyte(w0, 2), sbyte(w1, 2)), pack_exact(sbyte(w0, 3), sbyte(w1, 3))),
                 u.bq[g], acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = mul_h_at(acc[e], T.ks, e);
  }
}

// p (8 positions: rows 4kg..4kg+3 of T0 then of T1) times a per-position
// factor, split into bf16 hi + lo A operands
__device__ inline void split_a(const float (&ap)[8], bf16x8_t& a_hi, bf16x8_t& a_lo) {
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[j] = pack_bf16(ap[2 * j], ap[2 * j + 1]);
    const float h0 = __uint_as_float(__builtin_amdgcn_perm(0u, hi[j], 0x01000c0cu));
    lo[j] = pack_bf16(ap[2 * j] - h0, ap[2 * j + 1] - bf16_hi(hi[j]));
  }
  a_hi = bf8(hi[0], hi[1], hi[2], hi[3]);
  a_lo = bf8(lo[0], lo[1], lo[2], lo[3]);
}

// One step of two tiles.  va0 / va1: this lane's valid rows (4 bits) of each tile.
template <int KIND>
__device__ inline void step_mc(McUnit& u, const McTile<KIND>& T0, const McTile<KIND>& T1, uint32_t va0,
                               uint32_t va1, int lane) {
  float x0[4], x1[4];
  qk_mc<KIND>(u, T0, x0);
  qk_mc<KIND>(u, T1, x1);
  if (!__all((va0 & va1) == 15u)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] = ((va0 >> e) & 1u) ? x0[e] : -INFINITY;
      x1[e] = ((va1 >> e) & 1u) ? x1[e] : -INFINITY;
    }
  }
  float mx = max3(max3(x0[0], x0[1], x0[2]), max3(x0[3], x1[0], x1[1]), max3(x1[2], x1[3], -INFINITY));
  const float sc = KIND == kInt4Page ? kEnc * u.qk_scale : u.qk_scale;
  // lazy running max of a column, as in the single-query step
  if (__any(mx * sc > u.m + kRescale)) {
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mn = fmaxf(u.m, mx * sc);
    const float alpha = (mn == u.m) ? 1.0f : __builtin_amdgcn_exp2f(u.m - mn);
    u.l *= alpha;
    u.m = mn;
    // accumulator row e of lane (n, kg') is column 4kg' + e, held by lane 4kg' + e
    const int c0 = 4 * (lane >> 4);
    const f32x4_t f = {__shfl(alpha, c0, kWave), __shfl(alpha, c0 + 1, kWave), __shfl(alpha, c0 + 2, kWave),
                       __shfl(alpha, c0 + 3, kWave)};
#pragma unroll
    for (int t = 0; t < 8; ++t) u.o[t] *= f;
#pragma unroll
    for (int g = 0; g < 4; ++g) u.corr[g] *= f;
  }
  const float mneg = u.m == -INFINITY ? 0.0f : -u.m;
  float pr[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pr[e] = __builtin_amdgcn_exp2f(fmaf(x0[e], sc, mneg));
    pr[e + 4] = __builtin_amdgcn_exp2f(fmaf(x1[e], sc, mneg));
  }
  u.l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));

  if constexpr (KIND == kInt4Page) {
    constexpr uint32_t kNeg = 0xBF88BF88u;  // -(1 + 8/128) in both halves
    const bf16x8_t ones = bf8(kNeg, kNeg, kNeg, kNeg);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float ap[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ap[e] = mul_h_at(pr[e], T0.vs[g], e);
        ap[e + 4] = mul_h_at(pr[e + 4], T1.vs[g], e);
      }
      bf16x8_t a_hi, a_lo;
      split_a(ap, a_hi, a_lo);
      u.corr[g] = mfma(a_hi, ones, u.corr[g]);
      u.corr[g] = mfma(a_lo, ones, u.corr[g]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * g + tt, j = t & 3, w = t >> 2;
        const bf16x8_t bv = bf8(nib_pair_at(T0.v[w], j), nib_pair_at(T0.v[2 + w], j), nib_pair_at(T1.v[w], j),
                                nib_pair_at(T1.v[2 + w], j));
        f32x4_t c = u.o[t];
        c = mfma(a_hi, bv, c);
        c = mfma(a_lo, bv, c);
        u.o[t] = c;
      }
    }
  } else {
    float ap[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ap[e] = mul_h_at(pr[e] * (1.0f / kEnc), T0.vs, e);
      ap[e + 4] = mul_h_at(pr[e + 4] * (1.0f / kEnc), T1.vs, e);
    }
    bf16x8_t a_hi, a_lo;
    split_a(ap, a_hi, a_lo);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t a = T0.v[t], b = T1.v[t];
      const bf16x8_t bv = bf8(pack_exact(sbyte(a, 0), sbyte(a, 1)), pack_exact(sbyte(a, 2), sbyte(a, 3)),
                              pack_exact(sbyte(b, 0), sbyte(b, 1)), pack_exact(sbyte(b, 2), sbyte(b, 3)));
      f32x4_t c = u.o[t];
      c = mfma(a_hi, bv, c);
      c = mfma(a_lo, bv, c);
      u.o[t] = c;
    }
  }
}

// n tiles two at a time, two-stage register pipeline; loads past the end get
// an empty range (zeros), as in run_tiles.  mask(i) -> this lane's valid rows.
template <int KIND, class PtrFn, class MaskFn, class SetupFn>
__device__ inline void run_mc(McUnit& u, int n, PtrFn ptr, MaskFn mask, int lane, SetupFn setup) {
  if (n <= 0) return;
  const McOff off(lane & 15, lane >> 4);
  const int nsteps = (n + 1) >> 1;
  const int last = nsteps - 1;
  constexpr int kBytes = McTile<KIND>::kBytes;
  auto load = [&](McTile<KIND>& t0, McTile<KIND>& t1, int s) {
    const bool live = s <= last;
    s = s < last ? s : last;
    const int i = 2 * s;
    t0.load(TileSrc(ptr(i), live ? kBytes : 0), off);
    t1.load(TileSrc(ptr(i + 1 < n ? i + 1 : i), live && i + 1 < n ? kBytes : 0), off);
  };
  // per-wave LDS slots of the scale exchange, one per tile of a step
  __shared__ uint32_t scale_slots[kAttnThreads / kWave][2][kWave];
  uint32_t* slot0 = scale_slots[threadIdx.x / kWave][0];
  uint32_t* slot1 = scale_slots[threadIdx.x / kWave][1];
  auto run = [&](McTile<KIND>& t0, McTile<KIND>& t1, int s) {
    const int i = 2 * s;
    t0.gather(slot0, lane);
    t1.gather(slot1, lane);
    step_mc<KIND>(u, t0, t1, mask(i), i + 1 < n ? mask(i + 1) : 0u, lane);
  };
  // one stage: a second one measured 1.3% slower (registers)
  for (int s = 0; s < nsteps; ++s) {
    McTile<KIND> a0, a1;
    load(a0, a1, s);
    setup();
    run(a0, a1, s);
  }
}

// rows [lo, hi) of a 4-row run starting at row r: bits 0..3
__device__ inline uint32_t rows4(int r, int lo, int hi) {
  lo = lo - r;
  hi = hi - r;
  lo = lo < 0 ? 0 : lo;
  hi = hi > 4 ? 4 : hi;
  return hi > lo ? ((1u << hi) - 1u) & ~((1u << lo) - 1u) : 0u;
}

__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU, 8))) void attention_mc_kernel(
    DecodeParams p) {
  constexpr int D = 128, NT = 8;
  const int lane = threadIdx.x & (kWave - 1);
  const int ln = lane & 15, kg = lane >> 4;
  const int H = p.num_kv_heads, Hq = p.num_q_heads, G = Hq / H;
  const int S = p.n_sink, R = p.n_recent;
  const int T = p.nq, nqb = n_blocks(p);
  const uint32_t nitems = p.ws.header[1];
  const uint32_t units = nitems * uint32_t(H);
  if (units == 0) return;
  // units (item, kv head) from the pool; the next unit's ticket is drawn
  // when a unit starts
  const uint32_t nhead = head_items(nitems, gridDim.x);
  __shared__ uint32_t next_ticket;
  if (threadIdx.x == 0) next_ticket = 0u;
  __syncthreads();
  Ticket k = pool_issue(p, &next_ticket, uint32_t(H), nhead, units, lane);
  for (uint32_t t0 = pool_finish(k, uint32_t(H), nhead, units); t0 < units;
       t0 = pool_finish(k, uint32_t(H), nhead, units)) {
    k = pool_issue(p, &next_ticket, uint32_t(H), nhead, units, lane);
    const ItemDesc d = decode_item(load_item(p, t0 / uint32_t(H)));
    const int h = int(t0 % uint32_t(H));
    const int bseq = d.b / nqb, tb = (d.b % nqb) * p.tq;  // sequence, first query of the block
    const int nqs = T - tb < p.tq ? T - tb : p.tq;        // queries in the block
    const int N = d.N;
    const Regions g = regions_in(d.L, N, S, R);  // the block's union (its last query)

    // ---- this lane's QK column: query tb + ln / G, head ln % G
    const int qj = ln / G, hj = ln % G;
    const bool col_ok = qj < nqs;
    const int ncol = col_ok ? N - T + tb + qj + 1 : 0;  // positions the column sees: [0, ncol)

    McUnit u;
    uint4 qraw[4];
    bool pending = true;
    {
      const uint16_t* qrow = p.q + ((int64_t(bseq) * T + tb + (col_ok ? qj : 0)) * Hq + h * G + hj) * D;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        qraw[gg] = make_uint4(0u, 0u, 0u, 0u);
        if (col_ok) qraw[gg] = *reinterpret_cast<const uint4*>(qrow + 32 * gg + 8 * kg);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) u.o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) u.corr[gg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u.m = -INFINITY;
      u.l = 0.f;
      u.qk_scale = p.softmax_scale * kLog2e;
    }
    auto setup = [&]() {
      if (!pending) return;
      pending = false;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const uint32_t w0 = qraw[gg].x, w1 = qraw[gg].y, w2 = qraw[gg].z, w3 = qraw[gg].w;
        u.bq[gg] = bf8(__builtin_amdgcn_perm(w2, w0, 0x05040100u), __builtin_amdgcn_perm(w2, w0, 0x07060302u),
                       __builtin_amdgcn_perm(w3, w1, 0x05040100u), __builtin_amdgcn_perm(w3, w1, 0x07060302u));
        float qs = ((bf16_lo(w0) + bf16_hi(w0)) + (bf16_lo(w1) + bf16_hi(w1))) +
                   ((bf16_lo(w2) + bf16_hi(w2)) + (bf16_lo(w3) + bf16_hi(w3)));
        qs += __shfl_xor(qs, 16, kWave);
        qs += __shfl_xor(qs, 32, kWave);
        u.qs[gg] = qs;
      }
    };

    // ---- protected rows: INT8 side tiles of the first item
    if (d.ck == 0 && d.L > 0 && S + R > 0 && d.slot >= 0 && d.slot < p.num_slots) {
      const int nring = N > S ? (N - S < R ? N - S : R) : 0;
      const int ring0 = N - R > S ? N - R : S;
      const int rows = d.L > g.rb ? S + nring : g.se;
      const int ntiles = (rows + kPage - 1) / kPage;
      const int shift = R > 0 ? (ring0 - S) % R : 0;  // ring row of position ring0
      const int sink_end = ncol < S ? ncol : S;
      const uint8_t* sblk = p.side + (int64_t(d.slot) * H + h) * p.side_bytes;
      auto ptr = [&](int i) { return sblk + int64_t(i) * int8_tile_bytes(D); };
      auto mask = [&](int i) {
        uint32_t v = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rho = i * kPage + 4 * kg + e;
          bool ok;
          if (rho < S) {
            ok = rho < sink_end;
          } else {
            const int r = rho - S;
            const int pos = ring0 + (r - shift + R) % (R > 0 ? R : 1);
            ok = r < nring && pos < ncol;
          }
          v |= ok ? (1u << e) : 0u;
        }
        return v;
      };
      run_mc<kInt8Tile>(u, ntiles, ptr, mask, lane, setup);
    }

    // ---- middle pages of the item
    if (d.npg > 0) {
      int pid0 = 0;
      if (lane < d.npg) {
        const int64_t x = p.page_table[int64_t(bseq) * p.max_pages + d.first + lane];
        pid0 = (x < 0 || x >= p.num_pages) ? -1 : int(x);
      }
      auto ptr = [&](int i) {
        const int pid = __builtin_amdgcn_readlane(pid0, i);
        return p.pages + (int64_t(pid < 0 ? 0 : pid) * H + h) * p.block_bytes;
      };
      const int me = g.me < ncol ? g.me : ncol;  // this column's end of the INT4 region
      auto mask = [&](int i) {
        const int pid = __builtin_amdgcn_readlane(pid0, i);
        return pid < 0 ? 0u : rows4((d.first + i) * kPage + 4 * kg, g.mb, me);
      };
      run_mc<kInt4Page>(u, d.npg, ptr, mask, lane, setup);
    }

    // ---- finish: the column's denominator, then outputs or partials
    float lt = u.l;
    lt += __shfl_xor(lt, 16, kWave);
    lt += __shfl_xor(lt, 32, kWave);
    const int64_t pbase = d.pbase;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = 4 * kg + e;  // accumulator row e of this lane
      const float lh = __shfl(lt, col, kWave);
      const int cq = col / G, chj = col % G;
      if (cq < nqs) {
        const int64_t row = (int64_t(bseq) * T + tb + cq) * Hq + h * G + chj;
        const int64_t slot = pbase + int64_t(cq) * d.nitems + d.ck;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float o = u.o[t][e] + u.corr[t >> 1][e];
          const int c = 16 * t + ln;
          if (d.nitems == 1) {
            p.out[row * D + c] = f32_to_bf16_bits(lh > 0.f ? kEnc * o / lh : 0.f);
          } else {
            p.ws.partials[(slot * Hq + h * G + chj) * part_stride(D) + c] = kEnc * o;
          }
        }
      }
    }
    if (kg == 0 && col_ok) {
      const int64_t row = (int64_t(bseq) * T + tb + qj) * Hq + h * G + hj;
      if (d.nitems == 1) {
        if (p.lse) p.lse[row] = lt > 0.f ? (u.m + log2f(lt)) * kLn2 : -INFINITY;
      } else {
        float* part = p.ws.partials + ((pbase + int64_t(qj) * d.nitems + d.ck) * Hq + h * G + hj) * part_stride(D);
        part[D] = u.m;
        part[D + 1] = lt;
      }
    }
  }
  pool_leave(p, lane);
}

// ----------------------------------------------------------------- merge ---
// Exact log-sum-exp merge of the partials of split sequences ([NEWS]
// Interpretation para 3); a persistent grid strides over (split sequence,
// query head) pairs.  Items are taken eight at a time: the (m, l) of the eight
// (one per lane) and their output channels are loaded together, so a
// sequence of up to eight items costs one memory round trip.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  // A task is one (split block, query of the block, query head), merged by 16
  // lanes: each lane holds E consecutive channels and reads every item's m
  // and l itself, so the lanes of a task need no exchange and the four tasks
  // of a wave proceed independently.
  constexpr int QL = 16;      // lanes per task
  constexpr int E = D / QL;   // channels per lane
  constexpr int K = kMergeK;  // items per round
  constexpr int RS = part_stride(D);
  const int sub = threadIdx.x & (QL - 1);
  const int Hq = p.num_q_heads;
  const int64_t nt = int64_t(gridDim.x) * (blockDim.x / QL);
  const int nqb = n_blocks(p);
  const int64_t per = int64_t(p.tq) * Hq;  // (query of the block, head) pairs
  // A task's record is loaded before the count of split sequences is known
  // (the index clamped to the list's extent, the work blocks), so the two
  // loads overlap; a record past the count is never used.
  const int64_t last = int64_t(p.batch) * nqb - 1;
  auto record = [&](int64_t w) { return p.ws.merge_list[w / per < last ? w / per : last]; };
  int64_t w = int64_t(blockIdx.x) * (blockDim.x / QL) + threadIdx.x / QL;
  int4 rec = record(w);
  const int64_t tasks = int64_t(p.ws.header[3]) * per;
  for (; w < tasks; w += nt, rec = record(w)) {
    const int u = rec.x;
    const int j = int((w % per) / Hq), hq = int(w % Hq);
    if (j >= block_queries(p, u)) continue;
    const int b = (u / nqb) * p.nq + (u % nqb) * p.tq + j;  // output row: query t of sequence b
    const int n = rec.z;
    const float* base = p.ws.partials + ((int64_t(rec.y) + int64_t(j) * n) * Hq + hq) * RS;
    const int64_t stride = int64_t(Hq) * RS;
    float M = -INFINITY, l = 0.f, o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    for (int i0 = 0; i0 < n; i0 += K) {
      const int cnt = n - i0 < K ? n - i0 : K;
      float mi[K], li[K], v[K][E];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float* row = base + (i0 + (k < cnt ? k : 0)) * stride;
        const float2 ml = *reinterpret_cast<const float2*>(row + D);
        // an item without context rows, or none, weighs 0
        mi[k] = (k < cnt && ml.y > 0.f) ? ml.x : -INFINITY;
        li[k] = ml.y;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const float4 x = *reinterpret_cast<const float4*>(row + sub * E + 4 * q);
          v[k][4 * q] = x.x;
          v[k][4 * q + 1] = x.y;
          v[k][4 * q + 2] = x.z;
          v[k][4 * q + 3] = x.w;
        }
      }
      float mc = mi[0];
#pragma unroll
      for (int k = 1; k < K; ++k) mc = fmaxf(mc, mi[k]);
      const float Mn = fmaxf(M, mc);
      if (Mn == -INFINITY) continue;
      const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      l *= sc;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] *= sc;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float a = mi[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi[k] - Mn);
        l = fmaf(a, li[k], l);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = fmaf(a, v[k][e], o[e]);
      }
      M = Mn;
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint16_t* orow = p.out + (int64_t(b) * Hq + hq) * D + sub * E;
#pragma unroll
    for (int e = 0; e < E; e += 2)
      *reinterpret_cast<uint32_t*>(orow + e) =
          uint32_t(f32_to_bf16_bits(o[e] * inv)) | (uint32_t(f32_to_bf16_bits(o[e + 1] * inv)) << 16);
    if (p.lse && sub == 0) p.lse[int64_t(b) * Hq + hq] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
  }
}

// --------------------------------------------------------------- launch ---
template <class K>
int blocks_per_cu(K kernel) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), 256, 0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

template <int FMT, int D>
hipError_t launch_fd(DecodeParams p, unsigned phases, const AppendParams* append, hipStream_t stream) {
  constexpr int HB = 16 / (D / 32);
  const int cus = device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int G = p.num_q_heads / p.num_kv_heads;
  // several queries per sequence on INT4 pages at head_dim 128: one unit
  // holds 16 / G queries of the kv head's G heads
  const bool mc = FMT == kFmtKV4 && D == 128 && p.nq > 1 && G <= 16 && 16 % G == 0;
  p.tq = mc ? 16 / G : 1;
  // the work list is sized for the attention grid, so both use the same count
  const int blocks = cus;  // one workgroup per CU (the per-CU share of the list)
  p.resident_waves = blocks * (kAttnThreads / kWave);
  if (phases & 1u) {
    const int units_per_item = mc ? p.num_kv_heads : p.num_kv_heads * ((G + HB - 1) / HB);
    if (append && append->total_new > 0) {
      constexpr int AFMT = FMT == kFmtKV4Q8 ? kFmtKV4 : FMT;
      const int64_t waves = int64_t(append->total_new) * append->num_kv_heads;
      const unsigned blocks_a = unsigned(1 + (waves + 1024 / kWave - 1) / (1024 / kWave));
      hipLaunchKernelGGL((append_plan_kernel<AFMT, D / kWave>), dim3(blocks_a), dim3(1024), 0, stream, *append, p,
                         units_per_item);
    } else {
      hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, stream, p, units_per_item);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  } else if (append && append->total_new > 0) {
    const hipError_t err = launch_append(FMT == kFmtKV4Q8 ? kFmtKV4 : FMT, *append, D, stream);
    if (err != hipSuccess) return err;
  }
  if (phases & 2u) {
    if (mc) {
      hipLaunchKernelGGL(attention_mc_kernel, dim3(blocks), dim3(kAttnThreads), 0, stream, p);
    } else {
      hipLaunchKernelGGL((attention_kernel<FMT, D>), dim3(blocks), dim3(kAttnThreads), 0, stream, p);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (phases & 4u) {
    hipLaunchKernelGGL((merge_kernel<D>), dim3(cus * blocks_per_cu(merge_kernel<D>)), dim3(256), 0, stream, p);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <int FMT>
hipError_t launch_fmt(const DecodeParams& p, int head_dim, unsigned phases, const AppendParams* append,
                      hipStream_t stream) {
  return head_dim == 128 ? launch_fd<FMT, 128>(p, phases, append, stream)
                         : launch_fd<FMT, 64>(p, phases, append, stream);
}

}  // namespace


static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int64_t max_items_of(int32_t batch, int32_t max_pages) {
  const int64_t per_seq = (int64_t(max_pages) + kChunkPages - 1) / kChunkPages;
  return int64_t(batch) * (per_seq < 1 ? 1 : per_seq);
}

bool decode_units_fit(int32_t batch, int32_t max_pages, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim) {
  const int64_t hb = 16 / (head_dim / 32);
  const int64_t g = num_q_heads / num_kv_heads;
  const int64_t units = max_items_of(batch, max_pages) * num_kv_heads * ((g + hb - 1) / hb);
  return units < (int64_t(1) << 31);
}

size_t decode_workspace_bytes(int32_t batch, int32_t max_pages, int32_t num_q_heads, int32_t head_dim) {
  const int64_t max_items = max_items_of(batch, max_pages);
  size_t s = 256;                                   // header
  s += align256(sizeof(int32_t) * size_t(batch));      // item_base
  s += align256(sizeof(int4) * size_t(batch));         // merge_list
  s += align256(2 * sizeof(int4) * size_t(max_items)); // items
  s += align256(sizeof(float) * size_t(max_items) * num_q_heads * part_stride(head_dim));
  s += 2 * kCtrStride * sizeof(uint32_t);  // work counters
  return s;
}

DecodeWorkspace carve_workspace(void* base, int32_t batch, int32_t max_pages, int32_t num_q_heads,
                                int32_t head_dim) {
  const int64_t max_items = max_items_of(batch, max_pages);
  uint8_t* q = static_cast<uint8_t*>(base);
  DecodeWorkspace w;
  w.header = reinterpret_cast<uint32_t*>(q);
  q += 256;
  w.item_base = reinterpret_cast<int32_t*>(q);
  q += align256(sizeof(int32_t) * size_t(batch));
  w.merge_list = reinterpret_cast<int4*>(q);
  q += align256(sizeof(int4) * size_t(batch));
  w.items = reinterpret_cast<int4*>(q);
  q += align256(2 * sizeof(int4) * size_t(max_items));
  w.partials = reinterpret_cast<float*>(q);
  q += align256(sizeof(float) * size_t(max_items) * num_q_heads * part_stride(head_dim));
  w.ctr = reinterpret_cast<uint32_t*>(q);
  w.max_items = max_items;
  return w;
}

// ---------------------------------------------- allocation-free decode --
// Scratch of kv4_decode_attention_noalloc (the plan and the partials of one
// decode call), for callers that cannot allocate device memory.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device array: the
// device address is taken once per device, with that device current, and
// only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[KV4_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(int fmt, const DecodeParams& p, int head_dim, unsigned phases, hipStream_t stream,
                         const AppendParams* append) {
  if (fmt == kFmtKV4) return launch_fmt<kFmtKV4>(p, head_dim, phases, append, stream);
  if (fmt == kFmtKV4Q8) return launch_fmt<kFmtKV4Q8>(p, head_dim, phases, append, stream);
  if (fmt == kFmtKV8) return launch_fmt<kFmtKV8>(p, head_dim, phases, append, stream);
  return launch_fmt<kFmtBF16>(p, head_dim, phases, append, stream);
}

}  // namespace kv4

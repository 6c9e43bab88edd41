// append_body.h -- the per-(token, kv head) append work, shared by the
// append launch and the fused append + plan launch of the decode library.
//
// One wave per (new token, kv head).  Lane l holds E = D/64 consecutive
// channels (2 at head_dim 128, 1 at 64).  The quantizer is the calibration-free
// symmetric rule of the header (news summary "Async RL squeezes context into
// fewer decode steps; ...", Synopsis): scale = fp16_rne(min(amax/qmax, 65504)),
// code = clamp(rint(x / scale), -qmax, qmax), both divides IEEE fp32.  INT4
// uses 32-channel groups (qmax 7); the INT8 copy uses the whole row (qmax 127).
// No two positions share a byte in any format, so tokens of one sequence may
// be appended in one launch without atomics.
#pragma once
#include "kv4_common.h"
#include "kv4_launch.h"

namespace kv4 {
namespace {

// Largest b with cu[b] <= t (cu non-decreasing, cu[0] = 0 <= t < cu[batch]),
// searched by the whole wave: each round the 64 lanes probe evenly spaced
// entries of the current bracket, which shrinks it 64-fold (two rounds for
// 4096 sequences) instead of halving it per dependent load.
__device__ inline int find_seq(const int32_t* __restrict__ cu, int batch, int t, int lane) {
  int lo = 0, hi = batch;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int step = (hi - lo + kWave - 1) / kWave;
    const int idx = lo + lane * step;
    const bool le = idx < hi && cu[idx] <= t;  // true on a prefix of the lanes, lane 0 included
    const unsigned long long m = __ballot(le);
    const int last = 63 - __clzll((long long)m);
    lo = lo + last * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

template <int E>
__device__ inline void quantize(const float (&x)[E], float amax, float qmax, int (&code)[E], uint16_t& sbits) {
  sbits = quant_scale_bits(amax, qmax);
  const float s16 = f16_to_f32(sbits);
#pragma unroll
  for (int e = 0; e < E; ++e) code[e] = quant_code(x[e], s16, qmax);
}

template <int E>
__device__ inline void write_int8_row(uint8_t* __restrict__ tile, int r, int lane, const float (&k)[E],
                                      const float (&v)[E]) {
  constexpr int D = E * kWave;
  float ka = 0.f, va = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ka = fmaxf(ka, fabsf(k[e]));
    va = fmaxf(va, fabsf(v[e]));
  }
  ka = wave_max<kWave>(ka);
  va = wave_max<kWave>(va);
  int kc[E], vc[E];
  uint16_t ks, vs;
  quantize<E>(k, ka, 127.0f, kc, ks);
  quantize<E>(v, va, 127.0f, vc, vs);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int c = lane * E + e;
    tile[k8_byte(D, r, c)] = uint8_t(kc[e]);
    tile[v8_byte(D, r, c)] = uint8_t(vc[e]);
  }
  if (lane == 0) {
    *reinterpret_cast<uint16_t*>(tile + k8_scale(D, r)) = ks;
    *reinterpret_cast<uint16_t*>(tile + v8_scale(D, r)) = vs;
  }
}

template <int E>
__device__ inline void write_int4_row(uint8_t* __restrict__ blk, int r, int lane, const float (&k)[E],
                                      const float (&v)[E]) {
  constexpr int D = E * kWave;
  constexpr int LPG = kGroup / E;  // lanes per 32-channel group
  float ka = 0.f, va = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ka = fmaxf(ka, fabsf(k[e]));
    va = fmaxf(va, fabsf(v[e]));
  }
  ka = wave_max<LPG>(ka);  // xor offsets < LPG stay inside the group
  va = wave_max<LPG>(va);
  int kc[E], vc[E];
  uint16_t ks, vs;
  quantize<E>(k, ka, 7.0f, kc, ks);
  quantize<E>(v, va, 7.0f, vc, vs);
  const int grp = (lane * E) / kGroup;
  if ((lane % LPG) == 0) {
    *reinterpret_cast<uint16_t*>(blk + k4_scale(D, r, grp)) = ks;
    *reinterpret_cast<uint16_t*>(blk + v4_scale(D, r, grp)) = vs;
  }
  // K: a byte holds channels (2i, 2i+1) of this position.
  if constexpr (E == 2) {
    blk[k4_byte(D, r, lane * 2)] = uint8_t((kc[0] & 15) | ((kc[1] & 15) << 4));
  } else {
    int partner = __shfl_xor(kc[0], 1, kWave);
    if ((lane & 1) == 0) blk[k4_byte(D, r, lane)] = uint8_t((kc[0] & 15) | ((partner & 15) << 4));
  }
  // V: a byte holds channels c and c+16 (c/16 even) of this position; the
  // lane holding channel c+16 is lane + 16/E.
  constexpr int PART = 16 / E;
  int pv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) pv[e] = __shfl_xor(vc[e], PART, kWave);
  if (((lane * E / 16) & 1) == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int c = lane * E + e;
      blk[v4_byte(D, r, c)] = uint8_t((vc[e] & 15) | ((pv[e] & 15) << 4));
    }
  }
}

template <int E>
__device__ inline void write_bf16_row(uint8_t* __restrict__ tile, int r, int lane, const uint16_t (&k)[E],
                                      const uint16_t (&v)[E]) {
  constexpr int D = E * kWave;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int c = lane * E + e;
    *reinterpret_cast<uint16_t*>(tile + kb_byte(D, r, c)) = k[e];
    *reinterpret_cast<uint16_t*>(tile + vb_byte(D, r, c)) = v[e];
  }
}

// The append work of wave w: new token w / num_kv_heads, kv head
// w % num_kv_heads (waves past the last pair return).
template <int FMT, int E>
__device__ inline void append_row(const AppendParams& p, int64_t w) {
  constexpr int D = E * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int H = p.num_kv_heads;
  if (w >= int64_t(p.total_new) * H) return;
  const int t = int(w / H), h = int(w % H);
  // the new row's values do not depend on the sequence: load them first
  const uint16_t* kr = p.k_new + (int64_t(t) * H + h) * D + lane * E;
  const uint16_t* vr = p.v_new + (int64_t(t) * H + h) * D + lane * E;
  uint16_t kb[E], vb[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kb[e] = kr[e];
    vb[e] = vr[e];
  }
  // The sequence of token t: first the guess for equal token counts per
  // sequence (one token each in a decode step), whose cu_new entries,
  // length and slot are loaded together; a search when the guess is wrong.
  int b = int(int64_t(t) * p.batch / p.total_new);
  int c0 = p.cu_new[b], c1 = p.cu_new[b + 1], len = p.seq_lens[b];
  int slot = p.slot_ids ? p.slot_ids[b] : b;
  if (!(c0 <= t && t < c1)) {  // wave-uniform
    b = find_seq(p.cu_new, p.batch, t, lane);
    c0 = p.cu_new[b];
    c1 = p.cu_new[b + 1];
    len = p.seq_lens[b];
    slot = p.slot_ids ? p.slot_ids[b] : b;
  }
  const int pos = len - (c1 - c0) + (t - c0);
  if (pos < 0 || pos >= p.max_pages * kPage) return;  // outside the page table: skipped
  const int64_t pid = p.page_table[int64_t(b) * p.max_pages + pos / kPage];
  if (pid < 0 || pid >= p.num_pages) return;
  const int r = pos % kPage;

  float kf[E], vf[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kf[e] = bf16_to_f32(kb[e]);
    vf[e] = bf16_to_f32(vb[e]);
  }
  uint8_t* blk = p.pages + (pid * H + h) * int64_t(p.block_bytes);
  if constexpr (FMT == kFmtKV4) {
    write_int4_row<E>(blk, r, lane, kf, vf);
    const int S = p.n_sink, R = p.n_recent;
    // A ring row is written only by a position that is still among the last R
    // after this call, so positions of one call never share a ring row (the
    // result equals appending the tokens one at a time).
    if (pos < S || (R > 0 && pos >= len - R)) {
      if (slot >= 0 && slot < p.num_slots) {
        const int row = side_row(pos, S, R);
        uint8_t* tile = p.side + (int64_t(slot) * H + h) * int64_t(p.side_bytes) +
                        int64_t(row / kPage) * int64_t(int8_tile_bytes(D));
        write_int8_row<E>(tile, row % kPage, lane, kf, vf);
      }
    }
  } else if constexpr (FMT == kFmtKV8) {
    write_int8_row<E>(blk, r, lane, kf, vf);
  } else {
    write_bf16_row<E>(blk, r, lane, kb, vb);
  }
}

}  // namespace
}  // namespace kv4

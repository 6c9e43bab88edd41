// decode.hip -- single-token GQA decode attention over the paged caches.
//
// Three kernels on the caller's stream:
//   1. worklist  (1 workgroup): per sequence, the number of work items.  The
//      middle region is cut into chunks of `chunk_pages` INT4 pages; item 0
//      also carries the protected rows (INT8 sinks + recent ring).
//   2. attention (persistent grid, one wave per unit = item x kv head): the
//      online softmax over the item's rows.  A sequence with one item writes
//      the final bf16 output and lse directly; otherwise the item writes an
//      fp32 partial (o, m, l).
//   3. merge: exact log-sum-exp merge of the partials of split sequences.
// The regional merge is exact (news summary "Async RL squeezes context into
// fewer decode steps; ...", Interpretation paragraph 3): processing protected
// and middle rows in one online softmax, or in several partials merged by
// log-sum-exp, both equal one softmax over all positions.
#include "kv4_common.h"
#include "kv4_launch.h"

namespace kv4 {
namespace {

constexpr int kChunkPages = 32;

// ---------------------------------------------------------------- worklist --
__device__ inline int items_of(int L, int S, int R, int chunk_pages, int* mid_first_page, int* mid_last_page) {
  Regions g = regions(L, S, R);
  int np = 0;
  if (g.me > g.mb) {
    *mid_first_page = g.mb / kPage;
    *mid_last_page = (g.me - 1) / kPage;
    np = *mid_last_page - *mid_first_page + 1;
  } else {
    *mid_first_page = 0;
    *mid_last_page = -1;
  }
  int n = (np + chunk_pages - 1) / chunk_pages;
  return n < 1 ? 1 : n;
}

__global__ __launch_bounds__(1024) void worklist_kernel(DecodeParams p) {
  __shared__ int scan[1024];
  __shared__ int running;
  const int tid = threadIdx.x;
  if (tid == 0) running = 0;
  __syncthreads();
  for (int base = 0; base < p.batch; base += 1024) {
    const int b = base + tid;
    int n = 0, f, l;
    if (b < p.batch) {
      int L = p.seq_lens[b];
      L = L < 0 ? 0 : (L > p.max_pages * kPage ? p.max_pages * kPage : L);
      n = items_of(L, p.n_sink, p.n_recent, p.chunk_pages, &f, &l);
    }
    scan[tid] = n;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
      int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int start = running + scan[tid] - n;
    if (b < p.batch) {
      p.ws.item_base[b] = start;
      p.ws.item_count[b] = n;
      for (int k = 0; k < n; ++k) p.ws.items[start + k] = make_int2(b, k);
    }
    __syncthreads();
    if (tid == 1023) running += scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    p.ws.header[0] = 0u;
    p.ws.header[1] = uint32_t(running);
  }
}

// ------------------------------------------------------- row dequantization --
template <int E>
__device__ inline void load_int8_row(const uint8_t* __restrict__ tile, int r, int lane, float (&k)[E],
                                     float (&v)[E]) {
  constexpr int D = E * kWave;
  const float sk = f16_to_f32(*reinterpret_cast<const uint16_t*>(tile + k8_scale(D, r)));
  const float sv = f16_to_f32(*reinterpret_cast<const uint16_t*>(tile + v8_scale(D, r)));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    k[e] = float(int8_t(tile[k8_byte(D, r, c)])) * sk;
    v[e] = float(int8_t(tile[v8_byte(D, r, c)])) * sv;
  }
}

__device__ inline int nibble(uint8_t b, int high) {
  int n = high ? (b >> 4) : (b & 15);
  return n >= 8 ? n - 16 : n;
}

template <int E>
__device__ inline void load_int4_row(const uint8_t* __restrict__ blk, int r, int lane, float (&k)[E],
                                     float (&v)[E]) {
  constexpr int D = E * kWave;
  const int grp = (lane * E) / kGroup;
  const float sk = f16_to_f32(*reinterpret_cast<const uint16_t*>(blk + k4_scale(D, r, grp)));
  const float sv = f16_to_f32(*reinterpret_cast<const uint16_t*>(blk + v4_scale(D, r, grp)));
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    k[e] = float(nibble(blk[k4_byte(D, r, c)], c & 1)) * sk;
    v[e] = float(nibble(blk[v4_byte(D, r, c)], (c / 16) & 1)) * sv;
  }
}

template <int E>
__device__ inline void load_bf16_row(const uint8_t* __restrict__ tile, int r, int lane, float (&k)[E],
                                     float (&v)[E]) {
  constexpr int D = E * kWave;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    k[e] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(tile + kb_byte(D, r, c)));
    v[e] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(tile + vb_byte(D, r, c)));
  }
}

// ------------------------------------------------------------- attention ---
template <int E, int G>
struct Online {
  float q[G][E];
  float m[G], l[G], o[G][E];

  __device__ inline void init() {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) o[j][e] = 0.f;
    }
  }
  // One position: scores for the G heads, online softmax update.
  __device__ inline void step(const float (&k)[E], const float (&v)[E], float sm) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = fmaf(q[j][e], k[e], d);
      d = wave_sum<kWave>(d) * sm;
      const float mn = fmaxf(m[j], d);
      const float a = __expf(m[j] - mn);
      const float pj = __expf(d - mn);
      l[j] = l[j] * a + pj;
#pragma unroll
      for (int e = 0; e < E; ++e) o[j][e] = fmaf(pj, v[e], o[j][e] * a);
      m[j] = mn;
    }
  }
};

template <int FMT, int E, int G>
__global__ __launch_bounds__(256) void attention_kernel(DecodeParams p) {
  constexpr int D = E * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int H = p.num_kv_heads, Hq = p.num_q_heads;
  const int S = FMT == kFmtKV4 ? p.n_sink : 0;
  const int R = FMT == kFmtKV4 ? p.n_recent : 0;
  const int64_t units = int64_t(p.ws.header[1]) * H;
  for (;;) {
    int64_t u = 0;
    if (lane == 0) u = atomicAdd(&p.ws.header[0], 1u);
    u = __shfl(int(u), 0, kWave);
    if (u >= units) break;
    const int2 it = p.ws.items[u / H];
    const int h = int(u % H);
    const int b = it.x, chunk = it.y;
    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_pages * kPage ? p.max_pages * kPage : L);
    const Regions g = regions(L, S, R);

    Online<E, G> st;
    st.init();
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e)
        st.q[j][e] = bf16_to_f32(p.q[(int64_t(b) * Hq + h * G + j) * D + lane * E + e]);

    float k[E], v[E];
    if (FMT == kFmtKV4 && chunk == 0 && (g.se > 0 || g.rb < L)) {
      const int slot = p.slot_ids ? p.slot_ids[b] : b;
      if (slot >= 0 && slot < p.num_slots) {
        const uint8_t* sblk = p.side + (int64_t(slot) * H + h) * p.side_bytes;
        for (int pos = 0; pos < L; ++pos) {
          if (pos == g.se) pos = g.rb;  // skip the middle
          if (pos >= L) break;
          const int row = side_row(pos, S, R);
          load_int8_row<E>(sblk + int64_t(row / kPage) * int8_tile_bytes(D), row % kPage, lane, k, v);
          st.step(k, v, p.softmax_scale);
        }
      }
    }
    if (g.me > g.mb) {
      const int first = g.mb / kPage + chunk * p.chunk_pages;
      int last = first + p.chunk_pages - 1;
      if (last > (g.me - 1) / kPage) last = (g.me - 1) / kPage;
      for (int pg = first; pg <= last; ++pg) {
        const int64_t pid = p.page_table[int64_t(b) * p.max_pages + pg];
        if (pid < 0 || pid >= p.num_pages) continue;
        const uint8_t* blk = p.pages + (pid * H + h) * p.block_bytes;
        for (int r = 0; r < kPage; ++r) {
          const int pos = pg * kPage + r;
          if (pos < g.mb || pos >= g.me) continue;
          if constexpr (FMT == kFmtKV4) load_int4_row<E>(blk, r, lane, k, v);
          else if constexpr (FMT == kFmtKV8) load_int8_row<E>(blk, r, lane, k, v);
          else load_bf16_row<E>(blk, r, lane, k, v);
          st.step(k, v, p.softmax_scale);
        }
      }
    }

    const int nitems = p.ws.item_count[b];
    if (nitems == 1) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int hq = h * G + j;
        const float inv = st.l[j] > 0.f ? 1.0f / st.l[j] : 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
          p.out[(int64_t(b) * Hq + hq) * D + lane * E + e] = f32_to_bf16_bits(st.o[j][e] * inv);
        if (p.lse && lane == 0) p.lse[int64_t(b) * Hq + hq] = st.l[j] > 0.f ? st.m[j] + logf(st.l[j]) : -INFINITY;
      }
    } else {
      const int64_t slot = int64_t(p.ws.item_base[b] + chunk) * Hq;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float* part = p.ws.partials + (slot + h * G + j) * (D + 2);
#pragma unroll
        for (int e = 0; e < E; ++e) part[lane * E + e] = st.o[j][e];
        if (lane == 0) {
          part[D] = st.m[j];
          part[D + 1] = st.l[j];
        }
      }
    }
  }
}

// ----------------------------------------------------------------- merge ---
template <int E>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
  constexpr int D = E * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int Hq = p.num_q_heads;
  const int64_t w = int64_t(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (w >= int64_t(p.batch) * Hq) return;
  const int b = int(w / Hq), hq = int(w % Hq);
  const int n = p.ws.item_count[b];
  if (n <= 1) return;
  const int64_t base = int64_t(p.ws.item_base[b]) * Hq + hq;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, p.ws.partials[(base + int64_t(i) * Hq) * (D + 2) + D]);
  float l = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int i = 0; i < n; ++i) {
    const float* part = p.ws.partials + (base + int64_t(i) * Hq) * (D + 2);
    const float li = part[D + 1];
    if (li <= 0.f) continue;  // empty item
    const float a = __expf(part[D] - M);
    l += a * li;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(a, part[lane * E + e], o[e]);
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) p.out[(int64_t(b) * Hq + hq) * D + lane * E + e] = f32_to_bf16_bits(o[e] * inv);
  if (p.lse && lane == 0) p.lse[int64_t(b) * Hq + hq] = l > 0.f ? M + logf(l) : -INFINITY;
}

// --------------------------------------------------------------- launch ---
int persistent_blocks(const void* kernel) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return cus * per_cu;
}

template <int FMT, int E, int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const void* k = reinterpret_cast<const void*>(&attention_kernel<FMT, E, G>);
  const int blocks = persistent_blocks(k);
  if (blocks <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((attention_kernel<FMT, E, G>), dim3(blocks), dim3(256), 0, stream, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t waves = int64_t(p.batch) * p.num_q_heads;
  hipLaunchKernelGGL((merge_kernel<E>), dim3(unsigned((waves + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int FMT, int E>
hipError_t launch_e(const DecodeParams& p, hipStream_t stream) {
  switch (p.num_q_heads / p.num_kv_heads) {
    case 1: return launch_g<FMT, E, 1>(p, stream);
    case 2: return launch_g<FMT, E, 2>(p, stream);
    case 4: return launch_g<FMT, E, 4>(p, stream);
    case 8: return launch_g<FMT, E, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
hipError_t launch_fmt(const DecodeParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 128 ? launch_e<FMT, 2>(p, stream) : launch_e<FMT, 1>(p, stream);
}

}  // namespace

int32_t decode_chunk_pages() { return kChunkPages; }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t decode_workspace_bytes(int32_t batch, int32_t max_pages, int32_t num_q_heads, int32_t head_dim) {
  const int64_t per_seq = (int64_t(max_pages) + kChunkPages - 1) / kChunkPages;
  const int64_t max_items = int64_t(batch) * (per_seq < 1 ? 1 : per_seq);
  size_t s = 256;                                   // header
  s += align256(sizeof(int32_t) * size_t(batch));  // item_base
  s += align256(sizeof(int32_t) * size_t(batch));  // item_count
  s += align256(sizeof(int2) * size_t(max_items)); // items
  s += align256(sizeof(float) * size_t(max_items) * num_q_heads * (head_dim + 2));
  return s;
}

DecodeWorkspace carve_workspace(void* base, int32_t batch, int32_t max_pages, int32_t num_q_heads,
                                int32_t head_dim) {
  const int64_t per_seq = (int64_t(max_pages) + kChunkPages - 1) / kChunkPages;
  const int64_t max_items = int64_t(batch) * (per_seq < 1 ? 1 : per_seq);
  uint8_t* p = static_cast<uint8_t*>(base);
  DecodeWorkspace w;
  w.header = reinterpret_cast<uint32_t*>(p);
  p += 256;
  w.item_base = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(batch));
  w.item_count = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * size_t(batch));
  w.items = reinterpret_cast<int2*>(p);
  p += align256(sizeof(int2) * size_t(max_items));
  w.partials = reinterpret_cast<float*>(p);
  w.max_items = max_items;
  (void)num_q_heads;
  (void)head_dim;
  return w;
}

hipError_t launch_decode(int fmt, const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (fmt == kFmtKV4) return launch_fmt<kFmtKV4>(p, head_dim, stream);
  if (fmt == kFmtKV8) return launch_fmt<kFmtKV8>(p, head_dim, stream);
  return launch_fmt<kFmtBF16>(p, head_dim, stream);
}

}  // namespace kv4

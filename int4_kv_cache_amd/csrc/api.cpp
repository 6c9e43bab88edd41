// api.cpp -- the extern "C" boundary of libkv4: argument checks, sizes,
// workspace carving and kernel launches.  Nothing here touches device memory.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv4.h"
#include "kv4_common.h"
#include "kv4_launch.h"

namespace {

using kv4::kFmtBF16;
using kv4::kFmtKV4;
using kv4::kFmtKV8;

bool layout_valid(const kv4_layout* L) {
  return L && L->num_kv_heads > 0 && L->num_q_heads > 0 && L->num_q_heads % L->num_kv_heads == 0 &&
         L->n_sink >= 0 && L->n_recent >= 0;
}

kv4_status layout_check(const kv4_layout* L, int fmt) {
  if (!layout_valid(L)) return KV4_ERR_INVALID_ARG;
  if (L->head_dim != 64 && L->head_dim != 128) return KV4_ERR_UNSUPPORTED;
  if (L->page_size != 16 || L->group_size != 32) return KV4_ERR_UNSUPPORTED;
  const int g = L->num_q_heads / L->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KV4_ERR_UNSUPPORTED;
  if (L->flags & ~(KV4_LAYOUT_WIDE_PROTECTION | KV4_LAYOUT_INT8_QUERY)) return KV4_ERR_INVALID_ARG;
  const int max_prot = (L->flags & KV4_LAYOUT_WIDE_PROTECTION) ? KV4_WIDE_PROTECTION_MAX : kv4::kMaxProtected;
  if (fmt == kFmtKV4 && int64_t(L->n_sink) + L->n_recent > max_prot) return KV4_ERR_INVALID_ARG;
  return KV4_OK;
}

size_t block_bytes(const kv4_layout* L, int fmt) {
  if (!L || (L->head_dim != 64 && L->head_dim != 128)) return 0;
  const int D = L->head_dim;
  if (fmt == kFmtKV4) return kv4::int4_block_bytes(D);
  if (fmt == kFmtKV8) return kv4::int8_tile_bytes(D);
  return kv4::bf16_tile_bytes(D);
}

size_t side_bytes(const kv4_layout* L) {
  if (!L || (L->head_dim != 64 && L->head_dim != 128) || L->n_sink < 0 || L->n_recent < 0) return 0;
  return size_t(kv4::side_tiles(L->n_sink, L->n_recent)) * kv4::int8_tile_bytes(L->head_dim);
}

bool protected_set(const kv4_layout* L, int fmt) { return fmt == kFmtKV4 && L->n_sink + L->n_recent > 0; }

kv4_status cache_batch_check(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, int fmt) {
  if (!c || !b) return KV4_ERR_INVALID_ARG;
  if (!c->pages || c->num_pages <= 0) return KV4_ERR_INVALID_ARG;
  if (b->batch < 0 || b->max_pages <= 0) return KV4_ERR_INVALID_ARG;
  if (b->batch > 0 && (!b->page_table || !b->seq_lens)) return KV4_ERR_INVALID_ARG;
  if (protected_set(L, fmt) && (!c->side || c->num_slots <= 0)) return KV4_ERR_INVALID_ARG;
  return KV4_OK;
}

// Checks the append arguments and fills `p`; p.total_new = 0 when there is
// nothing to append (total 0 or an empty batch).
kv4_status append_params(int fmt, const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                         const uint16_t* k, const uint16_t* v, const int32_t* cu, int32_t total,
                         kv4::AppendParams& p) {
  kv4_status s = layout_check(L, fmt);
  if (s != KV4_OK) return s;
  s = cache_batch_check(L, c, b, fmt);
  if (s != KV4_OK) return s;
  if (total < 0) return KV4_ERR_INVALID_ARG;
  p = kv4::AppendParams{};
  if (total == 0 || b->batch == 0) return KV4_OK;
  if (!k || !v || !cu) return KV4_ERR_INVALID_ARG;
  p.pages = static_cast<uint8_t*>(c->pages);
  p.num_pages = c->num_pages;
  p.side = static_cast<uint8_t*>(c->side);
  p.num_slots = c->num_slots;
  p.page_table = b->page_table;
  p.max_pages = b->max_pages;
  p.seq_lens = b->seq_lens;
  p.slot_ids = b->slot_ids;
  p.batch = b->batch;
  p.k_new = k;
  p.v_new = v;
  p.cu_new = cu;
  p.total_new = total;
  p.num_kv_heads = L->num_kv_heads;
  p.n_sink = fmt == kFmtKV4 ? L->n_sink : 0;
  p.n_recent = fmt == kFmtKV4 ? L->n_recent : 0;
  p.block_bytes = int64_t(block_bytes(L, fmt));
  p.side_bytes = int64_t(side_bytes(L));
  if (!protected_set(L, fmt)) {
    p.side = nullptr;
    p.num_slots = 0;
  }
  return KV4_OK;
}

kv4_status append_impl(int fmt, const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                       const uint16_t* k, const uint16_t* v, const int32_t* cu, int32_t total,
                       hipStream_t stream) {
  kv4::AppendParams p;
  const kv4_status s = append_params(fmt, L, c, b, k, v, cu, total, p);
  if (s != KV4_OK || p.total_new == 0) return s;
  return kv4::launch_append(fmt, p, L->head_dim, stream) == hipSuccess ? KV4_OK : KV4_ERR_LAUNCH;
}

// Checks the decode arguments and fills `p` and the kernel format `kfmt`.
// With an empty batch it returns KV4_OK and sets p.batch = 0 (nothing to launch).
// check_only: every check, including the workspace size against ws_bytes, but
// no workspace address yet (ws may be null; p.ws is left empty).
kv4_status decode_params(int fmt, const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                         const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                         unsigned phases, int32_t nq, kv4::DecodeParams& p, int& kfmt, bool check_only = false) {
  if (phases < 1u || phases > 7u) return KV4_ERR_INVALID_ARG;
  if (nq < 1 || nq > KV4_MAX_QUERIES) return KV4_ERR_INVALID_ARG;
  kv4_status s = layout_check(L, fmt);
  if (s != KV4_OK) return s;
  if (!b) return KV4_ERR_INVALID_ARG;
  const bool plan_only = phases == KV4_PHASE_PLAN;
  if (plan_only) {
    if (b->batch < 0 || b->max_pages <= 0) return KV4_ERR_INVALID_ARG;
    if (b->batch > 0 && (!b->page_table || !b->seq_lens)) return KV4_ERR_INVALID_ARG;
  } else {
    s = cache_batch_check(L, c, b, fmt);
    if (s != KV4_OK) return s;
  }
  p = kv4::DecodeParams{};
  if (b->batch == 0) return KV4_OK;
  if (!ws && !check_only) return KV4_ERR_INVALID_ARG;
  if ((phases & (KV4_PHASE_ATTEND | KV4_PHASE_MERGE)) && !out) return KV4_ERR_INVALID_ARG;
  if ((phases & KV4_PHASE_ATTEND) && !q) return KV4_ERR_INVALID_ARG;
  if (!(sm > 0.0f) || sm > 3.0e38f) return KV4_ERR_INVALID_ARG;  // positive and finite
  // the kernels index work by b * nq + t
  if (int64_t(b->batch) * nq > int64_t(INT32_MAX)) return KV4_ERR_UNSUPPORTED;
  const int32_t nv = b->batch * nq;
  if (!kv4::decode_units_fit(nv, b->max_pages, L->num_q_heads, L->num_kv_heads, L->head_dim))
    return KV4_ERR_UNSUPPORTED;
  const size_t need = kv4::decode_workspace_bytes(nv, b->max_pages, L->num_q_heads, L->head_dim);
  if (ws_bytes < need) return KV4_ERR_WORKSPACE;
  if (c) {
    p.pages = static_cast<const uint8_t*>(c->pages);
    p.num_pages = c->num_pages;
    p.side = static_cast<const uint8_t*>(c->side);
    p.num_slots = c->num_slots;
  }
  p.page_table = b->page_table;
  p.max_pages = b->max_pages;
  p.seq_lens = b->seq_lens;
  p.slot_ids = b->slot_ids;
  p.batch = b->batch;
  p.nq = nq;
  p.tq = 1;  // set by the launcher for the kernel it picks
  p.q = q;
  p.softmax_scale = sm;
  p.out = out;
  p.lse = lse;
  p.num_q_heads = L->num_q_heads;
  p.num_kv_heads = L->num_kv_heads;
  p.n_sink = fmt == kFmtKV4 ? L->n_sink : 0;
  p.n_recent = fmt == kFmtKV4 ? L->n_recent : 0;
  p.block_bytes = int64_t(block_bytes(L, fmt));
  p.side_bytes = int64_t(side_bytes(L));
  if (!check_only) p.ws = kv4::carve_workspace(ws, nv, b->max_pages, L->num_q_heads, L->head_dim);
  if (!protected_set(L, fmt)) {
    p.side = nullptr;
    p.num_slots = 0;
  }
  kfmt = fmt;
  if (L->flags & KV4_LAYOUT_INT8_QUERY) {
    if (fmt != kFmtKV4) return KV4_ERR_UNSUPPORTED;
    kfmt = kv4::kFmtKV4Q8;
  }
  return KV4_OK;
}

kv4_status decode_impl(int fmt, const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                       const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                       unsigned phases, hipStream_t stream, int32_t nq = 1) {
  kv4::DecodeParams p;
  int kfmt = fmt;
  const kv4_status s = decode_params(fmt, L, c, b, q, sm, out, lse, ws, ws_bytes, phases, nq, p, kfmt);
  if (s != KV4_OK || p.batch == 0) return s;
  return kv4::launch_decode(kfmt, p, L->head_dim, phases, stream) == hipSuccess ? KV4_OK : KV4_ERR_LAUNCH;
}

// Append, then the selected decode phases; the plan shares the append's launch.
kv4_status append_decode_impl(int fmt, const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                              const uint16_t* k, const uint16_t* v, const int32_t* cu, int32_t total,
                              const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws,
                              size_t ws_bytes, unsigned phases, hipStream_t stream) {
  kv4::AppendParams a;
  kv4_status s = append_params(fmt, L, c, b, k, v, cu, total, a);
  if (s != KV4_OK) return s;
  kv4::DecodeParams p;
  int kfmt = fmt;
  s = decode_params(fmt, L, c, b, q, sm, out, lse, ws, ws_bytes, phases, 1, p, kfmt);
  if (s != KV4_OK || p.batch == 0) return s;
  return kv4::launch_decode(kfmt, p, L->head_dim, phases, stream, &a) == hipSuccess ? KV4_OK : KV4_ERR_LAUNCH;
}

constexpr unsigned kAllPhases = KV4_PHASE_PLAN | KV4_PHASE_ATTEND | KV4_PHASE_MERGE;

}  // namespace

extern "C" {

int32_t kv4_abi_version(void) { return KV4_ABI_VERSION; }

const char* kv4_status_string(int32_t s) {
  // an int, not the enum: callers may pass any code, and a C++ enum object
  // holding a value outside its enumerators' range is undefined
  switch (s) {
    case KV4_OK: return "ok";
    case KV4_ERR_INVALID_ARG: return "invalid argument";
    case KV4_ERR_UNSUPPORTED: return "unsupported shape";
    case KV4_ERR_WORKSPACE: return "workspace too small";
    case KV4_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

size_t kv4_block_bytes(const kv4_layout* L) { return block_bytes(L, kFmtKV4); }
size_t kv8_block_bytes(const kv4_layout* L) { return block_bytes(L, kFmtKV8); }
size_t kvbf16_block_bytes(const kv4_layout* L) { return block_bytes(L, kFmtBF16); }
size_t kv4_side_bytes(const kv4_layout* L) { return side_bytes(L); }

kv4_status kv4_append(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* k,
                      const uint16_t* v, const int32_t* cu, int32_t total, hipStream_t stream) {
  return append_impl(kFmtKV4, L, c, b, k, v, cu, total, stream);
}
kv4_status kv8_append(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* k,
                      const uint16_t* v, const int32_t* cu, int32_t total, hipStream_t stream) {
  return append_impl(kFmtKV8, L, c, b, k, v, cu, total, stream);
}
kv4_status kvbf16_append(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* k,
                         const uint16_t* v, const int32_t* cu, int32_t total, hipStream_t stream) {
  return append_impl(kFmtBF16, L, c, b, k, v, cu, total, stream);
}

kv4_status kv4_decode_workspace_size(const kv4_layout* L, int32_t batch, int32_t max_pages, size_t* bytes) {
  if (!layout_valid(L) || !bytes || batch < 0 || max_pages <= 0) return KV4_ERR_INVALID_ARG;
  if (L->head_dim != 64 && L->head_dim != 128) return KV4_ERR_UNSUPPORTED;
  *bytes = kv4::decode_workspace_bytes(batch, max_pages, L->num_q_heads, L->head_dim);
  return KV4_OK;
}

kv4_status kv4_decode_attention(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* q,
                                float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return decode_impl(kFmtKV4, L, c, b, q, sm, out, lse, ws, ws_bytes, kAllPhases, stream);
}
kv4_status kv8_decode_attention(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* q,
                                float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return decode_impl(kFmtKV8, L, c, b, q, sm, out, lse, ws, ws_bytes, kAllPhases, stream);
}
kv4_status kvbf16_decode_attention(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                   const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  return decode_impl(kFmtBF16, L, c, b, q, sm, out, lse, ws, ws_bytes, kAllPhases, stream);
}

kv4_status kv4_decode_phases(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* q,
                             float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes, uint32_t phases,
                             hipStream_t stream) {
  return decode_impl(kFmtKV4, L, c, b, q, sm, out, lse, ws, ws_bytes, phases, stream);
}
kv4_status kv8_decode_phases(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* q,
                             float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes, uint32_t phases,
                             hipStream_t stream) {
  return decode_impl(kFmtKV8, L, c, b, q, sm, out, lse, ws, ws_bytes, phases, stream);
}
kv4_status kvbf16_decode_phases(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b, const uint16_t* q,
                                float sm, uint16_t* out, float* lse, void* ws, size_t ws_bytes, uint32_t phases,
                                hipStream_t stream) {
  return decode_impl(kFmtBF16, L, c, b, q, sm, out, lse, ws, ws_bytes, phases, stream);
}

kv4_status kv4_append_decode_phases(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                    const uint16_t* k, const uint16_t* v, const int32_t* cu, int32_t total,
                                    const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws,
                                    size_t ws_bytes, uint32_t phases, hipStream_t stream) {
  return append_decode_impl(kFmtKV4, L, c, b, k, v, cu, total, q, sm, out, lse, ws, ws_bytes, phases, stream);
}
kv4_status kv8_append_decode_phases(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                    const uint16_t* k, const uint16_t* v, const int32_t* cu, int32_t total,
                                    const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws,
                                    size_t ws_bytes, uint32_t phases, hipStream_t stream) {
  return append_decode_impl(kFmtKV8, L, c, b, k, v, cu, total, q, sm, out, lse, ws, ws_bytes, phases, stream);
}
kv4_status kvbf16_append_decode_phases(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                       const uint16_t* k, const uint16_t* v, const int32_t* cu, int32_t total,
                                       const uint16_t* q, float sm, uint16_t* out, float* lse, void* ws,
                                       size_t ws_bytes, uint32_t phases, hipStream_t stream) {
  return append_decode_impl(kFmtBF16, L, c, b, k, v, cu, total, q, sm, out, lse, ws, ws_bytes, phases, stream);
}

kv4_status kv4_decode_attention_mq(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                   const uint16_t* q, int32_t num_queries, float sm, uint16_t* out, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(kFmtKV4, L, c, b, q, sm, out, lse, ws, ws_bytes, kAllPhases, stream, num_queries);
}
kv4_status kv8_decode_attention_mq(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                   const uint16_t* q, int32_t num_queries, float sm, uint16_t* out, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(kFmtKV8, L, c, b, q, sm, out, lse, ws, ws_bytes, kAllPhases, stream, num_queries);
}
kv4_status kvbf16_decode_attention_mq(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                      const uint16_t* q, int32_t num_queries, float sm, uint16_t* out,
                                      float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(kFmtBF16, L, c, b, q, sm, out, lse, ws, ws_bytes, kAllPhases, stream, num_queries);
}

kv4_status kv4_decode_attention_noalloc(const kv4_layout* L, const kv4_cache* c, const kv4_batch* b,
                                        const uint16_t* q, float sm, uint16_t* out, float* lse,
                                        hipStream_t stream) {
  // every argument check, and the batch's workspace size against the fixed
  // scratch, happens on the host before the scratch address is looked up
  kv4::DecodeParams p;
  int kfmt = kFmtKV4;
  const kv4_status s = decode_params(kFmtKV4, L, c, b, q, sm, out, lse, nullptr, KV4_NOALLOC_SCRATCH_BYTES,
                                     kAllPhases, 1, p, kfmt, /*check_only=*/true);
  if (s != KV4_OK || p.batch == 0) return s;
  void* ws = nullptr;
  if (kv4::noalloc_scratch(&ws) != hipSuccess) return KV4_ERR_LAUNCH;
  return decode_impl(kFmtKV4, L, c, b, q, sm, out, lse, ws, KV4_NOALLOC_SCRATCH_BYTES, kAllPhases, stream);
}

kv4_status kv4_cache_capacity(const kv4_layout* L, int32_t format, int32_t num_layers, const int32_t* seq_lens,
                              int32_t n, uint64_t budget, uint64_t* total, int32_t* fit) {
  if (!total || !fit || n < 0 || num_layers < 1 || (n > 0 && !seq_lens)) return KV4_ERR_INVALID_ARG;
  if (format != KV4_FORMAT_KV4 && format != KV4_FORMAT_KV8 && format != KV4_FORMAT_BF16) return KV4_ERR_INVALID_ARG;
  const int fmt = format == KV4_FORMAT_KV4 ? kFmtKV4 : (format == KV4_FORMAT_KV8 ? kFmtKV8 : kFmtBF16);
  const kv4_status s = layout_check(L, fmt);
  if (s != KV4_OK) return s;
  const uint64_t per_page = uint64_t(L->num_kv_heads) * block_bytes(L, fmt) * uint64_t(num_layers);
  const uint64_t per_seq = protected_set(L, fmt) ? uint64_t(L->num_kv_heads) * side_bytes(L) * uint64_t(num_layers) : 0;
  uint64_t sum = 0;
  int32_t k = 0;
  bool full = false;
  for (int32_t i = 0; i < n; ++i) {
    if (seq_lens[i] < 0) return KV4_ERR_INVALID_ARG;
    const uint64_t pages = (uint64_t(seq_lens[i]) + uint64_t(L->page_size) - 1) / uint64_t(L->page_size);
    sum += pages * per_page + per_seq;
    if (!full && sum <= budget) k = i + 1;
    else full = true;
  }
  *total = sum;
  *fit = k;
  return KV4_OK;
}

int32_t kv4_probe_blocks(void) { return kv4::probe_blocks(); }

kv4_status kv4_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16) return KV4_ERR_INVALID_ARG;
  return kv4::launch_probe(buf, bytes, sink, stream) == hipSuccess ? KV4_OK : KV4_ERR_LAUNCH;
}

}  // extern "C"

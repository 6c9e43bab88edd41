// kv4_launch.h -- kernel parameter blocks and launchers (host side of libkv4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kv4 {

struct AppendParams {
  uint8_t* pages;
  int64_t num_pages;
  uint8_t* side;
  int32_t num_slots;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* seq_lens;
  const int32_t* slot_ids;
  int32_t batch;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* cu_new;
  int32_t total_new;
  int32_t num_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int64_t block_bytes;
  int64_t side_bytes;
};

hipError_t launch_append(int fmt, const AppendParams& p, int head_dim, hipStream_t stream);

// Decode workspace: a header, the first partial slot of every sequence, the
// records of the sequences split over several items, the work items
// (costliest first) and the fp32 partial results of the split items.
struct DecodeWorkspace {
  uint32_t* header;      // [0] unused, [1] items, [2] chunk pages, [3] split sequences
  int32_t* item_base;    // [batch] first partial slot of a split sequence
  int4* merge_list;      // [batch] split sequences: {work index, first partial slot, items, 0}
  int4* items;           // [max_items][2] work-item descriptors (two int4 each)
  float* partials;       // [max_items][num_q_heads][head_dim + 4]: o, m, l, padding
  uint32_t* ctr;         // [2][32] work counters: finished waves, the tail's tickets
  int64_t max_items;
};

struct DecodeParams {
  const uint8_t* pages;
  int64_t num_pages;
  const uint8_t* side;
  int32_t num_slots;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* seq_lens;
  const int32_t* slot_ids;
  int32_t batch;
  int32_t nq;  // query tokens per sequence (the last nq positions)
  int32_t tq;  // queries per work block: work index u = b * ceil(nq / tq) + t / tq
  const uint16_t* q;
  float softmax_scale;
  uint16_t* out;
  float* lse;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int64_t block_bytes;
  int64_t side_bytes;
  int32_t resident_waves;  // attention waves resident on the device at once
  DecodeWorkspace ws;
};

size_t decode_workspace_bytes(int32_t batch, int32_t max_pages, int32_t num_q_heads, int32_t head_dim);
// whether the batch's work units can be numbered in 32 bits
bool decode_units_fit(int32_t batch, int32_t max_pages, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim);
DecodeWorkspace carve_workspace(void* base, int32_t batch, int32_t max_pages, int32_t num_q_heads,
                                int32_t head_dim);
// phases: bit 0 work list, bit 1 attention, bit 2 merge
// `append` (optional): new tokens stored before the decode phases run, in the
// same launch as the plan when `phases` holds it.
hipError_t launch_decode(int fmt, const DecodeParams& p, int head_dim, unsigned phases, hipStream_t stream,
                         const AppendParams* append = nullptr);

// Device address of this device's KV4_NOALLOC_SCRATCH_BYTES scratch array
// (looked up once per device; the current device's).
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
int32_t probe_blocks();

}  // namespace kv4

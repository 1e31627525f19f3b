// Host planner for one hybrid batch: validates the metadata and splits the work into prefill
// tile items and decode split-KV items (host-only code, no HIP calls).
#pragma once
#include <string>
#include <vector>

#include "../../include/pod_attn.h"
#include "pod_internal.h"

namespace pod {

struct Config {
  int hq = 0, hkv = 0, d = 0, page = 16, dtype = 0, mode = 0;
  float scale = 0.f;
  int decode_split_tokens = 0, prefill_split_cap = 0, wgs_per_cu = 0, flags = 0;
  int append_token_heads = kAppendTokenHeads;   // (token, KV head) pairs per KV append unit
  int extend_max_q = 0;         // chunks of at most this many rows run on the decode path (0: kExtendMaxQ, <0: never)
  int decode_items_per_wave = 0; // decode items per decode wave of the grid (0: 1, streams handles 2)
  int decode_taper = 8;         // the decode sequences claimed last take 1/decode_taper of the split length (< 2: off)
  int group() const { return hq / hkv; }
  int elem_bytes() const { return dtype == POD_ATTN_FP32 ? 4 : dtype == POD_ATTN_BF16 ? 2 : 1; }   // cache element
  int q_elem_bytes() const { return dtype == POD_ATTN_FP32 ? 4 : 2; }                           // q and out
  int lds_elem_bytes() const { return dtype == POD_ATTN_FP32 ? 4 : 2; }                         // prefill tile in LDS
};

struct Plan {
  std::vector<int32_t> pdesc, ddesc;   // kDescInts each
  std::vector<int32_t> pitems;         // prefill item table: kPItemHeader ints, then (desc, split << 16 | head)
  std::vector<int32_t> aunits;         // KV append units, kAUnitInts each
  int n_pdesc = 0, n_ddesc = 0, n_aunits = 0;
  int n_pf_items = 0, n_dc_items = 0;
  int n_pf_groups = 0, n_groups = 0, n_slots = 0;
  int tile_queries = 0, tile_cols = 0;
  int prefill_max_splits = 0, decode_split_tokens = 0, decode_max_splits = 0;
  int decode_max_cols = 0;      // widest decode-path descriptor: G, or n_q*G for small-q extends
  int num_small_extends = 0;    // prefill chunks planned on the decode path
  int total_q = 0, prefill_rows = 0;
  // Algorithmic work per share (prefill tiles / decode path): 4*D FLOPs per visible (query head,
  // key) pair; bytes = K and V once per KV head per context token, q and out once per row, one
  // int32 block-table entry per page.
  double prefill_flops = 0.0, decode_flops = 0.0;
  double prefill_bytes = 0.0, decode_bytes = 0.0;
  WorkspaceMap map{};
};

// Returns POD_ATTN_OK or an error status with *err set.
pod_attn_status validate_config(const pod_attn_config* c, Config* out, std::string* err);
pod_attn_status plan_batch(const Config& c, const pod_attn_batch* b, int num_cus, int wgs_per_cu,
                           Plan* out, std::string* err);
// Write the host-staged part of the workspace, [map.pdesc, map.copy_bytes), into dst (from dst[0]);
// [0, map.pdesc) (counters, tickets, claim counts) is zero-filled on the device.  Without
// with_units the staged part ends at map.aunits (no KV append this run).
void stage_plan(const Plan& p, const Config& c, uint8_t* dst, bool with_units);
// Expand descriptor-encoded items to the 16-int form of pod_attn_plan_inspect.
void expand_items(const Plan& p, const Config& c, std::vector<int32_t>* items);

}  // namespace pod

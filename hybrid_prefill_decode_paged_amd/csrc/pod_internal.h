// Internal layout shared by the host planner and the gfx950 kernels: work descriptors,
// workspace map and kernel parameter block.  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace pod {

constexpr int kPage = 16;            // tokens per KV page
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTileCols = 128;       // (query, head) columns of one prefill tile: 4 waves x 32
constexpr int kMaxGroup = 16;        // decode-path columns: one 16-wide MFMA block
constexpr int kExtendMaxQ = 16;      // default: prefill chunks of at most this many rows run on the decode path
constexpr int kPrefillKvTile = 64;   // keys per prefill inner iteration (4 pages)
constexpr int kCuSlots = 1024;       // hashed (XCC, SE, CU) slots for per-CU scheduler state
constexpr int kXcds = 8;             // accelerator complex dies (one L2 each)
constexpr int kPItemHeader = 16;     // prefill item table header: queue x = items [hdr[x], hdr[x+1])
constexpr int kMaxCombineSplits = 128;  // max KV splits of one group (LDS weight table rows)
constexpr int kCombineLdsPerWave = 16 * kMaxCombineSplits * 4;   // [16 columns][splits] floats

// A descriptor covers one prefill query tile or one decode sequence; it expands to
// Hkv * n_split work items, split-major: item = split * Hkv + kv_head, so that items taken
// one after another read the adjacent (page, head) slabs of the same pages.
enum DescField {
  kDSeq = 0,        // block-table row
  kDQRow,           // first q/out row
  kDNq,             // query rows (decode: 1)
  kDQPos,           // absolute position of the first query row
  kDKvLen,          // keys the tile needs: last query position + 1 (decode: ctx)
  kDNSplit,         // KV splits per head (>= 1)
  kDSplitTok,       // tokens per split (multiple of the kind's key step)
  kDItemBegin,      // decode: first item index of the descriptor
  kDGroupBegin,     // first combine group (one per head) when n_split > 1, else -1
  kDPartBase,       // first partial slot when n_split > 1
  kDNcols,          // columns = n_q * group
  kDescInts = 16
};

// KV append unit: the new tokens of one sequence that fall in one page (a run of consecutive
// slots), for a range of KV heads; one wave writes one unit before the attention launches.
enum AUnitField {
  kASeq = 0,        // block-table row
  kARow,            // q/k_new/v_new row of the first token
  kAPos,            // absolute position of the first token
  kANtok,           // tokens (1..16, one page)
  kAHead,           // first KV head
  kANh,             // KV heads
  kAUnitInts = 8
};
constexpr int kAppendTokenHeads = 16;   // token-heads per append unit (at most)

// Control block (int32 words at the start of the workspace), zeroed by every run.
enum CtrlWord {
  kCQueuePrefill = 0,
  kCQueueDecode = 64,
  kCStatus = 128,
  kCActivePrefill = 256,                    // [kCuSlots] prefill-role WGs now on each CU
  kCClaimsPrefillCu = 256 + kCuSlots,       // [kCuSlots] prefill items claimed per CU (every run)
  kCClaimsDecodeCu = 256 + 2 * kCuSlots,    // [kCuSlots] decode items claimed per CU (every run)
  kCQueuePrefillXcd = 256 + 3 * kCuSlots,   // [kXcds] prefill queues, one 128-byte line each
  kCtrlInts = kCQueuePrefillXcd + kXcds * 32
};
// Fused kernel: prefill-role workgroups allowed on one CU while decode work remains.  One, so
// that every CU keeps a decode workgroup streaming beside its matrix work.
constexpr int kPrefillPerCu = 1;

enum StatusBits { kStatusBadPage = 1 };

struct KernelParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  void* out;
  int32_t* ctrl;
  int32_t* tickets;          // [n_groups]
  int32_t* claims;           // [n_pf_items + n_dc_items] or null
  uint32_t* trace;           // [n_pf_items + n_dc_items][4] timeline records, or null
  const int32_t* pdesc;      // prefill descriptors
  const int32_t* pitems;     // prefill item table (header, then (desc, split << 16 | head) per item)
  const int32_t* ddesc;      // decode descriptors
  const float* k_scale;      // FP8 cache: [num_pages][Hkv] scale of each K slab, else null
  const float* v_scale;      // FP8 cache: [num_pages][Hkv] scale of each V slab, else null
  const void* k_new;         // [total_q][Hkv][D] keys of the new tokens (append), or null
  const void* v_new;         // [total_q][Hkv][D] values of the new tokens
  const int32_t* aunits;     // [n_aunits][kAUnitInts] append units (workspace copy)
  int n_aunits;
  float* part_o;             // [slots][D]
  float* part_lse;           // [slots], log2-domain log-sum-exp
  int n_pdesc, n_ddesc;
  int n_pf_items, n_dc_items;
  int n_pf_groups, n_groups; // groups [0, n_pf_groups) are prefill, the rest decode
  int hq, hkv, group, bt_stride, num_pages;
  float scale_log2;          // softmax scale * log2(e)
  int inline_combine;        // 1: the last-arriving decode split merges its group in-kernel (fused)
  int group_begin, group_end;// combine kernel range
  int combine_col_blocks;     // combine kernel: workgroups per group (16 columns each)
};

// Arguments of the plan-upload launch (which also writes the KV append in fused mode).
struct StageArgs {
  KernelParams p;            // append fields: k, v, bt, k_new, v_new, hkv, bt_stride, num_pages, n_aunits
  const void* src;           // pinned host staging buffer (its device-visible address)
  void* dst;                 // workspace
  int n_zero16, n_copy16;    // 16-byte words zero-filled, then copied from src
  int copy_wgs;              // workgroups [0, copy_wgs) upload the plan; the rest write append units
  const int32_t* units_host; // append units inside the staging buffer, or null
};

// LDS of one fused workgroup: four objects (K and V staging buffers 0 and 1 of the prefill tile,
// each also one wave's combine table), each the larger of a staged half (4 pages per buffer when
// a (page, head) slab of the tile's element type is at most 4 KiB, else 2) and a combine table.
// lds_elem_bytes is the tile's element size in LDS: 4 for fp32, 2 for bf16 and for the FP8
// cache (its codes are converted to bf16 when staged).  The kernels' geometry uses the same
// formula.
constexpr int fused_lds_bytes(int lds_elem_bytes, int d) {
  const int slab = kPage * d * lds_elem_bytes;
  const int half = (slab <= 4096 ? 4 : 2) * slab;
  return 4 * (half > kCombineLdsPerWave ? half : kCombineLdsPerWave);
}

// Workspace map (byte offsets), computed by the planner.
struct WorkspaceMap {
  size_t ctrl, tickets, claims, pdesc, pitems, ddesc, aunits, copy_bytes;  // [0, pdesc) zeroed, [pdesc, copy_bytes) staged from the host
  size_t part_o, part_lse, trace, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace pod

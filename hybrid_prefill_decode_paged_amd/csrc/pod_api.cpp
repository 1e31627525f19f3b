// C ABI of the hybrid-batch attention library: handle, planning, staging of the plan into the
// caller's workspace, and the three launch modes (fused, separate, two streams) that the
// Silicon & Systems digest "POD-Attention hybrid batching" compares (sections "Why
// concurrency alone is not enough" and "Reproduction and hardware evaluation"), with the
// diagnostics its section "Predictable latency and diagnostics" asks a runtime to expose.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/pod_attn.h"
#include "kernels.h"
#include "plan.h"

using namespace pod;

namespace {
thread_local std::string g_err;

pod_attn_status fail(pod_attn_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define POD_HIP(x)                                                                      \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) return fail(POD_ATTN_ERR_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

bool log_on() { return env_int("POD_ATTN_LOG", 0) != 0; }

struct StagingSlot {
  void* host = nullptr;            // pinned, fine-grained (read by the upload kernel over the host link)
  void* dev = nullptr;             // its device address
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};
constexpr int kRing = 4;
// Pinned staging bytes each ring slot gets at handle creation: plans of the measured workloads
// stage a few to ~70 KiB.  pod_attn_run grows a slot for a larger plan; pod_attn_run_noalloc,
// which allocates nothing, rejects such a plan instead.
constexpr size_t kStagingPrealloc = (size_t)256 << 10;

// Kernel-time record of one run: events around its attention kernels and its algorithmic work.
struct TimingSlot {
  hipEvent_t start = nullptr, end = nullptr;
  bool armed = false;
  uint64_t run = 0;
  double bytes = 0.0, flops = 0.0;
};
}  // namespace

struct pod_attn_handle {
  Config cfg;
  int device = 0;
  int num_cus = 0;
  int wgs_per_cu = 0;
  int fused_occupancy = 0;
  int fused_vgprs = 0;
  KernelSet ks;
  hipStream_t sA = nullptr, sB = nullptr;
  hipEvent_t evStart = nullptr, evA = nullptr, evB = nullptr;
  StagingSlot ring[kRing];
  int ring_next = 0;
  pod_attn_stats stats{};
  Plan last_plan;
  int mode_env = -1;
  hipEvent_t prof_start = nullptr, prof_end = nullptr;   // one-shot profiling events
  TimingSlot timing[kRing];         // kernel time of the last runs (one slot per run, round robin)
  int timing_next = 0;
  void* scratch = nullptr;          // pod_attn_run_noalloc's device scratch on this handle's device
};

extern "C" {

const char* pod_attn_last_error(void) { return g_err.c_str(); }

pod_attn_status pod_attn_create(const pod_attn_config* cfg, pod_attn_handle** out) {
  if (!out) return fail(POD_ATTN_ERR_INVALID_ARG, "null output handle pointer");
  *out = nullptr;
  Config c;
  std::string err;
  pod_attn_status st = validate_config(cfg, &c, &err);
  if (st != POD_ATTN_OK) return fail(st, err);

  int dev = 0, ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(POD_ATTN_ERR_NO_DEVICE, "no HIP device");
  POD_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  POD_HIP(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(POD_ATTN_ERR_NO_DEVICE, std::string("device is ") + prop.gcnArchName + ", built for gfx950");

  pod_attn_handle* h = new pod_attn_handle();
  h->cfg = c;
  h->device = dev;
  h->num_cus = prop.multiProcessorCount;
  h->ks = kernel_set(c.dtype, c.d);

  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, h->ks.fused, kThreads, 0) != hipSuccess) occ = 0;
  h->fused_occupancy = occ;
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, h->ks.fused) == hipSuccess) h->fused_vgprs = fa.numRegs;
  int w = c.wgs_per_cu > 0 ? c.wgs_per_cu : env_int("POD_ATTN_WGS_PER_CU", 0);
  if (w <= 0) w = std::min(occ, 2);
  h->wgs_per_cu = std::max(1, std::min(w, std::max(1, occ)));
  if (c.decode_split_tokens == 0) h->cfg.decode_split_tokens = env_int("POD_ATTN_DECODE_SPLIT_TOKENS", 0) / 128 * 128;
  if (c.prefill_split_cap == 0) h->cfg.prefill_split_cap = std::max(0, env_int("POD_ATTN_PREFILL_SPLIT_CAP", 0));
  h->cfg.append_token_heads = std::max(1, env_int("POD_ATTN_APPEND_TOKEN_HEADS", kAppendTokenHeads));
  h->cfg.decode_taper = env_int("POD_ATTN_DECODE_TAPER", h->cfg.decode_taper);
  h->cfg.decode_items_per_wave = std::max(0, env_int("POD_ATTN_DECODE_ITEMS_PER_WAVE", h->cfg.decode_items_per_wave));
  if (const char* m = std::getenv("POD_ATTN_MODE")) {
    if (!std::strcmp(m, "fused")) h->mode_env = POD_ATTN_MODE_FUSED;
    else if (!std::strcmp(m, "separate")) h->mode_env = POD_ATTN_MODE_SEPARATE;
    else if (!std::strcmp(m, "streams")) h->mode_env = POD_ATTN_MODE_STREAMS;
  }

  hipError_t e = hipSuccess;
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->sA, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->sB, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->evStart, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->evA, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->evB, hipEventDisableTiming);
  for (int i = 0; i < kRing && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&h->ring[i].done, hipEventDisableTiming);
  for (int i = 0; i < kRing && e == hipSuccess; ++i) {
    e = hipEventCreate(&h->timing[i].start);
    if (e == hipSuccess) e = hipEventCreate(&h->timing[i].end);
  }
  for (int i = 0; i < kRing && e == hipSuccess; ++i) {
    e = hipHostMalloc(&h->ring[i].host, kStagingPrealloc, hipHostMallocCoherent | hipHostMallocMapped);
    if (e == hipSuccess) e = hipHostGetDevicePointer(&h->ring[i].dev, h->ring[i].host, 0);
    if (e == hipSuccess) h->ring[i].cap = kStagingPrealloc;
  }
  if (e == hipSuccess) e = noalloc_scratch(dev, &h->scratch);
  if (e != hipSuccess) {
    pod_attn_destroy(h);
    return fail(POD_ATTN_ERR_HIP, std::string("stream/event/staging/scratch set-up: ") + hipGetErrorString(e));
  }
  h->stats.num_cus = h->num_cus;
  h->stats.wgs_per_cu = h->wgs_per_cu;
  h->stats.lds_bytes_per_wg = h->ks.fused_lds;
  h->stats.vgprs_per_lane = h->fused_vgprs;
  h->stats.prefill_kv_tile = h->ks.prefill_kv_tile;
  if (log_on())
    std::fprintf(stderr, "[pod_attn] create: Hq=%d Hkv=%d D=%d dtype=%d mode=%d cus=%d occ=%d wgs/cu=%d vgprs=%d lds=%d\n",
                 c.hq, c.hkv, c.d, c.dtype, c.mode, h->num_cus, occ, h->wgs_per_cu, h->fused_vgprs, h->ks.fused_lds);
  *out = h;
  return POD_ATTN_OK;
}

void pod_attn_destroy(pod_attn_handle* h) {
  if (!h) return;
  for (int i = 0; i < kRing; ++i) {
    if (h->ring[i].done) {
      if (h->ring[i].pending) (void)hipEventSynchronize(h->ring[i].done);
      (void)hipEventDestroy(h->ring[i].done);
    }
    if (h->ring[i].host) (void)hipHostFree(h->ring[i].host);
  }
  for (int i = 0; i < kRing; ++i) {
    if (h->timing[i].start) (void)hipEventDestroy(h->timing[i].start);
    if (h->timing[i].end) (void)hipEventDestroy(h->timing[i].end);
  }
  if (h->evStart) (void)hipEventDestroy(h->evStart);
  if (h->evA) (void)hipEventDestroy(h->evA);
  if (h->evB) (void)hipEventDestroy(h->evB);
  if (h->sA) (void)hipStreamDestroy(h->sA);
  if (h->sB) (void)hipStreamDestroy(h->sB);
  delete h;
}

// The configuration a batch is planned with: the handle's, in the mode its runs will launch
// (POD_ATTN_MODE, and separate kernels when the fused kernel cannot be resident), so that
// pod_attn_workspace_size and pod_attn_run plan alike.
static Config planning_config(const pod_attn_handle* h) {
  Config c = h->cfg;
  if (h->mode_env >= 0) c.mode = h->mode_env;
  if (c.mode == POD_ATTN_MODE_FUSED && h->fused_occupancy < 1) c.mode = POD_ATTN_MODE_SEPARATE;
  return c;
}

pod_attn_status pod_attn_workspace_size(pod_attn_handle* h, const pod_attn_batch* b, size_t* bytes) {
  if (!h || !bytes) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle or output");
  Plan p;
  std::string err;
  pod_attn_status st = plan_batch(planning_config(h), b, h->num_cus, h->wgs_per_cu, &p, &err);
  if (st != POD_ATTN_OK) return fail(st, err);
  *bytes = p.map.total;
  return POD_ATTN_OK;
}

static hipError_t launch(const void* fn, int grid, KernelParams& p, hipStream_t s) {
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

// Combine groups [g0, g1), whose groups have at most max_cols columns: one workgroup per
// (group, 16 columns).
static hipError_t launch_combine(pod_attn_handle* h, const KernelParams& base, int g0, int g1, int max_cols,
                                 hipStream_t s) {
  KernelParams c = base;
  c.group_begin = g0;
  c.group_end = g1;
  c.combine_col_blocks = (max_cols + 15) / 16;
  return launch(h->ks.combine, (g1 - g0) * c.combine_col_blocks, c, s);
}

// One run: plan, stage the plan, then (with k_new / v_new) the KV append and the attention
// launches of the chosen mode.
static pod_attn_status run_impl(pod_attn_handle* h, const void* q, const void* k_new, const void* v_new,
                                const void* k_cache, const void* v_cache, const float* k_scale,
                                const float* v_scale, const int32_t* block_tables, const pod_attn_batch* b,
                                void* out, void* workspace, size_t workspace_bytes, void* stream_,
                                bool noalloc = false) {
  if (!h) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle");
  if (noalloc) {
    workspace = h->scratch;
    workspace_bytes = kNoAllocScratchBytes;
  }
  const bool append = k_new != nullptr;
  const bool fp8 = h->cfg.dtype == POD_ATTN_FP8_E4M3;
  if (fp8 && append) return fail(POD_ATTN_ERR_UNSUPPORTED, "the KV append does not write an FP8 cache");
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr))
    return fail(POD_ATTN_ERR_INVALID_ARG, fp8 ? "an FP8_E4M3 cache needs k_scale and v_scale (pod_attn_run_scaled)"
                                              : "scales are only taken by FP8_E4M3 handles");
  if (((uintptr_t)k_scale | (uintptr_t)v_scale) & 3) return fail(POD_ATTN_ERR_INVALID_ARG, "scales must be 4-byte aligned");
  hipStream_t stream = (hipStream_t)stream_;
  const auto t0 = std::chrono::steady_clock::now();
  Plan p;
  std::string err;
  pod_attn_status st = plan_batch(planning_config(h), b, h->num_cus, h->wgs_per_cu, &p, &err);
  if (st != POD_ATTN_OK) return fail(st, err);
  const double plan_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
  if (p.total_q == 0) return POD_ATTN_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !out)
    return fail(POD_ATTN_ERR_INVALID_ARG, "null device buffer (q, k_cache, v_cache, block_tables or out)");
  if (!workspace) return fail(POD_ATTN_ERR_WORKSPACE, "null workspace");
  if (workspace_bytes < p.map.total)
    return fail(POD_ATTN_ERR_WORKSPACE, noalloc ? "the batch needs " + std::to_string(p.map.total) +
                                                      " workspace bytes; pod_attn_run_noalloc's scratch holds " +
                                                      std::to_string(kNoAllocScratchBytes)
                                                : "workspace has " + std::to_string(workspace_bytes) +
                                                      " bytes, needs " + std::to_string(p.map.total));
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out | (uintptr_t)workspace |
       (uintptr_t)k_new | (uintptr_t)v_new) & 15)
    return fail(POD_ATTN_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");

  // mode
  const int requested = h->mode_env >= 0 ? h->mode_env : h->cfg.mode;
  int mode = requested;
  int reason = h->mode_env >= 0 && h->mode_env != h->cfg.mode ? POD_ATTN_FALLBACK_ENV : POD_ATTN_FALLBACK_NONE;
  if (mode == POD_ATTN_MODE_FUSED) {
    if (h->fused_occupancy < 1) {
      mode = POD_ATTN_MODE_SEPARATE;
      reason = POD_ATTN_FALLBACK_OCCUPANCY;
    } else if (p.n_pf_items == 0) {
      reason = POD_ATTN_FALLBACK_NO_PREFILL;
    } else if (p.n_dc_items == 0) {
      reason = POD_ATTN_FALLBACK_NO_DECODE;
    }
  }

  // stage the plan through a pinned ring: the upload kernel zero-fills the counters and copies the
  // descriptors in (slot i is rewritten only after its upload kernel has run)
  StagingSlot& slot = h->ring[h->ring_next];
  h->ring_next = (h->ring_next + 1) % kRing;
  if (slot.pending) {
    POD_HIP(hipEventSynchronize(slot.done));
    slot.pending = false;
  }
  const size_t staged = (append ? p.map.copy_bytes : p.map.aunits) - p.map.pdesc;   // units only when appending
  if (noalloc && slot.cap < staged)
    return fail(POD_ATTN_ERR_WORKSPACE, "the plan stages " + std::to_string(staged) +
                                            " bytes; pod_attn_run_noalloc's staging slots hold " + std::to_string(slot.cap));
  if (slot.cap < staged) {
    if (slot.host) POD_HIP(hipHostFree(slot.host));
    slot.host = slot.dev = nullptr;
    slot.cap = 0;
    size_t cap = std::max<size_t>(staged * 2, 1 << 16);
    POD_HIP(hipHostMalloc(&slot.host, cap, hipHostMallocCoherent | hipHostMallocMapped));
    POD_HIP(hipHostGetDevicePointer(&slot.dev, slot.host, 0));
    slot.cap = cap;
  }
  uint8_t* ws = (uint8_t*)workspace;
  KernelParams kp{};
  kp.q = q; kp.k = k_cache; kp.v = v_cache; kp.bt = block_tables; kp.out = out;
  kp.ctrl = (int32_t*)(ws + p.map.ctrl);
  kp.tickets = (int32_t*)(ws + p.map.tickets);
  kp.claims = (h->cfg.flags & POD_ATTN_FLAG_DEBUG_CLAIMS) ? (int32_t*)(ws + p.map.claims) : nullptr;
  kp.trace = (h->cfg.flags & POD_ATTN_FLAG_TRACE) ? (uint32_t*)(ws + p.map.trace) : nullptr;
  kp.pdesc = (const int32_t*)(ws + p.map.pdesc);
  kp.pitems = (const int32_t*)(ws + p.map.pitems);
  kp.ddesc = (const int32_t*)(ws + p.map.ddesc);
  kp.part_o = (float*)(ws + p.map.part_o);
  kp.part_lse = (float*)(ws + p.map.part_lse);
  kp.k_new = k_new; kp.v_new = v_new;
  kp.k_scale = k_scale; kp.v_scale = v_scale;
  kp.aunits = (const int32_t*)(ws + p.map.aunits);
  kp.n_aunits = append ? p.n_aunits : 0;
  kp.n_pdesc = p.n_pdesc; kp.n_ddesc = p.n_ddesc;
  kp.n_pf_items = p.n_pf_items; kp.n_dc_items = p.n_dc_items;
  kp.n_pf_groups = p.n_pf_groups; kp.n_groups = p.n_groups;
  kp.hq = h->cfg.hq; kp.hkv = h->cfg.hkv; kp.group = h->cfg.group();
  kp.bt_stride = b->block_table_stride; kp.num_pages = b->num_pages_in_pool;
  kp.scale_log2 = h->cfg.scale * 1.4426950408889634f;

  // Plan upload (and, in fused mode, the KV append in the same launch).
  stage_plan(p, h->cfg, (uint8_t*)slot.host, append);
  {
    StageArgs a{};
    a.p = kp;
    a.src = slot.dev;
    a.dst = workspace;
    a.n_zero16 = (int)(p.map.pdesc / 16);
    a.n_copy16 = (int)(staged / 16);
    a.copy_wgs = (a.n_zero16 + a.n_copy16 + kThreads - 1) / kThreads;
    const bool fused_append = kp.n_aunits > 0 && mode == POD_ATTN_MODE_FUSED;
    if (!fused_append) a.p.n_aunits = 0;
    a.units_host = fused_append ? (const int32_t*)((const uint8_t*)slot.dev + (p.map.aunits - p.map.pdesc)) : nullptr;
    const int grid = a.copy_wgs + (a.p.n_aunits + kWaves - 1) / kWaves;
    void* args[] = {&a};
    POD_HIP(hipLaunchKernel(h->ks.stage, dim3(grid), dim3(kThreads), args, 0, stream));
  }
  POD_HIP(hipEventRecord(slot.done, stream));
  slot.pending = true;

  hipEvent_t prof_start = h->prof_start, prof_end = h->prof_end;
  h->prof_start = h->prof_end = nullptr;
  if (prof_start) POD_HIP(hipEventRecord(prof_start, stream));
  // Kernel time of this run, for the diagnostics: events around the attention kernels (the same
  // span the profiling hook brackets), kept with the run's algorithmic work.
  TimingSlot& tslot = h->timing[h->timing_next];
  h->timing_next = (h->timing_next + 1) % kRing;
  tslot.armed = false;
  POD_HIP(hipEventRecord(tslot.start, stream));
  int grid = 0;
  if (mode == POD_ATTN_MODE_FUSED) {
    kp.inline_combine = 1;                    // split groups merge in-kernel (last arriver)
    grid = h->num_cus * h->wgs_per_cu;
    POD_HIP(launch(h->ks.fused, grid, kp, stream));
  } else if (mode == POD_ATTN_MODE_SEPARATE) {
    kp.inline_combine = 0;
    if (kp.n_aunits) POD_HIP(launch(h->ks.append, (kp.n_aunits + kWaves - 1) / kWaves, kp, stream));
    if (p.n_pf_items) POD_HIP(launch(h->ks.prefill, p.n_pf_items, kp, stream));
    if (p.n_dc_items) POD_HIP(launch(h->ks.decode, (p.n_dc_items + kWaves - 1) / kWaves, kp, stream));
    if (p.n_pf_groups) POD_HIP(launch_combine(h, kp, 0, p.n_pf_groups, p.tile_cols, stream));
    if (p.n_groups > p.n_pf_groups) POD_HIP(launch_combine(h, kp, p.n_pf_groups, p.n_groups, p.decode_max_cols, stream));
  } else {
    kp.inline_combine = 0;
    if (kp.n_aunits) POD_HIP(launch(h->ks.append, (kp.n_aunits + kWaves - 1) / kWaves, kp, stream));
    POD_HIP(hipEventRecord(h->evStart, stream));
    POD_HIP(hipStreamWaitEvent(h->sA, h->evStart, 0));
    POD_HIP(hipStreamWaitEvent(h->sB, h->evStart, 0));
    if (p.n_pf_items) POD_HIP(launch(h->ks.prefill, p.n_pf_items, kp, h->sA));
    if (p.n_pf_groups) POD_HIP(launch_combine(h, kp, 0, p.n_pf_groups, p.tile_cols, h->sA));
    if (p.n_dc_items) POD_HIP(launch(h->ks.decode, (p.n_dc_items + kWaves - 1) / kWaves, kp, h->sB));
    if (p.n_groups > p.n_pf_groups) POD_HIP(launch_combine(h, kp, p.n_pf_groups, p.n_groups, p.decode_max_cols, h->sB));
    POD_HIP(hipEventRecord(h->evA, h->sA));
    POD_HIP(hipEventRecord(h->evB, h->sB));
    POD_HIP(hipStreamWaitEvent(stream, h->evA, 0));
    POD_HIP(hipStreamWaitEvent(stream, h->evB, 0));
  }
  if (prof_end) POD_HIP(hipEventRecord(prof_end, stream));
  POD_HIP(hipEventRecord(tslot.end, stream));

  pod_attn_stats& s = h->stats;
  s.runs += 1;
  if (mode == POD_ATTN_MODE_FUSED && reason == POD_ATTN_FALLBACK_NONE) s.runs_fused_path += 1;
  if (reason >= 0 && reason < POD_ATTN_NUM_FALLBACK_REASONS) s.fallback_runs[reason] += 1;
  s.algorithmic_bytes = p.prefill_bytes + p.decode_bytes;
  s.algorithmic_flops = p.prefill_flops + p.decode_flops;
  tslot.armed = true;
  tslot.run = s.runs;
  tslot.bytes = s.algorithmic_bytes;
  tslot.flops = s.algorithmic_flops;
  s.mode_requested = requested;
  s.mode_used = mode;
  s.fallback_reason = reason;
  s.num_prefill_items = p.n_pf_items;
  s.num_decode_items = p.n_dc_items;
  s.num_combine_groups = p.n_groups;
  s.prefill_tile_cols = p.tile_cols;
  s.prefill_tile_queries = p.tile_queries;
  s.prefill_max_splits = p.prefill_max_splits;
  s.decode_split_tokens = p.decode_split_tokens;
  s.decode_max_splits = p.decode_max_splits;
  s.grid_wgs = grid;
  s.prefill_wg_budget = mode == POD_ATTN_MODE_FUSED ? h->num_cus * kPrefillPerCu : 0;
  s.workspace_bytes = p.map.total;
  s.host_plan_us = plan_us;
  s.num_append_units = kp.n_aunits;
  s.num_small_extends = p.num_small_extends;
  if (log_on())
    std::fprintf(stderr, "[pod_attn] run: mode=%d reason=%d pf_items=%d dc_items=%d groups=%d split=%d grid=%d plan=%.1fus\n",
                 mode, reason, p.n_pf_items, p.n_dc_items, p.n_groups, p.decode_split_tokens, grid, plan_us);
  h->last_plan = std::move(p);
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_run(pod_attn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const pod_attn_batch* b, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return run_impl(h, q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_tables, b, out, workspace,
                  workspace_bytes, stream);
}

pod_attn_status pod_attn_run_noalloc(pod_attn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const pod_attn_batch* b, void* out, void* stream) {
  return run_impl(h, q, nullptr, nullptr, k_cache, v_cache, nullptr, nullptr, block_tables, b, out, nullptr, 0,
                  stream, true);
}

pod_attn_status pod_attn_run_scaled(pod_attn_handle* h, const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale, const int32_t* block_tables,
                                    const pod_attn_batch* b, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!k_scale || !v_scale) return fail(POD_ATTN_ERR_INVALID_ARG, "null k_scale or v_scale");
  return run_impl(h, q, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale, block_tables, b, out, workspace,
                  workspace_bytes, stream);
}

pod_attn_status pod_attn_run_append(pod_attn_handle* h, const void* q, const void* k_new, const void* v_new,
                                    void* k_cache, void* v_cache, const int32_t* block_tables,
                                    const pod_attn_batch* b, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!k_new || !v_new) return fail(POD_ATTN_ERR_INVALID_ARG, "null k_new or v_new");
  return run_impl(h, q, k_new, v_new, k_cache, v_cache, nullptr, nullptr, block_tables, b, out, workspace,
                  workspace_bytes, stream);
}

pod_attn_status pod_attn_set_kernel_events(pod_attn_handle* h, void* ev_start, void* ev_end) {
  if (!h) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle");
  h->prof_start = (hipEvent_t)ev_start;
  h->prof_end = (hipEvent_t)ev_end;
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(POD_ATTN_ERR_INVALID_ARG, "null buffer or sink");
  if (bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0)
    return fail(POD_ATTN_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and buf 16-byte aligned");
  const ProbeKernels pk = probe_kernels();
  size_t n16 = bytes / 16;
  void* args[] = {(void*)&buf, &n16, (void*)&sink};
  POD_HIP(hipLaunchKernel(pk.hbm_read, dim3(kProbeWgs), dim3(kThreads), args, 0, (hipStream_t)stream));
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_probe_mfma(int iters, float* sink, double* flops, void* stream) {
  if (!sink) return fail(POD_ATTN_ERR_INVALID_ARG, "null sink");
  if (iters < 1 || iters > (1 << 20)) return fail(POD_ATTN_ERR_INVALID_ARG, "iters must be in [1, 2^20]");
  const ProbeKernels pk = probe_kernels();
  void* args[] = {&iters, (void*)&sink};
  POD_HIP(hipLaunchKernel(pk.mfma, dim3(kProbeWgs), dim3(kThreads), args, 0, (hipStream_t)stream));
  if (flops) *flops = (double)kProbeWgs * kWaves * kProbeChains * (double)iters * (2.0 * 32 * 32 * 16);
  return POD_ATTN_OK;
}

// Kernel time of the newest run whose attention kernels have completed (non-blocking).
static void fill_timing(pod_attn_handle* h, pod_attn_stats* st) {
  st->timed_run = 0;
  st->kernel_us = -1.0;
  st->achieved_gbps = st->achieved_tflops = -1.0;
  const TimingSlot* best = nullptr;
  for (const TimingSlot& t : h->timing) {
    if (!t.armed || (best && t.run <= best->run)) continue;
    if (hipEventQuery(t.end) != hipSuccess) continue;
    best = &t;
  }
  float ms = 0.f;
  if (!best || hipEventElapsedTime(&ms, best->start, best->end) != hipSuccess || ms <= 0.f) return;
  st->timed_run = best->run;
  st->kernel_us = ms * 1e3;
  st->achieved_gbps = best->bytes / (ms * 1e-3) / 1e9;
  st->achieved_tflops = best->flops / (ms * 1e-3) / 1e12;
}

pod_attn_status pod_attn_get_stats(pod_attn_handle* h, pod_attn_stats* st) {
  if (!h || !st) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle or stats");
  *st = h->stats;
  fill_timing(h, st);
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_gather_kv(pod_attn_handle* h, const void* cache, int which, const int32_t* block_tables,
                                   int seq, int ctx, const pod_attn_batch* b, void* out_contig,
                                   int32_t* device_status, void* stream) {
  if (!h || !cache || !block_tables || !b || !out_contig) return fail(POD_ATTN_ERR_INVALID_ARG, "null argument");
  const bool fp8 = h->cfg.dtype == POD_ATTN_FP8_E4M3;
  if (!(which == 0 || which == 1 || (fp8 && (which == 2 || which == 3))))
    return fail(POD_ATTN_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V), or 2 / 3 (decoded, FP8_E4M3 handles)");
  if (seq < 0 || seq >= b->num_prefill + b->num_decode) return fail(POD_ATTN_ERR_INVALID_ARG, "seq out of range");
  if (ctx < 1 || (long)ctx > (long)b->block_table_stride * kPage) return fail(POD_ATTN_ERR_INVALID_ARG, "ctx out of range");
  const size_t total = (size_t)ctx * h->cfg.hkv * h->cfg.d;
  const int grid = (int)((total + kThreads - 1) / kThreads);
  const int32_t* row = block_tables + (size_t)seq * b->block_table_stride;
  int hkv = h->cfg.hkv, np = b->num_pages_in_pool;
  int32_t* status = device_status;
  if (((uintptr_t)status & 3) != 0) return fail(POD_ATTN_ERR_INVALID_ARG, "device_status must be 4-byte aligned");
  void* args[] = {(void*)&cache, &which, (void*)&row, &ctx, &hkv, &np, &out_contig, (void*)&status};
  POD_HIP(hipLaunchKernel(h->ks.gather, dim3(grid), dim3(kThreads), args, 0, (hipStream_t)stream));
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_read_device_status(pod_attn_handle* h, const void* workspace, void* stream,
                                            int32_t* status_word, int32_t* claims, int claims_cap, int* n_items,
                                            int32_t* pf_cu, int32_t* dc_cu, int cu_cap) {
  if (!h || !workspace) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle or workspace");
  POD_HIP(hipStreamSynchronize((hipStream_t)stream));
  const uint8_t* ws = (const uint8_t*)workspace;
  const Plan& p = h->last_plan;
  if (status_word) POD_HIP(hipMemcpy(status_word, ws + p.map.ctrl + 4 * kCStatus, 4, hipMemcpyDeviceToHost));
  const int n = p.n_pf_items + p.n_dc_items;
  if (n_items) *n_items = n;
  if (claims && claims_cap > 0 && (h->cfg.flags & POD_ATTN_FLAG_DEBUG_CLAIMS))
    POD_HIP(hipMemcpy(claims, ws + p.map.claims, 4 * (size_t)std::min(n, claims_cap), hipMemcpyDeviceToHost));
  const int m = std::min(cu_cap, (int)kCuSlots);
  if (pf_cu && m > 0) POD_HIP(hipMemcpy(pf_cu, ws + p.map.ctrl + 4 * kCClaimsPrefillCu, 4 * (size_t)m, hipMemcpyDeviceToHost));
  if (dc_cu && m > 0) POD_HIP(hipMemcpy(dc_cu, ws + p.map.ctrl + 4 * kCClaimsDecodeCu, 4 * (size_t)m, hipMemcpyDeviceToHost));
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_read_run_diagnostics(pod_attn_handle* h, const void* workspace, void* stream,
                                              pod_attn_run_diag* d) {
  if (!h || !workspace || !d) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle, workspace or output");
  POD_HIP(hipStreamSynchronize((hipStream_t)stream));
  const uint8_t* ws = (const uint8_t*)workspace;
  const Plan& p = h->last_plan;
  std::vector<int32_t> pf(kCuSlots), dc(kCuSlots);
  int32_t status = 0;
  POD_HIP(hipMemcpy(&status, ws + p.map.ctrl + 4 * kCStatus, 4, hipMemcpyDeviceToHost));
  POD_HIP(hipMemcpy(pf.data(), ws + p.map.ctrl + 4 * kCClaimsPrefillCu, 4 * (size_t)kCuSlots, hipMemcpyDeviceToHost));
  POD_HIP(hipMemcpy(dc.data(), ws + p.map.ctrl + 4 * kCClaimsDecodeCu, 4 * (size_t)kCuSlots, hipMemcpyDeviceToHost));
  pod_attn_run_diag r{};
  r.status_word = status;
  r.planned_prefill_items = p.n_pf_items;
  r.planned_decode_items = p.n_dc_items;
  r.min_prefill_share = 1.0;
  double share_sum = 0.0;
  int cus_any = 0;
  for (int i = 0; i < kCuSlots; ++i) {
    const int a = pf[i], b = dc[i];
    r.prefill_items += a;
    r.decode_items += b;
    r.cus_prefill += a > 0;
    r.cus_decode += b > 0;
    r.cus_both += a > 0 && b > 0;
    r.max_prefill_per_cu = std::max(r.max_prefill_per_cu, a);
    r.max_decode_per_cu = std::max(r.max_decode_per_cu, b);
    if (a + b > 0) {
      const double sh = (double)a / (a + b);
      share_sum += sh;
      r.min_prefill_share = std::min(r.min_prefill_share, sh);
      r.max_prefill_share = std::max(r.max_prefill_share, sh);
      ++cus_any;
    }
  }
  r.cus_any = cus_any;
  r.mean_prefill_share = cus_any ? share_sum / cus_any : 0.0;
  if (!cus_any) r.min_prefill_share = 0.0;
  r.prefill_decode_ratio = r.decode_items > 0 ? (double)r.prefill_items / r.decode_items : 0.0;
  pod_attn_stats st = h->stats;
  fill_timing(h, &st);
  r.run = st.runs;
  r.timed_run = st.timed_run;
  r.kernel_us = st.kernel_us;
  r.achieved_gbps = st.achieved_gbps;
  r.achieved_tflops = st.achieved_tflops;
  *d = r;
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_read_trace(pod_attn_handle* h, const void* workspace, void* stream, uint32_t* records,
                                    int cap, int* n_items) {
  if (!h || !workspace) return fail(POD_ATTN_ERR_INVALID_ARG, "null handle or workspace");
  if (!(h->cfg.flags & POD_ATTN_FLAG_TRACE)) return fail(POD_ATTN_ERR_INVALID_ARG, "handle was created without POD_ATTN_FLAG_TRACE");
  POD_HIP(hipStreamSynchronize((hipStream_t)stream));
  const Plan& p = h->last_plan;
  const int n = p.n_pf_items + p.n_dc_items;
  if (n_items) *n_items = n;
  if (records && cap > 0)
    POD_HIP(hipMemcpy(records, (const uint8_t*)workspace + p.map.trace, 16 * (size_t)std::min(n, cap), hipMemcpyDeviceToHost));
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_plan_inspect(const pod_attn_config* cfg, const pod_attn_batch* b, int num_cus, int wgs_per_cu,
                                      int32_t* items, int items_cap, int* n_items, pod_attn_stats* stats) {
  Config c;
  std::string err;
  pod_attn_status st = validate_config(cfg, &c, &err);
  if (st != POD_ATTN_OK) return fail(st, err);
  Plan p;
  st = plan_batch(c, b, num_cus, wgs_per_cu, &p, &err);
  if (st != POD_ATTN_OK) return fail(st, err);
  std::vector<int32_t> all;
  expand_items(p, c, &all);
  const int n = (int)(all.size() / 16);
  if (n_items) *n_items = n;
  if (items && items_cap > 0) std::memcpy(items, all.data(), 4 * 16 * (size_t)std::min(n, items_cap));
  if (stats) {
    pod_attn_stats s{};
    s.mode_requested = c.mode;
    s.mode_used = c.mode;
    s.num_prefill_items = p.n_pf_items;
    s.num_decode_items = p.n_dc_items;
    s.num_combine_groups = p.n_groups;
    s.prefill_tile_cols = p.tile_cols;
    s.prefill_tile_queries = p.tile_queries;
    s.prefill_max_splits = p.prefill_max_splits;
    s.decode_split_tokens = p.decode_split_tokens;
    s.decode_max_splits = p.decode_max_splits;
    s.num_cus = num_cus;
    s.wgs_per_cu = wgs_per_cu;
    s.num_small_extends = p.num_small_extends;
    s.workspace_bytes = p.map.total;
    *stats = s;
  }
  return POD_ATTN_OK;
}

pod_attn_status pod_attn_batch_signals(const pod_attn_config* cfg, const pod_attn_batch* b, int num_cus, int wgs_per_cu,
                                       double peak_gbps, double peak_tflops, pod_attn_signals* out) {
  if (!out) return fail(POD_ATTN_ERR_INVALID_ARG, "null output");
  Config c;
  std::string err;
  pod_attn_status st = validate_config(cfg, &c, &err);
  if (st != POD_ATTN_OK) return fail(st, err);
  Plan p;
  st = plan_batch(c, b, num_cus, wgs_per_cu, &p, &err);
  if (st != POD_ATTN_OK) return fail(st, err);
  if (peak_gbps <= 0.0) peak_gbps = 8000.0;
  if (peak_tflops <= 0.0) peak_tflops = c.dtype == POD_ATTN_FP32 ? 157.3 : 2500.0;   // FP8 cache: bf16 products
  pod_attn_signals s{};
  s.prefill_items = p.n_pf_items;
  s.decode_items = p.n_dc_items;
  s.combine_groups = p.n_groups;
  s.small_extends = p.num_small_extends;
  s.grid_wgs = num_cus * wgs_per_cu;
  s.lds_bytes_per_wg = fused_lds_bytes(c.lds_elem_bytes(), c.d);
  s.fallback_reason = p.n_pf_items == 0 ? POD_ATTN_FALLBACK_NO_PREFILL
                      : p.n_dc_items == 0 ? POD_ATTN_FALLBACK_NO_DECODE : POD_ATTN_FALLBACK_NONE;
  s.workspace_bytes = p.map.total;
  s.prefill_flops = p.prefill_flops;
  s.decode_flops = p.decode_flops;
  s.prefill_bytes = p.prefill_bytes;
  s.decode_bytes = p.decode_bytes;
  const double flops = p.prefill_flops + p.decode_flops, bytes = p.prefill_bytes + p.decode_bytes;
  s.intensity = bytes > 0.0 ? flops / bytes : 0.0;
  s.roofline_us = std::max(flops / (peak_tflops * 1e12), bytes / (peak_gbps * 1e9)) * 1e6;
  *out = s;
  return POD_ATTN_OK;
}

}  // extern "C"

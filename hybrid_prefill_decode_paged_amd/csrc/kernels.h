// Kernel entry points of one (dtype, head_dim) instantiation, as launchable function handles.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pod {

struct KernelSet {
  const void* fused = nullptr;     // persistent fused prefill + decode kernel (KernelParams)
  const void* prefill = nullptr;   // one workgroup per prefill item (KernelParams)
  const void* decode = nullptr;    // one workgroup per decode item (KernelParams)
  const void* combine = nullptr;   // one workgroup per combine group (KernelParams)
  const void* gather = nullptr;    // debug gather (cache, which, bt_row, ctx, hkv, num_pages, out, status)
  const void* stage = nullptr;     // plan upload, with the KV append in fused mode (StageArgs)
  const void* append = nullptr;    // KV append alone, one wave per unit (KernelParams)
  int fused_lds = 0;               // static LDS bytes of the fused kernel
  int prefill_kv_tile = 0;         // keys per prefill inner iteration
};

// dtype: 0 bf16, 1 fp32, 2 FP8 E4M3 cache with bf16 q/out; head_dim: 64 or 128.
KernelSet kernel_set(int dtype, int head_dim);

// Measurement probes (peaks on the machine at hand).
constexpr int kProbeWgs = 4096;    // workgroups of either probe
constexpr int kProbeChains = 8;    // independent 32x32x16 MFMA chains per wave
struct ProbeKernels {
  const void* hbm_read = nullptr;  // (const u32x4* buf, size_t n16, uint32_t* sink)
  const void* mfma = nullptr;      // (int iters, float* sink)
};
ProbeKernels probe_kernels();

// pod_attn_run_noalloc's device scratch: bytes per GPU, and its device address on `device`
// (which must be current), looked up on the first call per device and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)256 << 20;
hipError_t noalloc_scratch(int device, void** ptr);

}  // namespace pod

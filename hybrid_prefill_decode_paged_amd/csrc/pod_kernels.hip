// gfx950 (MI355X, CDNA4) kernels for fused hybrid-batch paged attention.
//
// Sources (web pages; sections as printed on them):
//   [POD] Silicon & Systems digest "POD-Attention hybrid batching"
//   [W6]  "Week 6: Beyond PyTorch: Custom Kernel과 vLLM"
//   [W4]  "LLMSO - W4 - Optimization & Frameworks"
//
// What every kernel computes is exact attention, softmax(scale * q K^T, causal by absolute
// position) V, over K/V read through block tables ([W6] "Attention에 적용하기",
// "Non-Causal vs. Causal Attention", "PagedAttention").  The kernels evaluate it with the
// online softmax: a running maximum m and running sum l per query column, the running output
// rescaled by exp(m_old - m_new) whenever the maximum grows, one division at the end ([W6]
// "FlashAttention의 single-pass 트릭"; [W4] "FlashAttention -- I/O를 줄이는 방향").  Key
// ranges that are split over several work items are merged by log-sum-exp ([W4]
// "FlashDecoding -- decode 단계의 병렬성 확보").  Exponentials are taken base 2 with
// log2(e) folded into the scale, which is the same function.
//
// Matrix layout on the MFMA units.  Both products run as 16x16 MFMA blocks with the keys on
// the M side and the (query, head) columns on the N side:
//   S^T[key][col]  = K[key][:] . Q[col][:]          (A = K rows, B = Q^T)
//   O^T[d][col]   += V^T[d][key] . P^T[key][col]     (A = V^T rows, B = P^T)
// so that the score block leaves the first MFMA in exactly the register layout the second one
// takes as its B operand (lane l holds column l%16 and keys 4*(l/16)+i), with no shuffles.
// The contraction index of an MFMA may be assigned to (lane group, register slot) in any way,
// as long as A and B agree; the KV page layout is chosen so that each lane's operand is one
// contiguous 16-byte (K) or 8-byte (V, bf16) load: K pages are [D/x][16][x] (16-byte chunks of
// x dims per token), V pages are [D][16] (tokens contiguous per dim).
//
// Decode items stream K/V straight from HBM into registers (no reuse, so no LDS staging), two
// pages per wave step with the next step's loads in flight; prefill tiles stage 64 keys of K
// and V in LDS (double-buffered) and share them across the four waves, each wave owning 32 of
// the tile's 128 query columns.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"
#include "pod_internal.h"

namespace pod {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define CPTR(T) const __attribute__((address_space(4))) T*

constexpr float kNegInf = -__builtin_huge_valf();

// Cache element types: bf16, fp32, or Fp8 -- OCP FP8 E4M3 codes with one float scale per
// (page, KV head) for K and one for V, q and out then being bf16.
struct Fp8 {};
template <typename T> struct ElemTraits;
template <> struct ElemTraits<__bf16> { static constexpr int kBytes = 2; };
template <> struct ElemTraits<float> { static constexpr int kBytes = 4; };
template <> struct ElemTraits<Fp8> { static constexpr int kBytes = 1; };
template <typename T> struct QOf { typedef T type; };       // q / out element type
template <> struct QOf<Fp8> { typedef __bf16 type; };
template <typename T> constexpr bool kIsFp8 = false;
template <> constexpr bool kIsFp8<Fp8> = true;

// Compile-time geometry of one (dtype, head_dim) instantiation.
template <typename T, int D> struct Geo {
  static constexpr int kBytes = ElemTraits<T>::kBytes;
  static constexpr int kEpc = 16 / kBytes;              // elements per 16-byte chunk
  static constexpr int kNch = D / kEpc;                 // 16-byte chunks per K row
  static constexpr int kNs = kIsFp8<T> ? D / 32 : kNch / 4;   // QK MFMA steps (bf16 MFMAs for Fp8)
  typedef typename QOf<T>::type QT;                     // q / out element
  static constexpr int kQBytes = sizeof(QT);
  typedef typename std::conditional<kIsFp8<T>, u32x2, u32x4>::type KReg;   // K operand as loaded, per step
  static constexpr int kSlab = kPage * D * kBytes;      // bytes of one (page, KV head) slab
  static constexpr int kCps = kSlab / 16;               // 16-byte chunks per slab
  // The prefill tile in LDS: FP8 codes are converted to bf16 when staged.
  static constexpr int kLdsBytes = kIsFp8<T> ? 2 : kBytes;
  static constexpr int kLdsSlab = kPage * D * kLdsBytes;                 // one staged (page, head)
  static constexpr int kTp = kLdsSlab <= 4096 ? 4 : 2;  // pages per prefill KV tile
  static constexpr int kTileKeys = kTp * kPage;
  static constexpr int kDb = D / 16;                    // 16-row blocks of O^T
  static constexpr int kStageChunks = 2 * kTp * kCps;   // K + V chunks of one prefill tile
  static constexpr int kStageR = kStageChunks / kThreads;
  static constexpr int kPrefillLds = 2 * 2 * kTp * kLdsSlab;           // 2 buffers x (K, V)
  // LDS is four separate objects: K and V staging buffers 0 and 1 of the prefill tile, each also
  // one wave's combine table.  Separate objects let the compiler's wait-count pass tell a read of
  // one buffer from the LDS-DMA loads in flight into another, so a tile's operand reads do not
  // wait for the next tile's staging loads.
  static constexpr int kObjBytes = kTp * kLdsSlab > kCombineLdsPerWave ? kTp * kLdsSlab : kCombineLdsPerWave;
  static constexpr int kFusedLds = 4 * kObjBytes;
  static_assert(kFusedLds == fused_lds_bytes(kLdsBytes, D), "host-side LDS figure matches the kernels");
  static_assert(kStageChunks % kThreads == 0, "tile must split evenly over the workgroup");
  static_assert(kTp % 2 == 0, "bf16 PV pairs pages");
};

// ------------------------------------------------------------------ page addressing
// One address generator for every reader of the paged cache (attention kernels and gather).
template <typename T, int D>
__device__ __forceinline__ const char* slab_ptr(const void* base, int page, int hkv, int g) {
  return (const char*)base + ((size_t)page * hkv + g) * Geo<T, D>::kSlab;
}
// byte offset, inside a K slab, of the 16-byte chunk c (dims c*x .. c*x+x-1) of token slot t
__device__ __forceinline__ int k_chunk_off(int c, int t) { return (c * kPage + t) * 16; }
// byte offset, inside a V slab, of dim d, token slot t
template <typename T>
__device__ __forceinline__ int v_elem_off(int d, int t) { return (d * kPage + t) * ElemTraits<T>::kBytes; }

// Reads block-table entry `pi` of row `btr` when the page holds keys (lim > 0); an entry
// outside the pool is never dereferenced: it is reported and its page counts as empty.
__device__ __forceinline__ int page_or_empty(CPTR(int32_t) btr, int pi, int& lim, int num_pages,
                                             int32_t* status) {
  int pg = 0;
  if (lim > 0) {
    pg = btr[pi];
    if ((unsigned)pg >= (unsigned)num_pages) {
      if ((threadIdx.x & 63) == 0) atomicOr(status, (int)kStatusBadPage);
      pg = 0;
      lim = 0;
    }
  } else {
    lim = 0;
  }
  return pg;
}

// ------------------------------------------------------------------ small primitives
__device__ __forceinline__ u32x4 ld16(const char* p) { return *(const u32x4*)p; }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// Streaming (nontemporal) load: decode reads every K/V byte exactly once, so its loads are
// marked not to be kept in the caches; measured 7-11% more HBM throughput on the decode share
// than ordinary loads.
template <typename V>
__device__ __forceinline__ V ld_stream(const char* p) { return __builtin_nontemporal_load((const V*)p); }

// Reductions over lanes l, l^16, l^32, l^48 with the gfx950 lane-swap instructions (VALU, no
// LDS round trip): v_permlane16_swap applied to (v, v) hands every lane the values of lanes
// l&~16 and l|16, i.e. its own and its partner's, in the same order on both partners, so the
// results are bit-identical across the four lanes.
__device__ __forceinline__ float max_over_groups(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));   // RNE
}

// One 16-byte chunk of contraction per lane: bf16 -> one 16x16x32 MFMA; fp32 -> four
// 16x16x4 MFMAs, element e of both chunks feeding the e-th.
__device__ __forceinline__ f32x4 mfma_chunk(u32x4 a, u32x4 b, f32x4 c, __bf16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_chunk(u32x4 a, u32x4 b, f32x4 c, float) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 mfma_chunk(u32x4 a, u32x4 b, f32x4 c, Fp8) {   // operands already bf16
  return mfma_chunk(a, b, c, __bf16());
}

// E4M3 -> bf16 for the Fp8 cache: gfx950 converts the two codes of a 16-bit half straight to
// a packed bf16 pair (OCP E4M3), here with a unit scale; every E4M3 value is exact in bf16, so
// nothing is rounded (NaN codes stay NaN).  Codes come lowest byte first.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t v) {
  const bf16x2v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
  const bf16x2v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(u32x2 v) {
  const u32x2 lo = e4m3x4_to_bf16(v.x), hi = e4m3x4_to_bf16(v.y);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}
// Eight E4M3 codes (lowest byte first) decoded exactly, times s, rounded to bf16 (nearest even):
// the values of an FP8 slab with its scale applied, as the bf16 tile takes them.
__device__ __forceinline__ uint32_t e4m3x2_scaled_bf16(uint32_t v, bool hi, float s) {
  const f32x2 x = hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v, 1.0f, false);
  return pack_bf16(x.x * s, x.y * s);
}
__device__ __forceinline__ u32x4 e4m3x8_scaled_bf16(u32x2 v, float s) {
  return u32x4{e4m3x2_scaled_bf16(v.x, false, s), e4m3x2_scaled_bf16(v.x, true, s),
               e4m3x2_scaled_bf16(v.y, false, s), e4m3x2_scaled_bf16(v.y, true, s)};
}
// The K operand of one MFMA step as the matrix unit takes it.
__device__ __forceinline__ u32x4 k_operand(u32x4 k) { return k; }
__device__ __forceinline__ u32x4 k_operand(u32x2 k) { return e4m3x8_to_bf16(k); }

// V^T operand of one page for one lane: 4 tokens (4q .. 4q+3) of dim d.
template <typename T> struct VOp;
template <> struct VOp<__bf16> { typedef u32x2 type; };
template <> struct VOp<float> { typedef u32x4 type; };
template <> struct VOp<Fp8> { typedef uint32_t type; };

// Zero the V^T elements of slots >= lim (tokens 4q .. 4q+3), so that 0 * (NaN in an unused
// slot) never enters the sum: masking selects, it does not multiply.
__device__ __forceinline__ u32x2 mask_vop(u32x2 v, int q, int lim) {
  const int t0 = 4 * q;
  uint32_t m0 = (t0 + 0 < lim ? 0x0000FFFFu : 0u) | (t0 + 1 < lim ? 0xFFFF0000u : 0u);
  uint32_t m1 = (t0 + 2 < lim ? 0x0000FFFFu : 0u) | (t0 + 3 < lim ? 0xFFFF0000u : 0u);
  return u32x2{v.x & m0, v.y & m1};
}
__device__ __forceinline__ u32x4 mask_vop(u32x4 v, int q, int lim) {
  const int t0 = 4 * q;
  return u32x4{t0 + 0 < lim ? v.x : 0u, t0 + 1 < lim ? v.y : 0u, t0 + 2 < lim ? v.z : 0u,
               t0 + 3 < lim ? v.w : 0u};
}

// PV for one pair of pages (bf16: one 16x16x32 MFMA; keys = 4 of each page per lane group).
__device__ __forceinline__ f32x4 pv_pair(u32x2 va, u32x2 vb, u32x4 pb, f32x4 c) {
  u32x4 a = {va.x, va.y, vb.x, vb.y};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, pb), c, 0, 0, 0);
}
// PV for one page in fp32: four 16x16x4 MFMAs, key 4q+i in the i-th.
__device__ __forceinline__ f32x4 pv_page_f32(u32x4 v, f32x4 p, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), p.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), p.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), p.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), p.w, c, 0, 0, 0);
  return c;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, f32x4 v);
template <> __device__ __forceinline__ void store4<__bf16>(__bf16* dst, f32x4 v) {
  u32x2 w = {pack_bf16(v.x, v.y), pack_bf16(v.z, v.w)};
  *(u32x2*)dst = w;
}
template <> __device__ __forceinline__ void store4<float>(float* dst, f32x4 v) { *(f32x4*)dst = v; }

// Descriptor lookup: last descriptor whose first item (or group) is <= key.
__device__ __forceinline__ int find_desc(CPTR(int32_t) descs, int n, int field, int key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (descs[mid * kDescInts + field] <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// This lane's index within its wave, through an empty asm statement (no instruction) that the
// compiler cannot see through: per-lane addresses derived from it are recomputed in each work item
// instead of being hoisted above a persistent kernel's claim loop and kept live (and spilled)
// across every item.
__device__ __forceinline__ int item_lane() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// The four LDS objects of a kernel (see Geo::kObjBytes): K and V staging buffers 0 and 1 of the
// prefill tile, and, for the decode role and the split merge, one combine table per wave.  The
// tile selects a buffer by a compile-time parity (its key loop is unrolled by two), so every
// access names one object.
struct Stage {
  char* k0;
  char* k1;
  char* v0;
  char* v1;
  __device__ __forceinline__ float* table(int w) const {
    return (float*)(w == 0 ? k0 : w == 1 ? k1 : w == 2 ? v0 : v1);
  }
};
template <int PAR> __device__ __forceinline__ char* kbuf_of(const Stage& B) { return PAR ? B.k1 : B.k0; }
template <int PAR> __device__ __forceinline__ char* vbuf_of(const Stage& B) { return PAR ? B.v1 : B.v0; }
template <int V> using Par = std::integral_constant<int, V>;

// ------------------------------------------------------------------ online-softmax update
// Per query column (lane l holds column l%16): x = raw scores of this block, -inf where masked,
// NV values per lane.  The running max m is kept in the log2 domain (scores times sl2 =
// scale*log2 e, sl2 > 0, so the max commutes with the scaling); updates m (identical in the 4
// lane groups) and l (this lane's partial sum), turns x into probabilities 2^(x*sl2 - m) and
// returns the rescale factor 2^(m_old - m_new) for the running output.
template <int NV>
__device__ __forceinline__ float softmax_update(float (&x)[NV], float sl2, float& m, float& l) {
  float mloc = x[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) mloc = fmaxf(mloc, x[i]);
  mloc = max_over_groups(mloc) * sl2;
  const float m_new = fmaxf(m, mloc);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = exp2_fast(m - m_use);
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = exp2_fast(__builtin_fmaf(x[i], sl2, -m_use));
  float part[NV];                                // pairwise sum: short dependency chain
#pragma unroll
  for (int i = 0; i < NV; ++i) part[i] = x[i];
#pragma unroll
  for (int w = NV / 2; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) part[i] = part[i] + part[i + w];
  const float sum = part[0];
  l = l * alpha + sum;
  m = m_new;
  return alpha;
}

// Rescale a running output only when some column's maximum moved (alpha == 1 exactly
// otherwise, so skipping the multiply changes nothing).
template <int N>
__device__ __forceinline__ void rescale(f32x4 (&o)[N], float alpha) {
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int b = 0; b < N; ++b) o[b] *= alpha;
  }
}

// ------------------------------------------------------------------ split partials
// Partials that another workgroup merges inside the same launch are written and read with
// device-scope (write-through / L2-bypassing) accesses: the writer's stores are complete once
// its vmcnt drains, so no cache-wide write-back is needed before the ticket is taken, and the
// merging wave never sees a stale line from its own L2.
__device__ __forceinline__ void store_part4(float* dst, f32x4 v) { *(f32x4*)dst = v; }
__device__ __forceinline__ void store_part1(float* dst, float v, bool coherent) {
  if (coherent) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *dst = v;
}
__device__ __forceinline__ float load_part1_coherent(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-coherent accesses to a run of partials, through a buffer resource over it:
// one 128-bit store or load per lane with the sc1 cache policy (written through past the
// writer's L2, read past the reader's), where 32-bit atomics would take four accesses and
// write partial memory lines four times.  Offsets are bytes from the resource base; the
// hardware drops accesses outside [0, bytes).
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kCachePolicyCoherent = 16;   // sc1
__device__ __forceinline__ BufRsrc part_rsrc(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);   // 32-bit data format
}
__device__ __forceinline__ void store_coherent4(BufRsrc r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCachePolicyCoherent);
}
__device__ __forceinline__ f32x4 load_coherent4(BufRsrc r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyCoherent));
}

// Prefill staging: one 16-byte chunk per lane from a (page, KV head) slab straight into LDS (lane
// i's chunk to dst + 16 i, dst wave-uniform), through a buffer resource over the slab (offsets
// past the slab are dropped by the hardware).  The buffer form of the LDS-DMA load, not the
// global one: the compiler's wait-count pass treats a global (flat) load that writes LDS as a
// pending access to both memory and LDS, and then drains every LDS read in flight at each
// operand wait of the tile.
// The LDS address of a lane is dst + 16 * lane: the load's immediate offset would be added to the
// LDS address as well as to the memory address, so it stays 0; the scalar offset moves only the
// memory address, and carries a unit's position in the slab, so that one resource serves every
// unit of a slab.
template <typename T, int D>
__device__ __forceinline__ BufRsrc slab_rsrc(const void* pool, int page, int hkv, int head) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slab_ptr<T, D>(pool, page, hkv, head)), (short)0,
                                           Geo<T, D>::kSlab, 0x00020000);
}
__device__ __forceinline__ void stage_chunk(BufRsrc r, int unit_off, int lane_off, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, lane_off, unit_off, 0, 0);
}

// Arrival of one split: every store of the calling wave has completed (vmcnt 0); one lane takes
// the group's ticket.  Returns, wave-uniformly, whether this split arrived last.
__device__ __forceinline__ int arrive_last(int32_t* ticket, int ns) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  int last = 0;
  if ((threadIdx.x & 63) == 0) last = atomicAdd(ticket, 1) == ns - 1;
  return __builtin_amdgcn_readfirstlane(last);
}

// ------------------------------------------------------------------ KV append
// The step's new tokens are written into their pages before attention reads them ([W6] "KV
// Cache": each step adds the new tokens' keys and values to the cache; [W6] "PagedAttention":
// position p of a sequence lives in slot p % 16 of the physical page that the sequence's
// block-table row names for logical page p / 16).  One wave writes one unit: a run of
// consecutive slots of one page for a range of KV heads, through a buffer resource over all
// KV-head slabs of that page with streaming stores (the attention kernels that read the pages
// start after this launch has completed).
// K: lane-consecutive stores are consecutive slots of one 16-byte chunk, i.e. contiguous bytes.
// V: where the run covers a whole 16-byte part of a dim (8 bf16 or 4 fp32 slots), a lane gathers
// the part's slots from the rows and stores the part, lanes covering consecutive parts; the
// run's remaining slots are written one element at a time, lanes covering consecutive dims.  A
// block-table entry outside the pool is not written through; the attention kernels, which read
// every page of the context, report it.
constexpr int kCachePolicyStream = 2;   // nt
template <typename T, int D>
__device__ void append_unit(const KernelParams& P, int seq, int row0, int pos0, int ntok, int h0, int nh) {
  using Gm = Geo<T, D>;
  constexpr int E = Gm::kBytes;
  const int lane = threadIdx.x & 63;
  const int slot0 = pos0 & (kPage - 1);
  const int pg = ((CPTR(int32_t))P.bt)[(size_t)seq * P.bt_stride + (pos0 >> 4)];
  if ((unsigned)pg < (unsigned)P.num_pages) {
    const int bytes = P.hkv * Gm::kSlab;
    const BufRsrc rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slab_ptr<T, D>(P.k, pg, P.hkv, 0)), (short)0, bytes, 0x00020000);
    const BufRsrc rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slab_ptr<T, D>(P.v, pg, P.hkv, 0)), (short)0, bytes, 0x00020000);
    const size_t row_bytes = (size_t)P.hkv * D * E;                 // one row of k_new / v_new
    const char* kn = (const char*)P.k_new + (size_t)row0 * row_bytes + (size_t)h0 * D * E;
    const char* vn = (const char*)P.v_new + (size_t)row0 * row_bytes + (size_t)h0 * D * E;
    // Batches carry no branches: a lane past the end reloads the last item and its stores get an
    // offset past the resource, which the hardware drops; so every load of a batch is in flight
    // before the first store waits.
    constexpr int kDrop = 1 << 30;
    constexpr int kV = Gm::kEpc;                   // elements per 16 bytes = slots per V part
    const int hd = D * E;                          // bytes of one head's row
    // K: items (head, chunk, token), token fastest; 4 per lane in flight.
    const int nk = nh * Gm::kNch * ntok;
    for (int i0 = 0; i0 < nk; i0 += 64 * 4) {
      u32x4 v[4];
      int off[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + 64 * j + lane, ic = min(i, nk - 1);
        const int t = ic % ntok, r = ic / ntok;
        const int c = r % Gm::kNch, hh = r / Gm::kNch;
        v[j] = ld16(kn + t * row_bytes + hh * hd + c * 16);
        off[j] = i < nk ? (h0 + hh) * Gm::kSlab + k_chunk_off(c, slot0 + t) : kDrop;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_buffer_store_b128(v[j], rk, off[j], 0, kCachePolicyStream);
    }
    // V, whole 16-byte parts (kV consecutive slots of one dim): parts [pf_lo, pf_hi) lie inside
    // the run.  Item (head, dim, part), part fastest, so that a store instruction's lanes write
    // whole consecutive lines; each item gathers its kV slots from kV rows (consecutive lanes read
    // consecutive dims of a row); 4 items per lane in flight.
    const int pf_lo = (slot0 + kV - 1) / kV, pf_hi = (slot0 + ntok) / kV;
    const int nfull = max(0, pf_hi - pf_lo);
    const int nvf = nh * D * nfull;
    for (int i0 = 0; i0 < nvf; i0 += 64 * 4) {
      u32x4 w[4];
      int off[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + 64 * j + lane, ic = min(i, nvf - 1);
        const int pp = pf_lo + ic % nfull, r = ic / nfull;
        const int d = r % D, hh = r / D;
        const char* src = vn + (size_t)(pp * kV - slot0) * row_bytes + hh * hd + d * E;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if constexpr (E == 2) {
            const uint32_t lo = *(const uint16_t*)(src + (2 * m) * row_bytes);
            const uint32_t hi = *(const uint16_t*)(src + (2 * m + 1) * row_bytes);
            w[j][m] = lo | (hi << 16);
          } else {
            w[j][m] = *(const uint32_t*)(src + m * row_bytes);
          }
        }
        off[j] = i < nvf ? (h0 + hh) * Gm::kSlab + v_elem_off<T>(d, pp * kV) : kDrop;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_buffer_store_b128(w[j], rv, off[j], 0, kCachePolicyStream);
    }
    // V, the run's other slots (before the first whole part and after the last), one element
    // each.  Item (head, slot, dim), dim fastest: a load instruction reads consecutive dims of a
    // row and a store instruction fills 4 elements of each line it touches; 16 per lane in flight.
    const int head_len = nfull > 0 ? pf_lo * kV - slot0 : ntok;
    const int npart = ntok - nfull * kV;
    const int nvp = nh * D * npart;
    for (int i0 = 0; i0 < nvp; i0 += 64 * 16) {
      uint32_t x[16];
      int off[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int i = i0 + 64 * j + lane, ic = min(i, nvp - 1);
        const int d = ic % D, r = ic / D;
        const int kk = r % npart, hh = r / npart;
        const int slot = kk < head_len ? slot0 + kk : pf_hi * kV + (kk - head_len);
        const char* src = vn + (size_t)(slot - slot0) * row_bytes + hh * hd + d * E;
        if constexpr (E == 2) x[j] = *(const uint16_t*)src;
        else x[j] = *(const uint32_t*)src;
        off[j] = i < nvp ? (h0 + hh) * Gm::kSlab + v_elem_off<T>(d, slot) : kDrop;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if constexpr (E == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)x[j], rv, off[j], 0, kCachePolicyStream);
        else __builtin_amdgcn_raw_buffer_store_b32(x[j], rv, off[j], 0, kCachePolicyStream);
      }
    }
  }
}

// ------------------------------------------------------------------ log-sum-exp combine
// out = sum_s w_s o_s / sum_s w_s with w_s = 2^(lse_s - max lse); empty splits weigh zero.
// In-kernel form, run by one wave for up to 16 columns of a group: the splits' lse values go to
// an LDS table `sw` ([16][ns] floats) with all loads in flight at once, the weights are formed
// once per column, then every (column, 4 dims) output sums its splits with 8 partial loads in
// flight.  Partials are read with device-scope loads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int D>
__device__ void combine_block_wave(const KernelParams& P, CPTR(int32_t) dsc, int head, int c0, float* sw) {
  const int lane = threadIdx.x & 63;
  const int ns = dsc[kDNSplit], ncols = dsc[kDNcols], q_row = dsc[kDQRow];
  const int nc = min(16, ncols - c0);
  const size_t base = (size_t)dsc[kDPartBase] + (size_t)head * ns * ncols;
  const int G = P.group;
  constexpr int kQ = D / 4;
  for (int i = lane; i < nc * ns; i += 64) {
    const int c = i / ns, sp = i - c * ns;
    sw[c * ns + sp] = load_part1_coherent(P.part_lse + base + (size_t)sp * ncols + c0 + c);
  }
  wave_lds_sync();
  if (lane < nc) {
    float M = kNegInf;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, sw[lane * ns + sp]);
    float sum = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float wgt = M == kNegInf ? 0.f : exp2_fast(sw[lane * ns + sp] - M);
      sw[lane * ns + sp] = wgt;
      sum += wgt;
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    for (int sp = 0; sp < ns; ++sp) sw[lane * ns + sp] *= inv;
  }
  wave_lds_sync();
  const int sstride = ncols * D * 4;                   // bytes between consecutive splits
  const BufRsrc grp = part_rsrc(P.part_o + base * D, ns * sstride);
  for (int pidx = lane; pidx < nc * kQ; pidx += 64) {
    const int c = pidx / kQ, d4 = pidx - c * kQ;
    const int src = ((c0 + c) * D + 4 * d4) * 4;
    const float* wc = sw + c * ns;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int sp = 0;
    for (; sp + 8 <= ns; sp += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = load_coherent4(grp, src + (sp + u) * sstride);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += wc[sp + u] * v[u];
    }
    for (; sp < ns; ++sp) acc += wc[sp] * load_coherent4(grp, src + sp * sstride);
    const int cc = c0 + c, qi = cc / G, hh = cc - qi * G;
    typedef typename QOf<T>::type QT;
    QT* dst = (QT*)P.out + ((size_t)(q_row + qi) * P.hq + head * G + hh) * D + 4 * d4;
    store4<QT>(dst, acc);
  }
}

// ------------------------------------------------------------------ decode item (one wave)
// One (decode sequence, KV head, key split) streamed by a single wave: the G query heads of
// the KV head are the columns of one 16-wide MFMA block; 32 keys (two pages) per step, with
// the next step's K/V loads in flight while the current step is computed.  Waves run their
// decode items independently (no workgroup barrier, no LDS).  A small-q extend piece (n_q
// query rows at positions q_pos .. q_pos+n_q-1, n_q*G <= 16) takes the same path: column n is
// query row n / G, head n % G, and on the steps that reach past q_pos each column sees the keys
// up to its own position ([W6] "Non-Causal vs. Causal Attention").
template <typename T, int D>
__device__ void decode_wave_item(const KernelParams& P, int item, float* sw) {
  using Gm = Geo<T, D>;
  typedef typename VOp<T>::type VT;
  CPTR(int32_t) descs = (CPTR(int32_t))P.ddesc;
  const int di = find_desc(descs, P.n_ddesc, kDItemBegin, item);
  CPTR(int32_t) dsc = descs + (size_t)di * kDescInts;
  const int ns = dsc[kDNSplit];
  const int local = item - dsc[kDItemBegin];
  const int split = local / P.hkv, head = local - split * P.hkv;   // adjacent items: adjacent heads

  const int lane = item_lane(), n = lane & 15, q = lane >> 4;
  const int G = P.group;
  const int seq = dsc[kDSeq], q_row = dsc[kDQRow], kv_len = dsc[kDKvLen];
  const int n_q = dsc[kDNq], ncols = dsc[kDNcols], q_pos = dsc[kDQPos];
  const int st = dsc[kDSplitTok];
  const int kv_begin = split * st;
  const int kv_end = min(kv_len, kv_begin + st);
  // Pages per step: 2 (the bf16 output product takes a page pair); 1 for an fp32 cache with
  // 128-dim heads, whose double-buffered step registers would otherwise exceed the budget.
  constexpr int kSp = (Gm::kBytes == 4 && D == 128) ? 1 : 2;
  constexpr int kStepTok = kSp * kPage;
  static_assert(kSp == 2 || Gm::kBytes == 4, "only the fp32 product takes single pages");
  const int n_steps = (kv_end - kv_begin + kStepTok - 1) / kStepTok;
  CPTR(int32_t) btr = (CPTR(int32_t))P.bt + (size_t)seq * P.bt_stride;
  const float sl2 = P.scale_log2;

  // Q^T operand: column n is query row q_row + n/G, head head*G + n%G (zero when n >= ncols).
  const int qi = n < ncols ? n / G : 0, hh = n < ncols ? n - qi * G : 0;
  const int cmax = q_pos + qi;                 // the last key column n sees
  u32x4 qop[Gm::kNs];
  {
    const char* qp = (const char*)P.q + ((size_t)(q_row + qi) * P.hq + head * G + hh) * (D * Gm::kQBytes);
#pragma unroll
    for (int s = 0; s < Gm::kNs; ++s) {
      u32x4 v = ld16(qp + (4 * s + q) * 16);
      qop[s] = n < ncols ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 o[Gm::kDb];
#pragma unroll
  for (int b = 0; b < Gm::kDb; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  typedef typename Gm::KReg KR;
  KR kA[kSp][Gm::kNs], kB[kSp][Gm::kNs];
  VT vA[kSp][Gm::kDb], vB[kSp][Gm::kDb];
  int limA[kSp], limB[kSp];
  float scA[2 * kSp], scB[2 * kSp];            // Fp8: K scales of the step's pages, then V scales

  auto load_step = [&](int step, KR (&kr)[kSp][Gm::kNs], VT (&vr)[kSp][Gm::kDb], int (&lim)[kSp],
                       float (&sc)[2 * kSp]) {
    const int tok0 = kv_begin + step * kStepTok;
#pragma unroll
    for (int p = 0; p < kSp; ++p) {
      const int pi = (tok0 >> 4) + p;
      int l = min(kPage, kv_end - pi * kPage);
      const int pg = __builtin_amdgcn_readfirstlane(page_or_empty(btr, pi, l, P.num_pages, P.ctrl + kCStatus));
      lim[p] = __builtin_amdgcn_readfirstlane(l);
      const char* kp = slab_ptr<T, D>(P.k, pg, P.hkv, head);
      const char* vp = slab_ptr<T, D>(P.v, pg, P.hkv, head);
      if constexpr (kIsFp8<T>) {
        // 8 codes per lane and step: dims 32s+8q .. +7 sit in 16-code chunk 2s + q/2, half q%2
#pragma unroll
        for (int s = 0; s < Gm::kNs; ++s) kr[p][s] = ld_stream<u32x2>(kp + k_chunk_off(2 * s + (q >> 1), n) + 8 * (q & 1));
        sc[p] = ((CPTR(float))P.k_scale)[(size_t)pg * P.hkv + head];
        sc[kSp + p] = ((CPTR(float))P.v_scale)[(size_t)pg * P.hkv + head];
      } else {
#pragma unroll
        for (int s = 0; s < Gm::kNs; ++s) kr[p][s] = ld_stream<u32x4>(kp + k_chunk_off(4 * s + q, n));
      }
#pragma unroll
      for (int b = 0; b < Gm::kDb; ++b) vr[p][b] = ld_stream<VT>(vp + v_elem_off<T>(16 * b + n, 4 * q));
    }
  };

  auto compute_step = [&](KR (&kr)[kSp][Gm::kNs], VT (&vr)[kSp][Gm::kDb], const int (&lim)[kSp],
                          const float (&sc)[2 * kSp], int tok0) {
    f32x4 sp[kSp];
#pragma unroll
    for (int p = 0; p < kSp; ++p) sp[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Gm::kNs; ++s) {
#pragma unroll
      for (int p = 0; p < kSp; ++p) sp[p] = mfma_chunk(k_operand(kr[p][s]), qop[s], sp[p], T());
    }
    if constexpr (kIsFp8<T>) {                 // the K scale of each page multiplies its scores
#pragma unroll
      for (int p = 0; p < kSp; ++p) sp[p] *= sc[p];
    }
    float x[4 * kSp];                          // key slot 4p + i: token 4q + i of page p
#pragma unroll
    for (int p = 0; p < kSp; ++p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * p + i] = (4 * q + i < lim[p]) ? sp[p][i] : kNegInf;
    }
    if (n_q > 1 && tok0 + kStepTok - 1 > q_pos) {   // extend rows: causal limit per column
#pragma unroll
      for (int p = 0; p < kSp; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (tok0 + kPage * p + 4 * q + i > cmax) x[4 * p + i] = kNegInf;
        }
      }
    }
    rescale(o, softmax_update<4 * kSp>(x, sl2, m_run, l_run));
    if constexpr (kIsFp8<T>) {
      // V codes -> bf16; the V scale of each page multiplies its probabilities in the product
      // only (the row sum already has them unscaled)
      u32x2 v8[2][Gm::kDb];
#pragma unroll
      for (int b = 0; b < Gm::kDb; ++b) {
        v8[0][b] = e4m3x4_to_bf16(vr[0][b]);
        v8[1][b] = e4m3x4_to_bf16(vr[1][b]);
      }
      if (lim[0] < kPage || lim[1] < kPage) {
#pragma unroll
        for (int b = 0; b < Gm::kDb; ++b) {
          v8[0][b] = mask_vop(v8[0][b], q, lim[0]);
          v8[1][b] = mask_vop(v8[1][b], q, lim[1]);
        }
      }
      const u32x4 pb = {pack_bf16(x[0] * sc[kSp], x[1] * sc[kSp]), pack_bf16(x[2] * sc[kSp], x[3] * sc[kSp]),
                        pack_bf16(x[4] * sc[kSp + 1], x[5] * sc[kSp + 1]), pack_bf16(x[6] * sc[kSp + 1], x[7] * sc[kSp + 1])};
#pragma unroll
      for (int b = 0; b < Gm::kDb; ++b) o[b] = pv_pair(v8[0][b], v8[1][b], pb, o[b]);
    } else {
#pragma unroll
      for (int p = 0; p < kSp; ++p) {
        if (lim[p] < kPage) {
#pragma unroll
          for (int b = 0; b < Gm::kDb; ++b) vr[p][b] = mask_vop(vr[p][b], q, lim[p]);
        }
      }
      if constexpr (Gm::kBytes == 2) {
        const u32x4 pb = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
#pragma unroll
        for (int b = 0; b < Gm::kDb; ++b) o[b] = pv_pair(vr[0][b], vr[1][b], pb, o[b]);
      } else {
#pragma unroll
        for (int p = 0; p < kSp; ++p) {
          const f32x4 pw = {x[4 * p], x[4 * p + 1], x[4 * p + 2], x[4 * p + 3]};
#pragma unroll
          for (int b = 0; b < Gm::kDb; ++b) o[b] = pv_page_f32(vr[p][b], pw, o[b]);
        }
      }
    }
  };

  // Two register sets; past the last step the prefetch re-reads the current step (cache hits,
  // results unused) so that every load is unconditional.
  int step = 0;
  load_step(0, kA, vA, limA, scA);
  for (;;) {
    int nxt = step + 1;
    load_step(nxt < n_steps ? nxt : step, kB, vB, limB, scB);
    compute_step(kA, vA, limA, scA, kv_begin + step * kStepTok);
    if (nxt >= n_steps) break;
    step = nxt;
    nxt = step + 1;
    load_step(nxt < n_steps ? nxt : step, kA, vA, limA, scA);
    compute_step(kB, vB, limB, scB, kv_begin + step * kStepTok);
    if (nxt >= n_steps) break;
    step = nxt;
  }

  // ---- epilogue: lane (n, q) holds O^T[16b + 4q + i][n]
  const float l_tot = sum_over_groups(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (n < ncols) {
    if (ns == 1) {
      typedef typename Gm::QT QT;
      QT* dst = (QT*)P.out + ((size_t)(q_row + qi) * P.hq + head * G + hh) * D + 4 * q;
#pragma unroll
      for (int b = 0; b < Gm::kDb; ++b) store4<QT>(dst + 16 * b, o[b] * inv);
    } else {
      const size_t run = (size_t)dsc[kDPartBase] + ((size_t)head * ns + split) * ncols;   // this split's slots
      const bool coh = P.inline_combine != 0;
      if (coh) {
        const BufRsrc r = part_rsrc(P.part_o + run * D, ncols * D * 4);
#pragma unroll
        for (int b = 0; b < Gm::kDb; ++b) store_coherent4(r, (n * D + 4 * q + 16 * b) * 4, o[b] * inv);
      } else {
        float* dst = P.part_o + (run + n) * D + 4 * q;
#pragma unroll
        for (int b = 0; b < Gm::kDb; ++b) store_part4(dst + 16 * b, o[b] * inv);
      }
      if (q == 0) store_part1(P.part_lse + run + n, l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf, coh);
    }
  }
  // Last arriver combines ([POD], "Virtual CTAs and per-SM balance": exact synchronisation
  // where partial results meet, and no wave ever waits for another).
  if (ns > 1 && P.inline_combine && arrive_last(P.tickets + dsc[kDGroupBegin] + head, ns))
    combine_block_wave<T, D>(P, dsc, head, 0, sw);
}

// ------------------------------------------------------------------ prefill item, fp32 cache
// One (query tile, KV head, key split): 128 columns = floor(128/G) queries x G heads; wave w
// owns columns 32w .. 32w+31 (two 16-wide blocks).  Keys advance 64 (or 32) at a time,
// staged in LDS by all 256 threads with the next tile's loads in flight.  (bf16 and FP8 caches
// take prefill_item_tile.)
template <typename T, int D>
__device__ void prefill_item(const KernelParams& P, CPTR(int32_t) dsc, int head, int split, const Stage& LB) {
  static_assert(sizeof(T) == 4 && !kIsFp8<T>, "the fp32 prefill item");
  using Gm = Geo<T, D>;
  const int lane = item_lane(), n = lane & 15, q = lane >> 4;
  const int w = wave_index();
  const int G = P.group;
  const int seq = dsc[kDSeq], q_row = dsc[kDQRow], n_q = dsc[kDNq], q_pos = dsc[kDQPos];
  const int kv_len = dsc[kDKvLen], ns = dsc[kDNSplit], st = dsc[kDSplitTok];
  const int ncols = n_q * G;
  const int kv_begin = split * st;
  const int kv_end = min(kv_len, kv_begin + st);
  const int n_tiles = (kv_end - kv_begin + Gm::kTileKeys - 1) / Gm::kTileKeys;
  CPTR(int32_t) btr = (CPTR(int32_t))P.bt + (size_t)seq * P.bt_stride;
  const float sl2 = P.scale_log2;

  // columns of this lane
  int pos[2];
  bool cval[2];
  u32x4 qop[2][Gm::kNs];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int c = 32 * w + 16 * nb + n;
    cval[nb] = c < ncols;
    const int cc = cval[nb] ? c : 0;
    const int qi = cc / G, hh = cc - qi * G;
    pos[nb] = q_pos + qi;
    const char* qp = (const char*)P.q + ((size_t)(q_row + qi) * P.hq + head * G + hh) * (D * Gm::kQBytes);
#pragma unroll
    for (int s = 0; s < Gm::kNs; ++s) {
      u32x4 v = ld16(qp + (4 * s + q) * 16);
      qop[nb][s] = cval[nb] ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int wc0 = 32 * w;
  const bool wave_active = wc0 < ncols;
  const int pmin = q_pos + wc0 / G;
  const int pmax = q_pos + (min(ncols, wc0 + 32) - 1) / G;

  f32x4 o[2][Gm::kDb];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int b = 0; b < Gm::kDb; ++b) o[nb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};

  // ---- staging: K and V pages of a key tile go HBM -> LDS directly (LDS-DMA, no registers);
  // instruction r of wave w moves linear chunks r*256 + 64w .. +63 of [K pages][V pages], one
  // 16-byte chunk per lane, into consecutive LDS.
  int lim_cur[Gm::kTp], lim_nxt[Gm::kTp];
  auto tile_pages = [&](int j, int (&lim)[Gm::kTp], int (&pg)[Gm::kTp]) {
    const int tb = kv_begin + j * Gm::kTileKeys;
#pragma unroll
    for (int p = 0; p < Gm::kTp; ++p) {
      const int pi = (tb >> 4) + p;
      int l = min(kPage, kv_end - pi * kPage);
      pg[p] = __builtin_amdgcn_readfirstlane(page_or_empty(btr, pi, l, P.num_pages, P.ctrl + kCStatus));
      lim[p] = __builtin_amdgcn_readfirstlane(l);
    }
  };
  auto kbuf = [&](auto par) { return kbuf_of<decltype(par)::value>(LB); };
  auto vbuf = [&](auto par) { return vbuf_of<decltype(par)::value>(LB); };
  auto issue_tile = [&](int j, auto b, int (&lim)[Gm::kTp]) {
    int pg[Gm::kTp];
    tile_pages(j, lim, pg);
#pragma unroll
    for (int r = 0; r < Gm::kStageR; ++r) {
      const int L0 = r * kThreads + 64 * w;                 // wave-uniform first chunk
      const int half = L0 / (Gm::kTp * Gm::kCps);
      const int rem0 = L0 - half * (Gm::kTp * Gm::kCps);
      const int p = rem0 / Gm::kCps, c0 = rem0 - p * Gm::kCps;
      int page = pg[0];
#pragma unroll
      for (int pp = 1; pp < Gm::kTp; ++pp) page = p == pp ? pg[pp] : page;
      const int c = c0 + lane;
      char* dst = (half ? vbuf(b) : kbuf(b)) + p * Gm::kSlab + c0 * 16;
      stage_chunk(slab_rsrc<T, D>(half ? P.v : P.k, page, P.hkv, head), 0, c * 16, dst);
    }
  };

  auto compute_tile = [&](auto b, int j, const int (&lim)[Gm::kTp]) {
    const int tb = kv_begin + j * Gm::kTileKeys;
    if (!wave_active || tb > pmax) return;                    // every key after every query
    bool full = tb + Gm::kTileKeys - 1 <= pmin;
#pragma unroll
    for (int p = 0; p < Gm::kTp; ++p) full = full && lim[p] == kPage;
    const char* kb = kbuf(b);
    const char* vb = vbuf(b);
    f32x4 S[2][Gm::kTp];
#pragma unroll
    for (int mb = 0; mb < Gm::kTp; ++mb) {
      u32x4 kop[Gm::kNs];
#pragma unroll
      for (int s = 0; s < Gm::kNs; ++s) kop[s] = *(const u32x4*)(kb + mb * Gm::kSlab + k_chunk_off(4 * s + q, n));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < Gm::kNs; ++s) acc = mfma_chunk(kop[s], qop[nb][s], acc, T());
        S[nb][mb] = acc;
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float x[4 * Gm::kTp];
      if (full) {                                  // wave-uniform: no key of the tile is masked
#pragma unroll
        for (int mb = 0; mb < Gm::kTp; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 * mb + i] = S[nb][mb][i];
      } else {
        const int rel = pos[nb] - tb - 4 * q;      // key slot 4q+i of page mb visible iff 16mb+i <= rel
#pragma unroll
        for (int mb = 0; mb < Gm::kTp; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = (4 * q + i < lim[mb]) & (mb * kPage + i <= rel);   // select, never multiply
            x[4 * mb + i] = ok ? S[nb][mb][i] : kNegInf;
          }
      }
      rescale(o[nb], softmax_update<4 * Gm::kTp>(x, sl2, m_run[nb], l_run[nb]));
#pragma unroll
      for (int mb = 0; mb < Gm::kTp; ++mb)
        S[nb][mb] = f32x4{x[4 * mb], x[4 * mb + 1], x[4 * mb + 2], x[4 * mb + 3]};
    }
    bool vmask = false;
#pragma unroll
    for (int p = 0; p < Gm::kTp; ++p) vmask = vmask || lim[p] < kPage;
#pragma unroll
    for (int mb = 0; mb < Gm::kTp; ++mb)
#pragma unroll
      for (int b2 = 0; b2 < Gm::kDb; ++b2) {
        const int d = 16 * b2 + n;
        u32x4 v = *(const u32x4*)(vb + mb * Gm::kSlab + v_elem_off<T>(d, 4 * q));
        if (vmask) v = mask_vop(v, q, lim[mb]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) o[nb][b2] = pv_page_f32(v, S[nb][mb], o[nb][b2]);
      }
  };
  // Tile j is staged in buffer j & 1 while tile j - 1 is computed; the loop is unrolled by two so
  // that each step names its buffers at compile time.
  auto step = [&](auto par, int j) {
    constexpr int PAR = decltype(par)::value;
    if (j + 1 < n_tiles) issue_tile(j + 1, Par<1 - PAR>(), lim_nxt);
    compute_tile(par, j, lim_cur);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < Gm::kTp; ++p) lim_cur[p] = lim_nxt[p];
  };
  if (n_tiles > 0) {
    issue_tile(0, Par<0>(), lim_cur);
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wave's LDS loads landed
    __syncthreads();
    for (int j = 0; j < n_tiles; j += 2) {
      step(Par<0>(), j);
      if (j + 1 < n_tiles) step(Par<1>(), j + 1);
    }
  }

  // ---- epilogue: normalise and write the output, or the split partial (o, lse)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l_tot = sum_over_groups(l_run[nb]);
    if (!cval[nb]) continue;
    const int c = 32 * w + 16 * nb + n;
    const int qi = c / G, hh = c - qi * G;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (ns == 1) {
      typedef typename Gm::QT QT;
      QT* dst = (QT*)P.out + ((size_t)(q_row + qi) * P.hq + head * G + hh) * D + 4 * q;
#pragma unroll
      for (int b2 = 0; b2 < Gm::kDb; ++b2) store4<QT>(dst + 16 * b2, o[nb][b2] * inv);
    } else {
      const size_t slot = (size_t)dsc[kDPartBase] + ((size_t)head * ns + split) * ncols + c;
      if (P.inline_combine) {                 // merged in-kernel by the group's last split (other dies read it)
        const BufRsrc r = part_rsrc(P.part_o + slot * D, D * 4);
#pragma unroll
        for (int b2 = 0; b2 < Gm::kDb; ++b2) store_coherent4(r, (4 * q + 16 * b2) * 4, o[nb][b2] * inv);
      } else {                                 // merged by the combine kernel
        float* dst = P.part_o + slot * D + 4 * q;
#pragma unroll
        for (int b2 = 0; b2 < Gm::kDb; ++b2) store_part4(dst + 16 * b2, o[nb][b2] * inv);
      }
      if (q == 0) store_part1(P.part_lse + slot, l_tot > 0.f ? m_run[nb] + __log2f(l_tot) : kNegInf, P.inline_combine != 0);
    }
  }
}

// ------------------------------------------------------------------ prefill tile, bf16
// Same item, same arithmetic, laid out for gfx950's LDS: every MFMA operand is one
// conflict-free 16-byte LDS read per lane, and the softmax spends as few VALU cycles per score
// as the method allows (the row sum runs on the matrix unit).
//
// Key -> row assignment of QK.  A 32-key pair of pages (pp) is scored as two 16-row blocks:
// block a holds keys 8r+i and block b keys 8r+4+i (r = row/4, i = row%4).  The MFMA output
// then gives lane group q the keys 8q .. 8q+7 of the pair (4 from a, 4 from b), i.e. one
// 16-byte chunk of a V row, so P^T feeds the PV product unshuffled and the V^T operand is a
// single b128 read.
//
// LDS tile (64 keys = 4 pages), one 1 KB unit per (page, group):
//   K unit (page p, chunk group s): the page's dim chunks 4s .. 4s+3 for its 16 tokens,
//     [chunk][slot][16 B], token t at slot kslot(p&1, t);
//   V unit (page p, dim group g): dims 32g .. 32g+31, [dim][half][16 B] (half h = tokens
//     8h .. 8h+7), i.e. the page's own byte order.
// Measured on gfx950 (LDS bank-conflict counter, one b128 read per lane): the K operand read
// conflicts two-way in the page's own order and not at all with the slot permutation, which is
// its own inverse, so the staging lane at slot i fetches source chunk kslot(p&1, i); the V
// operand read is conflict-free unpermuted.  Wave w stages page w of every tile: contiguous
// 1 KB HBM reads straight into LDS.
constexpr float kRescaleLog2 = 8.f;   // keep a stale running max while no probability exceeds 2^8

__device__ __forceinline__ int kslot(int par, int t) { return t ^ ((((t >> 3) & 1) ^ par) << 2); }

// Zero the bf16 V^T elements k >= lt of one lane's 8 token slots.
__device__ __forceinline__ u32x4 mask_v8(u32x4 v, int lt) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 2 * k;
    const uint32_t m = (t < lt ? 0x0000FFFFu : 0u) | (t + 1 < lt ? 0xFFFF0000u : 0u);
    r[k] = v[k] & m;
  }
  return r;
}

// The same tile for the bf16 cache (T = __bf16) and the FP8 cache (T = Fp8).  FP8: each wave
// stages its page's E4M3 codes (half the bytes) by LDS-DMA into the first units of the page's
// place, and once they have landed converts them in place into the bf16 layout above: each code
// decoded exactly, times the page's scale (K or V), rounded to bf16, once per workgroup.  From
// there on the tile is the bf16 one: no scale appears in the products, the softmax or the row
// sums.
template <typename T, int D>
__device__ void prefill_item_tile(const KernelParams& P, CPTR(int32_t) dsc, int head, int split, const Stage& LB) {
  constexpr bool kF8 = kIsFp8<T>;
  constexpr int kNs = D / 32;                  // QK steps of 32 dims
  constexpr int kKu = D / 32;                  // K units (1 KB) per page in LDS, bf16 layout
  constexpr int kVg = D / 32;                  // V units per page
  constexpr int kDma = Geo<T, D>::kSlab / 1024;   // 1 KB LDS-DMA pieces of a staged page
  constexpr int kDb = D / 16;                  // 16-dim blocks of O^T
  constexpr int kTp = 4, kTileKeys = kTp * kPage;
  constexpr int kKBytes = kTp * kKu * 1024;
  constexpr int kBufBytes = kKBytes + kTp * kVg * 1024;
  static_assert(kBufBytes * 2 == Geo<T, D>::kPrefillLds, "two staged tiles fill the prefill LDS");
  static_assert(kKBytes <= Geo<T, D>::kObjBytes && kTp * kVg * 1024 <= Geo<T, D>::kObjBytes, "a staged half fits its object");
  const int lane = item_lane(), n = lane & 15, q = lane >> 4;
  const int w = wave_index();
  const int G = P.group;
  const int seq = dsc[kDSeq], q_row = dsc[kDQRow], n_q = dsc[kDNq], q_pos = dsc[kDQPos];
  const int kv_len = dsc[kDKvLen], ns = dsc[kDNSplit], st = dsc[kDSplitTok];
  const int ncols = n_q * G;
  const int kv_begin = split * st;
  const int kv_end = min(kv_len, kv_begin + st);
  const int n_tiles = (kv_end - kv_begin + kTileKeys - 1) / kTileKeys;
  CPTR(int32_t) btr = (CPTR(int32_t))P.bt + (size_t)seq * P.bt_stride;
  const float sl2 = P.scale_log2;

  // Q^T operand: lane (column n, group q) holds dims 8(4s+q) .. +7 of its column.
  int pos[2];
  bool cval[2];
  u32x4 qop[2][kNs];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int c = 32 * w + 16 * nb + n;
    cval[nb] = c < ncols;
    const int cc = cval[nb] ? c : 0;
    const int qi = cc / G, hh = cc - qi * G;
    pos[nb] = q_pos + qi;
    const char* qp = (const char*)P.q + ((size_t)(q_row + qi) * P.hq + head * G + hh) * (D * 2);
#pragma unroll
    for (int s = 0; s < kNs; ++s) {
      u32x4 v = ld16(qp + (4 * s + q) * 16);
      qop[nb][s] = cval[nb] ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int wc0 = 32 * w;
  const bool wave_active = wc0 < ncols;
  const int pmin = q_pos + wc0 / G;
  const int pmax = q_pos + (min(ncols, wc0 + 32) - 1) / G;

  f32x4 o[2][kDb], lsum[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    lsum[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < kDb; ++b) o[nb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run[2] = {kNegInf, kNegInf};

  // lane-constant LDS offsets of the operand reads and of the staging sources
  const int par = n >> 3;
  const int t_a = 8 * ((n >> 2) & 1) + (n & 3);
  // K read = chunk q of the unit, 16 bytes
  const int koff_a = par * 1024 + (q * 16 + kslot(par, t_a)) * 16;
  const int koff_b = par * 1024 + (q * 16 + kslot(par, t_a + 4)) * 16;
  const int voff = (q >> 1) * 1024 + (2 * n + (q & 1)) * 16;
  // staging sources: bf16 K with the slot permutation; FP8 pages are copied in their own order
  // and permuted by the conversion
  const int src_k = kF8 ? lane * 16 : ((lane >> 4) * 16 + kslot(w & 1, lane & 15)) * 16;
  const int src_v = lane * 16;
  // FP8: the scale of this wave's page in each K buffer and in the V buffer being staged,
  // loaded with the staging (a vector load, counted with the LDS-DMA loads, so that no scalar
  // load is in flight beside the LDS reads) and applied when the page is converted
  float ks_own[2] = {1.f, 1.f}, vs_own = 1.f;
  auto scale_load = [&](const float* base, int page) {
    const BufRsrc r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base) + (size_t)page * P.hkv, (short)0,
                                                        P.hkv * 4, 0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, head * 4, 0, 0));
  };

  // LDS: K buffers 0 and 1, V buffers 0 and 1, four separate objects.  K(t) (tile t) lives in K
  // buffer t&1 and is staged two tiles ahead of the QK product that reads it, V(t) in V buffer
  // t&1 one tile ahead of its PV product, so that tile t's softmax can run beside tile t+1's QK.
  // Buffers are named by a compile-time parity (the loop below is unrolled by two).
  auto kbuf = [&](auto par) { return kbuf_of<decltype(par)::value>(LB); };
  auto vbuf = [&](auto par) { return vbuf_of<decltype(par)::value>(LB); };

  // Block-table entries, read one tile ahead: K and V each keep the entry of their own page of
  // the next tile they stage, so no staging waits for a scalar load, and page key counts are
  // arithmetic.  Absent pages past kv_end read the item's first entry, which exists.  Entries
  // outside the pool: the item's range is scanned once (every wave scans all of it, so all
  // agree); in an item that has one, such an entry becomes -1, is never dereferenced, its page
  // counts as absent, and page owners publish their key counts in s_lims.
  const int pfirst = kv_begin >> 4;
  bool clean;
  {
    bool bad = false;
    for (int i = pfirst + lane; i < (kv_end + kPage - 1) >> 4; i += 64)
      bad = bad | ((unsigned)btr[i] >= (unsigned)P.num_pages);
    clean = !__any(bad);
    if (!clean && threadIdx.x == 0) atomicOr(P.ctrl + kCStatus, (int)kStatusBadPage);
  }
  __shared__ int s_lims[2][kTp];
  auto page_lim = [&](int t, int p) {          // keys of page p of tile t (0: absent)
    return min(kPage, max(0, kv_end - (((kv_begin + t * kTileKeys) >> 4) + p) * kPage));
  };
  auto fetch_id = [&](int t) {                 // this wave's entry of tile t, as the table holds it
    return btr[page_lim(t, w) > 0 ? ((kv_begin + t * kTileKeys) >> 4) + w : pfirst];
  };
  // An entry is checked only when its page is staged, a tile after its load was issued, so that
  // no stage waits for the table read.
  auto usable = [&](int id) { return clean || (unsigned)id < (unsigned)P.num_pages ? id : -1; };
  int kpf, vpf;                                // entries of the next K / V tile to stage
  // Item with an entry outside the pool: tile t's key counts as its page owners published them
  // in stage_v (call after the barrier that follows).
  auto lims_after_barrier = [&](int t, int (&lim)[kTp]) {
    if (!clean) {
#pragma unroll
      for (int p = 0; p < kTp; ++p) lim[p] = s_lims[t & 1][p];
    }
  };

  // K(t): this wave stages page w of tile t into K buffer par = t & 1; returns whether it read
  // the page.
  auto stage_k = [&](auto par, int t) -> bool {
    const int own = usable(kpf), own_lim = own < 0 ? 0 : page_lim(t, w);
    if constexpr (kF8) ks_own[decltype(par)::value] = scale_load(P.k_scale, own < 0 ? 0 : own);
    kpf = fetch_id(t + 1);
    if (own_lim <= 0) return false;            // absent page: nothing is read
    char* dst = kbuf(par) + w * 1024;
    const BufRsrc r = slab_rsrc<T, D>(P.k, own, P.hkv, head);
    stage_chunk(r, 0, src_k, dst);
    if constexpr (kDma > 1) stage_chunk(r, 1024, src_k, dst + 4096);
    if constexpr (kDma > 2) stage_chunk(r, 2048, src_k, dst + 8192);
    if constexpr (kDma > 3) stage_chunk(r, 3072, src_k, dst + 12288);
    static_assert(kDma <= kKu && kKu <= 4, "K units per page");
    return true;
  };
  // V(t): key counts of the tile's pages into lim (item with an entry outside the pool: complete
  // only after the next barrier, see lims_after_barrier); this wave stages page w; returns its
  // count.
  auto stage_v = [&](auto par, int t, int (&lim)[kTp]) -> int {
    const int own = usable(vpf), own_lim = own < 0 ? 0 : page_lim(t, w);
#pragma unroll
    for (int p = 0; p < kTp; ++p) lim[p] = page_lim(t, p);
    if (!clean && lane == 0) s_lims[t & 1][w] = own_lim;
    if constexpr (kF8) vs_own = scale_load(P.v_scale, own < 0 ? 0 : own);
    vpf = fetch_id(t + 1);
    if (own_lim <= 0) return 0;
    char* dst = vbuf(par) + w * 1024;
    const BufRsrc r = slab_rsrc<T, D>(P.v, own, P.hkv, head);
    stage_chunk(r, 0, src_v, dst);
    if constexpr (kDma > 1) stage_chunk(r, 1024, src_v, dst + 4096);
    if constexpr (kDma > 2) stage_chunk(r, 2048, src_v, dst + 8192);
    if constexpr (kDma > 3) stage_chunk(r, 3072, src_v, dst + 12288);
    static_assert(kDma <= kVg && kVg <= 4, "V units per page");
    return own_lim;
  };
  // FP8, after this wave's staging loads have landed: convert its page of K buffer par in place
  // from the page's own order (FP8 chunk c of token t at byte (16c + t) * 16 of the staged
  // copy, 1 KB per unit) into the bf16 layout (bf16 chunks 2c and 2c+1 of that token, at the slot
  // whose source is t), each value decoded, times the page's K scale, rounded to bf16.  Every
  // lane reads all of its codes before any lane writes.
  auto convert_k = [&](auto par) {
    const float sc = ks_own[decltype(par)::value];
    char* kb = kbuf(par) + w * 1024;
    const int t = kslot(w & 1, lane & 15);     // source token of this lane's slot
    u32x4 c[kDma];
#pragma unroll
    for (int j = 0; j < kDma; ++j) c[j] = *(const u32x4*)(kb + j * 4096 + ((lane >> 4) * 16 + t) * 16);
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int c16 = 4 * j + (lane >> 4);     // FP8 chunk: dims 16 c16 .. 16 c16 + 15
      char* u = kb + (c16 >> 1) * 4096 + (2 * (c16 & 1) * 16 + (lane & 15)) * 16;
      *(u32x4*)u = e4m3x8_scaled_bf16(u32x2{c[j][0], c[j][1]}, sc);
      *(u32x4*)(u + 256) = e4m3x8_scaled_bf16(u32x2{c[j][2], c[j][3]}, sc);
    }
  };
  // FP8: the same for this wave's page of V buffer par (times the page's V scale): dim d's 16
  // codes (byte 16d of the staged copy) become its two 16-byte halves (tokens 0..7, 8..15) at
  // unit d/32, byte (d%32) * 32.
  auto convert_v = [&](auto par) {
    const float sc = vs_own;
    char* vb = vbuf(par) + w * 1024;
    u32x4 c[kDma];
#pragma unroll
    for (int j = 0; j < kDma; ++j) c[j] = *(const u32x4*)(vb + j * 4096 + lane * 16);
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const int d = 64 * j + lane;
      char* u = vb + (d >> 5) * 4096 + (d & 31) * 32;
      *(u32x4*)u = e4m3x8_scaled_bf16(u32x2{c[j][0], c[j][1]}, sc);
      *(u32x4*)(u + 16) = e4m3x8_scaled_bf16(u32x2{c[j][2], c[j][3]}, sc);
    }
  };
  // After this wave's staging loads have landed: zero the V slots of tokens >= lim of its page
  // (all of them for an absent page), so that a zero probability never meets a NaN or stale
  // value in the PV product.  Scores of those slots are masked by select.
  auto zero_v_tail = [&](auto par, int lim_own) {
    char* vu = vbuf(par) + w * 1024;
#pragma unroll
    for (int g = 0; g < kVg; ++g) {
      u32x4* cp = (u32x4*)(vu + g * 4096 + lane * 16);
      const u32x4 v = lim_own > 0 ? *cp : u32x4{0u, 0u, 0u, 0u};
      const int h = lane & 1;                  // the chunk holds tokens 8h .. 8h+7
      *cp = mask_v8(v, lim_own - 8 * h);
    }
  };

  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0 pairs
  typedef f32x4 Scores[2][2][2];               // S^T blocks [nb][pp][blk]

  // QK of one staged tile; the K operands of step k+1 are read while step k multiplies.
  auto qk = [&](const char* kb, Scores& S) {
    auto kread = [&](int k, u32x4 (&kop)[kNs]) {
      const int pp = k >> 1, blk = k & 1;
#pragma unroll
      for (int s = 0; s < kNs; ++s) kop[s] = *(const u32x4*)(kb + (s * 4 + 2 * pp) * 1024 + (blk ? koff_b : koff_a));
    };
    u32x4 kop0[kNs], kop1[kNs];
    kread(0, kop0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4 (&cur)[kNs] = (k & 1) ? kop1 : kop0;
      u32x4 (&nxt)[kNs] = (k & 1) ? kop0 : kop1;
      if (k + 1 < 4) kread(k + 1, nxt);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kNs; ++s) acc = mfma_chunk(cur[s], qop[nb][s], acc, __bf16());
        S[nb][k >> 1][k & 1] = acc;
      }
    }
  };
  // Causal and range mask of a tile that needs one: slot (pp, blk, i) of this lane is key
  // 32pp + 8q + 4blk + i of the tile, token 8(q&1) + 4blk + i of page 2pp + q/2, visible iff
  // 4blk + i <= bound(pp).  A select, never a multiply.
  auto apply_mask = [&](Scores& S, int tb, const int (&lim)[kTp]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int rel = pos[nb] - tb - 8 * q;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int lt = ((q >> 1) ? lim[2 * pp + 1] : lim[2 * pp]) - 8 * (q & 1);
        const int bound = min(rel - 32 * pp, lt - 1);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[nb][pp][blk][i] = 4 * blk + i <= bound ? S[nb][pp][blk][i] : kNegInf;
      }
    }
  };
  // Probabilities of a scored tile.  The running max m_run is a reference value that only moves
  // when a score exceeds it by more than 2^kRescaleLog2: any reference gives the same softmax as
  // long as numerator and denominator share it, and the bound keeps every probability <=
  // 2^kRescaleLog2.  So the common case takes the exponentials against the current reference
  // with no reduction first, and they issue beside the next tile's QK products; `probs` returns,
  // wave-uniformly, whether some column must move its reference (a probability above the bound,
  // or a column with none yet), and then `settle` takes the tile's per-column maxima, moves the
  // references that grew by more than the bound, rescales those columns' running output and sum by
  // 2^(m_old - m_new), and recomputes the probabilities.
  auto sval = [&](const Scores& S, int nb, int k) { return S[nb][k >> 3][(k >> 2) & 1][k & 3]; };
  auto col_max = [&](const Scores& S, int nb) {
    float m = fmaxf(sval(S, nb, 0), sval(S, nb, 1));
#pragma unroll
    for (int k = 2; k < 16; ++k) m = fmaxf(m, sval(S, nb, k));
    return m;
  };
  // whether some column's scores (raw, before the mask: a masked score only lowers a maximum)
  // exceed its reference by more than the bound, or a column has no reference yet
  auto needs_settle = [&](const Scores& S) -> bool {
    bool slow = false;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) slow = slow | (col_max(S, nb) * sl2 > m_run[nb] + kRescaleLog2) | (m_run[nb] == kNegInf);
    return __any(slow);
  };
  // masked scores: move the references that grew past the bound, rescale those columns
  auto settle = [&](const Scores& S) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mx = max_over_groups(col_max(S, nb)) * sl2;
      const bool grow = mx > m_run[nb] + kRescaleLog2;
      const float alpha = grow ? exp2_fast(m_run[nb] - mx) : 1.f;
      m_run[nb] = grow ? mx : m_run[nb];
#pragma unroll
      for (int b = 0; b < kDb; ++b) o[nb][b] *= alpha;
      lsum[nb] *= alpha;
    }
  };
  auto exps = [&](Scores& S) {                 // in place
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float mu = m_run[nb] == kNegInf ? 0.f : m_run[nb];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[nb][pp][blk][i] = exp2_fast(__builtin_fmaf(S[nb][pp][blk][i], sl2, -mu));
    }
  };
  // Product operands of the probabilities: bf16 pairs, keys 8q .. 8q+7 of a page pair per lane.
  auto pack = [&](const Scores& X, u32x4 (&pb)[2][2]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        float xp[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) xp[k] = sval(X, nb, 8 * pp + k);
        pb[nb][pp] = u32x4{pack_bf16(xp[0], xp[1]), pack_bf16(xp[2], xp[3]), pack_bf16(xp[4], xp[5]),
                           pack_bf16(xp[6], xp[7])};
      }
    }
  };
  // PV of one staged tile: V^T operands two blocks ahead of the products that use them; the row
  // sums come from the same P^T against a ones operand.
  auto pv = [&](const char* vb, const u32x4 (&pb)[2][2]) {
    auto vread = [&](int k) {
      const int pp = k / kDb, b2 = k % kDb;
      return *(const u32x4*)(vb + ((b2 >> 1) * 4 + 2 * pp) * 1024 + (b2 & 1) * 512 + voff);
    };
    constexpr int kPv = 2 * kDb;
    u32x4 vq[3];
    vq[0] = vread(0);
    vq[1] = vread(1);
#pragma unroll
    for (int k = 0; k < kPv; ++k) {
      const int pp = k / kDb, b2 = k % kDb;
      if (k + 2 < kPv) vq[(k + 2) % 3] = vread(k + 2);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) o[nb][b2] = mfma_chunk(vq[k % 3], pb[nb][pp], o[nb][b2], __bf16());
      if (b2 == kDb - 1) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) lsum[nb] = mfma_chunk(ones, pb[nb][pp], lsum[nb], __bf16());
      }
    }
  };

  // FP8: publish this wave's page scales of the tiles it just staged (lane 0; read by every wave
  // after the next barrier).  Deferred to the end of the iteration, when their loads are done.
  int lim_cur[kTp], lim_nxt[kTp];
  bool slow = true;                            // tile j's scores need a settle (always tile 0)
  // Iteration j: stage K(j+2) and V(j+1); QK(j+1) beside softmax(j) (one basic block, so the
  // matrix and vector units overlap); PV(j).  The product for tile j+1 past the last tile reads
  // a stale buffer and is discarded.
  auto iteration = [&](auto par, int j, Scores& Sc, Scores& Sn) {
    constexpr int PAR = decltype(par)::value;     // j & 1
    const int tb = kv_begin + j * kTileKeys;
    const bool more1 = j + 1 < n_tiles;
    const bool k_staged = j + 2 < n_tiles && stage_k(par, j + 2);
    int own_nv = kPage;
    if (more1) own_nv = stage_v(Par<1 - PAR>(), j + 1, lim_nxt);
    if (wave_active && tb <= pmax) {          // else every key follows every query of the wave
      const bool full = (tb + kTileKeys - 1 <= pmin) & (lim_cur[0] == kPage) & (lim_cur[1] == kPage) &
                        (lim_cur[2] == kPage) & (lim_cur[3] == kPage);
      if (!full) apply_mask(Sc, tb, lim_cur);
      if (slow) settle(Sc);
      qk(kbuf(Par<1 - PAR>()), Sn);
      exps(Sc);
      u32x4 pb[2][2];
      pack(Sc, pb);
      pv(vbuf(par), pb);
      slow = needs_settle(Sn);
    } else {
      // never read again (the wave's keys are done), but defined on this path too, so that no
      // tile's scores stay live across the loop's back edge
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) Sn[nb][pp][0] = Sn[nb][pp][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wave's staging loads landed
    if constexpr (kF8) {
      if (k_staged) convert_k(par);
      if (more1 && own_nv > 0) convert_v(Par<1 - PAR>());
    }
    if (own_nv < kPage) zero_v_tail(Par<1 - PAR>(), own_nv);
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTp; ++p) lim_cur[p] = lim_nxt[p];
    lims_after_barrier(j + 1, lim_cur);
  };

  if (n_tiles > 0) {
    Scores SA, SB;
    kpf = vpf = fetch_id(0);
    const bool k0 = stage_k(Par<0>(), 0);
    bool k1 = false;
    if (n_tiles > 1) k1 = stage_k(Par<1>(), 1);
    const int own0 = stage_v(Par<0>(), 0, lim_cur);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if constexpr (kF8) {
      if (k0) convert_k(Par<0>());
      if (k1) convert_k(Par<1>());
      if (own0 > 0) convert_v(Par<0>());
    }
    if (own0 < kPage) zero_v_tail(Par<0>(), own0);
    __syncthreads();
    lims_after_barrier(0, lim_cur);
    if (wave_active && kv_begin <= pmax) qk(kbuf(Par<0>()), SA);
    __syncthreads();                           // K buffer 0 is restaged by the first iteration
    for (int j = 0; j < n_tiles; j += 2) {
      iteration(Par<0>(), j, SA, SB);
      if (j + 1 < n_tiles) iteration(Par<1>(), j + 1, SB, SA);
    }
  }

  // ---- epilogue: normalise and write the output, or the split partial (o, lse)
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l_tot = lsum[nb][0];           // every row of the ones-product holds the column sum
    if (!cval[nb]) continue;
    const int c = 32 * w + 16 * nb + n;
    const int qi = c / G, hh = c - qi * G;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (ns == 1) {
      __bf16* dst = (__bf16*)P.out + ((size_t)(q_row + qi) * P.hq + head * G + hh) * D + 4 * q;
#pragma unroll
      for (int b2 = 0; b2 < kDb; ++b2) store4<__bf16>(dst + 16 * b2, o[nb][b2] * inv);
    } else {
      const size_t run = (size_t)dsc[kDPartBase] + ((size_t)head * ns + split) * ncols;   // this split's columns
      if (P.inline_combine) {                  // merged in-kernel by the group's last split
        const BufRsrc r = part_rsrc(P.part_o + run * D, ncols * D * 4);
#pragma unroll
        for (int b2 = 0; b2 < kDb; ++b2) store_coherent4(r, (c * D + 4 * q + 16 * b2) * 4, o[nb][b2] * inv);
      } else {                                 // merged by the combine kernel
        float* dst = P.part_o + (run + c) * D + 4 * q;
#pragma unroll
        for (int b2 = 0; b2 < kDb; ++b2) store_part4(dst + 16 * b2, o[nb][b2] * inv);
      }
      if (q == 0) store_part1(P.part_lse + run + c, l_tot > 0.f ? m_run[nb] + __log2f(l_tot) : kNegInf, P.inline_combine != 0);
    }
  }
}

// ------------------------------------------------------------------ item dispatch
// Prefill item: the whole workgroup.  Split partials (up to 128 columns x D floats per item) are
// merged in-kernel by the last-arriving split when inline_combine is set (fused mode; partials
// written through with 16-byte device-coherent stores), else by the combine kernel.
template <typename T, int D>
__device__ void run_prefill_item(const KernelParams& P, int item, const Stage& LB) {
  CPTR(int32_t) e = (CPTR(int32_t))P.pitems + kPItemHeader + 2 * (size_t)item;
  CPTR(int32_t) dsc = (CPTR(int32_t))P.pdesc + (size_t)e[0] * kDescInts;
  const int split = e[1] >> 16, head = e[1] & 0xFFFF;
  if constexpr (sizeof(T) == 2 || kIsFp8<T>) prefill_item_tile<T, D>(P, dsc, head, split, LB);
  else prefill_item<T, D>(P, dsc, head, split, LB);
  const int ns = dsc[kDNSplit];
  if (ns > 1 && P.inline_combine) {
    // Each wave's partial stores (write-through) complete before the barrier; thread 0 takes the
    // group's ticket; the workgroup holding the last split merges the group, each wave a block
    // of 16 columns at a time.  No workgroup waits for another.
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(P.tickets + dsc[kDGroupBegin] + head, 1) == ns - 1;
    __syncthreads();
    if (s_last) {
      float* sw = LB.table(wave_index());
      for (int c0 = 16 * wave_index(); c0 < dsc[kDNcols]; c0 += 16 * kWaves) combine_block_wave<T, D>(P, dsc, head, c0, sw);
    }
  }
  __syncthreads();   // LDS is reused by the next item
}

__device__ __forceinline__ int cu_slot() {
  const unsigned hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));     // HW_ID
  const unsigned xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11));    // XCC_ID[3:0]
  const unsigned cu = (hw >> 8) & 15u, sh = (hw >> 12) & 1u, se = (hw >> 13) & 3u;
  return (int)(((xcc & 7u) << 7) | (se << 5) | (sh << 4) | cu);
}

// Claim accounting: every run counts the items of each kind each CU claimed (the per-CU
// balance of the two kinds, read back as a run diagnostic); with POD_ATTN_FLAG_DEBUG_CLAIMS
// every item also counts its own claims.
__device__ __forceinline__ void note_claim(const KernelParams& P, int kind, int item, int cu) {
  if (P.claims) atomicAdd(P.claims + (kind == 0 ? 0 : P.n_pf_items) + item, 1);
  atomicAdd(P.ctrl + (kind == 0 ? kCClaimsPrefillCu : kCClaimsDecodeCu) + cu, 1);
}

// Timeline record of one work item (POD_ATTN_FLAG_TRACE): low 32 bits of the 100 MHz constant
// clock at the item's start and end, the CU slot that ran it, and its kind; one lane writes it.
__device__ __forceinline__ uint32_t clock100() { return (uint32_t)__builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t trace_start(const KernelParams& P) { return P.trace ? clock100() : 0u; }
__device__ __forceinline__ void trace_item(const KernelParams& P, int kind, int item, uint32_t t0, int cu) {
  if (P.trace) {
    const uint32_t t1 = clock100();
    *(u32x4*)(P.trace + 4 * ((size_t)(kind == 0 ? 0 : P.n_pf_items) + item)) = u32x4{t0, t1, (uint32_t)cu, (uint32_t)kind};
  }
}

// Prefill claim for a workgroup on XCC `xcc`: queue x is the item range [hdr[x], hdr[x+1]) of
// the item table, whole groups of tiles that read the same keys of the same KV head, so such
// tiles run on one die and reuse its L2; a workgroup whose queue is drained takes work from
// the other dies' queues.  Returns n_pf_items when every queue is drained.
__device__ __forceinline__ int claim_prefill(const KernelParams& P, int xcc) {
  CPTR(int32_t) hdr = (CPTR(int32_t))P.pitems;
  for (int k = 0; k < kXcds; ++k) {
    const int x = (xcc + k) & (kXcds - 1);
    const int b = hdr[x], n = hdr[x + 1] - b;
    if (n <= 0) continue;
    const int c = atomicAdd(P.ctrl + kCQueuePrefillXcd + 32 * x, 1);
    if (c < n) return b + c;
  }
  return P.n_pf_items;
}

// ------------------------------------------------------------------ kernels
// Fused persistent kernel: every workgroup loops, taking a role and claiming work of that kind.
// While decode work remains, at most kPrefillPerCu workgroups per CU hold the prefill role, so
// every CU keeps decode loads in flight beside its matrix work ([POD], "Virtual CTAs and per-SM balance": the scheduler places
// complementary work per SM).  A prefill-role workgroup works on one tile at a time with all
// four waves, taking tiles from its die's queue; a decode-role workgroup's four waves stream four
// adjacent decode items.  A workgroup whose kind is drained takes the other kind; the kernel
// ends when both are drained.
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void pod_fused_kernel(KernelParams P) {
  __shared__ __attribute__((aligned(16))) char lds_k0[Geo<T, D>::kObjBytes];
  __shared__ __attribute__((aligned(16))) char lds_k1[Geo<T, D>::kObjBytes];
  __shared__ __attribute__((aligned(16))) char lds_v0[Geo<T, D>::kObjBytes];
  __shared__ __attribute__((aligned(16))) char lds_v1[Geo<T, D>::kObjBytes];
  const Stage LB{lds_k0, lds_k1, lds_v0, lds_v1};
  __shared__ int s_role, s_item;
  const int tid = threadIdx.x;
  const int cu = cu_slot();
  const int xcc = cu >> 7;
  int* active = P.ctrl + kCActivePrefill + cu;
  bool pf_open = P.n_pf_items > 0, dc_open = P.n_dc_items > 0;
  bool counted = false;                       // thread 0: holds its CU's prefill slot
  for (;;) {
    if (tid == 0) {
      int role = -1;
      if (pf_open && dc_open) {
        const int a = atomicAdd(active, 1);
        if (a < kPrefillPerCu) {
          role = 0;
          counted = true;
        } else {
          atomicSub(active, 1);
          role = 1;
        }
      } else if (dc_open) {
        role = 1;
      } else if (pf_open) {
        role = 0;
      }
      s_role = role;
      if (role == 0) s_item = claim_prefill(P, xcc);
    }
    __syncthreads();
    const int role = s_role;
    int item = s_item;
    __syncthreads();
    if (role < 0) break;
    if (role == 1) {
      // The workgroup claims 4 consecutive items (adjacent KV heads of one key range) and each
      // wave streams one of them; the next block is claimed once the current one is done.
      float* sw = LB.table(wave_index());
      for (;;) {
        if (tid == 0) s_item = atomicAdd(P.ctrl + kCQueueDecode, kWaves);
        __syncthreads();
        const int base = s_item;
        __syncthreads();
        if (base >= P.n_dc_items) break;
        const int item = base + wave_index();
        if (item < P.n_dc_items) {
          if ((tid & 63) == 0) note_claim(P, 1, item, cu);
          const uint32_t t0 = trace_start(P);
          decode_wave_item<T, D>(P, item, sw);
          if ((tid & 63) == 0) trace_item(P, 1, item, t0, cu);
        }
      }
      dc_open = false;
      continue;
    }
    while (item < P.n_pf_items) {
      if (tid == 0) note_claim(P, 0, item, cu);
      const uint32_t t0 = trace_start(P);
      run_prefill_item<T, D>(P, item, LB);   // ends with a barrier
      if (tid == 0) trace_item(P, 0, item, t0, cu);
      if (tid == 0) s_item = claim_prefill(P, xcc);   // claim once idle
      __syncthreads();
      item = s_item;
      __syncthreads();
    }
    pf_open = false;
    if (tid == 0 && counted) {
      atomicSub(active, 1);
      counted = false;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void pod_prefill_kernel(KernelParams P) {
  __shared__ __attribute__((aligned(16))) char lds_k0[Geo<T, D>::kObjBytes];
  __shared__ __attribute__((aligned(16))) char lds_k1[Geo<T, D>::kObjBytes];
  __shared__ __attribute__((aligned(16))) char lds_v0[Geo<T, D>::kObjBytes];
  __shared__ __attribute__((aligned(16))) char lds_v1[Geo<T, D>::kObjBytes];
  const Stage LB{lds_k0, lds_k1, lds_v0, lds_v1};
  __shared__ int s_item;
  // one item per workgroup (the grid has n_pf_items workgroups), taken from this die's queue
  const int cu = cu_slot();
  if (threadIdx.x == 0) {
    s_item = claim_prefill(P, cu >> 7);
    if (s_item < P.n_pf_items) note_claim(P, 0, s_item, cu);
  }
  __syncthreads();
  const int item = s_item;
  if (item >= P.n_pf_items) return;
  const uint32_t t0 = trace_start(P);
  run_prefill_item<T, D>(P, item, LB);
  if (threadIdx.x == 0) trace_item(P, 0, item, t0, cu);
}

// Separate decode kernel: wave w of workgroup b takes decode item 4b + w.
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void pod_decode_kernel(KernelParams P) {
  const int item = (int)blockIdx.x * kWaves + wave_index();
  if (item >= P.n_dc_items) return;
  const int cu = cu_slot();
  if ((threadIdx.x & 63) == 0) note_claim(P, 1, item, cu);
  const uint32_t t0 = trace_start(P);
  decode_wave_item<T, D>(P, item, nullptr);   // no in-kernel combine here: the combine kernel merges
  if ((threadIdx.x & 63) == 0) trace_item(P, 1, item, t0, cu);
}

// Separate-mode combine: one workgroup per (group, block of 16 columns); the split weights of
// the block's columns are computed once into LDS, then every (column, 4 dims) is merged.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pod_combine_kernel(KernelParams P) {
  __shared__ float s_w[16][kMaxCombineSplits];
  __shared__ float s_inv[16];
  const int cb = P.combine_col_blocks;
  const int g = P.group_begin + (int)blockIdx.x / cb;
  const int blk = (int)blockIdx.x - ((int)blockIdx.x / cb) * cb;
  if (g >= P.group_end) return;
  const bool pf = g < P.n_pf_groups;
  CPTR(int32_t) descs = (CPTR(int32_t))(pf ? P.pdesc : P.ddesc);
  const int nd = pf ? P.n_pdesc : P.n_ddesc;
  const int di = find_desc(descs, nd, kDGroupBegin, g);
  CPTR(int32_t) dsc = descs + (size_t)di * kDescInts;
  const int head = g - dsc[kDGroupBegin];
  const int ns = dsc[kDNSplit], ncols = dsc[kDNcols], q_row = dsc[kDQRow];
  const int c0 = blk * 16;
  if (c0 >= ncols) return;
  const int nc = min(16, ncols - c0);
  const size_t base = (size_t)dsc[kDPartBase] + (size_t)head * ns * ncols;
  const int tid = threadIdx.x;
  for (int i = tid; i < nc * ns; i += kThreads) {
    const int c = i / ns, sp = i - c * ns;
    s_w[c][sp] = P.part_lse[base + (size_t)sp * ncols + c0 + c];
  }
  __syncthreads();
  if (tid < nc) {
    float M = kNegInf;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, s_w[tid][sp]);
    float sum = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float wgt = M == kNegInf ? 0.f : exp2_fast(s_w[tid][sp] - M);
      s_w[tid][sp] = wgt;
      sum += wgt;
    }
    s_inv[tid] = sum > 0.f ? 1.f / sum : 0.f;
  }
  __syncthreads();
  constexpr int kQ = D / 4;
  const int G = P.group;
  for (int idx = tid; idx < nc * kQ; idx += kThreads) {
    const int c = idx / kQ, d4 = idx - c * kQ;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < ns; ++sp) {
      const float wgt = s_w[c][sp];
      if (wgt > 0.f) acc += wgt * *(const f32x4*)(P.part_o + (base + (size_t)sp * ncols + c0 + c) * D + 4 * d4);
    }
    const int cc = c0 + c, qi = cc / G, hh = cc - qi * G;
    typedef typename QOf<T>::type QT;
    QT* dst = (QT*)P.out + ((size_t)(q_row + qi) * P.hq + head * G + hh) * D + 4 * d4;
    store4<QT>(dst, acc * s_inv[c]);
  }
}

// Debug gather: element (t, g, d) of one sequence, through the kernels' page addressing.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pod_gather_kernel(const void* cache, int which,
                                                             const int32_t* bt_row, int ctx, int hkv,
                                                             int num_pages, void* out, int32_t* status) {
  using Gm = Geo<T, D>;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)ctx * hkv * D;
  if (idx >= total) return;
  const int d = (int)(idx % D);
  const int g = (int)((idx / D) % hkv);
  const int t = (int)(idx / ((size_t)D * hkv));
  const int pg = bt_row[t >> 4];
  // element storage type: the cache's (raw codes for Fp8)
  typedef typename std::conditional<kIsFp8<T>, uint8_t, T>::type ST;
  ST val = ST(0);
  const char* p = nullptr;
  if ((unsigned)pg < (unsigned)num_pages) {
    const char* sp = slab_ptr<T, D>(cache, pg, hkv, g);
    const int slot = t & 15;
    p = (which & 1) == 0 ? sp + k_chunk_off(d / Gm::kEpc, slot) + (d % Gm::kEpc) * Gm::kBytes
                         : sp + v_elem_off<T>(d, slot);
    val = *(const ST*)p;
  } else if (status) {
    atomicOr(status, (int)kStatusBadPage);
  }
  if constexpr (kIsFp8<T>) {
    if (which & 2) {                 // decoded through the kernels' E4M3 -> bf16 conversion
      const u32x2 w = e4m3x4_to_bf16((uint32_t)val);
      ((uint16_t*)out)[idx] = (uint16_t)(w.x & 0xFFFFu);
      return;
    }
  }
  ((ST*)out)[idx] = val;
}

// Separate-mode KV append, launched after the plan upload and before the attention kernels:
// wave w of workgroup b writes unit 4b + w.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pod_append_kernel(KernelParams P) {
  const int u = (int)blockIdx.x * kWaves + wave_index();
  if (u >= P.n_aunits) return;
  CPTR(int32_t) a = (CPTR(int32_t))P.aunits + (size_t)u * kAUnitInts;
  if constexpr (!kIsFp8<T>) append_unit<T, D>(P, a[kASeq], a[kARow], a[kAPos], a[kANtok], a[kAHead], a[kANh]);
}

// Plan upload, launched before the attention kernels on the same stream: workgroups
// [0, copy_wgs) zero-fill the workspace's counter region [0, 16 n_zero16) and copy the
// descriptor region after it from the pinned host staging buffer (read over the host link), one
// 16-byte word per thread.  A kernel starts sooner after the previous kernel than a DMA copy's
// completion can release it.  In fused mode the KV append rides in the same launch: wave w of
// workgroup copy_wgs + b writes unit 4b + w, its fields read from the staging buffer (the
// workspace copy is being written by this launch), so the persistent kernel that follows reads
// an updated cache and has nothing to wait for.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pod_stage_kernel(StageArgs A) {
  const int b = (int)blockIdx.x;
  if (b < A.copy_wgs) {
    const int i = b * kThreads + (int)threadIdx.x;
    u32x4* dst = (u32x4*)A.dst;
    if (i < A.n_zero16) dst[i] = u32x4{0u, 0u, 0u, 0u};
    else if (i < A.n_zero16 + A.n_copy16) dst[i] = ((const u32x4*)A.src)[i - A.n_zero16];
    return;
  }
  const int u = (b - A.copy_wgs) * kWaves + wave_index();
  if (u >= A.p.n_aunits) return;
  const u32x4* f = (const u32x4*)(A.units_host + (size_t)u * kAUnitInts);
  const u32x4 f0 = f[0], f1 = f[1];          // every lane reads the same 32 bytes
  if constexpr (!kIsFp8<T>) append_unit<T, D>(A.p, __builtin_amdgcn_readfirstlane(f0[kASeq]), __builtin_amdgcn_readfirstlane(f0[kARow]),
                    __builtin_amdgcn_readfirstlane(f0[kAPos]), __builtin_amdgcn_readfirstlane(f0[kANtok]),
                    __builtin_amdgcn_readfirstlane(f1[kAHead - 4]), __builtin_amdgcn_readfirstlane(f1[kANh - 4]));
}

template <typename T, int D>
KernelSet make_set() {
  KernelSet s;
  s.fused = (const void*)&pod_fused_kernel<T, D>;
  s.prefill = (const void*)&pod_prefill_kernel<T, D>;
  s.decode = (const void*)&pod_decode_kernel<T, D>;
  s.combine = (const void*)&pod_combine_kernel<T, D>;
  s.gather = (const void*)&pod_gather_kernel<T, D>;
  s.stage = (const void*)&pod_stage_kernel<T, D>;
  s.append = (const void*)&pod_append_kernel<T, D>;
  s.fused_lds = Geo<T, D>::kFusedLds;
  s.prefill_kv_tile = Geo<T, D>::kTileKeys;
  return s;
}

// ------------------------------------------------------------------ measurement probes
// Streaming read of n16 16-byte chunks in 16 KiB blocks: wave v of the grid reads blocks v,
// v + waves, ..., with two blocks in flight (the next block's 16 loads per lane are issued before
// the current block is folded; consecutive lanes on consecutive chunks); each workgroup writes the
// XOR of its words to sink[wg] (so the read cannot be dropped, and a test can check that every
// byte was read).
__global__ __launch_bounds__(kThreads) void pod_probe_hbm_read_kernel(const u32x4* buf, size_t n16, uint32_t* sink) {
  constexpr int kPer = 16;                     // loads per lane per block
  constexpr size_t kBlock = 64 * kPer;         // chunks per block (16 KiB)
  const size_t nwaves = (size_t)gridDim.x * kWaves;
  const size_t lane = threadIdx.x & 63;
  uint32_t x = 0;
  auto load = [&](size_t blk, u32x4 (&v)[kPer]) {
    const size_t base = blk * kBlock + lane;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const size_t i = base + (size_t)j * 64;
      v[j] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto fold = [&](const u32x4 (&v)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  };
  size_t blk = (size_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  u32x4 a[kPer], b[kPer];
  if (blk * kBlock < n16) {
    load(blk, a);
    for (;;) {                                 // a holds block blk (in flight)
      size_t nx = blk + nwaves;
      const bool more = nx * kBlock < n16;
      if (more) load(nx, b);
      fold(a);
      if (!more) break;
      blk = nx;                                // b holds block blk
      nx = blk + nwaves;
      const bool more2 = nx * kBlock < n16;
      if (more2) load(nx, a);
      fold(b);
      if (!more2) break;
      blk = nx;
    }
  }
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  __shared__ uint32_t s_x[kWaves];
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

// Dense bf16 MFMA: every wave runs kProbeChains independent 32x32x16 accumulation chains for
// `iters` rounds (measured on gfx950 with 4096 x 4 waves: 8 chains of the 32x32 form reach 96% of
// the 2.5 PFLOP/s peak, 4 chains 90%; the 16x16x32 form needs 16 chains for 93%).  A is all ones and B all 2^-4, so each product adds exactly 1.0 to every
// accumulator element; lane 0 of each wave writes the sum of its chains' first elements
// (kProbeChains * iters) to sink[4 * wg + wave].
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(kThreads) void pod_probe_mfma_kernel(int iters, float* sink) {
  const uint32_t bv = iters > 0 ? 0x3D803D80u : 0u;    // bf16 2^-4 pairs, opaque to the compiler
  const u32x4 a = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4 b = {bv, bv, bv, bv};
  const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a), B = __builtin_bit_cast(bf16x8_t, b);
  f32x16 c[kProbeChains];
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k) {
#pragma unroll
    for (int e = 0; e < 16; ++e) c[k][e] = 0.f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kProbeChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c[k], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k) t += c[k][0];
  if ((threadIdx.x & 63) == 0) sink[4 * blockIdx.x + (threadIdx.x >> 6)] = t;
}

}  // namespace

ProbeKernels probe_kernels() {
  ProbeKernels p;
  p.hbm_read = (const void*)&pod_probe_hbm_read_kernel;
  p.mfma = (const void*)&pod_probe_mfma_kernel;
  return p;
}

KernelSet kernel_set(int dtype, int head_dim) {
  if (dtype == 0 && head_dim == 128) return make_set<__bf16, 128>();
  if (dtype == 0 && head_dim == 64) return make_set<__bf16, 64>();
  if (dtype == 2 && head_dim == 128) return make_set<Fp8, 128>();
  if (dtype == 2 && head_dim == 64) return make_set<Fp8, 64>();
  if (dtype == 1 && head_dim == 128) return make_set<float, 128>();
  return make_set<float, 64>();
}

}  // namespace pod

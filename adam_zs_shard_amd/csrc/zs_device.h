// zs_device.h -- device helpers shared by the gfx950 kernels of libzshard.
//
// The per-shard step is pure streaming: per element it reads P 16-bit
// gradients and the fp32 (w, m, v), writes (w, m, v) and one 16-bit working
// copy, and does O(P) flops.  At about 0.5 flop/byte it sits far below the
// fp32 vector ridge of the chip: the design goal is HBM bandwidth.
//  - Work comes in groups of 2048 elements, 8 per lane of a 256-lane
//    workgroup, at a workgroup-uniform base (SGPRs) plus per-lane byte
//    offsets.  In a full group, lane l of wave wv owns two quads: elements
//    512 wv + 4l + {0..3} and 512 wv + 256 + 4l + {0..3} of the group (the
//    lane map, Lanes below).  Every access is then a whole-line stream: each
//    8-byte access of a 16-bit array (gradients, working copy) covers 512
//    contiguous bytes per wave, each 16-byte access of an fp32 array (w, m,
//    v) 1 KiB, so no store instruction leaves a cache line half written.  The
//    last, partial group of a range keeps 8 consecutive elements per lane,
//    and so do the whole chunks of the single-tensor fused kernel (one
//    16-byte gradient load per rank and group), whose fp32 stores are made
//    whole-line by a cross-lane swap (st_f32x8_lines).
//  - Gradient reads are rank-major: for each rank in turn a wave issues its
//    first group's loads, uses them, then the other 27 groups' loads of the
//    chunk back to back (scheduling barriers stop the compiler from sinking
//    each load next to its use), then adds them into the per-group sums.
//    Every element receives the ranks in order 0..P-1: a left fold, one fp32
//    rounding per add, exactly the oracle's order.  All loads and stores are
//    non-temporal (each byte is touched once).
//  - Phase separation: HBM on this part streams reads alone far faster than
//    reads with any writes mixed in.  A workgroup therefore sums the
//    gradients of a whole chunk (28 groups, held in registers with one wave
//    per SIMD) before it touches w, m, v and the working copy, so reads and
//    writes reach the memory in separate stretches.
//  - One workgroup per CU.  Full chunks (28 groups) go round-robin; the
//    remainder (at most one chunk's worth, plus up to 14 scalar elements) is
//    dealt to the workgroups that got one chunk fewer, and is read with the
//    ranks batched, so the workgroups finish together.  Shards under half a
//    chunk per CU get no whole chunk: small_kernel deals their pieces over
//    three workgroups per CU instead.
//  - Soft barriers: with one workgroup per CU the CUs drift apart over the
//    rounds of chunks until reads and writes mix again; every few rounds a
//    soft barrier (soft_barrier below) pulls the grid back into step.
//  - No MFMA and no LDS on the single-tensor path (nothing is reused); the
//    multi-tensor path stages one chunk's descriptors in LDS.
// Arithmetic (rank-order fp32 mean, Adam moments, bias correction, update,
// round-to-nearest-even downcast) follows the pages cited in zshard.h:
// [DP-III] §(一) (Adam), §(四) steps 2-4; [EAI19] 通信原语 All-Reduce (mean);
// [ZP] 核心原理 and [ZA] §2.2 (fp32 update then the 16-bit working copy).
// Compiled with -ffp-contract=off and the pragma below: no FMA contraction;
// division and sqrt are the correctly rounded HIP defaults; fp32 denormals
// are kept.

#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "zs_internal.h"

#pragma clang fp contract(off)

namespace zs {
namespace {

// Vectors that may sit at any 2-byte (u16) or 4-byte (fp32) address: gfx950
// runs with unaligned access enabled, so these still compile to single
// global_load / global_store instructions of 8 or 16 bytes.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(2)));
typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));

// Groups whose rank sums are held in registers across the read-only phase of
// a full chunk (28 x 8 fp32 values per lane: with one wave per SIMD the
// kernel may use the whole 512-entry register file), the gradient loads a
// wave issues back to back, and the groups of the smaller chunks that take
// the remainder of a range.
constexpr int kGroupsMax = 28;
// Groups of loads per batch of a rank in the whole-chunk read phase (after
// the probe loads of group 0): fused_kernel issues the rest of the chunk, 27
// groups, in one batch; table_kernel keeps batches of 14.
constexpr int kLoadBatch = 28;
constexpr int kTableLoadBatch = 14;
static_assert(kGroupsMax % kLoadBatch == 0, "whole load batches per chunk");
static_assert(kGroupsMax % kTableLoadBatch == 0, "whole load batches per chunk");

// Soft barrier.  One workgroup per CU starts every round of chunks with its
// read phase, but the CUs do not run at one speed (some XCDs run 1-2.5%
// slower for a whole launch, and a round's time varies by 7-14% from CU to
// CU), so after a few rounds some CUs read gradients while others update,
// and HBM serves that mix more slowly than the two phases apart.  A grid-wide
// barrier would put them back in step but waits for the slowest workgroup
// every time.  This one waits only for most of the grid: thread 0 counts its
// workgroup in, then waits until kSoftPct percent of the grid has arrived,
// the last arrival has reset the count for the slot's next use, or
// kSoftCapTicks of the 100 MHz real-time clock have passed.  It orders no
// data (no workgroup reads what another writes), so results never depend on
// it, and the cap bounds every wait: a grid that is not all resident, or a
// launch on another stream sharing the counters, can cost time, never
// correctness.  The counters are file-scope device arrays, zero at load;
// each use of a slot brings its count back to zero.  Waiters poll them every
// ~3.4 us (the longest sleep): polling every 0.1 us was 0.1% (7.5B shard)
// and 0.4% (Llama table) slower.
constexpr unsigned int kSoftPct = 90;
constexpr uint64_t kSoftCapTicks = 20000;  // 200 us
constexpr int kSoftSlots = 64;
__device__ unsigned int g_soft_arrive[kSoftSlots];
__device__ unsigned int g_soft_gen[kSoftSlots];

// Barrier number j of a launch (j >= 1); every thread of the workgroup calls it.
__device__ __forceinline__ void soft_barrier(int j) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int s = j & (kSoftSlots - 1);
    const unsigned int g = gridDim.x;
    const unsigned int gen0 =
        __hip_atomic_load(&g_soft_gen[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned int old =
        __hip_atomic_fetch_add(&g_soft_arrive[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 >= g) {  // the last arrival: reset the slot, release the waiters
      __hip_atomic_store(&g_soft_arrive[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&g_soft_gen[s], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const unsigned int enough = (g * kSoftPct) / 100;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(&g_soft_gen[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 gen0 &&
             __hip_atomic_load(&g_soft_arrive[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                 enough) {
        __builtin_amdgcn_s_sleep(127);  // about 3.4 us between polls
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSoftCapTicks) break;
      }
    }
  }
  __syncthreads();
}

// Staging of the 16-bit working copy in whole chunks.  A shard's slice of
// the full working copy starts wherever s_k puts it (rank 63 of the 7.5B
// shard: 40 bytes into a 64-byte segment), so each wave's store of the copy
// would begin and end mid-line.  Instead each lane puts its values of every
// group into LDS at their place relative to the 128-byte line below the
// chunk's start (rounded down to 8 bytes: 8-byte LDS writes), and after the
// chunk's update the workgroup writes the chunk's 112 KiB out in 16-byte
// units on whole lines; only the two lines at the chunk's ends are partial,
// and each byte is still written by one workgroup (7.5B shard, fused step:
// 2.674 -> 2.651 ms in one process).
typedef uint32_t u32x4a16 __attribute__((ext_vector_type(4), aligned(16)));
typedef uint32_t u32x2a8 __attribute__((ext_vector_type(2), aligned(8)));
constexpr uint32_t kChunkCopyBytes = kGroupsMax * kBlock * kVec * 2;  // 114,688
constexpr uint32_t kCopyStage = kChunkCopyBytes + 128;

// The contiguous-map lane's 8 values of group u (y = u * 4096 + 16 * lane +
// the chunk's offset in its line rounded down to 8), or one quad of 4 values
// of the full-group map (stage_quad: y = u * 4096 + the quad's byte offset in
// the group + the same rounded offset).
__device__ __forceinline__ void stage_quad(unsigned char* lds, uint32_t y, u32x2 x) {
  *reinterpret_cast<u32x2a8*>(lds + y) = u32x2a8{x[0], x[1]};
}
__device__ __forceinline__ void stage_copy(unsigned char* lds, uint32_t y, u32x4 x) {
  reinterpret_cast<u32x2a8*>(lds + y)[0] = u32x2a8{x[0], x[1]};
  reinterpret_cast<u32x2a8*>(lds + y)[1] = u32x2a8{x[2], x[3]};
}

// The staged chunk out to bytes [a0 + d, a0 + d + kChunkCopyBytes), a0 on a
// 128-byte line; LDS byte y holds byte a0 + (d & 7) + y.
__device__ __forceinline__ void flush_copy(const unsigned char* lds, unsigned char* a0,
                                           uint32_t d) {
  const uint32_t r = d & 7u;
  const uint32_t end = d + kChunkCopyBytes;
  const uint32_t nunits = (end + 15u) / 16u;
  for (uint32_t i = threadIdx.x; i < nunits; i += kBlock) {
    const uint32_t b = 16u * i;
    if (b >= d && b + 16u <= end) {
      u32x4a16 x;
      if (r == 0) {
        x = *reinterpret_cast<const u32x4a16*>(lds + b);
      } else {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(lds + b - r);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = q[2 * j] | (static_cast<uint32_t>(q[2 * j + 1]) << 16);
      }
      __builtin_nontemporal_store(x, reinterpret_cast<u32x4a16*>(a0 + b));
    } else {
#pragma unroll
      for (uint32_t j = 0; j < 16u; j += 2u) {
        const uint32_t bj = b + j;
        if (bj >= d && bj < end)
          *reinterpret_cast<uint16_t*>(a0 + bj) =
              *reinterpret_cast<const uint16_t*>(lds + bj - r);
      }
    }
  }
}

constexpr int64_t kGroup = static_cast<int64_t>(kBlock) * kVec;  // elements per group

template <int DT>
__device__ __forceinline__ float widen_lo(uint32_t x) {
  if constexpr (DT == kF16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x & 0xffffu)));
  } else {
    return __builtin_bit_cast(float, x << 16);
  }
}

template <int DT>
__device__ __forceinline__ float widen_hi(uint32_t x) {
  if constexpr (DT == kF16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x >> 16)));
  } else {
    return __builtin_bit_cast(float, x & 0xffff0000u);
  }
}

template <int DT>
__device__ __forceinline__ float widen1(uint16_t h) {
  return widen_lo<DT>(static_cast<uint32_t>(h));
}

// fp32 -> 16 bits, round to nearest even (v_cvt_f16_f32 under the default
// rounding mode; v_cvt_pk_bf16_f32 on gfx950).
template <int DT>
__device__ __forceinline__ uint16_t narrow1(float x) {
  if constexpr (DT == kF16) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
}

template <int DT>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
  return static_cast<uint32_t>(narrow1<DT>(lo)) | (static_cast<uint32_t>(narrow1<DT>(hi)) << 16);
}

// One update of one element, in place.  Adam (both forms): the two moment
// products rounded, their sum rounded; bias correction by division;
// d = sqrt(v_hat) + eps; u = m_hat / d; w - lr*u.  The SGD forms touch only
// what they use: w - lr*g, or m = beta1*m + g then w - lr*m.
template <int FORM>
__device__ __forceinline__ void adam1(const Consts& c, float g, float& w, float& m, float& v) {
  if constexpr (FORM == kSgd) {  // w - lr*g; m, v unused
    w = w - c.LR * g;
    return;
  } else if constexpr (FORM == kSgdMomentum) {  // heavy-ball: m = beta1*m + g; w - lr*m
    m = c.B1 * m + g;
    w = w - c.LR * m;
    return;
  }
  const float mm = c.B1 * m + c.C1 * g;
  const float vv = c.B2 * v + c.C2 * (g * g);
  float mh, vh;
  if constexpr (FORM == kStandard) {
    m = mm;
    v = vv;
    mh = mm / c.BC1;
    vh = vv / c.BC2;
  } else {
    m = mm / c.BC1;
    v = vv / c.BC2;
    mh = m;
    vh = v;
  }
  const float d = __builtin_sqrtf(vh) + c.EPS;
  const float u = mh / d;
  w = w - c.LR * u;
}

// adam1's Adam forms in two halves over a lane's 8 elements, with the same
// operations in the same order per element: the moments (m, v as stored,
// and the corrected m_hat, v_hat), then the weights.  A group's stores of m
// and v can then go out before the divisions and square roots of the weight
// update, in two bursts instead of one (0.4% on the 64-rank shard, 1.2% on
// the update from a stored mean).
template <int FORM>
__device__ __forceinline__ void adam_moments8(const Consts& c, const float (&g)[8], float (&M)[8],
                                              float (&V)[8], float (&MH)[8], float (&VH)[8]) {
  static_assert(FORM == kStandard || FORM == kPage1Literal, "Adam forms only");
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float mm = c.B1 * M[j] + c.C1 * g[j];
    const float vv = c.B2 * V[j] + c.C2 * (g[j] * g[j]);
    if constexpr (FORM == kStandard) {
      M[j] = mm;
      V[j] = vv;
      MH[j] = mm / c.BC1;
      VH[j] = vv / c.BC2;
    } else {
      M[j] = mm / c.BC1;
      V[j] = vv / c.BC2;
      MH[j] = M[j];
      VH[j] = V[j];
    }
  }
}
__device__ __forceinline__ void adam_weights8(const Consts& c, const float (&MH)[8],
                                              const float (&VH)[8], float (&W)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = __builtin_sqrtf(VH[j]) + c.EPS;
    const float u = MH[j] / d;
    W[j] = W[j] - c.LR * u;
  }
}

template <class T>
__device__ __forceinline__ T* uniform_t(T* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  // Rebuilt as a global-memory pointer: a pointer that comes out of LDS is
  // otherwise generic, and generic (flat) accesses make every wait a full
  // drain (flat loads may return out of order), which serialises the loads.
  using GT = __attribute__((address_space(1))) T;
  return (T*)reinterpret_cast<GT*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ const uint16_t* uniform(const uint16_t* p) { return uniform_t(p); }

// Gradient pointer sources: kernel arguments, or a table staged in LDS.  The
// pointer of a rank is the same for the whole workgroup (uniform).
template <int PMAX>
struct GradArgs {
  const uint16_t* g[PMAX];
};

// The pointer table is the kernel's first argument, so it sits at offset 0 of
// the kernel-argument segment; reading it there (scalar loads from the
// constant address space) avoids any private copy of the by-value table.
typedef const uint16_t* const __attribute__((address_space(4)))* KernargTable;

struct ArgGrads {
  KernargTable t;
  __device__ __forceinline__ const uint16_t* get(int r) const { return t[r]; }
};

__device__ __forceinline__ ArgGrads kernarg_grads() {
  return ArgGrads{(KernargTable)(__builtin_amdgcn_kernarg_segment_ptr())};
}

// The rank pointers from a device array when the launch has one (more ranks
// than fit in the kernel arguments), else from the kernel arguments.  Both
// are read-only for the whole launch, so both are read with scalar loads.
__device__ __forceinline__ ArgGrads rank_grads(const void* table) {
  return table ? ArgGrads{reinterpret_cast<KernargTable>(reinterpret_cast<uintptr_t>(table))}
               : kernarg_grads();
}

struct LdsGrads {
  const uint16_t* const* s;
  __device__ __forceinline__ const uint16_t* get(int r) const { return uniform(s[r]); }
};

constexpr int kRankBatch = 8;
// Waves per SIMD (workgroups per CU) of the small-shard kernel.
constexpr int kSmallWaves = 3;

// ---- the lane maps -------------------------------------------------------
// Byte offsets of one lane inside a group, added to a workgroup-uniform base
// at the group's first element.  Full groups: quad A of 16-bit arrays at
// q16 (quad B at q16 + 512), of fp32 arrays at q32 (quad B at q32 + 1024).
// The partial group: 8 consecutive elements at c16 / c32.
struct Lanes {
  uint32_t q16, q32, c16, c32;
};

__device__ __forceinline__ Lanes lanes() {
  const uint32_t wv = threadIdx.x >> 6, l = threadIdx.x & 63u;
  const uint32_t q = wv * 512u + 4u * l;
  return Lanes{2u * q, 4u * q, 16u * threadIdx.x, 32u * threadIdx.x};
}

// The 8 gradients of a lane in a full group: quads A and B.
struct G8 {
  u32x2 a, b;
};

// Non-temporal loads (each byte is read once per step; plain gradient loads
// cost 10% on the 7.5B-parameter, 64-rank shard).
__device__ __forceinline__ G8 ld_g8(const uint16_t* base, const Lanes& L) {
  const char* p = reinterpret_cast<const char*>(base);
  return G8{__builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + L.q16)),
            __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + L.q16 + 512u))};
}
__device__ __forceinline__ u32x4 ld_grad(const uint16_t* base, uint32_t off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + off));
}
__device__ __forceinline__ f32x4 ld_f32x4(const float* base, uint32_t off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(base) + off));
}
// The fp32 state loads and all stores are non-temporal too: each byte of w,
// m, v and the working copy is read once and written once per step.
__device__ __forceinline__ void st_f32x4(float* base, uint32_t off, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(reinterpret_cast<char*>(base) + off));
}
__device__ __forceinline__ void st_u16x8(uint16_t* base, uint32_t off, u32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + off));
}
__device__ __forceinline__ void st_u16x4(uint16_t* base, uint32_t off, u32x2 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(reinterpret_cast<char*>(base) + off));
}

// The 8 fp32 values of a lane (quad A then quad B), loaded / stored.
__device__ __forceinline__ void ld_f8(const float* base, const Lanes& L, float (&x)[kVec]) {
  const f32x4 a = ld_f32x4(base, L.q32), b = ld_f32x4(base, L.q32 + 1024u);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void st_f8(float* base, const Lanes& L, const float (&x)[kVec]) {
  st_f32x4(base, L.q32, f32x4{x[0], x[1], x[2], x[3]});
  st_f32x4(base, L.q32 + 1024u, f32x4{x[4], x[5], x[6], x[7]});
}
template <int DT>
__device__ __forceinline__ void st_h8(uint16_t* base, const Lanes& L, const float (&x)[kVec]) {
  st_u16x4(base, L.q16, u32x2{narrow2<DT>(x[0], x[1]), narrow2<DT>(x[2], x[3])});
  st_u16x4(base, L.q16 + 512u, u32x2{narrow2<DT>(x[4], x[5]), narrow2<DT>(x[6], x[7])});
}

// Whole-line fp32 stores from the contiguous map.  Lane l of a wave holds 8
// consecutive values, its low quad X_l and high quad Y_l, 32 bytes at 32 l.
// Stored as they lie, each store instruction would write half of every
// 128-byte line it touches.  v_permlane32_swap trades lanes 32..63's X for
// lanes 0..31's Y, so the first instruction writes the wave's first KiB (X_l
// and Y_l of lanes 0..31) and the second its second KiB.  All 64 lanes must
// be active.
struct SwapOffs {
  uint32_t a, b;  // byte offsets of this lane's two stores
};
__device__ __forceinline__ SwapOffs swap_offs(uint32_t c32) {
  const bool hi = (threadIdx.x & 32u) != 0;
  // lane l >= 32 stores Y_{l-32} at 32 (l - 32) + 16, then its own Y_l;
  // lane l < 32 its own X_l, then X_{l+32} at 32 (l + 32)
  return SwapOffs{hi ? c32 - 1008u : c32, hi ? c32 + 16u : c32 + 1024u};
}
__device__ __forceinline__ void st_f32x8_lines(float* base, const SwapOffs& o,
                                               const float (&x)[kVec]) {
  f32x4 a, b;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // lanes 0..31 keep x[d] in a and receive lanes 32..63's x[d] in b;
    // lanes 32..63 receive lanes 0..31's x[4 + d] in a and keep x[4 + d] in b
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[d]),
                                                    __float_as_uint(x[4 + d]), false, false);
    a[d] = __uint_as_float(r[0]);
    b[d] = __uint_as_float(r[1]);
  }
  st_f32x4(base, o.a, a);
  st_f32x4(base, o.b, b);
}

// Which optimizer state a form reads and writes: Adam both moments, momentum
// SGD the momentum only, plain SGD neither (those pointers may be null).
template <int FORM>
constexpr bool kUsesM = FORM != kSgd;
template <int FORM>
constexpr bool kUsesV = FORM == kStandard || FORM == kPage1Literal;

template <bool USE>
__device__ __forceinline__ f32x4 ld_state(const float* base, uint32_t off) {
  if constexpr (USE) {
    return ld_f32x4(base, off);
  } else {
    return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
}
template <bool USE>
__device__ __forceinline__ void st_state(float* base, uint32_t off, f32x4 x) {
  if constexpr (USE) st_f32x4(base, off, x);
}
template <bool USE>
__device__ __forceinline__ float ld_state1(const float* p) {
  if constexpr (USE) {
    return *p;
  } else {
    return 0.0f;
  }
}
template <bool USE>
__device__ __forceinline__ void st_state1(float* p, float x) {
  if constexpr (USE) *p = x;
}

// ---- gradient folds --------------------------------------------------------
// Full groups (G8): acc[0..3] from quad A, acc[4..7] from quad B.
template <int GDT>
__device__ __forceinline__ void init8(float (&acc)[kVec], const G8& q) {
  acc[0] = widen_lo<GDT>(q.a.x); acc[1] = widen_hi<GDT>(q.a.x);
  acc[2] = widen_lo<GDT>(q.a.y); acc[3] = widen_hi<GDT>(q.a.y);
  acc[4] = widen_lo<GDT>(q.b.x); acc[5] = widen_hi<GDT>(q.b.x);
  acc[6] = widen_lo<GDT>(q.b.y); acc[7] = widen_hi<GDT>(q.b.y);
}
template <int GDT>
__device__ __forceinline__ void fold8(float (&acc)[kVec], const G8& q) {
  acc[0] = acc[0] + widen_lo<GDT>(q.a.x); acc[1] = acc[1] + widen_hi<GDT>(q.a.x);
  acc[2] = acc[2] + widen_lo<GDT>(q.a.y); acc[3] = acc[3] + widen_hi<GDT>(q.a.y);
  acc[4] = acc[4] + widen_lo<GDT>(q.b.x); acc[5] = acc[5] + widen_hi<GDT>(q.b.x);
  acc[6] = acc[6] + widen_lo<GDT>(q.b.y); acc[7] = acc[7] + widen_hi<GDT>(q.b.y);
}
// The partial group (u32x4): 8 consecutive elements.
template <int GDT>
__device__ __forceinline__ void init8(float (&acc)[kVec], const u32x4& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] = widen_lo<GDT>(q[j]);
    acc[2 * j + 1] = widen_hi<GDT>(q[j]);
  }
}
template <int GDT>
__device__ __forceinline__ void fold8(float (&acc)[kVec], const u32x4& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] = acc[2 * j] + widen_lo<GDT>(q[j]);
    acc[2 * j + 1] = acc[2 * j + 1] + widen_hi<GDT>(q[j]);
  }
}

// One lane's gradient vector of a group in either map.
template <bool FULL>
using GVec = std::conditional_t<FULL, G8, u32x4>;

template <bool FULL>
__device__ __forceinline__ GVec<FULL> ld_gvec(const uint16_t* base, const Lanes& L) {
  if constexpr (FULL) {
    return ld_g8(base, L);
  } else {
    return ld_grad(base, L.c16);
  }
}

// The loads of ranks r0 .. r0+B-1 for one lane's 8 elements of the group at
// e0, issued together (the scheduling barriers keep the compiler from sinking
// each load next to its use, which would leave one load in flight), then
// added in rank order.  CONT: acc already holds the fp32 sums of earlier
// ranks, so rank r0 = 0 of this call is added to it rather than starting the
// fold.
template <int B, int GDT, bool FULL, bool CONT = false, class Grads>
__device__ __forceinline__ void fold_batch(const Grads& gr, int r0, int64_t e0, const Lanes& L,
                                           float (&acc)[kVec]) {
  GVec<FULL> q[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    q[b] = ld_gvec<FULL>(gr.get(r0 + b) + e0, L);
    __builtin_amdgcn_sched_barrier(0);  // issued in rank order
  }
  if (!CONT && r0 == 0) {
    init8<GDT>(acc, q[0]);
  } else {
    fold8<GDT>(acc, q[0]);
  }
#pragma unroll
  for (int b = 1; b < B; ++b) fold8<GDT>(acc, q[b]);
  __builtin_amdgcn_sched_barrier(0);
}

// acc[j] = sum over ranks r = 0..p-1, in that order, of the lane's element
// j of the group at e0, in batches of 16 ranks, then one batch each of 8, 4,
// 2, 1 for the rest: at most 4 + P/16 memory round trips.
template <int GDT, bool FULL, bool CONT = false, int MAXB = 16, class Grads>
__device__ __forceinline__ void sum_ranks8(const Grads& gr, int p, int64_t e0, const Lanes& L,
                                           float (&acc)[kVec]) {
  int r0 = 0;
  if constexpr (MAXB >= 16) {
    for (; r0 + 16 <= p; r0 += 16) fold_batch<16, GDT, FULL, CONT>(gr, r0, e0, L, acc);
    if (r0 + 8 <= p) {
      fold_batch<8, GDT, FULL, CONT>(gr, r0, e0, L, acc);
      r0 += 8;
    }
  } else if constexpr (MAXB == 8) {
    for (; r0 + 8 <= p; r0 += 8) fold_batch<8, GDT, FULL, CONT>(gr, r0, e0, L, acc);
  } else {
    for (; r0 + 4 <= p; r0 += 4) fold_batch<4, GDT, FULL, CONT>(gr, r0, e0, L, acc);
  }
  if (r0 + 4 <= p) {
    fold_batch<4, GDT, FULL, CONT>(gr, r0, e0, L, acc);
    r0 += 4;
  }
  if (r0 + 2 <= p) {
    fold_batch<2, GDT, FULL, CONT>(gr, r0, e0, L, acc);
    r0 += 2;
  }
  if (r0 < p) fold_batch<1, GDT, FULL, CONT>(gr, r0, e0, L, acc);
}

// Two groups (at e0 and e1, in either map): both groups' loads of ranks
// r0 .. r0+B-1 in flight together, then the rank-order adds.
template <int B, int GDT, bool FULL, bool CONT = false, class Grads>
__device__ __forceinline__ void fold_batch2(const Grads& gr, int r0, int64_t e0, int64_t e1,
                                            const Lanes& L, float (&a)[kVec], float (&b)[kVec]) {
  GVec<FULL> qa[B], qb[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    qa[i] = ld_gvec<FULL>(gr.get(r0 + i) + e0, L);
    qb[i] = ld_gvec<FULL>(gr.get(r0 + i) + e1, L);
    if constexpr (FULL) __builtin_amdgcn_sched_barrier(0);  // issued in rank order
  }
  __builtin_amdgcn_sched_barrier(0);
  if (!CONT && r0 == 0) {
    init8<GDT>(a, qa[0]);
    init8<GDT>(b, qb[0]);
  } else {
    fold8<GDT>(a, qa[0]);
    fold8<GDT>(b, qb[0]);
  }
#pragma unroll
  for (int i = 1; i < B; ++i) {
    fold8<GDT>(a, qa[i]);
    fold8<GDT>(b, qb[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// MAXB caps the rank batch (16, 8 or 4): the small-shard kernel, with three
// waves per SIMD, takes 4; the chunk table's rest 8.
template <int GDT, int MAXB = 16, bool FULL = true, bool CONT = false, class Grads>
__device__ __forceinline__ void sum_ranks8x2(const Grads& gr, int p, int64_t e0, int64_t e1,
                                             const Lanes& L, float (&a)[kVec],
                                             float (&b)[kVec]) {
  int r0 = 0;
  if constexpr (MAXB >= 16) {
    for (; r0 + 16 <= p; r0 += 16) fold_batch2<16, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
    if (r0 + 8 <= p) {
      fold_batch2<8, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
      r0 += 8;
    }
  } else if constexpr (MAXB == 8) {
    for (; r0 + 8 <= p; r0 += 8) fold_batch2<8, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
  } else {
    for (; r0 + 4 <= p; r0 += 4) fold_batch2<4, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
  }
  if (r0 + 4 <= p) {
    fold_batch2<4, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
    r0 += 4;
  }
  if (r0 + 2 <= p) {
    fold_batch2<2, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
    r0 += 2;
  }
  if (r0 < p) fold_batch2<1, GDT, FULL, CONT>(gr, r0, e0, e1, L, a, b);
}

// Rank-order mean of one element, kRankBatch loads in flight per batch.
template <int GDT, class Grads>
__device__ __forceinline__ float mean1(const Grads& gr, int p, int64_t e, float PF) {
  float s = 0.0f;
  int r0 = 0;
  for (; r0 + kRankBatch <= p; r0 += kRankBatch) {
    uint16_t q[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) q[b] = gr.get(r0 + b)[e];
    __builtin_amdgcn_sched_barrier(0);
    s = r0 == 0 ? widen1<GDT>(q[0]) : s + widen1<GDT>(q[0]);
#pragma unroll
    for (int b = 1; b < kRankBatch; ++b) s = s + widen1<GDT>(q[b]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; r0 < p; ++r0) {
    const float x = widen1<GDT>(gr.get(r0)[e]);
    s = r0 == 0 ? x : s + x;
  }
  return s / PF;
}

// ---- the update of a group -------------------------------------------------
// The state of one full group at e0: its loads are issued first
// (load_group), then Adam and the downcast (apply_group) use them.  x: the
// rank sums (divided by P here) or, DIVIDE false, the mean.
struct GroupState {
  f32x4 w0, w1, m0, m1, v0, v1;
};

template <int FORM>
__device__ __forceinline__ GroupState load_group(const Lanes& L, const float* w, const float* m,
                                                 const float* v, int64_t e0) {
  return GroupState{ld_f32x4(w + e0, L.q32), ld_f32x4(w + e0, L.q32 + 1024u),
                    ld_state<kUsesM<FORM>>(m + e0, L.q32),
                    ld_state<kUsesM<FORM>>(m + e0, L.q32 + 1024u),
                    ld_state<kUsesV<FORM>>(v + e0, L.q32),
                    ld_state<kUsesV<FORM>>(v + e0, L.q32 + 1024u)};
}

template <int PDT, int FORM, bool DIVIDE = true, bool PARAM = true>
__device__ __forceinline__ void apply_group(const Consts& c, const Lanes& L, const GroupState& q,
                                            const float (&x)[kVec], float* w, float* m,
                                            float* v, uint16_t* par, int64_t e0) {
  float W[kVec] = {q.w0.x, q.w0.y, q.w0.z, q.w0.w, q.w1.x, q.w1.y, q.w1.z, q.w1.w};
  float M[kVec] = {q.m0.x, q.m0.y, q.m0.z, q.m0.w, q.m1.x, q.m1.y, q.m1.z, q.m1.w};
  float V[kVec] = {q.v0.x, q.v0.y, q.v0.z, q.v0.w, q.v1.x, q.v1.y, q.v1.z, q.v1.w};
  float* wb = w + e0;
  float* mb = m + e0;
  float* vb = v + e0;
  if constexpr (FORM == kStandard || FORM == kPage1Literal) {
    float g[kVec], MH[kVec], VH[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) g[j] = DIVIDE ? x[j] / c.PF : x[j];
    adam_moments8<FORM>(c, g, M, V, MH, VH);
    st_f8(mb, L, M);
    st_f8(vb, L, V);
    __builtin_amdgcn_sched_barrier(0);  // the moments go out before the weight arithmetic
    adam_weights8(c, MH, VH, W);
    st_f8(wb, L, W);
  } else {
#pragma unroll
    for (int j = 0; j < kVec; ++j) adam1<FORM>(c, DIVIDE ? x[j] / c.PF : x[j], W[j], M[j], V[j]);
    st_f8(wb, L, W);
    if constexpr (kUsesM<FORM>) st_f8(mb, L, M);
  }
  if constexpr (PARAM) st_h8<PDT>(par + e0, L, W);
}

// apply_group for the Adam forms with the next group's state loads (into
// `next`, when has_next) issued between the moment stores and the weight
// arithmetic, so they are in flight during the divisions (the chunk table's
// update phase: 0.4% on the 8-rank Llama-3-8B shard; the update from a
// stored mean, which also loads its gradient, was 0.8% slower this way).
template <int PDT, int FORM, bool DIVIDE = true, bool PARAM = true>
__device__ __forceinline__ void apply_group_pipe(const Consts& c, const Lanes& L,
                                                 const GroupState& q, const float (&x)[kVec],
                                                 float* w, float* m, float* v, uint16_t* par,
                                                 int64_t e0, bool has_next, GroupState& next) {
  float W[kVec] = {q.w0.x, q.w0.y, q.w0.z, q.w0.w, q.w1.x, q.w1.y, q.w1.z, q.w1.w};
  float M[kVec] = {q.m0.x, q.m0.y, q.m0.z, q.m0.w, q.m1.x, q.m1.y, q.m1.z, q.m1.w};
  float V[kVec] = {q.v0.x, q.v0.y, q.v0.z, q.v0.w, q.v1.x, q.v1.y, q.v1.z, q.v1.w};
  float g[kVec], MH[kVec], VH[kVec];
#pragma unroll
  for (int j = 0; j < kVec; ++j) g[j] = DIVIDE ? x[j] / c.PF : x[j];
  adam_moments8<FORM>(c, g, M, V, MH, VH);
  st_f8(m + e0, L, M);
  st_f8(v + e0, L, V);
  __builtin_amdgcn_sched_barrier(0);
  if (has_next) next = load_group<FORM>(L, w, m, v, e0 + kGroup);
  __builtin_amdgcn_sched_barrier(0);
  adam_weights8(c, MH, VH, W);
  st_f8(w + e0, L, W);
  if constexpr (PARAM) st_h8<PDT>(par + e0, L, W);
  __builtin_amdgcn_sched_barrier(0);
}

// The partial group: Adam + downcast of a lane's 8 consecutive elements at
// e0 + 8 * lane.  x holds the fp32 gradient mean, or (DIVIDE) the rank sums,
// divided by P here.
template <int PDT, int FORM, bool PARAM = true, bool DIVIDE = false>
__device__ __forceinline__ void adam8(const Consts& c, const float (&x)[kVec], float* w, float* m,
                                      float* v, uint16_t* par, int64_t e0, const Lanes& L) {
  float* wb = w + e0;
  float* mb = m + e0;
  float* vb = v + e0;
  const uint32_t lane32 = L.c32;
  const f32x4 w0 = ld_f32x4(wb, lane32), w1 = ld_f32x4(wb, lane32 + 16);
  const f32x4 m0 = ld_state<kUsesM<FORM>>(mb, lane32), m1 = ld_state<kUsesM<FORM>>(mb, lane32 + 16);
  const f32x4 v0 = ld_state<kUsesV<FORM>>(vb, lane32), v1 = ld_state<kUsesV<FORM>>(vb, lane32 + 16);
  float W[kVec] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float M[kVec] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
  float V[kVec] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    if constexpr (DIVIDE) {
      adam1<FORM>(c, x[j] / c.PF, W[j], M[j], V[j]);
    } else {
      adam1<FORM>(c, x[j], W[j], M[j], V[j]);
    }
  }
  st_f32x4(wb, lane32, f32x4{W[0], W[1], W[2], W[3]});
  st_f32x4(wb, lane32 + 16, f32x4{W[4], W[5], W[6], W[7]});
  st_state<kUsesM<FORM>>(mb, lane32, f32x4{M[0], M[1], M[2], M[3]});
  st_state<kUsesM<FORM>>(mb, lane32 + 16, f32x4{M[4], M[5], M[6], M[7]});
  st_state<kUsesV<FORM>>(vb, lane32, f32x4{V[0], V[1], V[2], V[3]});
  st_state<kUsesV<FORM>>(vb, lane32 + 16, f32x4{V[4], V[5], V[6], V[7]});
  if constexpr (PARAM)
    st_u16x8(par + e0, L.c16,
             u32x4{narrow2<PDT>(W[0], W[1]), narrow2<PDT>(W[2], W[3]), narrow2<PDT>(W[4], W[5]),
                   narrow2<PDT>(W[6], W[7])});
}

// Two full groups: both groups' state loads issued together, then the
// arithmetic and stores of each.
template <int PDT, int FORM, bool DIVIDE = true, bool PARAM = true>
__device__ __forceinline__ void adam8x2(const Consts& c, const float (&a)[kVec],
                                        const float (&b)[kVec], float* w, float* m, float* v,
                                        uint16_t* par, int64_t e0, int64_t e1, const Lanes& L) {
  const GroupState qa = load_group<FORM>(L, w, m, v, e0);
  const GroupState qb = load_group<FORM>(L, w, m, v, e1);
  __builtin_amdgcn_sched_barrier(0);
  apply_group<PDT, FORM, DIVIDE, PARAM>(c, L, qa, a, w, m, v, par, e0);
  apply_group<PDT, FORM, DIVIDE, PARAM>(c, L, qb, b, w, m, v, par, e1);
}

// ---- the rest of a range ---------------------------------------------------
// What whole kGroupsMax chunks do not cover, from vector left0 on (vectors of
// 8 elements after the head h): its full groups in pieces of two, then one
// full group if their count is odd, then the partial group, dealt one item
// per block.  Whole chunks go round-robin, so blocks nfull % nblk, ... have
// one chunk fewer than the rest: the items are dealt out starting there, then
// the scalar head and tail elements go to the next block.  All read the
// ranks in batches (several loads in flight per lane): an item is too small
// to batch over groups, and one load at a time would cost a full memory
// round trip per rank.
struct RestPlan {
  int64_t first_full;  // vector of the first full group
  int64_t nfg;         // full groups
  int64_t part;        // vectors in the partial group (0..kBlock-1)
  int64_t npairs;      // two-group pieces
  int64_t nitems;      // pieces, the odd full group, the partial group
  int64_t me;          // this block's place in the deal
};

__device__ __forceinline__ RestPlan rest_plan(int64_t nvec, int64_t left0, int64_t nfull,
                                              int64_t blk, int64_t nblk) {
  RestPlan r;
  r.first_full = left0;
  r.nfg = (nvec - left0) / kBlock;
  r.part = (nvec - left0) % kBlock;
  r.npairs = r.nfg / 2;
  r.nitems = r.npairs + (r.nfg & 1) + (r.part > 0 ? 1 : 0);
  const int64_t first = nfull % nblk;
  r.me = (blk - first + nblk) % nblk;
  return r;
}

// Full groups in the full-group lane map, the partial group in the
// contiguous one; MAXB caps the rank batch.
template <int GDT, int PDT, int FORM, int MAXB = 16, class Grads>
__device__ __forceinline__ void fused_rest(const Grads& gr, int p, float* __restrict__ w,
                                           float* __restrict__ m, float* __restrict__ v,
                                           uint16_t* __restrict__ par, int64_t len, int64_t h,
                                           int64_t nvec, int64_t left0, int64_t nfull,
                                           const Consts& c, int64_t blk, int64_t nblk,
                                           const Lanes& L) {
  const int tid = threadIdx.x;
  const RestPlan R = rest_plan(nvec, left0, nfull, blk, nblk);
  for (int64_t i = R.me; i < R.nitems; i += nblk) {
    if (i < R.npairs) {
      const int64_t e0 = h + (R.first_full + 2 * i * kBlock) * kVec;
      const int64_t e1 = e0 + kGroup;
      float a[kVec], b[kVec];
      sum_ranks8x2<GDT, MAXB>(gr, p, e0, e1, L, a, b);
      adam8x2<PDT, FORM>(c, a, b, w, m, v, par, e0, e1, L);
    } else if (i == R.npairs && (R.nfg & 1)) {
      const int64_t e0 = h + (R.first_full + 2 * R.npairs * kBlock) * kVec;
      float g[kVec];
      sum_ranks8<GDT, true, false, MAXB>(gr, p, e0, L, g);
      const GroupState q = load_group<FORM>(L, w, m, v, e0);
      apply_group<PDT, FORM>(c, L, q, g, w, m, v, par, e0);
    } else if (tid < R.part) {
      const int64_t e0 = h + (R.first_full + R.nfg * kBlock) * kVec;
      float g[kVec];
      sum_ranks8<GDT, false, false, MAXB>(gr, p, e0, L, g);
      adam8<PDT, FORM, true, true>(c, g, w, m, v, par, e0, L);
    }
  }
  if (R.me == R.nitems % nblk) {
    const int64_t t0 = h + nvec * kVec;
    const int64_t nsc = h + (len - t0);
    for (int64_t i = tid; i < nsc; i += kBlock) {
      const int64_t e = i < h ? i : t0 + (i - h);
      const float g = mean1<GDT>(gr, p, e, c.PF);
      float W = w[e], M = ld_state1<kUsesM<FORM>>(m + e), V = ld_state1<kUsesV<FORM>>(v + e);
      adam1<FORM>(c, g, W, M, V);
      w[e] = W;
      st_state1<kUsesM<FORM>>(m + e, M);
      st_state1<kUsesV<FORM>>(v + e, V);
      par[e] = narrow1<PDT>(W);
    }
  }
}

// A range of elements of one step: gradient pointers, fp32 state and working
// copy at the range's first element, the vector-group head, and its blocks.
template <class Grads>
struct Range {
  Grads gr;
  float* w;
  float* m;
  float* v;
  uint16_t* par;
  int64_t len;
  int head;
  int64_t blk, nblk;
};

// The chunk table of the multi-tensor step: one item per entry, one block
// each.  The block stages the entry's P gradient pointers and its piece
// descriptor in LDS.
struct TableSrc {
  const MtPiece* pieces;
  const uint16_t* const* gptrs;  // npieces * p pointers, piece-major
  const MtChunk* chunks;
  int64_t nchunks;
  int64_t chunk_elems;
  int p;
  __device__ __forceinline__ int64_t first() const { return blockIdx.x; }
  __device__ __forceinline__ int64_t count() const { return nchunks; }
  __device__ __forceinline__ int64_t stride() const { return gridDim.x; }
  __device__ __forceinline__ Range<LdsGrads> open(int64_t ch) const {
    __shared__ const uint16_t* s_g[kMaxP];
    __shared__ MtPiece s_piece;
    const MtChunk cc = chunks[ch];
    __syncthreads();  // the previous entry's readers of s_g / s_piece are done
    for (int r = threadIdx.x; r < p; r += kBlock)
      s_g[r] = gptrs[static_cast<int64_t>(cc.piece) * p + r] + cc.start;
    if (threadIdx.x == 0) s_piece = pieces[cc.piece];
    __syncthreads();
    const int64_t rest = s_piece.len - cc.start;
    const int64_t len = rest < chunk_elems ? rest : chunk_elems;
    const int head = (s_piece.head - static_cast<int>(cc.start & 7)) & 7;
    return Range<LdsGrads>{LdsGrads{s_g},
                           uniform_t(s_piece.w) + cc.start,
                           uniform_t(s_piece.m) + cc.start,
                           uniform_t(s_piece.v) + cc.start,
                           uniform_t(s_piece.param) + cc.start,
                           len, head, 0, 1};
  }
};

// Whole chunks used out of nfull: whole rounds over the nblk blocks, plus the
// last partial round when it fills at least half of the blocks.  A smaller
// last round goes to the rank-batched pieces instead, which every block
// shares (a shard of 109 chunks on 256 blocks would otherwise leave 147 CUs
// idle while 109 run one chunk each).
__device__ __forceinline__ int64_t whole_chunks(int64_t nfull, int64_t nblk) {
  const int64_t rem = nfull % nblk;
  return 2 * rem >= nblk ? nfull : nfull - rem;
}

template <int V>
using IC = std::integral_constant<int, V>;

template <class F>
void with_dt(int dt, F&& f) {
  if (dt == kF16) f(IC<kF16>{}); else f(IC<kBF16>{});
}

template <class F>
void with_form(int form, F&& f) {
  switch (form) {
    case kStandard: f(IC<kStandard>{}); break;
    case kPage1Literal: f(IC<kPage1Literal>{}); break;
    case kSgd: f(IC<kSgd>{}); break;
    default: f(IC<kSgdMomentum>{}); break;
  }
}

// Kernel-argument pointer tables of 64 or kKernargP ranks.
template <class F>
void with_pmax(int p, F&& f) {
  if (p <= 64) f(IC<64>{});
  else f(IC<kKernargP>{});
}

}  // namespace
}  // namespace zs

// zs_kernels.hip -- gfx950 kernels of libzshard.
//
// The per-shard step is pure streaming: per element it reads P 16-bit
// gradients and the fp32 (w, m, v), writes (w, m, v) and one 16-bit working
// copy, and does O(P) flops.  At about 0.5 flop/byte it sits far below the
// fp32 vector ridge of the chip: the design goal is HBM bandwidth.
//  - Each lane owns groups of 8 consecutive elements: one 16-byte load per
//    gradient rank, two per fp32 state array, one 16-byte store of the
//    16-bit copy.  Addresses are a workgroup-uniform base (SGPRs) plus a
//    fixed per-lane byte offset, so a wave64 access is 1 KiB contiguous.
//  - The loads of 8 ranks are issued back to back (scheduling barriers stop
//    the compiler from sinking each load next to its use); the adds then run
//    in rank order 0..P-1 as data arrives: a left fold, one fp32 rounding per
//    add, exactly the oracle's order.  Gradient loads are non-temporal.
//  - Phase separation: HBM on this part streams reads alone far faster than
//    reads with any writes mixed in.  A workgroup therefore sums the
//    gradients of a whole chunk (up to 28 groups per lane, held in registers
//    with one wave per SIMD) before it touches w, m, v and the working copy,
//    so reads and writes reach the memory in separate stretches.
//  - One workgroup per CU.  Full chunks (28 groups per lane) go round-robin;
//    the remainder is split evenly and run in 7-group chunks, so the
//    workgroups finish together.
//  - No MFMA and no LDS on the single-tensor path (nothing is reused); the
//    multi-tensor path stages one chunk's descriptors in LDS.
// Arithmetic (rank-order fp32 mean, Adam moments, bias correction, update,
// round-to-nearest-even downcast) follows the pages cited in zshard.h:
// [DP-III] §(一) (Adam), §(四) steps 2-4; [EAI19] 通信原语 All-Reduce (mean);
// [ZP] 核心原理 and [ZA] §2.2 (fp32 update then the 16-bit working copy).
// Compiled with -ffp-contract=off and the pragma below: no FMA contraction;
// division and sqrt are the correctly rounded HIP defaults; fp32 denormals
// are kept.

#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "zs_internal.h"

#pragma clang fp contract(off)

namespace zs {
namespace {

// 16-byte vectors that may sit at any 2-byte (u16) or 4-byte (fp32) address:
// gfx950 runs with unaligned access enabled, so these still compile to
// global_load_dwordx4 / global_store_dwordx4.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4 __attribute__((ext_vector_type(4), aligned(4)));

// Groups of 8 elements per lane whose rank sums are held in registers across
// the read-only phase of a chunk (28 x 8 fp32 values per lane: with one
// wave per SIMD the kernel may use the whole 512-entry register file).
constexpr int kGroupsMax = 28;

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

// One Adam update of one element, in place.  Operation order: the two moment
// products rounded, their sum rounded; bias correction by division;
// d = sqrt(v_hat) + eps; u = m_hat / d; w - lr*u.
template <int FORM>
__device__ __forceinline__ void adam1(const Consts& c, float g, float& w, float& m, float& v) {
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

__device__ __forceinline__ const uint16_t* uniform(const uint16_t* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return reinterpret_cast<const uint16_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <class T>
__device__ __forceinline__ T* uniform_t(T* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

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

struct LdsGrads {
  const uint16_t* const* s;
  __device__ __forceinline__ const uint16_t* get(int r) const { return uniform(s[r]); }
};

constexpr int kRankBatch = 8;

// 16-byte loads at a workgroup-uniform base plus a per-lane byte offset; the
// gradient loads are non-temporal (each byte is read once per step).
__device__ __forceinline__ u32x4 ld_grad(const uint16_t* base, uint32_t off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + off));
}
__device__ __forceinline__ u32x4 ld_u16x8(const uint16_t* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + off);
}
__device__ __forceinline__ f32x4 ld_f32x4(const float* base, uint32_t off) {
  return *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(base) + off);
}
__device__ __forceinline__ void st_f32x4(float* base, uint32_t off, f32x4 x) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(base) + off) = x;
}
__device__ __forceinline__ void st_u16x8(uint16_t* base, uint32_t off, u32x4 x) {
  *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + off) = x;
}

template <int GDT>
__device__ __forceinline__ void fold8(float (&acc)[kVec], const u32x4& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] = acc[2 * j] + widen_lo<GDT>(q[j]);
    acc[2 * j + 1] = acc[2 * j + 1] + widen_hi<GDT>(q[j]);
  }
}

template <int GDT>
__device__ __forceinline__ void init8(float (&acc)[kVec], const u32x4& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] = widen_lo<GDT>(q[j]);
    acc[2 * j + 1] = widen_hi<GDT>(q[j]);
  }
}

// acc[j] = sum over ranks r = 0..p-1, in that order, of widen(grad_r[e0 + 8*lane + j]).
// The loads of a batch of 8 ranks are issued together (the scheduling
// barriers keep the compiler from sinking each load next to its use, which
// would leave one load in flight per wave); the adds then run in rank order
// as the data arrives.  e0 is workgroup-uniform, lane16 = 16 * lane.
template <int GDT, class Grads>
__device__ __forceinline__ void sum_ranks8(const Grads& gr, int p, int64_t e0, uint32_t lane16,
                                           float (&acc)[kVec]) {
  int r0 = 0;
  for (; r0 + kRankBatch <= p; r0 += kRankBatch) {
    u32x4 q[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) q[b] = ld_grad(gr.get(r0 + b) + e0, lane16);
    __builtin_amdgcn_sched_barrier(0);
    if (r0 == 0) {
      init8<GDT>(acc, q[0]);
    } else {
      fold8<GDT>(acc, q[0]);
    }
#pragma unroll
    for (int b = 1; b < kRankBatch; ++b) fold8<GDT>(acc, q[b]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (r0 + kRankBatch / 2 <= p) {
    u32x4 q[kRankBatch / 2];
#pragma unroll
    for (int b = 0; b < kRankBatch / 2; ++b) q[b] = ld_grad(gr.get(r0 + b) + e0, lane16);
    __builtin_amdgcn_sched_barrier(0);
    if (r0 == 0) {
      init8<GDT>(acc, q[0]);
    } else {
      fold8<GDT>(acc, q[0]);
    }
#pragma unroll
    for (int b = 1; b < kRankBatch / 2; ++b) fold8<GDT>(acc, q[b]);
    __builtin_amdgcn_sched_barrier(0);
    r0 += kRankBatch / 2;
  }
  for (; r0 < p; ++r0) {
    const u32x4 q = ld_grad(gr.get(r0) + e0, lane16);
    if (r0 == 0) {
      init8<GDT>(acc, q);
    } else {
      fold8<GDT>(acc, q);
    }
  }
}

template <int GDT, class Grads>
__device__ __forceinline__ float mean1(const Grads& gr, int p, int64_t e, float PF) {
  float s = widen1<GDT>(gr.get(0)[e]);
  for (int r = 1; r < p; ++r) s = s + widen1<GDT>(gr.get(r)[e]);
  return s / PF;
}

// Adam + downcast of one lane's 8 elements at uniform element e0, from the
// fp32 gradient mean g.
template <int PDT, int FORM, bool PARAM = true>
__device__ __forceinline__ void adam8(const Consts& c, const float (&g)[kVec], float* w,
                                      float* m, float* v, uint16_t* par, int64_t e0,
                                      uint32_t lane16, uint32_t lane32) {
  float* wb = w + e0;
  float* mb = m + e0;
  float* vb = v + e0;
  const f32x4 w0 = ld_f32x4(wb, lane32), w1 = ld_f32x4(wb, lane32 + 16);
  const f32x4 m0 = ld_f32x4(mb, lane32), m1 = ld_f32x4(mb, lane32 + 16);
  const f32x4 v0 = ld_f32x4(vb, lane32), v1 = ld_f32x4(vb, lane32 + 16);
  float W[kVec] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float M[kVec] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
  float V[kVec] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int j = 0; j < kVec; ++j) adam1<FORM>(c, g[j], W[j], M[j], V[j]);
  st_f32x4(wb, lane32, f32x4{W[0], W[1], W[2], W[3]});
  st_f32x4(wb, lane32 + 16, f32x4{W[4], W[5], W[6], W[7]});
  st_f32x4(mb, lane32, f32x4{M[0], M[1], M[2], M[3]});
  st_f32x4(mb, lane32 + 16, f32x4{M[4], M[5], M[6], M[7]});
  st_f32x4(vb, lane32, f32x4{V[0], V[1], V[2], V[3]});
  st_f32x4(vb, lane32 + 16, f32x4{V[4], V[5], V[6], V[7]});
  if constexpr (PARAM)
    st_u16x8(par + e0, lane16,
             u32x4{narrow2<PDT>(W[0], W[1]), narrow2<PDT>(W[2], W[3]), narrow2<PDT>(W[4], W[5]),
                   narrow2<PDT>(W[6], W[7])});
}

// Sums are held in arrays of kGroupsPerArray groups (7 x 8 fp32 per lane);
// each array's loops unroll fully, so every index is a constant and the sums
// stay in registers.
constexpr int kGroupsPerArray = 7;
constexpr int kFullArrays = kGroupsMax / kGroupsPerArray;
static_assert(kFullArrays * kGroupsPerArray == kGroupsMax, "arrays must tile kGroupsMax");

// Read phase for the kGroupsPerArray groups starting at uniform group index
// gbase (groups gbase + u*kBlock + lane): rank sums into s.  Groups at or past
// glimit are skipped.
template <int GDT, class Grads>
__device__ __forceinline__ void read_groups(const Grads& gr, int p,
                                            float (&s)[kGroupsPerArray][kVec], int64_t gbase,
                                            int64_t glimit, int64_t h, uint32_t lane16) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kGroupsPerArray; ++u) {
    const int64_t gb = gbase + static_cast<int64_t>(u) * kBlock;
    if (gb + tid < glimit) sum_ranks8<GDT>(gr, p, h + gb * kVec, lane16, s[u]);
  }
}

// Update phase for the same groups: mean = sum / P, then Adam + downcast.
template <int PDT, int FORM>
__device__ __forceinline__ void update_groups(const Consts& c, float (&s)[kGroupsPerArray][kVec],
                                              int64_t gbase, int64_t glimit, int64_t h,
                                              float* w, float* m, float* v, uint16_t* par,
                                              uint32_t lane16, uint32_t lane32) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kGroupsPerArray; ++u) {
    const int64_t gb = gbase + static_cast<int64_t>(u) * kBlock;
    if (gb + tid < glimit) {
#pragma unroll
      for (int j = 0; j < kVec; ++j) s[u][j] = s[u][j] / c.PF;
      adam8<PDT, FORM>(c, s[u], w, m, v, par, h + gb * kVec, lane16, lane32);
    }
  }
}

// One chunk of NA * kGroupsPerArray groups per lane starting at group g0:
// first the read-only phase over all of its groups (sums in registers), then
// the update phase.  NA is a compile-time constant: a runtime bound on the
// group count here costs about a sixth of the bandwidth (the predicates get
// materialised and hoisted), so chunk sizes are fixed and only the range
// limit glimit is checked per lane.
template <int NA, int GDT, int PDT, int FORM, class Grads>
__device__ __forceinline__ void phase_chunk(const Grads& gr, int p, float* w, float* m, float* v,
                                            uint16_t* par, int64_t h, int64_t g0,
                                            int64_t glimit, const Consts& c, uint32_t lane16,
                                            uint32_t lane32) {
  constexpr int64_t A = static_cast<int64_t>(kGroupsPerArray) * kBlock;  // groups per array
  float s0[kGroupsPerArray][kVec], s1[kGroupsPerArray][kVec], s2[kGroupsPerArray][kVec],
      s3[kGroupsPerArray][kVec];
  static_assert(NA >= 1 && NA <= 4, "at most four sum arrays");
  read_groups<GDT>(gr, p, s0, g0, glimit, h, lane16);
  if constexpr (NA > 1) read_groups<GDT>(gr, p, s1, g0 + A, glimit, h, lane16);
  if constexpr (NA > 2) read_groups<GDT>(gr, p, s2, g0 + 2 * A, glimit, h, lane16);
  if constexpr (NA > 3) read_groups<GDT>(gr, p, s3, g0 + 3 * A, glimit, h, lane16);
  update_groups<PDT, FORM>(c, s0, g0, glimit, h, w, m, v, par, lane16, lane32);
  if constexpr (NA > 1) update_groups<PDT, FORM>(c, s1, g0 + A, glimit, h, w, m, v, par, lane16, lane32);
  if constexpr (NA > 2)
    update_groups<PDT, FORM>(c, s2, g0 + 2 * A, glimit, h, w, m, v, par, lane16, lane32);
  if constexpr (NA > 3)
    update_groups<PDT, FORM>(c, s3, g0 + 3 * A, glimit, h, w, m, v, par, lane16, lane32);
}

// The fused step on elements [0, len) of one range, phase-separated, shared
// by workgroups blk = 0..nblk-1.  Vector groups (8 elements per lane) start
// at element `head`.  Full chunks of kBlock * kGroupsMax groups go round-robin
// to the workgroups; the groups left after the last full chunk are split into
// nblk equal contiguous parts (whole multiples of kBlock groups), each
// processed in chunks of kBlock * kGroupsPerArray groups.  The scalar head
// and tail elements go to workgroup 0.
template <int GDT, int PDT, int FORM, class Grads>
__device__ __forceinline__ void fused_phased(const Grads& gr, int p, float* __restrict__ w,
                                             float* __restrict__ m, float* __restrict__ v,
                                             uint16_t* __restrict__ par, int64_t len, int head,
                                             const Consts& c, int64_t blk, int64_t nblk) {
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  const int tid = threadIdx.x;
  const uint32_t lane16 = static_cast<uint32_t>(tid) * 16u;
  const uint32_t lane32 = static_cast<uint32_t>(tid) * 32u;
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  constexpr int64_t kSmall = static_cast<int64_t>(kBlock) * kGroupsPerArray;
  const int64_t nfull = nvec / kFull;
  for (int64_t ch = blk; ch < nfull; ch += nblk)
    phase_chunk<kFullArrays, GDT, PDT, FORM>(gr, p, w, m, v, par, h, ch * kFull, nvec, c, lane16,
                                             lane32);
  const int64_t left0 = nfull * kFull;
  const int64_t nleft = nvec - left0;
  if (nleft > 0) {
    int64_t per = (nleft + nblk - 1) / nblk;
    per = (per + kBlock - 1) / kBlock * kBlock;
    const int64_t lo = left0 + blk * per;
    const int64_t hi = lo + per < nvec ? lo + per : nvec;
    for (int64_t g0 = lo; g0 < hi; g0 += kSmall)
      phase_chunk<1, GDT, PDT, FORM>(gr, p, w, m, v, par, h, g0, hi, c, lane16, lane32);
  }
  if (blk == 0) {
    const int64_t t0 = h + nvec * kVec;
    const int64_t nsc = h + (len - t0);
    for (int64_t i = tid; i < nsc; i += kBlock) {
      const int64_t e = i < h ? i : t0 + (i - h);
      const float g = mean1<GDT>(gr, p, e, c.PF);
      float W = w[e], M = m[e], V = v[e];
      adam1<FORM>(c, g, W, M, V);
      w[e] = W;
      m[e] = M;
      v[e] = V;
      par[e] = narrow1<PDT>(W);
    }
  }
}

template <int GDT, int PDT, int FORM, int PMAX>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_kernel(GradArgs<PMAX> ga, int p, float* __restrict__ w, float* __restrict__ m,
                  float* __restrict__ v, uint16_t* __restrict__ par, int64_t len, int head,
                  Consts c) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = kernarg_grads();
  fused_phased<GDT, PDT, FORM>(gr, p, w, m, v, par, len, head, c, blockIdx.x, gridDim.x);
}

// The fp32 mean of the P ranks alone, stored (the unfused first half).  Workgroup-uniform
// bases, 8 elements per lane, grid-stride over groups.
template <int GDT, int PMAX>
__global__ __launch_bounds__(kBlock) void mean_kernel(GradArgs<PMAX> ga, int p,
                                                      float* __restrict__ out, int64_t len,
                                                      int head, float PF) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = kernarg_grads();
  const int tid = threadIdx.x;
  const uint32_t lane16 = static_cast<uint32_t>(tid) * 16u;
  const uint32_t lane32 = static_cast<uint32_t>(tid) * 32u;
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  for (int64_t gb = static_cast<int64_t>(blockIdx.x) * kBlock; gb < nvec;
       gb += static_cast<int64_t>(gridDim.x) * kBlock) {
    if (gb + tid < nvec) {
      const int64_t e0 = h + gb * kVec;
      float g[kVec];
      sum_ranks8<GDT>(gr, p, e0, lane16, g);
#pragma unroll
      for (int j = 0; j < kVec; ++j) g[j] = g[j] / PF;
      float* ob = out + e0;
      st_f32x4(ob, lane32, f32x4{g[0], g[1], g[2], g[3]});
      st_f32x4(ob, lane32 + 16, f32x4{g[4], g[5], g[6], g[7]});
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t0 = h + nvec * kVec;
    const int64_t nsc = h + (len - t0);
    for (int64_t i = tid; i < nsc; i += kBlock) {
      const int64_t e = i < h ? i : t0 + (i - h);
      out[e] = mean1<GDT>(gr, p, e, PF);
    }
  }
}

// Adam + downcast from a stored fp32 gradient.
template <int PDT, int FORM, bool PARAM>
__global__ __launch_bounds__(kBlock) void adam_kernel(const float* __restrict__ gin,
                                                      float* __restrict__ w,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      uint16_t* __restrict__ par, int64_t len,
                                                      int head, Consts c) {
  const int tid = threadIdx.x;
  const uint32_t lane16 = static_cast<uint32_t>(tid) * 16u;
  const uint32_t lane32 = static_cast<uint32_t>(tid) * 32u;
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  for (int64_t gb = static_cast<int64_t>(blockIdx.x) * kBlock; gb < nvec;
       gb += static_cast<int64_t>(gridDim.x) * kBlock) {
    if (gb + tid < nvec) {
      const int64_t e0 = h + gb * kVec;
      const f32x4 a = ld_f32x4(gin + e0, lane32), b = ld_f32x4(gin + e0, lane32 + 16);
      const float g[kVec] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      adam8<PDT, FORM, PARAM>(c, g, w, m, v, par, e0, lane16, lane32);
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t0 = h + nvec * kVec;
    const int64_t nsc = h + (len - t0);
    for (int64_t i = tid; i < nsc; i += kBlock) {
      const int64_t e = i < h ? i : t0 + (i - h);
      float W = w[e], M = m[e], V = v[e];
      adam1<FORM>(c, gin[e], W, M, V);
      w[e] = W;
      m[e] = M;
      v[e] = V;
      if constexpr (PARAM) par[e] = narrow1<PDT>(W);
    }
  }
}

// Multi-tensor: one persistent launch over a chunk list, one workgroup per
// CU.  For each chunk the workgroup stages the chunk's piece descriptor and
// its p gradient pointers in LDS (every lane then reads the same entry), and
// runs the phase-separated body over the chunk with its own threads.
template <int GDT, int PDT, int FORM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void multi_kernel(const MtPiece* __restrict__ pieces, const uint16_t* const* __restrict__ gptrs,
                  const MtChunk* __restrict__ chunks, int64_t nchunks, int64_t chunk_elems, int p,
                  Consts c) {
  __shared__ const uint16_t* s_g[kMaxP];
  __shared__ MtPiece s_piece;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const MtChunk cc = chunks[ch];
    __syncthreads();  // the previous chunk's readers of s_g / s_piece are done
    for (int r = threadIdx.x; r < p; r += kBlock)
      s_g[r] = gptrs[static_cast<int64_t>(cc.piece) * p + r] + cc.start;
    if (threadIdx.x == 0) s_piece = pieces[cc.piece];
    __syncthreads();
    const int64_t plen = s_piece.len;
    const int64_t rest = plen - cc.start;
    const int64_t len = rest < chunk_elems ? rest : chunk_elems;
    const int head = (s_piece.head - static_cast<int>(cc.start & 7)) & 7;
    float* w = uniform_t(s_piece.w) + cc.start;
    float* m = uniform_t(s_piece.m) + cc.start;
    float* v = uniform_t(s_piece.v) + cc.start;
    uint16_t* par = uniform_t(s_piece.param) + cc.start;
    const LdsGrads gr{s_g};
    fused_phased<GDT, PDT, FORM>(gr, p, w, m, v, par, len, head, c, 0, 1);
  }
}

constexpr int kBlocksPerCU = 4;

int64_t grid_for(int64_t len) {
  const int64_t groups = len / kVec + 1;
  int64_t blocks = (groups + kBlock - 1) / kBlock;
  const int64_t cap = static_cast<int64_t>(cu_count()) * kBlocksPerCU;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return blocks;
}

template <int V>
using IC = std::integral_constant<int, V>;

template <class F>
void with_dt(int dt, F&& f) {
  if (dt == kF16) f(IC<kF16>{}); else f(IC<kBF16>{});
}

template <class F>
void with_form(int form, F&& f) {
  if (form == kStandard) f(IC<kStandard>{}); else f(IC<kPage1Literal>{});
}

template <class F>
void with_pmax(int p, F&& f) {
  if (p <= 8) f(IC<8>{});
  else if (p <= 64) f(IC<64>{});
  else f(IC<256>{});
}

}  // namespace

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_fused(const FusedLaunch& a) {
  // One workgroup per CU (the kernel runs one wave per SIMD).
  const int64_t h = a.head < a.len ? a.head : a.len;
  const int64_t nvec = (a.len - h) / kVec;
  int64_t grid = (nvec + kBlock - 1) / kBlock;
  const int64_t cu = cu_count();
  if (grid > cu) grid = cu;
  if (grid < 1) grid = 1;
  with_dt(a.gdt, [&](auto G) {
    with_dt(a.pdt, [&](auto H) {
      with_form(a.form, [&](auto F) {
        with_pmax(a.p, [&](auto PM) {
          constexpr int PMAX = decltype(PM)::value;
          GradArgs<PMAX> ga;
          for (int r = 0; r < PMAX; ++r) ga.g[r] = r < a.p ? a.grads[r] : nullptr;
          fused_kernel<decltype(G)::value, decltype(H)::value, decltype(F)::value, PMAX>
              <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                  ga, a.p, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
        });
      });
    });
  });
  return hipGetLastError();
}

hipError_t launch_mean(const MeanLaunch& a) {
  const int64_t grid = grid_for(a.len);
  with_dt(a.gdt, [&](auto G) {
    with_pmax(a.p, [&](auto PM) {
      constexpr int PMAX = decltype(PM)::value;
      GradArgs<PMAX> ga;
      for (int r = 0; r < PMAX; ++r) ga.g[r] = r < a.p ? a.grads[r] : nullptr;
      mean_kernel<decltype(G)::value, PMAX>
          <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
              ga, a.p, a.out, a.len, a.head, a.PF);
    });
  });
  return hipGetLastError();
}

hipError_t launch_adam(const AdamLaunch& a) {
  const int64_t grid = grid_for(a.len);
  with_dt(a.pdt, [&](auto H) {
    with_form(a.form, [&](auto F) {
      if (a.param)
        adam_kernel<decltype(H)::value, decltype(F)::value, true>
            <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                a.g, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
      else
        adam_kernel<decltype(H)::value, decltype(F)::value, false>
            <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                a.g, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
    });
  });
  return hipGetLastError();
}

hipError_t launch_multi(const MultiLaunch& a) {
  int64_t grid = static_cast<int64_t>(cu_count());
  if (grid > a.nchunks) grid = a.nchunks;
  if (grid < 1) grid = 1;
  with_dt(a.gdt, [&](auto G) {
    with_dt(a.pdt, [&](auto H) {
      with_form(a.form, [&](auto F) {
        multi_kernel<decltype(G)::value, decltype(H)::value, decltype(F)::value>
            <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                a.pieces, a.gptrs, a.chunks, a.nchunks, a.chunk_elems, a.p, a.c);
      });
    });
  });
  return hipGetLastError();
}

}  // namespace zs

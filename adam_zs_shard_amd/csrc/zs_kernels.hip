// zs_kernels.hip -- gfx950 kernels of libzshard.
//
// The per-shard step is pure streaming: per element it reads P 16-bit
// gradients and the fp32 (w, m, v), writes (w, m, v) and one 16-bit working
// copy, and does O(P) flops.  At 0.5 flop/byte it sits far below the fp32
// vector ridge of the chip, so the design goal is HBM bandwidth, not math:
//  - each lane owns groups of 8 consecutive elements: one 16-byte load per
//    gradient rank, two per fp32 state array, one 16-byte store of the
//    16-bit copy; consecutive lanes touch consecutive 16-byte words, so a
//    wave64 access is 1 KiB contiguous;
//  - the P rank loads of a group are issued in batches of 8 before their
//    adds, so each wave keeps 8 x 1 KiB of gradient reads in flight while
//    the adds stay in rank order 0..P-1 (the fold is a left fold: one fp32
//    rounding per add, in rank order, as the oracle does);
//  - the state loads are issued before the gradient loads so they overlap;
//  - grid-stride persistent blocks (a few workgroups per CU) walk the shard;
//  - no MFMA and no LDS on the single-tensor path: nothing is reused.
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

// Gradient pointer sources: kernel arguments, or a table staged in LDS.
template <int PMAX>
struct GradArgs {
  const uint16_t* g[PMAX];
};

template <int PMAX>
struct ArgGrads {
  const GradArgs<PMAX>& a;
  __device__ __forceinline__ const uint16_t* get(int r) const { return a.g[r]; }
};

struct LdsGrads {
  const uint16_t* const* s;
  __device__ __forceinline__ const uint16_t* get(int r) const { return uniform(s[r]); }
};

constexpr int kRankBatch = 8;

// acc[j] = (sum over r in rank order of widen(grad_r[e + j])) / PF, j < 8.
template <int GDT, class Grads>
__device__ __forceinline__ void mean8(const Grads& gr, int p, int64_t e, float (&acc)[kVec],
                                      float PF) {
  {
    u32x4 q[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b)
      if (b < p) q[b] = *reinterpret_cast<const u32x4*>(gr.get(b) + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = widen_lo<GDT>(q[0][j]);
      acc[2 * j + 1] = widen_hi<GDT>(q[0][j]);
    }
#pragma unroll
    for (int b = 1; b < kRankBatch; ++b) {
      if (b < p) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = acc[2 * j] + widen_lo<GDT>(q[b][j]);
          acc[2 * j + 1] = acc[2 * j + 1] + widen_hi<GDT>(q[b][j]);
        }
      }
    }
  }
  for (int r0 = kRankBatch; r0 < p; r0 += kRankBatch) {
    u32x4 q[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b)
      if (r0 + b < p) q[b] = *reinterpret_cast<const u32x4*>(gr.get(r0 + b) + e);
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
      if (r0 + b < p) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] = acc[2 * j] + widen_lo<GDT>(q[b][j]);
          acc[2 * j + 1] = acc[2 * j + 1] + widen_hi<GDT>(q[b][j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kVec; ++j) acc[j] = acc[j] / PF;
}

template <int GDT, class Grads>
__device__ __forceinline__ float mean1(const Grads& gr, int p, int64_t e, float PF) {
  float s = widen1<GDT>(gr.get(0)[e]);
  for (int r = 1; r < p; ++r) s = s + widen1<GDT>(gr.get(r)[e]);
  return s / PF;
}

__device__ __forceinline__ void load8(const float* p, float (&x)[kVec]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(float* p, const float (&x)[kVec]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

template <int PDT>
__device__ __forceinline__ void store8_16(uint16_t* p, const float (&x)[kVec]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{narrow2<PDT>(x[0], x[1]), narrow2<PDT>(x[2], x[3]),
                                       narrow2<PDT>(x[4], x[5]), narrow2<PDT>(x[6], x[7])};
}

// The fused step on elements [0, len) of one range, shared by threads
// tid = 0..nthr-1.  Vector groups start at element `head`; the scalar head
// and tail elements are spread over the first threads.
template <int GDT, int PDT, int FORM, class Grads>
__device__ __forceinline__ void fused_range(const Grads& gr, int p, float* __restrict__ w,
                                            float* __restrict__ m, float* __restrict__ v,
                                            uint16_t* __restrict__ par, int64_t len, int head,
                                            const Consts& c, int64_t tid, int64_t nthr) {
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  for (int64_t i = tid; i < nvec; i += nthr) {
    const int64_t e = h + i * kVec;
    float W[kVec], M[kVec], V[kVec], g[kVec];
    load8(w + e, W);
    load8(m + e, M);
    load8(v + e, V);
    mean8<GDT>(gr, p, e, g, c.PF);
#pragma unroll
    for (int j = 0; j < kVec; ++j) adam1<FORM>(c, g[j], W[j], M[j], V[j]);
    store8(w + e, W);
    store8(m + e, M);
    store8(v + e, V);
    store8_16<PDT>(par + e, W);
  }
  const int64_t t0 = h + nvec * kVec;
  const int64_t nsc = h + (len - t0);
  for (int64_t i = tid; i < nsc; i += nthr) {
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

template <int GDT, int PDT, int FORM, int PMAX>
__global__ __launch_bounds__(kBlock) void fused_kernel(GradArgs<PMAX> ga, int p,
                                                       float* __restrict__ w,
                                                       float* __restrict__ m,
                                                       float* __restrict__ v,
                                                       uint16_t* __restrict__ par, int64_t len,
                                                       int head, Consts c) {
  const ArgGrads<PMAX> gr{ga};
  fused_range<GDT, PDT, FORM>(gr, p, w, m, v, par, len, head, c,
                              static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x,
                              static_cast<int64_t>(gridDim.x) * kBlock);
}

template <int GDT, int PMAX>
__global__ __launch_bounds__(kBlock) void mean_kernel(GradArgs<PMAX> ga, int p,
                                                      float* __restrict__ out, int64_t len,
                                                      int head, float PF) {
  const ArgGrads<PMAX> gr{ga};
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nthr = static_cast<int64_t>(gridDim.x) * kBlock;
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  for (int64_t i = tid; i < nvec; i += nthr) {
    const int64_t e = h + i * kVec;
    float g[kVec];
    mean8<GDT>(gr, p, e, g, PF);
    store8(out + e, g);
  }
  const int64_t t0 = h + nvec * kVec;
  const int64_t nsc = h + (len - t0);
  for (int64_t i = tid; i < nsc; i += nthr) {
    const int64_t e = i < h ? i : t0 + (i - h);
    out[e] = mean1<GDT>(gr, p, e, PF);
  }
}

template <int PDT, int FORM, bool PARAM>
__global__ __launch_bounds__(kBlock) void adam_kernel(const float* __restrict__ gin,
                                                      float* __restrict__ w,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      uint16_t* __restrict__ par, int64_t len,
                                                      int head, Consts c) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nthr = static_cast<int64_t>(gridDim.x) * kBlock;
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  for (int64_t i = tid; i < nvec; i += nthr) {
    const int64_t e = h + i * kVec;
    float W[kVec], M[kVec], V[kVec], g[kVec];
    load8(gin + e, g);
    load8(w + e, W);
    load8(m + e, M);
    load8(v + e, V);
#pragma unroll
    for (int j = 0; j < kVec; ++j) adam1<FORM>(c, g[j], W[j], M[j], V[j]);
    store8(w + e, W);
    store8(m + e, M);
    store8(v + e, V);
    if constexpr (PARAM) store8_16<PDT>(par + e, W);
  }
  const int64_t t0 = h + nvec * kVec;
  const int64_t nsc = h + (len - t0);
  for (int64_t i = tid; i < nsc; i += nthr) {
    const int64_t e = i < h ? i : t0 + (i - h);
    float W = w[e], M = m[e], V = v[e];
    adam1<FORM>(c, gin[e], W, M, V);
    w[e] = W;
    m[e] = M;
    v[e] = V;
    if constexpr (PARAM) par[e] = narrow1<PDT>(W);
  }
}

// Multi-tensor: one persistent launch over a chunk list.  For each chunk the
// block stages the chunk's piece descriptor and its p gradient pointers in
// LDS, then runs the same per-range body with the block's threads.
template <int GDT, int PDT, int FORM>
__global__ __launch_bounds__(kBlock) void multi_kernel(const MtPiece* __restrict__ pieces,
                                                       const uint16_t* const* __restrict__ gptrs,
                                                       const MtChunk* __restrict__ chunks,
                                                       int64_t nchunks, int64_t chunk_elems,
                                                       int p, Consts c) {
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
    fused_range<GDT, PDT, FORM>(gr, p, w, m, v, par, len, head, c, threadIdx.x, kBlock);
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
  const int64_t grid = grid_for(a.len);
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
  int64_t grid = static_cast<int64_t>(cu_count()) * kBlocksPerCU;
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

// zs_unfused.hip -- the unfused pair: the stored rank mean, then the update from it.

#include "zs_device.h"

namespace zs {
namespace {

constexpr int kBlocksPerCU = 4;

// Output dtype of the stored mean: 0 (fp32), kF16 or kBF16.
template <class F>
void with_odt(int odt, F&& f) {
  if (odt == kF16) f(IC<kF16>{});
  else if (odt == kBF16) f(IC<kBF16>{});
  else f(IC<0>{});
}

int64_t grid_for(int64_t len) {
  const int64_t groups = len / kVec + 1;
  int64_t blocks = (groups + kBlock - 1) / kBlock;
  const int64_t cap = static_cast<int64_t>(cu_count()) * kBlocksPerCU;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return blocks;
}


// Where one pass of the stored mean puts its results (see MeanLaunch): the
// last pass divides the sums by P and stores the mean as fp32 (ODT 0) or
// rounded to nearest even in 16 bits; an earlier pass stores the fp32 sums,
// which the next pass continues.
template <int ODT>
struct MeanOut {
  void* out;
  int last;
  float PF;
  // the 8 consecutive elements at e0 of one lane (lane16 = 16 * lane)
  __device__ __forceinline__ void put8(int64_t e0, uint32_t lane16, const float (&s)[kVec]) const {
    if (last) {
      float g[kVec];
#pragma unroll
      for (int j = 0; j < kVec; ++j) g[j] = s[j] / PF;
      if constexpr (ODT == 0) {
        float* o = static_cast<float*>(out) + e0;
        st_f32x4(o, 2 * lane16, f32x4{g[0], g[1], g[2], g[3]});
        st_f32x4(o, 2 * lane16 + 16, f32x4{g[4], g[5], g[6], g[7]});
      } else {
        st_u16x8(static_cast<uint16_t*>(out) + e0, lane16,
                 u32x4{narrow2<ODT>(g[0], g[1]), narrow2<ODT>(g[2], g[3]),
                       narrow2<ODT>(g[4], g[5]), narrow2<ODT>(g[6], g[7])});
      }
    } else {
      float* o = static_cast<float*>(out) + e0;
      st_f32x4(o, 2 * lane16, f32x4{s[0], s[1], s[2], s[3]});
      st_f32x4(o, 2 * lane16 + 16, f32x4{s[4], s[5], s[6], s[7]});
    }
  }
  __device__ __forceinline__ void put1(int64_t e, float s) const {
    if (!last) {
      static_cast<float*>(out)[e] = s;
    } else if constexpr (ODT == 0) {
      static_cast<float*>(out)[e] = s / PF;
    } else {
      static_cast<uint16_t*>(out)[e] = narrow1<ODT>(s / PF);
    }
  }
};

// The fp32 sums of earlier passes for one lane's 8 elements at e0.
__device__ __forceinline__ void load_acc8(const float* acc, int64_t e0, uint32_t lane32,
                                          float (&s)[kVec]) {
  const f32x4 a = ld_f32x4(acc + e0, lane32), b = ld_f32x4(acc + e0, lane32 + 16);
  s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
  s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
}

// Rank-order sum of one element over this pass's p ranks, continuing the
// fp32 sum `init` of earlier passes when acc is set (kRankBatch loads in
// flight per batch).
template <int GDT, class Grads>
__device__ __forceinline__ float sum1(const Grads& gr, int p, int64_t e, bool cont, float init) {
  float s = init;
  int r0 = 0;
  for (; r0 + kRankBatch <= p; r0 += kRankBatch) {
    uint16_t q[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) q[b] = gr.get(r0 + b)[e];
    __builtin_amdgcn_sched_barrier(0);
    s = (!cont && r0 == 0) ? widen1<GDT>(q[0]) : s + widen1<GDT>(q[0]);
#pragma unroll
    for (int b = 1; b < kRankBatch; ++b) s = s + widen1<GDT>(q[b]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; r0 < p; ++r0) {
    const float x = widen1<GDT>(gr.get(r0)[e]);
    s = (!cont && r0 == 0) ? x : s + x;
  }
  return s;
}

// The stored mean's counterpart of fused_rest: the pieces left after the
// whole chunks, then the scalar head and tail, dealt the same way.
template <int GDT, int ODT, class Grads>
__device__ __forceinline__ void mean_rest(const Grads& gr, int p, const float* acc,
                                          const MeanOut<ODT>& mo, int64_t len, int64_t h,
                                          int64_t nvec, int64_t left0, int64_t nfull,
                                          int64_t blk, int64_t nblk, uint32_t lane16,
                                          uint32_t lane32) {
  const int tid = threadIdx.x;
  const int64_t first = nfull % nblk;
  const int64_t me = (blk - first + nblk) % nblk;
  constexpr int64_t kPiece = 2 * kBlock;
  const int64_t npieces = (nvec - left0 + kPiece - 1) / kPiece;
  for (int64_t i = me; i < npieces; i += nblk) {
    const int64_t gb = left0 + i * kPiece;
    const int64_t e0 = h + gb * kVec;
    const int64_t e1 = e0 + static_cast<int64_t>(kBlock) * kVec;
    if (gb + kBlock + tid < nvec) {
      float a[kVec], b[kVec];
      if (acc) {
        load_acc8(acc, e0, lane32, a);
        load_acc8(acc, e1, lane32, b);
        sum_ranks8x2<GDT, 16, true>(gr, p, e0, e1, lane16, a, b);
      } else {
        sum_ranks8x2<GDT>(gr, p, e0, e1, lane16, a, b);
      }
      mo.put8(e0, lane16, a);
      mo.put8(e1, lane16, b);
    } else if (gb + tid < nvec) {
      float g[kVec];
      if (acc) {
        load_acc8(acc, e0, lane32, g);
        sum_ranks8<GDT, true>(gr, p, e0, lane16, g);
      } else {
        sum_ranks8<GDT>(gr, p, e0, lane16, g);
      }
      mo.put8(e0, lane16, g);
    }
  }
  if (me == npieces % nblk) {
    const int64_t t0 = h + nvec * kVec;
    const int64_t nsc = h + (len - t0);
    for (int64_t i = tid; i < nsc; i += kBlock) {
      const int64_t e = i < h ? i : t0 + (i - h);
      mo.put1(e, sum1<GDT>(gr, p, e, acc != nullptr, acc ? acc[e] : 0.0f));
    }
  }
}

// The stored mean (the unfused first half) for shards with whole chunks:
// fused_kernel's read phase (same chunks, same probe-first rank loop, one
// workgroup per CU), then the chunk's results stored instead of the update.
// Written out in the kernel body for the reason given at fused_kernel.  A
// pass that continues earlier ranks starts from their fp32 sums (acc).
static_assert(kLoadBatch == kGroupsMax, "mean_chunk_kernel reads a chunk in one batch per rank");
template <int GDT, int ODT, int PMAX>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mean_chunk_kernel(GradArgs<PMAX> ga, int p, const float* acc, MeanOut<ODT> mo, int64_t len,
                       int head) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = kernarg_grads();
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  const uint32_t lane16 = threadIdx.x * 16u;
  const uint32_t lane32 = threadIdx.x * 32u;
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const int64_t nfull = whole_chunks(nvec / kFull, gridDim.x);
  const bool cont = acc != nullptr;
  for (int64_t ch = blockIdx.x; ch < nfull; ch += gridDim.x) {
    const int64_t g0 = ch * kFull;
    float s[kGroupsMax][kVec];
    if (cont) {
#pragma unroll
      for (int u = 0; u < kGroupsMax; ++u)
        load_acc8(acc, h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec, lane32, s[u]);
    }
    for (int r = 0; r < p; ++r) {
      const uint16_t* base = gr.get(r) + h + g0 * kVec;
      const bool start = !cont && r == 0;
      {
        const u32x4 q0 = ld_grad(base, lane16);
        __builtin_amdgcn_sched_barrier(0);
        if (start) {
          init8<GDT>(s[0], q0);
        } else {
          fold8<GDT>(s[0], q0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        u32x4 q[kLoadBatch - 1];
#pragma unroll
        for (int u = 0; u < kLoadBatch - 1; ++u)
          q[u] = ld_grad(base + static_cast<int64_t>(1 + u) * kBlock * kVec, lane16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kLoadBatch - 1; ++u) {
          if (start) {
            init8<GDT>(s[1 + u], q[u]);
          } else {
            fold8<GDT>(s[1 + u], q[u]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < kGroupsMax; ++u)
      mo.put8(h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec, lane16, s[u]);
  }
  mean_rest<GDT, ODT>(gr, p, acc, mo, len, h, nvec, nfull * kFull, nfull, blockIdx.x, gridDim.x,
                      lane16, lane32);
}

// The stored mean for smaller shards.  Workgroup-uniform bases, 8 elements
// per lane, grid-stride over groups.
template <int GDT, int ODT, int PMAX>
__global__ __launch_bounds__(kBlock) void mean_kernel(GradArgs<PMAX> ga, int p, const float* acc,
                                                      MeanOut<ODT> mo, int64_t len, int head) {
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
      if (acc) {
        load_acc8(acc, e0, lane32, g);
        sum_ranks8<GDT, true>(gr, p, e0, lane16, g);
      } else {
        sum_ranks8<GDT>(gr, p, e0, lane16, g);
      }
      mo.put8(e0, lane16, g);
    }
  }
  if (blockIdx.x == 0) {
    const int64_t t0 = h + nvec * kVec;
    const int64_t nsc = h + (len - t0);
    for (int64_t i = tid; i < nsc; i += kBlock) {
      const int64_t e = i < h ? i : t0 + (i - h);
      mo.put1(e, sum1<GDT>(gr, p, e, acc != nullptr, acc ? acc[e] : 0.0f));
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
  // Two vectors per lane per iteration, both vectors' loads in flight
  // together (14% faster than one on the 117M-element shard); the block whose
  // turn comes after the last whole pair takes the partial pair.
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock * 2;
  int64_t gb = static_cast<int64_t>(blockIdx.x) * kBlock * 2;
  for (; gb + 2 * kBlock <= nvec; gb += stride) {
    const int64_t e0 = h + gb * kVec;
    const int64_t e1 = e0 + static_cast<int64_t>(kBlock) * kVec;
    const f32x4 a0 = ld_f32x4(gin + e0, lane32), a1 = ld_f32x4(gin + e0, lane32 + 16);
    const f32x4 b0 = ld_f32x4(gin + e1, lane32), b1 = ld_f32x4(gin + e1, lane32 + 16);
    const float ga[kVec] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float gb2[kVec] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    adam8x2<PDT, FORM, false, PARAM>(c, ga, gb2, w, m, v, par, e0, e1, lane16, lane32);
  }
  for (; gb < nvec; gb += kBlock) {
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
      float W = w[e], M = ld_state1<kUsesM<FORM>>(m + e), V = ld_state1<kUsesV<FORM>>(v + e);
      adam1<FORM>(c, gin[e], W, M, V);
      w[e] = W;
      st_state1<kUsesM<FORM>>(m + e, M);
      st_state1<kUsesV<FORM>>(v + e, V);
      if constexpr (PARAM) par[e] = narrow1<PDT>(W);
    }
  }
}

// The update from a stored gradient (the unfused second half) for shards
// with whole chunks for at least half the CUs, in the shape of fused_kernel's
// update phase: whole chunks round-robin over one workgroup per CU (one wave
// per SIMD), the chunk's groups one after another.  16% faster than
// adam_kernel on the 117M-element shard.
template <int PDT, int FORM, bool PARAM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void adam_chunk_kernel(const float* __restrict__ gin, float* __restrict__ w,
                       float* __restrict__ m, float* __restrict__ v,
                       uint16_t* __restrict__ par, int64_t len, int head, Consts c) {
  const int tid = threadIdx.x;
  const uint32_t lane16 = static_cast<uint32_t>(tid) * 16u;
  const uint32_t lane32 = static_cast<uint32_t>(tid) * 32u;
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const int64_t nfull = nvec / kFull;
  for (int64_t ch = blockIdx.x; ch < nfull; ch += gridDim.x) {
    const int64_t g0 = ch * kFull;
#pragma unroll
    for (int u = 0; u < kGroupsMax; ++u) {
      const int64_t e0 = h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec;
      const f32x4 a = ld_f32x4(gin + e0, lane32), b = ld_f32x4(gin + e0, lane32 + 16);
      const float g[kVec] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      adam8<PDT, FORM, PARAM>(c, g, w, m, v, par, e0, lane16, lane32);
    }
  }
  // the vectors after the whole chunks (fewer than one chunk), grid-stride
  for (int64_t gb = nfull * kFull + static_cast<int64_t>(blockIdx.x) * kBlock; gb < nvec;
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
      float W = w[e], M = ld_state1<kUsesM<FORM>>(m + e), V = ld_state1<kUsesV<FORM>>(v + e);
      adam1<FORM>(c, gin[e], W, M, V);
      w[e] = W;
      st_state1<kUsesM<FORM>>(m + e, M);
      st_state1<kUsesV<FORM>>(v + e, V);
      if constexpr (PARAM) par[e] = narrow1<PDT>(W);
    }
  }
}

}  // namespace

hipError_t launch_mean(const MeanLaunch& a) {
  // Shards with whole chunks for at least half the CUs: mean_chunk_kernel,
  // one workgroup per CU; smaller ones: the grid-stride mean_kernel.
  const int64_t h = a.head < a.len ? a.head : a.len;
  const int64_t nvec = (a.len - h) / kVec;
  const int64_t cu = cu_count();
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const bool chunked = 2 * (nvec / kFull) >= cu;
  const int64_t grid = chunked ? cu : grid_for(a.len);
  // an earlier pass stores fp32 sums whatever the final dtype
  const int odt = a.last ? a.odt : 0;
  with_dt(a.gdt, [&](auto G) {
    with_odt(odt, [&](auto O) {
      with_pmax(a.p, [&](auto PM) {
        constexpr int GDT = decltype(G)::value, ODT = decltype(O)::value;
        constexpr int PMAX = decltype(PM)::value;
        GradArgs<PMAX> ga;
        for (int r = 0; r < PMAX; ++r) ga.g[r] = r < a.p ? a.grads[r] : nullptr;
        const MeanOut<ODT> mo{a.out, a.last, a.PF};
        if (chunked)
          mean_chunk_kernel<GDT, ODT, PMAX>
              <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                  ga, a.p, a.acc, mo, a.len, a.head);
        else
          mean_kernel<GDT, ODT, PMAX>
              <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                  ga, a.p, a.acc, mo, a.len, a.head);
      });
    });
  });
  return hipGetLastError();
}

hipError_t launch_adam(const AdamLaunch& a) {
  // Shards with whole chunks for at least half the CUs: adam_chunk_kernel,
  // one workgroup per CU; smaller ones: the grid-stride adam_kernel.
  const int64_t h = a.head < a.len ? a.head : a.len;
  const int64_t nvec = (a.len - h) / kVec;
  const int64_t cu = cu_count();
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const bool chunked = 2 * (nvec / kFull) >= cu;
  const int64_t grid = chunked ? cu : grid_for(a.len);
  const dim3 gd(static_cast<unsigned>(grid)), bd(kBlock);
  with_dt(a.pdt, [&](auto H) {
    with_form(a.form, [&](auto F) {
      constexpr int PDT = decltype(H)::value, FORM = decltype(F)::value;
      if (chunked && a.param)
        adam_chunk_kernel<PDT, FORM, true><<<gd, bd, 0, a.stream>>>(
            a.g, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
      else if (chunked)
        adam_chunk_kernel<PDT, FORM, false><<<gd, bd, 0, a.stream>>>(
            a.g, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
      else if (a.param)
        adam_kernel<PDT, FORM, true><<<gd, bd, 0, a.stream>>>(
            a.g, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
      else
        adam_kernel<PDT, FORM, false><<<gd, bd, 0, a.stream>>>(
            a.g, a.w, a.m, a.v, a.param, a.len, a.head, a.c);
    });
  });
  return hipGetLastError();
}

}  // namespace zs

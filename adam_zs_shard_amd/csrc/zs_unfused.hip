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
  // one lane's 8 elements of the group at e0, in the full-group map (FULL)
  // or 8 consecutive elements (the partial group)
  template <bool FULL>
  __device__ __forceinline__ void put8(int64_t e0, const Lanes& L, const float (&s)[kVec]) const {
    float g[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) g[j] = last ? s[j] / PF : s[j];
    if (last && ODT != 0) {
      constexpr int DT = ODT == 0 ? kF16 : ODT;
      uint16_t* o = static_cast<uint16_t*>(out) + e0;
      if constexpr (FULL) {
        st_h8<DT>(o, L, g);
      } else {
        st_u16x8(o, L.c16,
                 u32x4{narrow2<DT>(g[0], g[1]), narrow2<DT>(g[2], g[3]),
                       narrow2<DT>(g[4], g[5]), narrow2<DT>(g[6], g[7])});
      }
    } else {
      float* o = static_cast<float*>(out) + e0;
      if constexpr (FULL) {
        st_f8(o, L, g);
      } else {
        st_f32x4(o, L.c32, f32x4{g[0], g[1], g[2], g[3]});
        st_f32x4(o, L.c32 + 16, f32x4{g[4], g[5], g[6], g[7]});
      }
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

// The fp32 sums of earlier passes for one lane's 8 elements of the group at
// e0, in either map.
template <bool FULL>
__device__ __forceinline__ void load_acc8(const float* acc, int64_t e0, const Lanes& L,
                                          float (&s)[kVec]) {
  if constexpr (FULL) {
    ld_f8(acc + e0, L, s);
  } else {
    const f32x4 a = ld_f32x4(acc + e0, L.c32), b = ld_f32x4(acc + e0, L.c32 + 16);
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
  }
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

// One group's sums (either map), continuing acc when set.
template <int GDT, bool FULL, class Grads>
__device__ __forceinline__ void group_sums(const Grads& gr, int p, const float* acc, int64_t e0,
                                           const Lanes& L, float (&g)[kVec]) {
  if (acc) {
    load_acc8<FULL>(acc, e0, L, g);
    sum_ranks8<GDT, FULL, true>(gr, p, e0, L, g);
  } else {
    sum_ranks8<GDT, FULL>(gr, p, e0, L, g);
  }
}

// The stored mean's counterpart of fused_rest: the groups left after the
// whole chunks (pairs, the odd full group, the partial group), then the
// scalar head and tail, dealt the same way.
template <int GDT, int ODT, class Grads>
__device__ __forceinline__ void mean_rest(const Grads& gr, int p, const float* acc,
                                          const MeanOut<ODT>& mo, int64_t len, int64_t h,
                                          int64_t nvec, int64_t left0, int64_t nfull,
                                          int64_t blk, int64_t nblk, const Lanes& L) {
  const int tid = threadIdx.x;
  const RestPlan R = rest_plan(nvec, left0, nfull, blk, nblk);
  for (int64_t i = R.me; i < R.nitems; i += nblk) {
    if (i < R.npairs) {
      const int64_t e0 = h + (R.first_full + 2 * i * kBlock) * kVec;
      const int64_t e1 = e0 + kGroup;
      float a[kVec], b[kVec];
      if (acc) {
        load_acc8<true>(acc, e0, L, a);
        load_acc8<true>(acc, e1, L, b);
        sum_ranks8x2<GDT, 16, true, true>(gr, p, e0, e1, L, a, b);
      } else {
        sum_ranks8x2<GDT>(gr, p, e0, e1, L, a, b);
      }
      mo.template put8<true>(e0, L, a);
      mo.template put8<true>(e1, L, b);
    } else if (i == R.npairs && (R.nfg & 1)) {
      const int64_t e0 = h + (R.first_full + 2 * R.npairs * kBlock) * kVec;
      float g[kVec];
      group_sums<GDT, true>(gr, p, acc, e0, L, g);
      mo.template put8<true>(e0, L, g);
    } else if (tid < R.part) {
      const int64_t e0 = h + (R.first_full + R.nfg * kBlock) * kVec;
      float g[kVec];
      group_sums<GDT, false>(gr, p, acc, e0, L, g);
      mo.template put8<false>(e0, L, g);
    }
  }
  if (R.me == R.nitems % nblk) {
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
// Rounds of chunks between soft barriers (117M-element, 64-rank shard, 8
// rounds: every 2, 3 or 4 rounds 2.238 / 2.246 / 2.262 ms against 2.325 with
// none).
constexpr int kMeanSoftRounds = 2;
template <int GDT, int ODT, int PMAX>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mean_chunk_kernel(GradArgs<PMAX> ga, int p, const float* acc, MeanOut<ODT> mo, int64_t len,
                       int head) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = kernarg_grads();
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  const Lanes L = lanes();
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const int64_t nfull = whole_chunks(nvec / kFull, gridDim.x);
  const bool cont = acc != nullptr;
  // rounds of one whole chunk per workgroup, a soft barrier every
  // kMeanSoftRounds rounds
  const int64_t nrounds = (nfull + gridDim.x - 1) / gridDim.x;
  for (int64_t rd = 0; rd < nrounds; ++rd) {
    if (rd > 0 && rd % kMeanSoftRounds == 0)
      soft_barrier(static_cast<int>(rd / kMeanSoftRounds));
    const int64_t ch = blockIdx.x + rd * gridDim.x;
    if (ch >= nfull) continue;
    const int64_t g0 = ch * kFull;
    float s[kGroupsMax][kVec];
    if (cont) {
#pragma unroll
      for (int u = 0; u < kGroupsMax; ++u)
        load_acc8<true>(acc, h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec, L, s[u]);
    }
    for (int r = 0; r < p; ++r) {
      const uint16_t* base = gr.get(r) + h + g0 * kVec;
      const bool start = !cont && r == 0;
      {
        const G8 q0 = ld_g8(base, L);
        __builtin_amdgcn_sched_barrier(0);
        if (start) {
          init8<GDT>(s[0], q0);
        } else {
          fold8<GDT>(s[0], q0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        G8 q[kLoadBatch - 1];
#pragma unroll
        for (int u = 0; u < kLoadBatch - 1; ++u) {
          q[u] = ld_g8(base + (1 + u) * kGroup, L);
          __builtin_amdgcn_sched_barrier(0);  // issued in group order
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kLoadBatch - 1; ++u) {
          if (start) {
            init8<GDT>(s[1 + u], q[u]);
          } else {
            fold8<GDT>(s[1 + u], q[u]);
          }
          __builtin_amdgcn_sched_barrier(0);  // fold in load order
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < kGroupsMax; ++u)
      mo.template put8<true>(h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec, L, s[u]);
  }
  mean_rest<GDT, ODT>(gr, p, acc, mo, len, h, nvec, nfull * kFull, nfull, blockIdx.x, gridDim.x,
                      L);
}

// The stored mean for smaller shards, grid-stride over groups: full groups
// in the full-group map, then the partial group, then the scalar head and
// tail (block 0).
template <int GDT, int ODT, int PMAX>
__global__ __launch_bounds__(kBlock) void mean_kernel(GradArgs<PMAX> ga, int p, const float* acc,
                                                      MeanOut<ODT> mo, int64_t len, int head) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = kernarg_grads();
  const int tid = threadIdx.x;
  const Lanes L = lanes();
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  const int64_t nfg = nvec / kBlock, part = nvec % kBlock;
  for (int64_t gi = blockIdx.x; gi < nfg; gi += gridDim.x) {
    const int64_t e0 = h + gi * kGroup;
    float g[kVec];
    group_sums<GDT, true>(gr, p, acc, e0, L, g);
    mo.template put8<true>(e0, L, g);
  }
  if (part > 0 && blockIdx.x == nfg % gridDim.x && tid < part) {
    const int64_t e0 = h + nfg * kGroup;
    float g[kVec];
    group_sums<GDT, false>(gr, p, acc, e0, L, g);
    mo.template put8<false>(e0, L, g);
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

// The update of the scalar head and tail elements from a stored gradient.
template <int PDT, int FORM, bool PARAM>
__device__ __forceinline__ void adam_scalars(const Consts& c, const float* gin, float* w,
                                             float* m, float* v, uint16_t* par, int64_t len,
                                             int64_t h, int64_t nvec) {
  const int64_t t0 = h + nvec * kVec;
  const int64_t nsc = h + (len - t0);
  for (int64_t i = threadIdx.x; i < nsc; i += kBlock) {
    const int64_t e = i < h ? i : t0 + (i - h);
    float W = w[e], M = ld_state1<kUsesM<FORM>>(m + e), V = ld_state1<kUsesV<FORM>>(v + e);
    adam1<FORM>(c, gin[e], W, M, V);
    w[e] = W;
    st_state1<kUsesM<FORM>>(m + e, M);
    st_state1<kUsesV<FORM>>(v + e, V);
    if constexpr (PARAM) par[e] = narrow1<PDT>(W);
  }
}

// The update of one full group from a stored gradient (state and gradient
// loads issued together).
template <int PDT, int FORM, bool PARAM>
__device__ __forceinline__ void adam_group(const Consts& c, const Lanes& L, const float* gin,
                                           float* w, float* m, float* v, uint16_t* par,
                                           int64_t e0) {
  float g[kVec];
  ld_f8(gin + e0, L, g);
  const GroupState q = load_group<FORM>(L, w, m, v, e0);
  apply_group<PDT, FORM, false, PARAM>(c, L, q, g, w, m, v, par, e0);
}

// adam_group with the working copy staged in LDS (stage_quad) instead of
// stored: the quads go to y and y + 512.
template <int PDT, int FORM>
__device__ __forceinline__ void adam_group_staged(const Consts& c, const Lanes& L,
                                                  const float* gin, float* w, float* m, float* v,
                                                  int64_t e0, unsigned char* lds, uint32_t y) {
  float g[kVec];
  ld_f8(gin + e0, L, g);
  const GroupState q = load_group<FORM>(L, w, m, v, e0);
  float W[kVec] = {q.w0.x, q.w0.y, q.w0.z, q.w0.w, q.w1.x, q.w1.y, q.w1.z, q.w1.w};
  float M[kVec] = {q.m0.x, q.m0.y, q.m0.z, q.m0.w, q.m1.x, q.m1.y, q.m1.z, q.m1.w};
  float V[kVec] = {q.v0.x, q.v0.y, q.v0.z, q.v0.w, q.v1.x, q.v1.y, q.v1.z, q.v1.w};
  if constexpr (FORM == kStandard || FORM == kPage1Literal) {
    float MH[kVec], VH[kVec];
    adam_moments8<FORM>(c, g, M, V, MH, VH);
    st_f8(m + e0, L, M);
    st_f8(v + e0, L, V);
    __builtin_amdgcn_sched_barrier(0);  // the moments go out before the weight arithmetic
    adam_weights8(c, MH, VH, W);
    st_f8(w + e0, L, W);
  } else {
#pragma unroll
    for (int j = 0; j < kVec; ++j) adam1<FORM>(c, g[j], W[j], M[j], V[j]);
    st_f8(w + e0, L, W);
    if constexpr (kUsesM<FORM>) st_f8(m + e0, L, M);
  }
  stage_quad(lds, y, u32x2{narrow2<PDT>(W[0], W[1]), narrow2<PDT>(W[2], W[3])});
  stage_quad(lds, y + 512u, u32x2{narrow2<PDT>(W[4], W[5]), narrow2<PDT>(W[6], W[7])});
}

// Adam + downcast from a stored fp32 gradient, for smaller shards: pairs of
// full groups grid-stride (both groups' loads in flight together), then the
// odd full group and the partial group as two more items, then the scalars
// (block 0).
template <int PDT, int FORM, bool PARAM>
__global__ __launch_bounds__(kBlock) void adam_kernel(const float* __restrict__ gin,
                                                      float* __restrict__ w,
                                                      float* __restrict__ m,
                                                      float* __restrict__ v,
                                                      uint16_t* __restrict__ par, int64_t len,
                                                      int head, Consts c) {
  const int tid = threadIdx.x;
  const Lanes L = lanes();
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  const int64_t nfg = nvec / kBlock, part = nvec % kBlock;
  const int64_t npairs = nfg / 2;
  for (int64_t i = blockIdx.x; i < npairs; i += gridDim.x) {
    const int64_t e0 = h + 2 * i * kGroup, e1 = e0 + kGroup;
    float a[kVec], b[kVec];
    ld_f8(gin + e0, L, a);
    ld_f8(gin + e1, L, b);
    adam8x2<PDT, FORM, false, PARAM>(c, a, b, w, m, v, par, e0, e1, L);
  }
  if ((nfg & 1) && blockIdx.x == npairs % gridDim.x)
    adam_group<PDT, FORM, PARAM>(c, L, gin, w, m, v, par, h + (nfg - 1) * kGroup);
  if (part > 0 && blockIdx.x == (npairs + 1) % gridDim.x && tid < part) {
    const int64_t e0 = h + nfg * kGroup;
    const f32x4 a = ld_f32x4(gin + e0, L.c32), b = ld_f32x4(gin + e0, L.c32 + 16);
    const float g[kVec] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    adam8<PDT, FORM, PARAM>(c, g, w, m, v, par, e0, L);
  }
  if (blockIdx.x == 0) adam_scalars<PDT, FORM, PARAM>(c, gin, w, m, v, par, len, h, nvec);
}

// The update from a stored gradient (the unfused second half) for shards
// with whole chunks for at least half the CUs, in the shape of fused_kernel's
// update phase: whole chunks round-robin over one workgroup per CU (one wave
// per SIMD), the chunk's groups one after another; then the remaining full
// groups grid-stride, the partial group and the scalars.
template <int PDT, int FORM, bool PARAM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void adam_chunk_kernel(const float* __restrict__ gin, float* __restrict__ w,
                       float* __restrict__ m, float* __restrict__ v,
                       uint16_t* __restrict__ par, int64_t len, int head, Consts c) {
  const int tid = threadIdx.x;
  const Lanes L = lanes();
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const int64_t nfull = nvec / kFull;
  __shared__ __attribute__((aligned(16))) unsigned char copy_lds[PARAM ? kCopyStage : 16];
  for (int64_t ch = blockIdx.x; ch < nfull; ch += gridDim.x) {
    const int64_t g0 = ch * kFull;
    if constexpr (PARAM) {
      // the chunk's working copy staged in LDS, written out on whole lines
      unsigned char* const pc = reinterpret_cast<unsigned char*>(par + h + g0 * kVec);
      const uint32_t dl = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(pc) & 127u);
      const uint32_t ys = L.q16 + (dl & ~7u);
      __syncthreads();  // the previous chunk's flush has read the staged copy
#pragma unroll
      for (int u = 0; u < kGroupsMax; ++u)
        adam_group_staged<PDT, FORM>(c, L, gin, w, m, v,
                                     h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec,
                                     copy_lds, static_cast<uint32_t>(u) * (kBlock * kVec * 2) + ys);
      __syncthreads();
      flush_copy(copy_lds, pc - dl, dl);
    } else {
#pragma unroll
      for (int u = 0; u < kGroupsMax; ++u)
        adam_group<PDT, FORM, PARAM>(c, L, gin, w, m, v, par,
                                     h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec);
    }
  }
  const int64_t nfg = nvec / kBlock, part = nvec % kBlock;
  for (int64_t gi = nfull * kGroupsMax + blockIdx.x; gi < nfg; gi += gridDim.x)
    adam_group<PDT, FORM, PARAM>(c, L, gin, w, m, v, par, h + gi * kGroup);
  if (part > 0 && blockIdx.x == nfg % gridDim.x && tid < part) {
    const int64_t e0 = h + nfg * kGroup;
    const f32x4 a = ld_f32x4(gin + e0, L.c32), b = ld_f32x4(gin + e0, L.c32 + 16);
    const float g[kVec] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    adam8<PDT, FORM, PARAM>(c, g, w, m, v, par, e0, L);
  }
  if (blockIdx.x == 0) adam_scalars<PDT, FORM, PARAM>(c, gin, w, m, v, par, len, h, nvec);
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

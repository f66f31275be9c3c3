// zs_fused.h -- the single-tensor fused step kernels; zs_fused_f16.hip and
// zs_fused_bf16.hip instantiate them per gradient dtype.

#pragma once

#include "zs_device.h"

namespace zs {
namespace {

// Rounds of chunks between soft barriers (117M-element, 64-rank shard, 8
// rounds: every 2, 3 or 4 rounds 2.686 / 2.683 / 2.692 ms against 2.723 with
// none; every round no gain).
constexpr int kFusedSoftRounds = 3;

// Single-tensor fused step, one workgroup per CU.  The loop over whole chunks
// (nearly all of the bytes) is written out in the kernel body instead of going
// through helper functions: when the per-group sums cross a function
// boundary by reference, the callee is optimised on its own before inlining
// and the compiler peels the first rank out of the rank loop; the resulting
// schedule measured about 11% slower on MI355X (3.17 ms against 2.85 ms on a
// 117M-element, 64-rank shard) with bit-identical results.  Kept in this
// shape, the rank loop tests r == 0 per group and keeps a single loop body.
//
// The whole chunks keep the contiguous lane map (8 consecutive elements per
// lane, one 16-byte load per rank and group) rather than the full-group map
// of the other kernels.  Measured on the 117M-element, 64-rank shard, the
// full-group map makes each phase faster alone (reads 2.33 -> 2.29 ms,
// update 0.67 -> 0.60 ms) but the step slower (2.78 -> 2.85-2.89 ms): its
// dense full-line store bursts overlap worse with other CUs' read phases.
// Stored as they lie, this map's fp32 values would fill half of every cache
// line per store instruction (5% of the written bytes were repeated); a
// cross-lane swap before the stores (st_f32x8_lines) makes each instruction
// write whole lines, and the step 1.4% faster.  The loop is sensitive to its
// exact shape: scheduling barriers that force each load's issue order made
// it 9% slower (3.03 ms), and swapping the state loads the same way 6%.
template <int GDT, int PDT, int FORM, int PMAX>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_kernel(GradArgs<PMAX> ga, int p, float* __restrict__ w, float* __restrict__ m,
                  float* __restrict__ v, uint16_t* __restrict__ par, int64_t len, int head,
                  Consts c, const void* rank_table) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = rank_grads(rank_table);
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  const uint32_t lane16 = threadIdx.x * 16u;
  const uint32_t lane32 = threadIdx.x * 32u;
  const SwapOffs so = swap_offs(lane32);
  __shared__ __attribute__((aligned(16))) unsigned char copy_lds[kCopyStage];
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const int64_t nfull = whole_chunks(nvec / kFull, gridDim.x);
  // rounds of one whole chunk per workgroup, a soft barrier every
  // kFusedSoftRounds rounds
  const int64_t nrounds = (nfull + gridDim.x - 1) / gridDim.x;
  for (int64_t rd = 0; rd < nrounds; ++rd) {
    if (rd > 0 && rd % kFusedSoftRounds == 0)
      soft_barrier(static_cast<int>(rd / kFusedSoftRounds));
    const int64_t ch = blockIdx.x + rd * gridDim.x;
    if (ch >= nfull) continue;
    const int64_t g0 = ch * kFull;
    float s[kGroupsMax][kVec];
    // read phase: rank-major, kLoadBatch loads in flight per batch
    for (int r = 0; r < p; ++r) {
      const uint16_t* base = gr.get(r) + h + g0 * kVec;
      // Group 0 alone first, and used before the other loads go out: the
      // first access to this rank's pages takes the address-translation miss
      // with one load per wave waiting on it, not a whole batch (a batch
      // queued behind the miss fills the per-CU translation queue and stalls
      // every wave's loads).
      {
        const u32x4 q0 = ld_grad(base, lane16);
        __builtin_amdgcn_sched_barrier(0);
        if (r == 0) {
          init8<GDT>(s[0], q0);
        } else {
          fold8<GDT>(s[0], q0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {  // groups 1 .. kLoadBatch-1
        u32x4 q[kLoadBatch - 1];
#pragma unroll
        for (int u = 0; u < kLoadBatch - 1; ++u)
          q[u] = ld_grad(base + static_cast<int64_t>(1 + u) * kBlock * kVec, lane16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kLoadBatch - 1; ++u) {
          if (r == 0) {
            init8<GDT>(s[1 + u], q[u]);
          } else {
            fold8<GDT>(s[1 + u], q[u]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u0 = kLoadBatch; u0 < kGroupsMax; u0 += kLoadBatch) {
        u32x4 q[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u)
          q[u] = ld_grad(base + static_cast<int64_t>(u0 + u) * kBlock * kVec, lane16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          if (r == 0) {
            init8<GDT>(s[u0 + u], q[u]);
          } else {
            fold8<GDT>(s[u0 + u], q[u]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // update phase: mean, Adam, stores, group by group; state stores as whole
    // lines (1 KiB per wave instruction)
    if constexpr (FORM == kStandard || FORM == kPage1Literal) {
      // Each group's Adam in two halves: the m and v stores go out after the
      // moments, then the next group's state loads, then the weight
      // arithmetic and the w store, so the stores leave in two bursts and the
      // next loads are in flight during the divisions.  The working copy goes
      // to LDS (stage_copy) and out on whole lines after the chunk
      // (flush_copy).
      const int64_t eb = h + g0 * kVec;
      unsigned char* const pc = reinterpret_cast<unsigned char*>(par + eb);
      const uint32_t dl = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(pc) & 127u);
      const uint32_t ys = lane16 + (dl & ~7u);
      __syncthreads();  // the previous chunk's flush has read the staged copy
      f32x4 nw0 = ld_f32x4(w + eb, lane32), nw1 = ld_f32x4(w + eb, lane32 + 16);
      f32x4 nm0 = ld_f32x4(m + eb, lane32), nm1 = ld_f32x4(m + eb, lane32 + 16);
      f32x4 nv0 = ld_f32x4(v + eb, lane32), nv1 = ld_f32x4(v + eb, lane32 + 16);
#pragma unroll
      for (int u = 0; u < kGroupsMax; ++u) {
        const int64_t e0 = h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec;
        float* wb = w + e0;
        float* mb = m + e0;
        float* vb = v + e0;
        float W[kVec] = {nw0.x, nw0.y, nw0.z, nw0.w, nw1.x, nw1.y, nw1.z, nw1.w};
        float M[kVec] = {nm0.x, nm0.y, nm0.z, nm0.w, nm1.x, nm1.y, nm1.z, nm1.w};
        float V[kVec] = {nv0.x, nv0.y, nv0.z, nv0.w, nv1.x, nv1.y, nv1.z, nv1.w};
        float g[kVec], MH[kVec], VH[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) g[j] = s[u][j] / c.PF;
        adam_moments8<FORM>(c, g, M, V, MH, VH);
        st_f32x8_lines(mb, so, M);
        st_f32x8_lines(vb, so, V);
        __builtin_amdgcn_sched_barrier(0);
        if (u + 1 < kGroupsMax) {
          nw0 = ld_f32x4(wb + kGroup, lane32);
          nw1 = ld_f32x4(wb + kGroup, lane32 + 16);
          nm0 = ld_f32x4(mb + kGroup, lane32);
          nm1 = ld_f32x4(mb + kGroup, lane32 + 16);
          nv0 = ld_f32x4(vb + kGroup, lane32);
          nv1 = ld_f32x4(vb + kGroup, lane32 + 16);
        }
        __builtin_amdgcn_sched_barrier(0);
        adam_weights8(c, MH, VH, W);
        st_f32x8_lines(wb, so, W);
        stage_copy(copy_lds, static_cast<uint32_t>(u) * (kBlock * kVec * 2) + ys,
                   u32x4{narrow2<PDT>(W[0], W[1]), narrow2<PDT>(W[2], W[3]),
                         narrow2<PDT>(W[4], W[5]), narrow2<PDT>(W[6], W[7])});
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      flush_copy(copy_lds, pc - dl, dl);
    } else {
#pragma unroll
      for (int u = 0; u < kGroupsMax; ++u) {
        const int64_t e0 = h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec;
        float* wb = w + e0;
        float* mb = m + e0;
        const f32x4 w0 = ld_f32x4(wb, lane32), w1 = ld_f32x4(wb, lane32 + 16);
        const f32x4 m0 = ld_state<kUsesM<FORM>>(mb, lane32);
        const f32x4 m1 = ld_state<kUsesM<FORM>>(mb, lane32 + 16);
        float W[kVec] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float M[kVec] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        float V[kVec] = {};  // unused by the SGD forms
#pragma unroll
        for (int j = 0; j < kVec; ++j) adam1<FORM>(c, s[u][j] / c.PF, W[j], M[j], V[j]);
        st_f32x8_lines(wb, so, W);
        if constexpr (kUsesM<FORM>) st_f32x8_lines(mb, so, M);
        st_u16x8(par + e0, lane16,
                 u32x4{narrow2<PDT>(W[0], W[1]), narrow2<PDT>(W[2], W[3]),
                       narrow2<PDT>(W[4], W[5]), narrow2<PDT>(W[6], W[7])});
      }
    }
  }
  fused_rest<GDT, PDT, FORM>(gr, p, w, m, v, par, len, h, nvec, nfull * kFull, nfull, c,
                             blockIdx.x, gridDim.x, lanes());
}

// Single-tensor fused step for shards under half a whole chunk per CU, where
// fused_kernel would run no whole chunk at all: the same pieces of two
// groups, dealt over three workgroups per CU (three waves per SIMD, 168
// registers: no spills), in the full-group lane map with rank batches of 4.
// On the 16-rank, 6.25M-element shards: 63.2 us, against 63.8 with four
// workgroups per CU (128 registers, 5 spilled), 66.6 with the contiguous map
// and batches of 8, 68.8 with the contiguous map and batches of 4; one
// workgroup per CU was 4% slower.
template <int GDT, int PDT, int FORM, int PMAX>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kSmallWaves)))
void small_kernel(GradArgs<PMAX> ga, int p, float* __restrict__ w, float* __restrict__ m,
                  float* __restrict__ v, uint16_t* __restrict__ par, int64_t len, int head,
                  Consts c, const void* rank_table) {
  (void)ga;  // read through the kernel-argument segment, see kernarg_grads()
  const ArgGrads gr = rank_grads(rank_table);
  const int64_t h = head < len ? head : len;
  const int64_t nvec = (len - h) / kVec;
  fused_rest<GDT, PDT, FORM, 4>(gr, p, w, m, v, par, len, h, nvec, 0, 0, c, blockIdx.x,
                                gridDim.x, lanes());
}

}  // namespace

template <int GDT>
hipError_t launch_fused_g(const FusedLaunch& a) {
  // fused_kernel: one workgroup per CU (one wave per SIMD).  A shard under
  // half a whole chunk per CU would give it no whole chunk: small_kernel
  // deals that shard's pieces over kSmallWaves workgroups per CU, one piece
  // (two vectors per lane) per workgroup at least.
  const int64_t h = a.head < a.len ? a.head : a.len;
  const int64_t nvec = (a.len - h) / kVec;
  const int64_t cu = cu_count();
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const bool small = 2 * (nvec / kFull) < cu;
  int64_t grid, cap;
  if (small) {
    grid = (nvec + 2 * kBlock - 1) / (2 * kBlock);
    cap = cu * kSmallWaves;
  } else {
    grid = (nvec + kBlock - 1) / kBlock;
    cap = cu;
  }
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  with_dt(a.pdt, [&](auto H) {
    with_form(a.form, [&](auto F) {
      // with a device rank table the kernel arguments carry no pointers: the
      // smallest instance
      with_pmax(a.rank_table ? 1 : a.p, [&](auto PM) {
        constexpr int PMAX = decltype(PM)::value;
        GradArgs<PMAX> ga;
        for (int r = 0; r < PMAX; ++r) ga.g[r] = !a.rank_table && r < a.p ? a.grads[r] : nullptr;
        if (small)
          small_kernel<GDT, decltype(H)::value, decltype(F)::value, PMAX>
              <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                  ga, a.p, a.w, a.m, a.v, a.param, a.len, a.head, a.c, a.rank_table);
        else
          fused_kernel<GDT, decltype(H)::value, decltype(F)::value, PMAX>
              <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(
                  ga, a.p, a.w, a.m, a.v, a.param, a.len, a.head, a.c, a.rank_table);
      });
    });
  });
  return hipGetLastError();
}

}  // namespace zs

// zs_table.hip -- the multi-tensor chunk-table kernel and its launcher.

#include "zs_device.h"

namespace zs {
namespace {

// Multi-tensor fused step, one workgroup per CU, one wave per SIMD: for each
// chunk-table entry, the whole chunks of the entry, then its rest, by the
// block that took the entry.  The body is the single-tensor kernel's (see
// fused_kernel below for why it is written out rather than factored).
template <int GDT, int PDT, int FORM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void table_kernel(TableSrc src, int p, Consts c0, const StepTableDev* st) {
  // The step's constants: by value, or the step table's current entry
  // (launches captured once and replayed).  Past the table's end the launch
  // does nothing and flags the table.
  Consts c = c0;
  if (st) {
    const int64_t at = st->cursor;
    if (at < 0 || at >= st->nsteps) {
      if (blockIdx.x == 0 && threadIdx.x == 0) const_cast<StepTableDev*>(st)->exhausted = 1;
      return;
    }
    c = step_consts(st)[at];
  }
  const uint32_t lane16 = threadIdx.x * 16u;
  const uint32_t lane32 = threadIdx.x * 32u;
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  for (int64_t item = src.first(); item < src.count(); item += src.stride()) {
    const auto R = src.open(item);
    const auto& gr = R.gr;
    float* const w = R.w;
    float* const m = R.m;
    float* const v = R.v;
    uint16_t* const par = R.par;
    const int64_t h = R.head < R.len ? R.head : R.len;
    const int64_t nvec = (R.len - h) / kVec;
    const int64_t nfull = whole_chunks(nvec / kFull, R.nblk);
    for (int64_t ch = R.blk; ch < nfull; ch += R.nblk) {
      const int64_t g0 = ch * kFull;
      float s[kGroupsMax][kVec];
      // read phase: rank-major, kTableLoadBatch loads in flight per batch
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
        {  // groups 1 .. kTableLoadBatch-1
          u32x4 q[kTableLoadBatch - 1];
#pragma unroll
          for (int u = 0; u < kTableLoadBatch - 1; ++u)
            q[u] = ld_grad(base + static_cast<int64_t>(1 + u) * kBlock * kVec, lane16);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kTableLoadBatch - 1; ++u) {
            if (r == 0) {
              init8<GDT>(s[1 + u], q[u]);
            } else {
              fold8<GDT>(s[1 + u], q[u]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u0 = kTableLoadBatch; u0 < kGroupsMax; u0 += kTableLoadBatch) {
          u32x4 q[kTableLoadBatch];
#pragma unroll
          for (int u = 0; u < kTableLoadBatch; ++u)
            q[u] = ld_grad(base + static_cast<int64_t>(u0 + u) * kBlock * kVec, lane16);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kTableLoadBatch; ++u) {
            if (r == 0) {
              init8<GDT>(s[u0 + u], q[u]);
            } else {
              fold8<GDT>(s[u0 + u], q[u]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // update phase: mean, Adam, stores, kUG groups at a time.  One group,
      // as in fused_kernel: with two groups' state loads in flight the 8-rank
      // Llama-3-8B shard ran 0.7% slower and wrote 11% more bytes to HBM than
      // the model (one group: 4.5%).
      constexpr int kUG = 1;
      static_assert(kGroupsMax % kUG == 0, "whole update batches per chunk");
#pragma unroll
      for (int u0 = 0; u0 < kGroupsMax; u0 += kUG) {
        f32x4 A[kUG][6];
#pragma unroll
        for (int q = 0; q < kUG; ++q) {
          const int64_t e0 = h + (g0 + static_cast<int64_t>(u0 + q) * kBlock) * kVec;
          A[q][0] = ld_f32x4(w + e0, lane32);
          A[q][1] = ld_f32x4(w + e0, lane32 + 16);
          A[q][2] = ld_state<kUsesM<FORM>>(m + e0, lane32);
          A[q][3] = ld_state<kUsesM<FORM>>(m + e0, lane32 + 16);
          A[q][4] = ld_state<kUsesV<FORM>>(v + e0, lane32);
          A[q][5] = ld_state<kUsesV<FORM>>(v + e0, lane32 + 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kUG; ++q) {
          const int u = u0 + q;
          const int64_t e0 = h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec;
          float W[kVec] = {A[q][0].x, A[q][0].y, A[q][0].z, A[q][0].w, A[q][1].x, A[q][1].y, A[q][1].z, A[q][1].w};
          float M[kVec] = {A[q][2].x, A[q][2].y, A[q][2].z, A[q][2].w, A[q][3].x, A[q][3].y, A[q][3].z, A[q][3].w};
          float V[kVec] = {A[q][4].x, A[q][4].y, A[q][4].z, A[q][4].w, A[q][5].x, A[q][5].y, A[q][5].z, A[q][5].w};
#pragma unroll
          for (int j = 0; j < kVec; ++j) adam1<FORM>(c, s[u][j] / c.PF, W[j], M[j], V[j]);
          st_f32x4(w + e0, lane32, f32x4{W[0], W[1], W[2], W[3]});
          st_f32x4(w + e0, lane32 + 16, f32x4{W[4], W[5], W[6], W[7]});
          st_state<kUsesM<FORM>>(m + e0, lane32, f32x4{M[0], M[1], M[2], M[3]});
          st_state<kUsesM<FORM>>(m + e0, lane32 + 16, f32x4{M[4], M[5], M[6], M[7]});
          st_state<kUsesV<FORM>>(v + e0, lane32, f32x4{V[0], V[1], V[2], V[3]});
          st_state<kUsesV<FORM>>(v + e0, lane32 + 16, f32x4{V[4], V[5], V[6], V[7]});
          st_u16x8(par + e0, lane16,
                   u32x4{narrow2<PDT>(W[0], W[1]), narrow2<PDT>(W[2], W[3]),
                         narrow2<PDT>(W[4], W[5]), narrow2<PDT>(W[6], W[7])});
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // fp16 gradients take rank batches of 8 in the pieces: with 16 the
    // fp16 Adam instances spill 272 bytes; 8 leaves 44 and makes short-chunk
    // fp16 tables 5% faster (GPT-2 shard 7); bf16 keeps 16.
    fused_rest<GDT, PDT, FORM, GDT == kF16 ? 8 : 16>(gr, p, w, m, v, par, R.len, h, nvec,
                                                     nfull * kFull, nfull, c, R.blk, R.nblk,
                                                     lane16, lane32);
  }
}

}  // namespace

hipError_t launch_multi(const MultiLaunch& a) {
  int64_t grid = static_cast<int64_t>(cu_count());
  if (grid > a.nchunks) grid = a.nchunks;
  if (grid < 1) grid = 1;
  const TableSrc src{a.pieces, a.gptrs, a.chunks, a.nchunks, a.chunk_elems, a.p};
  with_dt(a.gdt, [&](auto G) {
    with_dt(a.pdt, [&](auto H) {
      with_form(a.form, [&](auto F) {
        table_kernel<decltype(G)::value, decltype(H)::value, decltype(F)::value>
            <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(src, a.p, a.c,
                                                                              a.steps);
      });
    });
  });
  return hipGetLastError();
}

}  // namespace zs

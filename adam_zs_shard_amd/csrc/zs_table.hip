// zs_table.hip -- the multi-tensor chunk-table kernel and its launcher.

#include "zs_device.h"

namespace zs {
namespace {

// Rounds of entries between soft barriers (8-rank Llama-3-8B shard, 69
// rounds: every 4, 5, 6 or 8 rounds 7.544 / 7.533 / 7.537 / 7.558 ms against
// 7.826 with none and 7.715 with a full grid-wide barrier every 12 rounds;
// every round 8.06).
constexpr int kTableSoftRounds = 6;

// Multi-tensor fused step, one workgroup per CU, one wave per SIMD: for each
// chunk-table entry, the whole chunks of the entry, then its rest, by the
// block that took the entry.  Entries go round-robin in rounds of gridDim.x,
// with a soft barrier every kTableSoftRounds rounds (every block takes it,
// with or without an entry in the round).  The body is the single-tensor
// kernel's (see fused_kernel for why it is written out rather than
// factored).
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
  const Lanes L = lanes();
  constexpr int64_t kFull = static_cast<int64_t>(kBlock) * kGroupsMax;
  const int64_t nrounds = (src.count() + src.stride() - 1) / src.stride();
  for (int64_t rd = 0; rd < nrounds; ++rd) {
    if (rd > 0 && rd % kTableSoftRounds == 0)
      soft_barrier(static_cast<int>(rd / kTableSoftRounds));
    const int64_t item = src.first() + rd * src.stride();
    if (item >= src.count()) continue;
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
          const G8 q0 = ld_g8(base, L);
          __builtin_amdgcn_sched_barrier(0);
          if (r == 0) {
            init8<GDT>(s[0], q0);
          } else {
            fold8<GDT>(s[0], q0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        {  // groups 1 .. kTableLoadBatch-1
          G8 q[kTableLoadBatch - 1];
#pragma unroll
          for (int u = 0; u < kTableLoadBatch - 1; ++u) {
            q[u] = ld_g8(base + (1 + u) * kGroup, L);
            __builtin_amdgcn_sched_barrier(0);  // issued in group order
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kTableLoadBatch - 1; ++u) {
            if (r == 0) {
              init8<GDT>(s[1 + u], q[u]);
            } else {
              fold8<GDT>(s[1 + u], q[u]);
            }
            __builtin_amdgcn_sched_barrier(0);  // fold in load order
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u0 = kTableLoadBatch; u0 < kGroupsMax; u0 += kTableLoadBatch) {
          G8 q[kTableLoadBatch];
#pragma unroll
          for (int u = 0; u < kTableLoadBatch; ++u) {
            q[u] = ld_g8(base + (u0 + u) * kGroup, L);
            __builtin_amdgcn_sched_barrier(0);  // issued in group order
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kTableLoadBatch; ++u) {
            if (r == 0) {
              init8<GDT>(s[u0 + u], q[u]);
            } else {
              fold8<GDT>(s[u0 + u], q[u]);
            }
            __builtin_amdgcn_sched_barrier(0);  // fold in load order
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // update phase: mean, Adam, stores, group by group (Adam: the next
      // group's state loads between each group's moment and weight halves)
      if constexpr (FORM == kStandard || FORM == kPage1Literal) {
        GroupState q = load_group<FORM>(L, w, m, v, h + g0 * kVec);
#pragma unroll
        for (int u = 0; u < kGroupsMax; ++u) {
          const int64_t e0 = h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec;
          GroupState qn = q;
          apply_group_pipe<PDT, FORM>(c, L, q, s[u], w, m, v, par, e0, u + 1 < kGroupsMax, qn);
          q = qn;
        }
      } else {
#pragma unroll
        for (int u = 0; u < kGroupsMax; ++u) {
          const int64_t e0 = h + (g0 + static_cast<int64_t>(u) * kBlock) * kVec;
          const GroupState q = load_group<FORM>(L, w, m, v, e0);
          apply_group<PDT, FORM>(c, L, q, s[u], w, m, v, par, e0);
        }
      }
    }
    // the rest in rank batches of 8 (1% faster than 16 on the 35-piece GPT-2
    // shard; with fp16 gradients, 16 spilled)
    fused_rest<GDT, PDT, FORM, 8>(gr, p, w, m, v, par, R.len, h, nvec, nfull * kFull, nfull, c,
                                  R.blk, R.nblk, L);
  }
}

// Tables whose entries are all shorter than a whole chunk (so table_kernel
// would run only its rest path): the same pieces of two groups, over two
// workgroups per CU (two waves per SIMD, 214 registers), rank batches of 16.
// On the 8-rank GPT-2 shards 2, 5 and 7 (16,384-element entries) 5-6%
// faster than table_kernel's one workgroup per CU; three workgroups per CU
// with batches of 4 gained 4%, four lost 2%.
constexpr int kTableRestWaves = 2;

template <int GDT, int PDT, int FORM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kTableRestWaves)))
void table_rest_kernel(TableSrc src, int p, Consts c0, const StepTableDev* st) {
  Consts c = c0;
  if (st) {
    const int64_t at = st->cursor;
    if (at < 0 || at >= st->nsteps) {
      if (blockIdx.x == 0 && threadIdx.x == 0) const_cast<StepTableDev*>(st)->exhausted = 1;
      return;
    }
    c = step_consts(st)[at];
  }
  const Lanes L = lanes();
  const int64_t nrounds = (src.count() + src.stride() - 1) / src.stride();
  for (int64_t rd = 0; rd < nrounds; ++rd) {
    const int64_t item = src.first() + rd * src.stride();
    if (item >= src.count()) continue;
    const auto R = src.open(item);
    const int64_t h = R.head < R.len ? R.head : R.len;
    const int64_t nvec = (R.len - h) / kVec;
    fused_rest<GDT, PDT, FORM, 16>(R.gr, p, R.w, R.m, R.v, R.par, R.len, h, nvec, 0, 0, c,
                                   R.blk, R.nblk, L);
  }
}

}  // namespace

hipError_t launch_multi(const MultiLaunch& a) {
  const TableSrc src{a.pieces, a.gptrs, a.chunks, a.nchunks, a.chunk_elems, a.p};
  const bool rest_only = a.chunk_elems < static_cast<int64_t>(kBlock) * kGroupsMax * kVec;
  int64_t grid = static_cast<int64_t>(cu_count()) * (rest_only ? kTableRestWaves : 1);
  if (grid > a.nchunks) grid = a.nchunks;
  if (grid < 1) grid = 1;
  if (rest_only) {
    with_dt(a.gdt, [&](auto G) {
      with_dt(a.pdt, [&](auto H) {
        with_form(a.form, [&](auto F) {
          table_rest_kernel<decltype(G)::value, decltype(H)::value, decltype(F)::value>
              <<<dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, a.stream>>>(src, a.p, a.c,
                                                                                a.steps);
        });
      });
    });
    return hipGetLastError();
  }
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

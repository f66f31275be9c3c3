// zs_probe.hip -- bandwidth probes for gfx950 (libzsprobe.so): plain stream
// kernels that read and write HBM in fixed ratios with no arithmetic beyond an
// XOR that keeps the loads live.  They are measurement tools, not part of
// the optimizer step: bench.py --ceiling times them to give the practical
// HBM ceiling of each read/write mix the step's workloads have.
//
// Layout: NR read streams and NW write streams, each `stream_bytes` apart
// inside one source and one destination allocation, each `nvec` 16-byte
// vectors long.  Every lane moves 16 bytes per stream per vector with
// non-temporal loads and stores (as the step's kernels do), so one wave
// instruction covers 1 KiB of contiguous memory.  Workgroups of 256 lanes
// walk the vectors grid-stride in units of U vectors per lane, all U x NR
// loads of a unit in flight before the first store.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zsprobe.h"
#include "zs_device.h"  // zs::soft_barrier, the library's pacing of whole-chunk rounds

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlock = 256;

template <int NR, int NW, int U>
__global__ __launch_bounds__(kBlock) void stream_kernel(const char* __restrict__ src,
                                                        char* __restrict__ dst,
                                                        int64_t stream_bytes, int64_t nvec,
                                                        u32x4* __restrict__ sink) {
  const int64_t lanes = static_cast<int64_t>(gridDim.x) * kBlock;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // whole units: vectors tid + j * lanes for j < U, then the next unit
  const int64_t unit = lanes * U;
  int64_t v0 = 0;
  for (; v0 + unit <= nvec; v0 += unit) {
    u32x4 q[NR][U];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int j = 0; j < U; ++j)
        q[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            src + r * stream_bytes) + v0 + j * lanes + tid);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      u32x4 x = q[0][j];
#pragma unroll
      for (int r = 1; r < NR; ++r) x ^= q[r][j];
      if constexpr (NW == 0) {
        acc ^= x;
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w)
          __builtin_nontemporal_store(x ^ static_cast<uint32_t>(w),
                                      reinterpret_cast<u32x4*>(dst + w * stream_bytes) + v0 +
                                          j * lanes + tid);
      }
    }
  }
  // the rest, one vector per lane at a time
  for (int64_t v = v0 + tid; v < nvec; v += lanes) {
    u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + v);
#pragma unroll
    for (int r = 1; r < NR; ++r)
      x ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * stream_bytes) + v);
    if constexpr (NW == 0) {
      acc ^= x;
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w)
        __builtin_nontemporal_store(x ^ static_cast<uint32_t>(w),
                                    reinterpret_cast<u32x4*>(dst + w * stream_bytes) + v);
    }
  }
  if constexpr (NW == 0) {
    if ((acc.x | acc.y | acc.z | acc.w) == 0x9e3779b9u) sink[tid & 255] = acc;  // keeps the loads
  }
}

// Phase-separated variant, one workgroup per CU: a workgroup takes chunks of
// G x 256 vectors per stream round-robin; for each read stream in turn it
// issues the G loads of the chunk back to back and folds them into G
// registers, then writes the G results to every write stream.  Reads and
// writes reach the memory in separate stretches, as in the step's
// whole-chunk kernels.
template <int NR, int NW, int G>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void phased_kernel(const char* __restrict__ src, char* __restrict__ dst, int64_t stream_bytes,
                   int64_t nvec, u32x4* __restrict__ sink) {
  constexpr int64_t kChunk = static_cast<int64_t>(G) * kBlock;
  const int64_t nchunk = nvec / kChunk;
  const int lane = threadIdx.x;
  u32x4 keep = {0u, 0u, 0u, 0u};
  for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
    const int64_t v0 = c * kChunk + lane;
    u32x4 acc[G];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      u32x4 q[G];
      const u32x4* sp = reinterpret_cast<const u32x4*>(src + r * stream_bytes) + v0;
#pragma unroll
      for (int u = 0; u < G; ++u) q[u] = __builtin_nontemporal_load(sp + u * kBlock);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < G; ++u) acc[u] = r == 0 ? q[u] : (acc[u] ^ q[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NW == 0) {
#pragma unroll
      for (int u = 0; u < G; ++u) keep ^= acc[u];
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        u32x4* dp = reinterpret_cast<u32x4*>(dst + w * stream_bytes) + v0;
#pragma unroll
        for (int u = 0; u < G; ++u)
          __builtin_nontemporal_store(acc[u] ^ static_cast<uint32_t>(w), dp + u * kBlock);
      }
    }
  }
  // vectors after the whole chunks, grid-stride
  for (int64_t v = nchunk * kChunk + static_cast<int64_t>(blockIdx.x) * kBlock + lane; v < nvec;
       v += static_cast<int64_t>(gridDim.x) * kBlock) {
    u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + v);
#pragma unroll
    for (int r = 1; r < NR; ++r)
      x ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * stream_bytes) + v);
    if constexpr (NW == 0) {
      keep ^= x;
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w)
        __builtin_nontemporal_store(x ^ static_cast<uint32_t>(w),
                                    reinterpret_cast<u32x4*>(dst + w * stream_bytes) + v);
    }
  }
  if constexpr (NW == 0) {
    if ((keep.x | keep.y | keep.z | keep.w) == 0x9e3779b9u) sink[lane] = keep;  // keeps the loads
  }
}

// The step's own read pattern and nothing else: P 16-bit rank buffers read
// in whole chunks of 28 groups of 2048 elements, round-robin over the
// workgroups; per chunk, rank by rank, each lane's first 16-byte load alone
// (its address translation taken with one load waiting), then the chunk's 27
// other loads back to back, every load widened (fp16) and added into fp32
// sums per element in rank order, as the fused step's read phase does.
constexpr int kStepGroups = 28;
constexpr int kStepRanks = 64;
struct StepRanks {
  const uint16_t* g[kStepRanks];
};

__device__ __forceinline__ float h_lo(uint32_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x & 0xffffu)));
}
__device__ __forceinline__ float h_hi(uint32_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(x >> 16)));
}
__device__ __forceinline__ void add8(float (&a)[8], const u32x4& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[2 * j] += h_lo(q[j]);
    a[2 * j + 1] += h_hi(q[j]);
  }
}

// PACED: rounds of one chunk per workgroup with the library's soft barrier
// every `pace` rounds; otherwise plain grid-stride over the chunks.
template <bool PACED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1)))
void step_reads_kernel(StepRanks R, int p, int64_t nchunks, int pace, u32x4* __restrict__ sink) {
  const uint32_t off = threadIdx.x * 16u;
  constexpr int64_t kChunk = static_cast<int64_t>(kStepGroups) * kBlock * 8;  // elements
  float keep = 0.0f;
  const int64_t nrounds = (nchunks + gridDim.x - 1) / gridDim.x;
  for (int64_t rd = 0; rd < nrounds; ++rd) {
    if constexpr (PACED) {
      if (rd > 0 && rd % pace == 0) zs::soft_barrier(static_cast<int>(rd / pace));
    }
    const int64_t ch = blockIdx.x + rd * gridDim.x;
    if (ch >= nchunks) continue;
    float s[kStepGroups][8];
#pragma unroll
    for (int u = 0; u < kStepGroups; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) s[u][j] = 0.0f;
    for (int r = 0; r < p; ++r) {
      const char* base = reinterpret_cast<const char*>(R.g[r] + ch * kChunk) + off;
      {
        const u32x4 q0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base));
        __builtin_amdgcn_sched_barrier(0);
        add8(s[0], q0);
        __builtin_amdgcn_sched_barrier(0);
      }
      u32x4 q[kStepGroups - 1];
#pragma unroll
      for (int u = 0; u < kStepGroups - 1; ++u)
        q[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(1 + u) * kBlock * 16));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kStepGroups - 1; ++u) add8(s[1 + u], q[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < kStepGroups; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) keep += s[u][j];
  }
  if (keep == 123456.0f) sink[threadIdx.x] = u32x4{1u, 2u, 3u, 4u};  // keeps the sums
}

template <int NR, int NW, int G>
hipError_t run_phased(const void* src, void* dst, int64_t stream_bytes, int64_t nvec, int grid,
                      void* sink, hipStream_t s) {
  phased_kernel<NR, NW, G><<<dim3(grid), dim3(kBlock), 0, s>>>(
      static_cast<const char*>(src), static_cast<char*>(dst), stream_bytes, nvec,
      static_cast<u32x4*>(sink));
  return hipGetLastError();
}

template <int NR, int NW, int U>
hipError_t run(const void* src, void* dst, int64_t stream_bytes, int64_t nvec, int grid,
               void* sink, hipStream_t s) {
  stream_kernel<NR, NW, U><<<dim3(grid), dim3(kBlock), 0, s>>>(
      static_cast<const char*>(src), static_cast<char*>(dst), stream_bytes, nvec,
      static_cast<u32x4*>(sink));
  return hipGetLastError();
}

}  // namespace

extern "C" {

int32_t zsp_stream(int32_t mix, const void* src, void* dst, int64_t stream_bytes, int64_t nvec,
                   int32_t grid, void* sink, void* stream) {
  if (!src || !sink || nvec < 0 || grid < 1 || stream_bytes < 16 * nvec) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (mix) {
    case ZSP_READ8: e = run<8, 0, 4>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_COPY: if (!dst) return 1; e = run<1, 1, 4>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_MIX_2_1: if (!dst) return 1; e = run<2, 1, 4>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_MIX_22_7: if (!dst) return 1; e = run<22, 7, 1>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_MIX_10_1: if (!dst) return 1; e = run<10, 1, 2>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_PHASED_READ8: e = run_phased<8, 0, 16>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_PHASED_COPY: if (!dst) return 1; e = run_phased<1, 1, 16>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_PHASED_2_1: if (!dst) return 1; e = run_phased<2, 1, 16>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_PHASED_22_7: if (!dst) return 1; e = run_phased<22, 7, 16>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_PHASED_10_1: if (!dst) return 1; e = run_phased<10, 1, 16>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    // pure reads: streams x loads in flight per stream
    case ZSP_READ1_U16: e = run<1, 0, 16>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_READ2_U8: e = run<2, 0, 8>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_READ4_U8: e = run<4, 0, 8>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_READ8_U8: e = run<8, 0, 8>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    case ZSP_READ1_U32: e = run<1, 0, 32>(src, dst, stream_bytes, nvec, grid, sink, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

static int32_t step_reads(const void* const* ranks, int32_t p, int64_t elems, int32_t grid,
                          int32_t pace, void* sink, void* stream) {
  if (!ranks || !sink || p < 1 || p > kStepRanks || elems < 0 || grid < 1 || pace < 0)
    return 1;
  StepRanks R;
  for (int r = 0; r < kStepRanks; ++r) {
    R.g[r] = r < p ? static_cast<const uint16_t*>(ranks[r]) : nullptr;
    if (r < p && !R.g[r]) return 1;
  }
  const int64_t nchunks = elems / (static_cast<int64_t>(kStepGroups) * kBlock * 8);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (pace > 0)
    step_reads_kernel<true><<<dim3(grid), dim3(kBlock), 0, s>>>(R, p, nchunks, pace,
                                                              static_cast<u32x4*>(sink));
  else
    step_reads_kernel<false><<<dim3(grid), dim3(kBlock), 0, s>>>(R, p, nchunks, 1,
                                                               static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int32_t zsp_step_reads(const void* const* ranks, int32_t p, int64_t elems, int32_t grid,
                       void* sink, void* stream) {
  return step_reads(ranks, p, elems, grid, 0, sink, stream);
}

int32_t zsp_step_reads_paced(const void* const* ranks, int32_t p, int64_t elems, int32_t grid,
                             int32_t pace_rounds, void* sink, void* stream) {
  if (pace_rounds < 1) return 1;
  return step_reads(ranks, p, elems, grid, pace_rounds, sink, stream);
}

int32_t zsp_streams(int32_t mix, int32_t* nread, int32_t* nwrite) {
  static const int32_t tab[][2] = {{8, 0}, {1, 1}, {2, 1}, {22, 7}, {10, 1},
                                   {8, 0}, {1, 1}, {2, 1}, {22, 7}, {10, 1},
                                   {1, 0}, {2, 0}, {4, 0}, {8, 0}, {1, 0}};
  if (mix < 0 || mix > ZSP_READ1_U32 || !nread || !nwrite) return 1;
  *nread = tab[mix][0];
  *nwrite = tab[mix][1];
  return 0;
}

}  // extern "C"

// zs_internal.h -- declarations shared by the host entry points and the HIP
// launchers of libzshard (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <vector>

#include "../../include/zshard.h"

namespace zs {

// Runs an entry point's body; a failure to obtain host memory or a thread
// (std::bad_alloc, std::system_error) becomes ZS_ERR_RESOURCE instead of an
// exception crossing the C interface.
template <class F>
zs_status guard(F&& f) noexcept {
  try {
    return f();
  } catch (...) {
    return ZS_ERR_RESOURCE;
  }
}


enum : int { kF16 = 1, kBF16 = 2 };
enum : int { kStandard = 0, kPage1Literal = 1, kSgd = 2, kSgdMomentum = 3 };

// Elements handled by one lane per vector group: 8 x 16-bit = one 16-byte
// load per gradient rank; 8 x fp32 = two 16-byte loads per state array.
constexpr int kVec = 8;
constexpr int kBlock = 256;             // 4 wave64 per workgroup
constexpr int kMaxP = 1024;             // matches ZS_MAX_P
// Ranks whose gradient pointers travel in one launch's kernel arguments
// (2 KiB of pointers); more ranks read their pointers from device memory.
constexpr int kKernargP = 256;

// The nine fp32 scalars of one step, each computed in double on the host and
// rounded once.
struct Consts {
  float B1, C1, B2, C2, BC1, BC2, LR, EPS, PF;
};

struct FusedLaunch {
  const uint16_t* grads[kMaxP];  // rank r's gradient at the shard's first element
  // Device array of the p pointers above (filled on the stream before the
  // step), or null: then p <= kKernargP and they go as kernel arguments.
  const uint16_t* const* rank_table;
  int p;
  int gdt, pdt, form;
  float* w;
  float* m;
  float* v;
  uint16_t* param;               // working copy at the shard's first element
  int64_t len;
  int head;                      // scalar elements before the first vector group
  Consts c;
  hipStream_t stream;
};

// One pass of the stored mean over up to kKernargP consecutive ranks.  The
// fp32 sums of the ranks before the pass (acc, or null on the first pass)
// are continued in rank order; the last pass divides by P and stores the
// mean as fp32 (odt 0) or rounded to nearest even in 16 bits (kF16 /
// kBF16), an earlier pass stores the fp32 partial sums.
struct MeanLaunch {
  const uint16_t* grads[kKernargP];
  int p;                  // ranks in this pass
  int gdt;
  int odt;
  const float* acc;
  void* out;
  int last;
  int64_t len;
  int head;
  float PF;               // f32(P), all ranks
  hipStream_t stream;
};

struct AdamLaunch {
  const float* g;
  float* w;
  float* m;
  float* v;
  uint16_t* param;  // may be null
  int pdt, form;
  int64_t len;
  int head;
  Consts c;
  hipStream_t stream;
};

// Device-side layout of a multi-tensor launch table (in the caller's
// workspace).  Sections start on 256-byte boundaries.
struct MtPiece {
  float* w;
  float* m;
  float* v;
  uint16_t* param;
  int64_t len;
  int32_t head;     // alignment head of the piece (elements, 0..7)
  int32_t reserved;
};
struct MtChunk {
  int32_t piece;
  int32_t reserved;
  int64_t start;    // first element of the chunk inside its piece
};
struct MtLayout {
  size_t pieces_off, gptr_off, chunks_off, total;
};
MtLayout mt_layout(int32_t npieces, int64_t nchunks, int32_t p);

// Step constants kept in device memory, for launches captured once and
// replayed: each launch applies entry `cursor`; a one-thread kernel advances
// the cursor after the step's launches.  A launch that finds the cursor at or
// past nsteps does nothing and sets `exhausted`.
struct StepTableDev {
  int64_t cursor;
  int64_t nsteps;
  int32_t exhausted;
  int32_t form;
  int32_t p;
  int32_t reserved;
  int64_t first_step;
  // followed by nsteps Consts entries at byte offset kStepTableHead
};
constexpr size_t kStepTableHead = 48;
__host__ __device__ inline const Consts* step_consts(const StepTableDev* t) {
  return reinterpret_cast<const Consts*>(reinterpret_cast<const char*>(t) + kStepTableHead);
}

struct MultiLaunch {
  const StepTableDev* steps;      // or null: the constants below
  const MtPiece* pieces;
  const uint16_t* const* gptrs;   // npieces * p pointers, piece-major
  const MtChunk* chunks;
  int64_t nchunks;
  int64_t chunk_elems;
  int p;
  int gdt, pdt, form;
  Consts c;
  hipStream_t stream;
};

hipError_t launch_fused(const FusedLaunch& a);
hipError_t launch_fused_f16(const FusedLaunch& a);
hipError_t launch_fused_bf16(const FusedLaunch& a);
hipError_t launch_mean(const MeanLaunch& a);
// The stored mean of len elements (grads[r] at the first one), in passes of
// up to kKernargP ranks: fp32 (odt 0, acc_buf = out) or rounded to 16 bits
// (acc_buf: fp32 sums between passes, needed when p > kKernargP).
hipError_t mean_range(const uint16_t* const* grads, int32_t p, int32_t gdt, int64_t len, int head,
                      void* out, int32_t odt, float* acc_buf, hipStream_t stream);
hipError_t launch_adam(const AdamLaunch& a);
hipError_t launch_multi(const MultiLaunch& a);
// dst[i] = src[i] for i < n (n <= kKernargP), on the stream.
hipError_t launch_rank_table(const uint16_t* const* src, int n, const uint16_t** dst,
                             hipStream_t stream);
// cursor += 1 in a step table, one thread.
hipError_t launch_step_advance(StepTableDev* t, hipStream_t stream);

// Elements (0..7) to peel before the first 8-element group so that the
// given 16-bit (a16) and fp32 (a32) streams, weighted by their bytes, start
// their groups as close to whole 128-byte lines as possible.
int choose_head(const std::vector<uintptr_t>& a16, const std::vector<uintptr_t>& a32);

// Bytes of the library's static device scratch (one copy per GPU): the rank
// pointer table of up to kMaxP ranks for the allocation-free fused step.
constexpr size_t kStaticScratchBytes = static_cast<size_t>(kMaxP) * sizeof(void*);
// Device address of the current device's static scratch, looked up once per
// device with that device current (hipGetSymbolAddress) and cached.
hipError_t static_scratch(void** out);

// Records e as this thread's last HIP error (zs_last_hip_error) and returns
// ZS_ERR_HIP.
int32_t hip_status(hipError_t e);

// Compute units of the current device (cached per device).
int cu_count();

}  // namespace zs

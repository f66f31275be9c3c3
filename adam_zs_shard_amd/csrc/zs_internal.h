// zs_internal.h -- declarations shared by the host entry points and the HIP
// launchers of libzshard (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace zs {

enum : int { kF16 = 1, kBF16 = 2 };
enum : int { kStandard = 0, kPage1Literal = 1, kSgd = 2, kSgdMomentum = 3 };

// Elements handled by one lane per vector group: 8 x 16-bit = one 16-byte
// load per gradient rank; 8 x fp32 = two 16-byte loads per state array.
constexpr int kVec = 8;
constexpr int kBlock = 256;             // 4 wave64 per workgroup
constexpr int kMaxP = 256;              // matches ZS_MAX_P

// The nine fp32 scalars of one step, each computed in double on the host and
// rounded once.
struct Consts {
  float B1, C1, B2, C2, BC1, BC2, LR, EPS, PF;
};

struct FusedLaunch {
  const uint16_t* grads[kMaxP];  // rank r's gradient at the shard's first element
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

struct MeanLaunch {
  const uint16_t* grads[kMaxP];
  int p;
  int gdt;
  float* out;
  int64_t len;
  int head;
  float PF;
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

struct MultiLaunch {
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
hipError_t launch_mean(const MeanLaunch& a);
hipError_t launch_adam(const AdamLaunch& a);
hipError_t launch_multi(const MultiLaunch& a);

// Compute units of the current device (cached per device).
int cu_count();

}  // namespace zs

// zs_common.hip -- device queries shared by the launchers.

#include "zs_device.h"

#include <mutex>

namespace zs {

// The allocation-free fused step's scratch: the rank pointer table, written
// by rank_table_kernel and read by the step's kernels.  Each GPU holds its own
// copy for the life of the process.  Host code must not use this name as an
// address (in host code it is a stand-in, not device memory): it takes the
// address from static_scratch() below.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};   // per device, guarded by g_scratch_mu

// Copies the n <= kKernargP rank pointers of this launch's kernel arguments
// into a device array, one pointer per lane.  The pointers are read through
// the kernel-argument segment (the by-value table is its first argument).
__global__ __launch_bounds__(kBlock) void rank_table_kernel(GradArgs<kKernargP> ga, int n,
                                                            const uint16_t** dst) {
  (void)ga;
  const KernargTable t = kernarg_grads().t;
  const int i = threadIdx.x;
  if (i < n) dst[i] = t[i];
}

// One thread: the step table's cursor moves to the next entry.
__global__ void step_advance_kernel(StepTableDev* st) {
  if (threadIdx.x == 0 && blockIdx.x == 0) st->cursor = st->cursor + 1;
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

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // once per device, with that device current: its own copy's address
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_rank_table(const uint16_t* const* src, int n, const uint16_t** dst,
                             hipStream_t stream) {
  GradArgs<kKernargP> ga;
  for (int r = 0; r < kKernargP; ++r) ga.g[r] = r < n ? src[r] : nullptr;
  rank_table_kernel<<<dim3(1), dim3(kBlock), 0, stream>>>(ga, n, dst);
  return hipGetLastError();
}

hipError_t launch_step_advance(StepTableDev* t, hipStream_t stream) {
  step_advance_kernel<<<dim3(1), dim3(64), 0, stream>>>(t);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedLaunch& a) {
  return a.gdt == kF16 ? launch_fused_f16(a) : launch_fused_bf16(a);
}

}  // namespace zs

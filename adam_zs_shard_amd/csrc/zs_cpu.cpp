// zs_cpu.cpp -- the optimizer-offload update of one shard on the host CPU.
//
// [ZA] §2.2 Offload 策略: the data-flow graph is cut along the 16-bit
// gradient and 16-bit parameter edges, so the GPU sends the shard's 16-bit
// gradient to host memory, the CPU runs the "Update Super Node" (Adam on the
// fp32 master weights and moments kept in host memory, then float2half), and
// the 16-bit parameters go back.  [ZA] §1.6.2 Optimizer Offload: the CPU side
// uses multithreading + SIMD so that it is not the bottleneck; in the
// multi-GPU case each GPU's 1/N shard has its own CPU process (§2.3 扩展性).
//
// The arithmetic is the canonical per-element sequence of the GPU path, on
// 8 lanes at a time with AVX2 and F16C: exact 16 -> 32-bit widening, every
// product, sum, quotient and square root rounded once to nearest-even (no
// FMA: the file is compiled with -ffp-contract=off), round-to-nearest-even
// downcast.  Each worker sets MXCSR to round-to-nearest with denormals kept.
// The 0..7 tail elements of a range go through the same 8-lane code on a
// padded copy, so there is no second arithmetic path.

#include <immintrin.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "zshard.h"

namespace {

constexpr int kF16 = ZS_F16;
constexpr int kBF16 = ZS_BF16;
constexpr uint32_t kMxcsrNearestNoFtz = 0x1F80u;  // all exceptions masked, RN, no FTZ/DAZ

struct HostConsts {
  float B1, C1, B2, C2, BC1, BC2, LR, EPS;
};

// Each constant computed in double and rounded once to fp32.
HostConsts host_consts(const zs_adam_hparams& hp) {
  const double t = static_cast<double>(hp.step);
  HostConsts c;
  c.B1 = static_cast<float>(hp.beta1);
  c.C1 = static_cast<float>(1.0 - hp.beta1);
  c.B2 = static_cast<float>(hp.beta2);
  c.C2 = static_cast<float>(1.0 - hp.beta2);
  c.BC1 = static_cast<float>(1.0 - std::pow(hp.beta1, t));
  c.BC2 = static_cast<float>(1.0 - std::pow(hp.beta2, t));
  c.LR = static_cast<float>(hp.lr);
  c.EPS = static_cast<float>(hp.eps);
  return c;
}

struct Job {
  const uint16_t* g;
  float* w;
  float* m;
  float* v;
  uint16_t* param;  // may be null
  HostConsts c;
};

#define ZS_AVX2 __attribute__((target("avx2,f16c")))

template <int GDT>
ZS_AVX2 inline __m256 widen8(const uint16_t* p) {
  const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i*>(p));
  if constexpr (GDT == kF16) {
    return _mm256_cvtph_ps(h);  // exact
  } else {
    return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
  }
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN of the same sign.
ZS_AVX2 inline __m128i to_bf16_8(__m256 x) {
  const __m256i b = _mm256_castps_si256(x);
  const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(b, 16), _mm256_set1_epi32(1));
  const __m256i rounded =
      _mm256_srli_epi32(_mm256_add_epi32(b, _mm256_add_epi32(_mm256_set1_epi32(0x7FFF), lsb)), 16);
  const __m256i mag = _mm256_and_si256(b, _mm256_set1_epi32(0x7FFFFFFF));
  const __m256i is_nan = _mm256_cmpgt_epi32(mag, _mm256_set1_epi32(0x7F800000));
  const __m256i quiet = _mm256_or_si256(_mm256_srli_epi32(b, 16), _mm256_set1_epi32(0x40));
  const __m256i r = _mm256_blendv_epi8(rounded, quiet, is_nan);
  // 8 x 32-bit (each < 2^16) -> 8 x 16-bit, in order
  const __m256i packed = _mm256_packus_epi32(r, r);
  return _mm256_castsi256_si128(_mm256_permute4x64_epi64(packed, 0x08));
}

template <int PDT>
ZS_AVX2 inline void narrow8(uint16_t* p, __m256 x) {
  __m128i h;
  if constexpr (PDT == kF16) {
    h = _mm256_cvtps_ph(x, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
  } else {
    h = to_bf16_8(x);
  }
  _mm_storeu_si128(reinterpret_cast<__m128i*>(p), h);
}

// One update of 8 elements (the order of the canonical sequence).
template <int FORM>
ZS_AVX2 inline void update8(const HostConsts& c, __m256 g, __m256& w, __m256& m, __m256& v) {
  const __m256 LR = _mm256_set1_ps(c.LR), B1 = _mm256_set1_ps(c.B1);
  if constexpr (FORM == ZS_SGD) {
    w = _mm256_sub_ps(w, _mm256_mul_ps(LR, g));
  } else if constexpr (FORM == ZS_SGD_MOMENTUM) {
    m = _mm256_add_ps(_mm256_mul_ps(B1, m), g);
    w = _mm256_sub_ps(w, _mm256_mul_ps(LR, m));
  } else {
    const __m256 mm = _mm256_add_ps(_mm256_mul_ps(B1, m), _mm256_mul_ps(_mm256_set1_ps(c.C1), g));
    const __m256 vv = _mm256_add_ps(_mm256_mul_ps(_mm256_set1_ps(c.B2), v),
                                    _mm256_mul_ps(_mm256_set1_ps(c.C2), _mm256_mul_ps(g, g)));
    __m256 mh, vh;
    if constexpr (FORM == ZS_ADAM_STANDARD) {
      m = mm;
      v = vv;
      mh = _mm256_div_ps(mm, _mm256_set1_ps(c.BC1));
      vh = _mm256_div_ps(vv, _mm256_set1_ps(c.BC2));
    } else {
      m = _mm256_div_ps(mm, _mm256_set1_ps(c.BC1));
      v = _mm256_div_ps(vv, _mm256_set1_ps(c.BC2));
      mh = m;
      vh = v;
    }
    const __m256 d = _mm256_add_ps(_mm256_sqrt_ps(vh), _mm256_set1_ps(c.EPS));
    w = _mm256_sub_ps(w, _mm256_mul_ps(LR, _mm256_div_ps(mh, d)));
  }
}

template <int FORM>
constexpr bool kUsesM = FORM != ZS_SGD;
template <int FORM>
constexpr bool kUsesV = FORM == ZS_ADAM_STANDARD || FORM == ZS_ADAM_PAGE1_LITERAL;

// Elements [i, i+8) from (g, w, m, v) at those addresses.
template <int GDT, int PDT, int FORM>
ZS_AVX2 inline void step8(const HostConsts& c, const uint16_t* g, float* w, float* m, float* v,
                          uint16_t* param) {
  __m256 W = _mm256_loadu_ps(w);
  __m256 M = kUsesM<FORM> ? _mm256_loadu_ps(m) : _mm256_setzero_ps();
  __m256 V = kUsesV<FORM> ? _mm256_loadu_ps(v) : _mm256_setzero_ps();
  update8<FORM>(c, widen8<GDT>(g), W, M, V);
  _mm256_storeu_ps(w, W);
  if constexpr (kUsesM<FORM>) _mm256_storeu_ps(m, M);
  if constexpr (kUsesV<FORM>) _mm256_storeu_ps(v, V);
  if (param) narrow8<PDT>(param, W);
}

template <int GDT, int PDT, int FORM>
ZS_AVX2 void run_range(const Job& j, int64_t lo, int64_t hi) {
  const unsigned int saved = _mm_getcsr();
  _mm_setcsr(kMxcsrNearestNoFtz);
  int64_t i = lo;
  for (; i + 8 <= hi; i += 8)
    step8<GDT, PDT, FORM>(j.c, j.g + i, j.w + i, kUsesM<FORM> ? j.m + i : nullptr,
                          kUsesV<FORM> ? j.v + i : nullptr, j.param ? j.param + i : nullptr);
  if (i < hi) {  // the tail, through the same 8-lane code on a padded copy
    const int64_t n = hi - i;
    alignas(32) uint16_t g8[8] = {0}, p8[8] = {0};
    alignas(32) float w8[8] = {0}, m8[8] = {0}, v8[8] = {0};
    std::memcpy(g8, j.g + i, 2 * n);
    std::memcpy(w8, j.w + i, 4 * n);
    if (kUsesM<FORM>) std::memcpy(m8, j.m + i, 4 * n);
    if (kUsesV<FORM>) std::memcpy(v8, j.v + i, 4 * n);
    step8<GDT, PDT, FORM>(j.c, g8, w8, m8, v8, j.param ? p8 : nullptr);
    std::memcpy(j.w + i, w8, 4 * n);
    if (kUsesM<FORM>) std::memcpy(j.m + i, m8, 4 * n);
    if (kUsesV<FORM>) std::memcpy(j.v + i, v8, 4 * n);
    if (j.param) std::memcpy(j.param + i, p8, 2 * n);
  }
  _mm_setcsr(saved);
}

using RangeFn = void (*)(const Job&, int64_t, int64_t);

template <int GDT, int PDT>
RangeFn pick_form(int form) {
  switch (form) {
    case ZS_ADAM_STANDARD: return run_range<GDT, PDT, ZS_ADAM_STANDARD>;
    case ZS_ADAM_PAGE1_LITERAL: return run_range<GDT, PDT, ZS_ADAM_PAGE1_LITERAL>;
    case ZS_SGD: return run_range<GDT, PDT, ZS_SGD>;
    default: return run_range<GDT, PDT, ZS_SGD_MOMENTUM>;
  }
}

RangeFn pick(int gdt, int pdt, int form) {
  if (gdt == kF16) return pdt == kF16 ? pick_form<kF16, kF16>(form) : pick_form<kF16, kBF16>(form);
  return pdt == kF16 ? pick_form<kBF16, kF16>(form) : pick_form<kBF16, kBF16>(form);
}

bool cpu_ok() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
}

struct Span {
  uintptr_t lo, hi;
};
bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace

namespace {

zs_status cpu_adam_body(const void* g, int32_t grad_dtype, float* w, float* m, float* v,
                        void* param, int32_t param_dtype, int64_t len, const zs_adam_hparams* hp,
                        int32_t threads) {
  if (!hp) return ZS_ERR_NULL;
  if (len < 0) return ZS_ERR_ARG;
  if (len > (int64_t{1} << 60)) return ZS_ERR_RANGE;
  if (grad_dtype != ZS_F16 && grad_dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (param && param_dtype != ZS_F16 && param_dtype != ZS_BF16) return ZS_ERR_DTYPE;
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
      !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || hp->step < 1 || hp->reserved != 0 ||
      hp->form < ZS_ADAM_STANDARD || hp->form > ZS_SGD_MOMENTUM)
    return ZS_ERR_ARG;
  if (len == 0) return ZS_OK;
  const bool um = hp->form != ZS_SGD;
  const bool uv = hp->form == ZS_ADAM_STANDARD || hp->form == ZS_ADAM_PAGE1_LITERAL;
  if (!g || !w || (um && !m) || (uv && !v)) return ZS_ERR_NULL;
  const uintptr_t b32 = 4u * static_cast<uintptr_t>(len), b16 = 2u * static_cast<uintptr_t>(len);
  std::vector<Span> writes = {{reinterpret_cast<uintptr_t>(w), reinterpret_cast<uintptr_t>(w) + b32}};
  if (um) writes.push_back({reinterpret_cast<uintptr_t>(m), reinterpret_cast<uintptr_t>(m) + b32});
  if (uv) writes.push_back({reinterpret_cast<uintptr_t>(v), reinterpret_cast<uintptr_t>(v) + b32});
  if (param)
    writes.push_back({reinterpret_cast<uintptr_t>(param), reinterpret_cast<uintptr_t>(param) + b16});
  const Span rd{reinterpret_cast<uintptr_t>(g), reinterpret_cast<uintptr_t>(g) + b16};
  for (size_t i = 0; i < writes.size(); ++i) {
    if (overlap(writes[i], rd)) return ZS_ERR_ALIAS;
    for (size_t k = i + 1; k < writes.size(); ++k)
      if (overlap(writes[i], writes[k])) return ZS_ERR_ALIAS;
  }
  if (!cpu_ok()) return ZS_ERR_UNSUPPORTED;

  const Job job{static_cast<const uint16_t*>(g), w, m, v, static_cast<uint16_t*>(param),
                host_consts(*hp)};
  const RangeFn fn = pick(grad_dtype, param ? param_dtype : ZS_F16, hp->form);
  // Threads: as asked (<= 0: all hardware threads), at most one per 64 Ki
  // elements; contiguous ranges whose bounds are multiples of 16 elements
  // (one 64-byte line of fp32), so no two threads write the same line.
  int64_t nt = threads > 0 ? threads : static_cast<int64_t>(std::thread::hardware_concurrency());
  nt = std::max<int64_t>(1, std::min<int64_t>(nt, (len + 65535) / 65536));
  const int64_t per = ((len + nt - 1) / nt + 15) / 16 * 16;
  // Ranges 1.. go to new threads; if the system refuses a thread (or the
  // pool's memory), the calling thread runs the ranges not handed out.  The
  // result does not depend on which thread runs a range.
  std::vector<std::thread> pool;
  int64_t t_next = 1;
  try {
    pool.reserve(static_cast<size_t>(nt - 1));
    for (; t_next < nt; ++t_next) {
      const int64_t lo = std::min(len, t_next * per), hi = std::min(len, lo + per);
      if (lo < hi) pool.emplace_back(fn, std::cref(job), lo, hi);
    }
  } catch (...) {
  }
  fn(job, 0, std::min(len, per));
  for (int64_t t = t_next; t < nt; ++t) {
    const int64_t lo = std::min(len, t * per), hi = std::min(len, lo + per);
    if (lo < hi) fn(job, lo, hi);
  }
  for (auto& th : pool) th.join();
  return ZS_OK;
}

}  // namespace

extern "C" zs_status zs_cpu_adam_step(const void* g, int32_t grad_dtype, float* w, float* m,
                                      float* v, void* param, int32_t param_dtype, int64_t len,
                                      const zs_adam_hparams* hp, int32_t threads) {
  try {
    return cpu_adam_body(g, grad_dtype, w, m, v, param, param_dtype, len, hp, threads);
  } catch (...) {
    return ZS_ERR_RESOURCE;
  }
}

// zs_oracle.cpp -- CPU ORACLE for the per-shard ZeRO optimizer step.
//
// TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
// and the benchmark's CPU-baseline leg may load this library.  It shares no
// source, header, table or constant generator with the HIP library: it is a
// plain, slow, element-at-a-time restatement of what the pages define, meant
// to be checked against them by eye.
//
// Pages cited (by title):
//   [DP-III]  深度学习专题：模型训练的数据并行（三）  (blog.csdn.net, lybugproducer)
//   [ZP]      ZeRO 原理：把模型状态切到多张 GPU 上       (hsichen.pages.dev)
//   [ZA]      ZeRO 技术原理：进阶与 Offload              (jianzhnie.github.io llmtechsite)
//   [EAI19]   高效AI 第19讲：分布式训练（第一部分）      (bittide.aicompass.dev)
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fPIC -shared, with no
// -ffast-math and no -march option, so every float operation below is one
// SSE2 scalar instruction rounded once to nearest-even (no FMA, no x87
// excess precision, denormals kept), and sqrtf/divss are correctly rounded.
//
// Every function here has a pin in tests/ (closed forms, brute force, the
// pages' printed numbers, numpy/torch routines).  None is "parity unpinned".

#include <cfenv>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>

static_assert(FLT_EVAL_METHOD == 0, "float expressions must be evaluated in float");
static_assert(sizeof(float) == 4 && sizeof(double) == 8, "IEEE binary32/binary64 expected");

namespace {

enum { DT_F16 = 1, DT_BF16 = 2 };
enum { FORM_STANDARD = 0, FORM_PAGE1_LITERAL = 1, FORM_SGD = 2, FORM_SGD_MOMENTUM = 3 };

uint32_t bits_of(float x) { uint32_t b; std::memcpy(&b, &x, 4); return b; }
float float_of(uint32_t b) { float x; std::memcpy(&x, &b, 4); return x; }

// ---------------------------------------------------------------------------
// 16-bit formats.  The mixed-precision scheme keeps gradients and the working
// copy of the parameters in 16 bits and the optimizer state in fp32
// ([ZA] §1.4 显存分析; [ZP] 核心原理, "parameters(fp32) ... 转换成fp16").
// ---------------------------------------------------------------------------

// binary16 -> binary32, from the format definition: sign, 5-bit exponent with
// bias 15, 10-bit fraction.  Every binary16 value is exactly a binary32 value.
float f16_to_f32(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double mag;
  if (e == 31) {
    if (f != 0) return sign ? -NAN : NAN;
    mag = INFINITY;
  } else if (e == 0) {
    mag = std::ldexp(static_cast<double>(f), -24);              // 0.f * 2^-14
  } else {
    mag = std::ldexp(static_cast<double>(1024 + f), e - 25);    // 1.f * 2^(e-15)
  }
  return static_cast<float>(sign ? -mag : mag);
}

// bfloat16 is, by definition, the upper 16 bits of a binary32 encoding.
float bf16_to_f32(uint16_t h) { return float_of(static_cast<uint32_t>(h) << 16); }

// Round |x| to the nearest multiple of the format's quantum, ties to even,
// for a format with `mant` fraction bits and minimum normal exponent `emin`.
// Returns the integer significand r and updates the binade exponent e so that
// the rounded magnitude is r * 2^(e - mant).
void round_to_format(double a, int mant, int emin, int64_t* r_out, int* e_out) {
  int e2;
  std::frexp(a, &e2);  // a in [2^(e2-1), 2^e2)
  int e = e2 - 1;
  if (e < emin) e = emin;  // below the normal range the quantum stays 2^(emin-mant)
  const double q = std::ldexp(a, mant - e);  // exact: scaling by a power of two
  int64_t r = static_cast<int64_t>(std::nearbyint(q));  // default mode: ties to even
  if (r == (int64_t{2} << mant)) {  // rounding carried into the next binade
    r = int64_t{1} << mant;
    e += 1;
  }
  *r_out = r;
  *e_out = e;
}

// binary32 -> binary16, round to nearest, ties to even; overflow gives +-inf,
// subnormals are produced, NaN stays a (quiet) NaN with its sign.
uint16_t f32_to_f16(float x) {
  const uint16_t sign = static_cast<uint16_t>((bits_of(x) >> 16) & 0x8000u);
  if (std::isnan(x)) return sign | 0x7e00u;
  if (std::isinf(x)) return sign | 0x7c00u;
  const double a = std::fabs(static_cast<double>(x));
  if (a == 0.0) return sign;
  int64_t r;
  int e;
  round_to_format(a, 10, -14, &r, &e);
  if (e > 15) return sign | 0x7c00u;                      // beyond 65504 after rounding
  if (r < 1024) return sign | static_cast<uint16_t>(r);   // subnormal, biased exponent 0
  return sign | static_cast<uint16_t>(((e + 15) << 10) | (r - 1024));
}

// binary32 -> bfloat16 (8-bit exponent like binary32, 7 fraction bits), same rules.
uint16_t f32_to_bf16(float x) {
  const uint16_t sign = static_cast<uint16_t>((bits_of(x) >> 16) & 0x8000u);
  if (std::isnan(x)) return sign | 0x7fc0u;
  if (std::isinf(x)) return sign | 0x7f80u;
  const double a = std::fabs(static_cast<double>(x));
  if (a == 0.0) return sign;
  int64_t r;
  int e;
  round_to_format(a, 7, -126, &r, &e);
  if (e > 127) return sign | 0x7f80u;
  if (r < 128) return sign | static_cast<uint16_t>(r);
  return sign | static_cast<uint16_t>(((e + 127) << 7) | (r - 128));
}

float widen(int dt, uint16_t h) { return dt == DT_F16 ? f16_to_f32(h) : bf16_to_f32(h); }
uint16_t narrow(int dt, float x) { return dt == DT_F16 ? f32_to_f16(x) : f32_to_bf16(x); }
bool dtype_ok(int dt) { return dt == DT_F16 || dt == DT_BF16; }

// ---------------------------------------------------------------------------
// Shard plan.  [DP-III] §(三) ZeRO-1 优化原理, 1. 步骤分析 (repeated in §(四)
// and §(五)): each of P GPUs manages M = ceil(N/P) parameters; GPU k (1-based)
// owns parameters s_k = 1+(k-1)M .. e_k = kM (1-based, inclusive).
// Restated 0-based and half-open, rank k in [0,P) owns [k*M, (k+1)*M), with
// both ends clamped to N because the page leaves the last shard implicit.
// ---------------------------------------------------------------------------
struct Shard { int64_t m, s, e; };

Shard plan(int64_t n, int32_t p, int32_t k) {
  Shard sh;
  sh.m = (n + p - 1) / p;  // ceil(N/P) for N >= 0, P >= 1
  const int64_t s1 = 1 + static_cast<int64_t>(k) * sh.m;  // page's s_{k+1}, 1-based
  const int64_t e1 = static_cast<int64_t>(k + 1) * sh.m;  // page's e_{k+1}, inclusive
  sh.s = s1 - 1 < n ? s1 - 1 : n;
  sh.e = e1 < n ? e1 : n;
  return sh;
}

// ---------------------------------------------------------------------------
// Adam scalars, each derived in double and rounded once to fp32.
// [DP-III] §(一) Adam 优化器: beta1, beta2 are hyper-parameters (usually 0.9
// and 0.999), eps a small constant, lr the learning rate; the bias-correction
// denominators are 1 - beta^t for the step t being produced.
// ---------------------------------------------------------------------------
struct Scalars { float B1, C1, B2, C2, BC1, BC2, LR, EPS, PF; };

Scalars derive(double lr, double b1, double b2, double eps, int64_t t, int32_t p) {
  Scalars c;
  c.B1 = static_cast<float>(b1);
  c.C1 = static_cast<float>(1.0 - b1);
  c.B2 = static_cast<float>(b2);
  c.C2 = static_cast<float>(1.0 - b2);
  c.BC1 = static_cast<float>(1.0 - std::pow(b1, static_cast<double>(t)));
  c.BC2 = static_cast<float>(1.0 - std::pow(b2, static_cast<double>(t)));
  c.LR = static_cast<float>(lr);
  c.EPS = static_cast<float>(eps);
  c.PF = static_cast<float>(static_cast<double>(p));
  return c;
}

// Mean of the P ranks' gradients for one element.  [EAI19] 通信原语, All-Reduce
// 和 All-Gather: g = (1/N) sum_i g_i.  [DP-III] §(四) ZeRO-2 step 2: the rank
// obtains elements s_k..e_k of every rank's gradient (reduce-scatter) and
// forms their mean.  Sum in fp32, left to right in rank order 0..P-1 starting
// from rank 0's value, then one division by P.
float mean_of(int gdt, int32_t p, const uint16_t* const* g, int64_t idx, float PF) {
  float s = widen(gdt, g[0][idx]);
  for (int32_t r = 1; r < p; ++r) s = s + widen(gdt, g[r][idx]);
  return s / PF;
}

// One Adam update of one element, in place on (w, m, v).
//   first moment   mm = beta1*m + (1-beta1)*g
//   second moment  vv = beta2*v + (1-beta2)*g^2
//   STANDARD: store the raw moving averages ([ZA] §1.1.1: exponentially
//     weighted moving averages of the gradient and its square; Kingma & Ba,
//     cited there as ref. 10) and bias-correct at use: mh = m/(1-b1^t),
//     vh = v/(1-b2^t).
//   PAGE1_LITERAL: [DP-III] §(一) moment/variance equations taken literally,
//     m_{t+1} = (b1 m_t + (1-b1) g)/(1-b1^{t+1}) and likewise v: the stored
//     moments are the corrected ones and are used as they are.
//   update  w' = w - lr * mh / (sqrt(vh) + eps)   ([DP-III] §(一) update
//     equation: eps added outside the square root).
// Each operation is rounded once, in the order written.
//
// The two SGD forms ride on the same call (m, v are left alone when unused):
//   SGD: w' = w - lr * g   ([DP-III] §(一), the SGD update equation).
//   SGD_MOMENTUM: m' = beta1*m + g; w' = w - lr * m'.  [ZA] §1.1.1 names
//     SGD with momentum and its stored momentum buffer but prints no formula;
//     this is the plain heavy-ball reading, coefficient beta1, m0 = 0.
void adam_one(const Scalars& c, int form, float g, float* w, float* m, float* v) {
  if (form == FORM_SGD) {
    *w = *w - (c.LR * g);
    return;
  }
  if (form == FORM_SGD_MOMENTUM) {
    *m = (c.B1 * *m) + g;
    *w = *w - (c.LR * *m);
    return;
  }
  const float mm = (c.B1 * *m) + (c.C1 * g);
  const float vv = (c.B2 * *v) + (c.C2 * (g * g));
  float mh, vh;
  if (form == FORM_STANDARD) {
    *m = mm;
    *v = vv;
    mh = *m / c.BC1;
    vh = *v / c.BC2;
  } else {
    *m = mm / c.BC1;
    *v = vv / c.BC2;
    mh = *m;
    vh = *v;
  }
  const float d = std::sqrt(vh) + c.EPS;
  const float u = mh / d;
  *w = *w - (c.LR * u);
}

bool hparams_ok(double lr, double b1, double b2, double eps, int64_t t, int form) {
  return std::isfinite(lr) && std::isfinite(eps) && b1 >= 0.0 && b1 < 1.0 && b2 >= 0.0 &&
         b2 < 1.0 && t >= 1 && form >= FORM_STANDARD && form <= FORM_SGD_MOMENTUM;
}

bool nearest_mode() { return std::fegetround() == FE_TONEAREST; }

}  // namespace

extern "C" {

// Status codes: 0 ok, 2 bad argument, 3 bad dtype, 8 rounding mode not nearest.

float oracle_f16_to_f32(uint16_t h) { return f16_to_f32(h); }
float oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }
uint16_t oracle_f32_to_f16(float x) { return f32_to_f16(x); }
uint16_t oracle_f32_to_bf16(float x) { return f32_to_bf16(x); }

int32_t oracle_widen(int32_t dt, const uint16_t* in, float* out, int64_t n) {
  if (!dtype_ok(dt)) return 3;
  for (int64_t i = 0; i < n; ++i) out[i] = widen(dt, in[i]);
  return 0;
}

int32_t oracle_narrow(int32_t dt, const float* in, uint16_t* out, int64_t n) {
  if (!dtype_ok(dt)) return 3;
  if (!nearest_mode()) return 8;
  for (int64_t i = 0; i < n; ++i) out[i] = narrow(dt, in[i]);
  return 0;
}

// M and, if the arrays are given, every rank's [s_k, e_k).
int32_t oracle_plan_shards(int64_t n, int32_t p, int64_t* m_out, int64_t* starts, int64_t* ends) {
  if (n < 0 || p < 1) return 2;
  for (int32_t k = 0; k < p; ++k) {
    const Shard sh = plan(n, p, k);
    if (m_out) *m_out = sh.m;
    if (starts) starts[k] = sh.s;
    if (ends) ends[k] = sh.e;
  }
  return 0;
}

// The nine fp32 scalars in the order B1 C1 B2 C2 BC1 BC2 LR EPS PF.
int32_t oracle_adam_scalars(double lr, double b1, double b2, double eps, int64_t t, int32_t p,
                            float* out9) {
  if (!hparams_ok(lr, b1, b2, eps, t, 0) || p < 1) return 2;
  const Scalars c = derive(lr, b1, b2, eps, t, p);
  const float v[9] = {c.B1, c.C1, c.B2, c.C2, c.BC1, c.BC2, c.LR, c.EPS, c.PF};
  std::memcpy(out9, v, sizeof v);
  return 0;
}

// fp32 mean over P ranks of n elements; grads[r] points at element 0 of the range.
int32_t oracle_grad_mean(int32_t gdt, int32_t p, const uint16_t* const* grads, int64_t n,
                         float* g_out) {
  if (!dtype_ok(gdt)) return 3;
  if (p < 1 || n < 0) return 2;
  const float PF = static_cast<float>(static_cast<double>(p));
  for (int64_t i = 0; i < n; ++i) g_out[i] = mean_of(gdt, p, grads, i, PF);
  return 0;
}

// Adam on n elements from an fp32 gradient; param (may be NULL) receives the
// 16-bit working copy of the updated weight ([ZP] 核心原理: the new fp32
// parameters are converted to fp16 to replace the working copy; [ZA] §2.2:
// the "Param update" and "float2half" nodes).
int32_t oracle_adam_apply(const float* g, float* w, float* m, float* v, uint16_t* param,
                          int32_t pdt, int64_t n, double lr, double b1, double b2, double eps,
                          int64_t t, int32_t form) {
  if (param && !dtype_ok(pdt)) return 3;
  if (!hparams_ok(lr, b1, b2, eps, t, form) || n < 0) return 2;
  if (!nearest_mode()) return 8;
  const Scalars c = derive(lr, b1, b2, eps, t, 1);
  for (int64_t i = 0; i < n; ++i) {
    adam_one(c, form, g[i], &w[i], &m[i], &v[i]);
    if (param) param[i] = narrow(pdt, w[i]);
  }
  return 0;
}

// The whole per-shard step on n elements given as compact arrays: grads[r]
// points at element 0 for rank r, w/m/v/param hold the same n elements.
int32_t oracle_step_elems(int32_t gdt, int32_t p, const uint16_t* const* grads, float* w,
                          float* m, float* v, uint16_t* param, int32_t pdt, int64_t n, double lr,
                          double b1, double b2, double eps, int64_t t, int32_t form) {
  if (!dtype_ok(gdt) || !dtype_ok(pdt)) return 3;
  if (p < 1 || n < 0 || !hparams_ok(lr, b1, b2, eps, t, form)) return 2;
  if (!nearest_mode()) return 8;
  const Scalars c = derive(lr, b1, b2, eps, t, p);
  for (int64_t i = 0; i < n; ++i) {
    const float g = mean_of(gdt, p, grads, i, c.PF);
    adam_one(c, form, g, &w[i], &m[i], &v[i]);
    param[i] = narrow(pdt, w[i]);
  }
  return 0;
}

// The per-shard step with the global index map.  Rank k of P over N
// parameters owns [s_k, e_k); element i of its w/m/v is global index
// j = s_k + i; rank r's gradient for j is grads[r][j - grad_base]; the working
// copy for j is param[j - param_base].  [DP-III] §(四) ZeRO-2 steps 2-4.
int32_t oracle_shard_step(int64_t n, int32_t p, int32_t k, const uint16_t* const* grads,
                          int32_t gdt, int64_t grad_base, float* w, float* m, float* v,
                          uint16_t* param, int32_t pdt, int64_t param_base, double lr, double b1,
                          double b2, double eps, int64_t t, int32_t form) {
  if (!dtype_ok(gdt) || !dtype_ok(pdt)) return 3;
  if (n < 0 || p < 1 || k < 0 || k >= p || !hparams_ok(lr, b1, b2, eps, t, form)) return 2;
  if (!nearest_mode()) return 8;
  const Shard sh = plan(n, p, k);
  const Scalars c = derive(lr, b1, b2, eps, t, p);
  for (int64_t j = sh.s; j < sh.e; ++j) {
    const int64_t i = j - sh.s;
    const float g = mean_of(gdt, p, grads, j - grad_base, c.PF);
    adam_one(c, form, g, &w[i], &m[i], &v[i]);
    param[j - param_base] = narrow(pdt, w[i]);
  }
  return 0;
}

// Many parameter tensors flattened in list order (gradient buckets, [ZA] §1.4
// ZeRO-R buffers and §1.5): which tensor holds flat index j, by prefix sums
// over the tensor sizes.  Returns the tensor index and its offset, or -1.
int32_t oracle_locate(const int64_t* numel, int32_t ntensors, int64_t j, int64_t* off) {
  int64_t start = 0;
  for (int32_t t = 0; t < ntensors; ++t) {
    if (j >= start && j < start + numel[t]) {
      *off = j - start;
      return t;
    }
    start += numel[t];
  }
  return -1;
}

// The pieces in which the flat range [lo, hi) meets each tensor, in list
// order: tensor index, offset inside the tensor, offset inside [lo, hi), length.
// Returns the piece count, or -1 if more than cap pieces would be needed.
int32_t oracle_shard_pieces(const int64_t* numel, int32_t ntensors, int64_t lo, int64_t hi,
                            int32_t* tensor, int64_t* tensor_off, int64_t* range_off,
                            int64_t* len, int32_t cap) {
  int32_t count = 0;
  int64_t start = 0;
  for (int32_t t = 0; t < ntensors; ++t) {
    const int64_t end = start + numel[t];
    const int64_t a = lo > start ? lo : start;
    const int64_t b = hi < end ? hi : end;
    if (a < b) {
      if (count == cap) return -1;
      tensor[count] = t;
      tensor_off[count] = a - start;
      range_off[count] = a - lo;
      len[count] = b - a;
      ++count;
    }
    start = end;
  }
  return count;
}

// Mixed-precision model-state bytes per parameter on one of `ndev` devices:
// fp16 parameters (2 B) + fp16 gradients (2 B) + K bytes of fp32 Adam state
// (master weights, momentum, variance: K = 12).  [ZA] §1.4 显存分析:
// 16Φ replicated, 4Φ + 12Φ/N (P_os), 2Φ + (2Φ + 12Φ)/N (P_os+g), 16Φ/N
// (P_os+g+p); [EAI19] ZeRO 和 FSDP: 2+2+12, 2+2+12/N, 2+2/N+12/N, 16/N.
double oracle_mp_bytes_per_param(int32_t stage, double ndev, double k_bytes) {
  switch (stage) {
    case 0: return 2.0 + 2.0 + k_bytes;
    case 1: return 2.0 + 2.0 + k_bytes / ndev;
    case 2: return 2.0 + (2.0 + k_bytes) / ndev;
    case 3: return (2.0 + 2.0 + k_bytes) / ndev;
    default: return -1.0;
  }
}

// Floats stored per GPU in the page-1 accounting (parameters, gradient,
// momentum, variance; no separate fp32 master copy), M = ceil(N/P):
// scheme 0 data-parallel SGD 2N, 1 data-parallel Adam 4N ([DP-III] §(二)),
// 2 ZeRO-1 2M+2N (§(三).2), 3 ZeRO-2 3M+N (§(四).2), 4 ZeRO-3 4M (§(五).2).
double oracle_p1_floats(int32_t scheme, int64_t n, int32_t p) {
  if (n < 0 || p < 1) return -1.0;
  const double N = static_cast<double>(n);
  const double M = static_cast<double>((n + p - 1) / p);
  switch (scheme) {
    case 0: return 2.0 * N;
    case 1: return 4.0 * N;
    case 2: return 2.0 * M + 2.0 * N;
    case 3: return 3.0 * M + N;
    case 4: return 4.0 * M;
    default: return -1.0;
  }
}

}  // extern "C"

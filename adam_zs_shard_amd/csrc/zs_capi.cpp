// zs_capi.cpp -- the C ABI of libzshard: argument checks, the shard plan, the
// fp32 constants, the alignment head, and the calls into the HIP launchers.
// Every argument error is returned before anything touches the device.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <vector>

#include "../../include/zshard.h"
#include "zs_internal.h"

static_assert(ZS_MAX_P == zs::kMaxP, "ZS_MAX_P and the kernel table size must agree");
static_assert(ZS_KERNARG_P == zs::kKernargP, "ZS_KERNARG_P and the kernel arguments must agree");
static_assert(ZS_STATIC_SCRATCH_BYTES == zs::kStaticScratchBytes, "static scratch size");
static_assert(sizeof(zs::StepTableDev) <= zs::kStepTableHead, "step table layout");

namespace {

thread_local int32_t g_last_hip_error = 0;

zs_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int32_t>(e);
  return ZS_ERR_HIP;
}

bool dtype_ok(int32_t dt) { return dt == ZS_F16 || dt == ZS_BF16; }

// Largest n accepted: keeps every byte offset (4 * n) far inside int64.
constexpr int64_t kMaxN = int64_t{1} << 60;

zs_status check_hparams(const zs_adam_hparams* hp) {
  if (!hp) return ZS_ERR_NULL;
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps)) return ZS_ERR_ARG;
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return ZS_ERR_ARG;
  if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return ZS_ERR_ARG;
  if (hp->step < 1) return ZS_ERR_ARG;
  if (hp->form < ZS_ADAM_STANDARD || hp->form > ZS_SGD_MOMENTUM) return ZS_ERR_ARG;
  if (hp->reserved != 0) return ZS_ERR_ARG;
  return ZS_OK;
}

// Optimizer state a form reads and writes: Adam m and v, momentum SGD m,
// plain SGD neither.
bool needs_m(int32_t form) { return form != ZS_SGD; }
bool needs_v(int32_t form) { return form == ZS_ADAM_STANDARD || form == ZS_ADAM_PAGE1_LITERAL; }

// fp32 constants of one step: each computed in double and rounded once.
zs::Consts make_consts(const zs_adam_hparams& hp, int32_t p) {
  zs::Consts c;
  const double t = static_cast<double>(hp.step);
  c.B1 = static_cast<float>(hp.beta1);
  c.C1 = static_cast<float>(1.0 - hp.beta1);
  c.B2 = static_cast<float>(hp.beta2);
  c.C2 = static_cast<float>(1.0 - hp.beta2);
  c.BC1 = static_cast<float>(1.0 - std::pow(hp.beta1, t));
  c.BC2 = static_cast<float>(1.0 - std::pow(hp.beta2, t));
  c.LR = static_cast<float>(hp.lr);
  c.EPS = static_cast<float>(hp.eps);
  c.PF = static_cast<float>(static_cast<double>(p));
  return c;
}

// M = ceil(n/p); rank k: [min(kM, n), min((k+1)M, n)).
void shard_bounds(int64_t n, int32_t p, int32_t k, int64_t* m, int64_t* s, int64_t* e) {
  const int64_t mm = n / p + (n % p != 0 ? 1 : 0);
  const int64_t lo = static_cast<int64_t>(k) * mm;
  const int64_t hi = lo + mm;
  *m = mm;
  *s = lo < n ? lo : n;
  *e = hi < n ? hi : n;
}

struct Range {
  uintptr_t lo, hi;
};
bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

size_t rank_table_bytes(int32_t p) {
  if (p <= ZS_KERNARG_P || p > ZS_MAX_P) return 0;
  return (static_cast<size_t>(p) * sizeof(void*) + 255u) & ~static_cast<size_t>(255u);
}

// Writes the p rank pointers into a device array, in launches of up to
// kKernargP pointers each, on the stream.
hipError_t fill_rank_table(const uint16_t* const* ptrs, int32_t p, void* dst, hipStream_t st) {
  auto** d = static_cast<const uint16_t**>(dst);
  for (int32_t r0 = 0; r0 < p; r0 += zs::kKernargP) {
    const int n = std::min<int32_t>(zs::kKernargP, p - r0);
    const hipError_t e = zs::launch_rank_table(ptrs + r0, n, d + r0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* zs_status_string(int32_t status) {
  switch (status) {
    case ZS_OK: return "ZS_OK";
    case ZS_ERR_NULL: return "ZS_ERR_NULL";
    case ZS_ERR_ARG: return "ZS_ERR_ARG";
    case ZS_ERR_DTYPE: return "ZS_ERR_DTYPE";
    case ZS_ERR_RANGE: return "ZS_ERR_RANGE";
    case ZS_ERR_ALIAS: return "ZS_ERR_ALIAS";
    case ZS_ERR_CAPACITY: return "ZS_ERR_CAPACITY";
    case ZS_ERR_HIP: return "ZS_ERR_HIP";
    case ZS_ERR_UNSUPPORTED: return "ZS_ERR_UNSUPPORTED";
    case ZS_ERR_RESOURCE: return "ZS_ERR_RESOURCE";
    default: return "ZS_ERR_UNKNOWN";
  }
}

int32_t zs_version(void) { return ZS_VERSION; }

int32_t zs_last_hip_error(void) { return g_last_hip_error; }

zs_status zs_plan_shards(int64_t n, int32_t p, int64_t* m_out, int64_t* starts, int64_t* ends) {
  if (n < 0 || p < 1) return ZS_ERR_ARG;
  if (n > kMaxN) return ZS_ERR_RANGE;
  for (int32_t k = 0; k < p; ++k) {
    int64_t m, s, e;
    shard_bounds(n, p, k, &m, &s, &e);
    if (m_out) *m_out = m;
    if (starts) starts[k] = s;
    if (ends) ends[k] = e;
  }
  return ZS_OK;
}

size_t zs_shard_workspace_bytes(int32_t p) { return rank_table_bytes(p); }

}  // extern "C"

namespace {

// The fused step; the rank pointer table of p > ZS_KERNARG_P ranks goes to
// the caller's workspace, or (use_static) to the library's static scratch.
zs_status fused_impl(const zs_shard_args* a, bool use_static) {
  if (!a) return ZS_ERR_NULL;
  if (a->p < 1 || a->p > ZS_MAX_P || a->k < 0 || a->k >= a->p || a->n < 0) return ZS_ERR_ARG;
  if (a->n > kMaxN) return ZS_ERR_RANGE;
  if (!dtype_ok(a->grad_dtype) || !dtype_ok(a->param_dtype)) return ZS_ERR_DTYPE;
  if (const zs_status st = check_hparams(a->hp)) return st;
  if (!a->grads) return ZS_ERR_NULL;
  int64_t m, s, e;
  shard_bounds(a->n, a->p, a->k, &m, &s, &e);
  const int64_t len = e - s;
  if (a->grad_base < 0 || a->grad_base > s || a->param_base < 0 || a->param_base > s)
    return ZS_ERR_RANGE;
  if (len == 0) return ZS_OK;
  const bool um = needs_m(a->hp->form), uv = needs_v(a->hp->form);
  if (!a->w || !a->param || (um && !a->m) || (uv && !a->v)) return ZS_ERR_NULL;
  for (int32_t r = 0; r < a->p; ++r)
    if (!a->grads[r]) return ZS_ERR_NULL;

  zs::FusedLaunch L;
  L.p = a->p;
  L.gdt = a->grad_dtype;
  L.pdt = a->param_dtype;
  L.form = a->hp->form;
  L.w = a->w;
  L.m = a->m;
  L.v = a->v;
  L.param = static_cast<uint16_t*>(a->param) + (s - a->param_base);
  L.len = len;
  L.c = make_consts(*a->hp, a->p);
  L.stream = static_cast<hipStream_t>(a->stream);

  std::vector<uintptr_t> a16, a32;
  std::vector<Range> reads;
  for (int32_t r = 0; r < a->p; ++r) {
    L.grads[r] = static_cast<const uint16_t*>(a->grads[r]) + (s - a->grad_base);
    const uintptr_t g0 = reinterpret_cast<uintptr_t>(L.grads[r]);
    reads.push_back({g0, g0 + 2u * static_cast<uintptr_t>(len)});
    a16.push_back(g0);
  }
  const uintptr_t pw = reinterpret_cast<uintptr_t>(L.w), pm = reinterpret_cast<uintptr_t>(L.m),
                  pv = reinterpret_cast<uintptr_t>(L.v),
                  pp = reinterpret_cast<uintptr_t>(L.param);
  const uintptr_t b32 = 4u * static_cast<uintptr_t>(len), b16 = 2u * static_cast<uintptr_t>(len);
  // only the buffers the form writes are checked (and used to pick the head)
  std::vector<Range> writes = {{pw, pw + b32}, {pp, pp + b16}};
  a32 = {pw};
  if (um) {
    writes.push_back({pm, pm + b32});
    a32.push_back(pm);
  }
  if (uv) {
    writes.push_back({pv, pv + b32});
    a32.push_back(pv);
  }
  for (size_t i = 0; i < writes.size(); ++i) {
    for (size_t j = i + 1; j < writes.size(); ++j)
      if (overlap(writes[i], writes[j])) return ZS_ERR_ALIAS;
    for (const Range& rd : reads)
      if (overlap(writes[i], rd)) return ZS_ERR_ALIAS;
  }
  a16.push_back(pp);
  L.head = zs::choose_head(a16, a32);
  L.rank_table = nullptr;
  if (a->p > ZS_KERNARG_P) {
    const size_t need = rank_table_bytes(a->p);
    void* table = nullptr;
    if (use_static) {
      if (need > zs::kStaticScratchBytes) return ZS_ERR_CAPACITY;
      const hipError_t e = zs::static_scratch(&table);
      if (e != hipSuccess) return hip_fail(e);
    } else {
      const uintptr_t pw_ = reinterpret_cast<uintptr_t>(a->workspace);
      if (!a->workspace || a->workspace_bytes < need || pw_ % 16u != 0) return ZS_ERR_CAPACITY;
      const Range wsr{pw_, pw_ + need};
      for (const Range& wr : writes)
        if (overlap(wsr, wr)) return ZS_ERR_ALIAS;
      for (const Range& rd : reads)
        if (overlap(wsr, rd)) return ZS_ERR_ALIAS;
      table = a->workspace;
    }
    L.rank_table = static_cast<const uint16_t* const*>(table);
    const hipError_t e = fill_rank_table(L.grads, a->p, table, L.stream);
    if (e != hipSuccess) return hip_fail(e);
  }

  const hipError_t err = zs::launch_fused(L);
  if (err != hipSuccess) return hip_fail(err);
  return ZS_OK;
}

}  // namespace

extern "C" {

zs_status zs_fused_shard_step(const zs_shard_args* a) {
  return zs::guard([&] { return fused_impl(a, false); });
}

zs_status zs_fused_shard_step_static(const zs_shard_args* a) {
  return zs::guard([&] { return fused_impl(a, true); });
}

}  // extern "C"

namespace {

// The stored mean, fp32 (odt 0) or rounded to 16 bits, in passes of up to
// kKernargP ranks; between passes the fp32 sums live in `partial` (g_out
// itself for an fp32 output).
zs_status mean_impl(const void* const* grads, int32_t grad_dtype, int64_t grad_base, int64_t n,
                    int32_t p, int32_t k, void* g_out, int32_t odt, float* partial,
                    void* stream) {
  if (p < 1 || p > ZS_MAX_P || k < 0 || k >= p || n < 0) return ZS_ERR_ARG;
  if (n > kMaxN) return ZS_ERR_RANGE;
  if (!dtype_ok(grad_dtype) || (odt != 0 && !dtype_ok(odt))) return ZS_ERR_DTYPE;
  if (!grads) return ZS_ERR_NULL;
  int64_t m, s, e;
  shard_bounds(n, p, k, &m, &s, &e);
  const int64_t len = e - s;
  if (grad_base < 0 || grad_base > s) return ZS_ERR_RANGE;
  if (len == 0) return ZS_OK;
  if (!g_out) return ZS_ERR_NULL;
  for (int32_t r = 0; r < p; ++r)
    if (!grads[r]) return ZS_ERR_NULL;
  const bool passes = p > ZS_KERNARG_P;
  float* acc_buf = odt == 0 ? static_cast<float*>(g_out) : partial;
  if (passes && !acc_buf) return ZS_ERR_NULL;

  const uintptr_t po = reinterpret_cast<uintptr_t>(g_out);
  const uintptr_t ob = (odt == 0 ? 4u : 2u) * static_cast<uintptr_t>(len);
  std::vector<Range> writes = {{po, po + ob}};
  const uintptr_t pa = reinterpret_cast<uintptr_t>(acc_buf);
  if (passes && odt != 0) {
    writes.push_back({pa, pa + 4u * static_cast<uintptr_t>(len)});
    if (overlap(writes[0], writes[1])) return ZS_ERR_ALIAS;
  }
  std::vector<const uint16_t*> gp(static_cast<size_t>(p));
  std::vector<uintptr_t> a16;
  for (int32_t r = 0; r < p; ++r) {
    gp[r] = static_cast<const uint16_t*>(grads[r]) + (s - grad_base);
    const uintptr_t g0 = reinterpret_cast<uintptr_t>(gp[r]);
    for (const Range& wr : writes)
      if (overlap(wr, Range{g0, g0 + 2u * static_cast<uintptr_t>(len)})) return ZS_ERR_ALIAS;
    a16.push_back(g0);
  }
  // the output is written once per element; an fp32 array weighs like the
  // state arrays, a 16-bit one like a gradient
  std::vector<uintptr_t> a32;
  if (odt == 0) a32.push_back(po); else a16.push_back(po);
  if (passes && odt != 0) a32.push_back(pa);

  const hipError_t err = zs::mean_range(gp.data(), p, grad_dtype, len, zs::choose_head(a16, a32),
                                        g_out, odt, acc_buf, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err);
  return ZS_OK;
}

}  // namespace

extern "C" {

zs_status zs_reduce_scatter_mean_local(const void* const* grads, int32_t grad_dtype,
                                       int64_t grad_base, int64_t n, int32_t p, int32_t k,
                                       float* g_out, void* stream) {
  return zs::guard(
      [&] { return mean_impl(grads, grad_dtype, grad_base, n, p, k, g_out, 0, nullptr, stream); });
}

zs_status zs_reduce_scatter_mean_local16(const void* const* grads, int32_t grad_dtype,
                                         int64_t grad_base, int64_t n, int32_t p, int32_t k,
                                         void* g_out, int32_t out_dtype, float* partial,
                                         void* stream) {
  if (!dtype_ok(out_dtype)) return ZS_ERR_DTYPE;
  return zs::guard([&] {
    return mean_impl(grads, grad_dtype, grad_base, n, p, k, g_out, out_dtype, partial, stream);
  });
}

static zs_status adam_step_body(const float* g, float* w, float* m, float* v, void* param,
                                int32_t param_dtype, int64_t len, const zs_adam_hparams* hp,
                                void* stream) {
  if (len < 0) return ZS_ERR_ARG;
  if (len > kMaxN) return ZS_ERR_RANGE;
  if (param && !dtype_ok(param_dtype)) return ZS_ERR_DTYPE;
  if (const zs_status st = check_hparams(hp)) return st;
  if (len == 0) return ZS_OK;
  const bool um = needs_m(hp->form), uv = needs_v(hp->form);
  if (!g || !w || (um && !m) || (uv && !v)) return ZS_ERR_NULL;
  const uintptr_t b32 = 4u * static_cast<uintptr_t>(len), b16 = 2u * static_cast<uintptr_t>(len);
  const uintptr_t pg = reinterpret_cast<uintptr_t>(g), pw = reinterpret_cast<uintptr_t>(w),
                  pm = reinterpret_cast<uintptr_t>(m), pv = reinterpret_cast<uintptr_t>(v),
                  pp = reinterpret_cast<uintptr_t>(param);
  std::vector<Range> writes = {{pw, pw + b32}};
  std::vector<uintptr_t> a32 = {pg, pw};
  if (um) {
    writes.push_back({pm, pm + b32});
    a32.push_back(pm);
  }
  if (uv) {
    writes.push_back({pv, pv + b32});
    a32.push_back(pv);
  }
  if (param) writes.push_back({pp, pp + b16});
  const Range rd{pg, pg + b32};
  for (size_t i = 0; i < writes.size(); ++i) {
    if (overlap(writes[i], rd)) return ZS_ERR_ALIAS;
    for (size_t j = i + 1; j < writes.size(); ++j)
      if (overlap(writes[i], writes[j])) return ZS_ERR_ALIAS;
  }
  zs::AdamLaunch L;
  L.g = g;
  L.w = w;
  L.m = m;
  L.v = v;
  L.param = static_cast<uint16_t*>(param);
  L.pdt = param ? param_dtype : ZS_F16;
  L.form = hp->form;
  L.len = len;
  L.c = make_consts(*hp, 1);
  L.stream = static_cast<hipStream_t>(stream);
  std::vector<uintptr_t> a16;
  if (param) a16.push_back(pp);
  L.head = zs::choose_head(a16, a32);
  const hipError_t err = zs::launch_adam(L);
  if (err != hipSuccess) return hip_fail(err);
  return ZS_OK;
}

zs_status zs_adam_step(const float* g, float* w, float* m, float* v, void* param,
                       int32_t param_dtype, int64_t len, const zs_adam_hparams* hp,
                       void* stream) {
  return zs::guard(
      [&] { return adam_step_body(g, w, m, v, param, param_dtype, len, hp, stream); });
}

// ---------------------------------------------------------------- multi

zs_status zs_plan_chunks(const int64_t* numel, int32_t ntensors, int32_t p, int32_t k,
                         int64_t chunk_elems, zs_piece* pieces, int32_t pieces_cap,
                         int32_t* npieces, int64_t* nchunks_out) {
  if (!npieces || (ntensors > 0 && !numel) || (pieces_cap > 0 && !pieces)) return ZS_ERR_NULL;
  if (ntensors < 0 || p < 1 || k < 0 || k >= p || pieces_cap < 0 || chunk_elems < 0)
    return ZS_ERR_ARG;
  int64_t n = 0;
  for (int32_t t = 0; t < ntensors; ++t) {
    if (numel[t] < 0) return ZS_ERR_ARG;
    n += numel[t];
    if (n > kMaxN) return ZS_ERR_RANGE;
  }
  int64_t m, s, e;
  shard_bounds(n, p, k, &m, &s, &e);
  // Walk the tensors with a running offset; each tensor [off, off + numel)
  // that meets [s, e) gives one piece.
  int32_t count = 0;
  int64_t chunks = 0;
  int64_t off = 0;
  for (int32_t t = 0; t < ntensors && off < e; ++t) {
    const int64_t lo = off > s ? off : s;
    const int64_t hi = off + numel[t] < e ? off + numel[t] : e;
    if (lo < hi) {
      if (count < pieces_cap) {
        zs_piece& pc = pieces[count];
        pc.tensor = t;
        pc.reserved = 0;
        pc.tensor_off = lo - off;
        pc.shard_off = lo - s;
        pc.len = hi - lo;
      }
      ++count;
      if (chunk_elems > 0) chunks += (hi - lo + chunk_elems - 1) / chunk_elems;
    }
    off += numel[t];
  }
  *npieces = count;
  if (nchunks_out) *nchunks_out = chunks;
  return count > pieces_cap ? ZS_ERR_CAPACITY : ZS_OK;
}

int64_t zs_mt_chunk_elems(int64_t shard_len, int32_t npieces, int32_t cu_count) {
  if (shard_len < 0 || npieces < 1) return 0;
  const int64_t cu = cu_count > 0 ? cu_count : zs::cu_count();
  constexpr int64_t whole = static_cast<int64_t>(zs::kBlock) * 28 * zs::kVec;  // 57,344
  if (shard_len >= 2 * whole * cu) return whole;
  const int64_t split = npieces == 1 ? cu : 4 * cu;
  const int64_t per = (shard_len + split - 1) / split;
  const int64_t c = (per + 2047) / 2048 * 2048;
  return c < 2048 ? 2048 : c;
}

zs_status zs_plan_buckets(const zs_piece* pieces, int32_t npieces, int64_t bucket_elems,
                          int32_t* bucket_of, int32_t* nbuckets) {
  if (!nbuckets || (npieces > 0 && (!pieces || !bucket_of))) return ZS_ERR_NULL;
  if (npieces < 0) return ZS_ERR_ARG;
  for (int32_t i = 0; i < npieces; ++i)
    if (pieces[i].len < 1) return ZS_ERR_ARG;
  int32_t b = 0;
  int64_t size = 0;
  for (int32_t i = 0; i < npieces; ++i) {
    bucket_of[i] = b;
    size += pieces[i].len;
    if (bucket_elems > 0 && size >= bucket_elems && i + 1 < npieces) {
      ++b;
      size = 0;
    }
  }
  *nbuckets = npieces > 0 ? b + 1 : 0;
  return ZS_OK;
}

}  // extern "C"

namespace zs {

int32_t hip_status(hipError_t e) { return hip_fail(e); }

// Elements to peel (0..7) before the first 8-element group, chosen for where
// the groups of each stream start.  A wave's access of a group covers 512 B
// (16-bit) or 1 KiB (fp32) of contiguous memory; when that span starts on a
// 128-byte line it moves whole lines, otherwise its first and last lines are
// partial, which HBM serves at a cost (the update alone on a 117M-element
// shard: 0.660 ms with every stream line-aligned, 0.675 with the 16-bit
// working copy 48 bytes into a line, 0.739 with the fp32 arrays 16 bytes into
// one).  So each stream scores by the alignment of its group starts: 128
// bytes 8, 64 bytes 6, 16 bytes 2 (an aligned 16-byte lane access), 8 bytes 1,
// weighted by its bytes per element: 2 for a 16-bit stream (gradients read,
// the working copy written), 8 for an fp32 array (the state, read and
// written).
int choose_head(const std::vector<uintptr_t>& a16, const std::vector<uintptr_t>& a32) {
  const auto level = [](uintptr_t x) {
    return x % 128u == 0 ? 8 : x % 64u == 0 ? 6 : x % 16u == 0 ? 2 : x % 8u == 0 ? 1 : 0;
  };
  int best = 0, best_score = -1;
  for (int h = 0; h < zs::kVec; ++h) {
    int score = 0;
    for (uintptr_t a : a16) score += 2 * level(a + 2u * h);
    for (uintptr_t a : a32) score += 8 * level(a + 4u * h);
    if (score > best_score) {
      best_score = score;
      best = h;
    }
  }
  return best;
}

hipError_t mean_range(const uint16_t* const* grads, int32_t p, int32_t gdt, int64_t len, int head,
                      void* out, int32_t odt, float* acc_buf, hipStream_t stream) {
  MeanLaunch L;
  L.gdt = gdt;
  L.odt = odt;
  L.len = len;
  L.head = head;
  L.PF = static_cast<float>(static_cast<double>(p));
  L.stream = stream;
  for (int32_t r0 = 0; r0 < p; r0 += kKernargP) {
    const int32_t np = std::min<int32_t>(kKernargP, p - r0);
    for (int32_t r = 0; r < np; ++r) L.grads[r] = grads[r0 + r];
    L.p = np;
    L.acc = r0 == 0 ? nullptr : acc_buf;
    L.last = r0 + np == p;
    L.out = L.last ? out : static_cast<void*>(acc_buf);
    const hipError_t err = launch_mean(L);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

MtLayout mt_layout(int32_t npieces, int64_t nchunks, int32_t p) {
  auto up = [](size_t x) { return (x + 255u) & ~static_cast<size_t>(255u); };
  MtLayout L;
  L.pieces_off = 0;
  L.gptr_off = up(sizeof(MtPiece) * static_cast<size_t>(npieces));
  L.chunks_off = L.gptr_off + up(sizeof(void*) * static_cast<size_t>(npieces) * p);
  L.total = L.chunks_off + up(sizeof(MtChunk) * static_cast<size_t>(nchunks));
  if (L.total == 0) L.total = 256;
  return L;
}
}  // namespace zs

extern "C" {

size_t zs_mt_workspace_bytes(int32_t npieces, int64_t nchunks, int32_t p) {
  if (npieces < 0 || nchunks < 0 || p < 1 || p > ZS_MAX_P) return 0;
  return zs::mt_layout(npieces, nchunks, p).total;
}

static zs_status mt_upload_body(const zs_piece* pieces, const zs_piece_ptrs* ptrs,
                                int32_t npieces, int32_t p, int32_t grad_dtype,
                                int32_t param_dtype, int64_t chunk_elems, void* workspace,
                                size_t ws_bytes, void* stream, zs_mt_table* table) {
  if (!table || !workspace || (npieces > 0 && (!pieces || !ptrs))) return ZS_ERR_NULL;
  if (p < 1 || p > ZS_MAX_P || npieces < 0 || chunk_elems < zs::kVec ||
      chunk_elems % zs::kVec != 0)
    return ZS_ERR_ARG;
  if (!dtype_ok(grad_dtype) || !dtype_ok(param_dtype)) return ZS_ERR_DTYPE;
  int64_t nchunks = 0;
  bool all_m = true, all_v = true;  // every piece has a momentum / variance buffer
  std::vector<Range> writes, reads;
  for (int32_t i = 0; i < npieces; ++i) {
    const int64_t len = pieces[i].len;
    if (len < 1 || len > kMaxN) return ZS_ERR_ARG;
    const zs_piece_ptrs& q = ptrs[i];
    if (!q.w || !q.param || !q.grads) return ZS_ERR_NULL;
    all_m = all_m && q.m;
    all_v = all_v && q.v;
    for (int32_t r = 0; r < p; ++r) {
      if (!q.grads[r]) return ZS_ERR_NULL;
      const uintptr_t g0 = reinterpret_cast<uintptr_t>(q.grads[r]);
      reads.push_back({g0, g0 + 2u * static_cast<uintptr_t>(len)});
    }
    const uintptr_t b32 = 4u * static_cast<uintptr_t>(len), b16 = 2u * static_cast<uintptr_t>(len);
    const uintptr_t pw = reinterpret_cast<uintptr_t>(q.w), pm = reinterpret_cast<uintptr_t>(q.m),
                    pv = reinterpret_cast<uintptr_t>(q.v),
                    pp = reinterpret_cast<uintptr_t>(q.param);
    writes.push_back({pw, pw + b32});
    if (q.m) writes.push_back({pm, pm + b32});
    if (q.v) writes.push_back({pv, pv + b32});
    writes.push_back({pp, pp + b16});
    nchunks += (len + chunk_elems - 1) / chunk_elems;
  }
  // Outputs must be pairwise disjoint and must not overlap any gradient range:
  // sort both lists and sweep, O((W + R) log(W + R)).
  auto by_lo = [](const Range& x, const Range& y) { return x.lo < y.lo; };
  std::sort(writes.begin(), writes.end(), by_lo);
  std::sort(reads.begin(), reads.end(), by_lo);
  for (size_t i = 1; i < writes.size(); ++i)
    if (writes[i].lo < writes[i - 1].hi) return ZS_ERR_ALIAS;
  {
    size_t j = 0;
    uintptr_t reach = 0;  // max hi over reads with lo < current write's hi
    for (const Range& wr : writes) {
      while (j < reads.size() && reads[j].lo < wr.hi) {
        if (reads[j].hi > reach) reach = reads[j].hi;
        ++j;
      }
      // a read that starts before wr.hi and ends after wr.lo overlaps wr
      if (reach > wr.lo) return ZS_ERR_ALIAS;
    }
  }
  const zs::MtLayout lay = zs::mt_layout(npieces, nchunks, p);
  if (reinterpret_cast<uintptr_t>(workspace) % 256u != 0 || ws_bytes < lay.total)
    return ZS_ERR_CAPACITY;

  std::vector<unsigned char> host(lay.total, 0);
  auto* hp_pieces = reinterpret_cast<zs::MtPiece*>(host.data() + lay.pieces_off);
  auto* hp_gptr = reinterpret_cast<const uint16_t**>(host.data() + lay.gptr_off);
  auto* hp_chunks = reinterpret_cast<zs::MtChunk*>(host.data() + lay.chunks_off);
  int64_t c = 0;
  for (int32_t i = 0; i < npieces; ++i) {
    const zs_piece_ptrs& q = ptrs[i];
    zs::MtPiece& d = hp_pieces[i];
    d.w = q.w;
    d.m = q.m;
    d.v = q.v;
    d.param = static_cast<uint16_t*>(q.param);
    d.len = pieces[i].len;
    d.reserved = 0;
    std::vector<uintptr_t> a16;
    for (int32_t r = 0; r < p; ++r) {
      hp_gptr[static_cast<int64_t>(i) * p + r] = static_cast<const uint16_t*>(q.grads[r]);
      a16.push_back(reinterpret_cast<uintptr_t>(q.grads[r]));
    }
    a16.push_back(reinterpret_cast<uintptr_t>(q.param));
    std::vector<uintptr_t> a32 = {reinterpret_cast<uintptr_t>(q.w)};
    if (q.m) a32.push_back(reinterpret_cast<uintptr_t>(q.m));
    if (q.v) a32.push_back(reinterpret_cast<uintptr_t>(q.v));
    d.head = zs::choose_head(a16, a32);
    for (int64_t st = 0; st < d.len; st += chunk_elems) {
      hp_chunks[c].piece = i;
      hp_chunks[c].reserved = 0;
      hp_chunks[c].start = st;
      ++c;
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipMemcpyAsync(workspace, host.data(), lay.total, hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return hip_fail(err);
  err = hipStreamSynchronize(s);
  if (err != hipSuccess) return hip_fail(err);
  table->workspace = workspace;
  table->nchunks = nchunks;
  table->chunk_elems = chunk_elems;
  table->npieces = npieces;
  table->p = p;
  table->grad_dtype = grad_dtype;
  table->param_dtype = param_dtype;
  table->state = (all_m ? ZS_STATE_M : 0) | (all_v ? ZS_STATE_V : 0);
  table->reserved = 0;
  return ZS_OK;
}

zs_status zs_mt_upload(const zs_piece* pieces, const zs_piece_ptrs* ptrs, int32_t npieces,
                       int32_t p, int32_t grad_dtype, int32_t param_dtype, int64_t chunk_elems,
                       void* workspace, size_t ws_bytes, void* stream, zs_mt_table* table) {
  return zs::guard([&] {
    return mt_upload_body(pieces, ptrs, npieces, p, grad_dtype, param_dtype, chunk_elems,
                          workspace, ws_bytes, stream, table);
  });
}

}  // extern "C"

namespace {

zs_status check_table(const zs_mt_table* t) {
  if (!t) return ZS_ERR_NULL;
  if (t->p < 1 || t->p > ZS_MAX_P || t->npieces < 0 || t->nchunks < 0 ||
      t->chunk_elems < zs::kVec || t->chunk_elems % zs::kVec != 0)
    return ZS_ERR_ARG;
  if (!dtype_ok(t->grad_dtype) || !dtype_ok(t->param_dtype)) return ZS_ERR_DTYPE;
  return ZS_OK;
}

zs_status launch_table(const zs_mt_table* t, int32_t form, const zs::Consts& c,
                       const zs::StepTableDev* steps, void* stream) {
  if (t->nchunks == 0) return ZS_OK;
  if ((needs_m(form) && !(t->state & ZS_STATE_M)) || (needs_v(form) && !(t->state & ZS_STATE_V)))
    return ZS_ERR_NULL;
  if (!t->workspace) return ZS_ERR_NULL;
  const zs::MtLayout lay = zs::mt_layout(t->npieces, t->nchunks, t->p);
  const auto* base = static_cast<const unsigned char*>(t->workspace);
  zs::MultiLaunch L;
  L.steps = steps;
  L.pieces = reinterpret_cast<const zs::MtPiece*>(base + lay.pieces_off);
  L.gptrs = reinterpret_cast<const uint16_t* const*>(base + lay.gptr_off);
  L.chunks = reinterpret_cast<const zs::MtChunk*>(base + lay.chunks_off);
  L.nchunks = t->nchunks;
  L.chunk_elems = t->chunk_elems;
  L.p = t->p;
  L.gdt = t->grad_dtype;
  L.pdt = t->param_dtype;
  L.form = form;
  L.c = c;
  L.stream = static_cast<hipStream_t>(stream);
  const hipError_t err = zs::launch_multi(L);
  if (err != hipSuccess) return hip_fail(err);
  return ZS_OK;
}

zs_status check_steps(const zs_step_table* st) {
  if (!st || !st->dev) return ZS_ERR_NULL;
  if (st->nsteps < 1 || st->nsteps > ZS_MAX_TABLE_STEPS || st->p < 1 || st->p > ZS_MAX_P ||
      st->form < ZS_ADAM_STANDARD ||
      st->form > ZS_SGD_MOMENTUM)
    return ZS_ERR_ARG;
  return ZS_OK;
}

}  // namespace

extern "C" {

zs_status zs_fused_shard_step_multi(const zs_mt_table* t, const zs_adam_hparams* hp,
                                    void* stream) {
  if (const zs_status st = check_table(t)) return st;
  if (const zs_status st = check_hparams(hp)) return st;
  return launch_table(t, hp->form, make_consts(*hp, t->p), nullptr, stream);
}

size_t zs_step_table_bytes(int32_t nsteps) {
  if (nsteps < 1 || nsteps > ZS_MAX_TABLE_STEPS) return 0;
  const size_t b = zs::kStepTableHead + sizeof(zs::Consts) * static_cast<size_t>(nsteps);
  return (b + 255u) & ~static_cast<size_t>(255u);
}

static zs_status step_table_init_body(const zs_adam_hparams* hp, int32_t p, int32_t nsteps,
                                      void* dev, size_t bytes, void* stream,
                                      zs_step_table* table) {
  if (!table || !dev) return ZS_ERR_NULL;
  if (const zs_status st = check_hparams(hp)) return st;
  if (p < 1 || p > ZS_MAX_P || nsteps < 1 || nsteps > ZS_MAX_TABLE_STEPS) return ZS_ERR_ARG;
  if (hp->step > INT64_MAX - nsteps) return ZS_ERR_RANGE;
  const size_t need = zs_step_table_bytes(nsteps);
  if (reinterpret_cast<uintptr_t>(dev) % 256u != 0 || bytes < need) return ZS_ERR_CAPACITY;
  std::vector<unsigned char> host(need, 0);
  auto* t = reinterpret_cast<zs::StepTableDev*>(host.data());
  t->cursor = 0;
  t->nsteps = nsteps;
  t->exhausted = 0;
  t->form = hp->form;
  t->p = p;
  t->reserved = 0;
  t->first_step = hp->step;
  auto* cs = reinterpret_cast<zs::Consts*>(host.data() + zs::kStepTableHead);
  for (int32_t i = 0; i < nsteps; ++i) {
    zs_adam_hparams h = *hp;
    h.step = hp->step + i;
    cs[i] = make_consts(h, p);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipMemcpyAsync(dev, host.data(), need, hipMemcpyHostToDevice, s);
  if (err != hipSuccess) return hip_fail(err);
  err = hipStreamSynchronize(s);
  if (err != hipSuccess) return hip_fail(err);
  table->dev = dev;
  table->first_step = hp->step;
  table->nsteps = nsteps;
  table->p = p;
  table->form = hp->form;
  table->reserved = 0;
  return ZS_OK;
}

zs_status zs_step_table_init(const zs_adam_hparams* hp, int32_t p, int32_t nsteps, void* dev,
                             size_t bytes, void* stream, zs_step_table* table) {
  return zs::guard(
      [&] { return step_table_init_body(hp, p, nsteps, dev, bytes, stream, table); });
}

zs_status zs_step_table_advance(const zs_step_table* table, void* stream) {
  if (const zs_status st = check_steps(table)) return st;
  const hipError_t err = zs::launch_step_advance(static_cast<zs::StepTableDev*>(table->dev),
                                                 static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err);
  return ZS_OK;
}

zs_status zs_step_table_status(const zs_step_table* table, int64_t* cursor, int32_t* exhausted,
                               void* stream) {
  if (const zs_status st = check_steps(table)) return st;
  unsigned char head[sizeof(zs::StepTableDev)];
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipMemcpyAsync(head, table->dev, sizeof(head), hipMemcpyDeviceToHost, s);
  if (err != hipSuccess) return hip_fail(err);
  err = hipStreamSynchronize(s);
  if (err != hipSuccess) return hip_fail(err);
  zs::StepTableDev t;
  std::memcpy(&t, head, sizeof(head));
  if (cursor) *cursor = t.cursor;
  if (exhausted) *exhausted = t.exhausted;
  return ZS_OK;
}

zs_status zs_fused_shard_step_multi_dev(const zs_mt_table* t, const zs_step_table* steps,
                                        void* stream) {
  if (const zs_status st = check_table(t)) return st;
  if (const zs_status st = check_steps(steps)) return st;
  if (steps->p != t->p) return ZS_ERR_ARG;
  return launch_table(t, steps->form, zs::Consts{},
                      static_cast<const zs::StepTableDev*>(steps->dev), stream);
}

}  // extern "C"

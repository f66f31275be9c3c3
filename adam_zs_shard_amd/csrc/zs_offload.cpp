// zs_offload.cpp -- the optimizer offload of one shard on one GPU: the
// pipeline around the host update.
//
// [ZA] §2.2 Offload 策略: the data-flow graph is cut along the 16-bit gradient
// and 16-bit parameter edges.  The GPU forms the shard's gradient (here: the
// rank-order mean of the P rank slices, rounded to 16 bits) and sends it to
// host memory bucket by bucket as the buckets fill, so the copies overlap the
// GPU's work; the CPU updates the fp32 master weights and moments kept in
// host memory and converts the result to 16 bits (the Update Super Node); the
// updated 16-bit parameters go back to the GPU while the CPU updates the
// next bucket.
// [ZA] §2.3 扩展性, delayed parameter update: the first N-1 steps update
// normally; at step N the CPU receives the gradient and does not update; from
// step N+1 on it applies the gradient received the step before while the GPU
// produces (and sends) the current step's.  zs_offload_step runs one step in
// any of the three modes; which mode each step takes is the caller's
// schedule.
//
// Per bucket b (contiguous element range [lo, hi) of the shard):
//   compute stream:  mean of the P ranks over [lo, hi), rounded -> g16_dev
//   d2h stream:      waits for that mean, copies it to g16_host[slot]
//   host:            waits for the copy (PLAIN) or not (DELAYED: the
//                    gradient is the one received last step); `threads`
//                    workers, started once per call, update the bucket
//                    into param_host
//   h2d stream:      copies param_host[lo, hi) into the working copy
// The call returns when every copy and update it started is complete.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "../../include/zshard.h"
#include "zs_internal.h"

namespace {

struct Span {
  uintptr_t lo, hi;
};
bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

bool dtype_ok(int32_t dt) { return dt == ZS_F16 || dt == ZS_BF16; }

// hipEvent_t handles owned by one call
struct Events {
  std::vector<hipEvent_t> ev;
  ~Events() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  hipError_t make(size_t n, unsigned flags = hipEventDisableTiming) {
    ev.assign(n, nullptr);
    for (auto& e : ev) {
      const hipError_t r = hipEventCreateWithFlags(&e, flags);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
};

constexpr int64_t kMaxBuckets = 4096;

}  // namespace

namespace {

zs_status offload_body(const zs_offload_args* a, const zs_adam_hparams* hp, int32_t mode,
                       int32_t slot) {
  if (!a || !hp) return ZS_ERR_NULL;
  if (mode < ZS_OFFLOAD_PLAIN || mode > ZS_OFFLOAD_DELAYED || slot < 0 || slot > 1)
    return ZS_ERR_ARG;
  if (a->p < 1 || a->p > ZS_MAX_P || a->k < 0 || a->k >= a->p || a->n < 0 ||
      a->bucket_elems < 0 || a->reserved != 0)
    return ZS_ERR_ARG;
  if (a->n > (int64_t{1} << 60)) return ZS_ERR_RANGE;
  if (!dtype_ok(a->grad_dtype) || !dtype_ok(a->param_dtype)) return ZS_ERR_DTYPE;
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
      !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || hp->step < 1 || hp->reserved != 0 ||
      hp->form < ZS_ADAM_STANDARD || hp->form > ZS_SGD_MOMENTUM)
    return ZS_ERR_ARG;
  // the shard [s, e) of rank k: M = ceil(n/p), both ends clamped to n
  const int64_t M = a->n / a->p + (a->n % a->p != 0 ? 1 : 0);
  const int64_t s = std::min(static_cast<int64_t>(a->k) * M, a->n);
  const int64_t e = std::min(s + M, a->n);
  const int64_t len = e - s;
  if (a->grad_base < 0 || a->grad_base > s || a->param_base < 0 || a->param_base > s)
    return ZS_ERR_RANGE;
  if (len == 0) return ZS_OK;
  const bool um = hp->form != ZS_SGD;
  const bool uv = hp->form == ZS_ADAM_STANDARD || hp->form == ZS_ADAM_PAGE1_LITERAL;
  const bool update = mode != ZS_OFFLOAD_RECEIVE;  // every mode receives
  if (!a->grads || !a->g16_dev || !a->g16_host[slot]) return ZS_ERR_NULL;
  if (mode == ZS_OFFLOAD_DELAYED && !a->g16_host[1 - slot]) return ZS_ERR_NULL;
  if (update && (!a->w || (um && !a->m) || (uv && !a->v) || !a->param || !a->param_host))
    return ZS_ERR_NULL;
  if (a->p > ZS_KERNARG_P && !a->partial) return ZS_ERR_NULL;
  for (int32_t r = 0; r < a->p; ++r)
    if (!a->grads[r]) return ZS_ERR_NULL;

  // device side: what the GPU writes must not overlap the gradients
  const uintptr_t b16 = 2u * static_cast<uintptr_t>(len), b32 = 4u * static_cast<uintptr_t>(len);
  std::vector<const uint16_t*> gp(static_cast<size_t>(a->p));
  std::vector<Span> dev_w = {{reinterpret_cast<uintptr_t>(a->g16_dev),
                              reinterpret_cast<uintptr_t>(a->g16_dev) + b16}};
  uint16_t* par_dev = static_cast<uint16_t*>(a->param) + (s - a->param_base);
  if (update)
    dev_w.push_back({reinterpret_cast<uintptr_t>(par_dev), reinterpret_cast<uintptr_t>(par_dev) + b16});
  if (a->p > ZS_KERNARG_P)
    dev_w.push_back({reinterpret_cast<uintptr_t>(a->partial),
                     reinterpret_cast<uintptr_t>(a->partial) + b32});
  for (size_t i = 0; i < dev_w.size(); ++i)
    for (size_t j = i + 1; j < dev_w.size(); ++j)
      if (overlap(dev_w[i], dev_w[j])) return ZS_ERR_ALIAS;
  for (int32_t r = 0; r < a->p; ++r) {
    gp[r] = static_cast<const uint16_t*>(a->grads[r]) + (s - a->grad_base);
    const Span g{reinterpret_cast<uintptr_t>(gp[r]), reinterpret_cast<uintptr_t>(gp[r]) + b16};
    for (const Span& w : dev_w)
      if (overlap(w, g)) return ZS_ERR_ALIAS;
  }
  // host side: the received gradient, the state and the staged parameters
  std::vector<Span> host_w = {{reinterpret_cast<uintptr_t>(a->g16_host[slot]),
                               reinterpret_cast<uintptr_t>(a->g16_host[slot]) + b16}};
  if (update) {
    host_w.push_back({reinterpret_cast<uintptr_t>(a->w), reinterpret_cast<uintptr_t>(a->w) + b32});
    if (um) host_w.push_back({reinterpret_cast<uintptr_t>(a->m), reinterpret_cast<uintptr_t>(a->m) + b32});
    if (uv) host_w.push_back({reinterpret_cast<uintptr_t>(a->v), reinterpret_cast<uintptr_t>(a->v) + b32});
    host_w.push_back({reinterpret_cast<uintptr_t>(a->param_host),
                      reinterpret_cast<uintptr_t>(a->param_host) + b16});
  }
  if (mode == ZS_OFFLOAD_DELAYED)
    host_w.push_back({reinterpret_cast<uintptr_t>(a->g16_host[1 - slot]),
                      reinterpret_cast<uintptr_t>(a->g16_host[1 - slot]) + b16});  // read
  for (size_t i = 0; i < host_w.size(); ++i)
    for (size_t j = i + 1; j < host_w.size(); ++j)
      if (overlap(host_w[i], host_w[j])) return ZS_ERR_ALIAS;

  const int64_t bucket = a->bucket_elems > 0 ? a->bucket_elems : len;
  const int64_t nb = (len + bucket - 1) / bucket;
  if (nb > kMaxBuckets) return ZS_ERR_ARG;

  const hipStream_t cs = static_cast<hipStream_t>(a->compute_stream);
  const hipStream_t ds = static_cast<hipStream_t>(a->d2h_stream);
  const hipStream_t hs = static_cast<hipStream_t>(a->h2d_stream);
  Events mean_done, copied;
  hipError_t err = mean_done.make(static_cast<size_t>(nb));
  // the host waits on `copied`: blocking events, so the waiting thread sleeps
  // instead of spinning on a core the update's workers need
  if (err == hipSuccess)
    err = copied.make(static_cast<size_t>(nb), hipEventDisableTiming | hipEventBlockingSync);
  auto fail = [](hipError_t x) { return static_cast<zs_status>(zs::hip_status(x)); };
  if (err != hipSuccess) return fail(err);

  auto* g16d = static_cast<uint16_t*>(a->g16_dev);
  auto* g16h_recv = static_cast<uint16_t*>(a->g16_host[slot]);
  std::vector<const uint16_t*> gb(static_cast<size_t>(a->p));
  std::vector<uintptr_t> a16, a32;
  a16.reserve(static_cast<size_t>(a->p) + 1);
  a32.reserve(1);

  // The host update's workers: thread t takes slice t of every bucket once
  // the bucket's gradient is on the host.  They start before anything is
  // enqueued, so a refused thread fails the call with nothing in flight.
  const auto* g16h_use = static_cast<const uint16_t*>(
      mode == ZS_OFFLOAD_DELAYED ? a->g16_host[1 - slot] : a->g16_host[slot]);
  auto* ph = static_cast<uint16_t*>(a->param_host);
  int64_t nt = a->threads > 0 ? a->threads
                              : static_cast<int64_t>(std::thread::hardware_concurrency());
  nt = std::max<int64_t>(1, std::min<int64_t>(nt, (bucket + 65535) / 65536));
  std::mutex mu;
  std::condition_variable cv_ready, cv_done;
  int64_t ready = mode == ZS_OFFLOAD_DELAYED ? nb : 0;  // buckets whose gradient is here
  std::vector<int64_t> done(static_cast<size_t>(nb), 0);  // workers finished per bucket
  zs_status worker_status = ZS_OK;
  auto stop = [&](zs_status st) {  // every waiting worker returns
    std::lock_guard<std::mutex> lk(mu);
    if (worker_status == ZS_OK) worker_status = st;
    cv_ready.notify_all();
  };
  auto work = [&](int64_t t) {
    for (int64_t b = 0; b < nb; ++b) {
      {
        std::unique_lock<std::mutex> lk(mu);
        cv_ready.wait(lk, [&] { return ready > b || worker_status != ZS_OK; });
        if (worker_status != ZS_OK) return;
      }
      const int64_t lo = b * bucket, hi = std::min(len, lo + bucket);
      const int64_t per = ((hi - lo + nt - 1) / nt + 15) / 16 * 16;
      const int64_t a0 = std::min(hi, lo + t * per), a1 = std::min(hi, a0 + per);
      zs_status st = ZS_OK;
      if (a0 < a1)
        st = zs_cpu_adam_step(g16h_use + a0, a->grad_dtype, a->w + a0, um ? a->m + a0 : nullptr,
                              uv ? a->v + a0 : nullptr, ph + a0, a->param_dtype, a1 - a0, hp, 1);
      std::lock_guard<std::mutex> lk(mu);
      if (st != ZS_OK && worker_status == ZS_OK) worker_status = st;
      ++done[static_cast<size_t>(b)];
      cv_done.notify_all();
      if (worker_status != ZS_OK) {
        cv_ready.notify_all();
        return;
      }
    }
  };
  // Joins the workers on every way out of this call.
  struct Pool {
    std::vector<std::thread> th;
    std::function<void()> on_exit;
    ~Pool() {
      if (on_exit) on_exit();
      for (auto& x : th)
        if (x.joinable()) x.join();
    }
  } pool;
  if (update) {
    try {
      pool.th.reserve(static_cast<size_t>(nt));
      for (int64_t t = 0; t < nt; ++t) pool.th.emplace_back(work, t);
    } catch (...) {
      stop(ZS_ERR_RESOURCE);
      return ZS_ERR_RESOURCE;  // ~Pool joins the workers already started
    }
  }
  // once the call ends, early or not, no worker waits for a bucket: any
  // non-OK status wakes the ones still waiting (after a normal end, none is)
  pool.on_exit = [&] { stop(ZS_ERR_HIP); };

  for (int64_t b = 0; b < nb; ++b) {
    const int64_t lo = b * bucket, hi = std::min(len, lo + bucket);
    a16.clear();
    a32.clear();
    for (int32_t r = 0; r < a->p; ++r) {
      gb[r] = gp[r] + lo;
      a16.push_back(reinterpret_cast<uintptr_t>(gb[r]));
    }
    a16.push_back(reinterpret_cast<uintptr_t>(g16d + lo));
    if (a->p > ZS_KERNARG_P) a32.push_back(reinterpret_cast<uintptr_t>(a->partial + lo));
    err = zs::mean_range(gb.data(), a->p, a->grad_dtype, hi - lo, zs::choose_head(a16, a32),
                         g16d + lo, a->grad_dtype, a->partial ? a->partial + lo : nullptr, cs);
    if (err == hipSuccess) err = hipEventRecord(mean_done.ev[b], cs);
    if (err == hipSuccess) err = hipStreamWaitEvent(ds, mean_done.ev[b], 0);
    if (err == hipSuccess)
      err = hipMemcpyAsync(g16h_recv + lo, g16d + lo, 2u * static_cast<size_t>(hi - lo),
                           hipMemcpyDeviceToHost, ds);
    if (err == hipSuccess) err = hipEventRecord(copied.ev[b], ds);
    if (err != hipSuccess) {
      stop(fail(err));
      (void)hipStreamSynchronize(ds);
      return fail(err);
    }
  }
  if (update) {
    zs_status st = ZS_OK;
    for (int64_t b = 0; b < nb && st == ZS_OK; ++b) {
      const int64_t lo = b * bucket, hi = std::min(len, lo + bucket);
      if (mode == ZS_OFFLOAD_PLAIN) {
        err = hipEventSynchronize(copied.ev[b]);
        std::lock_guard<std::mutex> lk(mu);
        if (err != hipSuccess) {
          st = fail(err);
          worker_status = st;
        } else {
          ready = b + 1;
        }
        cv_ready.notify_all();
        if (st != ZS_OK) break;
      }
      {
        std::unique_lock<std::mutex> lk(mu);
        cv_done.wait(lk, [&] { return done[static_cast<size_t>(b)] == nt || worker_status != ZS_OK; });
        if (worker_status != ZS_OK) {
          st = worker_status;
          break;
        }
      }
      err = hipMemcpyAsync(par_dev + lo, ph + lo, 2u * static_cast<size_t>(hi - lo),
                           hipMemcpyHostToDevice, hs);
      if (err != hipSuccess) {
        st = fail(err);
        stop(st);
      }
    }
    if (st != ZS_OK) {
      stop(st);
      (void)hipStreamSynchronize(ds);
      (void)hipStreamSynchronize(hs);
      return st;
    }
  }
  err = hipStreamSynchronize(ds);
  if (err == hipSuccess) err = hipStreamSynchronize(hs);
  if (err != hipSuccess) return fail(err);
  return ZS_OK;
}

}  // namespace

extern "C" zs_status zs_offload_step(const zs_offload_args* a, const zs_adam_hparams* hp,
                                     int32_t mode, int32_t slot) {
  return zs::guard([&] { return offload_body(a, hp, mode, slot); });
}

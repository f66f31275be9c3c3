// Runs the oracle's entry points on small inputs under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with g++; a
// finding aborts with a non-zero status).  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
int32_t oracle_widen(int32_t dt, const uint16_t* in, float* out, int64_t n);
int32_t oracle_narrow(int32_t dt, const float* in, uint16_t* out, int64_t n);
int32_t oracle_plan_shards(int64_t n, int32_t p, int64_t* m_out, int64_t* starts, int64_t* ends);
int32_t oracle_grad_mean(int32_t gdt, int32_t p, const uint16_t* const* grads, int64_t n,
                         float* g_out);
int32_t oracle_adam_apply(const float* g, float* w, float* m, float* v, uint16_t* param,
                          int32_t pdt, int64_t n, double lr, double b1, double b2, double eps,
                          int64_t t, int32_t form);
int32_t oracle_step_elems(int32_t gdt, int32_t p, const uint16_t* const* grads, float* w,
                          float* m, float* v, uint16_t* param, int32_t pdt, int64_t n, double lr,
                          double b1, double b2, double eps, int64_t t, int32_t form);
int32_t oracle_shard_step(int64_t n, int32_t p, int32_t k, const uint16_t* const* grads,
                          int32_t gdt, int64_t grad_base, float* w, float* m, float* v,
                          uint16_t* param, int32_t pdt, int64_t param_base, double lr, double b1,
                          double b2, double eps, int64_t t, int32_t form);
int32_t oracle_locate(const int64_t* numel, int32_t ntensors, int64_t j, int64_t* off);
int32_t oracle_shard_pieces(const int64_t* numel, int32_t ntensors, int64_t lo, int64_t hi,
                            int32_t* tensor, int64_t* tensor_off, int64_t* range_off,
                            int64_t* len, int32_t cap);
}

static int fails = 0;
static void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL %s\n", what);
    ++fails;
  }
}

int main() {
  // every 16-bit pattern through both conversions
  std::vector<uint16_t> bits(65536), back(65536);
  std::vector<float> f(65536);
  for (int i = 0; i < 65536; ++i) bits[i] = static_cast<uint16_t>(i);
  for (int dt = 1; dt <= 2; ++dt) {
    check(oracle_widen(dt, bits.data(), f.data(), 65536) == 0, "widen");
    check(oracle_narrow(dt, f.data(), back.data(), 65536) == 0, "narrow");
  }
  // shard plans with empty and ragged shards
  for (int64_t n = 0; n <= 17; ++n)
    for (int32_t p = 1; p <= 9; ++p) {
      std::vector<int64_t> s(p), e(p);
      int64_t m = 0;
      check(oracle_plan_shards(n, p, &m, s.data(), e.data()) == 0, "plan");
    }
  // a 3-rank mean, every form of the update, the whole step
  const int64_t n = 37;
  const int32_t p = 3;
  std::vector<std::vector<uint16_t>> g(p, std::vector<uint16_t>(n));
  std::vector<const uint16_t*> gp(p);
  for (int r = 0; r < p; ++r) {
    for (int64_t i = 0; i < n; ++i) g[r][i] = static_cast<uint16_t>(0x2000 + 37 * r + i);
    gp[r] = g[r].data();
  }
  std::vector<float> mean(n), w(n, 0.01f), m(n, 0.0f), v(n, 0.0f);
  std::vector<uint16_t> par(n);
  check(oracle_grad_mean(1, p, gp.data(), n, mean.data()) == 0, "mean");
  for (int32_t form = 0; form < 4; ++form)
    for (int64_t t = 1; t <= 3; ++t)
      check(oracle_adam_apply(mean.data(), w.data(), m.data(), v.data(), par.data(), 2, n, 1e-3,
                              0.9, 0.999, 1e-8, t, form) == 0,
            "adam_apply");
  check(oracle_step_elems(2, p, gp.data(), w.data(), m.data(), v.data(), par.data(), 1, n, 1e-3,
                          0.9, 0.999, 1e-8, 4, 0) == 0,
        "step_elems");
  // rank k = 1 of 4 over 50 elements, full-N gradient and parameter buffers
  const int64_t N = 50;
  std::vector<std::vector<uint16_t>> gf(4, std::vector<uint16_t>(N, 0x2400));
  std::vector<const uint16_t*> gfp(4);
  for (int r = 0; r < 4; ++r) gfp[r] = gf[r].data();
  std::vector<float> ws(13, 0.5f), ms(13, 0.0f), vs(13, 0.0f);
  std::vector<uint16_t> pf(N);
  check(oracle_shard_step(N, 4, 1, gfp.data(), 1, 0, ws.data(), ms.data(), vs.data(), pf.data(),
                          1, 0, 1e-3, 0.9, 0.999, 1e-8, 1, 1) == 0,
        "shard_step");
  // tensor-list maps
  const int64_t numel[5] = {3, 0, 7, 1, 11};
  int64_t off = 0;
  for (int64_t j = 0; j < 22; ++j) check(oracle_locate(numel, 5, j, &off) >= 0, "locate");
  std::vector<int32_t> tensor(5);
  std::vector<int64_t> toff(5), roff(5), len(5);
  check(oracle_shard_pieces(numel, 5, 2, 19, tensor.data(), toff.data(), roff.data(), len.data(),
                            5) == 4,
        "pieces");
  std::printf("%s\n", fails ? "oracle driver: failures" : "oracle driver: ok");
  return fails ? 1 : 0;
}

// Runs the host update (zs_cpu_adam_step, the optimizer-offload path) on
// ragged lengths, both 16-bit dtypes, every form and several thread counts
// under AddressSanitizer, UndefinedBehaviorSanitizer or ThreadSanitizer
// (built by tests/test_sanitizers.py with g++).  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "zshard.h"

int main() {
  int fails = 0;
  const int64_t lens[] = {1, 7, 15, 16, 17, 1000, 65537, 200003};
  for (int64_t n : lens)
    for (int32_t dt = ZS_F16; dt <= ZS_BF16; ++dt)
      for (int32_t form = ZS_ADAM_STANDARD; form <= ZS_SGD_MOMENTUM; ++form)
        for (int32_t threads : {1, 3, 8}) {
          std::vector<uint16_t> g(n), par(n);
          std::vector<float> w(n, 0.25f), m(n, 0.0f), v(n, 0.0f);
          for (int64_t i = 0; i < n; ++i) g[i] = static_cast<uint16_t>(0x1c00 + (i * 7919) % 0x2000);
          zs_adam_hparams hp{};
          hp.lr = 1e-3;
          hp.beta1 = 0.9;
          hp.beta2 = 0.999;
          hp.eps = 1e-8;
          hp.form = form;
          for (int64_t t = 1; t <= 2; ++t) {
            hp.step = t;
            const zs_status st = zs_cpu_adam_step(
                g.data(), dt, w.data(), form == ZS_SGD ? nullptr : m.data(),
                form == ZS_ADAM_STANDARD || form == ZS_ADAM_PAGE1_LITERAL ? v.data() : nullptr,
                par.data(), dt, n, &hp, threads);
            if (st == ZS_ERR_UNSUPPORTED) {
              std::printf("cpu update driver: no AVX2/F16C on this host\n");
              return 0;
            }
            if (st != ZS_OK) {
              std::printf("FAIL n=%lld dt=%d form=%d threads=%d: %d\n", (long long)n, dt, form,
                          threads, st);
              ++fails;
            }
          }
        }
  std::printf("%s\n", fails ? "cpu update driver: failures" : "cpu update driver: ok");
  return fails ? 1 : 0;
}

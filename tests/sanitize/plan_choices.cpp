// Host-only driver over the launch-plan header: prints the plan choices the
// dispatcher makes for the benchmark shapes (die grouping, step-major
// paths, LDS budget, weight staging), one line per shape, for
// tests/test_plan_cpu.py.
#include <cstdio>

#include "pdscan_plan.h"

using namespace pdscan;

static void show(const char* name, int mode, int B, int H, int L, int N, int K, int d, int u_shared, int bf16,
                 int chunk, int fold = 0, int n_out = 1) {
  Plan p;
  const bool ok = make_plan(p, mode, B, H, L, N, K, d, u_shared, bf16, chunk, fold, 0, n_out);
  const int hg = ok && mode == kModeFused && !p.fused16
                     ? xcd_head_groups(p.B, p.H, p.L, p.N, p.K, p.d, p.u_shared, p.in_bf16, p.fold_bu, p.nC)
                     : 0;
  std::printf("%s ok=%d fused16=%d step32=%d fold=%d gse=%d wst=%d S=%d G=%d nC=%d lds=%d limit=%d hg=%d tasks=%lld plain=%lld\n",
              name, ok ? 1 : 0, p.fused16, p.step32, p.fold_bu, p.gse, p.wst, p.S, p.G, p.nC, p.lds_bytes,
              p.lds_limit, hg, xcd_tasks(p, hg), xcd_tasks(p, 0));
}

int main() {
  show("impulse", kModeFused, 1, 32, 131072, 16, 8, 64, 0, 0, 512);
  show("impulse_c640", kModeFused, 1, 32, 131072, 16, 8, 64, 0, 0, 640);
  show("impulse_c768", kModeFused, 1, 32, 131072, 16, 8, 64, 0, 0, 768);
  show("impulse_c640_p2", kModeFused, 1, 32, 131072, 16, 8, 64, 0, 0, 640, 0, 2);
  show("base", kModeFused, 4, 8, 4096, 16, 8, 64, 0, 0, 256);
  show("timeseries", kModeFused, 8, 16, 16384, 32, 16, 128, 0, 1, 256);
  show("timeseries_c512", kModeFused, 8, 16, 16384, 32, 16, 128, 0, 1, 512);
  show("timeseries_k17", kModeFused, 8, 16, 16384, 32, 17, 128, 0, 1, 256);
  show("timeseries_fold", kModeFused, 8, 16, 16384, 32, 16, 128, 0, 1, 256, 1);
  show("lm_layer", kModeFused, 16, 24, 2048, 64, 32, 768, 1, 1, 128);
  show("lm_layer_fold", kModeFused, 16, 24, 2048, 64, 32, 768, 1, 1, 96, 1);
  show("lm_layer_fold_c128", kModeFused, 16, 24, 2048, 64, 32, 768, 1, 1, 128, 1);
  show("lm_layer_multi", kModeFused, 16, 24, 2048, 64, 32, 768, 1, 1, 64, 1, 2);
  show("lm_small", kModeFused, 3, 5, 260, 32, 16, 768, 1, 1, 128);
  show("lm_b1", kModeFused, 1, 24, 2048, 64, 32, 768, 1, 1, 128);
  show("timeseries_h96", kModeFused, 1, 96, 520, 32, 16, 128, 0, 1, 256);
  show("edge_d320", kModeFused, 1, 2, 300, 64, 32, 320, 0, 1, 128);
  show("edge_d384", kModeFused, 2, 1, 260, 64, 16, 384, 0, 1, 128);
  show("edge_d800", kModeFused, 1, 2, 130, 64, 3, 800, 0, 1, 128);
  return 0;
}

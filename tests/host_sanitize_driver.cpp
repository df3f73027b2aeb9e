// Sanitizer driver for the host-CPU projection (nvfp4::host::moe_decode, built from
// source without HIP): random layers of several shapes, NVFP4 and Q8_0 down projections,
// every instruction set the CPU has and several thread counts; outputs must match across
// thread counts bit for bit and the portable loop within FP32 rounding.
#include "../nvfp4_quantized_moe_02_amd/csrc/host.h"
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
using namespace nvfp4::host;
int main() {
  std::mt19937 rng(1);
  int fails = 0;
  for (int trial = 0; trial < 6; ++trial) {
    const int E = 5 + trial, H = 64 * (1 + trial % 3), I = 32 * (1 + trial % 4), T = 1 + trial * 3, k = 1 + trial % 8;
    const bool q8 = trial % 2;
    std::vector<uint8_t> gc((size_t)E * I * H / 2), uc(gc.size()), gs((size_t)E * I * H / 16), us(gs.size());
    std::vector<uint8_t> dc(q8 ? (size_t)E * H * I : (size_t)E * H * I / 2), ds(q8 ? (size_t)E * H * I / 32 * 2 : (size_t)E * H * I / 16);
    for (auto* v : {&gc, &uc, &dc}) for (auto& b : *v) b = rng() & 0xFF;
    for (auto* v : {&gs, &us}) for (auto& b : *v) b = 0x20 + rng() % 0x40;
    if (q8) { for (size_t i = 0; i < ds.size(); i += 2) { uint16_t h = 0x1800 + rng() % 0x800; memcpy(&ds[i], &h, 2); } }
    else for (auto& b : ds) b = 0x20 + rng() % 0x40;
    std::vector<float> gg(E, 0.5f), ug(E, 0.25f), dg(E, 2.f);
    Weight g{gc.data(), gs.data(), gg.data(), I, H, 0}, u{uc.data(), us.data(), ug.data(), I, H, 0};
    Weight d{dc.data(), ds.data(), q8 ? nullptr : dg.data(), H, I, q8 ? 1 : 0};
    std::vector<float> x((size_t)T * H);
    for (auto& v : x) v = std::uniform_real_distribution<float>(-1, 1)(rng);
    std::vector<int32_t> ids((size_t)T * k);
    for (auto& v : ids) v = (int)(rng() % (E + 2)) - 1;
    std::vector<float> w(ids.size(), 0.3f);
    std::vector<float> ref((size_t)T * H), out((size_t)T * H);
    moe_decode(x.data(), 0, T, H, I, g, u, d, E, ids.data(), w.data(), k, ref.data(), 1, kIsaPortable);
    for (int isa = kIsaPortable; isa <= best_isa(); ++isa) {
      std::vector<float> one((size_t)T * H);
      moe_decode(x.data(), 0, T, H, I, g, u, d, E, ids.data(), w.data(), k, one.data(), 1, isa);
      for (int nt : {2, 3, 8}) {
        moe_decode(x.data(), 0, T, H, I, g, u, d, E, ids.data(), w.data(), k, out.data(), nt, isa);
        if (memcmp(out.data(), one.data(), out.size() * 4)) { printf("trial %d isa %d nt %d: thread-count difference\n", trial, isa, nt); ++fails; }
      }
      double num = 0, den = 0;
      for (size_t i = 0; i < out.size(); ++i) { num += (out[i] - ref[i]) * (double)(out[i] - ref[i]); den += (double)ref[i] * ref[i]; }
      if (num > 1e-10 * den + 1e-30) { printf("trial %d isa %d: rel err %g\n", trial, isa, std::sqrt(num / den)); ++fails; }
    }
  }
  printf("%s (%d failures)\n", fails ? "FAIL" : "ok", fails);
  return fails != 0;
}

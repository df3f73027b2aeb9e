// Host-CPU projection shared by api.hip and host_decode.cpp (built by the host compiler,
// so this header holds plain C++ types only).
#pragma once
#include <stdint.h>

namespace nvfp4 {
namespace host {

// One projection of E experts in host memory; the layout of the device weights.
// fmt 0: NVFP4 (codes [E][N][K/2], E4M3 scales [E][N][K/16], global [E]);
// fmt 1: Q8_0 (int8 codes [E][N][K], fp16 scales [E][N][K/32], global [E] or null for 1).
struct Weight {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int N, K;
  int fmt;
};

// Instruction sets of the row kernels; kIsaAuto picks the widest the CPU has.
enum Isa { kIsaAuto = 0, kIsaPortable = 1, kIsaAvx2 = 2, kIsaAvx512 = 3 };

// The widest instruction set the running CPU supports (kIsaPortable .. kIsaAvx512).
int best_isa();

// The routed-expert projection on the host (arguments validated by the caller):
// out [T][H] fp32 = sum over valid pairs of w * gamma_down * (SiLU(g) * u) . Wdown.
// Returns the number of dropped pairs (ids outside [0, E)).
int64_t moe_decode(const void* x, int x_dtype, int T, int H, int I, const Weight& gate, const Weight& up,
                   const Weight& down, int E, const int32_t* ids, const float* wts, int topk, float* out,
                   int nthreads, int isa);

}  // namespace host
}  // namespace nvfp4

// Kernel launchers shared between the translation units of libnvfp4moe.so. Every
// launcher enqueues on `st` and returns hipGetLastError(); argument validation is the
// C-ABI layer's job (api.hip).
#pragma once
#include "common.h"

namespace nvfp4 {

// One projection of all experts. fmt 0: NVFP4 (codes [E][N][K/2], E4M3 scales [E][N][K/16],
// global [E]); fmt 1: Q8_0 (int8 codes [E][N][K], fp16 scales [E][N][K/32], global [E] or
// null for 1).
// Optionally one more expert, index `xe`, lives in tensors of its own (xcodes, xscales,
// xglobal: one expert's worth, the layer's shared expert); -1 means none.
struct WeightArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int N, K;
  int fmt;
  const uint8_t* xcodes = nullptr;
  const uint8_t* xscales = nullptr;
  const float* xglobal = nullptr;
  int xe = -1;
  // First code / scale byte of row n (0 <= n < N) of expert e; rowbytes = code bytes per
  // row, K / 2 for NVFP4 and K for Q8_0 (the caller knows the format at compile time).
  // X = false: the call has no separately stored expert (plain indexing, no select).
  template <bool X = true>
  __device__ const uint8_t* code_row(int e, size_t n, size_t rowbytes) const {
    if constexpr (X) return (e == xe ? xcodes : codes + (size_t)e * N * rowbytes) + n * rowbytes;
    return codes + ((size_t)e * N + n) * rowbytes;
  }
  template <bool X = true>
  __device__ const uint8_t* scale_row(int e, size_t n) const {
    if constexpr (X) return (e == xe ? xscales : scales + (size_t)e * N * (K / 16)) + n * (K / 16);
    return scales + ((size_t)e * N + n) * (K / 16);
  }
  // the expert's output scale; an NVFP4 projection always has one (one pointer select,
  // then one load: no branch between the loads a caller issues together)
  template <bool X = true>
  __device__ float gamma_nvfp4(int e) const {
    if constexpr (X) return *(e == xe ? xglobal : global + e);
    return global[e];
  }
  // the same for a projection that may have none (Q8_0: NULL means 1)
  template <bool X = true>
  __device__ float gamma(int e) const {
    if constexpr (X) {
      const float* g = e == xe ? xglobal : (global != nullptr ? global + e : nullptr);
      return g != nullptr ? *g : 1.0f;
    }
    return global != nullptr ? global[e] : 1.0f;
  }
};

struct TileDesc {
  int expert;
  int m0;
};

// A prefill GEMM block's work item: expert e, its rows [m0, m0 + rows) in sorted order
// (sorted positions base + m0 ...), N block nb.
struct TileCtx {
  int e, m0, rows, base, nb;
};

// SiLU for the prefill path's h: exp and reciprocal from the hardware approximations
// (about 1 ulp each).
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// elementwise.hip
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* global, int64_t rows,
                          int K, int out_dtype, void* out, hipStream_t st);
hipError_t launch_linear(const void* x, int x_dtype, int T, const uint8_t* codes, const uint8_t* scales,
                         const float* global, int N, int K, float* out, hipStream_t st);
hipError_t launch_quant_rows(const void* x, int x_dtype, int64_t rows, int cols, int8_t* q, float* scale,
                             hipStream_t st);
// NVFP4 activation rows (the W4A4 rule): cols % 16 == 0, 16-byte aligned rows; codes
// [rows][cols/2], scales [rows][cols/16] E4M3, g [rows] fp32.
hipError_t launch_quant_rows_nvfp4(const void* x, int x_dtype, int64_t rows, int cols, uint8_t* codes,
                                   uint8_t* scales, float* g, hipStream_t st);
// out[t][n] = sum over slots j (in order) of y[inv[t*topk + j]][n]; dropped slots skipped.
hipError_t launch_combine(const float* y, const int32_t* inv, int T, int topk, int H, void* out, int out_dtype,
                          hipStream_t st);

// route.hip
constexpr int kRouteChunk = 512;  // pairs per counting / scatter block
constexpr int kMaxExperts = 8192;
struct RouteWs {
  int32_t* counts;    // [E][nblk]
  int32_t* dropped;   // [nblk]
  int32_t* hdr;       // hdr[0] = dropped pairs, hdr[1] = tile count
  TileDesc* tiles;    // [max_tiles] (optional)
  int32_t* inv;       // [P] sorted position of each pair, -1 if dropped (optional)
};
int route_blocks(int64_t P);
// cvt_src (optional): bf16 activations [cvt_rows][cvt_cols] staged as fp16 into cvt_dst by
// extra blocks of the first launch, each row scaled by 2^cvt_exp[row] (cvt_cols a multiple
// of 8, rows 16-byte aligned).
hipError_t launch_route(const int32_t* ids, int64_t P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const RouteWs& ws, int tile_m, hipStream_t st, const void* cvt_src = nullptr,
                        void* cvt_dst = nullptr, int32_t* cvt_exp = nullptr, int cvt_rows = 0, int cvt_cols = 0);

// ids2 [T][k+1] / w2: the k routed slots (ids outside [0, E) as -1) and the shared expert
// (index E, weight 1) as slot k of every token.
hipError_t launch_append_shared(const int32_t* ids, const float* w, int64_t T, int k, int E, int32_t* ids2,
                                float* w2, hipStream_t st);

// decode.hip
constexpr int kDecodeMaxT = 8;
constexpr int kDecodeMaxPairs = 64;
constexpr int kDecodeMaxTH = 40960;
constexpr int kDecodeMaxH = 8192;  // T * H: the bf16 activations of a block live in LDS
// stage 0: gate/up + SwiGLU; 1: down + combine; 2: both in one persistent launch (falls
// back to 0 then 1 when the grid cannot be co-resident). hdr: [0] dropped pairs,
// [1] error flags, [2] grid-barrier spin-limit override, [4] the grid-barrier arrival
// counter, [6..7] its epoch; flags: per-block release flags (counter, error word,
// override and flags zero before first use; any epoch).
constexpr int kDecodeRowsPerBlock = 8;
inline size_t decode_flag_bytes(int H) { return (size_t)((H + kDecodeRowsPerBlock - 1) / kDecodeRowsPerBlock) * 128; }
hipError_t launch_decode(int stage, const void* x, int T, int H, int I, const WeightArgs& gate, const WeightArgs& up,
                         const WeightArgs& down, int E, const int32_t* ids, const float* w, int topk,
                         void* out, int out_dtype, float* h, int32_t* hdr, unsigned long long* flags,
                         hipStream_t st);

// router.hip: logits [T][E] fp32 (workspace), then ids/weights [T][k]. x_dtype 1 = bf16,
// 0 = fp32 (split exactly into three bf16 parts). E % 32 == 0, E <= 2048, k <= 64,
// H % 16 == 0 (H % 64 == 0 for few tokens). done: a completion counter, zero on entry
// and left zero (the single-launch path for up to 4 tokens counts its blocks on it).
hipError_t launch_router(const void* x, int x_dtype, int T, int H, const uint16_t* wr, int E, int k, float* logits,
                         int32_t* ids, float* wts, unsigned* done, hipStream_t st);

// prefill.hip
constexpr int kTileM = 128;
// act 0: fp16 activations with power-of-two row exponents (a_exp: x per token; h written
// as fp16 with one exponent per (sorted pair, gate/up block) into hexp); act 1: int8
// activations with fp32 row scales (a_scale), fp32 h.
// act: 0 fp16 x (a_exp), 1 int8 x (a_scale), 2 NVFP4 x (codes, a_scale = row scales,
// a_bscale = E4M3 block scales)
hipError_t launch_gemm_gateup(int act, const void* a, const float* a_scale, const uint8_t* a_bscale,
                              const int32_t* a_exp,
                              const int32_t* sorted_pairs, const int32_t* offsets, const TileDesc* tiles,
                              const int32_t* tile_count, int max_tiles, int topk, int H, int I,
                              const WeightArgs& gate, const WeightArgs& up, void* h, int32_t* hexp,
                              hipStream_t st);
// gate/up blocks along I (the number of h exponents per sorted pair in act 0)
int gateup_blocks(int I);
// prefill_i8.hip: the W4A8 GEMMs on int8 matrix cores (int8 activations with fp32 row
// scales; NVFP4 weights as exact int8 2*e2m1 with an fp32 rescale per 16-input group)
hipError_t launch_gemm_gateup_i8(const int8_t* a, const float* a_scale, const int32_t* sorted_pairs,
                                 const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                                 int max_tiles, int topk, int H, int I, const WeightArgs& gate, const WeightArgs& up,
                                 float* h, hipStream_t st);
hipError_t launch_gemm_down_i8(const int8_t* h, const float* h_scale, const int32_t* sorted_pairs,
                               const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count, int max_tiles,
                               int topk, int H, int I, const WeightArgs& down, const float* w, float* y,
                               hipStream_t st);
// y[pos][n] = gamma_down * w[pair] * (h[pos] . Wdown[n]) for every sorted position pos
hipError_t launch_gemm_down(int act, const void* h, const float* h_scale, const uint8_t* h_bscale,
                            const int32_t* hexp,
                            const int32_t* sorted_pairs, const int32_t* offsets, const TileDesc* tiles,
                            const int32_t* tile_count, int max_tiles, int topk, int H, int I,
                            const WeightArgs& down, const float* w, float* y, hipStream_t st);

}  // namespace nvfp4

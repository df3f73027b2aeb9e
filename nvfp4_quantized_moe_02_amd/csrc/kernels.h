// Kernel launchers shared between the translation units of libnvfp4moe.so. Every
// launcher enqueues on `st` and returns hipGetLastError(); argument validation is the
// C-ABI layer's job (api.hip).
#pragma once
#include "common.h"

namespace nvfp4 {

// One projection of all experts. fmt 0: NVFP4 (codes [E][N][K/2], E4M3 scales [E][N][K/16],
// global [E]); fmt 1: Q8_0 (int8 codes [E][N][K], fp16 scales [E][N][K/32], global [E] or
// null for 1).
struct WeightArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int N, K;
  int fmt;
};

struct TileDesc {
  int expert;
  int m0;
};

// elementwise.hip
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* global, int64_t rows,
                          int K, int out_dtype, void* out, hipStream_t st);
hipError_t launch_linear(const void* x, int x_dtype, int T, const uint8_t* codes, const uint8_t* scales,
                         const float* global, int N, int K, float* out, hipStream_t st);
hipError_t launch_quant_rows(const void* x, int x_dtype, int64_t rows, int cols, void* q, int q_f16,
                             float* scale, hipStream_t st);
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
// cvt_src (optional): n bf16 values converted to fp16 into cvt_dst by extra blocks of the
// first launch (n a multiple of 8).
hipError_t launch_route(const int32_t* ids, int64_t P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const RouteWs& ws, int tile_m, hipStream_t st, const void* cvt_src = nullptr,
                        void* cvt_dst = nullptr, int64_t cvt_n = 0);

// decode.hip
constexpr int kDecodeMaxT = 8;
constexpr int kDecodeMaxPairs = 64;
constexpr int kDecodeMaxTH = 40960;  // T * H: the bf16 activations of a block live in LDS
// stage 0: gate/up + SwiGLU; 1: down + combine; 2: both in one persistent launch (falls
// back to 0 then 1 when the grid cannot be co-resident). hdr: [0] dropped pairs,
// [1] error flags, [4..5] the grid-barrier counter; flags: decode_flag_bytes(H) of
// per-block release flags (counter and flags zero before first use).
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
hipError_t launch_gemm_gateup(int act, const void* a, const float* a_scale, const int32_t* sorted_pairs,
                              const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                              int max_tiles, int topk, int H, int I, const WeightArgs& gate,
                              const WeightArgs& up, void* h, hipStream_t st);
// y[pos][n] = gamma_down * w[pair] * (h[pos] . Wdown[n]) for every sorted position pos
hipError_t launch_gemm_down(int act, const void* h, const float* h_scale, const int32_t* sorted_pairs,
                            const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                            int max_tiles, int topk, int H, int I, const WeightArgs& down, const float* w,
                            float* y, hipStream_t st);

}  // namespace nvfp4

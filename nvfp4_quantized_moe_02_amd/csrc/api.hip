// The C ABI (include/nvfp4moe.h): argument validation, workspace layout and launch
// order. Every entry point validates all of its arguments before enqueueing anything.
#include "../../include/nvfp4moe.h"
#include "host.h"
#include "kernels.h"

#include <new>

using namespace nvfp4;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

bool weight_ok(const nvfp4_weight* w) {
  if (!w || (w->format != NVFP4_FMT_NVFP4 && w->format != NVFP4_FMT_Q8_0)) return false;
  return w->codes && w->scales && (w->global || w->format == NVFP4_FMT_Q8_0) && w->N > 0 && w->K > 0 &&
         (w->K % 32) == 0 && aligned(w->codes, 16) && aligned(w->scales, 16);
}

WeightArgs to_args(const nvfp4_weight* w) {
  return WeightArgs{w->codes, w->scales, w->global, w->N, w->K, w->format == NVFP4_FMT_Q8_0 ? 1 : 0};
}

// Workspace carving: offsets are computed identically by the size query and the call.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  }
};

struct RouteLayout {
  size_t hdr, counts, dropped, offsets, sorted, tiles, inv, end;
  int nblk, max_tiles;
};

RouteLayout route_layout(int64_t P, int E, bool with_tiles, Carver& c) {
  RouteLayout l;
  l.nblk = route_blocks(P);
  l.max_tiles = with_tiles ? (int)((P + kTileM - 1) / kTileM + (P < E ? P : E)) : 0;
  l.hdr = c.take(64);
  l.counts = c.take((size_t)E * l.nblk * 4);
  l.dropped = c.take((size_t)l.nblk * 4);
  l.offsets = c.take((size_t)(E + 1) * 4);
  l.sorted = c.take((size_t)P * 4);
  l.tiles = c.take((size_t)l.max_tiles * sizeof(TileDesc));
  l.inv = c.take(with_tiles ? (size_t)P * 4 : 0);
  l.end = c.off;
  return l;
}

struct PrefillLayout {
  RouteLayout r;
  size_t a16, sx, h, qh16, sh, y, end;
};

PrefillLayout prefill_layout(int T, int H, int I, int E, int topk, int act) {
  Carver c;
  PrefillLayout l;
  const int64_t P = (int64_t)T * topk;
  l.r = route_layout(P, E, true, c);
  const bool w4a8 = act != NVFP4_ACT_BF16;
  l.a16 = c.take((size_t)T * H * 2);
  l.sx = c.take(w4a8 ? (size_t)T * 4 : 0);
  l.h = c.take((size_t)P * I * (w4a8 ? 4 : 2));
  l.qh16 = c.take(w4a8 ? (size_t)P * I * 2 : 0);
  l.sh = c.take(w4a8 ? (size_t)P * 4 : 0);
  l.y = c.take((size_t)P * H * 4);
  l.end = c.off;
  return l;
}

struct DecodeLayout {
  size_t hdr, flags, h, end;
};

DecodeLayout decode_layout(int T, int H, int I, int topk) {
  Carver c;
  DecodeLayout l;
  l.hdr = c.take(64);
  l.flags = c.take(decode_flag_bytes(H));
  l.h = c.take((size_t)T * topk * I * 4);
  l.end = c.off;
  return l;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_EUNSUPPORTED: return "unsupported configuration";
    case NVFP4_EWORKSPACE: return "workspace too small";
    case NVFP4_EHIP: return "HIP runtime error";
    case NVFP4_ENOMEM: return "host memory or thread allocation failed";
    default: return "unknown status";
  }
}

int nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* global, int64_t rows, int32_t K,
                  int32_t out_dtype, void* out, void* stream) {
  if (!codes || !scales || !out || rows < 0 || K <= 0 || (K % 32) != 0) return NVFP4_EINVAL;
  if (out_dtype < NVFP4_F32 || out_dtype > NVFP4_F16) return NVFP4_EINVAL;
  if (!aligned(codes, 16) || !aligned(out, 16)) return NVFP4_EINVAL;
  (void)hipGetLastError();
  return hip_status(launch_dequant(codes, scales, global, rows, K, out_dtype, out, as_stream(stream)));
}

int nvfp4_linear(const void* x, int32_t x_dtype, int32_t T, const nvfp4_weight* w, int32_t expert, float* out,
                 void* stream) {
  if (!x || !out || T < 0 || expert < 0 || !weight_ok(w)) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (w->format != NVFP4_FMT_NVFP4) return NVFP4_EUNSUPPORTED;
  if (!aligned(x, 4)) return NVFP4_EINVAL;
  (void)hipGetLastError();
  const size_t er = (size_t)expert * w->N;
  return hip_status(launch_linear(x, x_dtype, T, w->codes + er * (w->K / 2), w->scales + er * (w->K / 16),
                                  w->global + expert, w->N, w->K, out, as_stream(stream)));
}

size_t nvfp4_route_workspace_size(int32_t T, int32_t topk, int32_t E) {
  if (T < 0 || topk < 1 || E < 1) return 0;
  Carver c;
  return route_layout((int64_t)T * topk, E, false, c).end;
}

int nvfp4_moe_route(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E, int32_t* expert_offsets,
                    int32_t* sorted_pairs, void* ws, size_t ws_bytes, void* stream) {
  if (!expert_offsets || !ws || T < 0 || topk < 1 || E < 1 || E > kMaxExperts) return NVFP4_EINVAL;
  if (T > 0 && (!topk_ids || !sorted_pairs)) return NVFP4_EINVAL;
  if ((int64_t)T * topk > (int64_t)1 << 30) return NVFP4_EUNSUPPORTED;
  if (!aligned(ws, 16)) return NVFP4_EINVAL;
  Carver c;
  const RouteLayout l = route_layout((int64_t)T * topk, E, false, c);
  if (ws_bytes < l.end) return NVFP4_EWORKSPACE;
  RouteWs rw{at<int32_t>(ws, l.counts), at<int32_t>(ws, l.dropped), at<int32_t>(ws, l.hdr), nullptr, nullptr};
  (void)hipGetLastError();
  return hip_status(
      launch_route(topk_ids, (int64_t)T * topk, E, expert_offsets, sorted_pairs, rw, kTileM, as_stream(stream)));
}

int nvfp4_quant_rows_i8(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, int8_t* q, float* scale,
                        void* stream) {
  if (!x || !q || !scale || rows < 0 || cols < 1) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (rows > 0x7fffffff) return NVFP4_EUNSUPPORTED;
  (void)hipGetLastError();
  return hip_status(launch_quant_rows(x, x_dtype, rows, cols, q, 0, scale, as_stream(stream)));
}

// Router workspace: a 256-byte header (the completion counter of the single-launch path,
// zero before first use and left zero by every call), then the fp32 logits [T][E].
constexpr size_t kRouterHeader = 256;

size_t nvfp4_router_workspace_size(int32_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return kRouterHeader + align_up((size_t)T * E * 4);
}

int nvfp4_router_topk(const void* x, int32_t x_dtype, int32_t T, int32_t H, const uint16_t* w_router, int32_t E,
                      int32_t topk, int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes,
                      void* stream) {
  if (T < 0 || H < 1 || E < 1 || topk < 1 || topk > E || !w_router || !ws) return NVFP4_EINVAL;
  if (T > 0 && (!x || !topk_ids || !topk_weights)) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(ws, 16) || !aligned(topk_ids, 4) ||
      !aligned(topk_weights, 4))
    return NVFP4_EINVAL;
  if ((H % 64) != 0 || (E % 32) != 0 || E > 2048 || topk > 64) return NVFP4_EUNSUPPORTED;
  if (ws_bytes < nvfp4_router_workspace_size(T, E)) return NVFP4_EWORKSPACE;
  if (T == 0) return NVFP4_OK;
  (void)hipGetLastError();
  return hip_status(launch_router(x, x_dtype == NVFP4_BF16 ? 1 : 0, T, H, w_router, E, topk,
                                  at<float>(ws, kRouterHeader), topk_ids, topk_weights, at<unsigned>(ws, 0),
                                  as_stream(stream)));
}

size_t nvfp4_moe_decode_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk) {
  (void)H;
  (void)E;
  if (T < 0 || I < 1 || topk < 1) return 0;
  return decode_layout(T, H, I, topk).end;
}

static int check_moe_common(const void* x, int32_t T, int32_t H, const nvfp4_weight* gate, const nvfp4_weight* up,
                            const nvfp4_weight* down, int32_t E, const int32_t* ids, const float* w, int32_t topk,
                            void* out, void* ws) {
  if (!ws || T < 0 || H < 1 || E < 1 || topk < 1) return NVFP4_EINVAL;
  if (T > 0 && (!x || !ids || !w || !out)) return NVFP4_EINVAL;  // T == 0 may pass empty (null) tensors
  if (!weight_ok(gate) || !weight_ok(up) || !weight_ok(down)) return NVFP4_EINVAL;
  const int I = gate->N;
  if (gate->K != H || up->K != H || up->N != I || down->N != H || down->K != I) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 16)) return NVFP4_EINVAL;
  if (gate->format != NVFP4_FMT_NVFP4 || up->format != NVFP4_FMT_NVFP4) return NVFP4_EUNSUPPORTED;
  return NVFP4_OK;
}

static int decode_impl(int first, int last, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                       const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                       const int32_t* topk_ids, const float* topk_weights, int32_t topk, void* out,
                       int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  int st = check_moe_common(x, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, ws);
  if (st != NVFP4_OK) return st;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_BF16) return NVFP4_EUNSUPPORTED;
  const int I = gate->N;
  if (T > kDecodeMaxT || T * topk > kDecodeMaxPairs || H > 8192 || I > 8192) return NVFP4_EUNSUPPORTED;
  if ((int64_t)T * H > kDecodeMaxTH) return NVFP4_EUNSUPPORTED;  // activations are staged in LDS
  const DecodeLayout l = decode_layout(T, H, I, topk);
  if (ws_bytes < l.end) return NVFP4_EWORKSPACE;
  if (T == 0) return NVFP4_OK;
  (void)hipGetLastError();
  // the full call runs as one persistent launch (mode 2); a single stage as mode 0 or 1
  const int mode = (first == 0 && last == 1) ? 2 : first;
  hipError_t e = launch_decode(mode, x, T, H, I, to_args(gate), to_args(up), to_args(down), E, topk_ids,
                               topk_weights, topk, out, out_dtype, at<float>(ws, l.h), at<int32_t>(ws, l.hdr),
                               at<unsigned long long>(ws, l.flags), as_stream(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

int nvfp4_moe_decode(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                     const nvfp4_weight* up, const nvfp4_weight* down, int32_t E, const int32_t* topk_ids,
                     const float* topk_weights, int32_t topk, void* out, int32_t out_dtype, void* ws,
                     size_t ws_bytes, void* stream) {
  return decode_impl(0, 1, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, out_dtype, ws,
                     ws_bytes, stream);
}

int nvfp4_moe_decode_stage(int32_t stage, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                           const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                           const int32_t* topk_ids, const float* topk_weights, int32_t topk, void* out,
                           int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (stage < 0 || stage > 1) return NVFP4_EINVAL;
  return decode_impl(stage, stage, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out,
                     out_dtype, ws, ws_bytes, stream);
}

size_t nvfp4_moe_prefill_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk, int32_t act) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || topk < 1) return 0;
  if (act < NVFP4_ACT_BF16 || act > NVFP4_ACT_W4A8_F16) return 0;
  return prefill_layout(T, H, I, E, topk, act).end;
}

static int prefill_impl(int first, int last, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                        const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                        const int32_t* topk_ids, const float* topk_weights, int32_t topk, int32_t act, void* out,
                        int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  int st = check_moe_common(x, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, ws);
  if (st != NVFP4_OK) return st;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (act < NVFP4_ACT_BF16 || act > NVFP4_ACT_W4A8_F16) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_BF16) return NVFP4_EUNSUPPORTED;
  if (act == NVFP4_ACT_W4A8) return NVFP4_EUNSUPPORTED;
  const int I = gate->N;
  if ((H % 256) != 0 || (I % 128) != 0 || E > kMaxExperts) return NVFP4_EUNSUPPORTED;
  if ((int64_t)T * topk > (int64_t)1 << 30) return NVFP4_EUNSUPPORTED;
  const PrefillLayout l = prefill_layout(T, H, I, E, topk, act);
  if (ws_bytes < l.end) return NVFP4_EWORKSPACE;
  if (T == 0) return NVFP4_OK;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const int64_t P = (int64_t)T * topk;
  float* y = at<float>(ws, l.y);
  int32_t* offsets = at<int32_t>(ws, l.r.offsets);
  int32_t* sorted = at<int32_t>(ws, l.r.sorted);
  int32_t* hdr = at<int32_t>(ws, l.r.hdr);
  TileDesc* tiles = at<TileDesc>(ws, l.r.tiles);
  void* a16 = at<void>(ws, l.a16);
  float* sx = at<float>(ws, l.sx);
  float* sh = at<float>(ws, l.sh);
  const int mode = act == NVFP4_ACT_BF16 ? 0 : 1;
  for (int stage = first; stage <= last; ++stage) {
    hipError_t e = hipSuccess;
    if (stage == 0) {  // route, stage the activations
      RouteWs rw{at<int32_t>(ws, l.r.counts), at<int32_t>(ws, l.r.dropped), hdr, tiles, at<int32_t>(ws, l.r.inv)};
      if (act == NVFP4_ACT_BF16) {
        e = launch_route(topk_ids, P, E, offsets, sorted, rw, kTileM, s, x, a16, (int64_t)T * H);
      } else {
        e = launch_route(topk_ids, P, E, offsets, sorted, rw, kTileM, s);
        if (e == hipSuccess) e = launch_quant_rows(x, NVFP4_BF16, T, H, a16, 1, sx, s);
      }
    } else if (stage == 1) {  // gate/up + SwiGLU (W4A8: then requantize h per row)
      e = launch_gemm_gateup(mode, a16, sx, sorted, offsets, tiles, hdr + 1, l.r.max_tiles, topk, H, I,
                             to_args(gate), to_args(up), at<void>(ws, l.h), s);
      if (e == hipSuccess && mode == 1)
        e = launch_quant_rows(at<void>(ws, l.h), NVFP4_F32, P, I, at<void>(ws, l.qh16), 1, sh, s);
    } else if (stage == 2) {  // down, scaled by gamma_d and the router weight, per pair
      const void* hA = mode == 0 ? at<void>(ws, l.h) : at<void>(ws, l.qh16);
      e = launch_gemm_down(mode, hA, sh, sorted, offsets, tiles, hdr + 1, l.r.max_tiles, topk, H, I,
                           to_args(down), topk_weights, y, s);
    } else {  // top-k combine in slot order, one rounding to the output dtype
      e = launch_combine(y, at<int32_t>(ws, l.r.inv), T, topk, H, out, out_dtype, s);
    }
    if (e != hipSuccess) return NVFP4_EHIP;
  }
  return NVFP4_OK;
}

int nvfp4_moe_prefill(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                      const nvfp4_weight* up, const nvfp4_weight* down, int32_t E, const int32_t* topk_ids,
                      const float* topk_weights, int32_t topk, int32_t act, void* out, int32_t out_dtype, void* ws,
                      size_t ws_bytes, void* stream) {
  return prefill_impl(0, 3, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, act, out, out_dtype,
                      ws, ws_bytes, stream);
}

int nvfp4_moe_prefill_stage(int32_t stage, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                            const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                            const int32_t* topk_ids, const float* topk_weights, int32_t topk, int32_t act, void* out,
                            int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (stage < 0 || stage > 3) return NVFP4_EINVAL;
  return prefill_impl(stage, stage, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, act, out,
                      out_dtype, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ host-CPU share
static bool host_weight_ok(const nvfp4_weight* w) {
  if (!w || (w->format != NVFP4_FMT_NVFP4 && w->format != NVFP4_FMT_Q8_0)) return false;
  return w->codes && w->scales && (w->global || w->format == NVFP4_FMT_Q8_0) && w->N > 0 && w->K > 0 &&
         (w->K % 32) == 0;
}

static host::Weight host_args(const nvfp4_weight* w) {
  return host::Weight{w->codes, w->scales, w->global, w->N, w->K, w->format == NVFP4_FMT_Q8_0 ? 1 : 0};
}

int32_t nvfp4_host_isa(void) { return host::best_isa(); }

int nvfp4_moe_decode_host(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                          const nvfp4_weight* up, const nvfp4_weight* down, int32_t E, const int32_t* topk_ids,
                          const float* topk_weights, int32_t topk, float* out, int32_t n_threads, int32_t isa,
                          int64_t* dropped) {
  if (T < 0 || H < 1 || E < 1 || topk < 1 || n_threads < 0) return NVFP4_EINVAL;
  if (T > 0 && (!x || !topk_ids || !topk_weights || !out)) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (isa < NVFP4_ISA_AUTO || isa > NVFP4_ISA_AVX512) return NVFP4_EINVAL;
  if (!host_weight_ok(gate) || !host_weight_ok(up) || !host_weight_ok(down)) return NVFP4_EINVAL;
  const int I = gate->N;
  if (gate->K != H || up->K != H || up->N != I || down->N != H || down->K != I) return NVFP4_EINVAL;
  if (gate->format != NVFP4_FMT_NVFP4 || up->format != NVFP4_FMT_NVFP4) return NVFP4_EUNSUPPORTED;
  if (isa > host::best_isa()) return NVFP4_EUNSUPPORTED;
  if ((int64_t)T * topk > 0x7fffffff) return NVFP4_EUNSUPPORTED;
  int64_t d = 0;
  if (T > 0) {
    try {
      d = host::moe_decode(x, x_dtype, T, H, I, host_args(gate), host_args(up), host_args(down), E, topk_ids,
                           topk_weights, topk, out, n_threads, isa);
    } catch (...) {  // std::bad_alloc, or std::system_error from creating a worker thread
      return NVFP4_ENOMEM;
    }
  }
  if (dropped) *dropped = d;
  return NVFP4_OK;
}

}  // extern "C"

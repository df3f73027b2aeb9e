// The C ABI (include/nvfp4moe.h): argument validation, workspace layout and launch
// order. Every entry point validates all of its arguments before enqueueing anything.
#include "../../include/nvfp4moe.h"
#include "host.h"
#include "kernels.h"

#include <mutex>
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

// The layer's shared expert, when a call has one: its three projections (one expert each,
// the routed experts' shapes and formats) become expert index E of the routed tensors.
WeightArgs to_args_shared(const nvfp4_weight* w, const nvfp4_weight* x, int xe) {
  WeightArgs a = to_args(w);
  if (x != nullptr) {
    a.xcodes = x->codes;
    a.xscales = x->scales;
    a.xglobal = x->global;
    a.xe = xe;
  }
  return a;
}

int check_shared(const nvfp4_weight* const* sh, const nvfp4_weight* gate, const nvfp4_weight* up,
                 const nvfp4_weight* down) {
  if (sh == nullptr) return NVFP4_OK;
  if (!weight_ok(sh[0]) || !weight_ok(sh[1]) || !weight_ok(sh[2])) return NVFP4_EINVAL;
  if (sh[0]->N != gate->N || sh[0]->K != gate->K || sh[1]->N != up->N || sh[1]->K != up->K ||
      sh[2]->N != down->N || sh[2]->K != down->K)
    return NVFP4_EINVAL;
  if (sh[0]->format != NVFP4_FMT_NVFP4 || sh[1]->format != NVFP4_FMT_NVFP4 || sh[2]->format != down->format)
    return NVFP4_EUNSUPPORTED;
  return NVFP4_OK;
}

// Bytes after the main workspace that hold the routing with the shared slot appended
// (ids [T][topk+1], then weights [T][topk+1]).
size_t shared_routing_bytes(int T, int topk) { return 2 * align_up((size_t)T * (topk + 1) * 4); }

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

// Prefill workspace regions (act BF16 | W4A8 | W4A4): staged x (fp16 | int8 | NVFP4 codes
// [T][H/2]) and its per-row exponents (int32) | scales (fp32) | scales (fp32), the W4A4
// block scales (E4M3 [T][H/16]); h in sorted-pair order (fp16 scaled per gate/up block |
// fp32 | fp32) with the block exponents (int32 [P][blocks] | absent | absent); the
// requantized h (absent | int8 [P][I] | codes [P][I/2]) with its row scales (fp32 [P]) and
// the W4A4 block scales (E4M3 [P][I/16]); y, each pair's scaled down row (fp32 [P][H]).
struct PrefillLayout {
  RouteLayout r;
  size_t xa, xs, xbs, h, hexp, qh, sh, qhbs, y, end;
  size_t xa_b, xs_b, xbs_b, h_b, hexp_b, qh_b, sh_b, qhbs_b, y_b;
};

PrefillLayout prefill_layout(int T, int H, int I, int E, int topk, int act) {
  Carver c;
  PrefillLayout l;
  const int64_t P = (int64_t)T * topk;
  l.r = route_layout(P, E, true, c);
  const bool rowq = act != NVFP4_ACT_BF16;  // activations quantized per row
  const bool f4 = act == NVFP4_ACT_W4A4;
  l.xa_b = f4 ? (size_t)T * H / 2 : (size_t)T * H * (rowq ? 1 : 2);
  l.xs_b = (size_t)T * 4;
  l.xbs_b = f4 ? (size_t)T * H / 16 : 0;
  l.h_b = (size_t)P * I * (rowq ? 4 : 2);
  l.hexp_b = rowq ? 0 : (size_t)P * gateup_blocks(I) * 4;
  l.qh_b = rowq ? (size_t)P * I / (f4 ? 2 : 1) : 0;
  l.sh_b = rowq ? (size_t)P * 4 : 0;
  l.qhbs_b = f4 ? (size_t)P * I / 16 : 0;
  l.y_b = (size_t)P * H * 4;
  l.xa = c.take(l.xa_b);
  l.xs = c.take(l.xs_b);
  l.xbs = c.take(l.xbs_b);
  l.h = c.take(l.h_b);
  l.hexp = c.take(l.hexp_b);
  l.qh = c.take(l.qh_b);
  l.sh = c.take(l.sh_b);
  l.qhbs = c.take(l.qhbs_b);
  l.y = c.take(l.y_b);
  l.end = c.off;
  return l;
}

struct DecodeLayout {
  size_t hdr, flags, h, end;
};

// The flag lines are reserved for the largest supported H, so calls with different H on
// one workspace never place h where an earlier call's flag lines are.
DecodeLayout decode_layout(int T, int H, int I, int topk) {
  (void)H;
  Carver c;
  DecodeLayout l;
  l.hdr = c.take(64);
  l.flags = c.take(decode_flag_bytes(kDecodeMaxH));
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
  return hip_status(launch_quant_rows(x, x_dtype, rows, cols, q, scale, as_stream(stream)));
}

int nvfp4_quant_rows_nvfp4(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, uint8_t* codes,
                           uint8_t* scales, float* g, void* stream) {
  if (!x || !codes || !scales || !g || rows < 0 || cols < 16 || cols % 16 != 0) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(g, 4)) return NVFP4_EINVAL;
  if (rows > 0x7fffffff) return NVFP4_EUNSUPPORTED;
  (void)hipGetLastError();
  return hip_status(launch_quant_rows_nvfp4(x, x_dtype, rows, cols, codes, scales, g, as_stream(stream)));
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

// dry: validate only (nothing is enqueued).
// dry: validate only (nothing is enqueued). shared: the layer's shared expert (gate, up,
// down) or null; with one, every token gets slot topk = the shared expert (index E, weight
// 1), and the routing with that slot is written after the main workspace first.
static int decode_impl(int first, int last, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                       const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                       const int32_t* topk_ids, const float* topk_weights, int32_t topk, void* out,
                       int32_t out_dtype, void* ws, size_t ws_bytes, void* stream, bool dry = false,
                       const nvfp4_weight* const* shared = nullptr) {
  int st = check_moe_common(x, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, ws);
  if (st != NVFP4_OK) return st;
  if ((st = check_shared(shared, gate, up, down)) != NVFP4_OK) return st;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_BF16) return NVFP4_EUNSUPPORTED;
  const int I = gate->N;
  const int keff = shared ? topk + 1 : topk;
  if (T > kDecodeMaxT || T * keff > kDecodeMaxPairs || H > kDecodeMaxH || I > 8192) return NVFP4_EUNSUPPORTED;
  if ((int64_t)T * H > kDecodeMaxTH) return NVFP4_EUNSUPPORTED;  // activations are staged in LDS
  const DecodeLayout l = decode_layout(T, H, I, keff);
  if (ws_bytes < l.end) return NVFP4_EWORKSPACE;
  if (T == 0 || dry) return NVFP4_OK;
  (void)hipGetLastError();
  // The decode kernel reads the caller's [T][topk] routing and, with a shared expert (index
  // E, the expert its WeightArgs hold apart), forms slot topk of every token itself.
  const nvfp4_weight* const* sh = shared;
  // the full call runs as one persistent launch (mode 2); a single stage as mode 0 or 1
  const int mode = (first == 0 && last == 1) ? 2 : first;
  hipError_t e = launch_decode(mode, x, T, H, I, to_args_shared(gate, sh ? sh[0] : nullptr, E),
                               to_args_shared(up, sh ? sh[1] : nullptr, E), to_args_shared(down, sh ? sh[2] : nullptr, E),
                               shared ? E + 1 : E, topk_ids, topk_weights, keff, out, out_dtype, at<float>(ws, l.h),
                               at<int32_t>(ws, l.hdr), at<unsigned long long>(ws, l.flags), as_stream(stream));
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

size_t nvfp4_moe_decode_shared_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk) {
  (void)E;
  if (T < 0 || I < 1 || topk < 1) return 0;
  return decode_layout(T, H, I, topk + 1).end;
}

int nvfp4_moe_decode_shared(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                            const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                            const nvfp4_weight* shared_gate, const nvfp4_weight* shared_up,
                            const nvfp4_weight* shared_down, const int32_t* topk_ids, const float* topk_weights,
                            int32_t topk, void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream) {
  const nvfp4_weight* sh[3] = {shared_gate, shared_up, shared_down};
  return decode_impl(0, 1, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, out_dtype, ws,
                     ws_bytes, stream, false, sh);
}

}  // extern "C"

// ------------------------------------------------------------------ decode without allocation
// Device scratch of nvfp4_moe_decode_noalloc: the decode workspace (header, barrier flag
// lines, h) in a static device array, one copy per GPU, held until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until set up

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The device address of this device's scratch (taken with the device current, once per
// device; the array's name in host code is only a stand-in). On that first set-up the
// header and the flag lines, the barrier state that must start at zero, are cleared by a
// fill kernel on the caller's stream (ahead of the call's own launch).
int scratch_for_device(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return NVFP4_EHIP;
    const DecodeLayout l = decode_layout(1, 1, 1, 1);  // header and flags sit first, for any shape
    zero_fill_kernel<<<dim3(16), 256, 0, s>>>(static_cast<uint4*>(p), l.h / 16);
    if (hipGetLastError() != hipSuccess) return NVFP4_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}
}  // namespace

extern "C" {

int nvfp4_moe_decode_noalloc(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                             const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                             const int32_t* topk_ids, const float* topk_weights, int32_t topk, void* out,
                             int32_t out_dtype, void* stream) {
  if (!gate || T < 0 || topk < 1) return NVFP4_EINVAL;
  const size_t need = nvfp4_moe_decode_workspace_size(T, H, gate->N, E, topk);
  if (need > kNoAllocScratchBytes) return NVFP4_EUNSUPPORTED;
  // every argument is checked before the set-up enqueues anything (a stand-in aligned,
  // non-null workspace pointer: validation never dereferences it)
  void* const probe = reinterpret_cast<void*>(uintptr_t(256));
  int st = decode_impl(0, 1, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, out_dtype, probe,
                       kNoAllocScratchBytes, stream, true);
  if (st != NVFP4_OK || T == 0) return st;
  void* ws = nullptr;
  st = scratch_for_device(as_stream(stream), &ws);
  if (st != NVFP4_OK) return st;
  return decode_impl(0, 1, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, out, out_dtype, ws,
                     kNoAllocScratchBytes, stream);
}

size_t nvfp4_moe_prefill_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk, int32_t act) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || topk < 1) return 0;
  if (act < NVFP4_ACT_BF16 || act > NVFP4_ACT_W4A4) return 0;
  return prefill_layout(T, H, I, E, topk, act).end;
}

// shared: the layer's shared expert (gate, up, down) or null; with one, the call routes
// E + 1 experts with topk + 1 slots per token, slot topk being the shared expert (index E,
// weight 1), from a routing written after the main workspace at the start of stage 0.
static int prefill_impl(int first, int last, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                        const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down, int32_t E0,
                        const int32_t* topk_ids0, const float* topk_weights0, int32_t topk0, int32_t act, void* out,
                        int32_t out_dtype, void* ws, size_t ws_bytes, void* stream,
                        const nvfp4_weight* const* shared = nullptr) {
  int st = check_moe_common(x, T, H, gate, up, down, E0, topk_ids0, topk_weights0, topk0, out, ws);
  if (st != NVFP4_OK) return st;
  if ((st = check_shared(shared, gate, up, down)) != NVFP4_OK) return st;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_EINVAL;
  if (act < NVFP4_ACT_BF16 || act > NVFP4_ACT_W4A4) return NVFP4_EINVAL;
  if (x_dtype != NVFP4_BF16) return NVFP4_EUNSUPPORTED;
  const int I = gate->N;
  const int E = shared ? E0 + 1 : E0, topk = shared ? topk0 + 1 : topk0;
  if ((H % 256) != 0 || (I % 128) != 0 || I > 8192 || E > kMaxExperts) return NVFP4_EUNSUPPORTED;
  if ((int64_t)T * topk > (int64_t)1 << 30) return NVFP4_EUNSUPPORTED;
  const PrefillLayout l = prefill_layout(T, H, I, E, topk, act);
  const size_t extra = shared ? shared_routing_bytes(T, topk0) : 0;
  if (ws_bytes < l.end + extra) return NVFP4_EWORKSPACE;
  if (T == 0) return NVFP4_OK;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const int32_t* topk_ids = shared ? at<int32_t>(ws, l.end) : topk_ids0;
  const float* topk_weights = shared ? at<float>(ws, l.end + extra / 2) : topk_weights0;
  const WeightArgs ga = to_args_shared(gate, shared ? shared[0] : nullptr, E0);
  const WeightArgs ua = to_args_shared(up, shared ? shared[1] : nullptr, E0);
  const WeightArgs da = to_args_shared(down, shared ? shared[2] : nullptr, E0);
  const int64_t P = (int64_t)T * topk;
  float* y = at<float>(ws, l.y);
  int32_t* offsets = at<int32_t>(ws, l.r.offsets);
  int32_t* sorted = at<int32_t>(ws, l.r.sorted);
  int32_t* hdr = at<int32_t>(ws, l.r.hdr);
  TileDesc* tiles = at<TileDesc>(ws, l.r.tiles);
  void* xa = at<void>(ws, l.xa);
  // GEMM activation mode: 0 fp16 (BF16), 1 int8 (W4A8, W4A8_F16), 2 NVFP4 (W4A4)
  const int mode = act == NVFP4_ACT_BF16 ? 0 : act == NVFP4_ACT_W4A4 ? 2 : 1;
  float* xscale = mode != 0 ? at<float>(ws, l.xs) : nullptr;
  int32_t* xexp = mode == 0 ? at<int32_t>(ws, l.xs) : nullptr;
  int32_t* hexp = mode == 0 ? at<int32_t>(ws, l.hexp) : nullptr;
  float* sh = mode != 0 ? at<float>(ws, l.sh) : nullptr;
  uint8_t* xbs = mode == 2 ? at<uint8_t>(ws, l.xbs) : nullptr;
  uint8_t* qhbs = mode == 2 ? at<uint8_t>(ws, l.qhbs) : nullptr;
  for (int stage = first; stage <= last; ++stage) {
    hipError_t e = hipSuccess;
    if (stage == 0) {  // route, stage the activations
      RouteWs rw{at<int32_t>(ws, l.r.counts), at<int32_t>(ws, l.r.dropped), hdr, tiles, at<int32_t>(ws, l.r.inv)};
      if (shared)
        e = launch_append_shared(topk_ids0, topk_weights0, T, topk0, E0, const_cast<int32_t*>(topk_ids),
                                 const_cast<float*>(topk_weights), s);
      if (e == hipSuccess && mode == 0) {
        e = launch_route(topk_ids, P, E, offsets, sorted, rw, kTileM, s, x, xa, xexp, T, H);
      } else if (e == hipSuccess) {
        e = launch_route(topk_ids, P, E, offsets, sorted, rw, kTileM, s);
        if (e == hipSuccess && mode == 1)
          e = launch_quant_rows(x, NVFP4_BF16, T, H, static_cast<int8_t*>(xa), xscale, s);
        else if (e == hipSuccess)
          e = launch_quant_rows_nvfp4(x, NVFP4_BF16, T, H, static_cast<uint8_t*>(xa), xbs, xscale, s);
      }
    } else if (stage == 1) {  // gate/up + SwiGLU (W4A8, W4A4: then requantize h per row)
      if (act == NVFP4_ACT_W4A8)
        e = launch_gemm_gateup_i8(static_cast<const int8_t*>(xa), xscale, sorted, offsets, tiles, hdr + 1,
                                  l.r.max_tiles, topk, H, I, ga, ua, at<float>(ws, l.h), s);
      else
        e = launch_gemm_gateup(mode, xa, xscale, xbs, xexp, sorted, offsets, tiles, hdr + 1, l.r.max_tiles, topk, H,
                               I, ga, ua, at<void>(ws, l.h), hexp, s);
      if (e == hipSuccess && mode == 1)
        e = launch_quant_rows(at<void>(ws, l.h), NVFP4_F32, P, I, at<int8_t>(ws, l.qh), sh, s);
      else if (e == hipSuccess && mode == 2)
        e = launch_quant_rows_nvfp4(at<void>(ws, l.h), NVFP4_F32, P, I, at<uint8_t>(ws, l.qh), qhbs, sh, s);
    } else if (stage == 2) {  // down, scaled by gamma_d and the router weight, per pair
      const void* hA = mode == 0 ? at<void>(ws, l.h) : at<void>(ws, l.qh);
      if (act == NVFP4_ACT_W4A8)
        e = launch_gemm_down_i8(static_cast<const int8_t*>(hA), sh, sorted, offsets, tiles, hdr + 1, l.r.max_tiles,
                                topk, H, I, da, topk_weights, y, s);
      else
        e = launch_gemm_down(mode, hA, sh, qhbs, hexp, sorted, offsets, tiles, hdr + 1, l.r.max_tiles, topk, H, I,
                             da, topk_weights, y, s);
    } else {  // top-k combine in slot order, one rounding to the output dtype
      e = launch_combine(y, at<int32_t>(ws, l.r.inv), T, topk, H, out, out_dtype, s);
    }
    if (e != hipSuccess) return NVFP4_EHIP;
  }
  return NVFP4_OK;
}

int nvfp4_moe_prefill_workspace_region(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk, int32_t act,
                                       int32_t region, size_t* offset, size_t* bytes) {
  if (!offset || !bytes || T < 0 || H < 1 || I < 1 || E < 1 || topk < 1) return NVFP4_EINVAL;
  if (act < NVFP4_ACT_BF16 || act > NVFP4_ACT_W4A4) return NVFP4_EINVAL;
  const PrefillLayout l = prefill_layout(T, H, I, E, topk, act);
  const size_t P = (size_t)T * topk;
  switch (region) {
    case NVFP4_WS_EXPERT_OFFSETS: *offset = l.r.offsets; *bytes = (size_t)(E + 1) * 4; break;
    case NVFP4_WS_SORTED_PAIRS: *offset = l.r.sorted; *bytes = P * 4; break;
    case NVFP4_WS_PAIR_POSITION: *offset = l.r.inv; *bytes = P * 4; break;
    case NVFP4_WS_X_STAGED: *offset = l.xa; *bytes = l.xa_b; break;
    case NVFP4_WS_X_ROWSCALE: *offset = l.xs; *bytes = l.xs_b; break;
    case NVFP4_WS_H: *offset = l.h; *bytes = l.h_b; break;
    case NVFP4_WS_H_EXP: *offset = l.hexp; *bytes = l.hexp_b; break;
    case NVFP4_WS_H_Q: *offset = l.qh; *bytes = l.qh_b; break;
    case NVFP4_WS_H_SCALE: *offset = l.sh; *bytes = l.sh_b; break;
    case NVFP4_WS_Y: *offset = l.y; *bytes = l.y_b; break;
    case NVFP4_WS_X_BLOCKSCALE: *offset = l.xbs; *bytes = l.xbs_b; break;
    case NVFP4_WS_H_BLOCKSCALE: *offset = l.qhbs; *bytes = l.qhbs_b; break;
    default: return NVFP4_EINVAL;
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

size_t nvfp4_moe_prefill_shared_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                                               int32_t act) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || topk < 1) return 0;
  if (act < NVFP4_ACT_BF16 || act > NVFP4_ACT_W4A4) return 0;
  return prefill_layout(T, H, I, E + 1, topk + 1, act).end + shared_routing_bytes(T, topk);
}

int nvfp4_moe_prefill_shared(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                             const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                             const nvfp4_weight* shared_gate, const nvfp4_weight* shared_up,
                             const nvfp4_weight* shared_down, const int32_t* topk_ids, const float* topk_weights,
                             int32_t topk, int32_t act, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                             void* stream) {
  const nvfp4_weight* sh[3] = {shared_gate, shared_up, shared_down};
  return prefill_impl(0, 3, x, x_dtype, T, H, gate, up, down, E, topk_ids, topk_weights, topk, act, out, out_dtype,
                      ws, ws_bytes, stream, sh);
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

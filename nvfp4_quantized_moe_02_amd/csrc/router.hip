// Router: logits = x . Wr^T with a bf16 router matrix [E][H], then per token the k largest
// logits (equal logits in expert-id order) and the softmax over those k. The pages feed
// the prompt path's BF16 projections, the router among them, with FP32-exact inputs
// ("Strata NVFP4" README); the routing rule is this library's reading (see the header).
//
// Logits run on bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation). A bf16
// input is one pass. An fp32 input is split exactly into three bf16 parts
// (x = b0 + b1 + b2 with b0 = bf16(x), b1 = bf16(x - b0), b2 = x - b0 - b1, exact for x in
// the normal range), so every product with a bf16 weight is exact and the sum is the fp32
// accumulation of exact products: three passes with the same weight fragments.
//
// Up to 64 tokens: a block covers 32 tokens x 32 experts, its 4 waves split the
// inputs and add their partial sums through LDS, so the router matrix is streamed by E/32
// blocks; fragments are loaded straight from memory. Many tokens: 128 x 128 tiles with the
// x tile shared through LDS (router_logits_tile_kernel).
#include "kernels.h"

namespace nvfp4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int CTRL>
__device__ __forceinline__ int dpp_movi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// The value of lane (lane ^ 16) / (lane ^ 32), by the row-swap moves (VALU, no LDS trip).
// A swap of v with itself leaves in its first result the lower row (half) copied over the
// upper one and in its second the upper copied over the lower.
__device__ __forceinline__ int xor16i(int v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane & 16) ? (int)r[0] : (int)r[1];
}
__device__ __forceinline__ int xor32i(int v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane & 32) ? (int)r[0] : (int)r[1];
}
__device__ __forceinline__ float xor16f(float v, int lane) { return __int_as_float(xor16i(__float_as_int(v), lane)); }
__device__ __forceinline__ float xor32f(float v, int lane) { return __int_as_float(xor32i(__float_as_int(v), lane)); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 inputs of one token: bf16 (one part) or fp32 split into three bf16 parts.
template <int XPARTS>
__device__ __forceinline__ void load_x8(const void* x, size_t off, bf16x8_t* parts) {
  if constexpr (XPARTS == 1) {
    parts[0] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off));
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t w[3][4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t h[3][2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float f = v[j + q];
        const uint32_t b0 = f32_to_bf16_rne(f);
        const float r1 = f - __uint_as_float(b0 << 16);  // exact
        const uint32_t b1 = f32_to_bf16_rne(r1);
        const float r2 = r1 - __uint_as_float(b1 << 16);  // exact, at most 8 significant bits
        h[0][q] = b0;
        h[1][q] = b1;
        h[2][q] = __float_as_uint(r2) >> 16;
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) w[p][j >> 1] = h[p][0] | (h[p][1] << 16);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) parts[p] = __builtin_bit_cast(bf16x8_t, make_uint4(w[p][0], w[p][1], w[p][2], w[p][3]));
  }
}

template <int XPARTS, bool KSPLIT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x, int T, int H,
                                                            const uint16_t* __restrict__ wr, int E,
                                                            float* __restrict__ logits) {
  __shared__ float red[KSPLIT ? 3 : 1][64][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.x * 32;
  const int e0 = blockIdx.y * (KSPLIT ? 32 : 128) + (KSPLIT ? 0 : wave * 32);
  if (!KSPLIT && e0 >= E) return;  // this wave's experts are past E (E % 32 == 0)
  const int tok = t0 + l32 < T ? t0 + l32 : T - 1;  // rows past T recompute row T-1 (not stored)
  const int ex = e0 + l32;
  const int k0 = KSPLIT ? wave * (H / 4) : 0, k1 = KSPLIT ? k0 + H / 4 : H;
  const uint16_t* wrow = wr + (size_t)ex * H;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // batches of U steps of 16 inputs, the next batch's loads issued before the current
  // batch's MFMAs. The step index is wave-uniform (a lane's input offset adds 8*half), so
  // the guards of a partial last batch are branches, not lane masks: a matrix instruction
  // ignores the lane mask, so a masked-off step would still be accumulated. Steps past the
  // end load the last step again and are skipped.
  constexpr int U = XPARTS == 1 ? 8 : 4;
  const int nsteps = (k1 - k0) >> 4;
  struct Batch {
    bf16x8_t x[U][XPARTS];
    bf16x8_t w[U];
  };
  auto load_batch = [&](int s0, Batch& b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + 16 * (s0 + u < nsteps ? s0 + u : nsteps - 1) + 8 * half;
      load_x8<XPARTS>(x, (size_t)tok * H + kk, b.x[u]);
      b.w[u] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wrow + kk));
    }
  };
  auto mma_batch = [&](int s0, const Batch& b) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < nsteps)
#pragma unroll
        for (int p = 0; p < XPARTS; ++p) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b.x[u][p], b.w[u], acc, 0, 0, 0);
  };
  Batch b0, b1;
  load_batch(0, b0);
  for (int s0 = 0; s0 < nsteps; s0 += 2 * U) {
    if (s0 + U < nsteps) load_batch(s0 + U, b1);
    mma_batch(s0, b0);
    if (s0 + U >= nsteps) break;
    if (s0 + 2 * U < nsteps) load_batch(s0 + 2 * U, b0);
    mma_batch(s0 + U, b1);
  }
  // acc[v]: token row 8*(v/4) + 4*half + v%4 of the tile, expert column l32
  if constexpr (KSPLIT) {
    if (wave > 0)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave - 1][lane][i] = acc[i];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = ((acc[i] + red[0][lane][i]) + red[1][lane][i]) + red[2][lane][i];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + 8 * (v >> 2) + 4 * half + (v & 3);
    if (t < T) logits[(size_t)t * E + ex] = acc[v];
  }
}

// One wave per token: k rounds of a wave-wide argmax (larger logit first, then the lower
// expert id; NaN logits rank below every number), then the softmax over the k selected
// logits (expf of the differences to the largest, IEEE division by their sum). `load(e)`
// reads the token's logit of expert e.
//
// Up to 512 experts (8 per lane) each lane first sorts its 8 candidates once, as 64-bit
// keys (the logit's order-preserving bits above, 2^32 - 1 - id below, so a larger key is a
// larger logit or, on equal logits, the lower id), and every round is one wave-wide max of
// the lanes' heads, after which the winning lane drops its head.
__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t v) {
  return ((uint64_t)(uint32_t)dpp_movi<CTRL>((int)(v >> 32)) << 32) | (uint32_t)dpp_movi<CTRL>((int)(uint32_t)v);
}
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v, int lane) {
  v = key_max(v, dpp_key<0xB1>(v));
  v = key_max(v, dpp_key<0x4E>(v));
  v = key_max(v, dpp_key<0x124>(v));
  v = key_max(v, dpp_key<0x128>(v));
  v = key_max(v, ((uint64_t)(uint32_t)xor16i((int)(v >> 32), lane) << 32) | (uint32_t)xor16i((int)(uint32_t)v, lane));
  v = key_max(v, ((uint64_t)(uint32_t)xor32i((int)(v >> 32), lane) << 32) | (uint32_t)xor32i((int)(uint32_t)v, lane));
  return v;
}

template <int NPL, class Load>  // logits per lane (E <= 64 * NPL)
__device__ __forceinline__ void topk_token(int lane, int E, int k, Load load, int32_t* __restrict__ ids,
                                           float* __restrict__ wts) {
  if constexpr (NPL == 8) {
    uint64_t key[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = lane + 64 * j;
      float f = e < E ? load(e) : 0.f;
      f = f == f ? (f == 0.f ? 0.f : f) : -__builtin_inff();  // NaN ranks lowest; -0 ties +0
      const uint32_t u = __float_as_uint(f);
      const uint32_t ou = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key[j] = e < E ? ((uint64_t)ou << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;  // 0: no expert
    }
    auto cas = [&](int i, int j) {
      const uint64_t a = key[i], b = key[j];
      key[i] = a > b ? a : b;
      key[j] = a > b ? b : a;
    };
    // 19-comparator sorting network for 8, descending
    cas(0, 2); cas(1, 3); cas(4, 6); cas(5, 7);
    cas(0, 4); cas(1, 5); cas(2, 6); cas(3, 7);
    cas(0, 1); cas(2, 3); cas(4, 5); cas(6, 7);
    cas(2, 4); cas(3, 5);
    cas(1, 4); cas(3, 6);
    cas(1, 2); cas(3, 4); cas(5, 6);
    uint64_t mine = 0;
    for (int r = 0; r < k; ++r) {
      const uint64_t m = wave_max_key(key[0], lane);
      if (lane == r) mine = m;
      const bool won = key[0] == m;  // keys are distinct: one lane
#pragma unroll
      for (int j = 0; j < 7; ++j) key[j] = won ? key[j + 1] : key[j];
      key[7] = won ? 0ull : key[7];
    }
    const uint32_t hi = (uint32_t)(mine >> 32);
    const float my_l = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
    const int my_id = (int)(0xFFFFFFFFu - (uint32_t)mine);
    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
    const float ez = lane < k ? expf(my_l - top) : 0.f;
    float s = ez;  // sum over the wave: rows by DPP, then the row swaps
    s += dpp_mov<0xB1>(s);
    s += dpp_mov<0x4E>(s);
    s += dpp_mov<0x124>(s);
    s += dpp_mov<0x128>(s);
    s += xor16f(s, lane);
    s += xor32f(s, lane);
    if (lane < k) {
      ids[lane] = my_id;
      wts[lane] = ez / s;
    }
    return;
  }
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    const float f = e < E ? load(e) : -__builtin_inff();
    v[j] = f == f ? f : -__builtin_inff();  // NaN ranks lowest
  }
  uint64_t taken = 0;  // bit j: this lane's value j is selected
  int my_id = 0;
  float my_l = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      const bool free = e < E && !((taken >> j) & 1);
      if (free && (v[j] > bv || (v[j] == bv && e < bi))) {
        bv = v[j];
        bi = e;
      }
    }
    auto take = [&](float ov, int oi) {
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    };
    // within each row of 16 lanes by DPP moves, then across the 4 rows by row swaps
    take(dpp_mov<0xB1>(bv), dpp_movi<0xB1>(bi));
    take(dpp_mov<0x4E>(bv), dpp_movi<0x4E>(bi));
    take(dpp_mov<0x124>(bv), dpp_movi<0x124>(bi));
    take(dpp_mov<0x128>(bv), dpp_movi<0x128>(bi));
    take(xor16f(bv, lane), xor16i(bi, lane));
    take(xor32f(bv, lane), xor32i(bi, lane));
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == r) {
      my_id = bi;
      my_l = bv;
    }
  }
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float ez = lane < k ? expf(my_l - top) : 0.f;
  float s = ez;  // sum over the wave: rows by DPP, then the row swaps
  s += dpp_mov<0xB1>(s);
  s += dpp_mov<0x4E>(s);
  s += dpp_mov<0x124>(s);
  s += dpp_mov<0x128>(s);
  s += xor16f(s, lane);
  s += xor32f(s, lane);
  if (lane < k) {
    ids[lane] = my_id;
    wts[lane] = ez / s;
  }
}

template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  topk_token<NPL>(lane, E, k, [row](int e) { return row[e]; }, ids + (size_t)t * k, wts + (size_t)t * k);
}

// Many tokens: a block covers 32*RB tokens x 128 experts; wave w computes the 32 experts
// 32w .. 32w+31 for all of them (RB row blocks), so each weight fragment feeds RB MFMAs
// (x parts: RB * XPARTS). The x tile is staged through LDS 64 inputs at a time (converted
// to its bf16 parts once), 16-byte chunks XOR-swizzled by row; weight fragments are loaded
// one 64-input chunk ahead.
template <int XPARTS, int RB>
__global__ __launch_bounds__(256) void router_logits_tile_kernel(const void* __restrict__ x, int T, int H,
                                                                 const uint16_t* __restrict__ wr, int E,
                                                                 float* __restrict__ logits) {
  constexpr int TM = 32 * RB;  // tokens per block
  __shared__ __attribute__((aligned(16))) uint16_t xs[XPARTS][TM * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int t0 = blockIdx.x * TM;
  const int e0 = blockIdx.y * 128 + wave * 32;
  const bool have = e0 < E;  // E % 32 == 0; waves past E still take part in the barriers
  const uint16_t* wrow = wr + (size_t)(have ? e0 + l32 : 0) * H;
  f32x16_t acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
  // staging: thread t holds 8 inputs (chunk t & 7) of rows (t >> 3) + 32 i, i < RB, loaded
  // one chunk ahead in registers, and stores their bf16 parts into LDS
  const int srow = tid >> 3, sch = tid & 7;
  typedef uint4 XRaw[XPARTS == 1 ? 1 : 2];
  auto load_xr = [&](int kc, XRaw* raw) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = srow + 32 * i;
      const size_t off = (size_t)(t0 + r < T ? t0 + r : T - 1) * H + kc + 8 * sch;
      if constexpr (XPARTS == 1) {
        raw[i][0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
      } else {
        raw[i][0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + off);
        raw[i][1] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + off + 4);
      }
    }
  };
  auto stage = [&](const XRaw* raw) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = srow + 32 * i;
      bf16x8_t parts[XPARTS];
      load_x8<XPARTS>(raw[i], 0, parts);
#pragma unroll
      for (int p = 0; p < XPARTS; ++p)
        *reinterpret_cast<uint4*>(&xs[p][r * 64 + ((sch ^ (r & 7)) << 3)]) = __builtin_bit_cast(uint4, parts[p]);
    }
  };
  auto load_w = [&](int kc, bf16x8_t* w) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      w[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(wrow + kc + 16 * s + 8 * half));
  };
  bf16x8_t wcur[4], wnext[4];
  XRaw xr[RB];
  load_w(0, wcur);
  load_xr(0, xr);
  for (int kc = 0; kc < H; kc += 64) {
    __syncthreads();  // the previous chunk's fragment reads are done
    stage(xr);
    if (kc + 64 < H) {
      load_w(kc + 64, wnext);
      load_xr(kc + 64, xr);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + half;  // 16-byte chunk of this lane's 8 inputs
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int r = rb * 32 + l32;
#pragma unroll
        for (int p = 0; p < XPARTS; ++p) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&xs[p][r * 64 + ((ch ^ (r & 7)) << 3)]));
          acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wcur[s], acc[rb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) wcur[s] = wnext[s];
  }
  if (!have) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = t0 + rb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
      if (t < T) logits[(size_t)t * E + e0 + l32] = acc[rb][v];
    }
}

// Decode sizes (T <= 8, x small enough for LDS): 16 lanes per expert row, 4 rows per wave,
// 16 experts per block; x (bf16 or fp32) in LDS; each lane issues all the weight loads of
// its row share (8 bf16 per 16-byte load) before the arithmetic: products in FP32 FMAs
// (each product exact inside the FMA), each lane's sum in input order, then a fixed
// 16-lane reduction.
//
// Up to one token per wave of a block (RANK), the same launch also ranks: logits are
// stored through to memory (agent scope), each block counts itself done on a counter in
// the workspace once its stores have completed, and the block that completes the count
// reads every logit back with agent-coherent loads and runs the top-k (one wave per
// token), then sets the counter back to zero. More tokens rank in a second launch.
// s_waitcnt immediate: no vector-memory operation of this wave outstanding.
constexpr int kRouterVmcnt0 = (7 << 4) | (0xF << 8);
// Waves per GEMV block (4 expert rows each). 1 and 2 measured slower: the ranking block then
// ranks several tokens per wave one after another.
constexpr int kRouterGemvWaves = 4;

template <int XT, int NPL, int WAVES, bool RANK>  // XT 1: bf16 x, 0: fp32 x; NPL: logits per lane in the
                                                  // top-k; RANK: this launch also ranks (T <= WAVES)
__global__ __launch_bounds__(64 * WAVES) void router_gemv_kernel(const void* __restrict__ x, int T, int H,
                                                          const uint16_t* __restrict__ wr, int E,
                                                          float* __restrict__ logits, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ wts,
                                                          unsigned* __restrict__ done) {
  extern __shared__ __attribute__((aligned(16))) char xl[];
  const int tid = threadIdx.x;
  const int n16 = T * H * (XT ? 2 : 4) / 16;
  for (int i = tid; i < n16; i += 64 * WAVES) reinterpret_cast<uint4*>(xl)[i] = reinterpret_cast<const uint4*>(x)[i];
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15;
  const int e = (blockIdx.x * WAVES + wave) * 4 + (lane >> 4);  // E % (4 * WAVES) == 0
  const uint16_t* row = wr + (size_t)e * H;
  const int nch = H >> 3;  // 8-input chunks; this lane takes l16, l16 + 16, ...
  float acc[kDecodeMaxT];
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) acc[t] = 0.f;
  constexpr int B = 16;  // chunks in flight per lane
  for (int c0 = l16; c0 < nch; c0 += 16 * B) {
    uint4 w[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + 16 * b;
      w[b] = c < nch ? *reinterpret_cast<const uint4*>(row + 8 * c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + 16 * b;
      if (c >= nch) break;
      const uint32_t wd[4] = {w[b].x, w[b].y, w[b].z, w[b].w};
      float wf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wf[2 * j] = __uint_as_float(wd[j] << 16);
        wf[2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
      }
#pragma unroll
      for (int t = 0; t < kDecodeMaxT; ++t) {
        if (t < T) {
          float xv[8];
          if (XT) {
            const uint4 q = reinterpret_cast<const uint4*>(xl)[(size_t)t * (H >> 3) + c];
            const uint32_t qd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              xv[2 * j] = __uint_as_float(qd[j] << 16);
              xv[2 * j + 1] = __uint_as_float(qd[j] & 0xFFFF0000u);
            }
          } else {
            const float4 qa = reinterpret_cast<const float4*>(xl)[((size_t)t * H + 8 * c) / 4];
            const float4 qb = reinterpret_cast<const float4*>(xl)[((size_t)t * H + 8 * c) / 4 + 1];
            xv[0] = qa.x; xv[1] = qa.y; xv[2] = qa.z; xv[3] = qa.w;
            xv[4] = qb.x; xv[5] = qb.y; xv[6] = qb.z; xv[7] = qb.w;
          }
          float a = acc[t];
#pragma unroll
          for (int j = 0; j < 8; ++j) a = fmaf(wf[j], xv[j], a);
          acc[t] = a;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) {
    if (t < T) {
      const float v = sum16(acc[t]);
      if (l16 == 0) __hip_atomic_store(logits + (size_t)t * E + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (!RANK) return;
  __builtin_amdgcn_s_waitcnt(kRouterVmcnt0);
  __syncthreads();
  __shared__ int last;
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == gridDim.x - 1;
    if (last) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  for (int t = wave; t < T; t += WAVES) {
    const float* row = logits + (size_t)t * E;
    topk_token<NPL>(
        lane, E, k, [row](int e) { return __hip_atomic_load(row + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); },
        ids + (size_t)t * k, wts + (size_t)t * k);
  }
}

template <int XT, int NPL, bool RANK>
static hipError_t launch_gemv(const void* x, int T, int H, const uint16_t* wr, int E, int k, float* logits,
                              int32_t* ids, float* wts, unsigned* done, size_t xbytes, hipStream_t st) {
  constexpr int W = kRouterGemvWaves;
  hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(router_gemv_kernel<XT, NPL, W, RANK>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)xbytes);
  if (ea != hipSuccess) return ea;
  router_gemv_kernel<XT, NPL, W, RANK><<<dim3((unsigned)(E / (4 * W))), 64 * W, xbytes, st>>>(
      x, T, H, wr, E, logits, k, ids, wts, done);
  return hipGetLastError();
}

hipError_t launch_router(const void* x, int x_dtype, int T, int H, const uint16_t* wr, int E, int k, float* logits,
                         int32_t* ids, float* wts, unsigned* done, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const size_t xbytes = (size_t)T * H * (x_dtype == 1 ? 2 : 4);
  if (T <= kRouterGemvWaves && xbytes <= 64 * 1024) {  // one launch: logits, then one wave per token ranks
    if (x_dtype == 1)
      return E <= 512 ? launch_gemv<1, 8, true>(x, T, H, wr, E, k, logits, ids, wts, done, xbytes, st)
                      : launch_gemv<1, 32, true>(x, T, H, wr, E, k, logits, ids, wts, done, xbytes, st);
    return E <= 512 ? launch_gemv<0, 8, true>(x, T, H, wr, E, k, logits, ids, wts, done, xbytes, st)
                    : launch_gemv<0, 32, true>(x, T, H, wr, E, k, logits, ids, wts, done, xbytes, st);
  } else if (T <= kDecodeMaxT && xbytes <= 64 * 1024) {
    hipError_t eg = x_dtype == 1 ? launch_gemv<1, 8, false>(x, T, H, wr, E, k, logits, ids, wts, done, xbytes, st)
                                 : launch_gemv<0, 8, false>(x, T, H, wr, E, k, logits, ids, wts, done, xbytes, st);
    if (eg != hipSuccess) return eg;
  } else if (T <= 64) {
    const dim3 g1((unsigned)((T + 31) / 32), (unsigned)(E / 32));
    if (x_dtype == 1) router_logits_kernel<1, true><<<g1, 256, 0, st>>>(x, T, H, wr, E, logits);
    else router_logits_kernel<3, true><<<g1, 256, 0, st>>>(x, T, H, wr, E, logits);
  } else {
    const dim3 g1((unsigned)((T + 63) / 64), (unsigned)((E + 127) / 128));
    if (x_dtype == 1) router_logits_tile_kernel<1, 2><<<g1, 256, 0, st>>>(x, T, H, wr, E, logits);
    else router_logits_tile_kernel<3, 2><<<g1, 256, 0, st>>>(x, T, H, wr, E, logits);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2((unsigned)((T + 3) / 4));
  if (E <= 512) router_topk_kernel<8><<<g2, 256, 0, st>>>(logits, T, E, k, ids, wts);
  else router_topk_kernel<32><<<g2, 256, 0, st>>>(logits, T, E, k, ids, wts);
  return hipGetLastError();
}

}  // namespace nvfp4

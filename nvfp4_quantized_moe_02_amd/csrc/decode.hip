// Decode path (1..8 tokens): HBM-bound NVFP4 GEMVs with FP32 arithmetic, the pages'
// quality profile for expert decode ("#1858 strata-safetensors": canonical FP32 expert
// decode). Two launches per layer:
//   1. gate/up + SwiGLU: one block per (unique expert, 16 intermediate rows); h in fp32.
//   2. down + top-k combine: each wave owns 4 output rows and sums every routed pair of
//      every token into them in a fixed order, so the result is deterministic.
// Both kernels derive the unique-expert list from topk_ids themselves (no host sync).
//
// Lane mapping: 16 lanes per weight row, each lane reads 16-byte chunks (32 inputs =
// two scale groups) with 128-bit loads; four rows per wave-wide load, so each load
// instruction covers 4 rows x 256 contiguous bytes.
#include "kernels.h"

namespace nvfp4 {

// Unique experts of the routed pairs, in order of first appearance. Every thread of
// the block calls this (it holds barriers); wave 0 does the work. s_ids receives each
// pair's id (or -1 when dropped), s_uniq the unique ids; returns their number.
__device__ int block_unique_experts(const int32_t* __restrict__ ids, int P, int E, int* s_ids, int* s_uniq,
                                    int* s_nu, int* s_drop) {
  const int tid = threadIdx.x;
  int e = -1;
  bool valid = false;
  if (tid < 64) {
    e = tid < P ? ids[tid] : -1;
    valid = tid < P && (unsigned)e < (unsigned)E;
    s_ids[tid] = valid ? e : -1;
  }
  __syncthreads();
  if (tid < 64) {
    bool first = valid;
    for (int q = 0; q < tid; ++q)
      if (s_ids[q] == e) first = false;
    const uint64_t fm = __ballot(first);
    const uint64_t dm = __ballot(tid < P && !valid);
    if (first) s_uniq[__popcll(fm & ((1ull << tid) - 1ull))] = e;
    if (tid == 0) {
      *s_nu = __popcll(fm);
      *s_drop = __popcll(dm);
    }
  }
  __syncthreads();
  return *s_nu;
}

// One 16-byte chunk (32 inputs, two scale groups) of a weight row dotted with bf16
// activations held as 16 packed pairs. Returns the scaled partial sum.
__device__ __forceinline__ float dot_chunk_bf16(const uint4 c, uint32_t sc, const uint32_t* xv) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p = part[i >> 1];
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(w[i]), __builtin_bit_cast(bf16x2_t, xv[4 * i + 0]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(w[i]), __builtin_bit_cast(bf16x2_t, xv[4 * i + 1]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(w[i]), __builtin_bit_cast(bf16x2_t, xv[4 * i + 2]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(w[i]), __builtin_bit_cast(bf16x2_t, xv[4 * i + 3]), p, false);
    part[i >> 1] = p;
  }
  return part[0] * e4m3_f32<0>(sc) + part[1] * e4m3_f32<1>(sc);
}

// ------------------------------------------------------------------ gate/up + SwiGLU
// CH = chunk iterations per lane = ceil(H / 32 / 16).
template <int CH>
__global__ __launch_bounds__(256) void decode_gateup_kernel(const uint16_t* __restrict__ x, int H, int I,
                                                            WeightArgs gate, WeightArgs up, int E,
                                                            const int32_t* __restrict__ ids, int P, int topk,
                                                            float* __restrict__ h, int32_t* __restrict__ hdr) {
  __shared__ int s_ids[64], s_uniq[64], s_pairs[64];
  __shared__ int s_nu, s_np, s_drop;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nu = block_unique_experts(ids, P, E, s_ids, s_uniq, &s_nu, &s_drop);
  if (tid < 64) {
    if (tid == 0 && blockIdx.x == 0 && blockIdx.y == 0) hdr[0] = s_drop;
    const int ex = (int)blockIdx.y < nu ? s_uniq[blockIdx.y] : -2;
    const bool match = tid < P && s_ids[tid] == ex;
    const uint64_t mm = __ballot(match);
    if (match) s_pairs[__popcll(mm & ((1ull << tid) - 1ull))] = tid;
    if (tid == 0) s_np = __popcll(mm);
  }
  __syncthreads();
  if ((int)blockIdx.y >= nu) return;
  const int e = s_uniq[blockIdx.y];
  const int np = s_np;
  const int row = blockIdx.x * 16 + wave * 4 + (lane >> 4);
  const int l16 = lane & 15;
  const int nch = H >> 5;  // 16-byte chunks per row
  if (row >= I) return;
  const size_t grow = (size_t)e * I + row;
  const uint8_t* gc = gate.codes + grow * (H / 2);
  const uint8_t* uc = up.codes + grow * (H / 2);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(gate.scales + grow * (H / 16));
  const uint16_t* us = reinterpret_cast<const uint16_t*>(up.scales + grow * (H / 16));
  uint4 gcode[CH], ucode[CH];
  uint32_t gsc[CH], usc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = l16 + 16 * c;
    if (ch < nch) {
      gcode[c] = *reinterpret_cast<const uint4*>(gc + ch * 16);
      ucode[c] = *reinterpret_cast<const uint4*>(uc + ch * 16);
      gsc[c] = gs[ch];
      usc[c] = us[ch];
    }
  }
  const float gg = gate.global[e], gu = up.global[e];
  for (int i = 0; i < np; ++i) {
    const int p = s_pairs[i];
    const int t = p / topk;
    const uint32_t* xr = reinterpret_cast<const uint32_t*>(x + (size_t)t * H);
    float ga = 0.f, ua = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = l16 + 16 * c;
      if (ch < nch) {
        uint32_t xv[16];
        const uint4* xp = reinterpret_cast<const uint4*>(xr + ch * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = xp[q];
          xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
        }
        ga += dot_chunk_bf16(gcode[c], gsc[c], xv);
        ua += dot_chunk_bf16(ucode[c], usc[c], xv);
      }
    }
    ga = sum16(ga);
    ua = sum16(ua);
    if (l16 == 0) h[(size_t)p * I + row] = silu(ga * gg) * (ua * gu);
  }
}

// ------------------------------------------------------------------ down + combine
// CH = chunk iterations per lane = ceil(I / 32 / 16). UB experts' rows are loaded
// before any is used, to keep enough bytes in flight.
template <int CH, int UB>
__global__ __launch_bounds__(128) void decode_down_kernel(const float* __restrict__ h, int H, int I,
                                                          WeightArgs down, int E, const int32_t* __restrict__ ids,
                                                          const float* __restrict__ w, int P, int topk, int T,
                                                          void* __restrict__ out, int out_dtype) {
  __shared__ int s_ids[64], s_uniq[64], s_list[64], s_start[65];
  __shared__ int s_nu, s_drop;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nu = block_unique_experts(ids, P, E, s_ids, s_uniq, &s_nu, &s_drop);
  // pairs grouped by unique expert, each group in pair order
  if (tid < 64) {
    int start = 0;
    for (int u = 0; u < nu; ++u) {
      const bool m = s_ids[tid] == s_uniq[u];
      const uint64_t mm = __ballot(m);
      if (m) s_list[start + __popcll(mm & ((1ull << tid) - 1ull))] = tid;
      if (tid == 0) s_start[u] = start;
      start += __popcll(mm);
    }
    if (tid == 0) s_start[nu] = start;
  }
  __syncthreads();
  const int row = blockIdx.x * 8 + wave * 4 + (lane >> 4);
  const int l16 = lane & 15;
  const int nch = I >> 5;
  const bool row_ok = row < H;
  float acc[kDecodeMaxT];
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) acc[t] = 0.f;
  for (int u0 = 0; u0 < nu; u0 += UB) {
    uint4 code[UB][CH];
    uint32_t sc[UB][CH];
#pragma unroll
    for (int b = 0; b < UB; ++b) {
      const int u = u0 + b;
      if (u < nu && row_ok) {
        const size_t grow = (size_t)s_uniq[u] * H + row;
        const uint8_t* rc = down.codes + grow * (I / 2);
        const uint16_t* rs = reinterpret_cast<const uint16_t*>(down.scales + grow * (I / 16));
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int ch = l16 + 16 * c;
          if (ch < nch) {
            code[b][c] = *reinterpret_cast<const uint4*>(rc + ch * 16);
            sc[b][c] = rs[ch];
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < UB; ++b) {
      const int u = u0 + b;
      if (u >= nu) break;
      const float gd = down.global[s_uniq[u]];
      for (int i = s_start[u]; i < s_start[u + 1]; ++i) {
        const int p = s_list[i];
        const int t = p / topk;
        const float* hr = h + (size_t)p * I;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int ch = l16 + 16 * c;
          if (ch < nch && row_ok) {
            const uint32_t wd[4] = {code[b][c].x, code[b][c].y, code[b][c].z, code[b][c].w};
            const float4* hp = reinterpret_cast<const float4*>(hr + ch * 32);
            float g2[2] = {0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 ha = hp[2 * q], hb = hp[2 * q + 1];
              const f32x2_t w0 = e2m1x2_f32<0>(wd[q]), w1 = e2m1x2_f32<1>(wd[q]);
              const f32x2_t w2 = e2m1x2_f32<2>(wd[q]), w3 = e2m1x2_f32<3>(wd[q]);
              float s = g2[q >> 1];
              s = fmaf(w0[0], ha.x, s); s = fmaf(w0[1], ha.y, s);
              s = fmaf(w1[0], ha.z, s); s = fmaf(w1[1], ha.w, s);
              s = fmaf(w2[0], hb.x, s); s = fmaf(w2[1], hb.y, s);
              s = fmaf(w3[0], hb.z, s); s = fmaf(w3[1], hb.w, s);
              g2[q >> 1] = s;
            }
            part += g2[0] * e4m3_f32<0>(sc[b][c]) + g2[1] * e4m3_f32<1>(sc[b][c]);
          }
        }
        const float coef = w[p] * gd;
#pragma unroll
        for (int tt = 0; tt < kDecodeMaxT; ++tt)
          if (tt == t) acc[tt] = fmaf(coef, part, acc[tt]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) {
    if (t >= T) break;
    const float v = sum16(acc[t]);
    if (l16 == 0 && row_ok) {
      if (out_dtype == 0) reinterpret_cast<float*>(out)[(size_t)t * H + row] = v;
      else reinterpret_cast<uint16_t*>(out)[(size_t)t * H + row] = f32_to_bf16_bits(v);
    }
  }
}

template <int CHG, int CHD>
static hipError_t launch_decode_t(int stage, const void* x, int T, int H, int I, const WeightArgs& gate,
                                  const WeightArgs& up, const WeightArgs& down, int E, const int32_t* ids,
                                  const float* w, int topk, void* out, int out_dtype, float* h, int32_t* hdr,
                                  hipStream_t st) {
  const int P = T * topk;
  if (stage == 0) {
    dim3 g1((I + 15) / 16, P);
    decode_gateup_kernel<CHG><<<g1, 256, 0, st>>>(reinterpret_cast<const uint16_t*>(x), H, I, gate, up, E, ids, P,
                                                  topk, h, hdr);
  } else {
    dim3 g2((H + 7) / 8);
    decode_down_kernel<CHD, 8><<<g2, 128, 0, st>>>(h, H, I, down, E, ids, w, P, topk, T, out, out_dtype);
  }
  return hipGetLastError();
}

hipError_t launch_decode(int stage, const void* x, int T, int H, int I, const WeightArgs& gate,
                         const WeightArgs& up, const WeightArgs& down, int E, const int32_t* ids, const float* w,
                         int topk, void* out, int out_dtype, float* h, int32_t* hdr, hipStream_t st) {
  const int chg = ((H >> 5) + 15) / 16;  // 1..16 for H <= 8192
  const int chd = ((I >> 5) + 15) / 16;
#define NVFP4_DEC(G, D)                                                                                          \
  if (chg <= G && chd <= D)                                                                                      \
    return launch_decode_t<G, D>(stage, x, T, H, I, gate, up, down, E, ids, w, topk, out, out_dtype, h, hdr, st);
  NVFP4_DEC(1, 1)
  NVFP4_DEC(2, 1)
  NVFP4_DEC(2, 2)
  NVFP4_DEC(4, 2)
  NVFP4_DEC(4, 4)
  NVFP4_DEC(8, 4)
  NVFP4_DEC(8, 8)
  NVFP4_DEC(16, 8)
  NVFP4_DEC(16, 16)
#undef NVFP4_DEC
  return hipErrorInvalidValue;
}

}  // namespace nvfp4

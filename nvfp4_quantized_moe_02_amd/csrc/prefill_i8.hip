// W4A8 prompt path on int8 matrix cores ("Strata NVFP4" README, "How it differs from
// upstream Strata": the int8 W4A8 prompt path that keeps 8-bit activations).
//
// The activations are int8 codes with an fp32 scale per row (the per-row rule of
// nvfp4_quant_rows_i8). The NVFP4 weights enter the matrix cores as exact int8 values
// 2 * e2m1 (0, +-1, +-2, +-3, +-4, +-6, +-8, +-12), so v_mfma_i32_32x32x16_i8 over one
// 16-input scale group gives the group's integer dot product exactly (at most
// 127 * 12 * 16 in magnitude). The group's E4M3 scale differs from group to group and
// from weight row to weight row, so it cannot ride through the matrix core: each group's
// int32 result is converted to fp32 and multiplied by e4m3 / 2 (exact: at most 15 + 4
// significant bits) into the fp32 accumulator. That is one conversion and one FMA per
// accumulator element per 16 inputs, 32 VALU instructions per matrix instruction, so this
// variant is bound by VALU issue, not by the matrix cores; the fp16 variant
// (NVFP4_ACT_W4A8_F16) computes the same product with the scale folded into exact fp16
// weights and is the faster one. A Q8_0 down projection's 32-input blocks span two
// matrix instructions that share one scale, so it rescales once per two.
//
// Layout. Tile = (expert, up to 128 routed rows) x one N block: 4 waves, each owning
// 32 weight rows per column block (gate/up: 32 gate and the same 32 up rows; down: 64
// rows). Per K-block of 64 inputs the block stages A (int8, [128][64]) and the weights
// of its 256 rows, unpacked to int8 ([256][64]), in LDS. Weights are unpacked with two
// byte-permute lookups per four codes (one for the positive values, one for the
// negative ones, chosen by the sign bit). The bytes of both operands are kept in the
// order (k0, k2, k4, k6, k1, k3, k5, k7) within each group of 8 inputs, which the
// weight unpack produces directly and A is permuted into while staged; the matrix core
// pairs equal byte positions, so the dot product is unchanged.
#include "kernels.h"

namespace nvfp4 {

typedef int i32x16_t_ __attribute__((ext_vector_type(16)));

constexpr int Q_BM = kTileM;   // rows per tile (the shared tile list)
constexpr int Q_KB = 64;       // inputs per K-block
constexpr int Q_WAVES = 4;
constexpr int Q_THREADS = 64 * Q_WAVES;
constexpr int Q_NCOL = 256;    // weight rows per block (gate/up: 128 gate + 128 up)

// Four E2M1 codes (the low nibble of each byte) -> four int8 values 2 * e2m1.
__device__ __forceinline__ uint32_t e2m1x4_i8(uint32_t nib) {
  const uint32_t sel = nib & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sel);  // 0 1 2 3 | 4 6 8 12
  const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sel);  // negated
  const uint32_t mask = ((nib >> 3) & 0x01010101u) * 0xFFu;
  return (neg & mask) | (pos & ~mask);
}

// 8 bytes in input order (lo = k0..k3, hi = k4..k7) -> (k0, k2, k4, k6 | k1, k3, k5, k7).
__device__ __forceinline__ uint2 even_odd(uint32_t lo, uint32_t hi) {
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x06040200u), __builtin_amdgcn_perm(hi, lo, 0x07050301u));
}

// LDS rows of 64 bytes: 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 3).
__device__ __forceinline__ int q_slot(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4); }

template <bool GATEUP, bool Q8, int NRB>
__device__ __forceinline__ void gemm_i8_tile(const TileCtx& tc, const int8_t* __restrict__ A, int K,
                                             const uint8_t* b0row, const uint8_t* b1row, const uint8_t* s0row,
                                             const uint8_t* s1row, const WeightArgs& w0, const WeightArgs& w1,
                                             void* __restrict__ out, int ldo, char* lds, const int* s_src,
                                             const float* s_coef) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nkb = K / Q_KB;
  char* As = lds;                   // [128][64] int8
  char* Bs = lds + Q_BM * 64;       // [256][64] int8

  // staging: thread t copies 32 bytes (two chunks) of A row t/2, and the codes of weight
  // row t (NVFP4: 32 bytes; Q8_0: 64 bytes) for one K-block
  const int arow = tid >> 1, ach = (tid & 1) * 2;
  const int8_t* asrc = A + (size_t)s_src[arow] * K + ach * 16;
  const size_t rowbytes = Q8 ? K : K / 2;
  const uint8_t* bsrc = (GATEUP && tid >= Q_NCOL / 2) ? b1row + (size_t)(tid - Q_NCOL / 2) * rowbytes
                                                      : b0row + (size_t)tid * rowbytes;
  constexpr int BCH = Q8 ? 4 : 2;  // 16-byte code chunks per weight row per K-block
  uint4 ar[2], br[BCH];
  uint32_t sr[2];
  // scale words: each lane's two weight rows (column blocks), 4 bytes per K-block
  // (NVFP4: the four groups' E4M3 bytes; Q8_0: the two blocks' fp16 scales)
  auto load = [&](int kb) {
    const int kc = kb < nkb ? kb : nkb - 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) ar[i] = *reinterpret_cast<const uint4*>(asrc + kc * Q_KB + i * 16);
#pragma unroll
    for (int i = 0; i < BCH; ++i) br[i] = *reinterpret_cast<const uint4*>(bsrc + kc * (Q8 ? 64 : 32) + i * 16);
    sr[0] = *reinterpret_cast<const uint32_t*>(s0row + kc * 4);
    sr[1] = *reinterpret_cast<const uint32_t*>(s1row + kc * 4);
  };

  f32x16_t acc[NRB][2];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] = 0.f;

  load(0);
  for (int kb = 0; kb < nkb; ++kb) {
    // A in even/odd byte order; the weights unpacked to int8 in the same order
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint2 lo = even_odd(ar[i].x, ar[i].y), hi = even_odd(ar[i].z, ar[i].w);
      *reinterpret_cast<uint4*>(As + q_slot(arow, ach + i)) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    if constexpr (Q8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 lo = even_odd(br[i].x, br[i].y), hi = even_odd(br[i].z, br[i].w);
        *reinterpret_cast<uint4*>(Bs + q_slot(tid, i)) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else {
      // 16 code bytes = 32 inputs = two chunks of 16 int8; a code word holds 8 inputs
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t w[4] = {br[i].x, br[i].y, br[i].z, br[i].w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = e2m1x4_i8(w[j] & 0x0F0F0F0Fu);           // k0 k2 k4 k6 of this word
          o[2 * j + 1] = e2m1x4_i8((w[j] >> 4) & 0x0F0F0F0Fu);  // k1 k3 k5 k7
        }
        *reinterpret_cast<uint4*>(Bs + q_slot(tid, 2 * i)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(Bs + q_slot(tid, 2 * i + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
    const uint32_t s0 = sr[0], s1 = sr[1];
    __syncthreads();
    load(kb + 1);  // the next K-block's bytes arrive while this one is computed
    // this lane's weight rows in the block tile: column block cb
    const int brow0 = GATEUP ? wave * 32 + l32 : wave * 64 + l32;
    const int brow1 = GATEUP ? Q_NCOL / 2 + wave * 32 + l32 : wave * 64 + 32 + l32;
#pragma unroll
    for (int g = 0; g < 4; g += (Q8 ? 2 : 1)) {
      // NVFP4: scale byte g of each column's word, times 1/2 (the weights are 2 * e2m1);
      // Q8_0: fp16 scale g/2, shared by groups g and g+1
      float sc0, sc1;
      if constexpr (Q8) {
        sc0 = (float)__builtin_bit_cast(f16x2_t, s0)[g >> 1];
        sc1 = (float)__builtin_bit_cast(f16x2_t, s1)[g >> 1];
      } else {
        sc0 = __builtin_amdgcn_cvt_f32_fp8((int)(s0 >> (8 * g)), 0) * 0.5f;
        sc1 = __builtin_amdgcn_cvt_f32_fp8((int)(s1 >> (8 * g)), 0) * 0.5f;
      }
      long bf0[2], bf1[2];
#pragma unroll
      for (int q = 0; q < (Q8 ? 2 : 1); ++q) {
        const int gg = g + q;
        bf0[q] = *reinterpret_cast<const long*>(Bs + q_slot(brow0, gg) + half * 8);
        bf1[q] = *reinterpret_cast<const long*>(Bs + q_slot(brow1, gg) + half * 8);
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int ar_ = rb * 32 + l32;
        i32x16_t_ c0 = {}, c1 = {};
#pragma unroll
        for (int q = 0; q < (Q8 ? 2 : 1); ++q) {
          const long af = *reinterpret_cast<const long*>(As + q_slot(ar_, g + q) + half * 8);
          c0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(af, bf0[q], c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(af, bf1[q], c1, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[rb][0][i] = fmaf((float)c0[i], sc0, acc[rb][0][i]);
          acc[rb][1][i] = fmaf((float)c1[i], sc1, acc[rb][1][i]);
        }
      }
    }
    __syncthreads();  // every wave has read this K-block's tiles
  }

  // Accumulator element i of lane (half, l32): row rb*32 + 8*(i/4) + 4*half + i%4 of the
  // tile, weight row l32 of the column block.
  if constexpr (GATEUP) {
    const float gg = w0.gamma_nvfp4(tc.e), gu = w1.gamma_nvfp4(tc.e);
    const int col = tc.nb * (Q_NCOL / 2) + wave * 32 + l32;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const float xs = s_coef[r];
        const float h = silu_fast(acc[rb][0][i] * (xs * gg)) * (acc[rb][1][i] * (xs * gu));
        if (r < tc.rows) reinterpret_cast<float*>(out)[(size_t)(tc.base + tc.m0 + r) * ldo + col] = h;
      }
  } else {
    const float gd = w0.gamma(tc.e);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const float c = s_coef[r] * gd;
        if (r < tc.rows) {
          float* yrow = reinterpret_cast<float*>(out) + (size_t)(tc.base + tc.m0 + r) * ldo + tc.nb * Q_NCOL;
          yrow[wave * 64 + l32] = acc[rb][0][i] * c;
          yrow[wave * 64 + 32 + l32] = acc[rb][1][i] * c;
        }
      }
  }
}

// GATEUP: gate/up + SwiGLU into fp32 h (w0 = gate, w1 = up); else down (w0 = down),
// each pair's row times gamma_d, its router weight and its h scale, into y.
template <bool GATEUP, bool Q8>
__global__ __launch_bounds__(Q_THREADS, 2) void moe_gemm_i8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, const TileDesc* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    int topk, int K, int NB, WeightArgs w0, WeightArgs w1, const float* __restrict__ route_w,
    void* __restrict__ out, int ldo) {
  __shared__ __attribute__((aligned(16))) char lds[Q_BM * 64 + Q_NCOL * 64];
  __shared__ int s_src[Q_BM];
  __shared__ float s_coef[Q_BM];

  // XCD-aware order: consecutive logical tiles run on the same XCD
  const int total = *tile_count * NB;
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
  if (jj >= per) return;
  const int L = xcd * per + jj;
  if (L >= total) return;
  TileCtx tc;
  const int tile = L / NB;
  tc.nb = L - tile * NB;
  const TileDesc td = tiles[tile];
  tc.e = td.expert;
  tc.m0 = td.m0;
  tc.base = offsets[tc.e];
  const int Me = offsets[tc.e + 1] - tc.base;
  tc.rows = Me - tc.m0 < Q_BM ? Me - tc.m0 : Q_BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31;
  if (tid < Q_BM) {
    const int r = tid < tc.rows ? tid : tc.rows - 1;  // padding rows repeat the last row
    const int pos = tc.base + tc.m0 + r;
    const int p = sorted_pairs[pos];
    if (GATEUP) {
      s_src[tid] = p / topk;
      s_coef[tid] = a_scale[p / topk];
    } else {
      s_src[tid] = pos;
      s_coef[tid] = route_w[p] * a_scale[pos];
    }
  }
  const uint8_t *b0row, *b1row, *s0row, *s1row;
  // scale bytes per weight row: NVFP4 K/16 E4M3, Q8_0 K/32 fp16
  if (GATEUP) {
    const size_t row0 = (size_t)tc.nb * (Q_NCOL / 2);
    b0row = w0.code_row(tc.e, row0, K / 2);
    b1row = w1.code_row(tc.e, row0, K / 2);
    s0row = w0.scale_row(tc.e, row0 + wave * 32 + l32);
    s1row = w1.scale_row(tc.e, row0 + wave * 32 + l32);
  } else {
    const size_t row0 = (size_t)tc.nb * Q_NCOL;
    b0row = w0.code_row(tc.e, row0, Q8 ? K : K / 2);
    b1row = b0row;
    s0row = w0.scale_row(tc.e, row0 + wave * 64 + l32);
    s1row = w0.scale_row(tc.e, row0 + wave * 64 + 32 + l32);
  }
  __syncthreads();
  const int nrb = (tc.rows + 31) >> 5;
  const int8_t* Ab = A;
#define NVFP4_I8_TILE(R) \
  gemm_i8_tile<GATEUP, Q8, R>(tc, Ab, K, b0row, b1row, s0row, s1row, w0, w1, out, ldo, lds, s_src, s_coef)
  if (nrb == 4)
    NVFP4_I8_TILE(4);
  else if (nrb == 3)
    NVFP4_I8_TILE(3);
  else if (nrb == 2)
    NVFP4_I8_TILE(2);
  else
    NVFP4_I8_TILE(1);
#undef NVFP4_I8_TILE
}

static inline unsigned grid_i8(int max_tiles, int NB) {
  const long long g = (long long)max_tiles * NB;
  return (unsigned)(((g + 7) / 8) * 8);
}

hipError_t launch_gemm_gateup_i8(const int8_t* a, const float* a_scale, const int32_t* sorted_pairs,
                                 const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                                 int max_tiles, int topk, int H, int I, const WeightArgs& gate, const WeightArgs& up,
                                 float* h, hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  const int NB = I / (Q_NCOL / 2);
  moe_gemm_i8_kernel<true, false><<<grid_i8(max_tiles, NB), Q_THREADS, 0, st>>>(
      a, a_scale, sorted_pairs, offsets, tiles, tile_count, topk, H, NB, gate, up, nullptr, h, I);
  return hipGetLastError();
}

hipError_t launch_gemm_down_i8(const int8_t* h, const float* h_scale, const int32_t* sorted_pairs,
                               const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count, int max_tiles,
                               int topk, int H, int I, const WeightArgs& down, const float* w, float* y,
                               hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  const int NB = H / Q_NCOL;
  if (down.fmt == 1)
    moe_gemm_i8_kernel<false, true><<<grid_i8(max_tiles, NB), Q_THREADS, 0, st>>>(
        h, h_scale, sorted_pairs, offsets, tiles, tile_count, topk, I, NB, down, down, w, y, H);
  else
    moe_gemm_i8_kernel<false, false><<<grid_i8(max_tiles, NB), Q_THREADS, 0, st>>>(
        h, h_scale, sorted_pairs, offsets, tiles, tile_count, topk, I, NB, down, down, w, y, H);
  return hipGetLastError();
}

}  // namespace nvfp4

// Prefill path: grouped GEMMs over the routed pairs on gfx950 matrix cores, one launch
// per stage for all experts ("Strata NVFP4" README, "How it differs from upstream
// Strata": an MMQ group's experts gathered in one launch; prompt chunks up to 32K
// tokens, each streaming every expert of a layer once).
//
// Tile = (expert, 128 routed rows) x one N block; 4 waves. Each wave owns a 128 x 64
// output block (4 x 2 blocks of v_mfma_f32_32x32x16_f16). The A operand (activations,
// fp16) is staged through LDS, double-buffered, 64 inputs per K-block; rows are
// gathered by token for gate/up and contiguous for down. The B operand never touches
// LDS: each lane loads the 16 code bytes and 2 scale bytes its fragment needs with one
// 128-bit load and unpacks them exactly to fp16 (exponent-scaled convert, then one
// packed fp16 multiply by the scale's mantissa factor), so every weight byte is read
// once per tile and decoded once per wave. Within a K-block the reduction order of the
// 64 inputs is permuted (lane half 0 takes inputs 0..31, half 1 inputs 32..63); A uses
// the same permutation, so the dot products are unchanged.
//
// gate/up: wave w computes gate and up for the same 32 intermediate indices, so SwiGLU
// runs in registers: h = SiLU(gamma_g * g) * (gamma_u * u) (gate scale before SiLU, the
// "Strata NVFP4" README's per-projection output scale). down: the epilogue multiplies by
// gamma_d and the router weight and adds into an fp32 [T][H] accumulator.
#include "kernels.h"

namespace nvfp4 {

constexpr int BM = kTileM;
constexpr int KBLK = 64;
constexpr int LDS_STRIDE = 72;  // fp16 per LDS row: 64 + 8 padding (144 B, conflict-free 128-bit reads)

struct BRaw {
  uint4 c;     // 32 codes
  uint32_t s;  // 2 scale bytes (groups of this lane's 32 inputs)
};

__device__ __forceinline__ BRaw load_braw(const uint8_t* rowc, const uint8_t* rows, int kb, int half) {
  BRaw r;
  r.c = *reinterpret_cast<const uint4*>(rowc + kb * 32 + half * 16);
  r.s = *reinterpret_cast<const uint16_t*>(rows + kb * 4 + half * 2);
  return r;
}

__device__ __forceinline__ uint32_t word_of(const uint4& c, int s) {
  return s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
}

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8_t bfrag(uint32_t word, const F16Scale& sc) {
  f16x2_t o[4];
  unpack8_f16(word, sc, o);
  const f16x4_t lo = __builtin_shufflevector(o[0], o[1], 0, 1, 2, 3);
  const f16x4_t hi = __builtin_shufflevector(o[2], o[3], 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// GATEUP: gate/up + SwiGLU (w0 = gate, w1 = up), else down + combine (w0 = down).
// ASCALE: multiply by a per-row activation scale (the W4A8 int8 scales).
// HOUT32: gate/up writes fp32 h (for the int8 requantization), else fp16 h.
template <bool GATEUP, bool ASCALE, bool HOUT32>
__global__ __launch_bounds__(256, 2) void moe_gemm_f16_kernel(
    const uint16_t* __restrict__ A, const float* __restrict__ a_scale, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, const TileDesc* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    int topk, int K, int NB, WeightArgs w0, WeightArgs w1, const float* __restrict__ route_w,
    void* __restrict__ out, int ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ int s_src[BM];
  __shared__ int s_tok[BM];
  __shared__ float s_coef[BM];

  // XCD-aware order: consecutive logical tiles (the N blocks of one row tile, which
  // share their A rows) run on the same XCD and its L2.
  const int total = *tile_count * NB;
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
  if (jj >= per) return;
  const int L = xcd * per + jj;
  if (L >= total) return;
  const int tile = L / NB, nb = L - tile * NB;
  const TileDesc td = tiles[tile];
  const int e = td.expert, m0 = td.m0;
  const int base = offsets[e];
  const int Me = offsets[e + 1] - base;
  const int rows = Me - m0 < BM ? Me - m0 : BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  if (tid < BM) {
    const int r = tid < rows ? tid : rows - 1;  // padding rows repeat the last row
    const int pos = base + m0 + r;
    const int p = sorted_pairs[pos];
    if (GATEUP) {
      s_src[tid] = p / topk;
      s_coef[tid] = ASCALE ? a_scale[p / topk] : 1.0f;
    } else {
      s_src[tid] = pos;
      s_tok[tid] = p / topk;
      s_coef[tid] = route_w[p] * (ASCALE ? a_scale[pos] : 1.0f);
    }
  }

  const uint8_t* bc[2];
  const uint8_t* bs[2];
  if (GATEUP) {
    const size_t grow = (size_t)e * w0.N + nb * 128 + wave * 32 + l32;
    bc[0] = w0.codes + grow * (K / 2);
    bs[0] = w0.scales + grow * (K / 16);
    bc[1] = w1.codes + grow * (K / 2);
    bs[1] = w1.scales + grow * (K / 16);
  } else {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const size_t grow = (size_t)e * w0.N + nb * 256 + wave * 64 + cb * 32 + l32;
      bc[cb] = w0.codes + grow * (K / 2);
      bs[cb] = w0.scales + grow * (K / 16);
    }
  }
  __syncthreads();

  const int nkb = K / KBLK;
  const int arow = tid >> 3, achunk = tid & 7;
  const uint16_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) asrc[i] = A + (size_t)s_src[arow + 32 * i] * K + achunk * 8;

  f32x16_t acc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] = 0.f;

  uint4 areg[4];
  BRaw braw[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) areg[i] = *reinterpret_cast<const uint4*>(asrc[i]);
  braw[0] = load_braw(bc[0], bs[0], 0, half);
  braw[1] = load_braw(bc[1], bs[1], 0, half);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(&As[0][(arow + 32 * i) * LDS_STRIDE + achunk * 8]) = areg[i];

  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    const BRaw cur0 = braw[0], cur1 = braw[1];
    const bool more = kb + 1 < nkb;
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) areg[i] = *reinterpret_cast<const uint4*>(asrc[i] + (kb + 1) * KBLK);
      braw[0] = load_braw(bc[0], bs[0], kb + 1, half);
      braw[1] = load_braw(bc[1], bs[1], kb + 1, half);
    }
    const F16Scale sc00 = f16_scale(e4m3_f32<0>(cur0.s)), sc01 = f16_scale(e4m3_f32<1>(cur0.s));
    const F16Scale sc10 = f16_scale(e4m3_f32<0>(cur1.s)), sc11 = f16_scale(e4m3_f32<1>(cur1.s));
    const uint16_t* Ab = As[kb & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f16x8_t b0 = bfrag(word_of(cur0.c, s), s < 2 ? sc00 : sc01);
      const f16x8_t b1 = bfrag(word_of(cur1.c, s), s < 2 ? sc10 : sc11);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f16x8_t a =
            *reinterpret_cast<const f16x8_t*>(Ab + (rb * 32 + l32) * LDS_STRIDE + half * 32 + s * 8);
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc[rb][1], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&As[(kb + 1) & 1][(arow + 32 * i) * LDS_STRIDE + achunk * 8]) = areg[i];
    }
  }

  if (GATEUP) {
    const float gg = w0.global[e], gu = w1.global[e];
    const int jcol = nb * 128 + wave * 32 + l32;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        if (r < rows) {
          const float xs = s_coef[r];
          const float g = acc[rb][0][i] * xs * gg;
          const float u = acc[rb][1][i] * xs * gu;
          const float hv = silu(g) * u;
          const size_t o = (size_t)(base + m0 + r) * ldo + jcol;
          if (HOUT32) reinterpret_cast<float*>(out)[o] = hv;
          else reinterpret_cast<uint16_t*>(out)[o] = f32_to_f16_bits(hv);
        }
      }
  } else {
    const float gd = w0.global[e];
    float* o = reinterpret_cast<float*>(out);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = rb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        if (r < rows) {
          const float c = s_coef[r] * gd;
          float* orow = o + (size_t)s_tok[r] * ldo + nb * 256 + wave * 64 + l32;
          unsafeAtomicAdd(orow, acc[rb][0][i] * c);
          unsafeAtomicAdd(orow + 32, acc[rb][1][i] * c);
        }
      }
  }
}

static inline unsigned grid_for(int max_tiles, int NB) {
  const long long g = (long long)max_tiles * NB;
  return (unsigned)(((g + 7) / 8) * 8);
}

hipError_t launch_gemm_gateup(int act, const void* a, const float* a_scale, const int32_t* sorted_pairs,
                              const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                              int max_tiles, int topk, int H, int I, const WeightArgs& gate,
                              const WeightArgs& up, void* h, hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  const int NB = I / 128;
  const dim3 grid(grid_for(max_tiles, NB));
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a);
  if (act == 0)
    moe_gemm_f16_kernel<true, false, false><<<grid, 256, 0, st>>>(A, a_scale, sorted_pairs, offsets, tiles,
                                                                  tile_count, topk, H, NB, gate, up, nullptr, h, I);
  else
    moe_gemm_f16_kernel<true, true, true><<<grid, 256, 0, st>>>(A, a_scale, sorted_pairs, offsets, tiles,
                                                                tile_count, topk, H, NB, gate, up, nullptr, h, I);
  return hipGetLastError();
}

hipError_t launch_gemm_down(int act, const void* h, const float* h_scale, const int32_t* sorted_pairs,
                            const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                            int max_tiles, int topk, int H, int I, const WeightArgs& down, const float* w,
                            float* out_acc, hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  const int NB = H / 256;
  const dim3 grid(grid_for(max_tiles, NB));
  const uint16_t* A = reinterpret_cast<const uint16_t*>(h);
  if (act == 0)
    moe_gemm_f16_kernel<false, false, false><<<grid, 256, 0, st>>>(A, h_scale, sorted_pairs, offsets, tiles,
                                                                   tile_count, topk, I, NB, down, down, w,
                                                                   out_acc, H);
  else
    moe_gemm_f16_kernel<false, true, false><<<grid, 256, 0, st>>>(A, h_scale, sorted_pairs, offsets, tiles,
                                                                  tile_count, topk, I, NB, down, down, w,
                                                                  out_acc, H);
  return hipGetLastError();
}

}  // namespace nvfp4

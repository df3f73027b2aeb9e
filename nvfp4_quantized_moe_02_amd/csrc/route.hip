// Token-to-expert routing: a stable counting sort of the (token, slot) pairs by expert,
// in three launches (per-chunk histograms, one scan, per-chunk scatter). The result is
// deterministic and equals a stable sort by expert id: pairs of one expert keep their
// pair order p = t * topk + j. This replaces the pages' per-expert waits with one launch
// per stage for all experts ("Strata NVFP4" README, "How it differs from upstream
// Strata": an MMQ group's experts gathered in one launch after one wait).
#include "kernels.h"

namespace nvfp4 {

int route_blocks(int64_t P) { return (int)((P + kRouteChunk - 1) / kRouteChunk); }

// Blocks [0, nblk): expert histogram of one chunk of kRouteChunk pairs. Blocks after that
// (optional) stage the bf16 activations as fp16 for the prefill GEMMs, one wave per token
// row: the row is scaled by 2^e, e chosen so that its largest magnitude lands in
// [2^14, 2^15), so every bf16 value of the row above 2^-17 of that magnitude is exact in
// fp16 and nothing overflows, whatever the row's range; e goes to cvt_exp[row] and the
// gate/up epilogue multiplies by 2^-e (exact). Rows holding an infinity or a NaN, and
// all-zero rows, take e = 0. The routing grid is small, so the staging runs beside it in
// the same launch.
__device__ __forceinline__ int f16_stage_exponent(float absmax) {
  if (!(absmax > 0.f) || !(absmax <= 3.402823466e38f)) return 0;  // zero, inf or NaN
  return 15 - __builtin_amdgcn_frexp_expf(absmax);  // absmax in [2^(x-1), 2^x) -> [2^14, 2^15)
}

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                          int nblk, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ dropped,
                                                          const uint4* __restrict__ cvt_src,
                                                          uint4* __restrict__ cvt_dst, int32_t* __restrict__ cvt_exp,
                                                          int cvt_rows, int cvt_row8) {
  extern __shared__ int32_t hist[];
  __shared__ int32_t drop;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b >= nblk) {
    const int row = (b - nblk) * 4 + (tid >> 6), lane = tid & 63;
    if (row >= cvt_rows) return;
    const uint4* src = cvt_src + (size_t)row * cvt_row8;
    float m = 0.f;
    for (int i = lane; i < cvt_row8; i += 64) {
      const uint4 v = src[i];
      const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(bf16_lo(in[j])), fabsf(bf16_hi(in[j]))));
    }
    const int e = f16_stage_exponent(wave_max(m));
    uint4* dst = cvt_dst + (size_t)row * cvt_row8;
    for (int i = lane; i < cvt_row8; i += 64) {
      const uint4 v = src[i];
      const uint32_t in[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = (uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(bf16_lo(in[j]), e)) |
               ((uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(bf16_hi(in[j]), e)) << 16);
      dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (lane == 0) cvt_exp[row] = e;
    return;
  }
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  if (tid == 0) drop = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)b * kRouteChunk;
  const int64_t p1 = p0 + kRouteChunk < P ? p0 + kRouteChunk : P;
  int mydrop = 0;
  for (int64_t p = p0 + tid; p < p1; p += 256) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    else ++mydrop;
  }
  if (mydrop) atomicAdd(&drop, mydrop);
  __syncthreads();
  for (int e = tid; e < E; e += 256) counts[(size_t)e * nblk + b] = hist[e];
  if (tid == 0) dropped[b] = drop;
}

// Exclusive block scan of one int per thread (1024 threads); returns the exclusive
// prefix and writes the total to *total.
__device__ int block_scan_1024(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[1023];
  __syncthreads();
  return incl - v;
}

// One wave per expert: that expert's chunk counts (contiguous, e-major) -> exclusive
// prefix in place (the expert-local base of each chunk), and the expert's total into
// totals[e].
__global__ __launch_bounds__(256) void route_expert_scan_kernel(int E, int nblk, int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  int32_t* c = counts + (size_t)e * nblk;
  int run = 0;
  for (int b0 = 0; b0 < nblk; b0 += 64) {
    const int b = b0 + lane;
    const int v = b < nblk ? c[b] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off, 64);
      if (lane >= off) incl += u;
    }
    if (b < nblk) c[b] = run + incl - v;
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) totals[e] = run;
}

// One block of 1024 threads: expert totals (in offsets[0..E); all zero when there are no
// chunks) -> exclusive offsets in place and offsets[E]; the dropped total; -1 padding of
// sorted_pairs; the tile list.
__global__ __launch_bounds__(1024) void route_scan_kernel(int E, int nblk, int64_t P, const int32_t* __restrict__ dropped,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ hdr, TileDesc* __restrict__ tiles,
                                                          int tile_m) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  const int start = tid * per < E ? tid * per : E;
  const int end = start + per < E ? start + per : E;
  int local = 0;
  for (int i = start; i < end; ++i) local += nblk ? offsets[i] : 0;
  int total;
  int run = block_scan_1024(local, sh, &total);
  int my = 0;  // tiles of tile_m rows per expert, in expert order
  for (int i = start; i < end; ++i) {
    const int c = nblk ? offsets[i] : 0;
    offsets[i] = run;
    run += c;
    my += (c + tile_m - 1) / tile_m;
  }
  int d = 0;
  for (int b = tid; b < nblk; b += 1024) d += dropped[b];
  int dtotal;
  block_scan_1024(d, sh, &dtotal);
  if (tid == 0) {
    offsets[E] = total;
    hdr[0] = dtotal;
  }
  for (int64_t i = total + tid; i < P; i += 1024) sorted_pairs[i] = -1;
  if (tiles == nullptr) return;
  int ntiles;
  int base = block_scan_1024(my, sh, &ntiles);
  __syncthreads();  // offsets of this thread's range are final (written above by this thread)
  for (int i = start; i < end; ++i) {
    const int cnt = (i + 1 < end ? offsets[i + 1] : run) - offsets[i];
    for (int m0 = 0; m0 < cnt; m0 += tile_m) tiles[base++] = TileDesc{i, m0};
  }
  if (tid == 0) hdr[1] = ntiles;
}

// One block of 4 waves per chunk, 256 pairs per round. Within a wave, lanes holding the
// same expert are ranked in lane order (a match built from ballots over the id bits); the
// four waves of a round then take their positions from the running per-expert position in
// wave order, one wave per barrier-separated phase, so the scatter is stable.
__global__ __launch_bounds__(256) void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                            int nblk, const int32_t* __restrict__ bases,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pairs,
                                                            int32_t* __restrict__ inv) {
  extern __shared__ int32_t run[];  // [E] next sorted position per expert
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) run[e] = offsets[e] + bases[(size_t)e * nblk + b];
  __syncthreads();
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const int64_t p0 = (int64_t)b * kRouteChunk;
  const int64_t p1 = p0 + kRouteChunk < P ? p0 + kRouteChunk : P;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int64_t base = p0; base < p1; base += 256) {
    const int64_t p = base + tid;
    const int e = p < p1 ? ids[p] : -1;
    const bool valid = p < p1 && (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const uint64_t bb = __ballot(set);
      m &= set ? bb : ~bb;
    }
    int pos = -1;
    for (int w = 0; w < 4; ++w) {
      if (wave == w && valid) {
        pos = run[e] + __popcll(m & lt);
        if ((m >> lane) == 1ull) run[e] = pos + 1;  // highest lane of its expert
      }
      __syncthreads();
    }
    if (valid) sorted_pairs[pos] = (int32_t)p;
    if (inv != nullptr && p < p1) inv[p] = pos;  // sorted position of pair p, -1 if dropped
  }
}

hipError_t launch_route(const int32_t* ids, int64_t P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const RouteWs& ws, int tile_m, hipStream_t st, const void* cvt_src, void* cvt_dst,
                        int32_t* cvt_exp, int cvt_rows, int cvt_cols) {
  const int nblk = route_blocks(P);
  const int rows = cvt_src != nullptr ? cvt_rows : 0;
  const int64_t cvt_blocks = (rows + 3) / 4;
  if (nblk + cvt_blocks > 0) {
    route_count_kernel<<<dim3((unsigned)(nblk + cvt_blocks)), 256, (size_t)E * sizeof(int32_t), st>>>(
        ids, P, E, nblk, ws.counts, ws.dropped, reinterpret_cast<const uint4*>(cvt_src),
        reinterpret_cast<uint4*>(cvt_dst), cvt_exp, rows, cvt_cols / 8);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nblk > 0) {
    route_expert_scan_kernel<<<dim3((unsigned)((E + 3) / 4)), 256, 0, st>>>(E, nblk, ws.counts, offsets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  route_scan_kernel<<<1, 1024, 0, st>>>(E, nblk, P, ws.dropped, offsets, sorted_pairs, ws.hdr, ws.tiles, tile_m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nblk > 0) {
    route_scatter_kernel<<<nblk, 256, (size_t)E * sizeof(int32_t), st>>>(ids, P, E, nblk, ws.counts, offsets,
                                                                        sorted_pairs, ws.inv);
    e = hipGetLastError();
  }
  return e;
}

// Routing of a layer with a shared expert, as one more slot of every token: ids2 [T][k+1]
// holds the token's k routed ids (those outside [0, E) as -1, so they stay dropped when E + 1
// experts are routed) and then E, the shared expert's index; w2 the router weights and 1.
__global__ __launch_bounds__(256) void append_shared_kernel(const int32_t* __restrict__ ids,
                                                            const float* __restrict__ w, int64_t T, int k, int E,
                                                            int32_t* __restrict__ ids2, float* __restrict__ w2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * (k + 1)) return;
  const int64_t t = i / (k + 1);
  const int j = (int)(i - t * (k + 1));
  if (j < k) {
    const int e = ids[t * k + j];
    ids2[i] = (unsigned)e < (unsigned)E ? e : -1;
    w2[i] = w[t * k + j];
  } else {
    ids2[i] = E;
    w2[i] = 1.0f;
  }
}

hipError_t launch_append_shared(const int32_t* ids, const float* w, int64_t T, int k, int E, int32_t* ids2,
                                float* w2, hipStream_t st) {
  const int64_t n = T * (k + 1);
  if (n == 0) return hipSuccess;
  append_shared_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(ids, w, T, k, E, ids2, w2);
  return hipGetLastError();
}

}  // namespace nvfp4

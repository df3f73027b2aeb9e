// Token-to-expert routing: a stable counting sort of the (token, slot) pairs by expert,
// in three launches (per-chunk histograms, one scan, per-chunk scatter). The result is
// deterministic and equals a stable sort by expert id: pairs of one expert keep their
// pair order p = t * topk + j. This replaces the pages' per-expert waits with one launch
// per stage for all experts ("Strata NVFP4" README, "How it differs from upstream
// Strata": an MMQ group's experts gathered in one launch after one wait).
#include "kernels.h"

namespace nvfp4 {

int route_blocks(int64_t P) { return (int)((P + kRouteChunk - 1) / kRouteChunk); }

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                          int nblk, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ dropped) {
  extern __shared__ int32_t hist[];
  __shared__ int32_t drop;
  const int b = blockIdx.x, tid = threadIdx.x;
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

// One block of 1024 threads: counts (e-major, chunk-minor) -> bases in place, expert
// offsets, the dropped total, -1 padding of sorted_pairs, and the tile list.
__global__ __launch_bounds__(1024) void route_scan_kernel(int E, int nblk, int64_t P, int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ dropped,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ hdr, TileDesc* __restrict__ tiles,
                                                          int tile_m) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  const int n = E * nblk;
  const int per = (n + 1023) / 1024;
  const int start = tid * per < n ? tid * per : n;
  const int end = start + per < n ? start + per : n;
  int local = 0;
  for (int i = start; i < end; ++i) local += counts[i];
  int total;
  int run = block_scan_1024(local, sh, &total);
  for (int i = start; i < end; ++i) {
    const int c = counts[i];
    counts[i] = run;
    run += c;
  }
  int d = 0;
  for (int b = tid; b < nblk; b += 1024) d += dropped[b];
  int dtotal;
  block_scan_1024(d, sh, &dtotal);
  __syncthreads();
  for (int e = tid; e < E; e += 1024) offsets[e] = nblk ? counts[(size_t)e * nblk] : 0;
  if (tid == 0) {
    offsets[E] = total;
    hdr[0] = dtotal;
  }
  for (int64_t i = total + tid; i < P; i += 1024) sorted_pairs[i] = -1;
  if (tiles == nullptr) return;
  __syncthreads();
  // tiles of tile_m rows per expert, in expert order
  int my = 0;
  for (int e = tid; e < E; e += 1024) {
    const int cnt = ((e + 1 < E) ? offsets[e + 1] : total) - offsets[e];
    my += (cnt + tile_m - 1) / tile_m;
  }
  int ntiles;
  int base = block_scan_1024(my, sh, &ntiles);
  for (int e = tid; e < E; e += 1024) {
    const int cnt = ((e + 1 < E) ? offsets[e + 1] : total) - offsets[e];
    for (int m0 = 0; m0 < cnt; m0 += tile_m) tiles[base++] = TileDesc{e, m0};
  }
  if (tid == 0) hdr[1] = ntiles;
}

// One wave per chunk: walks its pairs in order, 64 at a time; lanes holding the same
// expert get consecutive slots in lane order (a match built from ballots over the id
// bits), so the scatter is stable.
__global__ __launch_bounds__(64) void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                           int nblk, const int32_t* __restrict__ bases,
                                                           int32_t* __restrict__ sorted_pairs,
                                                           int32_t* __restrict__ inv) {
  extern __shared__ int32_t run[];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = bases[(size_t)e * nblk + b];
  __syncthreads();
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const int64_t p0 = (int64_t)b * kRouteChunk;
  const int64_t p1 = p0 + kRouteChunk < P ? p0 + kRouteChunk : P;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int64_t base = p0; base < p1; base += 64) {
    const int64_t p = base + lane;
    const int e = p < p1 ? ids[p] : -1;
    const bool valid = p < p1 && (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = valid && ((e >> bit) & 1);
      const uint64_t bb = __ballot(set);
      m &= set ? bb : ~bb;
    }
    int pos = 0;
    if (valid) pos = run[e] + __popcll(m & lt);
    __syncthreads();
    if (valid) {
      sorted_pairs[pos] = (int32_t)p;
      if ((m >> lane) == 1ull) run[e] += __popcll(m);
    }
    if (inv != nullptr && p < p1) inv[p] = valid ? pos : -1;  // sorted position of pair p
    __syncthreads();
  }
}

hipError_t launch_route(const int32_t* ids, int64_t P, int E, int32_t* offsets, int32_t* sorted_pairs,
                        const RouteWs& ws, int tile_m, hipStream_t st) {
  const int nblk = route_blocks(P);
  const size_t lds = (size_t)E * sizeof(int32_t);
  if (nblk > 0) {
    route_count_kernel<<<nblk, 256, lds, st>>>(ids, P, E, nblk, ws.counts, ws.dropped);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  route_scan_kernel<<<1, 1024, 0, st>>>(E, nblk, P, ws.counts, ws.dropped, offsets, sorted_pairs, ws.hdr,
                                        ws.tiles, tile_m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nblk > 0) {
    route_scatter_kernel<<<nblk, 64, lds, st>>>(ids, P, E, nblk, ws.counts, sorted_pairs, ws.inv);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace nvfp4

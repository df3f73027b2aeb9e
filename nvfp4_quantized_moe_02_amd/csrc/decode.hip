// Decode path (1..8 tokens): HBM-bound NVFP4 GEMVs with FP32 arithmetic, the pages'
// quality profile for expert decode ("#1858 strata-safetensors": canonical FP32 expert
// decode). A decode round is dominated by the expert bytes it moves ("Strata NVFP4"
// README, "Limits"), so the whole layer runs as ONE persistent launch:
//
//   setup    every block derives the unique-expert list from topk_ids and copies the
//            bf16 activations into LDS.
//   phase 1  gate/up + SwiGLU: units of (unique expert, 4 intermediate rows) are spread
//            over all waves of the grid; h (fp32) goes to the workspace.
//   barrier  one arrival per block on an agent-scope counter; the last arrival writes
//            every block's release flag, each block polls its own (bounded spin).
//   phase 2  down + top-k combine: block b owns output rows 8b .. 8b+7; every block
//            copies h into LDS once; each wave covers all 8 rows (8 lanes per row) for
//            the unique experts w, w+8, ..., sums its experts' pairs in a fixed order, and
//            the 8 waves' partials are added in wave order, so the result is
//            deterministic. Each wave issues the loads of its first down weights as soon
//            as its block has arrived at the barrier, so that traffic overlaps the wait
//            and the h copy while phase 1 has the memory system to itself.
//
// The same device code also runs as two ordinary launches (phase 1, then phase 2) for
// the staged entry point and for shapes whose grid cannot be co-resident or whose h does
// not fit in LDS (the launch boundary then makes h visible); both forms
// give bit-identical results. Both derive the unique-expert list from topk_ids
// themselves (no host synchronization).
//
// Lane mapping: gate/up rows take 16 lanes each, down rows 8 (I = 768 has 24 input chunks:
// 3 per lane with 8 lanes, where 16 lanes left a quarter of the lanes' second chunk empty;
// measured 7% faster at 4 tokens, 3% at 1). Each lane reads 16-byte chunks (32 inputs =
// two scale groups) with 128-bit loads, so one load instruction reads 4 rows x 256 (or 8
// rows x 128) contiguous bytes. A Q8_0 down projection (template parameter Q8) keeps the
// mapping with 32-byte chunks (32 int8 weights, one fp16 scale).
#include "kernels.h"

namespace nvfp4 {

constexpr int kDecWaves = 8;     // waves per block
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kRowsPerBlock = kDecodeRowsPerBlock;  // output rows per block in phase 2
// down experts a wave loads at once (8 rows each): 3, or 2 for Q8_0's twice-as-wide rows
template <bool Q8>
constexpr int kUBof = Q8 ? 2 : 3;
constexpr int kDownLanes = 8;     // lanes per down row in phase 2 (a wave covers the block's 8 rows)
constexpr int kCopyBatch = 8;     // 16-byte loads in flight per thread when copying h into LDS

struct DecodeSmem {
  int ids[64];    // each pair's expert id, or -1 when dropped
  int uniq[64];   // unique experts in ascending id order
  int list[64];   // pairs grouped by unique expert, each group in pair order
  int start[65];  // group boundaries in list
  float wp[64];   // router weight of each pair
  int nu, drop, ok, last, spin;
  unsigned long long epoch;
  float part[kDecWaves][kRowsPerBlock][kDecodeMaxT];
};

// Dynamic LDS: x (bf16, T x H) then, when it fits, h (fp32, P x I). Both are stored in
// 16-byte-padded chunks (x: 64 B of data per 80 B, h: 128 B per 144 B), so the lanes of a
// row group, which read consecutive chunks (16 of x, 8 of h at a time), hit distinct banks.
extern __shared__ __attribute__((aligned(16))) char dec_lds[];

__host__ __device__ inline size_t x_lds_bytes(int T, int H) { return (size_t)T * (H / 32) * 80; }
__host__ __device__ inline size_t h_lds_bytes(int P, int I) { return (size_t)P * (I / 32) * 144; }
__device__ inline const uint4* x_lds_chunk(int t, int H, int ch) {
  return reinterpret_cast<const uint4*>(dec_lds + (size_t)t * (H / 32) * 80 + ch * 80);
}
__device__ inline const float* h_lds_chunk(int H_T_bytes, int p, int I, int ch) {
  return reinterpret_cast<const float*>(dec_lds + H_T_bytes + (size_t)p * (I / 32) * 144 + ch * 144);
}

struct DecodeArgs {
  const uint16_t* x;
  int T, H, I, E, P, topk;
  WeightArgs gate, up, down;
  const int32_t* ids;
  const float* w;
  float* h;
  void* out;
  int out_dtype;
  int32_t* hdr;                  // [0] dropped pairs, [1] error flags, [2] spin-limit override
  unsigned* barrier;             // grid barrier arrival counter (zero between calls)
  unsigned long long* epoch;     // grid barrier epoch (grows by one per fused call)
  unsigned long long* flags;     // grid barrier release flags, one 128-byte line per block
  int spin_limit;
  int h_in_lds;                  // phase 2 reads h from LDS (P * I * 4 bytes fit)
};



// Sum over each group of 8 lanes (quad swaps, then the half-row mirror), in every lane.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  return v;
}

// s_waitcnt immediate: no vector-memory operation of this wave outstanding.
constexpr int kVmcnt0 = (7 << 4) | (0xF << 8);

// Setup, called by every thread of the block (it holds barriers). The loads of the
// routing ids, the router weights and the activations are issued together; wave 0 then
// forms the unique-expert list (ascending ids) and the pair list of each unique expert
// with one ballot per id bit.
__device__ void decode_prepare(DecodeSmem& sm, const DecodeArgs& a, bool copy_x) {
  const int tid = threadIdx.x;
  int e = -1;
  float wv = 0.f;
  if (tid < 64 && tid < a.P) {
    if (a.gate.xe >= 0) {
      // a shared expert (index xe) is slot topk - 1 of every token, weight 1; the caller's
      // ids and weights are [T][topk - 1], and their ids outside [0, xe) are dropped
      const int kk = a.topk - 1, t = tid / a.topk, j = tid - t * a.topk;
      if (j < kk) {
        e = a.ids[t * kk + j];
        wv = a.w[t * kk + j];
        if ((unsigned)e >= (unsigned)a.gate.xe) e = -1;
      } else {
        e = a.gate.xe;
        wv = 1.0f;
      }
    } else {
      e = a.ids[tid];
      wv = a.w[tid];
    }
  }
  if (copy_x) {
    const int n16 = a.T * a.H / 8;  // 16-byte pieces, 4 per 32-input chunk
    const uint4* xs = reinterpret_cast<const uint4*>(a.x);
    for (int i = tid; i < n16; i += kDecThreads)
      *reinterpret_cast<uint4*>(dec_lds + (i >> 2) * 80 + (i & 3) * 16) = xs[i];
  }
  if (tid < 64) {
    const bool valid = tid < a.P && (unsigned)e < (unsigned)a.E;
    const int ev = valid ? e : -1;
    sm.ids[tid] = ev;
    sm.wp[tid] = wv;
    // Group the pairs by expert, experts in ascending id order, pairs in pair order, with
    // no loop over the experts: from the top bit of the id down, one ballot per bit
    // narrows each lane's mask of lanes with the same id and collects the lanes with a
    // smaller id. A pair's list position is the count of smaller-id pairs plus its rank
    // among its expert's pairs; the lowest lane of an expert writes the group entry.
    const uint64_t lt = (1ull << tid) - 1ull;
    const uint64_t vm = __ballot(valid);
    const uint64_t dm = __ballot(tid < a.P && !valid);
    uint64_t less = 0ull, same = valid ? vm : 0ull;
    // One token: its valid slots are taken in slot order, each as its own group (an
    // expert named twice is read twice); this skips the ballots, the slowest part of the
    // set-up at one token.
    const int nbits = a.T == 1 ? 0 : 32 - __builtin_clz((unsigned)(a.E > 1 ? a.E - 1 : 1));
    if (a.T == 1) {
      same = valid ? (1ull << tid) : 0ull;
      less = vm & lt;
    }
    for (int b = nbits - 1; b >= 0; --b) {
      const bool bit = (ev >> b) & 1;
      const uint64_t mb = __ballot(bit);
      less |= bit ? (same & ~mb) : 0ull;
      same &= bit ? mb : ~mb;
    }
    const bool first = valid && (same & lt) == 0ull;
    const uint64_t fm = __ballot(first);
    if (valid) sm.list[__popcll(less) + __popcll(same & lt)] = tid;
    if (first) {
      const int g = __popcll(fm & less);  // distinct smaller ids
      sm.uniq[g] = ev;
      sm.start[g] = __popcll(less);
    }
    if (tid == 0) {
      const int nu = __popcll(fm);
      sm.start[nu] = __popcll(vm);
      sm.nu = nu;
      sm.drop = __popcll(dm);
      // grid-barrier spin limit: the workspace header's override word when nonzero
      // (negative: no polling, every waiting block gives up at once)
      const int ov = a.hdr[2];
      sm.spin = ov > 0 ? ov : ov < 0 ? 0 : a.spin_limit;
      // the barrier epoch of this call (read before this block arrives at the barrier)
      sm.epoch = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
}

// One 16-byte chunk (32 inputs, two scale groups) of a weight row dotted with bf16
// activations held as 16 packed pairs; returns the scaled partial sum.
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

// One 16-byte chunk of a down row dotted with 32 fp32 h values.
__device__ __forceinline__ float dot_chunk_f32(const uint4 c, uint32_t sc, const float* __restrict__ hp) {
  const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
  const float4* h4 = reinterpret_cast<const float4*>(hp);
  float g2[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 ha = h4[2 * q], hb = h4[2 * q + 1];
    const f32x2_t w0 = e2m1x2_f32<0>(wd[q]), w1 = e2m1x2_f32<1>(wd[q]);
    const f32x2_t w2 = e2m1x2_f32<2>(wd[q]), w3 = e2m1x2_f32<3>(wd[q]);
    float s = g2[q >> 1];
    s = fmaf(w0[0], ha.x, s); s = fmaf(w0[1], ha.y, s);
    s = fmaf(w1[0], ha.z, s); s = fmaf(w1[1], ha.w, s);
    s = fmaf(w2[0], hb.x, s); s = fmaf(w2[1], hb.y, s);
    s = fmaf(w3[0], hb.z, s); s = fmaf(w3[1], hb.w, s);
    g2[q >> 1] = s;
  }
  return g2[0] * e4m3_f32<0>(sc) + g2[1] * e4m3_f32<1>(sc);
}

// One Q8_0 block (32 int8 weights in two 16-byte words, fp16 scale bits in `sc`) dotted
// with 32 fp32 h values: FP32 products and sums, the scale applied once per block.
__device__ __forceinline__ float dot_chunk_q8(const uint4 c0, const uint4 c1, uint32_t sc,
                                              const float* __restrict__ hp) {
  const uint32_t wd[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float4* h4 = reinterpret_cast<const float4*>(hp);
  float g2[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 hv = h4[q];
    const int32_t w = (int32_t)wd[q];
    float s = g2[q & 1];
    s = fmaf((float)((w << 24) >> 24), hv.x, s);
    s = fmaf((float)((w << 16) >> 24), hv.y, s);
    s = fmaf((float)((w << 8) >> 24), hv.z, s);
    s = fmaf((float)(w >> 24), hv.w, s);
    g2[q & 1] = s;
  }
  return (g2[0] + g2[1]) * (float)__builtin_bit_cast(_Float16, (uint16_t)sc);
}

// ---- phase 1: a unit is (unique expert slot u, intermediate rows 4q .. 4q+3)
template <int CH>
struct GateUpRows {
  uint4 gc[CH], uc[CH];
  uint32_t gs[CH], us[CH];
  float gg, gu;  // the expert's global scales, loaded with its rows
};

// X: the call has a separately stored (shared) expert, index a.gate.xe
template <int CH, bool X>
__device__ __forceinline__ void gateup_load(const DecodeArgs& a, int e_in, int row, int l16, GateUpRows<CH>& r) {
  const int nch = a.H >> 5;
  // the unit's expert is the same for the whole wave: with a shared expert, keep it (and
  // the selected weight bases) scalar
  const int e = X ? __builtin_amdgcn_readfirstlane(e_in) : e_in;
  const uint8_t* gc = a.gate.code_row<X>(e, row, a.H / 2);
  const uint8_t* uc = a.up.code_row<X>(e, row, a.H / 2);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(a.gate.scale_row<X>(e, row));
  const uint16_t* us = reinterpret_cast<const uint16_t*>(a.up.scale_row<X>(e, row));
  r.gg = a.gate.gamma_nvfp4<X>(e);
  r.gu = a.up.gamma_nvfp4<X>(e);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = l16 + 16 * c;
    if (ch < nch) {
      r.gc[c] = *reinterpret_cast<const uint4*>(gc + ch * 16);
      r.uc[c] = *reinterpret_cast<const uint4*>(uc + ch * 16);
      r.gs[c] = gs[ch];
      r.us[c] = us[ch];
    }
  }
}

template <int CH>
__device__ __forceinline__ void gateup_compute(const DecodeArgs& a, const DecodeSmem& sm, int u, int row, int l16,
                                               const GateUpRows<CH>& r) {
  const int nch = a.H >> 5;
  const float gg = r.gg, gu = r.gu;
  for (int i = sm.start[u]; i < sm.start[u + 1]; ++i) {
    const int p = sm.list[i];
    const int t = p / a.topk;
    float ga = 0.f, ua = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = l16 + 16 * c;
      if (ch < nch) {
        uint32_t xv[16];
        const uint4* xr = x_lds_chunk(t, a.H, ch);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = xr[q];
          xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
        }
        ga += dot_chunk_bf16(r.gc[c], r.gs[c], xv);
        ua += dot_chunk_bf16(r.uc[c], r.us[c], xv);
      }
    }
    ga = sum16(ga);
    ua = sum16(ua);
    // h goes to memory with an agent-coherent (write-through) store: blocks on other
    // XCDs read it after the grid barrier without any L2 writeback or invalidation.
    if (l16 == 0)
      __hip_atomic_store(a.h + (size_t)p * a.I + row, silu(ga * gg) * (ua * gu), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// All waves of the grid share the phase-1 units, two at a time per wave. The loads of
// the first two units are issued by the caller (before the gamma loads and the barrier
// that publishes them).
template <int CH>
struct Phase1 {
  GateUpRows<CH> r0, r1;
  int j;
};

template <int CH, bool X>
__device__ __forceinline__ void phase1_issue(const DecodeArgs& a, const DecodeSmem& sm, int j, Phase1<CH>& st) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, rq = lane >> 4;
  const int quads = a.I >> 2;
  const int units = sm.nu * quads;
  const int nw = gridDim.x * kDecWaves;
  st.j = j;
  if (j < units) {
    const int u0 = j / quads;
    gateup_load<CH, X>(a, sm.uniq[u0], (j - u0 * quads) * 4 + rq, l16, st.r0);
  }
  if (j + nw < units) {
    const int u1 = (j + nw) / quads;
    gateup_load<CH, X>(a, sm.uniq[u1], (j + nw - u1 * quads) * 4 + rq, l16, st.r1);
  }
}

template <int CH, bool X>
__device__ void phase1(const DecodeArgs& a, const DecodeSmem& sm, Phase1<CH>& st) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, rq = lane >> 4;
  const int quads = a.I >> 2;
  const int units = sm.nu * quads;
  const int nw = gridDim.x * kDecWaves;
  for (int j = st.j; j < units; j += 2 * nw) {
    if (j != st.j) phase1_issue<CH, X>(a, sm, j, st);
    const int u0 = j / quads;
    gateup_compute<CH>(a, sm, u0, (j - u0 * quads) * 4 + rq, l16, st.r0);
    if (j + nw < units) {
      const int u1 = (j + nw) / quads;
      gateup_compute<CH>(a, sm, u1, (j + nw - u1 * quads) * 4 + rq, l16, st.r1);
    }
  }
}

// ---- phase 2: wave w covers the block's 8 rows (8 lanes per row) for the unique experts
// w + 8i.
template <int CH, bool Q8>
struct DownRows {
  static constexpr int kUB = kUBof<Q8>;
  uint4 c[kUB][CH][Q8 ? 2 : 1];  // NVFP4: 16 bytes (32 inputs); Q8_0: 32 bytes
  uint32_t s[kUB][CH];           // NVFP4: two E4M3 bytes; Q8_0: fp16 bits
  float gd[kUB];  // global scales of the experts, loaded with their rows
  // the experts' pairs: list positions [ps, pe); the first pair and its router weight are
  // read here, ahead of the h exchange, so phase 2 starts without an LDS round trip
  int ps[kUB], pe[kUB], p0[kUB];
  float w0[kUB];
};

__device__ __forceinline__ int down_expert(int wave, int ub) { return wave + kDecWaves * ub; }

// Loads the weight chunks of this wave's experts ub0 .. ub0+kUB-1 for output row `row`;
// experts beyond the unique list get an empty pair range and rows beyond H zero codes,
// scales and global scale (they add exactly 0).
template <int CH, bool Q8, bool X>
__device__ __forceinline__ void down_load(const DecodeArgs& a, const DecodeSmem& sm, int ub0, int row, int l16,
                                          DownRows<CH, Q8>& d) {
  const int wave = threadIdx.x >> 6;
  const int nch = a.I >> 5;
#pragma unroll
  for (int b = 0; b < kUBof<Q8>; ++b) {
    const int u = down_expert(wave, ub0 + b);
    const bool have = u < sm.nu;
    d.ps[b] = have ? sm.start[u] : 0;
    d.pe[b] = have ? sm.start[u + 1] : 0;
    d.p0[b] = have ? sm.list[d.ps[b]] : 0;
    d.w0[b] = have ? sm.wp[d.p0[b]] : 0.f;
    const bool ok = have && row < a.H;
    d.gd[b] = ok ? a.down.gamma<X>(X ? __builtin_amdgcn_readfirstlane(sm.uniq[u]) : sm.uniq[u]) : 0.f;
    // per row: NVFP4 I/2 code bytes and I/16 scale bytes; Q8_0 I code bytes and I/32 fp16
    const int ue = ok ? sm.uniq[u] : 0;
    const size_t rr = ok ? (size_t)row : 0;
    const int uex = X ? __builtin_amdgcn_readfirstlane(have ? sm.uniq[u] : 0) : ue;  // one expert per wave and b
    const uint8_t* rc = a.down.code_row<X>(uex, rr, Q8 ? a.I : a.I / 2);
    const uint16_t* rs = reinterpret_cast<const uint16_t*>(a.down.scale_row<X>(uex, rr));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = l16 + kDownLanes * c;
      const bool ld = ok && ch < nch;
#pragma unroll
      for (int v = 0; v < (Q8 ? 2 : 1); ++v)
        d.c[b][c][v] = ld ? *reinterpret_cast<const uint4*>(rc + ch * (Q8 ? 32 : 16) + 16 * v) : make_uint4(0, 0, 0, 0);
      d.s[b][c] = ld ? (uint32_t)rs[ch] : 0u;
    }
  }
}

// One pair's partial dot products for this lane's chunks: all h reads are issued before
// the arithmetic (chunks past I read chunk 0 and meet zero weights).
template <int CH, bool Q8, bool HLDS>
__device__ __forceinline__ float down_pair(const DecodeArgs& a, const DownRows<CH, Q8>& d, int b, int p, int l16,
                                           int xb) {
  const int nch = a.I >> 5;
  float part = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = l16 + kDownLanes * c < nch ? l16 + kDownLanes * c : 0;
    const float* hp = HLDS ? h_lds_chunk(xb, p, a.I, ch) : a.h + (size_t)p * a.I + ch * 32;
    if constexpr (Q8)
      part += dot_chunk_q8(d.c[b][c][0], d.c[b][c][1], d.s[b][c], hp);
    else
      part += dot_chunk_f32(d.c[b][c][0], d.s[b][c], hp);
  }
  return part;
}

template <int CH, bool Q8, bool HLDS>
__device__ __forceinline__ void down_accum(const DecodeArgs& a, const DecodeSmem& sm, const DownRows<CH, Q8>& d,
                                           int l16, float (&acc)[kDecodeMaxT]) {
  const int xb = (int)x_lds_bytes(a.T, a.H);
#pragma unroll
  for (int b = 0; b < kUBof<Q8>; ++b) {
    if (d.ps[b] >= d.pe[b]) break;  // uniform: this wave has no expert b (nor later ones)
    {
      const int p = d.p0[b];
      const float part = down_pair<CH, Q8, HLDS>(a, d, b, p, l16, xb);
      const int t = p / a.topk;
      const float coef = d.w0[b] * d.gd[b];
#pragma unroll
      for (int tt = 0; tt < kDecodeMaxT; ++tt)
        if (tt == t) acc[tt] = fmaf(coef, part, acc[tt]);
    }
    for (int i = d.ps[b] + 1; i < d.pe[b]; ++i) {
      const int p = sm.list[i];
      const float part = down_pair<CH, Q8, HLDS>(a, d, b, p, l16, xb);
      const int t = p / a.topk;
      const float coef = sm.wp[p] * d.gd[b];
#pragma unroll
      for (int tt = 0; tt < kDecodeMaxT; ++tt)
        if (tt == t) acc[tt] = fmaf(coef, part, acc[tt]);
    }
    // one expert's h reads in flight at a time (keeps the register count down)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Grid barrier over gridDim.x co-resident blocks. h was stored write-through (agent
// scope), so arrival only needs every wave's stores complete (vmcnt 0) before one
// relaxed atomic per block on the arrival counter. Every block read the call's epoch
// before arriving; the block whose arrival completes the count (it has seen every other
// arrival) writes epoch + 1 into every block's flag (one 128-byte line each, so the
// waiting blocks poll different lines instead of one), resets the counter to zero and
// stores epoch + 1 as the next call's epoch. A block waits until its flag reaches
// epoch + 1. So every call starts with a zero counter whatever the previous call's grid
// size was, and stale flags (at most the previous epoch) never release a wait. Readers
// then load h with agent-coherent loads. The arrival and the wait are two calls, so a block
// can issue loads in between.
__device__ void barrier_arrive(const DecodeArgs& a, DecodeSmem& sm) {
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.barrier, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = old + 1 == gridDim.x;
    sm.ok = 1;
  }
  __syncthreads();
  if (sm.last) {
    const unsigned long long target = sm.epoch + 1;
    for (unsigned b = threadIdx.x; b < gridDim.x; b += kDecThreads)
      __hip_atomic_store(a.flags + (size_t)b * 16, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
      __hip_atomic_store(a.barrier, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.epoch, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The wait half of the barrier (the last arriver does not wait). Returns false (and sets
// bit 0 of hdr[1]) if the wait exceeds the spin limit, so every wave exits.
__device__ bool barrier_wait(const DecodeArgs& a, DecodeSmem& sm) {
  if (sm.last) return true;
  const unsigned long long target = sm.epoch + 1;
  if (threadIdx.x == 0) {
    const unsigned long long* f = a.flags + (size_t)blockIdx.x * 16;
    int n = 0;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++n > sm.spin) {
        sm.ok = 0;
        __hip_atomic_fetch_or(a.hdr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  return sm.ok != 0;
}

// MODE 0: phase 1 only; MODE 1: phase 2 only; MODE 2: both with the grid barrier.
// Q8: the down projection is Q8_0. X: one expert (the shared one) is stored apart.
template <int MODE, int CHG, int CHD, bool Q8, bool X>
__global__ __launch_bounds__(kDecThreads, 1) void decode_kernel(DecodeArgs a) {
  __shared__ DecodeSmem sm;
  decode_prepare(sm, a, MODE != 1);
  if (blockIdx.x == 0 && threadIdx.x == 0 && MODE != 1) a.hdr[0] = sm.drop;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l8 = lane & (kDownLanes - 1);
  const int row = blockIdx.x * kRowsPerBlock + lane / kDownLanes;  // phase 2: every wave, all 8 rows
  Phase1<CHG> p1;
  // First unit of this wave: at one token block-major (a block's waves take 32 adjacent
  // rows of one expert), else wave-major (unit j on wave j / grid of block j % grid), which
  // spreads the units beyond the first round over all blocks (measured: 1 token 13.8 us
  // block-major vs 14.6 wave-major; 4 tokens 29.8 vs 28.9).
  const int j0 = a.T == 1 ? (int)blockIdx.x * kDecWaves + wave : wave * (int)gridDim.x + (int)blockIdx.x;
  if (MODE != 1) phase1_issue<CHG, X>(a, sm, j0, p1);
  DownRows<CHD, Q8> d;
  if (MODE == 1) down_load<CHD, Q8, X>(a, sm, 0, row, l8, d);
  if (MODE != 1) phase1<CHG, X>(a, sm, p1);
  if (MODE == 0) return;
  // The fused form issues its first down-weight loads once it has arrived at the grid
  // barrier: they then overlap the wait instead of sharing the memory system with the
  // gate/up loads of phase 1.
  if (MODE == 2) barrier_arrive(a, sm);
  if (MODE == 2) down_load<CHD, Q8, X>(a, sm, 0, row, l8, d);
  if (MODE == 2 && !barrier_wait(a, sm)) {
    // the wait gave up: this block's output rows are written as NaN, never left stale
    if (tid < kRowsPerBlock * a.T) {
      const int r = blockIdx.x * kRowsPerBlock + (tid & 7), t = tid >> 3;
      if (r < a.H) {
        if (a.out_dtype == 0) reinterpret_cast<float*>(a.out)[(size_t)t * a.H + r] = __builtin_nanf("");
        else reinterpret_cast<uint16_t*>(a.out)[(size_t)t * a.H + r] = 0x7FC0;
      }
    }
    return;
  }
  if (a.h_in_lds) {
    // agent-coherent 128-bit loads (cache policy sc1) of h into LDS. Above 4 pieces per
    // thread, kCopyBatch loads are in flight per thread before their LDS stores (one or
    // two memory round trips instead of one per piece: -2 us at 4 tokens); one token's
    // 3 pieces per thread measured faster one at a time.
    const int n16 = a.P * a.I / 4;  // 16-byte pieces, 8 per 32-value chunk
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc(a.h, 0, (int)((size_t)a.P * a.I * 4), 0x00020000);
    char* hd = dec_lds + x_lds_bytes(a.T, a.H);
    if (n16 <= 4 * kDecThreads) {
      for (int i = tid; i < n16; i += kDecThreads)
        *reinterpret_cast<uint4*>(hd + (i >> 3) * 144 + (i & 7) * 16) =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(hr, i * 16, 0, 16));
    } else {
      for (int b0 = 0; b0 < n16; b0 += kCopyBatch * kDecThreads) {  // block-uniform bounds
        uint4 v[kCopyBatch];
#pragma unroll
        for (int k = 0; k < kCopyBatch; ++k)  // pieces past the end of h read as zero
          if (b0 + k * kDecThreads < n16)
            v[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 hr, (b0 + k * kDecThreads + tid) * 16, 0, 16));
#pragma unroll
        for (int k = 0; k < kCopyBatch; ++k) {
          const int i = b0 + k * kDecThreads + tid;
          if (b0 + k * kDecThreads < n16 && i < n16)
            *reinterpret_cast<uint4*>(hd + (i >> 3) * 144 + (i & 7) * 16) = v[k];
        }
      }
    }
    __syncthreads();
  }

  float acc[kDecodeMaxT];
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) acc[t] = 0.f;
  const int per_wave = (sm.nu - wave + kDecWaves - 1) / kDecWaves;  // experts of this wave
  for (int ub0 = 0; ub0 < per_wave; ub0 += kUBof<Q8>) {
    if (ub0 > 0) down_load<CHD, Q8, X>(a, sm, ub0, row, l8, d);
    if (a.h_in_lds) down_accum<CHD, Q8, true>(a, sm, d, l8, acc);
    else down_accum<CHD, Q8, false>(a, sm, d, l8, acc);
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxT; ++t) {
    if (t < a.T) {
      const float v = sum8(acc[t]);
      if (l8 == 0) sm.part[wave][lane / kDownLanes][t] = v;
    }
  }
  __syncthreads();
  if (tid < kRowsPerBlock * a.T) {
    const int q8 = tid & 7, t = tid >> 3;  // row within the block, token
    float v = sm.part[0][q8][t];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) v += sm.part[w][q8][t];  // wave order
    const int r = blockIdx.x * kRowsPerBlock + q8;
    if (r < a.H) {
      if (a.out_dtype == 0) reinterpret_cast<float*>(a.out)[(size_t)t * a.H + r] = v;
      else reinterpret_cast<uint16_t*>(a.out)[(size_t)t * a.H + r] = f32_to_bf16_bits(v);
    }
  }
}

// Dynamic LDS budget of one block (of the 160 KiB per CU, the rest is static LDS).
constexpr size_t kDecLdsBudget = 152 * 1024;

static size_t decode_lds_bytes(const DecodeArgs& a) {
  return x_lds_bytes(a.T, a.H) + (a.h_in_lds ? h_lds_bytes(a.P, a.I) : 0);
}

template <int MODE, int CHG, int CHD, bool Q8, bool X>
static hipError_t launch_mode(const DecodeArgs& a, hipStream_t st) {
  const size_t lds = decode_lds_bytes(a);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<MODE, CHG, CHD, Q8, X>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((a.H + kRowsPerBlock - 1) / kRowsPerBlock);
  decode_kernel<MODE, CHG, CHD, Q8, X><<<grid, kDecThreads, lds, st>>>(a);
  return hipGetLastError();
}

// The fused form needs every block of its grid resident at once.
template <int CHG, int CHD, bool Q8, bool X>
static bool fused_fits(const DecodeArgs& a) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<2, CHG, CHD, Q8, X>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds_bytes(a)) != hipSuccess)
    return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<2, CHG, CHD, Q8, X>, kDecThreads,
                                                   decode_lds_bytes(a)) != hipSuccess)
    return false;
  return (long long)((a.H + kRowsPerBlock - 1) / kRowsPerBlock) <= (long long)cus * per_cu;
}

template <int CHG, int CHD, bool Q8, bool X>
static hipError_t launch_decode_q(int stage, const DecodeArgs& a, hipStream_t st) {
  if (stage == 0) return launch_mode<0, CHG, CHD, Q8, X>(a, st);
  if (stage == 1) return launch_mode<1, CHG, CHD, Q8, X>(a, st);
  // fused only when h fits in LDS: phase 2 then reads h once, with agent-coherent loads
  if (a.h_in_lds && fused_fits<CHG, CHD, Q8, X>(a)) return launch_mode<2, CHG, CHD, Q8, X>(a, st);
  const hipError_t e = launch_mode<0, CHG, CHD, Q8, X>(a, st);
  return e != hipSuccess ? e : launch_mode<1, CHG, CHD, Q8, X>(a, st);
}

template <int CHG, int CHD>
static hipError_t launch_decode_t(int stage, const DecodeArgs& a, hipStream_t st) {
  const bool x = a.gate.xe >= 0;
  if (a.down.fmt == 1)
    return x ? launch_decode_q<CHG, CHD, true, true>(stage, a, st) : launch_decode_q<CHG, CHD, true, false>(stage, a, st);
  return x ? launch_decode_q<CHG, CHD, false, true>(stage, a, st) : launch_decode_q<CHG, CHD, false, false>(stage, a, st);
}

hipError_t launch_decode(int stage, const void* x, int T, int H, int I, const WeightArgs& gate, const WeightArgs& up,
                         const WeightArgs& down, int E, const int32_t* ids, const float* w, int topk, void* out,
                         int out_dtype, float* h, int32_t* hdr, unsigned long long* flags, hipStream_t st) {
  DecodeArgs a;
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.T = T; a.H = H; a.I = I; a.E = E; a.P = T * topk; a.topk = topk;
  a.gate = gate; a.up = up; a.down = down;
  a.ids = ids; a.w = w; a.h = h; a.out = out; a.out_dtype = out_dtype;
  a.hdr = hdr;
  a.barrier = reinterpret_cast<unsigned*>(hdr + 4);
  a.epoch = reinterpret_cast<unsigned long long*>(hdr + 6);
  a.flags = flags;
  a.spin_limit = 1 << 22;
  a.h_in_lds = 0;
  a.h_in_lds = decode_lds_bytes(a) + h_lds_bytes(a.P, I) <= kDecLdsBudget ? 1 : 0;
  const int chg = ((H >> 5) + 15) / 16;  // 1..16 for H <= 8192
  const int chd = ((I >> 5) + kDownLanes - 1) / kDownLanes;
#define NVFP4_DEC(G, D) \
  if (chg <= G && chd <= D) return launch_decode_t<G, D>(stage, a, st);
  NVFP4_DEC(1, 1)
  NVFP4_DEC(2, 1)
  NVFP4_DEC(2, 2)
  NVFP4_DEC(4, 2)
  NVFP4_DEC(4, 3)
  NVFP4_DEC(4, 4)
  NVFP4_DEC(8, 4)
  NVFP4_DEC(8, 8)
  NVFP4_DEC(16, 8)
  NVFP4_DEC(16, 16)
  NVFP4_DEC(16, 32)
#undef NVFP4_DEC
  return hipErrorInvalidValue;
}

}  // namespace nvfp4

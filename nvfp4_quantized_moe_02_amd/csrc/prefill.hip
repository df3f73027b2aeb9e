// Prefill path: grouped GEMMs over the routed pairs on gfx950 matrix cores, one launch
// per stage for all experts ("Strata NVFP4" README, "How it differs from upstream
// Strata": an MMQ group's experts gathered in one launch; prompt chunks up to 32K
// tokens, each streaming every expert of a layer once).
//
// Tile = (expert, up to 128 routed rows) x one N block of WPB*64 weight rows; WPB = 8
// waves when the shape allows, else 4. Each wave owns an NRB*32 x 64 output block (NRB row
// blocks x 2 column blocks of v_mfma_f32_32x32x16_f16), where NRB = ceil(rows / 32) is a
// template parameter, so partial tiles skip the empty row blocks without branches in the
// K loop.
//
// A (activations, fp16): loaded two K-blocks (of 64 inputs) ahead into registers and
// stored to a 2-stage LDS ring at the top of the iteration that uses it.
// Each LDS row holds 64 inputs (8 slots of 16 bytes); slot c of row r holds chunk
// c ^ (r & 7), so the 32 rows of an MFMA fragment read hit 8 distinct slots (no bank
// conflicts). Rows are gathered by token for gate/up and contiguous for down.
//
// B (NVFP4 weights): the block stages its weight rows' codes GK K-blocks at a
// time with coalesced loads (consecutive threads read one row's GK*32 contiguous bytes)
// one group ahead in registers, stores each group to an XOR-swizzled LDS tile, and every
// lane reads its fragment's 16 code bytes per K-block from there. Each lane loads its
// column's scale bytes for four K-blocks at once. The unpack to fp16 is exact: E2M1 codes
// and the E4M3 scale both convert exactly to fp16, and their product (at most 5
// significant bits) is exact in one packed fp16 multiply; each weight is decoded once per
// block. Within a K-block the reduction order of the 64 inputs is permuted (lane half 0
// takes inputs 0..31, half 1 inputs 32..63); A is read with the same permutation, so the
// dot products are unchanged.
//
// Inside a K-block each lane reads its A fragments two ahead of their MFMAs (the LDS
// latency hides under the MFMAs in between), unpacks the B fragments of the next step
// right after issuing the current step's last MFMA, and issues the global loads of later
// K-blocks spread over the MFMAs: all waves issuing them in one burst after the barrier
// made each wave queue in the address unit before its first MFMA.
//
// gate/up: wave w computes gate and up for the same 32 intermediate indices, so SwiGLU
// runs in registers: h = SiLU(gamma_g * g) * (gamma_u * u) (gate scale before SiLU, the
// "Strata NVFP4" README's per-projection output scale); the weights are the MFMA's first
// operand, so each lane ends with four adjacent h values of a row and stores them directly.
// down: the epilogue multiplies by gamma_d and the router weight and writes each pair's
// fp32 row through LDS as whole 1 KB row segments; a separate combine sums the slots of
// each token in slot order, so the result is deterministic.
#include <type_traits>

#include "kernels.h"

namespace nvfp4 {

constexpr int BM = kTileM;
constexpr int KBLK = 64;                        // inputs per K-block
constexpr int NSTAGE = 2;                       // LDS stages of A
constexpr int STAGE_BYTES = BM * KBLK * 2;      // 16 KiB per stage

__device__ __forceinline__ uint32_t word_of(const uint4& c, int s) {
  return s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
}

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x8_t bfrag(uint32_t word, _Float16 sc) {
  f16x2_t o[4];
  unpack8_f16(word, sc, o);
  const f16x4_t lo = __builtin_shufflevector(o[0], o[1], 0, 1, 2, 3);
  const f16x4_t hi = __builtin_shufflevector(o[2], o[3], 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Q8_0 fragment: 8 int8 weights (two words) -> fp16 exactly (each byte with its sign bit
// flipped, q + 128, becomes the mantissa of the fp16 value 1024 + q + 128 by a byte
// permute; subtracting 1152 is exact), then one fp16 multiply by the block scale d: the
// one rounding of the path's operands (relative error at most 2^-11).
__device__ __forceinline__ f16x8_t bfrag_q8(uint32_t lo, uint32_t hi, _Float16 d) {
  const uint32_t u0 = lo ^ 0x80808080u, u1 = hi ^ 0x80808080u;
  const f16x2_t k = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2_t dd = {d, d};
  const f16x2_t o0 = (__builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) - k) * dd;
  const f16x2_t o1 = (__builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) - k) * dd;
  const f16x2_t o2 = (__builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) - k) * dd;
  const f16x2_t o3 = (__builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) - k) * dd;
  const f16x4_t lo4 = __builtin_shufflevector(o0, o1, 0, 1, 2, 3);
  const f16x4_t hi4 = __builtin_shufflevector(o2, o3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// SiLU for the fp16/fp32 h of the prefill path: exp and reciprocal from the hardware
// approximations (about 1 ulp each).
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

struct TileCtx {
  int e, m0, rows, base, nb;
};

// Scale bytes are loaded KQ K-blocks at a time (4 * KQ bytes of one column's scale row
// per lane, 16-byte aligned for KQ = 4 when K is a multiple of 256, 8-byte for KQ = 2);
// one byte permute per two K-blocks keeps the two bytes of each K-block this lane uses.
template <int KQ>
struct ScaleRaw;
template <>
struct ScaleRaw<4> {
  typedef uint4 type;
};
template <>
struct ScaleRaw<2> {
  typedef uint2 type;
};

// B tile of a block: NCB = WPB * 64 weight rows (gate/up: WPB*32 gate rows, then the
// same WPB*32 up rows; down: WPB*64 rows), GK K-blocks at a time, in LDS.
template <int WPB, int GK>
struct BTile {
  static constexpr int NCB = WPB * 64;
  static constexpr int ROWB = GK * 32;                  // code bytes of one row per group
  static constexpr int CPR = GK * 2;                    // 16-byte chunks per row per group
  static constexpr int SHIFT = GK == 2 ? 1 : 0;         // swizzle: chunk ^ ((row >> SHIFT) & (CPR-1))
  static constexpr int BYTES = NCB * ROWB;
  static constexpr int CH = BYTES / (WPB * 64 * 16);    // 16-byte chunks staged per thread
  static constexpr int RPT = WPB * 64 / CPR;            // rows covered by one staging round
  __device__ static int slot(int row, int ch) { return row * ROWB + ((ch ^ ((row >> SHIFT) & (CPR - 1))) << 4); }
};

template <bool GATEUP, bool ASCALE, bool HOUT32, int NRB, int KQ, int WPB, int GK, bool Q8>
__device__ __forceinline__ void gemm_tile(const TileCtx& tc, const uint16_t* __restrict__ A, int K,
                                          const uint8_t* b0row, const uint8_t* b1row,
                                          const uint8_t* const* bs, const WeightArgs& w0,
                                          const WeightArgs& w1, void* __restrict__ out, int ldo, char* lds,
                                          const int* s_src, const float* s_coef) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nkb = K / KBLK;

  // A: thread t copies 16-byte chunk t & 7 of rows (t >> 3) + RPR*i, i < NA, of a
  // K-block; it stores chunk c of row r into slot c ^ (r & 7) of that LDS row. With 8
  // waves and an odd NRB the last round also copies 32 rows the MFMAs never read (padding
  // rows of the tile, so in bounds), which keeps the loop free of branches.
  constexpr int RPR = WPB * 8;
  constexpr int NA = (NRB * 32 + RPR - 1) / RPR;
  const int arow = tid >> 3, achunk = tid & 7;
  const uint16_t* asrc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) asrc[i] = A + (size_t)s_src[arow + RPR * i] * K + achunk * 8;
  const int aslot = ((achunk ^ (arow & 7)) << 4);

  // B codes: the block's NCB weight rows, GK K-blocks (GK*32 bytes of each row) per
  // group. Thread t stages chunks j*(WPB*64) + t of the group tile, i.e. chunk t % CPR of
  // rows j*RPT + t / CPR: CPR consecutive threads read one row's GK*32 contiguous bytes.
  // They go to LDS once per group; each lane then reads its fragments from there.
  // Q8_0 (down only): a group is one K-block, 64 int8 weights per row (the tile geometry
  // of two NVFP4 K-blocks).
  constexpr int GKB = Q8 ? 1 : GK;  // K-blocks per B group
  typedef BTile<WPB, Q8 ? 2 : GK> BT;
  const size_t rowbytes = Q8 ? K : K / 2;
  char* btiles = lds + NSTAGE * STAGE_BYTES;
  const int brow = tid / BT::CPR, bch = tid % BT::CPR;
  const int ngb = nkb / GKB;
  auto load_bg = [&](int g, int j) -> uint4 {
    const int gc = g < ngb ? g : ngb - 1;  // past the end: refetch the last group (never used)
    const int row = j * BT::RPT + brow;
    // gate/up: rows [0, NCB/2) are gate rows, [NCB/2, NCB) the same up rows (j is a
    // compile-time index, so the tensor choice is too)
    const uint8_t* base = (GATEUP && j * BT::RPT >= BT::NCB / 2) ? b1row + (size_t)(row - BT::NCB / 2) * rowbytes
                                                                 : b0row + (size_t)row * rowbytes;
    return *reinterpret_cast<const uint4*>(base + gc * BT::ROWB + bch * 16);
  };
  // tile row of this lane's fragment in column block cb
  const int frow0 = GATEUP ? wave * 32 + l32 : wave * 64 + l32;
  const int frow1 = GATEUP ? BT::NCB / 2 + wave * 32 + l32 : wave * 64 + 32 + l32;
  // Scales: K-block kb of a column holds 4 bytes (NVFP4: groups 4kb .. 4kb+3; Q8_0: the
  // fp16 scales of blocks 2kb, 2kb+1); lane half h uses bytes 2h and 2h+1 either way. A
  // group of KQ K-blocks is one load per column.
  typedef typename ScaleRaw<KQ>::type SRaw;
  const int ngrp = nkb / KQ;
  auto load_s = [&](int j, int cb) -> SRaw {
    const int jc = j < ngrp ? j : ngrp - 1;
    return *reinterpret_cast<const SRaw*>(bs[cb] + jc * (4 * KQ));
  };
  const uint32_t psel = half ? 0x07060302u : 0x05040100u;
  // compact word c holds, for K-blocks 2c and 2c+1 of the group, this lane's two bytes each
  auto compact = [&](const SRaw& r, uint32_t* c) {
    if constexpr (KQ == 4) {
      c[0] = __builtin_amdgcn_perm(r.y, r.x, psel);
      c[1] = __builtin_amdgcn_perm(r.w, r.z, psel);
    } else {
      c[0] = __builtin_amdgcn_perm(r.y, r.x, psel);
    }
  };
  auto load_a = [&](int kb, int i) -> uint4 {
    const int kc = kb < nkb ? kb : nkb - 1;
    return *reinterpret_cast<const uint4*>(asrc[i] + kc * KBLK);
  };

  f32x16_t acc[NRB][2];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] = 0.f;

  // Two K-blocks of A in registers; B codes one group ahead in registers. Iteration kb:
  // store A(kb) into LDS stage kb & 1, barrier; at a group start also store the staged
  // group into the B tile (every wave finished the previous group's reads at the barrier),
  // barrier, and stage the next group; issue A(kb+2); compute K-block kb.
  // The scales of the next group are loaded two K-blocks before the end of a scale group
  // and compacted at its end, inside the same loop iteration (a value carried across the
  // back-edge while loads are in flight makes the compiler drain every load there).
  uint4 aq[2][NA];
  uint4 bg[BT::CH];
  SRaw sq[2] = {load_s(0, 0), load_s(0, 1)};
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < BT::CH; ++j) bg[j] = load_bg(0, j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
#pragma unroll
    for (int i = 0; i < NA; ++i) aq[d][i] = load_a(d, i);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint32_t sc0[KQ / 2], sc1[KQ / 2];
  compact(sq[0], sc0);
  compact(sq[1], sc1);

  auto kstep = [&](auto qpos, int kb) {
    constexpr int Q = decltype(qpos)::value;  // position in the scale group
    constexpr int R = Q & 1;                  // LDS stage / register ring slot
    char* st = lds + R * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<uint4*>(st + (arow + RPR * i) * 128 + aslot) = aq[R][i];
    // A(kb) visible to all waves. Stage R was last read in iteration kb-2, and every wave
    // finished those reads before passing the barrier of iteration kb-1.
    __syncthreads();
    if constexpr (Q % GKB == 0) {
#pragma unroll
      for (int j = 0; j < BT::CH; ++j)
        *reinterpret_cast<uint4*>(btiles + BT::slot(j * BT::RPT + brow, bch)) = bg[j];
      __syncthreads();
    }
    const char* btile = btiles;
    // The next B group (at a group start) and A(kb+2) are loaded spread over the MFMAs of
    // this K-block: a burst of loads from every wave right after the barrier queues in the
    // address unit and holds back each wave's first MFMAs.
    constexpr int NBL = (Q % GKB == 0) ? BT::CH : 0;
    constexpr int NLD = NBL + NA;
    auto issue_loads = [&](int idx, int nf) {
#pragma unroll
      for (int g = 0; g < NLD; ++g) {
        if (g * nf / NLD == idx) {
          if (g < NBL) bg[g < NBL ? g : 0] = load_bg(kb / GKB + 1, g < NBL ? g : 0);
          else aq[R][g - NBL] = load_a(kb + 2, g - NBL);
        }
      }
    };
    // NVFP4: K-block q of the group is chunks 2q (half 0) and 2q+1 (half 1) of a row, one
    // 16-byte chunk per lane; Q8_0: chunks 2*half and 2*half+1, 32 bytes per lane
    constexpr int q = Q % GKB;
    const uint4 cur0 = *reinterpret_cast<const uint4*>(btile + BT::slot(frow0, Q8 ? 2 * half : 2 * q + half));
    const uint4 cur1 = *reinterpret_cast<const uint4*>(btile + BT::slot(frow1, Q8 ? 2 * half : 2 * q + half));
    uint4 cur0b = cur0, cur1b = cur1;
    if constexpr (Q8) {
      cur0b = *reinterpret_cast<const uint4*>(btile + BT::slot(frow0, 2 * half + 1));
      cur1b = *reinterpret_cast<const uint4*>(btile + BT::slot(frow1, 2 * half + 1));
    }
    // NVFP4: the lane's two 16-group scales (E4M3 -> fp16); Q8_0: its block scale d twice
    f16x2_t s0, s1;
    if constexpr (Q8) {
      const _Float16 d0 = __builtin_bit_cast(f16x2_t, sc0[Q >> 1])[Q & 1];
      const _Float16 d1 = __builtin_bit_cast(f16x2_t, sc1[Q >> 1])[Q & 1];
      s0 = f16x2_t{d0, d0};
      s1 = f16x2_t{d1, d1};
    } else {
      s0 = e4m3x2_f16<(Q & 1) != 0>(sc0[Q >> 1]);
      s1 = e4m3x2_f16<(Q & 1) != 0>(sc1[Q >> 1]);
    }
    // the B fragment of step s (inputs 32*half + 8s .. +7 of the K-block)
    auto bstep = [&](const uint4& c, const uint4& cb, f16x2_t sc, int s) -> f16x8_t {
      if constexpr (Q8) {
        const uint4& w = s < 2 ? c : cb;
        return (s & 1) ? bfrag_q8(w.z, w.w, sc[0]) : bfrag_q8(w.x, w.y, sc[0]);
      } else {
        return bfrag(word_of(c, s), sc[s >> 1]);
      }
    };
    // A fragments are read LA fragments ahead of their MFMAs (a ring of LA+1), so the LDS
    // latency of each read hides under the MFMAs issued in between; the B fragments of
    // step s+1 are unpacked right after the last MFMA of step s is issued.
    constexpr int NF = 4 * NRB, LA = 2;
    f16x8_t ring[LA + 1];
    auto read_a = [&](int idx) -> f16x8_t {
      const int s = idx / NRB, rb = idx % NRB;
      const int row = rb * 32 + l32, chunk = half * 4 + s;
      return *reinterpret_cast<const f16x8_t*>(st + row * 128 + ((chunk ^ (row & 7)) << 4));
    };
#pragma unroll
    for (int i = 0; i < LA; ++i) ring[i] = read_a(i);
    f16x8_t b0 = bstep(cur0, cur0b, s0, 0);
    f16x8_t b1 = bstep(cur1, cur1b, s1, 0);
#pragma unroll
    for (int idx = 0; idx < NF; ++idx) {
      if (idx + LA < NF) ring[(idx + LA) % (LA + 1)] = read_a(idx + LA);
      issue_loads(idx, NF);
      __builtin_amdgcn_sched_barrier(0);
      const int s = idx / NRB, rb = idx % NRB;
      // gate/up: weights as the first operand (output-major accumulators, see the epilogue)
      if constexpr (GATEUP) {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, ring[idx % (LA + 1)], acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, ring[idx % (LA + 1)], acc[rb][1], 0, 0, 0);
      } else {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[idx % (LA + 1)], b0, acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[idx % (LA + 1)], b1, acc[rb][1], 0, 0, 0);
      }
      if (rb == NRB - 1 && s < 3) {
        b0 = bstep(cur0, cur0b, s0, s + 1);
        b1 = bstep(cur1, cur1b, s1, s + 1);
      }
    }
  };
  // nkb is a multiple of KQ
  for (int j = 0; j < ngrp; ++j) {
    const int kb = j * KQ;
    if constexpr (KQ == 4) {
      kstep(std::integral_constant<int, 0>{}, kb);
      kstep(std::integral_constant<int, 1>{}, kb + 1);
      sq[0] = load_s(j + 1, 0);
      sq[1] = load_s(j + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      kstep(std::integral_constant<int, 2>{}, kb + 2);
      kstep(std::integral_constant<int, 3>{}, kb + 3);
    } else {
      sq[0] = load_s(j + 1, 0);
      sq[1] = load_s(j + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      kstep(std::integral_constant<int, 0>{}, kb);
      kstep(std::integral_constant<int, 1>{}, kb + 1);
    }
    compact(sq[0], sc0);
    compact(sq[1], sc1);
  }

  if constexpr (GATEUP) {
    // The weights are the first MFMA operand, so element v of acc[rb][cb] is intermediate
    // index 8*(v/4) + 4*half + v%4 of the wave's 32, for token row rb*32 + l32: four
    // consecutive v are four adjacent h values of one row, stored as one 8-byte (fp16) or
    // 16-byte (fp32) piece straight to memory.
    const float gg = w0.global[tc.e], gu = w1.global[tc.e];
    const int col0 = tc.nb * (WPB * 32) + wave * 32 + 4 * half;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + l32;
      const float xs = s_coef[r];
      const float cg = xs * gg, cu = xs * gu;
      const size_t rowoff = (size_t)(tc.base + tc.m0 + r) * ldo + col0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          hv[v] = silu_fast(acc[rb][0][4 * g + v] * cg) * (acc[rb][1][4 * g + v] * cu);
        if (r < tc.rows) {
          if constexpr (HOUT32) {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + rowoff + 8 * g) =
                f32x4_t{hv[0], hv[1], hv[2], hv[3]};
          } else {
            const uint2 pk = {(uint32_t)f32_to_f16_bits(hv[0]) | ((uint32_t)f32_to_f16_bits(hv[1]) << 16),
                              (uint32_t)f32_to_f16_bits(hv[2]) | ((uint32_t)f32_to_f16_bits(hv[3]) << 16)};
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + rowoff + 8 * g) = pk;
          }
        }
      }
    }
  } else {
    // y[pos][n] = gamma_d * coef[pos] * acc, fp32, in sorted order; the combine kernel sums
    // each token's slots. One row block at a time goes through LDS ([32][NCOL] fp32, 16-byte
    // chunks XOR-swizzled by row), so every store is a full 16 bytes and a wave writes whole
    // 1 KB row segments; the stores are non-temporal (y is read once, by the combine). The
    // kernel's LDS holds 32 * NCOL * 4 bytes.
    constexpr int NCOL = WPB * 64;
    const float gd = w0.global ? w0.global[tc.e] : 1.0f;  // a Q8_0 down may have no tensor scale
    float* y = reinterpret_cast<float*>(out);
    float* yl = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      __syncthreads();  // the A stages / the previous row block are no longer read
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = (i >> 2) * 8 + half * 4 + (i & 3);
        const float c = s_coef[rb * 32 + rr] * gd;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int col = wave * 64 + cb * 32 + l32;
          yl[rr * NCOL + (((col >> 2) ^ (rr & 7)) << 2) + (col & 3)] = acc[rb][cb][i] * c;
        }
      }
      __syncthreads();
      for (int k = tid; k < 32 * (NCOL / 4); k += WPB * 64) {
        const int rr = k / (NCOL / 4), cc = k % (NCOL / 4);
        const int r = rb * 32 + rr;
        if (r < tc.rows) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(yl + rr * NCOL + ((cc ^ (rr & 7)) << 2));
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(y + (size_t)(tc.base + tc.m0 + r) * ldo +
                                                                     tc.nb * NCOL + cc * 4));
        }
      }
    }
  }
}

// GATEUP: gate/up + SwiGLU (w0 = gate, w1 = up), else down + combine (w0 = down).
// ASCALE: multiply by a per-row activation scale (the W4A8 int8 scales).
// HOUT32: gate/up writes fp32 h (for the int8 requantization), else fp16 h.
template <bool GATEUP, bool ASCALE, bool HOUT32, int KQ, int WPB, int GK, bool Q8 = false>
__global__ __launch_bounds__(WPB * 64, 8 / WPB) void moe_gemm_f16_kernel(
    const uint16_t* __restrict__ A, const float* __restrict__ a_scale, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, const TileDesc* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    int topk, int K, int NB, WeightArgs w0, WeightArgs w1, const float* __restrict__ route_w,
    void* __restrict__ out, int ldo) {
  // A stages and the B tile; the down epilogue reuses them (32 rows x WPB*64 fp32)
  constexpr int kMain = NSTAGE * STAGE_BYTES + BTile<WPB, Q8 ? 2 : GK>::BYTES;
  constexpr int kEpi = GATEUP ? 0 : 32 * WPB * 64 * 4;
  constexpr int kLds = kMain > kEpi ? kMain : kEpi;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ int s_src[BM];
  __shared__ float s_coef[BM];

  // XCD-aware order: consecutive logical tiles (the N blocks of one row tile, then the
  // row tiles of one expert) run on the same XCD and share its L2.
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
  tc.rows = Me - tc.m0 < BM ? Me - tc.m0 : BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31;
  if (tid < BM) {
    const int r = tid < tc.rows ? tid : tc.rows - 1;  // padding rows repeat the last row
    const int pos = tc.base + tc.m0 + r;
    const int p = sorted_pairs[pos];
    if (GATEUP) {
      s_src[tid] = p / topk;
      s_coef[tid] = ASCALE ? a_scale[p / topk] : 1.0f;
    } else {
      s_src[tid] = pos;
      s_coef[tid] = route_w[p] * (ASCALE ? a_scale[pos] : 1.0f);
    }
  }

  // first weight row of the block in each tensor; per-lane scale rows of its fragments
  const uint8_t* b0row;
  const uint8_t* b1row;
  const uint8_t* bs[2];
  if (GATEUP) {
    const size_t row0 = (size_t)tc.e * w0.N + tc.nb * (WPB * 32);
    b0row = w0.codes + row0 * (K / 2);
    b1row = w1.codes + row0 * (K / 2);
    bs[0] = w0.scales + (row0 + wave * 32 + l32) * (K / 16);
    bs[1] = w1.scales + (row0 + wave * 32 + l32) * (K / 16);
  } else {
    const size_t row0 = (size_t)tc.e * w0.N + tc.nb * (WPB * 64);
    b0row = w0.codes + row0 * (Q8 ? K : K / 2);
    b1row = b0row;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) bs[cb] = w0.scales + (row0 + wave * 64 + cb * 32 + l32) * (K / 16);
  }
  __syncthreads();

  const int nrb = (tc.rows + 31) >> 5;
  if (nrb == 4)
    gemm_tile<GATEUP, ASCALE, HOUT32, 4, KQ, WPB, GK, Q8>(tc, A, K, b0row, b1row, bs, w0, w1, out, ldo, lds, s_src, s_coef);
  else if (nrb == 3)
    gemm_tile<GATEUP, ASCALE, HOUT32, 3, KQ, WPB, GK, Q8>(tc, A, K, b0row, b1row, bs, w0, w1, out, ldo, lds, s_src, s_coef);
  else if (nrb == 2)
    gemm_tile<GATEUP, ASCALE, HOUT32, 2, KQ, WPB, GK, Q8>(tc, A, K, b0row, b1row, bs, w0, w1, out, ldo, lds, s_src, s_coef);
  else
    gemm_tile<GATEUP, ASCALE, HOUT32, 1, KQ, WPB, GK, Q8>(tc, A, K, b0row, b1row, bs, w0, w1, out, ldo, lds, s_src, s_coef);
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
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a);
  // 8 waves (256 intermediate indices per block) when I allows, else 4 (128); H is a
  // multiple of 256, so scale groups of 4 K-blocks; B groups of 2 K-blocks.
#define NVFP4_GU(ASC, H32, WPB, GK)                                                                      \
  moe_gemm_f16_kernel<true, ASC, H32, 4, WPB, GK><<<grid_for(max_tiles, I / (WPB * 32)), WPB * 64, 0, st>>>( \
      A, a_scale, sorted_pairs, offsets, tiles, tile_count, topk, H, I / (WPB * 32), gate, up, nullptr, h, I)
  const bool w8 = I % 256 == 0;
  if (act == 0) {
    if (w8)
      NVFP4_GU(false, false, 8, 2);
    else
      NVFP4_GU(false, false, 4, 2);
  } else {
    if (w8)
      NVFP4_GU(true, true, 8, 2);
    else
      NVFP4_GU(true, true, 4, 2);
  }
#undef NVFP4_GU
  return hipGetLastError();
}

hipError_t launch_gemm_down(int act, const void* h, const float* h_scale, const int32_t* sorted_pairs,
                            const int32_t* offsets, const TileDesc* tiles, const int32_t* tile_count,
                            int max_tiles, int topk, int H, int I, const WeightArgs& down, const float* w,
                            float* y, hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(h);
  // 8 waves (512 outputs per block) when H allows, else 4 (256); scale groups of 4
  // K-blocks when I is a multiple of 256, else 2; B groups of 2 K-blocks.
#define NVFP4_DOWN(ASC, KQ, WPB)                                                                           \
  do {                                                                                                     \
    const dim3 grid = grid_for(max_tiles, H / (WPB * 64));                                                 \
    if (down.fmt == 1)                                                                                     \
      moe_gemm_f16_kernel<false, ASC, false, KQ, WPB, 2, true><<<grid, WPB * 64, 0, st>>>(                 \
          A, h_scale, sorted_pairs, offsets, tiles, tile_count, topk, I, H / (WPB * 64), down, down, w, y, H); \
    else                                                                                                   \
      moe_gemm_f16_kernel<false, ASC, false, KQ, WPB, 2><<<grid, WPB * 64, 0, st>>>(                       \
          A, h_scale, sorted_pairs, offsets, tiles, tile_count, topk, I, H / (WPB * 64), down, down, w, y, H); \
  } while (0)
#define NVFP4_DOWN_W(ASC, KQ) \
  if (H % 512 == 0)           \
    NVFP4_DOWN(ASC, KQ, 8);   \
  else                        \
    NVFP4_DOWN(ASC, KQ, 4);
  const bool q4 = I % 256 == 0;
  if (act == 0) {
    if (q4) {
      NVFP4_DOWN_W(false, 4)
    } else {
      NVFP4_DOWN_W(false, 2)
    }
  } else {
    if (q4) {
      NVFP4_DOWN_W(true, 4)
    } else {
      NVFP4_DOWN_W(true, 2)
    }
  }
#undef NVFP4_DOWN_W
#undef NVFP4_DOWN
  return hipGetLastError();
}

}  // namespace nvfp4

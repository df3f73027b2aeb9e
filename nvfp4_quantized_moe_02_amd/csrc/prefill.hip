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
// stored to a 2-stage LDS ring at the top of the iteration that uses it. The gate/up GEMM
// on fp16 activations (the prefill's default) instead loads A, the B codes and the scale
// bytes straight into LDS (global_load_lds_dwordx4, 4 A stages, explicit vmcnt waits before
// each K-block's barrier): no staging registers and no LDS store instructions.
// Each LDS row holds 64 inputs (8 slots of 16 bytes); chunk c of row r sits in slot
// c ^ ((r >> 1) & 7). gfx950's LDS serves a 128-bit read 16 lanes (256 bytes, all 64
// banks) per cycle, and the 16 rows of such a lane group then cover every bank once: the
// row's parity picks the 128-byte half, the slot the 16 bytes within it (with the slot
// keyed on r & 7, rows r and r + 8 collided: measured 38% of LDS-active cycles in bank
// conflicts, none with this key). Rows are gathered by token for gate/up and contiguous
// for down.
//
// B (NVFP4 weights): the block stages its weight rows' codes GK K-blocks at a
// time with coalesced loads (consecutive threads read one row's GK*32 contiguous bytes)
// one group ahead in registers, stores each group to one of two XOR-swizzled LDS tiles
// (alternating, so a group is stored beside A before the K-block's one barrier), and
// every lane reads its fragment's 16 code bytes per K-block from there. Each lane loads its
// column's scale bytes for four K-blocks at once. The unpack to fp16 is exact: E2M1 codes
// and the E4M3 scale both convert exactly to fp16, and their product (at most 5
// significant bits) is exact in one packed fp16 multiply; each weight is decoded once per
// block. Within a K-block the reduction order of the 64 inputs is permuted (lane half 0
// takes inputs 0..31, half 1 inputs 32..63); A is read with the same permutation, so the
// dot products are unchanged.
//
// Inside a K-block each lane reads its A fragments two ahead of their MFMAs (the LDS
// latency hides under the MFMAs in between), unpacks the B fragments of the next step
// between the current step's MFMAs, and issues the global loads of later
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

// Direct-to-LDS staging for the gate/up GEMM on fp16 activations (the one mode whose A
// needs no conversion): A and B go from memory straight into their swizzled LDS slots with
// global_load_lds_dwordx4 (each lane's 16 bytes land at the wave's LDS window + 16 * lane,
// so the XOR swizzle is applied to the source chunk a lane loads), with four A stages.
#ifndef NVFP4_GATEUP_DLDS
#define NVFP4_GATEUP_DLDS 1
#endif
template <bool GATEUP, int AM, int KQ, bool Q8>
constexpr bool direct_lds() {
  return NVFP4_GATEUP_DLDS && GATEUP && AM == 0 && KQ == 4 && !Q8;
}
constexpr int NSTAGE_DL = 4;  // A stages with direct-to-LDS loads: K-block kb in stage kb & 3

typedef __attribute__((address_space(3))) char* lds_ptr_t;
// 16 bytes per lane from gsrc into the wave's LDS window at ldst (wave-uniform) + 16 * lane.
// Written as asm: the compiler, seeing the builtin's LDS write, waits for it to land
// (vmcnt(0)) before every later LDS read, which would serialize the prefetch. The
// instruction writes no register (the data goes to LDS), and its waits are explicit here:
// wait_vm before the barrier that publishes the stage, wait_vm<0> before the block ends.
__device__ __forceinline__ void load_lds16(const void* gsrc, char* ldst) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)ldst);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(m) : "memory", "m0");
}
// wait until at most N vector memory operations of this wave are outstanding (gfx9
// s_waitcnt encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

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

// 8 int8 values (two words) -> 8 fp16 exactly: each byte with its sign bit flipped,
// q + 128, becomes the mantissa of the fp16 value 1024 + q + 128 by a byte permute, and
// subtracting 1152 is exact.
__device__ __forceinline__ f16x8_t i8x8_f16(uint32_t lo, uint32_t hi) {
  const uint32_t u0 = lo ^ 0x80808080u, u1 = hi ^ 0x80808080u;
  const f16x2_t k = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2_t o0 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) - k;
  const f16x2_t o1 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) - k;
  const f16x2_t o2 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) - k;
  const f16x2_t o3 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) - k;
  const f16x4_t lo4 = __builtin_shufflevector(o0, o1, 0, 1, 2, 3);
  const f16x4_t hi4 = __builtin_shufflevector(o2, o3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Q8_0 fragment: 8 int8 weights -> fp16 exactly, then one fp16 multiply by the block
// scale d: the one rounding of the path's operands (relative error at most 2^-11).
__device__ __forceinline__ f16x8_t bfrag_q8(uint32_t lo, uint32_t hi, _Float16 d) {
  const f16x8_t v = i8x8_f16(lo, hi);
  const f16x8_t dd = {d, d, d, d, d, d, d, d};
  return v * dd;
}

// fp16 bits of 2^-d for a right shift by d >= 0 bits (subnormal for d > 14, zero past 24).
__device__ __forceinline__ uint32_t f16_pow2_neg(int d) {
  return d <= 14 ? (uint32_t)(15 - d) << 10 : d <= 24 ? 1u << (24 - d) : 0u;
}


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
  // swizzle: chunk ^ ((row >> SHIFT) & (CPR-1)); a 16-lane fragment read (16 rows) then
  // covers all 64 banks once (row & (256/ROWB - 1) picks the bank block, the key the slot)
  static constexpr int SHIFT = GK == 2 ? 2 : 3;
  static constexpr int BYTES = NCB * ROWB;
  static constexpr int CH = BYTES / (WPB * 64 * 16);    // 16-byte chunks staged per thread
  static constexpr int RPT = WPB * 64 / CPR;            // rows covered by one staging round
  __device__ static int slot(int row, int ch) { return row * ROWB + ((ch ^ ((row >> SHIFT) & (CPR - 1))) << 4); }
};

// Activation modes. A_F16: fp16 activations staged with a power-of-two exponent per row
// (gate/up: the token row's, from the staging launch; down: h stored per gate/up block
// with that block's exponent, brought to the row's smallest exponent while A is staged into
// LDS); the epilogue multiplies by 2^-exponent with ldexp, so no operand overflows or
// underflows fp16 whatever the activations' range. A_I8: int8 activations (1 byte each,
// converted to fp16 exactly when staged) with an fp32 scale per row (the W4A8 path).
// A_F4: NVFP4 activations (E2M1 codes, two per byte, and an E4M3 scale per 16 inputs)
// with an fp32 scale per row (the W4A4 path); code * scale is exact in fp16 (as for the
// weights), so the operands are exact and the row scale multiplies at the accumulator.
constexpr int A_F16 = 0, A_I8 = 1, A_F4 = 2;
constexpr int kMaxHSeg = 64;  // gate/up blocks along I that the down GEMM can rescale (I <= 8192)

template <bool GATEUP, int AM, int NRB, int KQ, int WPB, int GK, bool Q8>
__device__ __forceinline__ void gemm_tile(const TileCtx& tc, const void* __restrict__ A,
                                          const uint8_t* __restrict__ Abs, int K,
                                          const uint8_t* b0row, const uint8_t* b1row,
                                          const uint8_t* const* bs, const WeightArgs& w0,
                                          const WeightArgs& w1, void* __restrict__ out, int ldo, char* lds,
                                          const int* s_src, const float* s_coef, const int* s_exp,
                                          const uint8_t* s_hd, int seg_shift, float* s_red,
                                          int32_t* __restrict__ hexp_out, int NB) {
  constexpr bool HOUT32 = GATEUP && AM != A_F16;
  constexpr bool DL = direct_lds<GATEUP, AM, KQ, Q8>();
  // A_F4 raw chunk: x = the 8 codes, y = the K-block's 4 scale bytes
  typedef typename std::conditional<AM == A_F16, uint4, uint2>::type ARaw;
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
  // bytes per K-block of one A row in memory (A_F4: codes; its scales are 4 more)
  constexpr int KBB = AM == A_F16 ? KBLK * 2 : AM == A_I8 ? KBLK : KBLK / 2;
  const char* asrc[NA];
  const uint8_t* absrc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const size_t row = (size_t)s_src[arow + RPR * i];
    asrc[i] = reinterpret_cast<const char*>(A) + row * (K / KBLK) * KBB + achunk * (KBB / 8);
    absrc[i] = AM == A_F4 ? Abs + row * (K / kGroup) : nullptr;
  }
  const int aslot = ((achunk ^ ((arow >> 1) & 7)) << 4);
  const int ashift = 8 * (achunk >> 1);  // A_F4: the chunk's scale byte in the K-block's word
  // DL: lane L of wave w fills slot L & 7 of row 8w + L/8 (+ RPR*i), so it loads the chunk
  // that the swizzle puts there: chunk (L & 7) ^ key(row)
  const char* adl[NA];
  if constexpr (DL) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = arow + RPR * i;
      adl[i] = reinterpret_cast<const char*>(A) + (size_t)s_src[row] * K * 2 + ((achunk ^ ((row >> 1) & 7)) << 4);
    }
  }

  // B codes: the block's NCB weight rows, GK K-blocks (GK*32 bytes of each row) per
  // group. Thread t stages chunks j*(WPB*64) + t of the group tile, i.e. chunk t % CPR of
  // rows j*RPT + t / CPR: CPR consecutive threads read one row's GK*32 contiguous bytes.
  // They go to LDS once per group; each lane then reads its fragments from there.
  // Q8_0 (down only): a group is one K-block, 64 int8 weights per row (the tile geometry
  // of two NVFP4 K-blocks).
  constexpr int GKB = Q8 ? 1 : GK;  // K-blocks per B group
  typedef BTile<WPB, Q8 ? 2 : GK> BT;
  const size_t rowbytes = Q8 ? K : K / 2;
  char* btiles = lds + (DL ? NSTAGE_DL : NSTAGE) * STAGE_BYTES;
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
  // DL: group g's staging round j straight into tile t: lane L of wave w fills slot L % CPR
  // of tile row j*RPT + 16w + L/CPR (the thread's brow), loading the chunk the swizzle
  // puts there
  auto load_bg_dl = [&](int g, int j, char* tile) {
    const int gc = g < ngb ? g : ngb - 1;
    const int row = j * BT::RPT + brow;
    const uint8_t* base = (GATEUP && j * BT::RPT >= BT::NCB / 2) ? b1row + (size_t)(row - BT::NCB / 2) * rowbytes
                                                                 : b0row + (size_t)row * rowbytes;
    const int ch = bch ^ ((row >> BT::SHIFT) & (BT::CPR - 1));
    load_lds16(base + gc * BT::ROWB + ch * 16, tile + (j * BT::RPT + (tid >> 6) * (64 / BT::CPR)) * BT::ROWB);
  };
  auto load_a_dl = [&](int kb, int i) {
    const int kc = kb < nkb ? kb : nkb - 1;
    load_lds16(adl[i] + kc * KBLK * 2, lds + (kb & (NSTAGE_DL - 1)) * STAGE_BYTES + (RPR * i + 8 * (tid >> 6)) * 128);
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
  // DL: a scale group's bytes (16 per weight row: KQ = 4 K-blocks) straight into scale tile
  // (group & 1), thread t filling tile row t (the gate rows, then the up rows); every lane
  // then reads its two columns' 16 bytes from there. Scale loads into registers would make
  // the compiler, which cannot see the asm loads, drain every load (vmcnt(0)) before using
  // them.
  char* stiles = btiles + 2 * BT::BYTES;
  const uint8_t* sdl = nullptr;
  if constexpr (DL) {
    const size_t srow0 = (size_t)tc.nb * (WPB * 32);
    sdl = tid < BT::NCB / 2 ? w0.scale_row(tc.e, srow0 + tid) : w1.scale_row(tc.e, srow0 + tid - BT::NCB / 2);
  }
  auto load_s_dl = [&](int j) {
    const int jc = j < ngrp ? j : ngrp - 1;
    load_lds16(sdl + jc * (4 * KQ), stiles + (j & 1) * (BT::NCB * 16) + (tid >> 6) * 1024);
  };
  auto read_s_dl = [&](int j, SRaw* q) {
    const char* t = stiles + (j & 1) * (BT::NCB * 16);
    q[0] = *reinterpret_cast<const SRaw*>(t + (wave * 32 + l32) * 16);
    q[1] = *reinterpret_cast<const SRaw*>(t + (BT::NCB / 2 + wave * 32 + l32) * 16);
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
  auto load_a = [&](int kb, int i) -> ARaw {
    const int kc = kb < nkb ? kb : nkb - 1;
    if constexpr (AM == A_F4)
      return make_uint2(*reinterpret_cast<const uint32_t*>(asrc[i] + kc * KBB),
                        *reinterpret_cast<const uint32_t*>(absrc[i] + kc * 4));
    else
      return *reinterpret_cast<const ARaw*>(asrc[i] + kc * KBB);
  };
  // the 8 fp16 values a thread stores for row arow + RPR*i of K-block kb
  auto a_fp16 = [&](const ARaw& v, int kb, int i) -> uint4 {
    if constexpr (AM == A_I8) {
      return __builtin_bit_cast(uint4, i8x8_f16(v.x, v.y));
    } else if constexpr (AM == A_F4) {
      const _Float16 sc = e4m3x2_f16<false>((v.y >> ashift) & 0xFFu)[0];
      return __builtin_bit_cast(uint4, bfrag(v.x, sc));
    } else if constexpr (!GATEUP) {
      const uint32_t m = f16_pow2_neg(s_hd[(arow + RPR * i) * kMaxHSeg + (kb >> seg_shift)]);
      const f16x2_t mm = __builtin_bit_cast(f16x2_t, m | (m << 16));
      return make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.x) * mm),
                        __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.y) * mm),
                        __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.z) * mm),
                        __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.w) * mm));
    } else {
      (void)kb;
      (void)i;
      return v;
    }
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
  ARaw aq[2][NA];
  uint4 bg[BT::CH];
  SRaw sq[2];
  if constexpr (DL) {
    // scale group 0, then the order of the loop's own issue (B group, then A): B(0) and
    // A(0), then A(1); the first group's scales are read once A(0) has landed
    load_s_dl(0);
#pragma unroll
    for (int j = 0; j < BT::CH; ++j) load_bg_dl(0, j, btiles);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int i = 0; i < NA; ++i) load_a_dl(d, i);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<NA>();
    __syncthreads();
    read_s_dl(0, sq);
  } else {
    sq[0] = load_s(0, 0);
    sq[1] = load_s(0, 1);
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
  }
  uint32_t sc0[KQ / 2], sc1[KQ / 2];
  compact(sq[0], sc0);
  compact(sq[1], sc1);

  auto kstep = [&](auto qpos, int kb) {
    constexpr int Q = decltype(qpos)::value;  // position in the scale group
    constexpr int R = Q & 1;                  // LDS stage / register ring slot
    char* st = lds + (DL ? Q : R) * STAGE_BYTES;
    if constexpr (DL) {
      // This wave's direct loads of A(kb) (and, at a group start, of the B group) are
      // complete once no more than the loads issued after them are outstanding: those of
      // the previous K-block (A(kb+1); its B group when it started one) and the scale load
      // issued between positions 1 and 2 of a scale group. Loads complete in order.
      constexpr int kAfter = NA + (((Q + 3) % 4) % GKB == 0 ? BT::CH : 0) + (Q == 2 ? 1 : 0);
      wait_vm<kAfter>();
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        *reinterpret_cast<uint4*>(st + (arow + RPR * i) * 128 + aslot) = a_fp16(aq[R][i], kb, i);
      // At a group start the staged B group goes to tile (group & 1): that tile was last
      // read in the group before the previous one, which every wave finished before passing
      // the previous group's first barrier.
      if constexpr (Q % GKB == 0) {
        char* bt = btiles + ((kb / GKB) & 1) * BT::BYTES;
#pragma unroll
        for (int j = 0; j < BT::CH; ++j) *reinterpret_cast<uint4*>(bt + BT::slot(j * BT::RPT + brow, bch)) = bg[j];
      }
    }
    // A(kb) (and the B group) visible to all waves. Stage R was last read in iteration
    // kb-2, and every wave finished those reads before passing the barrier of iteration
    // kb-1 (DL: the stage and tile the loads issued below fill were last read in K-block
    // kb-2 and in the previous group, both finished before this barrier).
    __syncthreads();
    // DL: the next scale group's bytes (loaded before position 2, so landed before this
    // barrier at position 3) into registers, compacted at the group's end
    if constexpr (DL && Q == 3) read_s_dl(kb / KQ + 1, sq);
    const char* btile = btiles + ((kb / GKB) & 1) * BT::BYTES;
    // The next B group (at a group start) and A(kb+2) are loaded spread over the MFMAs of
    // this K-block: a burst of loads from every wave right after the barrier queues in the
    // address unit and holds back each wave's first MFMAs.
    constexpr int NBL = (Q % GKB == 0) ? BT::CH : 0;
    constexpr int NLD = NBL + NA;
    auto issue_loads = [&](int idx, int nf) {
#pragma unroll
      for (int g = 0; g < NLD; ++g) {
        if (g * nf / NLD == idx) {
          if constexpr (DL) {
            if (g < NBL) load_bg_dl(kb / GKB + 1, g < NBL ? g : 0, btiles + ((kb / GKB + 1) & 1) * BT::BYTES);
            else load_a_dl(kb + 2, g - NBL);
          } else {
            if (g < NBL) bg[g < NBL ? g : 0] = load_bg(kb / GKB + 1, g < NBL ? g : 0);
            else aq[R][g - NBL] = load_a(kb + 2, g - NBL);
          }
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
    // step s+1 are unpacked between the MFMAs of step s into a second pair of registers.
    constexpr int NF = 4 * NRB, LA = 2;
    f16x8_t ring[LA + 1];
    auto read_a = [&](int idx) -> f16x8_t {
      const int s = idx / NRB, rb = idx % NRB;
      const int row = rb * 32 + l32, chunk = half * 4 + s;
      return *reinterpret_cast<const f16x8_t*>(st + row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4));
    };
#pragma unroll
    for (int i = 0; i < LA; ++i) ring[i] = read_a(i);
    f16x8_t b0 = bstep(cur0, cur0b, s0, 0);
    f16x8_t b1 = bstep(cur1, cur1b, s1, 0);
    f16x8_t n0 = b0, n1 = b1;
#pragma unroll
    for (int idx = 0; idx < NF; ++idx) {
      if (idx + LA < NF) ring[(idx + LA) % (LA + 1)] = read_a(idx + LA);
      issue_loads(idx, NF);
      __builtin_amdgcn_sched_barrier(0);
      const int s = idx / NRB, rb = idx % NRB;
      // gate/up: weights as the first operand (output-major accumulators, see the epilogue)
      if constexpr (GATEUP)
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, ring[idx % (LA + 1)], acc[rb][0], 0, 0, 0);
      else
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[idx % (LA + 1)], b0, acc[rb][0], 0, 0, 0);
      // the next step's fragments are unpacked between this step's MFMAs (column block 0
      // after row block 0, column block 1 after row block NRB / 2) into n0 / n1
      if (s < 3 && rb == 0) n0 = bstep(cur0, cur0b, s0, s + 1);
      if constexpr (GATEUP)
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, ring[idx % (LA + 1)], acc[rb][1], 0, 0, 0);
      else
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ring[idx % (LA + 1)], b1, acc[rb][1], 0, 0, 0);
      if (s < 3 && rb == NRB / 2) n1 = bstep(cur1, cur1b, s1, s + 1);
      if (rb == NRB - 1 && s < 3) {
        b0 = n0;
        b1 = n1;
      }
    }
  };
  // nkb is a multiple of KQ
  for (int j = 0; j < ngrp; ++j) {
    const int kb = j * KQ;
    if constexpr (KQ == 4) {
      kstep(std::integral_constant<int, 0>{}, kb);
      kstep(std::integral_constant<int, 1>{}, kb + 1);
      if constexpr (DL) {
        load_s_dl(j + 1);
      } else {
        sq[0] = load_s(j + 1, 0);
        sq[1] = load_s(j + 1, 1);
      }
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
  // DL: the loads issued past the last K-block (refetches, never read) land before the
  // block can end and its LDS be handed to another block
  if constexpr (DL) wait_vm<0>();

  if constexpr (GATEUP) {
    // The weights are the first MFMA operand, so element v of acc[rb][cb] is intermediate
    // index 8*(v/4) + 4*half + v%4 of the wave's 32, for token row rb*32 + l32: four
    // consecutive v are four adjacent h values of one row, stored as one 8-byte (fp16) or
    // 16-byte (fp32) piece straight to memory.
    const float gg = w0.gamma_nvfp4(tc.e), gu = w1.gamma_nvfp4(tc.e);
    const int col0 = tc.nb * (WPB * 32) + wave * 32 + 4 * half;
    float hv[NRB][16];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if constexpr (AM != A_F16) {
          const float xs = s_coef[r];
          hv[rb][v] = silu_fast(acc[rb][0][v] * (xs * gg)) * (acc[rb][1][v] * (xs * gu));
        } else {
          // g = gamma_g * 2^-e * acc: the gamma product rounds once, the power of two is exact
          const int ex = -s_exp[r];
          hv[rb][v] = silu_fast(__builtin_amdgcn_ldexpf(acc[rb][0][v] * gg, ex)) *
                      __builtin_amdgcn_ldexpf(acc[rb][1][v] * gu, ex);
        }
      }
    }
    // fp16 h (A_F16): each row of the block's WPB*32 intermediate indices is stored times
    // 2^eb, eb chosen so that the row's largest magnitude in this block lands in
    // [2^14, 2^15) (zero, infinite or NaN maxima take eb = 0); eb goes to hexp_out. The
    // block maximum is reduced over the two lane halves and then over the waves in LDS.
    int eb[NRB];
    if constexpr (!HOUT32) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float m = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) m = fmaxf(m, fabsf(hv[rb][v]));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (half == 0) s_red[wave * BM + rb * 32 + l32] = m;
      }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int r = rb * 32 + l32;
        float m = s_red[r];
#pragma unroll
        for (int w = 1; w < WPB; ++w) m = fmaxf(m, s_red[w * BM + r]);
        eb[rb] = (m > 0.f && m <= 3.402823466e38f) ? 15 - __builtin_amdgcn_frexp_expf(m) : 0;
        if (wave == 0 && half == 0 && r < tc.rows) hexp_out[(size_t)(tc.base + tc.m0 + r) * NB + tc.nb] = eb[rb];
      }
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 32 + l32;
      const size_t rowoff = (size_t)(tc.base + tc.m0 + r) * ldo + col0;
      if (r < tc.rows) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if constexpr (HOUT32) {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + rowoff + 8 * g) =
                f32x4_t{hv[rb][4 * g], hv[rb][4 * g + 1], hv[rb][4 * g + 2], hv[rb][4 * g + 3]};
          } else {
            uint32_t pk[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
              pk[j] = (uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(hv[rb][4 * g + 2 * j], eb[rb])) |
                      ((uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(hv[rb][4 * g + 2 * j + 1], eb[rb])) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + rowoff + 8 * g) = make_uint2(pk[0], pk[1]);
          }
        }
      }
    }
  } else {
    // y[pos][n] = gamma_d * coef[pos] * acc (A_F16: times 2^-e of the row, by ldexp), fp32,
    // in sorted order; the combine kernel sums each token's slots. One row block at a time
    // goes through LDS ([32][NCOL] fp32, 16-byte chunks XOR-swizzled by row), so every
    // store is a full 16 bytes and a wave writes whole 1 KB row segments; the stores are
    // non-temporal (y is read once, by the combine). The kernel's LDS holds
    // 32 * NCOL * 4 bytes.
    constexpr int NCOL = WPB * 64;
    const float gd = w0.gamma(tc.e);  // a Q8_0 down may have no tensor scale (1)
    float* y = reinterpret_cast<float*>(out);
    float* yl = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      __syncthreads();  // the A stages / the previous row block are no longer read
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = (i >> 2) * 8 + half * 4 + (i & 3);
        const float c = s_coef[rb * 32 + rr] * gd;
        const int ex = AM == A_F16 ? -s_exp[rb * 32 + rr] : 0;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int col = wave * 64 + cb * 32 + l32;
          float v = acc[rb][cb][i] * c;
          if constexpr (AM == A_F16) v = __builtin_amdgcn_ldexpf(v, ex);
          yl[rr * NCOL + (((col >> 2) ^ (rr & 7)) << 2) + (col & 3)] = v;
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
// AM: the activation mode (A_F16, A_I8 or A_F4, above).
// a_scale: A_I8 / A_F4 row scales (gate/up: per token; down: per sorted position).
// a_bscale: A_F4 block scales (E4M3, one per 16 inputs of a row).
// a_exp: A_F16 exponents (gate/up: per token; down: per sorted position and gate/up block,
// [P][nbh], whose blocks span 2^seg_shift K-blocks of the down GEMM).
// hexp_out: gate/up A_F16 only, the exponents of the fp16 h it writes ([P][NB]).
template <bool GATEUP, int AM, int KQ, int WPB, int GK, bool Q8 = false>
__global__ __launch_bounds__(WPB * 64, 8 / WPB) void moe_gemm_f16_kernel(
    const void* __restrict__ A, const float* __restrict__ a_scale, const uint8_t* __restrict__ a_bscale,
    const int32_t* __restrict__ a_exp, int nbh,
    int seg_shift, const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ offsets,
    const TileDesc* __restrict__ tiles, const int32_t* __restrict__ tile_count, int topk, int K, int NB,
    WeightArgs w0, WeightArgs w1, const float* __restrict__ route_w, void* __restrict__ out, int ldo,
    int32_t* __restrict__ hexp_out) {
  // A stages and the B tile; the down epilogue reuses them (32 rows x WPB*64 fp32)
  constexpr bool kDl = direct_lds<GATEUP, AM, KQ, Q8>();
  constexpr int kMain = (kDl ? NSTAGE_DL : NSTAGE) * STAGE_BYTES + 2 * BTile<WPB, Q8 ? 2 : GK>::BYTES +
                        (kDl ? 2 * WPB * 64 * 16 : 0);  // + the two scale tiles
  constexpr int kEpi = GATEUP ? 0 : 32 * WPB * 64 * 4;
  constexpr int kLds = kMain > kEpi ? kMain : kEpi;
  constexpr bool kHd = !GATEUP && AM == A_F16;    // down rescales A per gate/up block
  constexpr bool kRed = GATEUP && AM == A_F16;    // gate/up reduces the row maxima of h
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ int s_src[BM];
  __shared__ float s_coef[BM];
  __shared__ int s_exp[BM];
  __shared__ uint8_t s_hd[kHd ? BM * kMaxHSeg : 1];
  __shared__ float s_red[kRed ? WPB * BM : 1];

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
      s_coef[tid] = AM != A_F16 ? a_scale[p / topk] : 1.0f;
      s_exp[tid] = AM == A_F16 ? a_exp[p / topk] : 0;
    } else {
      s_src[tid] = pos;
      s_coef[tid] = route_w[p] * (AM != A_F16 ? a_scale[pos] : 1.0f);
      if constexpr (kHd) {
        // the row's smallest exponent (its largest block), and each block's shift down to it
        const int32_t* ex = a_exp + (size_t)pos * nbh;
        int emin = ex[0];
        for (int b = 1; b < nbh; ++b) emin = min(emin, ex[b]);
        for (int b = 0; b < nbh; ++b) s_hd[tid * kMaxHSeg + b] = (uint8_t)min(ex[b] - emin, 31);
        s_exp[tid] = emin;
      } else {
        s_exp[tid] = 0;
      }
    }
  }

  // first weight row of the block in each tensor; per-lane scale rows of its fragments
  const uint8_t* b0row;
  const uint8_t* b1row;
  const uint8_t* bs[2];
  if (GATEUP) {
    const size_t row0 = (size_t)tc.nb * (WPB * 32);
    b0row = w0.code_row(tc.e, row0, K / 2);
    b1row = w1.code_row(tc.e, row0, K / 2);
    bs[0] = w0.scale_row(tc.e, row0 + wave * 32 + l32);
    bs[1] = w1.scale_row(tc.e, row0 + wave * 32 + l32);
  } else {
    const size_t row0 = (size_t)tc.nb * (WPB * 64);
    b0row = w0.code_row(tc.e, row0, Q8 ? K : K / 2);
    b1row = b0row;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) bs[cb] = w0.scale_row(tc.e, row0 + wave * 64 + cb * 32 + l32);
  }
  __syncthreads();

  const int nrb = (tc.rows + 31) >> 5;
#define NVFP4_TILE(R)                                                                                            \
  gemm_tile<GATEUP, AM, R, KQ, WPB, GK, Q8>(tc, A, a_bscale, K, b0row, b1row, bs, w0, w1, out, ldo, lds, s_src, s_coef, \
                                            s_exp, s_hd, seg_shift, s_red, hexp_out, NB)
  if (nrb == 4)
    NVFP4_TILE(4);
  else if (nrb == 3)
    NVFP4_TILE(3);
  else if (nrb == 2)
    NVFP4_TILE(2);
  else
    NVFP4_TILE(1);
#undef NVFP4_TILE
}

static inline unsigned grid_for(int max_tiles, int NB) {
  const long long g = (long long)max_tiles * NB;
  return (unsigned)(((g + 7) / 8) * 8);
}

hipError_t launch_gemm_gateup(int act, const void* a, const float* a_scale, const uint8_t* a_bscale,
                              const int32_t* a_exp,
                              const int32_t* sorted_pairs, const int32_t* offsets, const TileDesc* tiles,
                              const int32_t* tile_count, int max_tiles, int topk, int H, int I,
                              const WeightArgs& gate, const WeightArgs& up, void* h, int32_t* hexp,
                              hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  // 8 waves (256 intermediate indices per block) when I allows, else 4 (128); H is a
  // multiple of 256, so scale groups of 4 K-blocks; B groups of 2 K-blocks.
#define NVFP4_GU(AM, WPB)                                                                                  \
  moe_gemm_f16_kernel<true, AM, 4, WPB, 2><<<grid_for(max_tiles, I / (WPB * 32)), WPB * 64, 0, st>>>(      \
      a, a_scale, a_bscale, a_exp, 0, 0, sorted_pairs, offsets, tiles, tile_count, topk, H, I / (WPB * 32), \
      gate, up, nullptr, h, I, hexp)
  const bool w8 = I % 256 == 0;
  if (act == 0) {
    if (w8)
      NVFP4_GU(A_F16, 8);
    else
      NVFP4_GU(A_F16, 4);
  } else if (act == 1) {
    if (w8)
      NVFP4_GU(A_I8, 8);
    else
      NVFP4_GU(A_I8, 4);
  } else {
    if (w8)
      NVFP4_GU(A_F4, 8);
    else
      NVFP4_GU(A_F4, 4);
  }
#undef NVFP4_GU
  return hipGetLastError();
}

int gateup_blocks(int I) { return I % 256 == 0 ? I / 256 : I / 128; }

hipError_t launch_gemm_down(int act, const void* h, const float* h_scale, const uint8_t* h_bscale,
                            const int32_t* hexp,
                            const int32_t* sorted_pairs, const int32_t* offsets, const TileDesc* tiles,
                            const int32_t* tile_count, int max_tiles, int topk, int H, int I,
                            const WeightArgs& down, const float* w, float* y, hipStream_t st) {
  if (max_tiles == 0) return hipSuccess;
  // fp16 h: one exponent per gate/up block of 256 (or 128) intermediate indices, i.e. per
  // 4 (or 2) K-blocks of this GEMM
  const int nbh = gateup_blocks(I);
  const int seg_shift = I % 256 == 0 ? 2 : 1;
  // 8 waves (512 outputs per block) when H allows, else 4 (256); scale groups of 4
  // K-blocks when I is a multiple of 256, else 2; B groups of 2 K-blocks.
#define NVFP4_DOWN(AM, KQ, WPB)                                                                             \
  do {                                                                                                      \
    const dim3 grid = grid_for(max_tiles, H / (WPB * 64));                                                  \
    if (down.fmt == 1)                                                                                      \
      moe_gemm_f16_kernel<false, AM, KQ, WPB, 2, true><<<grid, WPB * 64, 0, st>>>(                          \
          h, h_scale, h_bscale, hexp, nbh, seg_shift, sorted_pairs, offsets, tiles, tile_count, topk, I,     \
          H / (WPB * 64),                                                                                   \
          down, down, w, y, H, nullptr);                                                                    \
    else                                                                                                    \
      moe_gemm_f16_kernel<false, AM, KQ, WPB, 2><<<grid, WPB * 64, 0, st>>>(                                \
          h, h_scale, h_bscale, hexp, nbh, seg_shift, sorted_pairs, offsets, tiles, tile_count, topk, I,     \
          H / (WPB * 64),                                                                                   \
          down, down, w, y, H, nullptr);                                                                    \
  } while (0)
#define NVFP4_DOWN_W(AM, KQ) \
  if (H % 512 == 0)          \
    NVFP4_DOWN(AM, KQ, 8);   \
  else                       \
    NVFP4_DOWN(AM, KQ, 4);
  const bool q4 = I % 256 == 0;
  if (act == 0) {
    if (q4) {
      NVFP4_DOWN_W(A_F16, 4)
    } else {
      NVFP4_DOWN_W(A_F16, 2)
    }
  } else if (act == 1) {
    if (q4) {
      NVFP4_DOWN_W(A_I8, 4)
    } else {
      NVFP4_DOWN_W(A_I8, 2)
    }
  } else {
    if (q4) {
      NVFP4_DOWN_W(A_F4, 4)
    } else {
      NVFP4_DOWN_W(A_F4, 2)
    }
  }
#undef NVFP4_DOWN_W
#undef NVFP4_DOWN
  return hipGetLastError();
}

}  // namespace nvfp4

// Host-CPU share of the routed experts ("Strata NVFP4" README: AVX-512 NVFP4 kernels for
// the CPU share of the experts, an AVX2 path on CPUs without AVX-512, that share read from
// host DRAM). The projection is the decode path's: every weight decoded exactly (an E2M1
// value times its E4M3 scale, or a Q8_0 int8 times its fp16 scale, is exact in fp32), FP32
// dot products, the FP32 global scale at each projection's output, SwiGLU in FP32, h kept
// in FP32, and the routed pairs added into each output row in a fixed order.
//
// Work split: phase 1 hands out (unique expert, 16 intermediate rows) units and writes
// h[pair][I]; phase 2 hands out 16-row blocks of the output, and each block adds its pairs
// unique expert by unique expert (order of first appearance), pairs in pair order. Which
// thread runs a unit never changes a value, so results do not depend on the thread count.
// Each weight row is read once per batch of up to 8 pairs that share its expert.
//
// Built by the host compiler for baseline x86-64; the AVX2 and AVX-512 row kernels carry
// their own target attributes and are chosen at run time from what the CPU reports.
#include "host.h"

#include <immintrin.h>
#include <sched.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace nvfp4 {
namespace host {
namespace {

constexpr int kRows = 8;  // pairs that share one read of a weight row

// ------------------------------------------------------------------ element decoding
alignas(64) constexpr float kE2M1[16] = {0.f,  0.5f,  1.f,  1.5f,  2.f,  3.f,  4.f,  6.f,
                                         -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};
alignas(32) constexpr float kE2M1Mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};

// E4M3 (bias 7, no infinities, S.1111.111 is NaN): every byte as fp32.
struct E4M3Table {
  float v[256];
  E4M3Table() {
    for (int b = 0; b < 256; ++b) {
      const int e = (b >> 3) & 15, m = b & 7;
      float f;
      if ((b & 0x7F) == 0x7F) f = std::nanf("");
      else if (e == 0) f = std::ldexp((float)m, -9);
      else f = std::ldexp(1.f + m / 8.f, e - 7);
      v[b] = (b & 0x80) ? -f : f;
    }
  }
};
const E4M3Table kE4M3;

// IEEE binary16 bits to fp32 (exact).
inline float half_bits_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  float f;
  if (e == 0) {
    f = std::ldexp((float)m, -24);
  } else if (e == 31) {
    const uint32_t u = 0x7F800000u | (m << 13);
    std::memcpy(&f, &u, 4);
  } else {
    f = std::ldexp((float)(1024 + m), (int)e - 25);
  }
  return sign ? -f : f;
}

inline float bf16_bits_to_float(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ------------------------------------------------------------------ row kernels
// y[q] = sum_k W[k] * x[q][k] for one weight row and NR input rows (NR <= kRows).
// NVFP4 row: codes K/2 bytes (input 2j in the low nibble of byte j), scales K/16 bytes.
// Q8_0 row: codes K int8, scales K/32 fp16.
typedef void (*DotFn)(const uint8_t*, const uint8_t*, const float* const*, int, float*);

template <int NR>
void dot_nvfp4_portable(const uint8_t* c, const uint8_t* s, const float* const* x, int K, float* y) {
  float acc[NR] = {};
  for (int g = 0; g < K / 16; ++g) {
    const float sc = kE4M3.v[s[g]];
    for (int j = 0; j < 16; ++j) {
      const float w = kE2M1[(c[g * 8 + j / 2] >> (4 * (j & 1))) & 15] * sc;  // exact
      for (int q = 0; q < NR; ++q) acc[q] += w * x[q][g * 16 + j];
    }
  }
  for (int q = 0; q < NR; ++q) y[q] = acc[q];
}

template <int NR>
void dot_q8_portable(const uint8_t* c, const uint8_t* s, const float* const* x, int K, float* y) {
  float acc[NR] = {};
  for (int b = 0; b < K / 32; ++b) {
    uint16_t hb;
    std::memcpy(&hb, s + 2 * b, 2);
    const float d = half_bits_to_float(hb);
    for (int j = 0; j < 32; ++j) {
      const float w = (float)(int8_t)c[b * 32 + j] * d;  // exact: 11 x 8 significant bits
      for (int q = 0; q < NR; ++q) acc[q] += w * x[q][b * 32 + j];
    }
  }
  for (int q = 0; q < NR; ++q) y[q] = acc[q];
}

#define AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx512dq")))
#define AVX2 __attribute__((target("avx2,fma")))

// AVX-512 NVFP4 rows take their input in "pair order": within each group of 16 inputs,
// position 2m holds input m and position 2m+1 input 8+m. Then one 8-byte broadcast of a
// group's codes and one per-lane shift leave nibble m of the low dword in lane 2m and
// nibble m of the high dword in lane 2m+1, a 16-lane permute (it reads index bits 0..3)
// maps them to values, and no byte unpacking is needed. Two FMA chains per input row.
inline int pair_order(int k) {
  const int j = k & 15;
  return (k & ~15) | (j < 8 ? 2 * j : 2 * (j - 8) + 1);
}

template <int NR>
AVX512 void dot_nvfp4_avx512(const uint8_t* c, const uint8_t* s, const float* const* x, int K, float* y) {
  const __m512 lut = _mm512_load_ps(kE2M1);
  const __m512i shift = _mm512_set_epi32(28, 28, 24, 24, 20, 20, 16, 16, 12, 12, 8, 8, 4, 4, 0, 0);
  __m512 a0[NR], a1[NR];
  for (int q = 0; q < NR; ++q) a0[q] = a1[q] = _mm512_setzero_ps();
  for (int g = 0; g < K / 16; g += 2) {
    long long q0, q1;
    std::memcpy(&q0, c + g * 8, 8);
    std::memcpy(&q1, c + g * 8 + 8, 8);
    const __m512 w0 = _mm512_mul_ps(_mm512_permutexvar_ps(_mm512_srlv_epi32(_mm512_set1_epi64(q0), shift), lut),
                                    _mm512_set1_ps(kE4M3.v[s[g]]));
    const __m512 w1 = _mm512_mul_ps(_mm512_permutexvar_ps(_mm512_srlv_epi32(_mm512_set1_epi64(q1), shift), lut),
                                    _mm512_set1_ps(kE4M3.v[s[g + 1]]));
    for (int q = 0; q < NR; ++q) {
      a0[q] = _mm512_fmadd_ps(w0, _mm512_loadu_ps(x[q] + g * 16), a0[q]);
      a1[q] = _mm512_fmadd_ps(w1, _mm512_loadu_ps(x[q] + g * 16 + 16), a1[q]);
    }
  }
  for (int q = 0; q < NR; ++q) y[q] = _mm512_reduce_add_ps(_mm512_add_ps(a0[q], a1[q]));
}

template <int NR>
AVX512 void dot_q8_avx512(const uint8_t* c, const uint8_t* s, const float* const* x, int K, float* y) {
  __m512 a0[NR], a1[NR];
  for (int q = 0; q < NR; ++q) a0[q] = a1[q] = _mm512_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {
    uint16_t hb;
    std::memcpy(&hb, s + 2 * b, 2);
    const __m512 d = _mm512_set1_ps(half_bits_to_float(hb));
    const __m128i c0 = _mm_loadu_si128(reinterpret_cast<const __m128i*>(c + b * 32));
    const __m128i c1 = _mm_loadu_si128(reinterpret_cast<const __m128i*>(c + b * 32 + 16));
    const __m512 w0 = _mm512_mul_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(c0)), d);
    const __m512 w1 = _mm512_mul_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(c1)), d);
    for (int q = 0; q < NR; ++q) {
      a0[q] = _mm512_fmadd_ps(w0, _mm512_loadu_ps(x[q] + b * 32), a0[q]);
      a1[q] = _mm512_fmadd_ps(w1, _mm512_loadu_ps(x[q] + b * 32 + 16), a1[q]);
    }
  }
  for (int q = 0; q < NR; ++q) y[q] = _mm512_reduce_add_ps(_mm512_add_ps(a0[q], a1[q]));
}

AVX2 inline float hsum256(__m256 v) {
  __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  s = _mm_add_ps(s, _mm_movehl_ps(s, s));
  s = _mm_add_ss(s, _mm_shuffle_ps(s, s, 1));
  return _mm_cvtss_f32(s);
}

// 8 inputs from one code dword: lane i shifted right by 4i holds nibble i (input i) in
// its low bits; magnitude by an 8-lane permute (it reads index bits 0..2), sign from index
// bit 3 moved to bit 31.
AVX2 inline __m256 e2m1x8(uint32_t codes, __m256 mag) {
  const __m256i idx = _mm256_srlv_epi32(_mm256_set1_epi32((int)codes), _mm256_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28));
  const __m256i sgn = _mm256_and_si256(_mm256_slli_epi32(idx, 28), _mm256_set1_epi32((int)0x80000000u));
  return _mm256_or_ps(_mm256_permutevar8x32_ps(mag, idx), _mm256_castsi256_ps(sgn));
}

template <int NR>
AVX2 void dot_nvfp4_avx2(const uint8_t* c, const uint8_t* s, const float* const* x, int K, float* y) {
  const __m256 mag = _mm256_load_ps(kE2M1Mag);
  __m256 a0[NR], a1[NR];
  for (int q = 0; q < NR; ++q) a0[q] = a1[q] = _mm256_setzero_ps();
  for (int g = 0; g < K / 16; ++g) {
    uint32_t d0, d1;
    std::memcpy(&d0, c + g * 8, 4);
    std::memcpy(&d1, c + g * 8 + 4, 4);
    const __m256 sc = _mm256_set1_ps(kE4M3.v[s[g]]);
    const __m256 w0 = _mm256_mul_ps(e2m1x8(d0, mag), sc);
    const __m256 w1 = _mm256_mul_ps(e2m1x8(d1, mag), sc);
    for (int q = 0; q < NR; ++q) {
      const float* xp = x[q] + g * 16;
      a0[q] = _mm256_fmadd_ps(w0, _mm256_loadu_ps(xp), a0[q]);
      a1[q] = _mm256_fmadd_ps(w1, _mm256_loadu_ps(xp + 8), a1[q]);
    }
  }
  for (int q = 0; q < NR; ++q) y[q] = hsum256(_mm256_add_ps(a0[q], a1[q]));
}

template <int NR>
AVX2 void dot_q8_avx2(const uint8_t* c, const uint8_t* s, const float* const* x, int K, float* y) {
  __m256 a0[NR], a1[NR];
  for (int q = 0; q < NR; ++q) a0[q] = a1[q] = _mm256_setzero_ps();
  for (int b = 0; b < K / 32; ++b) {
    uint16_t hb;
    std::memcpy(&hb, s + 2 * b, 2);
    const __m256 d = _mm256_set1_ps(half_bits_to_float(hb));
    __m256 w[4];
    for (int i = 0; i < 4; ++i) {
      const __m128i ci = _mm_loadl_epi64(reinterpret_cast<const __m128i*>(c + b * 32 + 8 * i));
      w[i] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(ci)), d);
    }
    for (int q = 0; q < NR; ++q) {
      const float* xp = x[q] + b * 32;
      a0[q] = _mm256_fmadd_ps(w[0], _mm256_loadu_ps(xp), a0[q]);
      a1[q] = _mm256_fmadd_ps(w[1], _mm256_loadu_ps(xp + 8), a1[q]);
      a0[q] = _mm256_fmadd_ps(w[2], _mm256_loadu_ps(xp + 16), a0[q]);
      a1[q] = _mm256_fmadd_ps(w[3], _mm256_loadu_ps(xp + 24), a1[q]);
    }
  }
  for (int q = 0; q < NR; ++q) y[q] = hsum256(_mm256_add_ps(a0[q], a1[q]));
}

// Row-kernel table: [format][isa - 1][rows - 1].
#define ROW_TABLE(fn) {fn<1>, fn<2>, fn<3>, fn<4>, fn<5>, fn<6>, fn<7>, fn<8>}
const DotFn kDot[2][3][kRows] = {
    {ROW_TABLE(dot_nvfp4_portable), ROW_TABLE(dot_nvfp4_avx2), ROW_TABLE(dot_nvfp4_avx512)},
    {ROW_TABLE(dot_q8_portable), ROW_TABLE(dot_q8_avx2), ROW_TABLE(dot_q8_avx512)},
};
#undef ROW_TABLE

inline void row_ptrs(const Weight& w, int e, int r, const uint8_t** c, const uint8_t** s) {
  const size_t row = (size_t)e * w.N + r;
  if (w.fmt == 1) {
    *c = w.codes + row * (size_t)w.K;
    *s = w.scales + row * (size_t)(w.K / 32) * 2;
  } else {
    *c = w.codes + row * (size_t)(w.K / 2);
    *s = w.scales + row * (size_t)(w.K / 16);
  }
}

// ------------------------------------------------------------------ thread pool
// Persistent workers, created on first use and kept for the life of the process (a
// forked child starts a pool of its own). One job at a time; the calling thread works too.
// A job is published as one atomic word (generation << 16 | helper count), so a worker
// decides from a single snapshot whether it takes part; workers take the caller's MXCSR
// (denormal and rounding modes), so every unit is computed the same way on any thread. Idle workers spin for a short
// while before they sleep, since decode calls come back to back and a sleeping thread
// takes tens of microseconds to wake.
class Pool {
 public:
  void run(int n, int threads, const std::function<void(int)>& f) {
    std::lock_guard<std::mutex> one_job(call_mu_);
    threads = std::max(1, std::min({threads, n, kMaxThreads}));
    if (threads == 1) {
      for (int i = 0; i < n; ++i) f(i);
      return;
    }
    while (started_ < threads - 1) {  // counted only once running (creation may throw)
      std::thread([this, id = started_] { loop(id); }).detach();
      ++started_;
    }
    job_.store(&f, std::memory_order_relaxed);
    n_.store(n, std::memory_order_relaxed);
    csr_.store(_mm_getcsr(), std::memory_order_relaxed);  // the caller's denormal and rounding modes
    next_.store(0, std::memory_order_relaxed);
    busy_.store(threads - 1, std::memory_order_relaxed);
    {
      std::lock_guard<std::mutex> lk(mu_);  // a worker about to sleep sees the new word or is woken
      const uint64_t gen = (state_.load(std::memory_order_relaxed) >> 16) + 1;
      state_.store(gen << 16 | (uint64_t)(threads - 1), std::memory_order_release);
    }
    if (sleepers_.load(std::memory_order_acquire) > 0) cv_.notify_all();
    drain(f, n);
    while (busy_.load(std::memory_order_acquire) != 0) _mm_pause();
  }

 private:
  static constexpr int kMaxThreads = 1024;
  static constexpr int kSpin = 1 << 14;

  void drain(const std::function<void(int)>& f, int n) {
    for (int i; (i = next_.fetch_add(1, std::memory_order_relaxed)) < n;) f(i);
  }
  void loop(int id) {
    uint64_t seen = 0;
    for (;;) {
      uint64_t st = state_.load(std::memory_order_acquire);
      for (int i = 0; (st >> 16) == (seen >> 16) && i < kSpin; ++i) {
        _mm_pause();
        st = state_.load(std::memory_order_acquire);
      }
      if ((st >> 16) == (seen >> 16)) {
        std::unique_lock<std::mutex> lk(mu_);
        sleepers_.fetch_add(1, std::memory_order_acq_rel);
        cv_.wait(lk, [&] { return (state_.load(std::memory_order_acquire) >> 16) != (seen >> 16); });
        sleepers_.fetch_sub(1, std::memory_order_acq_rel);
        st = state_.load(std::memory_order_acquire);
      }
      seen = st;
      if (id >= (int)(st & 0xFFFF)) continue;  // not a helper of this job
      _mm_setcsr(csr_.load(std::memory_order_relaxed));
      drain(*job_.load(std::memory_order_relaxed), n_.load(std::memory_order_relaxed));
      busy_.fetch_sub(1, std::memory_order_release);
    }
  }

  std::mutex call_mu_, mu_;
  std::condition_variable cv_;
  std::atomic<uint64_t> state_{0};
  std::atomic<const std::function<void(int)>*> job_{nullptr};
  std::atomic<int> n_{0}, next_{0}, busy_{0}, sleepers_{0};
  std::atomic<unsigned> csr_{0};
  int started_ = 0;
};

Pool& pool() {
  static std::mutex mu;
  static Pool* p = nullptr;
  static pid_t owner = 0;
  std::lock_guard<std::mutex> lk(mu);
  if (!p || owner != getpid()) {  // never freed: detached workers wait on it until exit
    p = new Pool;
    owner = getpid();
  }
  return *p;
}

int default_threads() {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) return std::max(1, CPU_COUNT(&set));
  return std::max(1u, std::thread::hardware_concurrency());
}

}  // namespace

int best_isa() {
  static const int isa = [] {
    __builtin_cpu_init();
    if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
        __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq"))
      return (int)kIsaAvx512;
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return (int)kIsaAvx2;
    return (int)kIsaPortable;
  }();
  return isa;
}

int64_t moe_decode(const void* x, int x_dtype, int T, int H, int I, const Weight& gate, const Weight& up,
                   const Weight& down, int E, const int32_t* ids, const float* wts, int topk, float* out,
                   int nthreads, int isa) {
  const int64_t P = (int64_t)T * topk;
  const int level = (isa == kIsaAuto ? best_isa() : isa) - 1;
  const DotFn* dgu = kDot[0][level];
  const DotFn* ddn = kDot[down.fmt == 1 ? 1 : 0][level];
  nthreads = nthreads <= 0 ? default_threads() : std::min(nthreads, default_threads());

  // inputs of the AVX-512 NVFP4 rows are stored in pair order (x here, h in phase 1)
  const bool px = level == kIsaAvx512 - 1, ph = px && down.fmt == 0;

  // activations in fp32 (bf16 widens exactly)
  std::vector<float> xf((size_t)T * H);
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < H; ++k) {
      const size_t i = (size_t)t * H + k;
      xf[(size_t)t * H + (px ? pair_order(k) : k)] =
          x_dtype == 1 ? bf16_bits_to_float(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
    }

  // pairs grouped by expert: unique experts in order of first appearance, pairs in order
  std::vector<int> uniq, start, list;
  int64_t dropped = 0;
  {
    std::vector<int> slot(E, -1), count;
    for (int64_t p = 0; p < P; ++p) {
      const int e = ids[p];
      if (e < 0 || e >= E) {
        ++dropped;
        continue;
      }
      if (slot[e] < 0) {
        slot[e] = (int)uniq.size();
        uniq.push_back(e);
        count.push_back(0);
      }
      ++count[slot[e]];
    }
    start.assign(uniq.size() + 1, 0);
    for (size_t u = 0; u < uniq.size(); ++u) start[u + 1] = start[u] + count[u];
    list.resize(start.back());
    std::vector<int> fill(start.begin(), start.end() - 1);
    for (int64_t p = 0; p < P; ++p) {
      const int e = ids[p];
      if (e >= 0 && e < E) list[fill[slot[e]]++] = (int)p;
    }
  }
  const int U = (int)uniq.size();
  std::fill(out, out + (size_t)T * H, 0.f);
  if (U == 0) return dropped;

  // phase 1: h[p][i] = SiLU(gate) * up for every valid pair
  std::vector<float> h((size_t)P * I);
  const int rb1 = (I + 15) / 16;
  pool().run(U * rb1, nthreads, [&](int j) {
    const int u = j / rb1, r0 = (j % rb1) * 16, r1 = std::min(I, r0 + 16);
    const int e = uniq[u];
    const float gg = gate.global[e], gu = up.global[e];
    for (int i0 = start[u]; i0 < start[u + 1]; i0 += kRows) {
      const int n = std::min(kRows, start[u + 1] - i0);
      const float* xr[kRows];
      for (int q = 0; q < n; ++q) xr[q] = xf.data() + (size_t)(list[i0 + q] / topk) * H;
      for (int r = r0; r < r1; ++r) {
        const uint8_t *gc, *gs, *uc, *us;
        row_ptrs(gate, e, r, &gc, &gs);
        row_ptrs(up, e, r, &uc, &us);
        float g[kRows], v[kRows];
        dgu[n - 1](gc, gs, xr, H, g);
        dgu[n - 1](uc, us, xr, H, v);
        for (int q = 0; q < n; ++q) {
          const float z = g[q] * gg;
          h[(size_t)list[i0 + q] * I + (ph ? pair_order(r) : r)] = z / (1.f + std::exp(-z)) * (v[q] * gu);
        }
      }
    }
  });

  // phase 2: 16-row blocks of out; pairs added unique expert by unique expert, in pair order
  const int rb2 = (H + 15) / 16;
  pool().run(rb2, nthreads, [&](int j) {
    const int r0 = j * 16, r1 = std::min(H, r0 + 16);
    for (int u = 0; u < U; ++u) {
      const int e = uniq[u];
      const float gd = down.global ? down.global[e] : 1.f;
      for (int i0 = start[u]; i0 < start[u + 1]; i0 += kRows) {
        const int n = std::min(kRows, start[u + 1] - i0);
        const float* hr[kRows];
        for (int q = 0; q < n; ++q) hr[q] = h.data() + (size_t)list[i0 + q] * I;
        for (int r = r0; r < r1; ++r) {
          const uint8_t *dc, *ds;
          row_ptrs(down, e, r, &dc, &ds);
          float y[kRows];
          ddn[n - 1](dc, ds, hr, I, y);
          for (int q = 0; q < n; ++q) {
            const int p = list[i0 + q];
            out[(size_t)(p / topk) * H + r] += wts[p] * (gd * y[q]);
          }
        }
      }
    }
  });
  return dropped;
}

}  // namespace host
}  // namespace nvfp4

// Host expert executor: the CPU branch of a decode step.
//
// [FT] = "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
// Execution" (arXiv 2608.16157).  [FT] §3.2: experts of the CPU set C execute in
// place from the host-resident pool and return gate-weighted per-token partial
// outputs, concurrently with the GPU path.  [FT] §4.1 "Graph-resident CPU
// execution": a persistent pool of workers pinned to cores, with SIMD kernels
// that stay bound by host memory bandwidth.
//
// Work of one call: phase 1 computes h = silu(W_gate x) * (W_up x) for every
// (expert, use) with rows of W_gate/W_up dealt to workers in blocks; phase 2
// computes partial[t][c] = sum over the uses (expert, t, gate) of
// gate * (W_down[c] . h) with output rows dealt in blocks, so every output row
// is owned by one worker.  Each weight row is read once and applied to all the
// uses of its expert.  MXFP4 records (OCP MX v1.0: E2M1 codes, one E8M0 scale per
// 32 consecutive elements of a row) are dequantised in registers through a
// 16-entry table, exactly (every E2M1 value times a power of two is an fp32).
#include <immintrin.h>
#include <pthread.h>
#include <sched.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "internal.h"

namespace ft {
namespace {

constexpr int MAXV = 8;  // activation vectors applied per weight row pass

using RowDotsFn = void (*)(const uint16_t* w, int n, const float* const* xs, int nx, float* out);

void row_dots_scalar(const uint16_t* w, int n, const float* const* xs, int nx, float* out) {
  float acc[MAXV] = {0};
  for (int i = 0; i < n; ++i) {
    uint32_t u = (uint32_t)w[i] << 16;
    float wf;
    std::memcpy(&wf, &u, 4);
    for (int v = 0; v < nx; ++v) acc[v] += wf * xs[v][i];
  }
  for (int v = 0; v < nx; ++v) out[v] = acc[v];
}

__attribute__((target("avx2,fma"))) void row_dots_avx2(const uint16_t* w, int n,
                                                         const float* const* xs, int nx,
                                                         float* out) {
  __m256 acc[MAXV];
  for (int v = 0; v < MAXV; ++v) acc[v] = _mm256_setzero_ps();
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    const __m128i a = _mm_loadu_si128(reinterpret_cast<const __m128i*>(w + i));
    const __m256 wf = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(a), 16));
    for (int v = 0; v < nx; ++v) acc[v] = _mm256_fmadd_ps(wf, _mm256_loadu_ps(xs[v] + i), acc[v]);
  }
  for (int v = 0; v < nx; ++v) {
    __m128 s = _mm_add_ps(_mm256_castps256_ps128(acc[v]), _mm256_extractf128_ps(acc[v], 1));
    s = _mm_hadd_ps(s, s);
    s = _mm_hadd_ps(s, s);
    float r = _mm_cvtss_f32(s);
    for (int j = i; j < n; ++j) {
      uint32_t u = (uint32_t)w[j] << 16;
      float wf;
      std::memcpy(&wf, &u, 4);
      r += wf * xs[v][j];
    }
    out[v] = r;
  }
}

__attribute__((target("avx512f,avx512bw"))) void row_dots_avx512(const uint16_t* w, int n,
                                                                   const float* const* xs, int nx,
                                                                   float* out) {
  __m512 acc[MAXV];
  for (int v = 0; v < MAXV; ++v) acc[v] = _mm512_setzero_ps();
  int i = 0;
  for (; i + 16 <= n; i += 16) {
    const __m256i a = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + i));
    const __m512 wf = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(a), 16));
    for (int v = 0; v < nx; ++v) acc[v] = _mm512_fmadd_ps(wf, _mm512_loadu_ps(xs[v] + i), acc[v]);
  }
  for (int v = 0; v < nx; ++v) {
    float r = _mm512_reduce_add_ps(acc[v]);
    for (int j = i; j < n; ++j) {
      uint32_t u = (uint32_t)w[j] << 16;
      float wf;
      std::memcpy(&wf, &u, 4);
      r += wf * xs[v][j];
    }
    out[v] = r;
  }
}

// ---- MXFP4 rows: codes (n/2 bytes, low nibble first) and n/32 E8M0 scales ----
using MxRowDotsFn = void (*)(const uint8_t* codes, const uint8_t* sc, int n, const float* const* xs, int nx,
                             float* out);

constexpr float kE2M1[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                             -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

// 2^(s - 127) for an E8M0 byte: the exponent field itself, or 2^-127 (subnormal) for s = 0
inline float e8m0_f(uint8_t s) {
  const uint32_t u = s ? (uint32_t)s << 23 : 0x00400000u;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

void mx_row_dots_scalar(const uint8_t* codes, const uint8_t* sc, int n, const float* const* xs, int nx,
                        float* out) {
  float acc[MAXV] = {0};
  for (int b = 0; b < n / 32; ++b) {
    float w[32];
    const float s = e8m0_f(sc[b]);
    for (int i = 0; i < 16; ++i) {
      w[2 * i] = kE2M1[codes[16 * b + i] & 15] * s;
      w[2 * i + 1] = kE2M1[codes[16 * b + i] >> 4] * s;
    }
    for (int v = 0; v < nx; ++v)
      for (int i = 0; i < 32; ++i) acc[v] += w[i] * xs[v][32 * b + i];
  }
  for (int v = 0; v < nx; ++v) out[v] = acc[v];
}

__attribute__((target("avx2,fma"))) void mx_row_dots_avx2(const uint8_t* codes, const uint8_t* sc, int n,
                                                            const float* const* xs, int nx, float* out) {
  const __m256 mag = _mm256_setr_ps(0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f);
  const __m128i m4 = _mm_set1_epi8(0x0f);
  __m256 acc[MAXV];
  for (int v = 0; v < MAXV; ++v) acc[v] = _mm256_setzero_ps();
  for (int b = 0; b < n / 32; ++b) {
    const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + 16 * b));
    const __m128i lo = _mm_and_si128(raw, m4);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m4);
    const __m128i el[2] = {_mm_unpacklo_epi8(lo, hi), _mm_unpackhi_epi8(lo, hi)};  // elements 0..15, 16..31
    const __m256 s = _mm256_set1_ps(e8m0_f(sc[b]));
    __m256 w[4];
    for (int q = 0; q < 4; ++q) {
      const __m128i src = (q & 1) ? _mm_srli_si128(el[q >> 1], 8) : el[q >> 1];
      const __m256i c = _mm256_cvtepu8_epi32(src);
      const __m256 m = _mm256_permutevar8x32_ps(mag, c);
      const __m256 sign = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_and_si256(c, _mm256_set1_epi32(8)), 28));
      w[q] = _mm256_mul_ps(_mm256_xor_ps(m, sign), s);
    }
    for (int v = 0; v < nx; ++v)
      for (int q = 0; q < 4; ++q) acc[v] = _mm256_fmadd_ps(w[q], _mm256_loadu_ps(xs[v] + 32 * b + 8 * q), acc[v]);
  }
  for (int v = 0; v < nx; ++v) {
    __m128 t = _mm_add_ps(_mm256_castps256_ps128(acc[v]), _mm256_extractf128_ps(acc[v], 1));
    t = _mm_hadd_ps(t, t);
    t = _mm_hadd_ps(t, t);
    out[v] = _mm_cvtss_f32(t);
  }
}

// The 32 weights of block b: codes through a 16-entry table scaled by the block's
// E8M0 scale (elements 0..15 in w0, 16..31 in w1).
__attribute__((target("avx512f,avx512bw"))) inline void mx_block_weights(const uint8_t* codes, const uint8_t* sc,
                                                                         int b, __m512 lut, __m512& w0,
                                                                         __m512& w1) {
  const __m128i m4 = _mm_set1_epi8(0x0f);
  const __m128i raw = _mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + 16 * b));
  const __m128i lo = _mm_and_si128(raw, m4);
  const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m4);
  const __m512 lut_s = _mm512_mul_ps(lut, _mm512_set1_ps(e8m0_f(sc[b])));
  w0 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpacklo_epi8(lo, hi)), lut_s);
  w1 = _mm512_permutexvar_ps(_mm512_cvtepu8_epi32(_mm_unpackhi_epi8(lo, hi)), lut_s);
}

// Independent accumulators per activation vector (two per block, four over two
// blocks when there is one vector) keep the FMA latency off the critical path.
__attribute__((target("avx512f,avx512bw"))) void mx_row_dots_avx512(const uint8_t* codes, const uint8_t* sc, int n,
                                                                      const float* const* xs, int nx, float* out) {
  const __m512 lut = _mm512_loadu_ps(kE2M1);
  const int nb = n / 32;
  if (nx == 1) {
    const float* x = xs[0];
    __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps(), a2 = _mm512_setzero_ps(), a3 = _mm512_setzero_ps();
    int b = 0;
    for (; b + 2 <= nb; b += 2) {
      __m512 w0, w1, w2, w3;
      mx_block_weights(codes, sc, b, lut, w0, w1);
      mx_block_weights(codes, sc, b + 1, lut, w2, w3);
      a0 = _mm512_fmadd_ps(w0, _mm512_loadu_ps(x + 32 * b), a0);
      a1 = _mm512_fmadd_ps(w1, _mm512_loadu_ps(x + 32 * b + 16), a1);
      a2 = _mm512_fmadd_ps(w2, _mm512_loadu_ps(x + 32 * b + 32), a2);
      a3 = _mm512_fmadd_ps(w3, _mm512_loadu_ps(x + 32 * b + 48), a3);
    }
    for (; b < nb; ++b) {
      __m512 w0, w1;
      mx_block_weights(codes, sc, b, lut, w0, w1);
      a0 = _mm512_fmadd_ps(w0, _mm512_loadu_ps(x + 32 * b), a0);
      a1 = _mm512_fmadd_ps(w1, _mm512_loadu_ps(x + 32 * b + 16), a1);
    }
    out[0] = _mm512_reduce_add_ps(_mm512_add_ps(_mm512_add_ps(a0, a1), _mm512_add_ps(a2, a3)));
    return;
  }
  __m512 acc0[MAXV], acc1[MAXV];
  for (int v = 0; v < MAXV; ++v) acc0[v] = acc1[v] = _mm512_setzero_ps();
  for (int b = 0; b < nb; ++b) {
    __m512 w0, w1;
    mx_block_weights(codes, sc, b, lut, w0, w1);
    for (int v = 0; v < nx; ++v) {
      acc0[v] = _mm512_fmadd_ps(w0, _mm512_loadu_ps(xs[v] + 32 * b), acc0[v]);
      acc1[v] = _mm512_fmadd_ps(w1, _mm512_loadu_ps(xs[v] + 32 * b + 16), acc1[v]);
    }
  }
  for (int v = 0; v < nx; ++v) out[v] = _mm512_reduce_add_ps(_mm512_add_ps(acc0[v], acc1[v]));
}

MxRowDotsFn g_mx_row_dots = nullptr;

RowDotsFn pick_row_dots(const char** name) {
  __builtin_cpu_init();
  if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw")) {
    *name = "avx512";
    g_mx_row_dots = mx_row_dots_avx512;
    return row_dots_avx512;
  }
  if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) {
    *name = "avx2";
    g_mx_row_dots = mx_row_dots_avx2;
    return row_dots_avx2;
  }
  *name = "scalar";
  g_mx_row_dots = mx_row_dots_scalar;
  return row_dots_scalar;
}

const char* g_simd_name = nullptr;
RowDotsFn g_row_dots = nullptr;
std::once_flag g_simd_once;

inline float silu_f(float z) { return z / (1.0f + std::exp(-z)); }

}  // namespace

class CpuPool {
 public:
  explicit CpuPool(int threads) {
    std::call_once(g_simd_once, [] { g_row_dots = pick_row_dots(&g_simd_name); });
    cpu_set_t mask;
    CPU_ZERO(&mask);
    std::vector<int> cpus;
    if (sched_getaffinity(0, sizeof(mask), &mask) == 0)
      for (int c = 0; c < CPU_SETSIZE; ++c)
        if (CPU_ISSET(c, &mask)) cpus.push_back(c);
    // By default one worker per CPU of the affinity mask except the first two,
    // which are left to the calling thread (it also works while it waits) and to
    // the HIP runtime; each worker is pinned to its own CPU.
    const int ncpu = cpus.empty() ? (int)std::thread::hardware_concurrency() : (int)cpus.size();
    const int reserved = ncpu > 4 ? 2 : (ncpu > 1 ? 1 : 0);
    if (threads <= 0) threads = std::max(1, ncpu - reserved);
    nthreads_ = threads;
    for (int i = 0; i < threads; ++i) {
      workers_.emplace_back([this] { run(); });
      if ((int)cpus.size() > reserved) {
        cpu_set_t one;
        CPU_ZERO(&one);
        CPU_SET(cpus[reserved + (i % (cpus.size() - reserved))], &one);
        pthread_setaffinity_np(workers_.back().native_handle(), sizeof(one), &one);
      }
    }
  }

  ~CpuPool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
      gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }

  int threads() const { return nthreads_; }
  double last_work_us() const { return t_done_us_; }
  int last_caller_items() const { return caller_items_; }

  void submit(const uint16_t* x, int T, int d, int d_ff, int fmt, const CpuExpert* ex, int n_exp,
              float* partial) {
    T_ = T;
    d_ = d;
    d_ff_ = d_ff;
    mx_ = fmt == FT_W_MXFP4;
    ex_ = ex;
    n_exp_ = n_exp;
    partial_ = partial;
    xf_.resize((size_t)T * d);
    for (size_t i = 0; i < (size_t)T * d; ++i) {
      uint32_t u = (uint32_t)x[i] << 16;
      std::memcpy(&xf_[i], &u, 4);
    }
    std::memset(partial, 0, sizeof(float) * (size_t)T * d);
    use_base_.assign(n_exp + 1, 0);
    for (int e = 0; e < n_exp; ++e) use_base_[e + 1] = use_base_[e] + ex[e].n_use;
    h_.resize((size_t)use_base_[n_exp] * d_ff);
    blocks1_ = (d_ff + RB1 - 1) / RB1;
    items1_ = n_exp * blocks1_;
    items2_ = (d + RB2 - 1) / RB2;
    // publish: the job fields above happen-before any item grab of this generation
    const uint64_t g = (gen_.load(std::memory_order_relaxed) + 1) & 0xffffffffu;
    cur_ = g;
    done1_.store(0, std::memory_order_relaxed);
    done2_.store(0, std::memory_order_relaxed);
    t_submit_ = std::chrono::steady_clock::now();
    next1_.store(g << 32, std::memory_order_release);
    next2_.store(g << 32, std::memory_order_release);
    {
      std::lock_guard<std::mutex> lk(mu_);
      gen_.store(g, std::memory_order_release);
    }
    cv_.notify_all();
  }

  // The caller works on the current call too, then waits for every item to finish.
  void wait() {
    caller_items_ = work(cur_);
    for (int spins = 0; done2_.load(std::memory_order_acquire) < items2_; ++spins) {
      if (spins < 4096)
        _mm_pause();
      else
        std::this_thread::yield();
    }
  }

 private:
  static constexpr int kSpinUs = 20000;
  static constexpr int RB1 = 16;  // W_gate/W_up rows per phase-1 item
  static constexpr int RB2 = 32;  // output rows per phase-2 item

  // Takes the next item of generation g from a tagged counter (gen << 32 | index);
  // -1 when the counter belongs to another call or is exhausted.
  static int grab(std::atomic<uint64_t>& next, uint64_t g, int items) {
    uint64_t v = next.load(std::memory_order_acquire);
    for (;;) {
      if ((v >> 32) != g) return -1;
      const int i = (int)(v & 0xffffffffu);
      if (i >= items) return -1;
      if (next.compare_exchange_weak(v, v + 1, std::memory_order_acq_rel, std::memory_order_acquire)) return i;
    }
  }

  // Phase 1 items, then (once all phase-1 items of this call are done) phase 2
  // items.  A thread that is descheduled while holding no item delays nothing.
  int work(uint64_t g) {
    int n = 0;
    for (int it; (it = grab(next1_, g, items1_)) >= 0; ++n) {
      phase1(it);
      done1_.fetch_add(1, std::memory_order_acq_rel);
    }
    for (int spins = 0; done1_.load(std::memory_order_acquire) < items1_; ++spins) {
      if ((next1_.load(std::memory_order_acquire) >> 32) != g) return n;  // call already over
      if (spins < 4096)
        _mm_pause();
      else
        std::this_thread::yield();
    }
    for (int it; (it = grab(next2_, g, items2_)) >= 0; ++n) {
      phase2(it);
      if (done2_.fetch_add(1, std::memory_order_acq_rel) == items2_ - 1)
        t_done_us_ = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_submit_).count();
    }
    return n;
  }

  void phase1(int item) {
    const int e = item / blocks1_;
    const int r0 = (item % blocks1_) * RB1;
    const int r1 = std::min(d_ff_, r0 + RB1);
    const CpuExpert& X = ex_[e];
    const uint16_t* wg = static_cast<const uint16_t*>(X.rec);
    const uint16_t* wu = wg + (size_t)d_ff_ * d_;
    const uint8_t* rb = static_cast<const uint8_t*>(X.rec);
    const size_t mc = (size_t)d_ff_ * d_ / 2, ms = (size_t)d_ff_ * d_ / 32;  // MXFP4 code / scale bytes per matrix
    const float* xs[MAXV];
    float zg[MAXV], zu[MAXV];
    for (int u0 = 0; u0 < X.n_use; u0 += MAXV) {
      const int nx = std::min(MAXV, X.n_use - u0);
      for (int v = 0; v < nx; ++v) xs[v] = xf_.data() + (size_t)X.use[u0 + v].t * d_;
      for (int r = r0; r < r1; ++r) {
        if (mx_) {
          g_mx_row_dots(rb + (size_t)r * (d_ / 2), rb + 3 * mc + (size_t)r * (d_ / 32), d_, xs, nx, zg);
          g_mx_row_dots(rb + mc + (size_t)r * (d_ / 2), rb + 3 * mc + ms + (size_t)r * (d_ / 32), d_, xs, nx, zu);
        } else {
          g_row_dots(wg + (size_t)r * d_, d_, xs, nx, zg);
          g_row_dots(wu + (size_t)r * d_, d_, xs, nx, zu);
        }
        for (int v = 0; v < nx; ++v)
          h_[(size_t)(use_base_[e] + u0 + v) * d_ff_ + r] = silu_f(zg[v]) * zu[v];
      }
    }
  }

  void phase2(int item) {
    const int c0 = item * RB2;
    const int c1 = std::min(d_, c0 + RB2);
    const float* hs[MAXV];
    float o[MAXV];
    for (int e = 0; e < n_exp_; ++e) {
      const CpuExpert& X = ex_[e];
      const uint16_t* wd = static_cast<const uint16_t*>(X.rec) + (size_t)2 * d_ff_ * d_;
      const uint8_t* rb = static_cast<const uint8_t*>(X.rec);
      const size_t mc = (size_t)d_ff_ * d_ / 2, ms = (size_t)d_ff_ * d_ / 32;
      for (int u0 = 0; u0 < X.n_use; u0 += MAXV) {
        const int nx = std::min(MAXV, X.n_use - u0);
        for (int v = 0; v < nx; ++v) hs[v] = h_.data() + (size_t)(use_base_[e] + u0 + v) * d_ff_;
        for (int c = c0; c < c1; ++c) {
          if (mx_)
            g_mx_row_dots(rb + 2 * mc + (size_t)c * (d_ff_ / 2), rb + 3 * mc + 2 * ms + (size_t)c * (d_ff_ / 32), d_ff_,
                          hs, nx, o);
          else
            g_row_dots(wd + (size_t)c * d_ff_, d_ff_, hs, nx, o);
          for (int v = 0; v < nx; ++v) partial_[(size_t)X.use[u0 + v].t * d_ + c] += X.use[u0 + v].gate * o[v];
        }
      }
    }
  }

  void run() {
    uint64_t seen = 0;
    for (;;) {
      // spin for the next call for up to kSpinUs, then sleep: decode calls with a
      // CPU set arrive a few layers apart and waking a sleeping pool is slow
      const auto spin_end = std::chrono::steady_clock::now() + std::chrono::microseconds(kSpinUs);
      for (int i = 0; gen_.load(std::memory_order_acquire) == seen; ++i) {
        _mm_pause();
        if ((i & 255) == 255 && std::chrono::steady_clock::now() > spin_end) break;
      }
      if (gen_.load(std::memory_order_acquire) == seen) {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_.load(std::memory_order_acquire) != seen || stop_; });
      }
      seen = gen_.load(std::memory_order_acquire);
      if (stop_) return;
      work(seen);
    }
  }

  int nthreads_ = 1;
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::atomic<uint64_t> gen_{0};
  uint64_t cur_ = 0;
  std::atomic<bool> stop_{false};

  int T_ = 0, d_ = 0, d_ff_ = 0, n_exp_ = 0;
  bool mx_ = false;
  const CpuExpert* ex_ = nullptr;
  float* partial_ = nullptr;
  std::vector<float> xf_, h_;
  std::vector<int> use_base_;
  int blocks1_ = 0, items1_ = 0, items2_ = 0;
  std::atomic<uint64_t> next1_{0}, next2_{0};
  std::atomic<int> done1_{0}, done2_{0};
  std::chrono::steady_clock::time_point t_submit_{};
  double t_done_us_ = 0.0;
  int caller_items_ = 0;
};

CpuPool* cpu_pool_create(int threads) { return new CpuPool(threads); }
void cpu_pool_destroy(CpuPool* p) { delete p; }
int cpu_pool_threads(const CpuPool* p) { return p->threads(); }
void cpu_pool_submit(CpuPool* p, const uint16_t* x, int T, int d, int d_ff, int fmt, const CpuExpert* ex,
                     int n_exp, float* partial) {
  p->submit(x, T, d, d_ff, fmt, ex, n_exp, partial);
}
void cpu_pool_wait(CpuPool* p) { p->wait(); }
double cpu_pool_last_work_us(const CpuPool* p) { return p->last_work_us(); }
int cpu_pool_last_caller_items(const CpuPool* p) { return p->last_caller_items(); }
const char* cpu_simd_name() {
  std::call_once(g_simd_once, [] { g_row_dots = pick_row_dots(&g_simd_name); });
  return g_simd_name;
}

}  // namespace ft

// A CPU build of a HIP kernel source: one host thread per lane, a workgroup
// at a time.  __syncthreads waits for every live lane of the workgroup;
// cross-lane operations (ds_bpermute, __shfl_*, the fp8 MFMA) wait for every
// live lane of the wave, exchange through a per-wave table and wait again.
// A lane that leaves the kernel stops counting for both, as a finished wave
// stops counting for a hardware barrier.  Every wait has a time limit: a
// wait that does not complete reports which barrier, block and lane it was
// and aborts, so a barrier a lane never reaches, or a collective some lanes
// skip, shows as an error instead of a hang.  With the host build under
// AddressSanitizer every global and LDS access is bounds-checked.
//
// The fp8 MFMA (v_mfma_f32_16x16x128_f8f6f4, E4M3 operands, no block scale)
// is computed exactly in binary64 and rounded once to binary32, with the
// operand layout the kernel source assumes: lane l holds row (A) or column
// (B) l % 16 and K bytes [32 (l / 16), +32); the result gives lane l column
// l % 16, rows 4 (l / 16) + r.
#pragma once

#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <type_traits>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define __align__(n) __attribute__((aligned(n)))

namespace emu {

struct Idx {
  unsigned x = 0, y = 0, z = 0;
};
inline thread_local Idx thread_idx, block_idx;
inline Idx grid_dim, block_dim;

// Seconds a wait may last before it counts as a deadlock (EMU_WAIT_S, 30).
inline int wait_limit_s() {
  const char* e = std::getenv("EMU_WAIT_S");
  const int v = e ? std::atoi(e) : 0;
  return v > 0 ? v : 30;
}

// A barrier whose party count is the number of live lanes.
class Barrier {
 public:
  void init(int n) { n_ = n; }
  void wait(const char* what) {
    std::unique_lock<std::mutex> lk(m_);
    const long gen = gen_;
    if (++count_ >= n_) {
      count_ = 0;
      ++gen_;
      cv_.notify_all();
      return;
    }
    if (!cv_.wait_for(lk, std::chrono::seconds(wait_limit_s()), [&] { return gen_ != gen; })) {
      std::fprintf(stderr, "DEADLOCK at a %s wait: %d of %d live lanes arrived (block %u, lane %u)\n",
                   what, count_, n_, block_idx.x, thread_idx.x);
      std::fflush(stderr);
      std::abort();
    }
  }
  void leave() {
    std::lock_guard<std::mutex> lk(m_);
    --n_;
    if (n_ > 0 && count_ >= n_) {
      count_ = 0;
      ++gen_;
      cv_.notify_all();
    }
  }

 private:
  std::mutex m_;
  std::condition_variable cv_;
  int n_ = 0, count_ = 0;
  long gen_ = 0;
};

struct Wave {
  Barrier bar;
  uint64_t slot[64];
  uint8_t a[64][32], b[64][32];
};

struct Block {
  Barrier bar;
  std::vector<Wave> waves;
  explicit Block(unsigned threads) : waves((threads + 63) / 64) {
    bar.init((int)threads);
    for (unsigned w = 0; w < waves.size(); ++w) {
      const unsigned lanes = threads - 64 * w < 64 ? threads - 64 * w : 64;
      waves[w].bar.init((int)lanes);
    }
  }
};
inline thread_local Block* cur_block = nullptr;

inline int lane() { return (int)(thread_idx.x & 63u); }
inline Wave& wave() { return cur_block->waves[thread_idx.x / 64]; }

template <class T>
T exchange(T v, int src) {
  static_assert(sizeof(T) <= 8, "one register");
  Wave& w = wave();
  uint64_t bits = 0;
  std::memcpy(&bits, &v, sizeof(T));
  w.slot[lane()] = bits;
  w.bar.wait("cross-lane");
  const uint64_t r = w.slot[src & 63];
  w.bar.wait("cross-lane");
  T out;
  std::memcpy(&out, &r, sizeof(T));
  return out;
}

inline int bpermute(int addr, int v) { return exchange(v, (addr >> 2) & 63); }
template <class T>
T shfl_xor(T v, int mask) {
  return exchange(v, lane() ^ mask);
}
template <class T>
T shfl_up(T v, unsigned d) {
  const int src = lane() - (int)d;
  return exchange(v, src < 0 ? lane() : src);
}

inline void syncthreads() { cur_block->bar.wait("__syncthreads"); }

inline double e4m3(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e ? std::ldexp(1.0 + m / 8.0, e - 7) : std::ldexp(m / 8.0, -6);
  return s ? -v : v;
}

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

inline v4f_t mfma_fp8(v8i_t a, v8i_t b, v4f_t c) {
  Wave& w = wave();
  const int l = lane();
  std::memcpy(w.a[l], &a, 32);
  std::memcpy(w.b[l], &b, 32);
  w.bar.wait("MFMA");
  v4f_t d;
  const int j = l % 16;
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * (l / 16) + r;
    double s = 0.0;
    for (int k = 0; k < 128; ++k)
      s += e4m3(w.a[i + 16 * (k / 32)][k % 32]) * e4m3(w.b[j + 16 * (k / 32)][k % 32]);
    d[r] = (float)(s + (double)c[r]);
  }
  w.bar.wait("MFMA");
  return d;
}

template <class T>
T unreachable(const char* what) {
  std::fprintf(stderr, "device builtin %s is not emulated\n", what);
  std::abort();
}

// A launch: the workgroups one after another, each with one thread per lane.
template <class K, class... A>
void launch(K kernel, dim3 g, dim3 b, A... args) {
  grid_dim = Idx{g.x, g.y, g.z};
  block_dim = Idx{b.x, b.y, b.z};
  for (unsigned bx = 0; bx < g.x; ++bx) {
    Block blk(b.x);
    std::vector<std::thread> ts;
    ts.reserve(b.x);
    for (unsigned t = 0; t < b.x; ++t) {
      ts.emplace_back([&, t, bx] {
        thread_idx = Idx{t, 0, 0};
        block_idx = Idx{bx, 0, 0};
        cur_block = &blk;
        kernel(args...);
        blk.waves[t / 64].bar.leave();
        blk.bar.leave();
      });
    }
    for (auto& th : ts) th.join();
  }
}

}  // namespace emu

#define threadIdx emu::thread_idx
#define blockIdx emu::block_idx
#define gridDim emu::grid_dim
#define blockDim emu::block_dim
#define __syncthreads() emu::syncthreads()
#define __shfl_xor(v, m) emu::shfl_xor(v, m)
#define __shfl_up(v, d) emu::shfl_up(v, d)
#define hipLaunchKernelGGL(k, g, b, shmem, stream, ...) emu::launch(k, g, b, __VA_ARGS__)
#define hipGetLastError() 0

#define __builtin_amdgcn_ds_bpermute(addr, v) emu::bpermute(addr, v)
#define __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, ...) emu::mfma_fp8(a, b, c)
#define __builtin_amdgcn_fence(order, scope) ((void)0)
#define __builtin_amdgcn_wave_barrier() ((void)0)
#define __builtin_amdgcn_update_dpp(...) emu::unreachable<int>("update_dpp")
#define __builtin_amdgcn_cvt_pk_fp8_f32(...) emu::unreachable<int>("cvt_pk_fp8_f32")
#define __builtin_amdgcn_cvt_f32_fp8(...) emu::unreachable<float>("cvt_f32_fp8")
#define __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(...) emu::unreachable<unsigned>("cvt_scalef32_pk_fp4_f32")

inline float __uint_as_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint32_t __float_as_uint(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
inline uint32_t max(uint32_t a, uint32_t b) { return a > b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }

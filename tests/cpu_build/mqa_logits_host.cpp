// The indexer-logits kernel source (mqa_logits.hip) built for the CPU with the
// stand-ins of emu.h, run through the library's own launcher on inputs from
// a file.  Usage: mqa_logits_host <input> <output>.
//
// Input (little-endian): int64 num_q, num_heads, num_k, row_cols, row_stride;
// then q codes [num_q, num_heads, 128] u8, k codes [num_k, 128] u8, k_scale
// [num_k] f32, weights [num_q, num_heads] f32, ks [num_q] i32, ke [num_q] i32.
// Output: the logits buffer [num_q, row_stride] f32, every element first set
// to -1234.5 so that elements the kernel does not write can be told apart.
#include <hip/hip_runtime.h>

#include "mqa_logits.hip"

#include <cstdio>
#include <vector>

template <class T>
static bool read_n(FILE* f, std::vector<T>& v, size_t n) {
  v.resize(n);
  return n == 0 || std::fread(v.data(), sizeof(T), n, f) == n;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 2;
  }
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  int64_t hdr[5];
  if (std::fread(hdr, sizeof(int64_t), 5, f) != 5) return 2;
  const int64_t M = hdr[0], H = hdr[1], N = hdr[2], cols = hdr[3], stride = hdr[4];
  std::vector<uint8_t> q, k;
  std::vector<float> ksc, w;
  std::vector<int32_t> ks, ke;
  if (!read_n(f, q, (size_t)(M * H * 128)) || !read_n(f, k, (size_t)(N * 128)) ||
      !read_n(f, ksc, (size_t)N) || !read_n(f, w, (size_t)(M * H)) ||
      !read_n(f, ks, (size_t)M) || !read_n(f, ke, (size_t)M))
    return 2;
  std::fclose(f);
  // exactly sized heap buffers: an access past any of them is an error
  // under AddressSanitizer
  std::vector<float> logits((size_t)(M * stride), -1234.5f);
  const pkv::MqaLogitsArgs a{q.data(), H * 128, k.data(), ksc.data(), w.data(), ks.data(),
                             ke.data(), logits.data(), stride, cols, (int32_t)M, (int32_t)H, N};
  const int rc = pkv::launch_fp8_mqa_logits(a, nullptr);
  if (rc != 0) return 3;
  FILE* o = std::fopen(argv[2], "wb");
  if (!o) return 2;
  std::fwrite(logits.data(), sizeof(float), logits.size(), o);
  std::fclose(o);
  std::printf("launched %lld workgroups\n", (long long)((M + 7) / 8));
  return 0;
}

// A C++ client of libpkv that uses the HIP runtime directly -- hipMalloc'd
// buffers, its own stream, no PyTorch -- to run the fp8 store and the gather
// of what it stored.  Usage: pkv_hip_client <input> <output>.
//
// Input (little-endian): int64 T, D, B, num_blocks, page_stride, R, max_blocks;
// then k bf16 bits [T, D] u16, slot_mapping [T] i64, cache [num_blocks,
// page_stride] u8, block_table [R, max_blocks] i32, cu_seq_lens [R + 1] i32,
// k_fp8 [rows, D] u8 and k_scale [rows, 4] u8 with rows = cu_seq_lens[R] + 3
// (their initial bytes).  Output: the cache, k_fp8 and k_scale after the two
// calls, in that order.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "pkv.h"

namespace {

template <class T>
bool read_n(FILE* f, std::vector<T>& v, size_t n) {
  v.resize(n);
  return n == 0 || std::fread(v.data(), sizeof(T), n, f) == n;
}

template <class T>
T* to_device(const std::vector<T>& v) {
  void* p = nullptr;
  if (hipMalloc(&p, v.size() * sizeof(T) + 16) != hipSuccess) return nullptr;
  if (!v.empty() && hipMemcpy(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return nullptr;
  return static_cast<T*>(p);
}

template <class T>
bool to_host(std::vector<T>& v, const T* p) {
  return v.empty() || hipMemcpy(v.data(), p, v.size() * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 2;
  }
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  int64_t h[7];
  if (std::fread(h, sizeof(int64_t), 7, f) != 7) return 2;
  const int64_t T = h[0], D = h[1], B = h[2], nb = h[3], stride = h[4], R = h[5], maxb = h[6];
  std::vector<uint16_t> k;
  std::vector<int64_t> slots;
  std::vector<uint8_t> cache, kf, ks;
  std::vector<int32_t> table, cu;
  if (!read_n(f, k, (size_t)(T * D)) || !read_n(f, slots, (size_t)T) ||
      !read_n(f, cache, (size_t)(nb * stride)) || !read_n(f, table, (size_t)(R * maxb)) ||
      !read_n(f, cu, (size_t)(R + 1)))
    return 2;
  const int64_t rows = (int64_t)cu[(size_t)R] + 3;
  if (!read_n(f, kf, (size_t)(rows * D)) || !read_n(f, ks, (size_t)(rows * 4))) return 2;
  std::fclose(f);

  uint16_t* dk = to_device(k);
  int64_t* dslots = to_device(slots);
  uint8_t* dcache = to_device(cache);
  int32_t* dtable = to_device(table);
  int32_t* dcu = to_device(cu);
  uint8_t* dkf = to_device(kf);
  uint8_t* dks = to_device(ks);
  if (!dk || !dslots || !dcache || !dtable || !dcu || !dkf || !dks) return 3;
  hipStream_t s = nullptr;
  if (hipStreamCreate(&s) != hipSuccess) return 3;

  int rc = pkv_store_indexer_k_fp8(dk, D, PKV_DTYPE_BF16, dslots, T, dcache, nb, stride,
                                   (int32_t)B, (int32_t)D, s);
  if (rc != PKV_OK) {
    std::fprintf(stderr, "store: %d %s\n", rc, pkv_last_error());
    return 4;
  }
  rc = pkv_gather_indexer_k_fp8(dcache, dkf, dks, dtable, dcu, (int32_t)R, (int32_t)maxb, rows,
                                nb, stride, (int32_t)B, (int32_t)D, s);
  if (rc != PKV_OK) {
    std::fprintf(stderr, "gather: %d %s\n", rc, pkv_last_error());
    return 4;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return 5;
  if (!to_host(cache, dcache) || !to_host(kf, dkf) || !to_host(ks, dks)) return 5;
  (void)hipStreamDestroy(s);
  for (void* p : {(void*)dk, (void*)dslots, (void*)dcache, (void*)dtable, (void*)dcu, (void*)dkf,
                  (void*)dks})
    (void)hipFree(p);

  FILE* o = std::fopen(argv[2], "wb");
  if (!o) return 2;
  std::fwrite(cache.data(), 1, cache.size(), o);
  std::fwrite(kf.data(), 1, kf.size(), o);
  std::fwrite(ks.data(), 1, ks.size(), o);
  std::fclose(o);
  std::printf("hip client ok\n");
  return 0;
}

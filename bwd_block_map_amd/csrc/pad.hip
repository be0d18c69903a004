// Head dimensions below HD: the library runs the HD kernels on copies whose
// rows are widened with zeros (a zero column adds nothing to a score, and the
// extra output columns are dropped), then narrows the results back. Rows are
// the innermost dimension in every layout, so one row copy covers BHSD, BSHD
// and TND alike.
#include "kernels.hpp"

namespace vsa {

namespace {

template <class T>
__global__ __launch_bounds__(256) void widen_rows_kernel(const T* __restrict__ src,
                                                         T* __restrict__ dst, long long rows, int D) {
  const long long n = rows * HD;
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n; x += (long long)gridDim.x * 256) {
    const long long r = x / HD;
    const int d = (int)(x - r * HD);
    dst[x] = d < D ? src[r * D + d] : T(0);
  }
}

template <class T>
__global__ __launch_bounds__(256) void narrow_rows_kernel(const T* __restrict__ src,
                                                          T* __restrict__ dst, long long rows, int D) {
  const long long n = rows * D;
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n; x += (long long)gridDim.x * 256) {
    const long long r = x / D;
    dst[x] = src[r * HD + (x - r * D)];
  }
}

__global__ __launch_bounds__(256) void copy_words_kernel(const uint32_t* __restrict__ src,
                                                        uint32_t* __restrict__ dst, long long n) {
  for (long long x = (long long)blockIdx.x * 256 + threadIdx.x; x < n; x += (long long)gridDim.x * 256)
    dst[x] = src[x];
}

unsigned grid_of(long long n) {
  const long long g = (n + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

}  // namespace

hipError_t launch_widen_rows(const void* src, void* dst, long long rows, int D, int elem_bytes,
                             hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (elem_bytes == 2)
    widen_rows_kernel<uint16_t><<<grid_of(rows * HD), 256, 0, st>>>(
        (const uint16_t*)src, (uint16_t*)dst, rows, D);
  else
    widen_rows_kernel<float><<<grid_of(rows * HD), 256, 0, st>>>((const float*)src, (float*)dst,
                                                                 rows, D);
  return hipGetLastError();
}

hipError_t launch_narrow_rows(const void* src, void* dst, long long rows, int D, int elem_bytes,
                              hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (elem_bytes == 2)
    narrow_rows_kernel<uint16_t><<<grid_of(rows * D), 256, 0, st>>>(
        (const uint16_t*)src, (uint16_t*)dst, rows, D);
  else
    narrow_rows_kernel<float><<<grid_of(rows * D), 256, 0, st>>>((const float*)src, (float*)dst,
                                                                 rows, D);
  return hipGetLastError();
}

hipError_t launch_copy_words(const void* src, void* dst, long long words, hipStream_t st) {
  if (words <= 0) return hipSuccess;
  copy_words_kernel<<<grid_of(words), 256, 0, st>>>((const uint32_t*)src, (uint32_t*)dst, words);
  return hipGetLastError();
}

}  // namespace vsa

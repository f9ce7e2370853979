// Read and write kernels of known traffic, for scaling the hardware's memory
// counters (rocprofv3 FETCH_SIZE / WRITE_SIZE) to bytes.  Not part of the
// layer: built into its own library (libqmoe_calib.so) and used by the
// benchmark's calibration mode only.  Each kernel touches every byte of its
// buffer exactly once, with one of the access shapes the layer's kernels use:
//   lines      64 lanes read 1 KB contiguous per instruction (whole 128-byte
//              lines), the shape of the small-batch GEMV kernels;
//   halflines  lane (r = l % 16, q = l / 16) reads 16 bytes at
//              r * row_bytes + 16 q + 64 kb: 16 rows x 64 bytes per
//              instruction, the shape of the grouped GEMM's weight loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void __launch_bounds__(256) read_lines_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;   // keeps the loads; practically never stores
}

__global__ void __launch_bounds__(256) read_halflines_kernel(const uint8_t* __restrict__ src,
                                                             size_t rows, uint32_t row_bytes,
                                                             uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave = ((size_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const size_t row = wave * 16 + (lane & 15);
  uint32_t acc = 0;
  if (row < rows) {
    const uint8_t* p = src + row * row_bytes + 16 * (lane >> 4);
    for (uint32_t kb = 0; kb < row_bytes / 64; ++kb) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + 64 * (size_t)kb);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) write_lines_kernel(uint4* __restrict__ dst, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    dst[i] = make_uint4((uint32_t)i, 1u, 2u, 3u);
}

}  // namespace

extern "C" {

// src: `bytes` (a multiple of 16) of device memory; sink: 256 uint32 of device memory.
int qmoe_calib_read_lines(const void* src, size_t bytes, void* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(read_lines_kernel, dim3(4096), dim3(256), 0, s,
                     static_cast<const uint4*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// rows x row_bytes (row_bytes a multiple of 64) of device memory.
int qmoe_calib_read_halflines(const void* src, size_t rows, uint32_t row_bytes, void* sink,
                              hipStream_t s) {
  if (row_bytes % 64 != 0) return 2;
  const size_t waves = (rows + 15) / 16;
  hipLaunchKernelGGL(read_halflines_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), rows, row_bytes, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int qmoe_calib_write_lines(void* dst, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(write_lines_kernel, dim3(4096), dim3(256), 0, s, static_cast<uint4*>(dst),
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"

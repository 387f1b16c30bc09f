// The calibration stream: a kernel with no arithmetic that reads and writes
// given byte counts in one pass, with the 16-byte vector accesses and the
// non-temporal hints of the fused kernels. Timed with the read/write mix of a
// workload, it states the streaming rate this GPU reaches in practice for
// that mix, beside the 8 TB/s peak.
//
// Thread j of n_out = write_bytes / 16 writes unit j of dst: the XOR of the
// source units j, j + n_out, j + 2 n_out, ... below n_in = read_bytes / 16
// (every source unit is read exactly once), or, past the source, the unit
// index itself. Consecutive threads touch consecutive units, so every
// wavefront access covers 1 KiB of contiguous bytes.
#include "anq_device.h"
#include "anq_internal.h"

namespace anq {

template <bool NT>
__global__ void __launch_bounds__(256) stream_kernel(const uint8_t* src, int64_t n_in,
                                                     uint8_t* dst, int64_t n_out) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n_out) return;
  U4 v;
  if (j < n_in) {
    v = ld16s<NT>(src + (size_t)j * 16);
  } else {
    v.w[0] = (uint32_t)j;
    v.w[1] = (uint32_t)(j >> 32);
    v.w[2] = 0u;
    v.w[3] = 0u;
  }
  for (int64_t k = j + n_out; k < n_in; k += n_out) {
    const U4 u = ld16s<NT>(src + (size_t)k * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) v.w[i] ^= u.w[i];
  }
  st16s<NT>(dst + (size_t)j * 16, v);
}

int launch_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, bool nt,
                  void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n_in = read_bytes / 16, n_out = write_bytes / 16;
  const int64_t grid = (n_out + 255) / 256;  // <= 2^31 - 1, checked by the front end
  const uint8_t* sb = static_cast<const uint8_t*>(src);
  uint8_t* db = static_cast<uint8_t*>(dst);
  if (nt)
    hipLaunchKernelGGL(stream_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, sb, n_in, db,
                       n_out);
  else
    hipLaunchKernelGGL(stream_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, sb, n_in, db,
                       n_out);
  return (int)hipGetLastError();
}

}  // namespace anq

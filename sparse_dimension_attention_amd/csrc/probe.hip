// Streaming-read bandwidth probe: the measured denominator next to the vendor's HBM peak.  Each
// workgroup reads one contiguous slice of the buffer in 16-byte pieces with the decode kernel's
// load (non-temporal, 1 KiB per wavefront instruction), sixteen pieces in flight per lane (64 KiB
// per workgroup per round), and folds them into one word per workgroup, so that nothing but the
// reads is timed.  Contiguous slices per workgroup sustain about 7.0 TB/s on MI355X at any grid
// from 256 to 8192 workgroups; a grid-stride walk over the same buffer reads 5.3 to 6.4 TB/s.
#include "aqua_internal.h"

namespace aqua {
namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

template <int NF>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4v *__restrict__ buf,
                                                          size_t n16, size_t per,
                                                          uint32_t *__restrict__ sink) {
  __shared__ uint32_t s_acc[4];
  const size_t lo = static_cast<size_t>(blockIdx.x) * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  size_t i = lo + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (NF - 1) * 256 < hi; i += NF * 256) {
    u32x4v r[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) r[j] = __builtin_nontemporal_load(buf + i + j * 256);
#pragma unroll
    for (int j = 0; j < NF; ++j) acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
  }
  for (; i < hi; i += 256) {
    const u32x4v r = __builtin_nontemporal_load(buf + i);
    acc ^= r.x ^ r.y ^ r.z ^ r.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink,
                              hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t per = (n16 + blocks - 1) / blocks;  // a workgroup past the end reads nothing
  stream_read_kernel<16><<<dim3(blocks), dim3(256), 0, s>>>(static_cast<const u32x4v *>(buf),
                                                            n16, per, sink);
  return hipGetLastError();
}

}  // namespace aqua

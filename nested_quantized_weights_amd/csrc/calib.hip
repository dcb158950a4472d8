// A plain streaming read: the bandwidth any kernel of this library that
// reads its bytes once can reach on this device. It is the denominator of
// the "fraction of achievable" figures next to the fraction of the
// published HBM peak. Each thread reads 16-byte pieces with the same
// nontemporal hint the GEMV and attention kernels use, four in flight per
// iteration, and folds them into one word so that no load is dead; each
// workgroup then xors its word into *sink.
#include "nibble.h"

namespace {

__global__ void __launch_bounds__(256) read_stream_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = nest::ldnt16(src + i), b = nest::ldnt16(src + i + stride);
    const uint4 c = nest::ldnt16(src + i + 2 * stride), d = nest::ldnt16(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = nest::ldnt16(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o, 64));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(sink, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

}  // namespace

extern "C" int nest_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  const char* what = "nest_read_stream";
  if (!src || !sink) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (bytes == 0 || bytes % 16) return nest::fail(NEST_ESHAPE, "%s: bytes must be a positive multiple of 16", what);
  if (!nest::aligned16(src)) return nest::fail(NEST_EALIGN, "%s: src must be 16-byte aligned", what);
  // as many workgroups as fit on the chip at once (at most eight per CU)
  const int blocks = nest::resident_blocks(reinterpret_cast<const void*>(read_stream_kernel), 256, 0);
  read_stream_kernel<<<dim3(static_cast<unsigned>(blocks < 2048 ? blocks : 2048)), 256, 0,
                       nest::as_stream(stream)>>>(static_cast<const uint4*>(src), bytes / 16, sink);
  return nest::check_launch(what);
}

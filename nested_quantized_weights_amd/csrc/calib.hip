// A plain streaming read: the bandwidth any kernel of this library that
// reads its bytes once can reach on this device. It is the denominator of
// the "fraction of achievable" figures next to the fraction of the
// published HBM peak. Each thread reads eight 16-byte pieces with the same
// nontemporal hint the GEMV and attention kernels use, all in flight
// together, and folds them into one word; a thread stores that word to
// *sink only if it equals a fixed constant, which keeps every load live
// without any contended write. The grid gives every thread one
// such batch (up to 65536 workgroups, then a grid-stride loop): on MI355X
// this shape measured fastest among 4 to 16 pieces per thread and 1024 to
// 131072 workgroups, about 6.5 TB/s over 2 GiB.
#include "nibble.h"

namespace {

constexpr int kPieces = 8;
constexpr int kMaxBlocks = 65536;

__global__ void __launch_bounds__(256) read_stream_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kPieces - 1) * stride < n16; i += kPieces * stride) {
    uint4 v[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) v[u] = nest::ldnt16(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kPieces; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = nest::ldnt16(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

extern "C" int nest_read_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  const char* what = "nest_read_stream";
  if (!src || !sink) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (bytes == 0 || bytes % 16) return nest::fail(NEST_ESHAPE, "%s: bytes must be a positive multiple of 16", what);
  if (!nest::aligned16(src)) return nest::fail(NEST_EALIGN, "%s: src must be 16-byte aligned", what);
  const size_t n16 = bytes / 16;
  const size_t want = (n16 + 256 * kPieces - 1) / (256 * kPieces);
  const unsigned blocks = static_cast<unsigned>(want < kMaxBlocks ? (want > 0 ? want : 1) : kMaxBlocks);
  read_stream_kernel<<<dim3(blocks), 256, 0, nest::as_stream(stream)>>>(static_cast<const uint4*>(src), n16, sink);
  return nest::check_launch(what);
}

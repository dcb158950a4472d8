// Internal: nibble-plane and activation operands for v_mfma_i32_16x16x64_i8.
//
// A lane holds 16 bytes of an MFMA operand: a row (or column) chosen by
// lane & 15, and a k-quarter chosen by lane >> 4. A group of 128 reduction
// elements is split into two MFMAs, one over the even and one over the odd
// elements of each k-quarter, so that both operands come straight from the
// plane bytes:
//   16 plane bytes (32 nibbles, element 2j in the low nibble of byte j):
//     even operand byte b of word t = (w_t << 4) & 0xF0 -> 16 * code[8t + 2b]
//     odd  operand byte b of word t =  w_t       & 0xF0 -> 16 * code[8t + 2b + 1]
//   32 activation bytes: v_perm_b32 gathers the even and the odd bytes into
//   the same positions.
// The MFMA k-order is the same permutation for both operands, so the group
// sum is unchanged, and every product carries the factor 16 (removed
// exactly by an arithmetic shift).
#pragma once

#include "common.h"

namespace nest {

constexpr int kGroup = 128;
constexpr unsigned kHiNib = 0xF0F0F0F0u;

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 32 activation bytes (elements 0..31 of a k-quarter) -> even / odd operands.
__device__ __forceinline__ void split_act(uint4 a0, uint4 a1, v4i& be, v4i& bo) {
  be[0] = __builtin_amdgcn_perm(a0.y, a0.x, 0x06040200u);
  be[1] = __builtin_amdgcn_perm(a0.w, a0.z, 0x06040200u);
  be[2] = __builtin_amdgcn_perm(a1.y, a1.x, 0x06040200u);
  be[3] = __builtin_amdgcn_perm(a1.w, a1.z, 0x06040200u);
  bo[0] = __builtin_amdgcn_perm(a0.y, a0.x, 0x07050301u);
  bo[1] = __builtin_amdgcn_perm(a0.w, a0.z, 0x07050301u);
  bo[2] = __builtin_amdgcn_perm(a1.y, a1.x, 0x07050301u);
  bo[3] = __builtin_amdgcn_perm(a1.w, a1.z, 0x07050301u);
}

// 16 plane bytes (32 nibbles) -> even / odd operands holding 16 * code.
__device__ __forceinline__ void split_nib(uint4 w, v4i& e, v4i& o) {
  e[0] = (w.x << 4) & kHiNib;
  e[1] = (w.y << 4) & kHiNib;
  e[2] = (w.z << 4) & kHiNib;
  e[3] = (w.w << 4) & kHiNib;
  o[0] = w.x & kHiNib;
  o[1] = w.y & kHiNib;
  o[2] = w.z & kHiNib;
  o[3] = w.w & kHiNib;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Blocks of `kernel` that fit on the chip at once (cached per kernel and
// dynamic LDS size).
int resident_blocks(const void* kernel, int threads, size_t dyn_lds);

// Counter zone at the start of every workspace of the GEMV entry points
// (draft_gemv*, verify_gemm*, verify_accept*), the same for every entry point
// and shape: [0, 256) the argmax kernels' finished-block counter, then one
// finished-slice counter per row block of the batched verify (at most
// kMaxSplitRowBlocks), which the row argmax of more than 16 rows takes in
// turn as one finished-chunk counter per row. Counters are zero at rest, every call returns the
// ones it used to zero, and no call stores data in the zone, so one
// workspace serves calls of any of these entry points and shapes in turn.
constexpr size_t kSplitCounterOff = 256;
constexpr int kMaxSplitRowBlocks = 1024;
constexpr size_t kCounterZoneBytes = kSplitCounterOff + 4 * kMaxSplitRowBlocks;

// Batched verify (M > 16 rows): one launch for up to 144 rows. Shapes whose
// groups are split over several blocks need the row blocks' counters (zero
// before the launch; the launch leaves them zero) and
// verify_batched_slot_bytes(M, K, N) bytes of partial sums (16-byte
// aligned, no initial contents); other shapes need neither (0 bytes).
// Without counters (null) the groups are never split. With refine null the
// launch computes the draft's product over the base plane alone (acc_dbg
// then holds the base plane's exact group sums).
size_t verify_batched_slot_bytes(int M, int K, int N);
int launch_verify_batched(const int8_t* qa, const float* sa, int M, int K, const uint8_t* base,
                          const uint8_t* refine, const float* scales, int N, float* y,
                          int32_t* acc_dbg, unsigned* counters, void* slots, size_t slot_bytes,
                          hipStream_t st);

}  // namespace nest

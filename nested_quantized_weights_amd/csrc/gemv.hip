// Draft and verify products for up to 16 activation rows over the dual-plane
// nested weights (BitNest, Figure 3: the draft reads the base plane, the
// target reads both), the fused LM-head argmax, and the greedy accept step
// of a round ("How Speculative Decoding Speeds Up Inference", numbered round
// steps, Table 1).
//
// gfx950 mapping. One wave owns a tile of 16 weight rows. Per group of 128
// weights, v_mfma_i32_16x16x64_i8 takes the activations as the A operand
// (row m = lane & 15) and the weights as the B operand (column n = tile row
// lane & 15). Both operands are built from raw bytes (see nibble.h). D then
// gives lane l the entries m = 4*(l>>4) + r, n = n0 + (l & 15). All M <= 4
// rows sit in registers r < M of lanes 0..15, so a one-row draft folds a
// single register, and each lane needs the scale of only one weight row.
// The fp32 fold runs in registers in ascending group order, as the
// reference fold does:
//   draft:  A_b = R_b >> 4,            run = fmaf(s,        A_b, run)
//   verify: A_v = R_b + (R_r >> 4),    run = fmaf(s * 2^-4, A_v, run)
// R_b and R_r are the exact int32 MFMA sums over 16*q_b and 16*q_r. With
// one segment per tile the result is bit-identical to the reference. With
// S > 1 segments, the waves of a block fold contiguous group ranges, and
// the partial sums are added in segment order.
//
// When the M x K activation bytes fit, each block stages them once in LDS,
// already split into even/odd operand order, so the main loop streams
// only the planes and scales from HBM. The *_x entry points take fp32
// activations instead: every block quantizes them itself while staging
// (s_a = max|x|/127 per row, q = clamp(rint(x/s_a), +-127), the rule of
// nest_act_quant), so the round needs no separate quantization launch.
// Blocks loop over tiles with a grid stride, and the grid is at most what
// fits on the chip.
//
// The argmax path keeps per-lane best (value, index) keys across tiles and
// writes one key per row and block into the caller's workspace; the last
// block to finish (a counter in the workspace, zero between calls) reduces
// every block's keys and writes the argmax or, for verify_accept, applies
// the accept rule. Why the last block sees every key: each block writes
// its keys with agent-scope atomic stores (on gfx950 these carry sc1 and
// are written through to the agent's coherence point rather than left in
// one XCD's L2), waits until those stores are acknowledged (s_waitcnt 0
// covers stores on this architecture), and only then increments the
// counter with an agent-scope atomic. The block whose increment returns
// gridDim - 1 therefore runs after every other block's keys have reached
// the coherence point, and it reads them with agent-scope atomic loads
// (sc1, served from that point). This is the ordering a release/acquire
// pair would give, without the release's write-back of the whole L2, which
// nothing here needs because no plain store carries data between blocks.
#include <type_traits>

#include "nibble.h"

namespace {

using nest::kGroup;
using nest::ld16;

constexpr int kMaxArgmaxBlocks = 4096;
constexpr int kLdsActMax = 48 * 1024;     // largest M*K staged in LDS from int8 activations
constexpr int kLdsActMaxX = 128 * 1024;   // largest M*K the fp32-activation path stages

struct FinishArgs {
  const unsigned long long* partials;
  int nparts, M;
  int32_t* argmax_out;  // draft: [M]
  int B, k;             // accept: B sequences of k+1 rows
  const int32_t* draft;
  int32_t* target;
  int32_t* n_emitted;
  int32_t* emitted;
  int32_t* len;   // accept: [B] committed lengths advanced by n_emitted (nullable)
  int32_t* next;  // accept: [B] the last emitted token, the next round's input (nullable)
  bool accept;    // apply the greedy accept rule (else write argmax_out)
};

struct GemvArgs {
  const int8_t* qa;
  const float* sa;
  const float* x;  // fp32 activations (the *_x entry points), else null
  int M, K;
  const uint8_t* base;
  const uint8_t* refine;
  const float* scales;
  int N, G, nseg;
  float* y;
  int32_t* acc_dbg;
  unsigned long long* partials;  // argmax: [gridDim.x][16]
  unsigned* done;                // argmax: finished-block counter (zero at launch)
  FinishArgs fin;                // argmax: what the last block writes
};


// LDS slot of the even (p = 0) or odd (p = 1) operand of activation row m,
// k-quarter kq, group g.
__device__ __forceinline__ int lds_slot(int g, int p, int kq, int m, int M) {
  return ((g * 2 + p) * 4 + kq) * M + m;
}

__device__ __forceinline__ uint32_t quant4(float4 v, float s, float r) {
  return (static_cast<uint32_t>(quant_act(v.x, s, r)) & 0xFFu) |
         ((static_cast<uint32_t>(quant_act(v.y, s, r)) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(quant_act(v.z, s, r)) & 0xFFu) << 16) |
         ((static_cast<uint32_t>(quant_act(v.w, s, r)) & 0xFFu) << 24);
}

__device__ __forceinline__ float absmax4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Code 16 elements (an "item") with the row's (s, 1/s) and store their even
// and odd bytes into the two operand slots of their k-quarter. Item idx of
// a row covers elements [16*idx, 16*idx + 16): group idx >> 3, k-quarter
// (idx >> 1) & 3, half idx & 1 of that quarter.
// The fast half of quant_act without its branch: the code of rint(x * r),
// and `near` set when x * r is within 3e-5 of a half-integer or r is not
// finite (then the caller recomputes with the exact quotient).
__device__ __forceinline__ uint32_t code_fast(float x, float r, bool& near) {
  const float t = x * r;
  near |= !(fabsf(t - floorf(t) - 0.5f) > 3.0e-5f);
  const float q = fminf(fmaxf(rintf(t), -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int>(q)) & 0xFFu;
}

__device__ __forceinline__ uint32_t quant4_fast(float4 v, float r, bool& near) {
  return code_fast(v.x, r, near) | (code_fast(v.y, r, near) << 8) | (code_fast(v.z, r, near) << 16) |
         (code_fast(v.w, r, near) << 24);
}

__device__ __forceinline__ void store_item(uint2* lds2, int M, int m, int idx, const float4 (&v)[4],
                                           float s, float r) {
  const int half = idx & 1, q = (idx >> 1) & 3, g = idx >> 3;
  // 16 codes without branches; one exact pass for the rare item that holds
  // a near-tie (or a zero / tiny row scale)
  bool near = !(r < INFINITY);
  uint32_t w0 = quant4_fast(v[0], r, near), w1 = quant4_fast(v[1], r, near), w2 = quant4_fast(v[2], r, near),
           w3 = quant4_fast(v[3], r, near);
  if (near) {
    w0 = quant4(v[0], s, r);
    w1 = quant4(v[1], s, r);
    w2 = quant4(v[2], s, r);
    w3 = quant4(v[3], s, r);
  }
  lds2[lds_slot(g, 0, q, m, M) * 2 + half] =
      make_uint2(__builtin_amdgcn_perm(w1, w0, 0x06040200u), __builtin_amdgcn_perm(w3, w2, 0x06040200u));
  lds2[lds_slot(g, 1, q, m, M) * 2 + half] =
      make_uint2(__builtin_amdgcn_perm(w1, w0, 0x07050301u), __builtin_amdgcn_perm(w3, w2, 0x07050301u));
}

// Per-token int8 quantization of fp32 activations x [M][K], written straight
// into the LDS operand layout, in two steps so that the kernel can request
// its first weights in between: vector loads return in issue order, so x
// must be requested before the weights for staging to wait on x alone.
// Thread t owns items t, t + NT, ... of the flattened rows; its first ITEMS
// items are loaded at once and kept in registers (one round trip when
// M*K <= 16*ITEMS*NT). Row maxima of |x| merge through an LDS max on the
// float bits (they order like the values for x >= 0); items past the first
// ITEMS*NT are read once for the maximum and again for coding.
template <int ITEMS>
struct XItems {
  float4 v[ITEMS][4];
  int row[ITEMS];
};

// Items base + t + j*NT (j < ITEMS) of the flattened rows. Branch-free: a
// clamped (in-bounds) load for every item, used only if its index is below
// total, so that a wait for these loads can leave later ones outstanding.
template <int NT, int ITEMS>
__device__ __forceinline__ void stage_x_batch(const float* __restrict__ x, int K, int ipr, int total, int base,
                                              XItems<ITEMS>& it) {
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int h = base + static_cast<int>(threadIdx.x) + j * NT, hc = min(h, total - 1), m = hc / ipr;
    it.row[j] = h < total ? m : -1;
    const float4* src = reinterpret_cast<const float4*>(x + static_cast<size_t>(m) * K) + 4 * (hc - m * ipr);
#pragma unroll
    for (int e = 0; e < 4; ++e) it.v[j][e] = src[e];
  }
}

template <int NT, int ITEMS>
__device__ __forceinline__ void stage_x_issue(const float* __restrict__ x, int M, int K, int G,
                                              XItems<ITEMS>& it) {
  stage_x_batch<NT, ITEMS>(x, K, G * 8, M * G * 8, 0, it);
}

template <int NT, int ITEMS>
__device__ __forceinline__ void stage_x_finish(const float* __restrict__ x, int M, int K, int G, uint4* lds,
                                               float* sa_sh, unsigned* amax_sh, const XItems<ITEMS>& it) {
  const int t = threadIdx.x;
  const int ipr = G * 8, total = M * ipr;
  if (t < 16) amax_sh[t] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (it.row[j] >= 0)
      atomicMax(&amax_sh[it.row[j]],
                __float_as_uint(fmaxf(fmaxf(absmax4(it.v[j][0]), absmax4(it.v[j][1])),
                                      fmaxf(absmax4(it.v[j][2]), absmax4(it.v[j][3])))));
  for (int h = t + ITEMS * NT; h < total; h += NT) {
    const int m = h / ipr;
    const float4* src = reinterpret_cast<const float4*>(x + static_cast<size_t>(m) * K) + 4 * (h - m * ipr);
    atomicMax(&amax_sh[m], __float_as_uint(fmaxf(fmaxf(absmax4(src[0]), absmax4(src[1])),
                                                 fmaxf(absmax4(src[2]), absmax4(src[3])))));
  }
  __syncthreads();
  // every thread derives the scales it needs from the row maxima itself
  // (the same IEEE operations, so the same values everywhere); thread m
  // also records row m's for the fold
  auto scale = [&](int m) { return __uint_as_float(amax_sh[m]) / 127.0f; };
  if (t < M) {
    const float s = scale(t);
    sa_sh[t] = s;
    sa_sh[16 + t] = 1.0f / s;
  }
  uint2* lds2 = reinterpret_cast<uint2*>(lds);
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (it.row[j] >= 0) {
      const float s = scale(it.row[j]);
      store_item(lds2, M, it.row[j], t + j * NT - it.row[j] * ipr, it.v[j], s, 1.0f / s);
    }
  for (int h = t + ITEMS * NT; h < total; h += NT) {
    const int m = h / ipr;
    const float4* src = reinterpret_cast<const float4*>(x + static_cast<size_t>(m) * K) + 4 * (h - m * ipr);
    const float4 w[4] = {src[0], src[1], src[2], src[3]};
    const float s = scale(m);
    store_item(lds2, M, m, h - m * ipr, w, s, 1.0f / s);
  }
  __syncthreads();
}

// int8 activations qa [M][K] -> the LDS operand layout, in the same two
// steps: unit u (32 bytes: row u % M, k-quarter (u / M) & 3, group u / 4M)
// of the first UNITS per thread is loaded before the weights are requested.
template <int UNITS>
struct QItems {
  uint4 a[UNITS], b[UNITS];
};

template <int NT, int UNITS>
__device__ __forceinline__ void stage_q_issue(const int8_t* __restrict__ qa, int M, int K, int G,
                                              QItems<UNITS>& it) {
  const int total = M * G * 4;
#pragma unroll
  for (int j = 0; j < UNITS; ++j) {
    const int u = min(static_cast<int>(threadIdx.x) + j * NT, total - 1);  // clamped, branch-free
    const int m = u % M, rest = u / M, q = rest & 3, g = rest >> 2;
    const int8_t* src = qa + static_cast<size_t>(m) * K + g * kGroup + q * 32;
    it.a[j] = ld16(src);
    it.b[j] = ld16(src + 16);
  }
}

template <int NT, int UNITS>
__device__ __forceinline__ void stage_q_finish(const int8_t* __restrict__ qa, int M, int K, int G, uint4* lds,
                                               const QItems<UNITS>& it) {
  const int total = M * G * 4;
  auto put = [&](int u, uint4 a0, uint4 a1) {
    const int m = u % M, rest = u / M, q = rest & 3, g = rest >> 2;
    v4i e, o;
    nest::split_act(a0, a1, e, o);
    lds[lds_slot(g, 0, q, m, M)] = __builtin_bit_cast(uint4, e);
    lds[lds_slot(g, 1, q, m, M)] = __builtin_bit_cast(uint4, o);
  };
#pragma unroll
  for (int j = 0; j < UNITS; ++j) {
    const int u = threadIdx.x + j * NT;
    if (u < total) put(u, it.a[j], it.b[j]);
  }
  for (int u = threadIdx.x + UNITS * NT; u < total; u += NT) {
    const int m = u % M, rest = u / M, q = rest & 3, g = rest >> 2;
    const int8_t* src = qa + static_cast<size_t>(m) * K + g * kGroup + q * 32;
    put(u, ld16(src), ld16(src + 16));
  }
  __syncthreads();
}

template <int PLANES, int MR, bool DBG, bool LDSACT>
__device__ __forceinline__ void gemv_group(const GemvArgs& a, const uint4* lds, const int8_t* pa, int kq,
                                           int mrow, int n, int g, uint4 wb, uint4 wr, float s,
                                           float (&run)[MR]) {
  v4i xe, xo;
  if (LDSACT) {
    xe = __builtin_bit_cast(v4i, lds[lds_slot(g, 0, kq, mrow, a.M)]);
    xo = __builtin_bit_cast(v4i, lds[lds_slot(g, 1, kq, mrow, a.M)]);
  } else {
    const int8_t* p = pa + static_cast<size_t>(g) * kGroup;
    nest::split_act(ld16(p), ld16(p + 16), xe, xo);
  }
  v4i wbe, wbo;
  nest::split_nib(wb, wbe, wbo);
  const v4i z = {0, 0, 0, 0};
  v4i rb = nest::mfma_i8(xe, wbe, z);
  rb = nest::mfma_i8(xo, wbo, rb);
  v4i acc;
  if (PLANES == 2) {
    v4i wre, wro;
    nest::split_nib(wr, wre, wro);
    v4i rr = nest::mfma_i8(xe, wre, z);
    rr = nest::mfma_i8(xo, wro, rr);
    acc = rb + (rr >> 4);
  } else {
    acc = rb >> 4;
  }
  const float sc = PLANES == 2 ? s * 0.0625f : s;
#pragma unroll
  for (int r = 0; r < MR; ++r) run[r] = fmaf(sc, static_cast<float>(acc[r]), run[r]);
  if (DBG && n < a.N) {
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int m = 4 * kq + r;
      if (m < a.M) a.acc_dbg[(static_cast<size_t>(m) * a.N + n) * a.G + g] = acc[r];
    }
  }
}

// Four consecutive groups of one lane's weight row: 16 plane bytes per
// group and plane, and the four scales.
struct Quad {
  uint4 b0, b1, b2, b3, r0, r1, r2, r3;
  float4 s;
};

// A lane's place in the tile layout (nestspec.h, nest_tile): for tile t and
// group g, the planes hold 1 KB = [k-quarter][16 rows][16 bytes], so lane
// (kq, c) reads 16 bytes at ((t*G + g)*4 + kq)*256 + c*16 and a wave's load
// covers the whole kilobyte; the scales hold [quad][16 rows][4], so lane c
// reads the float4 of groups 4u..4u+3 at ((t*Gq + u)*16 + c)*4.
struct TilePtr {
  const uint8_t* pb;  // group 0 of the lane's 16 bytes; group g adds g * 1024
  const uint8_t* pr;
  const float* ps;    // quad 0 of the lane's scales; quad u adds u * 64
};

template <int PLANES>
__device__ __forceinline__ TilePtr tile_ptr(const GemvArgs& a, int t, int kq, int c) {
  const size_t pl = (static_cast<size_t>(t) * a.G * 4 + kq) * 256 + c * 16;
  TilePtr p;
  p.pb = a.base + pl;
  p.pr = PLANES == 2 ? a.refine + pl : nullptr;
  p.ps = a.scales + (static_cast<size_t>(t) * ((a.G + 3) / 4) * 16 + c) * 4;
  return p;
}

template <int PLANES>
__device__ __forceinline__ void load_quad(const TilePtr& p, int g, Quad& q) {
  q.b0 = nest::ldnt16(p.pb + static_cast<size_t>(g) * 1024);
  q.b1 = nest::ldnt16(p.pb + static_cast<size_t>(g + 1) * 1024);
  q.b2 = nest::ldnt16(p.pb + static_cast<size_t>(g + 2) * 1024);
  q.b3 = nest::ldnt16(p.pb + static_cast<size_t>(g + 3) * 1024);
  if (PLANES == 2) {
    q.r0 = nest::ldnt16(p.pr + static_cast<size_t>(g) * 1024);
    q.r1 = nest::ldnt16(p.pr + static_cast<size_t>(g + 1) * 1024);
    q.r2 = nest::ldnt16(p.pr + static_cast<size_t>(g + 2) * 1024);
    q.r3 = nest::ldnt16(p.pr + static_cast<size_t>(g + 3) * 1024);
  } else {
    q.r0 = q.r1 = q.r2 = q.r3 = make_uint4(0, 0, 0, 0);
  }
  q.s = nest::ldnt_f4(p.ps + static_cast<size_t>(g / 4) * 64);
}

// Fold groups [g0, g1) of one tile (A4: 4-aligned bounds; cur holds the
// quad at g0, already loaded). The next quad is loaded while the current one
// is multiplied. Without A4 the groups are loaded one at a time.
template <int PLANES, int MR, bool DBG, bool A4, bool LDSACT>
__device__ __forceinline__ void gemv_segment(const GemvArgs& a, const uint4* lds, const TilePtr& tp,
                                             const int8_t* pa, int kq, int mrow, int n, int g0, int g1,
                                             float (&run)[MR], Quad& cur) {
  if (A4) {
    for (int g = g0; g < g1; g += 4) {
      Quad q;
      const bool more = g + 4 < g1;
      if (more) load_quad<PLANES>(tp, g + 4, q);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g, cur.b0, cur.r0, cur.s.x, run);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 1, cur.b1, cur.r1, cur.s.y, run);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 2, cur.b2, cur.r2, cur.s.z, run);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 3, cur.b3, cur.r3, cur.s.w, run);
      if (more) cur = q;
    }
  } else {
    for (int g = g0; g < g1; ++g) {
      const uint4 wb = nest::ldnt16(tp.pb + static_cast<size_t>(g) * 1024);
      const uint4 wr = PLANES == 2 ? nest::ldnt16(tp.pr + static_cast<size_t>(g) * 1024) : make_uint4(0, 0, 0, 0);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g, wb, wr,
                                          tp.ps[static_cast<size_t>(g / 4) * 64 + (g & 3)], run);
    }
  }
}

// The same with D quads in flight: q[i] holds the quad at g0 + 4i (when it
// exists), all already requested; the quad D ahead is requested while q[0]
// is multiplied. Used by the argmax GEMVs, whose waves take two or three
// whole tiles each: in the last third of a launch only the three-tile waves
// still stream, and the deeper queue keeps enough bytes in flight per CU.
template <int PLANES, int MR, bool DBG, bool LDSACT, int D>
__device__ __forceinline__ void gemv_segment_d(const GemvArgs& a, const uint4* lds, const TilePtr& tp,
                                               const int8_t* pa, int kq, int mrow, int n, int g0, int g1,
                                               float (&run)[MR], Quad (&qs)[D]) {
  for (int g = g0; g < g1; g += 4) {
    Quad q;
    const bool more = g + 4 * D < g1;
    if (more) load_quad<PLANES>(tp, g + 4 * D, q);
    const Quad& cur = qs[0];
    gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g, cur.b0, cur.r0, cur.s.x, run);
    gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 1, cur.b1, cur.r1, cur.s.y, run);
    gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 2, cur.b2, cur.r2, cur.s.z, run);
    gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 3, cur.b3, cur.r3, cur.s.w, run);
#pragma unroll
    for (int i = 0; i + 1 < D; ++i) qs[i] = qs[i + 1];
    if (more) qs[D - 1] = q;
  }
}

// WAVES waves per block; a tile takes nseg consecutive waves (nseg | WAVES).
// ARGMAX requires nseg == 1. XQ: fp32 activations, quantized while staging
// (requires LDSACT). The first quad of each wave's first tile is requested
// before the activations are staged, so staging overlaps the first HBM
// round trip of the weights.
// Waves per SIMD the register allocation must allow. The streams need
// enough bytes in flight; the targets are the largest that compile without
// spills for each fold (the one-row, one-plane fold trades a fourth wave
// for a second quad in flight, measured faster; the debug build is left
// unconstrained).
// Quads in flight per wave for the argmax GEMVs (see gemv_segment_d): two
// for one plane; the two-plane fold keeps one (a second, at two waves per
// SIMD, measured no faster), and three for one plane was slower.
constexpr int prefetch_depth(int planes) { return planes == 1 ? 2 : 1; }

constexpr int occupancy_target(int planes, int mr, bool dbg, bool unstaged_depth2 = false) {
  // the two-plane fold with two quads in flight (unstaged activations)
  // needs the register budget of two waves per SIMD
  return dbg ? 1 : planes == 2 ? (unstaged_depth2 ? 2 : 3) : mr == 1 ? 3 : 4;
}

template <int PLANES, int MR, int WAVES, bool ARGMAX, bool DBG, bool A4, bool LDSACT, bool XQ>
__global__ void __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(occupancy_target(PLANES, MR, DBG, !ARGMAX && A4 && !LDSACT))))
gemv_kernel(GemvArgs a) {
  static_assert(!XQ || LDSACT, "fp32 activations are quantized into LDS");
  extern __shared__ uint4 lds_act[];
  // the wave index is the same in every lane: values derived from it stay
  // in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int S = a.nseg, per_iter = WAVES / S;
  const int T = (a.N + 15) / 16;
  // Tiles: the block's per_iter wave groups (S waves each) are numbered
  // across the grid, and group gg takes the contiguous tiles
  // [gg T / NG, (gg+1) T / NG): every group gets within one tile of the
  // same share, so the CUs' shares are even too.
  const int NG = static_cast<int>(gridDim.x) * per_iter;
  const int gg = static_cast<int>(blockIdx.x) * per_iter + wave / S;
  const int t_lo = static_cast<int>(static_cast<long long>(gg) * T / NG);
  const int t_hi = static_cast<int>(static_cast<long long>(gg + 1) * T / NG);
  const int J = (T + NG - 1) / NG;  // the most tiles a group takes
  const int seg = wave % S, G = a.G;
  const int unit = A4 ? 4 : 1, units = G / unit;
  const int g_begin = static_cast<int>(static_cast<long long>(seg) * units / S) * unit;
  const int g_end = static_cast<int>(static_cast<long long>(seg + 1) * units / S) * unit;
  const int kq = lane >> 4, c = lane & 15;
  const int mrow = min(c, a.M - 1);  // A-operand row of this lane (rows past M fill unused D rows)
  const int8_t* pa = LDSACT ? nullptr : a.qa + static_cast<size_t>(mrow) * a.K + kq * 32;

  // activations first (returns come back in issue order), then the first
  // weight quad, then the rest of staging
  constexpr int kXItems = MR == 1 ? (WAVES == 4 ? 1 : 2)
                                  : (WAVES >= 16 || PLANES == 1) ? (WAVES >= 16 ? 1 : 2) : (WAVES == 8 ? 3 : 4);
  constexpr int kQUnits = MR == 1 ? 1 : (WAVES >= 16 ? 1 : 3);
  XItems<XQ ? kXItems : 1> xi;
  QItems<(LDSACT && !XQ) ? kQUnits : 1> qi;
  if (XQ) stage_x_issue<WAVES * 64>(a.x, a.M, a.K, G, xi);
  else if (LDSACT) stage_q_issue<WAVES * 64>(a.qa, a.M, a.K, G, qi);

  // branch-free first quad: tile and group clamped into range; it is only
  // used when this wave's first tile exists and its segment is not empty
  // quads in flight per wave: the argmax GEMVs as prefetch_depth says; the
  // two-plane products whose activations are not staged (long rows, e.g.
  // the 5-row down projection) keep two (their waves walk a chain of quads,
  // each a round trip; 19.9 -> 17.8 us for 5 x 18944 x 3584), the rest one
  constexpr int kDepth = (A4 && !DBG) ? (ARGMAX ? prefetch_depth(PLANES) : (PLANES == 2 && !LDSACT ? 2 : 1)) : 1;
  Quad qs[kDepth];
  Quad& cur = qs[0];
  if (A4) {
    const TilePtr tp0 = tile_ptr<PLANES>(a, min(t_lo, T - 1), kq, c);
#pragma unroll
    for (int i = 0; i < kDepth; ++i) load_quad<PLANES>(tp0, min(g_begin + 4 * i, G - 4), qs[i]);
  }

  __shared__ float sa_sh[32];  // [0, 16): s_a per row; [16, 32): 1 / s_a
  __shared__ unsigned amax_sh[16];
  if (XQ) stage_x_finish<WAVES * 64>(a.x, a.M, a.K, G, lds_act, sa_sh, amax_sh, xi);
  else if (LDSACT) stage_q_finish<WAVES * 64>(a.qa, a.M, a.K, G, lds_act, qi);

  unsigned long long best[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) best[r] = 0;
  float s_a[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) s_a[r] = XQ ? sa_sh[min(4 * kq + r, a.M - 1)] : a.sa[min(4 * kq + r, a.M - 1)];

  // One tile of this wave's range. The first tile (its first quads already
  // in flight) is an instance of its own: as one loop with a first-iteration
  // test, the compiler kept more registers live and spilled some (the
  // one-plane argmax kernels over several rows).
  __shared__ float part[WAVES][MR][64];  // segment sums (S > 1)
  auto tile = [&](int j, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    const int n0 = (t_lo + j) * 16;
    const bool tile_ok = t_lo + j < t_hi;
    const int n = n0 + c;  // this lane's output column (weight row)
    const TilePtr tp = tile_ptr<PLANES>(a, n0 / 16, kq, c);
    float run[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) run[r] = 0.0f;
    // the first tile's first quad was requested before staging
    if (A4 && tile_ok && !kFirst && g_begin < g_end) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i)
        if (g_begin + 4 * i < g_end) load_quad<PLANES>(tp, g_begin + 4 * i, qs[i]);
    }
    if (tile_ok) {
      if constexpr (kDepth > 1) {
        gemv_segment_d<PLANES, MR, DBG, LDSACT, kDepth>(a, lds_act, tp, pa, kq, mrow, n, g_begin, g_end, run, qs);
      } else {
        gemv_segment<PLANES, MR, DBG, A4, LDSACT>(a, lds_act, tp, pa, kq, mrow, n, g_begin, g_end, run, cur);
      }
    }

    if (ARGMAX) {
      if (tile_ok && n < a.N) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          if (4 * kq + r < a.M) {
            const float v = run[r] * s_a[r];
            if (a.y) a.y[static_cast<size_t>(4 * kq + r) * a.N + n] = v;
            best[r] = umax64(best[r], argmax_key(v, static_cast<uint32_t>(n)));
          }
        }
      }
      return;
    }

    float tot[MR];
    if (S > 1) {
#pragma unroll
      for (int r = 0; r < MR; ++r) part[wave][r][lane] = run[r];
      __syncthreads();
      if (seg == 0) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          float t = part[wave][r][lane];
          for (int s2 = 1; s2 < S; ++s2) t += part[wave + s2][r][lane];
          tot[r] = t;
        }
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int r = 0; r < MR; ++r) tot[r] = run[r];
    }
    if (seg != 0 || !tile_ok || n >= a.N) return;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int m = 4 * kq + r;
      if (m < a.M) a.y[static_cast<size_t>(m) * a.N + n] = tot[r] * s_a[r];
    }
  };
  if (J > 0) tile(0, std::true_type{});
  for (int j = 1; j < J; ++j) tile(j, std::false_type{});

  if (ARGMAX) {
    // best over the 16 lanes of each k-quarter group, then over the waves
    __shared__ unsigned long long bw[WAVES][16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      unsigned long long k = r < MR ? best[r < MR ? r : 0] : 0ull;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) k = umax64(k, shfl_xor_u64(k, o));
      if (c == 0) bw[wave][4 * kq + r] = k;
    }
    __syncthreads();
    if (threadIdx.x < 16) {
      unsigned long long k = 0;
      for (int w = 0; w < WAVES; ++w) k = umax64(k, bw[w][threadIdx.x]);
      unsigned long long* slot = a.partials + static_cast<size_t>(blockIdx.x) * 16 + threadIdx.x;
      __hip_atomic_store(slot, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // The last block to finish reduces every block's keys (the ordering
    // argument is in the file header), then leaves the counter at zero for
    // the next launch that uses this workspace.
    __shared__ int last_sh;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) last_sh = atomicAdd(a.done, 1u) == gridDim.x - 1;
    __syncthreads();
    if (last_sh) {
      FinishArgs f = a.fin;
      f.partials = a.partials;
      f.nparts = gridDim.x;
      f.M = a.M;
      finish_reduce<WAVES * 64>(f);
      if (threadIdx.x == 0) atomicExch(a.done, 0u);
    }
  }
}

// Reduce the per-block argmax keys of f.partials (f.nparts blocks, f.M live
// rows) and write the argmaxes, or apply the greedy accept rule (f.accept).
// NT threads; thread t reads the keys of blocks t, t + NT, ..., all loads
// issued before any is used, so the reduction waits for one round trip to
// memory. Rows are then reduced per wave (shuffles) and across the waves
// (LDS). The keys were written by other blocks of the running kernel with
// agent-scope stores and are read with agent-scope loads.
// The greedy accept rule for sequence b, given the target (argmax) of each
// of its k+1 rows, tgt(b*(k+1) + j): slot i's draft d_i is checked against
// the target of row i-1, and the first mismatch ends the round. Writes the
// targets, the emitted count and tokens, and advances the lengths.
template <typename Tgt>
__device__ void accept_sequence(const FinishArgs& f, int b, Tgt tgt) {
  const int k1 = f.k + 1;
  int acc = 0;
  while (acc < f.k && f.draft[b * f.k + acc] == tgt(b * k1 + acc)) ++acc;
  f.n_emitted[b] = acc + 1;
  for (int j = 0; j < k1; ++j) {
    const int32_t tj = tgt(b * k1 + j);
    f.target[b * k1 + j] = tj;
    f.emitted[b * k1 + j] = j <= acc ? tj : -1;
  }
  if (f.len) f.len[b] += acc + 1;
  if (f.next) f.next[b] = tgt(b * k1 + acc);
}

template <int NT>
__device__ void finish_reduce(const FinishArgs& f) {
  constexpr int kPer = kMaxArgmaxBlocks / NT, kW = NT / 64;
  __shared__ unsigned long long red[16][kW];
  __shared__ int32_t tgt[16];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  unsigned long long best[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) best[r] = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = t + j * NT;
    if (b < f.nparts) {
      const unsigned long long* p = f.partials + static_cast<size_t>(b) * 16;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < f.M)
          best[i] = umax64(best[i], __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < f.M) {
      unsigned long long k = best[r];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) k = umax64(k, shfl_xor_u64(k, o));
      if (lane == 0) red[r][wave] = k;
    }
  }
  __syncthreads();
  if (t < f.M) {
    unsigned long long k = 0;
    for (int w = 0; w < kW; ++w) k = umax64(k, red[t][w]);
    tgt[t] = static_cast<int32_t>(argmax_key_index(k));
    if (!f.accept) f.argmax_out[t] = tgt[t];
  }
  __syncthreads();
  if (f.accept && t < f.B) accept_sequence(f, t, [&](int r) { return tgt[r]; });
}

// More than 16 rows (the drafts of several sequences, or verify_accept over
// several sequences or k >= 16): the batched kernel writes the logits to y,
// then each row's argmax is taken with the same keys as the fused path (the
// largest value, the lowest index among equal ones) by C workgroups per row,
// one per chunk of L values (L a multiple of 4). With C > 1 the chunks'
// keys meet through the handoff of the file header: each workgroup
// publishes its key with an agent-scope store, waits for it, and counts in
// on its row's counter; the row's last workgroup reduces the C keys, writes
// the row's index and returns the counter to zero.
__global__ void __launch_bounds__(256) row_argmax_kernel(const float* __restrict__ y, int V, int C, int L,
                                                         unsigned long long* keys, unsigned* counters,
                                                         int32_t* index) {
  __shared__ unsigned long long red[4];
  __shared__ int last_sh;
  const int t = threadIdx.x;
  const int row = static_cast<int>(blockIdx.x) / C, c = static_cast<int>(blockIdx.x) - row * C;
  const int lo = c * L, hi = min(lo + L, V);
  const float* yr = y + static_cast<size_t>(row) * V;
  unsigned long long k = 0;
  // the largest key does not depend on the order the values are visited
  // in: 16-byte loads where the rows allow them, else one value at a time
  int n0 = lo;
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
    const float4* y4 = reinterpret_cast<const float4*>(yr);
#pragma unroll 4
    for (int i = (lo >> 2) + t; i < (hi >> 2); i += 256) {
      const float4 v = y4[i];
      const uint32_t n = 4 * static_cast<uint32_t>(i);
      k = umax64(umax64(k, umax64(argmax_key(v.x, n), argmax_key(v.y, n + 1))),
                 umax64(argmax_key(v.z, n + 2), argmax_key(v.w, n + 3)));
    }
    n0 = hi;
  }
#pragma unroll 8
  for (int n = n0 + t; n < hi; n += 256) k = umax64(k, argmax_key(yr[n], static_cast<uint32_t>(n)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) k = umax64(k, shfl_xor_u64(k, o));
  if ((t & 63) == 0) red[t >> 6] = k;
  __syncthreads();
  const unsigned long long best = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
  if (C == 1) {
    if (t == 0) index[row] = static_cast<int32_t>(argmax_key_index(best));
    return;
  }
  if (t == 0) __hip_atomic_store(keys + static_cast<size_t>(row) * C + c, best, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) last_sh = atomicAdd(counters + row, 1u) == static_cast<unsigned>(C - 1);
  __syncthreads();
  if (last_sh && t < 64) {
    unsigned long long b = 0;
    for (int j = t; j < C; j += 64)
      b = umax64(b, __hip_atomic_load(keys + static_cast<size_t>(row) * C + j, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) b = umax64(b, shfl_xor_u64(b, o));
    if (t == 0) {
      index[row] = static_cast<int32_t>(argmax_key_index(b));
      atomicExch(counters + row, 0u);
    }
  }
}

__global__ void __launch_bounds__(64) accept_rows_kernel(const int32_t* index, FinishArgs f) {
  for (int b = threadIdx.x; b < f.B; b += 64) accept_sequence(f, b, [&](int r) { return index[r]; });
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int pick_split(int tiles, int G, int max_split) {
  // Enough waves to keep HBM busy (~8 per CU), at least two groups each.
  int s = 1;
  while (s < max_split && static_cast<long long>(tiles) * s < 2048 && G / (2 * s) >= 2) s *= 2;
  return s;
}

// The two-plane fold needs more than the 128 VGPRs a wave of a 1024-thread
// block may hold, so it uses at most 8 waves per block.
int max_split(int planes) { return planes == 2 ? 8 : 16; }

template <int PLANES, int MR, int WAVES, bool ARGMAX, bool DBG, bool A4, bool LDSACT, bool XQ>
int launch_one(const GemvArgs& a, hipStream_t st, const char* what, int max_blocks, int* used) {
  auto kern = gemv_kernel<PLANES, MR, WAVES, ARGMAX, DBG, A4, LDSACT, XQ>;
  const size_t lds = LDSACT ? static_cast<size_t>(a.M) * a.K : 0;
  if (lds > 64 * 1024) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       kLdsActMaxX);
    if (attr != hipSuccess)
      return nest::fail(NEST_EHIP, "%s: cannot raise the LDS limit: %s", what, hipGetErrorString(attr));
  }
  const int per_iter = WAVES / a.nseg;
  const int iters = ((a.N + 15) / 16 + per_iter - 1) / per_iter;
  // As many blocks as fit at once (a whole number per CU, so no CU carries
  // a larger share of blocks than another), at most one tile per wave group.
  const int fit = min(max_blocks, nest::resident_blocks(reinterpret_cast<const void*>(kern), WAVES * 64, lds));
  const int blocks = min(fit, iters);
  if (used) *used = blocks;
  kern<<<dim3(blocks), dim3(WAVES * 64), lds, st>>>(a);
  return nest::check_launch(what);
}

template <int PLANES, int MR, bool ARGMAX, bool DBG, bool A4, bool LDSACT, bool XQ>
int launch_waves(const GemvArgs& a, hipStream_t st, const char* what, int max_blocks, int* used) {
  // the exact-fold argmax GEMVs (one tile per wave) run 8 waves per block:
  // fewer blocks to dispatch and to stage activations for
  if constexpr (ARGMAX) return launch_one<PLANES, MR, 8, ARGMAX, DBG, A4, LDSACT, XQ>(a, st, what, max_blocks, used);
  if (a.nseg <= 4)
    return launch_one<PLANES, MR, 4, ARGMAX, DBG, A4, LDSACT, XQ>(a, st, what, max_blocks, used);
  if constexpr (!ARGMAX) {
    if (PLANES == 2 || a.nseg == 8)
      return launch_one<PLANES, MR, 8, false, DBG, A4, LDSACT, XQ>(a, st, what, max_blocks, used);
    if constexpr (PLANES == 1)
      return launch_one<PLANES, MR, 16, false, DBG, A4, LDSACT, XQ>(a, st, what, max_blocks, used);
  }
  return NEST_EHIP;
}

// Kernel choice: one-row (MR = 1) or up-to-16-row (MR = 4) fold; A4 (groups
// in quads) when G % 4 == 0; LDS-staged activations when M*K fits; the fp32
// activation path (a.x set) always stages, quantizing on the way.
template <int PLANES, bool ARGMAX, bool DBG>
int launch_gemv(const GemvArgs& a, hipStream_t st, const char* what, int max_blocks, int* used) {
  const bool a4 = a.G % 4 == 0;
  const bool stage = a.x || (a4 && static_cast<long long>(a.M) * a.K <= kLdsActMax);
  if constexpr (!DBG) {
    if (a.x) {
      if (a.M == 1)
        return a4 ? launch_waves<PLANES, 1, ARGMAX, false, true, true, true>(a, st, what, max_blocks, used)
                  : launch_waves<PLANES, 1, ARGMAX, false, false, true, true>(a, st, what, max_blocks, used);
      return a4 ? launch_waves<PLANES, 4, ARGMAX, false, true, true, true>(a, st, what, max_blocks, used)
                : launch_waves<PLANES, 4, ARGMAX, false, false, true, true>(a, st, what, max_blocks, used);
    }
  }
  const bool ldsact = stage;
  if (a.M == 1) {
    if (ldsact) return launch_waves<PLANES, 1, ARGMAX, DBG, true, true, false>(a, st, what, max_blocks, used);
    if (a4) return launch_waves<PLANES, 1, ARGMAX, DBG, true, false, false>(a, st, what, max_blocks, used);
    return launch_waves<PLANES, 1, ARGMAX, DBG, false, false, false>(a, st, what, max_blocks, used);
  }
  if (ldsact) return launch_waves<PLANES, 4, ARGMAX, DBG, true, true, false>(a, st, what, max_blocks, used);
  if (a4) return launch_waves<PLANES, 4, ARGMAX, DBG, true, false, false>(a, st, what, max_blocks, used);
  return launch_waves<PLANES, 4, ARGMAX, DBG, false, false, false>(a, st, what, max_blocks, used);
}

size_t argmax_ws_bytes(int N) {
  const int iters = ((N + 15) / 16 + 3) / 4;
  return static_cast<size_t>(min(iters, kMaxArgmaxBlocks)) * 16 * sizeof(unsigned long long);
}

// Workspace of the GEMV entry points (all offsets 256-byte aligned):
//   [0, C)               the counter zone (C = nest::kCounterZoneBytes): the
//                        argmax kernels' finished-block counter and the
//                        batched verify's finished-slice counters; zero
//                        before the first call, and every call leaves it zero
//   [C, C + P)           per-block argmax keys, P = argmax_ws_bytes(N)
//   then, for fp32 activations (the *_x entry points), M*K int8 codes and M
//   fp32 row scales, used when the codes are made by a separate
//   nest_act_quant launch rather than inside the GEMV, and the batched
//   verify's partial sums when it splits the groups.
// verify_gemm with int8 rows over more than 16 rows uses the counter zone
// and then the partial sums. Only counters ever live in the zone, at the
// same offsets for every entry point and shape, so calls of different
// shapes and entry points can take turns on one workspace.
constexpr size_t kCounterBytes = nest::kCounterZoneBytes;
static_assert(kCounterBytes % 256 == 0, "the counter zone keeps the 256-byte alignment");
constexpr size_t round256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// The batched verify's partial sums (its groups split over blocks), for the
// launches of up to 144 rows that an M-row call makes (the largest is the
// first, of min(M, 144) rows).
size_t batched_ws_bytes(int64_t M, int64_t K, int64_t N) {
  if (M <= 16 || N > (1LL << 30) || K > (1LL << 24)) return 0;
  return round256(nest::verify_batched_slot_bytes(static_cast<int>(M < 144 ? M : 144), static_cast<int>(K),
                                                  static_cast<int>(N)));
}

// verify_gemm's workspace with int8 rows: the counter zone and the partial
// sums, or nothing when no launch splits the groups.
size_t verify_int8_ws_bytes(int64_t M, int64_t K, int64_t N) {
  const size_t slots = batched_ws_bytes(M, K, N);
  return slots ? kCounterBytes + slots : 0;
}

// Chunks per row of the row argmax (more than 16 rows): about 1024
// workgroups over all rows, each chunk at least 2048 values, at most one
// row counter per row of the counter zone.
int row_chunks(int64_t M, int64_t V) {
  if (M >= nest::kMaxSplitRowBlocks) return 1;
  int64_t c = (1024 + M - 1) / M;
  const int64_t cap = V / 2048;
  if (c > cap) c = cap;
  if (c > 64) c = 64;
  return c < 1 ? 1 : static_cast<int>(c);
}

// The row argmax's chunk keys [M][C] and row indices [M] (int32, after the
// keys) over more than 16 rows.
size_t row_keys_bytes(int64_t M, int64_t V) {
  return static_cast<size_t>(M) * row_chunks(M, V) * sizeof(unsigned long long);
}

// The keys region: per-block argmax keys, or the row argmax's keys and
// indices over more than 16 rows.
size_t keys_bytes(int64_t M, int64_t N) {
  const size_t blocks = argmax_ws_bytes(static_cast<int>(N));
  const size_t rows = M > 16 ? row_keys_bytes(M, N) + static_cast<size_t>(M) * sizeof(int32_t) : 0;
  return round256(blocks > rows ? blocks : rows);
}


size_t gemv_ws_bytes(int64_t M, int64_t K, int64_t N, bool x) {
  size_t n = kCounterBytes + keys_bytes(M, N);
  if (x) n += round256(static_cast<size_t>(M) * K) + round256(static_cast<size_t>(M) * sizeof(float)) +
              batched_ws_bytes(M, K, N);
  return n;
}

struct Workspace {
  unsigned* counter;
  unsigned* split_counters;  // the batched verify's, in the counter zone
  unsigned long long* partials;
  int8_t* codes;  // fp32-activation paths only
  float* code_scales;
  void* batched;  // fp32-activation verify of more than 16 rows: the batched kernel's workspace
};

Workspace carve(void* ws, int64_t M, int64_t K, int64_t N) {
  char* p = static_cast<char*>(ws);
  Workspace w{};
  w.counter = reinterpret_cast<unsigned*>(p);
  w.split_counters = reinterpret_cast<unsigned*>(p + nest::kSplitCounterOff);
  w.partials = reinterpret_cast<unsigned long long*>(p + kCounterBytes);
  char* c = p + kCounterBytes + keys_bytes(M, N);
  w.codes = reinterpret_cast<int8_t*>(c);
  w.code_scales = reinterpret_cast<float*>(c + round256(static_cast<size_t>(M) * K));
  w.batched = reinterpret_cast<char*>(w.code_scales) + round256(static_cast<size_t>(M) * sizeof(float));
  return w;
}

// Launch the row argmax over M rows of V logits; index gets each row's
// argmax. Keys and row counters come from the workspace.
int launch_row_argmax(const float* y, int64_t M, int64_t V, const Workspace& w, int32_t* index,
                      hipStream_t st, const char* what) {
  const int C = row_chunks(M, V);
  const int64_t L = (((V + C - 1) / C) + 3) & ~static_cast<int64_t>(3);
  row_argmax_kernel<<<static_cast<unsigned>(M * C), 256, 0, st>>>(y, (int)V, C, (int)L, w.partials,
                                                                    w.split_counters, index);
  return nest::check_launch(what);
}

// The exact-fold argmax GEMV; its last block reduces the keys.
template <int PLANES, bool DBG>
int launch_argmax(GemvArgs a, const FinishArgs& f0, bool accept, const Workspace& w, hipStream_t st,
                  const char* what) {
  a.nseg = 1;
  a.done = w.counter;
  a.partials = w.partials;
  a.fin = f0;
  a.fin.accept = accept;
  return launch_gemv<PLANES, true, DBG>(a, st, what, kMaxArgmaxBlocks, nullptr);
}

// Activations of a call: int8 codes with their row scales, or fp32 values
// that the kernel quantizes itself.
struct Act {
  const int8_t* qa;
  const float* sa;
  const float* x;
};

int check_common(const char* what, const Act& act, int64_t M, int64_t K, const uint8_t* base,
                 const float* scales, int64_t N, int64_t group) {
  if (!base || !scales) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (act.x ? false : (!act.qa || !act.sa)) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (M < 1 || K < 1 || N < 1) return nest::fail(NEST_EINVAL, "%s: empty shape", what);
  if (group != kGroup)
    return nest::fail(NEST_EUNSUPPORTED, "%s: group=%lld (kernels handle 128)", what, (long long)group);
  if (K % kGroup) return nest::fail(NEST_ESHAPE, "%s: K=%lld is not a multiple of 128", what, (long long)K);
  if (K > (1LL << 24) || N > (1LL << 30) || M > (1LL << 20))
    return nest::fail(NEST_EUNSUPPORTED, "%s: shape too large", what);
  if (!nest::aligned16(base) || !nest::aligned16(scales))
    return nest::fail(NEST_EALIGN, "%s: planes and scales must be 16-byte aligned", what);
  if (act.x) {
    if (!nest::aligned16(act.x)) return nest::fail(NEST_EALIGN, "%s: x must be 16-byte aligned", what);
  } else if (!nest::aligned16(act.qa)) {
    return nest::fail(NEST_EALIGN, "%s: qa must be 16-byte aligned", what);
  }
  return NEST_OK;
}

int check_ws(const char* what, const void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return nest::fail(NEST_EWORKSPACE, "%s: workspace needs %zu bytes", what, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return nest::fail(NEST_EALIGN, "%s: workspace must be 256-byte aligned", what);
  return NEST_OK;
}

// fp32 activations are quantized inside the GEMV when they fit its LDS
// budget. A separate nest_act_quant launch into the workspace comes first
// when they do not fit, or when several rows would be quantized again by
// each of many blocks (N*M*K at least kQuantFirst: there one launch is
// cheaper than the blocks' staging; measured on the 5- and 9-row verify of
// 3584x37888 and 18944x3584 linears). The codes are the same either way.
constexpr double kQuantFirst = 1.2e8;

bool needs_quantize_first(int64_t M, int64_t K, int64_t N, bool by_size) {
  const bool fits = M <= 16 && M * K <= kLdsActMaxX;
  const bool heavy = by_size && M >= 2 && static_cast<double>(N) * M * K >= kQuantFirst;
  return !fits || heavy;
}

int quantize_first(Act& act, int64_t M, int64_t K, int64_t N, const Workspace& w, hipStream_t st,
                   bool by_size) {
  if (!act.x || !needs_quantize_first(M, K, N, by_size)) return NEST_OK;
  const int rc = nest_act_quant(act.x, M, K, w.codes, w.code_scales, st);
  if (rc) return rc;
  act = Act{w.codes, w.code_scales, nullptr};
  return NEST_OK;
}

GemvArgs make_args(const Act& act, int64_t M, int64_t K, const uint8_t* base, const uint8_t* refine,
                   const float* scales, int64_t N, float* y, int32_t* acc_dbg) {
  GemvArgs a{};
  a.qa = act.qa; a.sa = act.sa; a.x = act.x;
  a.M = (int)M; a.K = (int)K; a.base = base; a.refine = refine; a.scales = scales;
  a.N = (int)N; a.G = (int)(K / kGroup); a.y = y; a.acc_dbg = acc_dbg;
  return a;
}

int draft_impl(const char* what, const Act& act, int64_t M, int64_t K, const uint8_t* base,
               const float* scales, int64_t N, int64_t group, float* y, int32_t* argmax,
               int32_t* acc_dbg, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(what, act, M, K, base, scales, N, group);
  if (rc) return rc;
  if (!y && !argmax) return nest::fail(NEST_EINVAL, "%s: need y or argmax", what);
  if (M > 16 && !y) return nest::fail(NEST_EINVAL, "%s: more than 16 rows need y for the products", what);
  if (M > 65535) return nest::fail(NEST_EUNSUPPORTED, "%s: M=%lld > 65535", what, (long long)M);
  if (act.x || argmax) {
    rc = check_ws(what, ws, ws_bytes, gemv_ws_bytes(M, K, N, act.x != nullptr));
    if (rc) return rc;
  }
  hipStream_t st = nest::as_stream(stream);
  const Workspace w = ws ? carve(ws, M, K, N) : Workspace{};
  Act act2 = act;
  rc = quantize_first(act2, M, K, N, w, st, true);
  if (rc) return rc;
  if (M > 16) {
    // more rows (the drafts of more than 16 sequences): the batched kernel
    // over the base plane alone (no refinement plane, groups not split),
    // then the row argmaxes with the fused path's keys
    for (int64_t m0 = 0; m0 < M; m0 += 144) {
      const int64_t mc = M - m0 < 144 ? M - m0 : 144;
      rc = nest::launch_verify_batched(act2.qa + m0 * K, act2.sa + m0, (int)mc, (int)K, base, nullptr, scales,
                                       (int)N, y + m0 * N, acc_dbg ? acc_dbg + m0 * N * (K / kGroup) : nullptr,
                                       nullptr, nullptr, 0, st);
      if (rc) return rc;
    }
    if (!argmax) return NEST_OK;
    return launch_row_argmax(y, M, N, w, argmax, st, what);
  }
  GemvArgs a = make_args(act2, M, K, base, nullptr, scales, N, y, acc_dbg);
  if (argmax) {
    FinishArgs f{};
    f.argmax_out = argmax;
    return acc_dbg ? launch_argmax<1, true>(a, f, false, w, st, what)
                   : launch_argmax<1, false>(a, f, false, w, st, what);
  }
  a.nseg = pick_split((a.N + 15) / 16, a.G, max_split(1));
  return acc_dbg ? launch_gemv<1, false, true>(a, st, what, 1 << 30, nullptr)
                 : launch_gemv<1, false, false>(a, st, what, 1 << 30, nullptr);
}

int verify_impl(const char* what, const Act& act, int64_t M, int64_t K, const uint8_t* base,
                const uint8_t* refine, const float* scales, int64_t N, int64_t group, float* y,
                int32_t* acc_dbg, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(what, act, M, K, base, scales, N, group);
  if (rc) return rc;
  if (!refine || !y) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (!nest::aligned16(refine)) return nest::fail(NEST_EALIGN, "%s: refine not 16-byte aligned", what);
  if (act.x) {
    rc = check_ws(what, ws, ws_bytes, gemv_ws_bytes(M, K, N, true));
    if (rc) return rc;
  }
  hipStream_t st = nest::as_stream(stream);
  Act act2 = act;
  // the batched kernel's counters (in the counter zone) and partial sums
  unsigned* bcnt = nullptr;
  void* bslots = nullptr;
  const size_t bslot_bytes = batched_ws_bytes(M, K, N);
  if (act.x) {
    const Workspace w = carve(ws, M, K, N);
    rc = quantize_first(act2, M, K, N, w, st, true);
    if (rc) return rc;
    bcnt = w.split_counters;
    bslots = w.batched;
  } else if (bslot_bytes) {
    rc = check_ws(what, ws, ws_bytes, verify_int8_ws_bytes(M, K, N));
    if (rc) return rc;
    bcnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + nest::kSplitCounterOff);
    bslots = static_cast<char*>(ws) + kCounterBytes;
  }
  if (M <= 16) {
    GemvArgs a = make_args(act2, M, K, base, refine, scales, N, y, acc_dbg);
    a.nseg = pick_split((a.N + 15) / 16, a.G, max_split(2));
    return acc_dbg ? launch_gemv<2, false, true>(a, st, what, 1 << 30, nullptr)
                   : launch_gemv<2, false, false>(a, st, what, 1 << 30, nullptr);
  }
  // More rows (int8 activations only): the batched kernel, in chunks of up to 144 rows.
  for (int64_t m0 = 0; m0 < M; m0 += 144) {
    const int64_t mc = M - m0 < 144 ? M - m0 : 144;
    rc = nest::launch_verify_batched(act2.qa + m0 * K, act2.sa + m0, (int)mc, (int)K, base, refine, scales,
                                     (int)N, y + m0 * N,
                                     acc_dbg ? acc_dbg + m0 * N * (K / kGroup) : nullptr, bcnt, bslots,
                                     bslot_bytes, st);
    if (rc) return rc;
  }
  return NEST_OK;
}

int accept_impl(const char* what, const Act& act, int64_t B, int64_t k, int64_t K, const uint8_t* base,
                const uint8_t* refine, const float* scales, int64_t V, int64_t group,
                const int32_t* draft, int32_t* target, int32_t* n_emitted, int32_t* emitted, float* y,
                int32_t* len, int32_t* next, void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || k < 0) return nest::fail(NEST_EINVAL, "%s: B=%lld k=%lld", what, (long long)B, (long long)k);
  if (B * (k + 1) > 65535)
    return nest::fail(NEST_EUNSUPPORTED, "%s: B*(k+1)=%lld > 65535", what, (long long)(B * (k + 1)));
  const int64_t M = B * (k + 1);
  if (M > 16 && !y) return nest::fail(NEST_EINVAL, "%s: more than 16 rows need y for the logits", what);
  int rc = check_common(what, act, M, K, base, scales, V, group);
  if (rc) return rc;
  if (!refine || !target || !n_emitted || !emitted || (k > 0 && !draft))
    return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (!nest::aligned16(refine)) return nest::fail(NEST_EALIGN, "%s: refine not 16-byte aligned", what);
  if (V > 0x7fffffffLL) return nest::fail(NEST_EUNSUPPORTED, "%s: V too large", what);
  rc = check_ws(what, ws, ws_bytes, gemv_ws_bytes(M, K, V, act.x != nullptr));
  if (rc) return rc;
  hipStream_t st = nest::as_stream(stream);
  const Workspace w = carve(ws, M, K, V);
  Act act2 = act;  // the LM head stays with in-kernel quantization whenever it fits
  rc = quantize_first(act2, M, K, V, w, st, false);
  if (rc) return rc;
  FinishArgs f{};
  f.B = (int)B; f.k = (int)k; f.draft = draft; f.target = target; f.n_emitted = n_emitted;
  f.emitted = emitted; f.len = len; f.next = next;
  if (M > 16) {
    // the batched kernel (groups never split: no room for partial sums is
    // asked of the caller) writes y, then the row argmaxes and the rule
    for (int64_t m0 = 0; m0 < M; m0 += 144) {
      const int64_t mc = M - m0 < 144 ? M - m0 : 144;
      rc = nest::launch_verify_batched(act2.qa + m0 * K, act2.sa + m0, (int)mc, (int)K, base, refine, scales,
                                       (int)V, y + m0 * V, nullptr, nullptr, nullptr, 0, st);
      if (rc) return rc;
    }
    int32_t* rows = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(w.partials) + row_keys_bytes(M, V));
    rc = launch_row_argmax(y, M, V, w, rows, st, what);
    if (rc) return rc;
    accept_rows_kernel<<<1, 64, 0, st>>>(rows, f);
    return nest::check_launch(what);
  }
  GemvArgs a = make_args(act2, M, K, base, refine, scales, V, y, nullptr);
  return launch_argmax<2, false>(a, f, true, w, st, what);
}

}  // namespace

extern "C" size_t draft_gemv_workspace_size(int64_t M, int64_t N) {
  if (M < 1 || N < 1 || N > (1LL << 30)) return 0;
  return gemv_ws_bytes(M, 0, N, false);
}

extern "C" size_t verify_accept_workspace_size(int64_t B, int64_t k, int64_t V) {
  if (B < 1 || k < 0 || V < 1 || V > (1LL << 30)) return 0;
  return gemv_ws_bytes(B * (k + 1), 0, V, false);
}

extern "C" size_t nest_gemv_x_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M < 1 || K < 1 || N < 1 || N > (1LL << 30) || K > (1LL << 24) || M > (1LL << 20)) return 0;
  return gemv_ws_bytes(M, K, N, true);
}

extern "C" int draft_gemv(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                          const uint8_t* base, const float* scales, int64_t N, int64_t group,
                          float* y, int32_t* argmax, int32_t* acc_dbg, void* ws, size_t ws_bytes,
                          void* stream) {
  return draft_impl("draft_gemv", Act{qa, sa, nullptr}, M, K, base, scales, N, group, y, argmax,
                    acc_dbg, ws, ws_bytes, stream);
}

extern "C" int draft_gemv_x(const float* x, int64_t M, int64_t K, const uint8_t* base,
                            const float* scales, int64_t N, int64_t group, float* y,
                            int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  if (!x) return nest::fail(NEST_EINVAL, "draft_gemv_x: null pointer");
  return draft_impl("draft_gemv_x", Act{nullptr, nullptr, x}, M, K, base, scales, N, group, y, argmax,
                    nullptr, ws, ws_bytes, stream);
}

extern "C" size_t verify_gemm_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M < 1 || K < 1 || N < 1) return 0;
  return verify_int8_ws_bytes(M, K, N);
}

extern "C" int verify_gemm(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                           const uint8_t* base, const uint8_t* refine, const float* scales,
                           int64_t N, int64_t group, float* y, int32_t* acc_dbg, void* ws,
                           size_t ws_bytes, void* stream) {
  return verify_impl("verify_gemm", Act{qa, sa, nullptr}, M, K, base, refine, scales, N, group, y,
                     acc_dbg, ws, ws_bytes, stream);
}

extern "C" int verify_gemm_x(const float* x, int64_t M, int64_t K, const uint8_t* base,
                             const uint8_t* refine, const float* scales, int64_t N, int64_t group,
                             float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x) return nest::fail(NEST_EINVAL, "verify_gemm_x: null pointer");
  return verify_impl("verify_gemm_x", Act{nullptr, nullptr, x}, M, K, base, refine, scales, N, group,
                     y, nullptr, ws, ws_bytes, stream);
}

extern "C" int verify_accept(const int8_t* qa, const float* sa, int64_t B, int64_t k, int64_t K,
                             const uint8_t* base, const uint8_t* refine, const float* scales,
                             int64_t V, int64_t group, const int32_t* draft, int32_t* target,
                             int32_t* n_emitted, int32_t* emitted, float* y, int32_t* len,
                             int32_t* next, void* ws, size_t ws_bytes, void* stream) {
  return accept_impl("verify_accept", Act{qa, sa, nullptr}, B, k, K, base, refine, scales, V, group,
                     draft, target, n_emitted, emitted, y, len, next, ws, ws_bytes, stream);
}

extern "C" int verify_accept_x(const float* x, int64_t B, int64_t k, int64_t K, const uint8_t* base,
                               const uint8_t* refine, const float* scales, int64_t V, int64_t group,
                               const int32_t* draft, int32_t* target, int32_t* n_emitted,
                               int32_t* emitted, float* y, int32_t* len, int32_t* next, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!x) return nest::fail(NEST_EINVAL, "verify_accept_x: null pointer");
  return accept_impl("verify_accept_x", Act{nullptr, nullptr, x}, B, k, K, base, refine, scales, V,
                     group, draft, target, n_emitted, emitted, y, len, next, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// verify_accept_x without a caller workspace, for callers that cannot
// allocate: the workspace is a file-scope device array of kStaticScratch
// bytes, one copy per device, held until the process ends.
// ---------------------------------------------------------------------------

#include <mutex>

namespace {

constexpr size_t kStaticScratch = size_t{1} << 20;
constexpr int kMaxDevices = 64;

// Zero when the library loads; the only part that must be zero before a
// call (the counter zone at its start) is returned to zero by every call,
// and the rest needs no initial contents.
__device__ __align__(256) unsigned char scratch[kStaticScratch];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (with that device current); the host-side name of the array is not
// a device address and is never passed to a kernel.
int static_scratch(const char* what, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nest::fail(NEST_EHIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return nest::fail(NEST_EUNSUPPORTED, "%s: device %d", what, dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return nest::fail(NEST_EHIP, "%s: hipGetSymbolAddress: %s", what, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NEST_OK;
}

}  // namespace

extern "C" int verify_accept_x_static(const float* x, int64_t B, int64_t k, int64_t K, const uint8_t* base,
                                      const uint8_t* refine, const float* scales, int64_t V, int64_t group,
                                      const int32_t* draft, int32_t* target, int32_t* n_emitted,
                                      int32_t* emitted, float* y, int32_t* len, int32_t* next, void* stream) {
  const char* what = "verify_accept_x_static";
  if (!x) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (B < 1 || k < 0 || K < 1 || V < 1 || B * (k + 1) > 16 || K > (1LL << 24) || V > (1LL << 30))
    return nest::fail(NEST_EINVAL, "%s: B=%lld k=%lld K=%lld V=%lld", what, (long long)B, (long long)k,
                      (long long)K, (long long)V);
  const size_t need = gemv_ws_bytes(B * (k + 1), K, V, true);
  if (need > kStaticScratch)
    return nest::fail(NEST_EUNSUPPORTED, "%s: needs %zu bytes of scratch, more than its %zu", what, need,
                      kStaticScratch);
  void* ws = nullptr;
  const int rc = static_scratch(what, &ws);
  if (rc) return rc;
  return accept_impl(what, Act{nullptr, nullptr, x}, B, k, K, base, refine, scales, V, group, draft, target,
                     n_emitted, emitted, y, len, next, ws, kStaticScratch, stream);
}

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
// only the planes and scales from HBM. Blocks loop over tiles with a grid
// stride, and the grid is at most what fits on the chip. The argmax path
// keeps per-lane best (value, index) keys across tiles and writes one key
// per row and block. A second small kernel reduces the keys and, for
// verify_accept, applies the accept rule. The kernel boundary makes the
// keys visible, with no cross-block fence or atomic.
#include "nibble.h"

namespace {

using nest::kGroup;
using nest::ld16;

constexpr int kMaxArgmaxBlocks = 4096;
constexpr int kLdsActMax = 48 * 1024;  // largest M*K staged in LDS

struct GemvArgs {
  const int8_t* qa;
  const float* sa;
  int M, K;
  const uint8_t* base;
  const uint8_t* refine;
  const float* scales;
  int N, G, nseg;
  float* y;
  int32_t* acc_dbg;
  unsigned long long* partials;  // argmax: [gridDim.x][16]
};

struct FinishArgs {
  const unsigned long long* partials;
  int nparts, M;
  int32_t* argmax_out;  // draft: [M]
  int B, k;             // accept: B sequences of k+1 rows
  const int32_t* draft;
  int32_t* target;
  int32_t* n_emitted;
  int32_t* emitted;
};

// LDS slot of the even (p = 0) or odd (p = 1) operand of activation row m,
// k-quarter kq, group g.
__device__ __forceinline__ int lds_slot(int g, int p, int kq, int m, int M) {
  return ((g * 2 + p) * 4 + kq) * M + m;
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

// Fold groups [g0, g1) of one tile. A4: G % 4 == 0 and the segment is
// 4-aligned, so the lane's scales load as one float4 per four groups and
// the plane stream is software-pipelined by four groups.
template <int PLANES, int MR, bool DBG, bool A4, bool LDSACT>
__device__ __forceinline__ void gemv_segment(const GemvArgs& a, const uint4* lds, const uint8_t* pb,
                                             const uint8_t* pr, const float* ps, const int8_t* pa,
                                             int kq, int mrow, int n, int g0, int g1, float (&run)[MR]) {
  if (A4) {
    uint4 b0, b1, b2, b3, r0, r1, r2, r3;
    auto load = [&](int g, uint4& x0, uint4& x1, uint4& x2, uint4& x3, uint4& y0, uint4& y1,
                    uint4& y2, uint4& y3) {
      x0 = ld16(pb + static_cast<size_t>(g) * 64);
      x1 = ld16(pb + static_cast<size_t>(g + 1) * 64);
      x2 = ld16(pb + static_cast<size_t>(g + 2) * 64);
      x3 = ld16(pb + static_cast<size_t>(g + 3) * 64);
      if (PLANES == 2) {
        y0 = ld16(pr + static_cast<size_t>(g) * 64);
        y1 = ld16(pr + static_cast<size_t>(g + 1) * 64);
        y2 = ld16(pr + static_cast<size_t>(g + 2) * 64);
        y3 = ld16(pr + static_cast<size_t>(g + 3) * 64);
      } else {
        y0 = y1 = y2 = y3 = make_uint4(0, 0, 0, 0);
      }
    };
    if (g0 < g1) load(g0, b0, b1, b2, b3, r0, r1, r2, r3);
    for (int g = g0; g < g1; g += 4) {
      uint4 nb0, nb1, nb2, nb3, nr0, nr1, nr2, nr3;
      if (g + 4 < g1) load(g + 4, nb0, nb1, nb2, nb3, nr0, nr1, nr2, nr3);
      const float4 s = *reinterpret_cast<const float4*>(ps + g);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g, b0, r0, s.x, run);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 1, b1, r1, s.y, run);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 2, b2, r2, s.z, run);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g + 3, b3, r3, s.w, run);
      b0 = nb0; b1 = nb1; b2 = nb2; b3 = nb3;
      r0 = nr0; r1 = nr1; r2 = nr2; r3 = nr3;
    }
  } else {
    for (int g = g0; g < g1; ++g) {
      const uint4 wb = ld16(pb + static_cast<size_t>(g) * 64);
      const uint4 wr = PLANES == 2 ? ld16(pr + static_cast<size_t>(g) * 64) : make_uint4(0, 0, 0, 0);
      gemv_group<PLANES, MR, DBG, LDSACT>(a, lds, pa, kq, mrow, n, g, wb, wr, ps[g], run);
    }
  }
}

// WAVES waves per block; a tile takes nseg consecutive waves (nseg | WAVES).
// ARGMAX requires nseg == 1.
template <int PLANES, int MR, int WAVES, bool ARGMAX, bool DBG, bool A4, bool LDSACT>
__global__ void __launch_bounds__(WAVES * 64) gemv_kernel(GemvArgs a) {
  extern __shared__ uint4 lds_act[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int S = a.nseg, per_iter = WAVES / S;
  const int T = (a.N + 15) / 16, iters = (T + per_iter - 1) / per_iter;
  const int seg = wave % S, G = a.G;
  const int unit = A4 ? 4 : 1, units = G / unit;
  const int g_begin = static_cast<int>(static_cast<long long>(seg) * units / S) * unit;
  const int g_end = static_cast<int>(static_cast<long long>(seg + 1) * units / S) * unit;
  const int kq = lane >> 4, c = lane & 15;
  const int mrow = min(c, a.M - 1);  // A-operand row of this lane (rows past M fill unused D rows)
  const size_t rowb = static_cast<size_t>(a.K / 2);
  const int8_t* pa = a.qa + static_cast<size_t>(mrow) * a.K + kq * 32;

  if (LDSACT) {
    // stage all M x K activation bytes once, split into operand order
    const int units32 = a.M * G * 4;
    for (int u = threadIdx.x; u < units32; u += WAVES * 64) {
      const int m = u % a.M, rest = u / a.M, q = rest & 3, g = rest >> 2;
      const int8_t* src = a.qa + static_cast<size_t>(m) * a.K + g * kGroup + q * 32;
      v4i e, o;
      nest::split_act(ld16(src), ld16(src + 16), e, o);
      lds_act[lds_slot(g, 0, q, m, a.M)] = __builtin_bit_cast(uint4, e);
      lds_act[lds_slot(g, 1, q, m, a.M)] = __builtin_bit_cast(uint4, o);
    }
    __syncthreads();
  }

  unsigned long long best[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) best[r] = 0;
  float s_a[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) s_a[r] = a.sa[min(4 * kq + r, a.M - 1)];

  for (int it = blockIdx.x; it < iters; it += gridDim.x) {
    const int n0 = (it * per_iter + wave / S) * 16;
    const bool tile_ok = n0 < a.N;
    const int n = n0 + c;  // this lane's output column (weight row)
    const int wrow = min(n, a.N - 1);
    const uint8_t* pb = a.base + wrow * rowb + kq * 16;
    const uint8_t* pr = PLANES == 2 ? a.refine + wrow * rowb + kq * 16 : nullptr;
    const float* ps = a.scales + static_cast<size_t>(wrow) * G;
    float run[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) run[r] = 0.0f;
    if (tile_ok)
      gemv_segment<PLANES, MR, DBG, A4, LDSACT>(a, lds_act, pb, pr, ps, pa, kq, mrow, n, g_begin,
                                                g_end, run);

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
      continue;
    }

    float tot[MR];
    if (S > 1) {
      __shared__ float part[WAVES][MR][64];
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
    if (seg != 0 || !tile_ok || n >= a.N) continue;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int m = 4 * kq + r;
      if (m < a.M) a.y[static_cast<size_t>(m) * a.N + n] = tot[r] * s_a[r];
    }
  }

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
      a.partials[static_cast<size_t>(blockIdx.x) * 16 + threadIdx.x] = k;
    }
  }
}

// Reduce the per-block argmax keys; ACCEPT also applies the accept rule.
// One block of 1024 threads: 64 strands per row.
template <bool ACCEPT>
__global__ void __launch_bounds__(1024) argmax_finish_kernel(FinishArgs f) {
  __shared__ unsigned long long red[64][16];
  __shared__ int32_t tgt[16];
  const int m = threadIdx.x & 15, p = threadIdx.x >> 4;
  unsigned long long k = 0;
#pragma unroll 8
  for (int b = p; b < f.nparts; b += 64) k = umax64(k, f.partials[static_cast<size_t>(b) * 16 + m]);
  red[p][m] = k;
  __syncthreads();
  if (threadIdx.x < 16) {
    unsigned long long t = 0;
    for (int q = 0; q < 64; ++q) t = umax64(t, red[q][threadIdx.x]);
    tgt[threadIdx.x] = static_cast<int32_t>(argmax_key_index(t));
    if (!ACCEPT && threadIdx.x < f.M) f.argmax_out[threadIdx.x] = tgt[threadIdx.x];
  }
  __syncthreads();
  if (ACCEPT && threadIdx.x < f.B) {
    // One thread per sequence: slot i's draft d_i is checked against
    // t_{i-1}; the first mismatch ends the round.
    const int b = threadIdx.x, k1 = f.k + 1;
    int acc = 0;
    while (acc < f.k && f.draft[b * f.k + acc] == tgt[b * k1 + acc]) ++acc;
    f.n_emitted[b] = acc + 1;
    for (int j = 0; j < k1; ++j) {
      f.target[b * k1 + j] = tgt[b * k1 + j];
      f.emitted[b * k1 + j] = j <= acc ? tgt[b * k1 + j] : -1;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int pick_split(int tiles, int G) {
  // Enough waves to keep HBM busy (~8 per CU), at least two groups each.
  int s = 1;
  while (s < 16 && static_cast<long long>(tiles) * s < 2048 && G / (2 * s) >= 2) s *= 2;
  return s;
}

template <int PLANES, int MR, int WAVES, bool ARGMAX, bool DBG, bool A4, bool LDSACT>
int launch_one(const GemvArgs& a, hipStream_t st, const char* what, int max_blocks, int* used) {
  auto kern = gemv_kernel<PLANES, MR, WAVES, ARGMAX, DBG, A4, LDSACT>;
  const size_t lds = LDSACT ? static_cast<size_t>(a.M) * a.K : 0;
  const int per_iter = WAVES / a.nseg;
  const int iters = ((a.N + 15) / 16 + per_iter - 1) / per_iter;
  int blocks = min(iters, nest::resident_blocks(reinterpret_cast<const void*>(kern), WAVES * 64, lds));
  blocks = min(blocks, max_blocks);
  if (used) *used = blocks;
  kern<<<dim3(blocks), dim3(WAVES * 64), lds, st>>>(a);
  return nest::check_launch(what);
}

template <int PLANES, int MR, bool ARGMAX, bool DBG, bool A4, bool LDSACT>
int launch_waves(const GemvArgs& a, hipStream_t st, const char* what, int max_blocks, int* used) {
  if (ARGMAX || a.nseg <= 4)
    return launch_one<PLANES, MR, 4, ARGMAX, DBG, A4, LDSACT>(a, st, what, max_blocks, used);
  if constexpr (!ARGMAX) {
    if (a.nseg == 8) return launch_one<PLANES, MR, 8, false, DBG, A4, LDSACT>(a, st, what, max_blocks, used);
    return launch_one<PLANES, MR, 16, false, DBG, A4, LDSACT>(a, st, what, max_blocks, used);
  }
  return NEST_EHIP;
}

template <int PLANES, bool ARGMAX, bool DBG>
int launch_gemv(const GemvArgs& a, hipStream_t st, const char* what, int max_blocks, int* used) {
  const bool a4 = a.G % 4 == 0 && nest::aligned16(a.scales);
  const bool ldsact = a4 && static_cast<long long>(a.M) * a.K <= kLdsActMax;
  if (a.M == 1) {
    if (ldsact) return launch_waves<PLANES, 1, ARGMAX, DBG, true, true>(a, st, what, max_blocks, used);
    if (a4) return launch_waves<PLANES, 1, ARGMAX, DBG, true, false>(a, st, what, max_blocks, used);
    return launch_waves<PLANES, 1, ARGMAX, DBG, false, false>(a, st, what, max_blocks, used);
  }
  if (ldsact) return launch_waves<PLANES, 4, ARGMAX, DBG, true, true>(a, st, what, max_blocks, used);
  if (a4) return launch_waves<PLANES, 4, ARGMAX, DBG, true, false>(a, st, what, max_blocks, used);
  return launch_waves<PLANES, 4, ARGMAX, DBG, false, false>(a, st, what, max_blocks, used);
}

size_t argmax_ws_bytes(int N) {
  const int iters = ((N + 15) / 16 + 3) / 4;
  return static_cast<size_t>(min(iters, kMaxArgmaxBlocks)) * 16 * sizeof(unsigned long long);
}

// The exact-fold argmax GEMV and its finishing kernel.
template <int PLANES, bool DBG>
int launch_argmax(GemvArgs a, const FinishArgs& f0, bool accept, hipStream_t st, const char* what) {
  a.nseg = 1;
  int used = 0;
  int rc = launch_gemv<PLANES, true, DBG>(a, st, what, kMaxArgmaxBlocks, &used);
  if (rc) return rc;
  FinishArgs f = f0;
  f.partials = a.partials;
  f.nparts = used;
  f.M = a.M;
  if (accept)
    argmax_finish_kernel<true><<<1, 1024, 0, st>>>(f);
  else
    argmax_finish_kernel<false><<<1, 1024, 0, st>>>(f);
  return nest::check_launch(what);
}

int check_common(const char* what, const int8_t* qa, const float* sa, int64_t M, int64_t K,
                 const uint8_t* base, const float* scales, int64_t N, int64_t group) {
  if (!qa || !sa || !base || !scales) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (M < 1 || K < 1 || N < 1) return nest::fail(NEST_EINVAL, "%s: empty shape", what);
  if (group != kGroup)
    return nest::fail(NEST_EUNSUPPORTED, "%s: group=%lld (kernels handle 128)", what, (long long)group);
  if (K % kGroup) return nest::fail(NEST_ESHAPE, "%s: K=%lld is not a multiple of 128", what, (long long)K);
  if (K > (1LL << 24) || N > (1LL << 30) || M > (1LL << 20))
    return nest::fail(NEST_EUNSUPPORTED, "%s: shape too large", what);
  if (!nest::aligned16(qa) || !nest::aligned16(base))
    return nest::fail(NEST_EALIGN, "%s: qa and planes must be 16-byte aligned", what);
  return NEST_OK;
}

}  // namespace

extern "C" size_t draft_gemv_workspace_size(int64_t M, int64_t N) {
  (void)M;
  if (N < 1 || N > (1LL << 30)) return 0;
  return argmax_ws_bytes(static_cast<int>(N));
}

extern "C" size_t verify_accept_workspace_size(int64_t B, int64_t k, int64_t V) {
  (void)B;
  (void)k;
  if (V < 1 || V > (1LL << 30)) return 0;
  return argmax_ws_bytes(static_cast<int>(V));
}

extern "C" int draft_gemv(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                          const uint8_t* base, const float* scales, int64_t N, int64_t group,
                          float* y, int32_t* argmax, int32_t* acc_dbg, void* ws, size_t ws_bytes,
                          void* stream) {
  const char* what = "draft_gemv";
  int rc = check_common(what, qa, sa, M, K, base, scales, N, group);
  if (rc) return rc;
  if (M > 16) return nest::fail(NEST_EUNSUPPORTED, "draft_gemv: M=%lld > 16", (long long)M);
  if (!y && !argmax) return nest::fail(NEST_EINVAL, "draft_gemv: need y or argmax");
  GemvArgs a{};
  a.qa = qa; a.sa = sa; a.M = (int)M; a.K = (int)K; a.base = base; a.scales = scales;
  a.N = (int)N; a.G = (int)(K / kGroup); a.y = y; a.acc_dbg = acc_dbg;
  hipStream_t st = nest::as_stream(stream);
  if (argmax) {
    if (!ws || ws_bytes < argmax_ws_bytes(a.N))
      return nest::fail(NEST_EWORKSPACE, "draft_gemv: workspace needs %zu bytes", argmax_ws_bytes(a.N));
    a.partials = static_cast<unsigned long long*>(ws);
    FinishArgs f{};
    f.argmax_out = argmax;
    return acc_dbg ? launch_argmax<1, true>(a, f, false, st, what)
                   : launch_argmax<1, false>(a, f, false, st, what);
  }
  a.nseg = pick_split((a.N + 15) / 16, a.G);
  return acc_dbg ? launch_gemv<1, false, true>(a, st, what, 1 << 30, nullptr)
                 : launch_gemv<1, false, false>(a, st, what, 1 << 30, nullptr);
}

extern "C" int verify_gemm(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                           const uint8_t* base, const uint8_t* refine, const float* scales,
                           int64_t N, int64_t group, float* y, int32_t* acc_dbg, void* stream) {
  const char* what = "verify_gemm";
  int rc = check_common(what, qa, sa, M, K, base, scales, N, group);
  if (rc) return rc;
  if (!refine || !y) return nest::fail(NEST_EINVAL, "verify_gemm: null pointer");
  if (!nest::aligned16(refine)) return nest::fail(NEST_EALIGN, "verify_gemm: refine not 16-byte aligned");
  hipStream_t st = nest::as_stream(stream);
  if (M <= 16) {
    GemvArgs a{};
    a.qa = qa; a.sa = sa; a.M = (int)M; a.K = (int)K; a.base = base; a.refine = refine;
    a.scales = scales; a.N = (int)N; a.G = (int)(K / kGroup); a.y = y; a.acc_dbg = acc_dbg;
    a.nseg = pick_split((a.N + 15) / 16, a.G);
    return acc_dbg ? launch_gemv<2, false, true>(a, st, what, 1 << 30, nullptr)
                   : launch_gemv<2, false, false>(a, st, what, 1 << 30, nullptr);
  }
  // More rows: the batched kernel, in chunks of up to 144 rows.
  for (int64_t m0 = 0; m0 < M; m0 += 144) {
    const int64_t mc = M - m0 < 144 ? M - m0 : 144;
    rc = nest::launch_verify_batched(qa + m0 * K, sa + m0, (int)mc, (int)K, base, refine, scales,
                                     (int)N, y + m0 * N,
                                     acc_dbg ? acc_dbg + m0 * N * (K / kGroup) : nullptr, st);
    if (rc) return rc;
  }
  return NEST_OK;
}

extern "C" int verify_accept(const int8_t* qa, const float* sa, int64_t B, int64_t k, int64_t K,
                             const uint8_t* base, const uint8_t* refine, const float* scales,
                             int64_t V, int64_t group, const int32_t* draft, int32_t* target,
                             int32_t* n_emitted, int32_t* emitted, float* y, void* ws,
                             size_t ws_bytes, void* stream) {
  const char* what = "verify_accept";
  if (B < 1 || k < 0) return nest::fail(NEST_EINVAL, "verify_accept: B=%lld k=%lld", (long long)B, (long long)k);
  if (B * (k + 1) > 16)
    return nest::fail(NEST_EUNSUPPORTED, "verify_accept: B*(k+1)=%lld > 16", (long long)(B * (k + 1)));
  int rc = check_common(what, qa, sa, B * (k + 1), K, base, scales, V, group);
  if (rc) return rc;
  if (!refine || !target || !n_emitted || !emitted || (k > 0 && !draft))
    return nest::fail(NEST_EINVAL, "verify_accept: null pointer");
  if (!nest::aligned16(refine)) return nest::fail(NEST_EALIGN, "verify_accept: refine not 16-byte aligned");
  if (V > 0x7fffffffLL) return nest::fail(NEST_EUNSUPPORTED, "verify_accept: V too large");
  if (!ws || ws_bytes < argmax_ws_bytes((int)V))
    return nest::fail(NEST_EWORKSPACE, "verify_accept: workspace needs %zu bytes", argmax_ws_bytes((int)V));
  GemvArgs a{};
  a.qa = qa; a.sa = sa; a.M = (int)(B * (k + 1)); a.K = (int)K; a.base = base; a.refine = refine;
  a.scales = scales; a.N = (int)V; a.G = (int)(K / kGroup); a.y = y;
  a.partials = static_cast<unsigned long long*>(ws);
  FinishArgs f{};
  f.B = (int)B; f.k = (int)k; f.draft = draft; f.target = target; f.n_emitted = n_emitted;
  f.emitted = emitted;
  return launch_argmax<2, false>(a, f, true, nest::as_stream(stream), what);
}

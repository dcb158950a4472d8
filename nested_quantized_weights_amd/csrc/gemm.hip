// Batched verify over both planes (BitNest, Figure 3: the target reads the
// base and the refinement plane) for more than 16 activation rows, e.g. 16
// sequences x (k+1) = 144 rows.
//
// One wave owns a 16-row weight tile in the tile layout (the MFMA A operand:
// row lane & 15, k-quarter lane >> 4; one contiguous kilobyte per group) and
// all CT 16-row column tiles of activations. Per
// group, the plane bytes are unpacked once and reused for every column
// tile: two v_mfma_i32_16x16x64_i8 per plane and tile. The fp32 fold stays
// in registers, one run per (column tile, row) entry, in ascending group
// order. A block of four waves may split a tile's groups into S <= 4
// contiguous segments, whose partial sums are added in segment order.
#include "nibble.h"

namespace {

using nest::kGroup;

struct GemmArgs {
  const int8_t* qa;
  const float* sa;
  int M, K;
  const uint8_t* base;
  const uint8_t* refine;
  const float* scales;
  int N, G, nseg;
  float* y;
  int32_t* acc_dbg;
};

template <int CT, bool DBG>
__device__ __forceinline__ void gemm_group(const GemmArgs& a, const int8_t* pa, int col, int n_out0, int g,
                                           uint4 wb, uint4 wr, float4 s, float (&run)[CT][4]) {
  v4i wbe, wbo, wre, wro;
  nest::split_nib(wb, wbe, wbo);
  nest::split_nib(wr, wre, wro);
  const float sc[4] = {s.x * 0.0625f, s.y * 0.0625f, s.z * 0.0625f, s.w * 0.0625f};
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    // activation row c*16 + col (clamped; rows past M only fill unused columns)
    const int m = min(c * 16 + col, a.M - 1);
    const int8_t* p = pa + static_cast<size_t>(m) * a.K + static_cast<size_t>(g) * kGroup;
    v4i xe, xo;
    nest::split_act(nest::ld16(p), nest::ld16(p + 16), xe, xo);
    const v4i z = {0, 0, 0, 0};
    v4i rb = nest::mfma_i8(wbe, xe, z);
    rb = nest::mfma_i8(wbo, xo, rb);
    v4i rr = nest::mfma_i8(wre, xe, z);
    rr = nest::mfma_i8(wro, xo, rr);
    const v4i acc = rb + (rr >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) run[c][r] = fmaf(sc[r], static_cast<float>(acc[r]), run[c][r]);
    if (DBG && c * 16 + col < a.M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n_out0 + r;
        if (n < a.N) a.acc_dbg[(static_cast<size_t>(c * 16 + col) * a.N + n) * a.G + g] = acc[r];
      }
    }
  }
}

template <int CT, bool DBG>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int S = a.nseg, per_iter = 4 / S;
  const int T = (a.N + 15) / 16, iters = (T + per_iter - 1) / per_iter;
  const int seg = wave % S, G = a.G;
  const int g_begin = static_cast<int>(static_cast<long long>(seg) * G / S);
  const int g_end = static_cast<int>(static_cast<long long>(seg + 1) * G / S);
  const int kq = lane >> 4, col = lane & 15;
  const int Gq = (G + 3) / 4;
  const int8_t* pa = a.qa + kq * 32;
  __shared__ float part[4][CT][4][64];

  for (int it = blockIdx.x; it < iters; it += gridDim.x) {
    const int n0 = (it * per_iter + wave / S) * 16;
    const bool tile_ok = n0 < a.N;
    const int n_out0 = n0 + 4 * kq;
    // tile layout: lane (kq, col) reads 16 bytes of row n0 + col at
    // ((t*G + g)*4 + kq)*256 + col*16; the scales of rows n0 + 4kq + r sit at
    // ((t*Gq + g/4)*16 + 4kq + r)*4 + g%4 (padded rows and groups hold 0)
    const size_t t = static_cast<size_t>(n0 / 16);
    const uint8_t* pb = a.base + (t * G * 4 + kq) * 256 + col * 16;
    const uint8_t* pr = a.refine + (t * G * 4 + kq) * 256 + col * 16;
    const float* ps = a.scales + (t * Gq * 16 + 4 * kq) * 4;
    float run[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) run[c][r] = 0.0f;
    if (tile_ok) {
      for (int g = g_begin; g < g_end; ++g) {
        const uint4 wb = nest::ldnt16(pb + static_cast<size_t>(g) * 1024);
        const uint4 wr = nest::ldnt16(pr + static_cast<size_t>(g) * 1024);
        const float* pq = ps + static_cast<size_t>(g / 4) * 64 + (g & 3);
        const float4 s = make_float4(pq[0], pq[4], pq[8], pq[12]);
        gemm_group<CT, DBG>(a, pa, col, n_out0, g, wb, wr, s, run);
      }
    }
    float tot[CT][4];
    if (S > 1) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][c][r][lane] = run[c][r];
      __syncthreads();
      if (seg == 0) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float t = part[wave][c][r][lane];
            for (int s2 = 1; s2 < S; ++s2) t += part[wave + s2][c][r][lane];
            tot[c][r] = t;
          }
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[c][r] = run[c][r];
    }
    if (seg != 0 || !tile_ok) continue;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int m = c * 16 + col;
      if (m >= a.M) continue;
      const float sm = a.sa[m];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n_out0 + r;
        if (n < a.N) a.y[static_cast<size_t>(m) * a.N + n] = tot[c][r] * sm;
      }
    }
  }
}

template <int CT, bool DBG>
int launch(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  const int tiles = (a.N + 15) / 16;
  a.nseg = 1;
  while (a.nseg < 4 && tiles * a.nseg < 1024 && a.G / (2 * a.nseg) >= 2) a.nseg *= 2;
  auto kern = gemm_kernel<CT, DBG>;
  const int per_iter = 4 / a.nseg;
  const int iters = (tiles + per_iter - 1) / per_iter;
  const int blocks = min(iters, nest::resident_blocks(reinterpret_cast<const void*>(kern), 256, 0));
  kern<<<dim3(blocks), dim3(256), 0, st>>>(a);
  return nest::check_launch("verify_gemm(batched)");
}

template <bool DBG>
int launch_ct(const GemmArgs& a, int CT, hipStream_t st) {
  switch (CT) {
    case 2: return launch<2, DBG>(a, st);
    case 3: return launch<3, DBG>(a, st);
    case 4: return launch<4, DBG>(a, st);
    case 5: return launch<5, DBG>(a, st);
    case 6: return launch<6, DBG>(a, st);
    case 7: return launch<7, DBG>(a, st);
    case 8: return launch<8, DBG>(a, st);
    default: return launch<9, DBG>(a, st);
  }
}

}  // namespace

namespace nest {

int launch_verify_batched(const int8_t* qa, const float* sa, int M, int K, const uint8_t* base,
                          const uint8_t* refine, const float* scales, int N, float* y,
                          int32_t* acc_dbg, hipStream_t st) {
  GemmArgs a{};
  a.qa = qa; a.sa = sa; a.M = M; a.K = K; a.base = base; a.refine = refine; a.scales = scales;
  a.N = N; a.G = K / kGroup; a.y = y; a.acc_dbg = acc_dbg;
  const int CT = (M + 15) / 16;
  return acc_dbg ? launch_ct<true>(a, CT, st) : launch_ct<false>(a, CT, st);
}

}  // namespace nest

// Draft and verify products over the dual-plane nested weights (BitNest,
// Figure 3: the draft reads the base plane, the target reads both), the
// fused LM-head argmax, and the greedy accept step of a round ("How
// Speculative Decoding Speeds Up Inference", numbered round steps, Table 1).
//
// Layout on gfx950. One wave owns a tile of 16 weight rows. Per group of
// 128 weights, lane l loads 16 bytes of each plane: row (l & 15) of the
// tile, k-quarter (l >> 4). The nibbles become int8 operands of
// v_mfma_i32_16x16x64_i8 without any cross-lane traffic:
//   even elements: (w << 4) & 0xF0F0F0F0   (16 * code)
//   odd  elements:  w       & 0xF0F0F0F0   (16 * code)
// The activation operand holds the same k-quarter of activation row
// (l & 15). It is split into even and odd bytes by v_perm_b32 to match. One
// group is two MFMAs per plane. The D tile gives lane l column m = l & 15
// and rows 4*(l>>4)+r, so the per-group fp32 fold stays in registers and
// runs in ascending group order, as the reference fold does.
//   draft:  A_b = R_b >> 4,            run = fmaf(s,        A_b, run)
//   verify: A_v = R_b + (R_r >> 4),    run = fmaf(s * 2^-4, A_v, run)
// where R_b and R_r are the MFMA sums over 16*q_b and 16*q_r (all exact
// int32). With one segment per tile the result is bit-identical to the
// reference fold. With S > 1 segments the waves of a block fold contiguous
// group ranges, and their partial sums are added in segment order.
#include "common.h"

namespace {

constexpr int kGroup = 128;
constexpr unsigned kHiNib = 0xF0F0F0F0u;
constexpr int kWsHeader = 256;  // bytes: the arrival counter, padded

struct GemvArgs {
  const int8_t* qa;
  const float* sa;
  int M, K;
  const uint8_t* base;
  const uint8_t* refine;
  const float* scales;
  int N, G;
  int nseg;
  float* y;
  int32_t* acc_dbg;
  // argmax / accept epilogue
  unsigned int* counter;
  unsigned long long* partials;  // [gridDim.x][16]
  int32_t* argmax_out;           // [M] (draft) or unused (accept)
  int B, k;                      // accept: B sequences of k+1 rows
  const int32_t* draft;
  int32_t* target;
  int32_t* n_emitted;
  int32_t* emitted;
};

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

template <int PLANES, int CT>
struct GroupData {
  uint4 wb, wr;
  float s[4];
};

// One group of the tile: accumulate into run[CT][4].
template <int PLANES, int CT, bool DBG>
__device__ __forceinline__ void do_group(const GemvArgs& a, const GroupData<PLANES, CT>& d,
                                         const int8_t* pa, int g, int col, int n_out0,
                                         const uint4* pre_a, float (&run)[CT][4]) {
  v4i wbe, wbo, wre, wro;  // weight operands: base / refine, even / odd
  split_nib(d.wb, wbe, wbo);
  if (PLANES == 2) split_nib(d.wr, wre, wro);
  float sc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sc[r] = PLANES == 2 ? d.s[r] * 0.0625f : d.s[r];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    uint4 a0, a1;
    if (pre_a) {
      a0 = pre_a[0];
      a1 = pre_a[1];
    } else {
      const int m = c * 16 + col;
      if (m < a.M) {
        const int8_t* p = pa + static_cast<size_t>(c * 16) * a.K + static_cast<size_t>(g) * kGroup;
        a0 = *reinterpret_cast<const uint4*>(p);
        a1 = *reinterpret_cast<const uint4*>(p + 16);
      } else {
        a0 = make_uint4(0, 0, 0, 0);
        a1 = a0;
      }
    }
    v4i xe, xo;
    split_act(a0, a1, xe, xo);
    const v4i z = {0, 0, 0, 0};
    v4i rb = mfma_i8(wbe, xe, z);
    rb = mfma_i8(wbo, xo, rb);
    v4i acc;
    if (PLANES == 2) {
      v4i rr = mfma_i8(wre, xe, z);
      rr = mfma_i8(wro, xo, rr);
      acc = rb + (rr >> 4);
    } else {
      acc = rb >> 4;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) run[c][r] = fmaf(sc[r], static_cast<float>(acc[r]), run[c][r]);
    if (DBG) {
      const int m = c * 16 + col;
      if (m < a.M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n_out0 + r;
          if (n < a.N) a.acc_dbg[(static_cast<size_t>(m) * a.N + n) * a.G + g] = acc[r];
        }
      }
    }
  }
}

// WAVES waves per block; a tile takes nseg consecutive waves (nseg | WAVES).
// ARGMAX requires nseg == 1 and CT == 1. ACCEPT implies ARGMAX.
template <int PLANES, int CT, int WAVES, bool ARGMAX, bool ACCEPT, bool DBG>
__global__ void __launch_bounds__(WAVES * 64) gemv_kernel(GemvArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int S = a.nseg;
  const int tile = blockIdx.x * (WAVES / S) + wave / S;
  const int seg = wave % S;
  const int n0 = tile * 16;
  const bool tile_ok = n0 < a.N;
  const int G = a.G;
  const int g_begin = static_cast<int>(static_cast<long long>(seg) * G / S);
  const int g_end = static_cast<int>(static_cast<long long>(seg + 1) * G / S);

  const int kq = lane >> 4, col = lane & 15;
  const int n_out0 = n0 + 4 * kq;  // rows of this lane's D entries: n_out0 + r
  const size_t rowb = static_cast<size_t>(a.K / 2);
  const int arow = min(n0 + col, a.N - 1);
  const uint8_t* pb = a.base + arow * rowb + kq * 16;
  const uint8_t* pr = PLANES == 2 ? a.refine + arow * rowb + kq * 16 : nullptr;
  const int8_t* pa = a.qa + static_cast<size_t>(col) * a.K + kq * 32;  // row c*16+col, added per tile
  const float* ps[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ps[r] = a.scales + static_cast<size_t>(min(n_out0 + r, a.N - 1)) * G;

  float run[CT][4];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) run[c][r] = 0.0f;

  if (tile_ok) {
    constexpr int U = CT == 1 ? 4 : 2;
    int g = g_begin;
    for (; g + U <= g_end; g += U) {
      GroupData<PLANES, CT> d[U];
      uint4 act[U][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        d[u].wb = *reinterpret_cast<const uint4*>(pb + static_cast<size_t>(g + u) * 64);
        if (PLANES == 2) d[u].wr = *reinterpret_cast<const uint4*>(pr + static_cast<size_t>(g + u) * 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) d[u].s[r] = ps[r][g + u];
        if (CT == 1) {
          if (col < a.M) {
            const int8_t* p = pa + static_cast<size_t>(g + u) * kGroup;
            act[u][0] = *reinterpret_cast<const uint4*>(p);
            act[u][1] = *reinterpret_cast<const uint4*>(p + 16);
          } else {
            act[u][0] = make_uint4(0, 0, 0, 0);
            act[u][1] = act[u][0];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        do_group<PLANES, CT, DBG>(a, d[u], pa, g + u, col, n_out0, CT == 1 ? act[u] : nullptr, run);
    }
    for (; g < g_end; ++g) {
      GroupData<PLANES, CT> d;
      d.wb = *reinterpret_cast<const uint4*>(pb + static_cast<size_t>(g) * 64);
      if (PLANES == 2) d.wr = *reinterpret_cast<const uint4*>(pr + static_cast<size_t>(g) * 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) d.s[r] = ps[r][g];
      do_group<PLANES, CT, DBG>(a, d, pa, g, col, n_out0, nullptr, run);
    }
  }

  if (!ARGMAX) {
    float tot[CT][4];
    if (WAVES > 1 && S > 1) {
      __shared__ float part[WAVES][CT][4][64];
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][c][r][lane] = run[c][r];
      __syncthreads();
      if (seg != 0) return;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float t = part[wave][c][r][lane];
          for (int s = 1; s < S; ++s) t += part[wave + s][c][r][lane];
          tot[c][r] = t;
        }
    } else {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[c][r] = run[c][r];
    }
    if (!tile_ok) return;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int m = c * 16 + col;
      if (m >= a.M) continue;
      const float s_a = a.sa[m];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n_out0 + r;
        if (n < a.N) a.y[static_cast<size_t>(m) * a.N + n] = tot[c][r] * s_a;
      }
    }
    return;
  }

  // ---- argmax epilogue (nseg == 1, CT == 1): exact fold, per-block best ----
  __shared__ unsigned long long best[WAVES][16];
  __shared__ unsigned long long red[WAVES * 4][16];
  __shared__ int32_t tgt[16];
  __shared__ int last;
  {
    unsigned long long key = 0;
    if (tile_ok && col < a.M) {
      const float s_a = a.sa[col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n_out0 + r;
        if (n < a.N) {
          const float v = run[0][r] * s_a;
          if (a.y) a.y[static_cast<size_t>(col) * a.N + n] = v;
          key = umax64(key, argmax_key(v, static_cast<uint32_t>(n)));
        }
      }
    }
    key = umax64(key, shfl_xor_u64(key, 16));
    key = umax64(key, shfl_xor_u64(key, 32));
    if (lane < 16) best[wave][lane] = key;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    unsigned long long k = 0;
    for (int w = 0; w < WAVES; ++w) k = umax64(k, best[w][threadIdx.x]);
    a.partials[static_cast<size_t>(blockIdx.x) * 16 + threadIdx.x] = k;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (prev == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  {
    // Thread t reduces column t & 15 over blocks p, p + P, p + 2P, ...
    // (p = t >> 4, P = WAVES * 4), then one thread per column folds the P
    // strands. The maximum of u64 keys does not depend on the order.
    constexpr int P = WAVES * 4;
    const int m = threadIdx.x & 15, p = threadIdx.x >> 4;
    unsigned long long k = 0;
    for (unsigned b = p; b < gridDim.x; b += P)
      k = umax64(k, a.partials[static_cast<size_t>(b) * 16 + m]);
    red[p][m] = k;
    __syncthreads();
    if (threadIdx.x < 16) {
      unsigned long long f = 0;
      for (int q = 0; q < P; ++q) f = umax64(f, red[q][threadIdx.x]);
      tgt[threadIdx.x] = static_cast<int32_t>(argmax_key_index(f));
      if (!ACCEPT && threadIdx.x < a.M) a.argmax_out[threadIdx.x] = tgt[threadIdx.x];
    }
    __syncthreads();
  }
  if (ACCEPT && threadIdx.x < a.B) {
    // One thread per sequence: slot i's draft d_i is checked against
    // t_{i-1}; the first mismatch ends the round.
    const int b = threadIdx.x, k1 = a.k + 1;
    int acc = 0;
    while (acc < a.k && a.draft[b * a.k + acc] == tgt[b * k1 + acc]) ++acc;
    a.n_emitted[b] = acc + 1;
    for (int j = 0; j < k1; ++j) {
      a.target[b * k1 + j] = tgt[b * k1 + j];
      a.emitted[b * k1 + j] = j <= acc ? tgt[b * k1 + j] : -1;
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int PLANES, int CT, int WAVES, bool ARGMAX, bool ACCEPT, bool DBG>
int launch_one(const GemvArgs& a, int blocks, hipStream_t st, const char* what) {
  gemv_kernel<PLANES, CT, WAVES, ARGMAX, ACCEPT, DBG><<<dim3(blocks), dim3(WAVES * 64), 0, st>>>(a);
  return nest::check_launch(what);
}

template <int PLANES, int CT, bool DBG>
int launch_split(GemvArgs a, hipStream_t st, const char* what) {
  const int tiles = (a.N + 15) / 16;
  const int S = CT == 1 ? a.nseg : min(a.nseg, 4);
  a.nseg = S;
  const int waves = S <= 4 ? 4 : S;
  const int blocks = (tiles + waves / S - 1) / (waves / S);
  if constexpr (CT == 1) {
    switch (waves) {
      case 4: return launch_one<PLANES, CT, 4, false, false, DBG>(a, blocks, st, what);
      case 8: return launch_one<PLANES, CT, 8, false, false, DBG>(a, blocks, st, what);
      default: return launch_one<PLANES, CT, 16, false, false, DBG>(a, blocks, st, what);
    }
  } else {
    return launch_one<PLANES, CT, 4, false, false, DBG>(a, blocks, st, what);
  }
}

template <int PLANES, bool DBG>
int launch_ct(GemvArgs a, int CT, hipStream_t st, const char* what) {
  switch (CT) {
    case 1: return launch_split<PLANES, 1, DBG>(a, st, what);
    case 2: return launch_split<PLANES, 2, DBG>(a, st, what);
    case 3: return launch_split<PLANES, 3, DBG>(a, st, what);
    case 4: return launch_split<PLANES, 4, DBG>(a, st, what);
    case 5: return launch_split<PLANES, 5, DBG>(a, st, what);
    case 6: return launch_split<PLANES, 6, DBG>(a, st, what);
    case 7: return launch_split<PLANES, 7, DBG>(a, st, what);
    case 8: return launch_split<PLANES, 8, DBG>(a, st, what);
    default: return launch_split<PLANES, 9, DBG>(a, st, what);
  }
}

constexpr int kArgmaxWaves = 4;

int argmax_blocks(int N) { return ((N + 15) / 16 + kArgmaxWaves - 1) / kArgmaxWaves; }

size_t argmax_ws_bytes(int N) {
  return kWsHeader + static_cast<size_t>(argmax_blocks(N)) * 16 * sizeof(unsigned long long);
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
    a.nseg = 1;
    a.counter = static_cast<unsigned int*>(ws);
    a.partials = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + kWsHeader);
    a.argmax_out = argmax;
    const int blocks = argmax_blocks(a.N);
    return acc_dbg ? launch_one<1, 1, kArgmaxWaves, true, false, true>(a, blocks, st, what)
                   : launch_one<1, 1, kArgmaxWaves, true, false, false>(a, blocks, st, what);
  }
  a.nseg = pick_split((a.N + 15) / 16, a.G);
  return acc_dbg ? launch_ct<1, true>(a, 1, st, what) : launch_ct<1, false>(a, 1, st, what);
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
  // Row chunks of up to 144 (nine 16-row column tiles) per launch.
  for (int64_t m0 = 0; m0 < M; m0 += 144) {
    const int64_t mc = M - m0 < 144 ? M - m0 : 144;
    GemvArgs a{};
    a.qa = qa + m0 * K; a.sa = sa + m0; a.M = (int)mc; a.K = (int)K; a.base = base;
    a.refine = refine; a.scales = scales; a.N = (int)N; a.G = (int)(K / kGroup);
    a.y = y + m0 * N;
    a.acc_dbg = acc_dbg ? acc_dbg + m0 * N * (K / kGroup) : nullptr;
    const int CT = (int)((mc + 15) / 16);
    a.nseg = pick_split((a.N + 15) / 16, a.G);
    rc = acc_dbg ? launch_ct<2, true>(a, CT, st, what) : launch_ct<2, false>(a, CT, st, what);
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
  a.scales = scales; a.N = (int)V; a.G = (int)(K / kGroup); a.nseg = 1; a.y = y;
  a.counter = static_cast<unsigned int*>(ws);
  a.partials = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + kWsHeader);
  a.B = (int)B; a.k = (int)k; a.draft = draft; a.target = target; a.n_emitted = n_emitted;
  a.emitted = emitted;
  return launch_one<2, 1, kArgmaxWaves, true, true, false>(a, argmax_blocks(a.N), nest::as_stream(stream), what);
}

// Nested quantization (BitNest, Figure 2: a base, then the remaining error
// as a refinement; Figure 3: two independent 4-bit planes), the nested KV
// cache builder (Figure 4), and per-token int8 activations.
//
// Each quantization group is one wave. Lanes read the group coalesced for
// the max-abs pass, then each lane codes adjacent element pairs, which are
// one byte in each plane. Every division is IEEE fp32 (correctly rounded,
// HIP's default), rintf rounds ties to even, and the residual is one fmaf,
// so the codes are those of the rule in nestspec.h bit for bit.
#include "common.h"

namespace {

__device__ __forceinline__ void nest_codes(float w, float s, float s16, int& qb, int& qr) {
  if (s == 0.0f) {
    qb = 0;
    qr = 0;
    return;
  }
  int b = static_cast<int>(rintf(w / s));
  b = b < -7 ? -7 : (b > 7 ? 7 : b);
  float e = fmaf(-s, static_cast<float>(b), w);
  int r = 0;
  if (s16 != 0.0f) {
    float u = rintf(e / s16);
    u = u < -8.0f ? -8.0f : (u > 7.0f ? 7.0f : u);
    r = static_cast<int>(u);
  }
  qb = b;
  qr = r;
}

// One wave per group. Group gi covers src[gi*group, (gi+1)*group) in both
// layouts. VT selects the dim-major plane order that the V cache uses
// inside a block: plane element e is (dim e/blk, token e%blk), which is
// the source element (e%blk)*d + e/blk of the token-major block.
template <bool VT>
__global__ void __launch_bounds__(256) pack_groups_kernel(const float* __restrict__ src,
                                                          int64_t num_groups, int64_t group,
                                                          int64_t d, int64_t blk,
                                                          uint8_t* __restrict__ base,
                                                          uint8_t* __restrict__ refine,
                                                          float* __restrict__ scales) {
  const int64_t gi = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (gi >= num_groups) return;  // uniform per wave; no block-level sync below
  const float* g = src + gi * group;

  float m = 0.0f;
  for (int64_t e = lane; e < group; e += 64) m = fmaxf(m, fabsf(g[e]));
  m = wave_max(m);
  const float s = m / 7.0f;
  const float s16 = s * 0.0625f;
  if (lane == 0) scales[gi] = s;

  uint8_t* pb = base + gi * (group / 2);
  uint8_t* pr = refine + gi * (group / 2);
  for (int64_t p = lane; p < group / 2; p += 64) {
    float w0, w1;
    if (VT) {
      const int64_t e = 2 * p, t = e % blk, j = e / blk;
      w0 = g[t * d + j];
      w1 = g[(t + 1) * d + j];
    } else {
      w0 = g[2 * p];
      w1 = g[2 * p + 1];
    }
    int b0, r0, b1, r1;
    nest_codes(w0, s, s16, b0, r0);
    nest_codes(w1, s, s16, b1, r1);
    pb[p] = static_cast<uint8_t>((b0 & 15) | ((b1 & 15) << 4));
    pr[p] = static_cast<uint8_t>((r0 & 15) | ((r1 & 15) << 4));
  }
}

// Block-wide maximum for blocks of 1024 threads (16 waves).
__device__ __forceinline__ float block_max_1024(float m, float* red) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) r = fmaxf(r, red[w]);
  return r;
}

// One block of 1024 threads per activation row. When K % 4 == 0 and the
// row fits in PER float4 per thread, the row is read once into registers.
template <int PER>
__global__ void __launch_bounds__(1024) act_quant_kernel(const float* __restrict__ x, int64_t K,
                                                         int8_t* __restrict__ qa,
                                                         float* __restrict__ sa) {
  __shared__ float red[16];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * K;
  int8_t* q = qa + row * K;
  if (PER > 0) {
    float4 v[PER > 0 ? PER : 1];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t e = (static_cast<int64_t>(i) * 1024 + threadIdx.x) * 4;
      v[i] = e < K ? *reinterpret_cast<const float4*>(xr + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    m = block_max_1024(m, red);
    const float s = m / 127.0f, r = 1.0f / s;
    if (threadIdx.x == 0) sa[row] = s;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t e = (static_cast<int64_t>(i) * 1024 + threadIdx.x) * 4;
      if (e < K) {
        char4 c;
        c.x = static_cast<signed char>(quant_act(v[i].x, s, r));
        c.y = static_cast<signed char>(quant_act(v[i].y, s, r));
        c.z = static_cast<signed char>(quant_act(v[i].z, s, r));
        c.w = static_cast<signed char>(quant_act(v[i].w, s, r));
        *reinterpret_cast<char4*>(q + e) = c;
      }
    }
  } else {
    float m = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += 1024) m = fmaxf(m, fabsf(xr[k]));
    m = block_max_1024(m, red);
    const float s = m / 127.0f, r = 1.0f / s;
    if (threadIdx.x == 0) sa[row] = s;
    for (int64_t k = threadIdx.x; k < K; k += 1024) q[k] = static_cast<int8_t>(quant_act(xr[k], s, r));
  }
}

// Row-major planes and scales -> the tile layout the GEMV/GEMM kernels read
// (nestspec.h, nest_tile). One thread writes one 16-byte piece of a plane:
// piece o is (tile t, group g, k-quarter q, row r) with r = o % 16,
// q = (o / 16) % 4, g = (o / 64) % G, t = o / (64 G), copied from row
// 16t + r, bytes 64g + 16q .. +15 (zero past the last row). Scales: float f
// is (tile t, quad u, row r, i) with i = f % 4, r = (f / 4) % 16,
// u = (f / 64) % Gq, t = f / (64 Gq): scale (16t + r, 4u + i), zero when the
// row or group is padding.
__global__ void __launch_bounds__(256) tile_planes_kernel(const uint4* __restrict__ src, int64_t rows,
                                                          int64_t G, int64_t pieces, uint4* __restrict__ dst) {
  const int64_t o = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (o >= pieces) return;
  const int64_t r = o & 15, q = (o >> 4) & 3, tg = o >> 6, g = tg % G, t = tg / G;
  const int64_t n = 16 * t + r;
  dst[o] = n < rows ? src[n * (G * 4) + g * 4 + q] : make_uint4(0, 0, 0, 0);
}

__global__ void __launch_bounds__(256) tile_scales_kernel(const float* __restrict__ src, int64_t rows, int64_t G,
                                                          int64_t count, float* __restrict__ dst) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (f >= count) return;
  const int64_t Gq = (G + 3) / 4;
  const int64_t i = f & 3, r = (f >> 2) & 15, uq = f >> 6, u = uq % Gq, t = uq / Gq;
  const int64_t n = 16 * t + r, g = 4 * u + i;
  dst[f] = (n < rows && g < G) ? src[n * G + g] : 0.0f;
}

int launch_pack(bool vt, const float* src, int64_t num_groups, int64_t group, int64_t d,
                int64_t blk, uint8_t* base, uint8_t* refine, float* scales, hipStream_t st,
                const char* what) {
  const int64_t blocks = (num_groups + 3) / 4;
  if (blocks > 0x7fffffffLL) return nest::fail(NEST_EUNSUPPORTED, "%s: too many groups", what);
  if (vt)
    pack_groups_kernel<true><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(
        src, num_groups, group, d, blk, base, refine, scales);
  else
    pack_groups_kernel<false><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(
        src, num_groups, group, d, blk, base, refine, scales);
  return nest::check_launch(what);
}

}  // namespace

extern "C" int nest_pack(const float* w, int64_t rows, int64_t cols, int64_t group, uint8_t* base,
                         uint8_t* refine, float* scales, void* stream) {
  if (!w || !base || !refine || !scales) return nest::fail(NEST_EINVAL, "nest_pack: null pointer");
  if (rows < 1 || cols < 2)
    return nest::fail(NEST_EINVAL, "nest_pack: rows=%lld cols=%lld", (long long)rows, (long long)cols);
  if (group < 2 || group % 2 || cols % group)
    return nest::fail(NEST_ESHAPE, "nest_pack: group=%lld must be even and divide cols=%lld",
                      (long long)group, (long long)cols);
  return launch_pack(false, w, rows * (cols / group), group, 1, 1, base, refine, scales,
                     nest::as_stream(stream), "nest_pack");
}

extern "C" int kv_nest_pack(const float* k, const float* v, int64_t n_kv_heads, int64_t capacity,
                            int64_t head_dim, int64_t block, uint8_t* k_base, uint8_t* k_refine,
                            float* k_scale, uint8_t* v_base, uint8_t* v_refine, float* v_scale,
                            void* stream) {
  if (!k || !v || !k_base || !k_refine || !k_scale || !v_base || !v_refine || !v_scale)
    return nest::fail(NEST_EINVAL, "kv_nest_pack: null pointer");
  if (n_kv_heads < 1 || capacity < 1 || head_dim < 2 || block < 2)
    return nest::fail(NEST_EINVAL, "kv_nest_pack: bad sizes");
  if (head_dim % 2 || block % 2 || capacity % block)
    return nest::fail(NEST_ESHAPE, "kv_nest_pack: need even d and block, capacity %% block == 0");
  const int64_t groups = n_kv_heads * (capacity / block), gsz = block * head_dim;
  hipStream_t st = nest::as_stream(stream);
  int rc = launch_pack(false, k, groups, gsz, head_dim, block, k_base, k_refine, k_scale, st,
                       "kv_nest_pack(K)");
  if (rc) return rc;
  return launch_pack(true, v, groups, gsz, head_dim, block, v_base, v_refine, v_scale, st,
                     "kv_nest_pack(V)");
}

extern "C" int nest_act_quant(const float* x, int64_t M, int64_t K, int8_t* qa, float* sa,
                              void* stream) {
  if (!x || !qa || !sa) return nest::fail(NEST_EINVAL, "nest_act_quant: null pointer");
  if (M < 1 || K < 1 || M > 0x7fffffffLL)
    return nest::fail(NEST_EINVAL, "nest_act_quant: M=%lld K=%lld", (long long)M, (long long)K);
  const dim3 grid(static_cast<unsigned>(M)), block(1024);
  hipStream_t st = nest::as_stream(stream);
  const bool vec = K % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(qa) & 3) == 0;
  const int64_t per = (K / 4 + 1023) / 1024;
  if (vec && per <= 1)
    act_quant_kernel<1><<<grid, block, 0, st>>>(x, K, qa, sa);
  else if (vec && per <= 2)
    act_quant_kernel<2><<<grid, block, 0, st>>>(x, K, qa, sa);
  else if (vec && per <= 5)
    act_quant_kernel<5><<<grid, block, 0, st>>>(x, K, qa, sa);
  else if (vec && per <= 8)
    act_quant_kernel<8><<<grid, block, 0, st>>>(x, K, qa, sa);
  else
    act_quant_kernel<0><<<grid, block, 0, st>>>(x, K, qa, sa);
  return nest::check_launch("nest_act_quant");
}

extern "C" size_t nest_tile_plane_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 128 || cols % 128 || rows > (1LL << 34) || cols > (1LL << 30)) return 0;
  return static_cast<size_t>((rows + 15) / 16) * 16 * static_cast<size_t>(cols / 2);
}

extern "C" size_t nest_tile_scale_count(int64_t rows, int64_t cols, int64_t group) {
  if (group != 128 || nest_tile_plane_bytes(rows, cols) == 0) return 0;
  return static_cast<size_t>((rows + 15) / 16) * 64 * static_cast<size_t>((cols / 128 + 3) / 4);
}

extern "C" int nest_tile(const uint8_t* base, const uint8_t* refine, const float* scales, int64_t rows,
                         int64_t cols, int64_t group, uint8_t* base_t, uint8_t* refine_t, float* scales_t,
                         void* stream) {
  const char* what = "nest_tile";
  if (!base || !scales || !base_t || !scales_t) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (!refine != !refine_t) return nest::fail(NEST_EINVAL, "%s: refine and refine_t go together", what);
  if (group != 128) return nest::fail(NEST_EUNSUPPORTED, "%s: group=%lld (the tile layout uses 128)", what,
                                      (long long)group);
  if (rows < 1 || cols < 128 || cols % 128)
    return nest::fail(NEST_ESHAPE, "%s: rows=%lld cols=%lld (cols must be a multiple of 128)", what,
                      (long long)rows, (long long)cols);
  if (nest_tile_plane_bytes(rows, cols) == 0) return nest::fail(NEST_EUNSUPPORTED, "%s: shape too large", what);
  if (!nest::aligned16(base) || !nest::aligned16(base_t) || (refine && (!nest::aligned16(refine) ||
                                                                        !nest::aligned16(refine_t))))
    return nest::fail(NEST_EALIGN, "%s: planes must be 16-byte aligned", what);
  const int64_t G = cols / 128;
  const int64_t pieces = static_cast<int64_t>(nest_tile_plane_bytes(rows, cols) / 16);
  const int64_t count = static_cast<int64_t>(nest_tile_scale_count(rows, cols, group));
  hipStream_t st = nest::as_stream(stream);
  const dim3 b(256);
  tile_planes_kernel<<<dim3(static_cast<unsigned>((pieces + 255) / 256)), b, 0, st>>>(
      reinterpret_cast<const uint4*>(base), rows, G, pieces, reinterpret_cast<uint4*>(base_t));
  if (refine)
    tile_planes_kernel<<<dim3(static_cast<unsigned>((pieces + 255) / 256)), b, 0, st>>>(
        reinterpret_cast<const uint4*>(refine), rows, G, pieces, reinterpret_cast<uint4*>(refine_t));
  tile_scales_kernel<<<dim3(static_cast<unsigned>((count + 255) / 256)), b, 0, st>>>(scales, rows, G, count,
                                                                                       scales_t);
  return nest::check_launch(what);
}

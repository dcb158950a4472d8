// Nested quantization (BitNest, Figure 2: a base, then the remaining error
// as a refinement; Figure 3: two independent 4-bit planes), the nested KV
// cache builder (Figure 4), and per-token int8 activations.
//
// Each quantization group is one wave. Lanes read the group coalesced for
// the max-abs pass, then each lane codes adjacent element pairs, which are
// one byte in each plane. Every division is IEEE fp32 (correctly rounded,
// HIP's default), rintf rounds ties to even, and the residual is one fmaf,
// so the codes are those of the rule in nestspec.h bit for bit.
#include "quant.h"

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
    // clamped, branch-free loads: all PER of them are in flight together
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t e = (static_cast<int64_t>(i) * 1024 + threadIdx.x) * 4;
      v[i] = *reinterpret_cast<const float4*>(xr + (e < K ? e : K - 4));
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t e = (static_cast<int64_t>(i) * 1024 + threadIdx.x) * 4;
      if (e >= K) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
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

// KV append. Block b of kv head h, K or V, is coded by kAppendSplit
// workgroups, each over its own share of the element pairs. Every one of
// them takes the block's max |v| itself (tokens before pos from the shadow
// slot b % 2, later ones straight from the new values, tokens past the valid
// end as 0), so the workgroups never wait on one another; part 0 also
// writes the block's new tokens into the shadow and the scale. Codes follow
// nest_codes: K token-major (element t*d + j), V dim-major (element
// j*blk + t).
constexpr int kAppendSplit = 16;

struct AppendArgs {
  uint8_t *kb, *kr, *vb, *vr;
  float *ks, *vs;
  float *shk, *shv;              // [Hkv][2][blk][d]
  const float *knew, *vnew;      // [Hkv][n][d]
  int64_t cap, d, blk, pos, n;   // pos: the first position, or an offset added to *pos_dev
  const int32_t* pos_dev;        // device word holding the rest of the position, or null
};

__global__ void __launch_bounds__(256) kv_append_kernel(AppendArgs a) {
  __shared__ float red[4];
  // the first position: host value, plus the device word when given; an
  // append that would not fit in the cache writes nothing
  if (a.pos_dev) {
    a.pos += *a.pos_dev;
    if (a.pos < 0 || a.pos + a.n > a.cap) return;
  }
  const int64_t b = a.pos / a.blk + blockIdx.x, h = blockIdx.y;
  if (b > (a.pos + a.n - 1) / a.blk) return;  // a block the append does not touch
  const bool is_v = (blockIdx.z & 1) == 1;
  const int part = static_cast<int>(blockIdx.z >> 1);
  const int64_t t0 = b * a.blk, nb = a.cap / a.blk;
  float* sh = (is_v ? a.shv : a.shk) + (h * 2 + (b & 1)) * a.blk * a.d;
  const float* nw = (is_v ? a.vnew : a.knew) + h * a.n * a.d;  // token pos + i at nw[i*d]
  const int64_t hi = a.pos + a.n < t0 + a.blk ? a.pos + a.n : t0 + a.blk;
  const int64_t valid = hi - t0;
  const int64_t old_end = a.pos > t0 ? a.pos - t0 : 0;  // tokens [0, old_end) come from the shadow
  auto value = [&](int64_t t, int64_t j) -> float {
    if (t >= valid) return 0.0f;
    return t < old_end ? sh[t * a.d + j] : nw[(t0 + t - a.pos) * a.d + j];
  };
  // 1. the block's max |v| over its valid tokens: the shadow's tokens
  // [0, old_end) and the new ones [old_end, valid) are two contiguous runs
  // (read as float4 when aligned, so that a block takes one round trip)
  float m = 0.0f;
  auto absmax_run = [&](const float* src, int64_t n) {
    if ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && (n & 3) == 0) {
#pragma unroll 16
      for (int64_t i = 4 * static_cast<int64_t>(threadIdx.x); i < n; i += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(src + i);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      }
    } else {
      for (int64_t i = threadIdx.x; i < n; i += 256) m = fmaxf(m, fabsf(src[i]));
    }
  };
  absmax_run(sh, old_end * a.d);
  absmax_run(nw + (t0 + old_end - a.pos) * a.d, (valid - old_end) * a.d);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m / 7.0f, s16 = s * 0.0625f, rs = 1.0f / s, rs16 = 1.0f / s16;
  if (part == 0) {
    if (threadIdx.x == 0) (is_v ? a.vs : a.ks)[h * nb + b] = s;
    for (int64_t i = threadIdx.x; i < (valid - old_end) * a.d; i += 256)
      sh[old_end * a.d + i] = nw[(t0 + old_end - a.pos) * a.d + i];
  }
  // 2. this part's element pairs (element e, e+1 share a byte)
  uint8_t* pb = (is_v ? a.vb : a.kb) + (h * a.cap + t0) * a.d / 2;
  uint8_t* pr = (is_v ? a.vr : a.kr) + (h * a.cap + t0) * a.d / 2;
  const int64_t pairs = a.blk * a.d / 2;
  const int64_t p0 = pairs * part / kAppendSplit, p1 = pairs * (part + 1) / kAppendSplit;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
    const int64_t e = 2 * p;
    float w0, w1;
    if (is_v) {  // tokens t, t+1 of dim j
      const int64_t j = e / a.blk, t = e % a.blk;
      w0 = value(t, j);
      w1 = value(t + 1, j);
    } else {     // dims j, j+1 of token t
      const int64_t t = e / a.d, j = e % a.d;
      w0 = value(t, j);
      w1 = value(t, j + 1);
    }
    int b0, r0, b1, r1;
    nest::nest_codes_fast(w0, s, s16, rs, rs16, b0, r0);
    nest::nest_codes_fast(w1, s, s16, rs, rs16, b1, r1);
    pb[p] = static_cast<uint8_t>((b0 & 15) | ((b1 & 15) << 4));
    pr[p] = static_cast<uint8_t>((r0 & 15) | ((r1 & 15) << 4));
  }
}

// Copy tokens [blk * floor(ctx/blk), ctx) of every head from full fp32 K/V
// [Hkv][src_len][d] into their shadow slot.
__global__ void __launch_bounds__(256) kv_shadow_fill_kernel(const float* __restrict__ src, int64_t src_len,
                                                             int64_t d, int64_t blk, int64_t ctx,
                                                             float* __restrict__ sh) {
  const int64_t h = blockIdx.y, b = ctx / blk, t0 = b * blk, n = (ctx - t0) * d;
  float* dst = sh + (h * 2 + (b & 1)) * blk * d;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    dst[i] = src[(h * src_len + t0) * d + i];
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

namespace {
int check_kv(const char* what, const nest_kv* kv) {
  if (!kv || !kv->k_base || !kv->k_refine || !kv->v_base || !kv->v_refine || !kv->k_scale || !kv->v_scale)
    return nest::fail(NEST_EINVAL, "%s: null cache pointer", what);
  if (kv->n_kv_heads < 1 || kv->head_dim < 2 || kv->head_dim % 2 || kv->block < 2 || kv->block % 2 ||
      kv->capacity < kv->block || kv->capacity % kv->block)
    return nest::fail(NEST_ESHAPE, "%s: bad cache shape", what);
  if (kv->n_kv_heads > 65535) return nest::fail(NEST_EUNSUPPORTED, "%s: too many kv heads", what);
  return NEST_OK;
}
}  // namespace

extern "C" size_t kv_nest_shadow_floats(int64_t n_kv_heads, int64_t head_dim, int64_t block) {
  if (n_kv_heads < 1 || head_dim < 2 || block < 2) return 0;
  return static_cast<size_t>(n_kv_heads) * 2 * static_cast<size_t>(block) * static_cast<size_t>(head_dim);
}

extern "C" int kv_nest_shadow_fill(const nest_kv* kv, const float* k, const float* v, int64_t src_len,
                                   int64_t ctx_len, float* shadow_k, float* shadow_v, void* stream) {
  const char* what = "kv_nest_shadow_fill";
  int rc = check_kv(what, kv);
  if (rc) return rc;
  if (!k || !v || !shadow_k || !shadow_v) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (ctx_len < 0 || ctx_len > src_len || ctx_len > kv->capacity)
    return nest::fail(NEST_EINVAL, "%s: need 0 <= ctx_len <= src_len, capacity", what);
  if (ctx_len % kv->block == 0) return nest::ok();  // no open block to carry
  const dim3 grid(static_cast<unsigned>((kv->block * kv->head_dim + 255) / 256),
                  static_cast<unsigned>(kv->n_kv_heads));
  hipStream_t st = nest::as_stream(stream);
  kv_shadow_fill_kernel<<<grid, 256, 0, st>>>(k, src_len, kv->head_dim, kv->block, ctx_len, shadow_k);
  kv_shadow_fill_kernel<<<grid, 256, 0, st>>>(v, src_len, kv->head_dim, kv->block, ctx_len, shadow_v);
  return nest::check_launch(what);
}

extern "C" int kv_nest_append(const nest_kv* kv, float* shadow_k, float* shadow_v, const float* k_new,
                              const float* v_new, const int32_t* pos_dev, int64_t pos, int64_t n,
                              void* stream) {
  const char* what = "kv_nest_append";
  int rc = check_kv(what, kv);
  if (rc) return rc;
  if (!shadow_k || !shadow_v || !k_new || !v_new) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (n < 1 || n > kv->block || (!pos_dev && (pos < 0 || pos + n > kv->capacity)) ||
      (pos_dev && (pos < -kv->capacity || pos > kv->capacity)))
    return nest::fail(NEST_EINVAL, "%s: need pos >= 0, 1 <= n <= block, pos + n <= capacity (pos=%lld n=%lld)",
                      what, (long long)pos, (long long)n);
  AppendArgs a{};
  a.kb = const_cast<uint8_t*>(kv->k_base); a.kr = const_cast<uint8_t*>(kv->k_refine);
  a.vb = const_cast<uint8_t*>(kv->v_base); a.vr = const_cast<uint8_t*>(kv->v_refine);
  a.ks = const_cast<float*>(kv->k_scale); a.vs = const_cast<float*>(kv->v_scale);
  a.shk = shadow_k; a.shv = shadow_v; a.knew = k_new; a.vnew = v_new;
  a.cap = kv->capacity; a.d = kv->head_dim; a.blk = kv->block; a.pos = pos; a.n = n; a.pos_dev = pos_dev;
  // n <= block tokens touch at most two blocks; with the position on the
  // device both are launched and the kernel skips one the append misses
  const int64_t touched = pos_dev ? 2 : (pos + n - 1) / kv->block - pos / kv->block + 1;
  kv_append_kernel<<<dim3(static_cast<unsigned>(touched), static_cast<unsigned>(kv->n_kv_heads),
                          2 * kAppendSplit),
                     256, 0, nest::as_stream(stream)>>>(a);
  return nest::check_launch(what);
}

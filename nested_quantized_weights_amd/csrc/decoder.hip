// Glue of a small synthetic decoder built from the nested linears and the
// nested KV cache: token embedding, residual add + RMSNorm, rotary position
// embedding with the q/k/v split, and SwiGLU. None of this is on the pages;
// it is the plain pre-norm decoder (Llama / Qwen style) that the round is
// run through end to end ("How Speculative Decoding Speeds Up Inference",
// section "The same output as the large model alone": with greedy decoding
// every kept token is the target's own top choice).
//
// Each output row depends on its own input row only and is computed in the
// same order whatever the number of rows, so a position comes out
// bit-identical whether it is processed alone (one token per pass) or
// inside a batch of k+1 (a verify pass).
#include "common.h"

namespace {

constexpr int kNormThreads = 256;

// out[m] = table[tokens[m]] (a zero row for an id outside [0, V)).
__global__ void __launch_bounds__(256) embed_kernel(const float* table, int V, int H, const int32_t* tokens,
                                                    float* out) {
  const int m = blockIdx.y;
  const int t = tokens[m];
  const bool ok = t >= 0 && t < V;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < H; i += gridDim.x * 256)
    out[static_cast<size_t>(m) * H + i] = ok ? table[static_cast<size_t>(t) * H + i] : 0.0f;
}

// x[m] += y[m] (when y is set), then out[m] = x[m] / sqrt(mean(x[m]^2) + eps) * gamma.
// One block per row; each thread sums its strided elements in order, then
// the wave butterflies and the waves in order: a fixed order per row.
__global__ void __launch_bounds__(kNormThreads) add_rmsnorm_kernel(float* x, const float* y, const float* gamma,
                                                                   int H, float eps, float* out) {
  __shared__ float part[kNormThreads / 64];
  const int m = blockIdx.x;
  float* xr = x + static_cast<size_t>(m) * H;
  const float* yr = y ? y + static_cast<size_t>(m) * H : nullptr;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < H; i += kNormThreads) {
    float v = xr[i];
    if (yr) {
      v += yr[i];
      xr[i] = v;
    }
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += part[w];
  const float r = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
  float* o = out + static_cast<size_t>(m) * H;
  for (int i = threadIdx.x; i < H; i += kNormThreads) o[i] = xr[i] * r * gamma[i];
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  // round to nearest, ties to even (finite inputs)
  const uint32_t b = __float_as_uint(f);
  return static_cast<uint16_t>((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

struct RopeArgs {
  const float* qkv;  // [M][(Hq + 2 Hkv) d]
  int M, Hq, Hkv, d;
  int64_t pos0;            // position of row 0, or an offset added to *pos_dev
  const int32_t* pos_dev;  // device word holding the rest of the position, or null
  float log2_theta;
  int token_major;  // K/V out as [M][Hkv][d] (1) or [Hkv][M][d] (0)
  uint16_t* q;      // bf16 [M][Hq][d]
  float* k;
  float* v;
};

// One block per (row, head), d/2 threads: the rotate-half rotary embedding
// on q and k at position pos0 + m with frequency theta^(-2i/d) for pair
// (i, i + d/2); q rounded to bf16, v copied.
__global__ void __launch_bounds__(64) rope_split_kernel(RopeArgs a) {
  const int m = blockIdx.x, h = blockIdx.y, i = threadIdx.x, half = a.d / 2;
  const int64_t pos = a.pos0 + (a.pos_dev ? *a.pos_dev : 0) + m;
  const float* src = a.qkv + static_cast<size_t>(m) * (a.Hq + 2 * a.Hkv) * a.d + static_cast<size_t>(h) * a.d;
  for (int j = i; j < half; j += 64) {
    const float x1 = src[j], x2 = src[j + half];
    if (h < a.Hq + a.Hkv) {
      const float inv_freq = exp2f(-(2.0f * static_cast<float>(j) / static_cast<float>(a.d)) * a.log2_theta);
      const float ang = static_cast<float>(pos) * inv_freq;
      float s, c;
      sincosf(ang, &s, &c);
      const float o1 = x1 * c - x2 * s, o2 = x2 * c + x1 * s;
      if (h < a.Hq) {
        uint16_t* q = a.q + (static_cast<size_t>(m) * a.Hq + h) * a.d;
        q[j] = to_bf16(o1);
        q[j + half] = to_bf16(o2);
      } else {
        const int kh = h - a.Hq;
        float* k = a.k + (a.token_major ? (static_cast<size_t>(m) * a.Hkv + kh) * a.d
                                        : (static_cast<size_t>(kh) * a.M + m) * a.d);
        k[j] = o1;
        k[j + half] = o2;
      }
    } else {
      const int vh = h - a.Hq - a.Hkv;
      float* v = a.v + (a.token_major ? (static_cast<size_t>(m) * a.Hkv + vh) * a.d
                                      : (static_cast<size_t>(vh) * a.M + m) * a.d);
      v[j] = x1;
      v[j + half] = x2;
    }
  }
}

// out[m][i] = silu(gu[m][i]) * gu[m][I + i], silu(g) = g / (1 + exp(-g)).
__global__ void __launch_bounds__(256) swiglu_kernel(const float* gu, int I, float* out) {
  const int m = blockIdx.y;
  const float* r = gu + static_cast<size_t>(m) * 2 * I;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < I; i += gridDim.x * 256) {
    const float g = r[i];
    out[static_cast<size_t>(m) * I + i] = g / (1.0f + expf(-g)) * r[I + i];
  }
}

int check_rows(const char* what, int64_t M, int64_t H) {
  if (M < 1 || H < 1) return nest::fail(NEST_EINVAL, "%s: empty shape", what);
  if (M > 65535 || H > (1 << 24)) return nest::fail(NEST_EUNSUPPORTED, "%s: shape too large", what);
  return NEST_OK;
}

unsigned col_blocks(int64_t n) { return static_cast<unsigned>(n < 256 * 64 ? (n + 255) / 256 : 64); }

}  // namespace

extern "C" int nest_embed(const float* table, int64_t V, int64_t H, const int32_t* tokens, int64_t M, float* out,
                          void* stream) {
  const char* what = "nest_embed";
  if (!table || !tokens || !out) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  int rc = check_rows(what, M, H);
  if (rc) return rc;
  if (V < 1 || V > 0x7fffffffLL) return nest::fail(NEST_EINVAL, "%s: V=%lld", what, (long long)V);
  embed_kernel<<<dim3(col_blocks(H), static_cast<unsigned>(M)), 256, 0, nest::as_stream(stream)>>>(
      table, static_cast<int>(V), static_cast<int>(H), tokens, out);
  return nest::check_launch(what);
}

extern "C" int nest_add_rmsnorm(float* x, const float* y, const float* gamma, int64_t M, int64_t H, float eps,
                                float* out, void* stream) {
  const char* what = "nest_add_rmsnorm";
  if (!x || !gamma || !out) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  int rc = check_rows(what, M, H);
  if (rc) return rc;
  if (!(eps >= 0.0f)) return nest::fail(NEST_EINVAL, "%s: eps must be >= 0", what);
  add_rmsnorm_kernel<<<static_cast<unsigned>(M), kNormThreads, 0, nest::as_stream(stream)>>>(
      x, y, gamma, static_cast<int>(H), eps, out);
  return nest::check_launch(what);
}

extern "C" int nest_rope_split(const float* qkv, int64_t M, const int32_t* pos_dev, int64_t pos0,
                               int64_t n_q_heads, int64_t n_kv_heads,
                               int64_t head_dim, float theta, int token_major, uint16_t* q, float* k, float* v,
                               void* stream) {
  const char* what = "nest_rope_split";
  if (!qkv || !q || !k || !v) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  int rc = check_rows(what, M, head_dim);
  if (rc) return rc;
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads + 2 * n_kv_heads > 65535 || head_dim % 2 ||
      (!pos_dev && pos0 < 0) || pos0 > (1LL << 24) || pos0 < -(1LL << 24))
    return nest::fail(NEST_EINVAL, "%s: heads=%lld/%lld head_dim=%lld pos0=%lld", what, (long long)n_q_heads,
                      (long long)n_kv_heads, (long long)head_dim, (long long)pos0);
  if (!(theta > 1.0f)) return nest::fail(NEST_EINVAL, "%s: theta must be > 1", what);
  RopeArgs a{qkv, static_cast<int>(M), static_cast<int>(n_q_heads), static_cast<int>(n_kv_heads),
             static_cast<int>(head_dim), pos0, pos_dev, log2f(theta), token_major ? 1 : 0, q, k, v};
  rope_split_kernel<<<dim3(static_cast<unsigned>(M), static_cast<unsigned>(n_q_heads + 2 * n_kv_heads)), 64, 0,
                      nest::as_stream(stream)>>>(a);
  return nest::check_launch(what);
}

extern "C" int nest_swiglu(const float* gate_up, int64_t M, int64_t I, float* out, void* stream) {
  const char* what = "nest_swiglu";
  if (!gate_up || !out) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  int rc = check_rows(what, M, I);
  if (rc) return rc;
  swiglu_kernel<<<dim3(col_blocks(I), static_cast<unsigned>(M)), 256, 0, nest::as_stream(stream)>>>(
      gate_up, static_cast<int>(I), out);
  return nest::check_launch(what);
}

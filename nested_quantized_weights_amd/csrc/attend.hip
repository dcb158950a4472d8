// Decode attention over the nested KV cache (BitNest, Figure 4). The draft
// attends the base view and reads only the base planes. Verification
// attends the full view, 16*q_b + q_r at s/16, reading both planes. Entries
// past ctx_len are never read, and the caller's length update discards a
// rejected suffix.
//
// gfx950 design (flash-decoding). Work unit = (kv head, 128-token block).
// A block of 4 waves takes 4*bpw consecutive blocks of one head, and each
// wave keeps an online softmax over its blocks. The waves merge in LDS in a
// fixed order. A second kernel merges the blocks' partial (max, sum, O)
// with log-sum-exp weights, also in a fixed order. Both products use
// v_mfma_f32_16x16x32_f16:
//   S^T = K Q^T : A = 16 tokens x 32 dims of K codes, B = Q^T (16 query rows)
//   O^T += V^T P^T : A = 16 dims x 32 tokens of V codes, B = P^T
// Cache codes become exact f16 integers without converts. v_perm_b32 puts
// a nibble-or-byte u under the exponent byte 0x64 (the f16 1024 + u). One
// v_pk_add_f16 then removes the offset exactly (1032 for a 4-bit base code,
// 1160 for the 8-bit code 16*q_b + q_r biased by 136). Inside a block, token
// tile 2j+e row 4q+i holds token 32q + 8j + 4e + i. Then the S^T tile that
// a lane holds is exactly the P^T operand it needs, and each lane's V codes
// for a dim tile are 16 contiguous bytes of the dim-major V block.
// Query values enter as f16 (bf16 -> f16 is exact in the normal range).
// Softmax runs in the log2 domain with exp2f.
#include "common.h"

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kBlk = 128;
constexpr float kLog2e = 1.4426950408889634f;

struct AttArgs {
  const uint16_t* q;
  int nq, Hq, grp, R;  // R = nq * grp query rows per kv head
  int ctx, nbv;        // visible length and visible blocks
  const uint8_t *kb, *kr, *vb, *vr;
  const float *ks, *vs;
  int cap, nb;         // capacity and blocks per head in the planes
  int bpw, nchunk;     // blocks per wave, chunks (workgroups) per head
  float* part_ml;      // [Hkv][nchunk][R][2]  (max in log2 domain, sum)
  float* part_o;       // [Hkv][nchunk][R][128]
  float* out;          // [nq][Hq][128]
};

__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t x, uint32_t y) { return (x & m) | (y & ~m); }

__device__ __forceinline__ uint32_t sub_h2(uint32_t v, uint32_t off) {
  h2 a = __builtin_bit_cast(h2, v), b = __builtin_bit_cast(h2, off);
  return __builtin_bit_cast(uint32_t, a - b);
}

// Four bytes u (each < 256) -> two VGPRs of f16 pairs 1024+u in the order
// (byte0, byte1) and (byte2, byte3).
__device__ __forceinline__ void bytes_to_h(uint32_t bytes, uint32_t off, uint32_t& p01, uint32_t& p23) {
  const uint32_t c64 = 0x64646464u;
  p01 = sub_h2(__builtin_amdgcn_perm(c64, bytes, 0x04010400u), off);
  p23 = sub_h2(__builtin_amdgcn_perm(c64, bytes, 0x04030402u), off);
}

// One 32-bit word of codes (8 elements e0..e7, e_{2b} in the low nibble of
// byte b) -> 8 f16 code values in the order [e0 e2 e4 e6 e1 e3 e5 e7].
template <int VIEW>
__device__ __forceinline__ v8h codes_to_h8(uint32_t wb, uint32_t wr) {
  uint32_t ev, od, off;
  const uint32_t xb = wb ^ 0x88888888u;
  if (VIEW == 0) {
    ev = xb & 0x0F0F0F0Fu;          // q_b + 8 of even elements
    od = (xb >> 4) & 0x0F0F0F0Fu;   // of odd elements
    off = 0x64086408u;              // f16 1032 = 1024 + 8, twice
  } else {
    const uint32_t xr = wr ^ 0x88888888u;
    ev = bfi(0xF0F0F0F0u, xb << 4, xr);  // 16*(q_b+8) + (q_r+8) = c + 136
    od = bfi(0xF0F0F0F0u, xb, xr >> 4);
    off = 0x64886488u;                   // f16 1160 = 1024 + 136, twice
  }
  uint32_t r[4];
  bytes_to_h(ev, off, r[0], r[1]);
  bytes_to_h(od, off, r[2], r[3]);
  v4i t = {(int)r[0], (int)r[1], (int)r[2], (int)r[3]};
  return __builtin_bit_cast(v8h, t);
}

__device__ __forceinline__ v4f mfma_h(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ _Float16 bf16_to_h(uint16_t b) {
  return static_cast<_Float16>(__uint_as_float(static_cast<uint32_t>(b) << 16));
}

template <int RT, int VIEW>
__global__ void __launch_bounds__(256) attend_kernel(AttArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int h = blockIdx.y, chunk = blockIdx.x;

  // Query operands: row rt*16 + c16, k-step s holds dims 32*q4 + 8*s + [0 2 4 6 1 3 5 7].
  v8h qop[RT][4];
  int pos[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = rt * 16 + c16;
    pos[rt] = -1;
    if (rho < a.R) {
      const int i = rho / a.grp, g = rho % a.grp;
      pos[rt] = a.ctx - a.nq + i;
      const uint16_t* qr = a.q + (static_cast<size_t>(i) * a.Hq + h * a.grp + g) * kD + 32 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint16_t* p = qr + 8 * s;
        v8h v;
        v[0] = bf16_to_h(p[0]); v[1] = bf16_to_h(p[2]); v[2] = bf16_to_h(p[4]); v[3] = bf16_to_h(p[6]);
        v[4] = bf16_to_h(p[1]); v[5] = bf16_to_h(p[3]); v[6] = bf16_to_h(p[5]); v[7] = bf16_to_h(p[7]);
        qop[rt][s] = v;
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qop[rt][s] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  float m[RT], l[RT];
  v4f O[RT][8];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[rt][dt] = v4f{0, 0, 0, 0};
  }

  const float sm_scale = (VIEW ? 0.0625f : 1.0f) * 0.08838834764831845f * kLog2e;  // 1/sqrt(128)
  const int first = chunk * 4 * a.bpw;
  for (int t = 0; t < a.bpw; ++t) {
    const int blk = first + wave + 4 * t;
    if (blk >= a.nbv) break;  // uniform per wave
    const int t0 = blk * kBlk;
    const size_t hb = static_cast<size_t>(h) * a.nb + blk;

    // K: token tile tt = 2j+e, row c16 = 4*qq+i -> token 32*qq + 8*j + 4*e + i.
    uint4 kw[8], kwr[8], vw[8], vwr[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int tok = 32 * (c16 >> 2) + 8 * (tt >> 1) + 4 * (tt & 1) + (c16 & 3);
      const size_t off = (static_cast<size_t>(h) * a.cap + t0 + tok) * (kD / 2) + 16 * q4;
      kw[tt] = *reinterpret_cast<const uint4*>(a.kb + off);
      if (VIEW) kwr[tt] = *reinterpret_cast<const uint4*>(a.kr + off);
    }
    // V: dim tile dt, dim row dt*16 + c16, tokens 32*q4 .. 32*q4+31.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const size_t off = (hb * kD + dt * 16 + c16) * (kBlk / 2) + 16 * q4;
      vw[dt] = *reinterpret_cast<const uint4*>(a.vb + off);
      if (VIEW) vwr[dt] = *reinterpret_cast<const uint4*>(a.vr + off);
    }
    const float ck = a.ks[hb] * sm_scale;
    const float sv = VIEW ? a.vs[hb] * 0.0625f : a.vs[hb];

    // S^T tiles
    v4f S[RT][8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const uint32_t w0[4] = {kw[tt].x, kw[tt].y, kw[tt].z, kw[tt].w};
      uint32_t w1[4] = {0, 0, 0, 0};
      if (VIEW) { w1[0] = kwr[tt].x; w1[1] = kwr[tt].y; w1[2] = kwr[tt].z; w1[3] = kwr[tt].w; }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) S[rt][tt] = v4f{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v8h av = codes_to_h8<VIEW>(w0[s], w1[s]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) S[rt][tt] = mfma_h(av, qop[rt][s], S[rt][tt]);
      }
    }

    // online softmax (log2 domain) for the row this lane carries
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mb = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + 32 * q4 + 8 * (tt >> 1) + 4 * (tt & 1) + i;
          const float v = tok <= pos[rt] ? S[rt][tt][i] * ck : -INFINITY;
          S[rt][tt][i] = v;
          mb = fmaxf(mb, v);
        }
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      const float mn = fmaxf(m[rt], mb);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2f(m[rt] - mu);
      float ls = 0.0f;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(S[rt][tt][i] - mu);
          S[rt][tt][i] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      l[rt] = l[rt] * alpha + ls;
      m[rt] = mn;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[rt][dt] *= alpha;
    }

    // O^T += V^T P^T ; P pre-scaled by the block's V scale
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v8h pb[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const v4f e0 = S[rt][2 * j], e1 = S[rt][2 * j + 1];
        v8h p;
        p[0] = (_Float16)(e0[0] * sv); p[1] = (_Float16)(e0[2] * sv);
        p[2] = (_Float16)(e1[0] * sv); p[3] = (_Float16)(e1[2] * sv);
        p[4] = (_Float16)(e0[1] * sv); p[5] = (_Float16)(e0[3] * sv);
        p[6] = (_Float16)(e1[1] * sv); p[7] = (_Float16)(e1[3] * sv);
        pb[rt] = p;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint32_t wb = j == 0 ? vw[dt].x : j == 1 ? vw[dt].y : j == 2 ? vw[dt].z : vw[dt].w;
        uint32_t wr = 0;
        if (VIEW) wr = j == 0 ? vwr[dt].x : j == 1 ? vwr[dt].y : j == 2 ? vwr[dt].z : vwr[dt].w;
        const v8h av = codes_to_h8<VIEW>(wb, wr);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) O[rt][dt] = mfma_h(av, pb[rt], O[rt][dt]);
      }
    }
  }

  // ---- merge the 4 waves in LDS, in the fixed order 3, 2, 1, 0 ----
  __shared__ float ml[4][RT * 16][2];
  __shared__ float buf[RT * 16][kD + 4];
  if (q4 == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      ml[wave][rt * 16 + c16][0] = m[rt];
      ml[wave][rt * 16 + c16][1] = l[rt];
    }
  }
  __syncthreads();
  float f[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + c16;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[w][row][0]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    f[rt] = exp2f(m[rt] - Mu);
  }
  for (int w = 3; w >= 0; --w) {
    if (wave == w) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* p = &buf[rt * 16 + c16][dt * 16 + 4 * q4 + i];
            const float v = O[rt][dt][i] * f[rt];
            *p = (w == 3) ? v : *p + v;
          }
    }
    __syncthreads();
  }
  // write this workgroup's partial: rows < R
  const size_t pbase = (static_cast<size_t>(h) * a.nchunk + chunk) * a.R;
  for (int idx = threadIdx.x; idx < a.R * kD; idx += 256) {
    const int row = idx / kD, dim = idx % kD;
    a.part_o[(pbase + row) * kD + dim] = buf[row][dim];
  }
  if (threadIdx.x < a.R) {
    const int row = threadIdx.x;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[w][row][0]);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float L = 0.0f;
    for (int w = 0; w < 4; ++w) L += ml[w][row][1] * exp2f(ml[w][row][0] - Mu);
    a.part_ml[(pbase + row) * 2 + 0] = M;
    a.part_ml[(pbase + row) * 2 + 1] = L;
  }
}

// One block of 256 threads per (row, kv head). The chunk weights
// 2^(m_c - M) go to LDS. Then each half-block sums the chunks of one parity
// for all 128 dims, and the two halves are added (a fixed order).
constexpr int kCombineChunks = 1024;  // chunks handled per LDS pass

__global__ void __launch_bounds__(256) combine_kernel(AttArgs a) {
  __shared__ float wts[kCombineChunks];
  __shared__ float red[8];
  __shared__ float half_acc[kD];
  const int row = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const size_t base = static_cast<size_t>(h) * a.nchunk * a.R + row;  // partial of chunk c: base + c*R
  float M = -INFINITY;
  for (int c = t; c < a.nchunk; c += 256) M = fmaxf(M, a.part_ml[(base + static_cast<size_t>(c) * a.R) * 2]);
  M = wave_max(M);
  if ((t & 63) == 0) red[t >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float Mu = M == -INFINITY ? 0.0f : M;
  __syncthreads();
  float L = 0.0f, acc = 0.0f;
  const int dim = t & (kD - 1), par = t >> 7;
  for (int c0 = 0; c0 < a.nchunk; c0 += kCombineChunks) {
    const int cn = min(kCombineChunks, a.nchunk - c0);
    for (int c = t; c < cn; c += 256) {
      const size_t pr = base + static_cast<size_t>(c0 + c) * a.R;
      const float mc = a.part_ml[pr * 2];
      const float w = mc == -INFINITY ? 0.0f : exp2f(mc - Mu);
      wts[c] = w;
      L += w * a.part_ml[pr * 2 + 1];
    }
    __syncthreads();
    for (int c = par; c < cn; c += 2) {
      const float w = wts[c];
      if (w != 0.0f) acc += a.part_o[(base + static_cast<size_t>(c0 + c) * a.R) * kD + dim] * w;
    }
    __syncthreads();
  }
  // total denominator: block sum of L
  L = wave_sum(L);
  if ((t & 63) == 0) red[4 + (t >> 6)] = L;
  if (par == 1) half_acc[dim] = acc;
  __syncthreads();
  if (par == 0) {
    const float Lt = (red[4] + red[5]) + (red[6] + red[7]);
    const int i = row / a.grp, g = row % a.grp;
    a.out[(static_cast<size_t>(i) * a.Hq + h * a.grp + g) * kD + dim] = (acc + half_acc[dim]) / Lt;
  }
}

struct Plan {
  int nbv, bpw, nchunk, RT;
  size_t ws;
};

Plan make_plan(int64_t nq, int64_t Hq, int64_t Hkv, int64_t ctx) {
  Plan p{};
  const int64_t R = nq * (Hq / Hkv);
  p.nbv = static_cast<int>((ctx + kBlk - 1) / kBlk);
  p.bpw = 1;
  // keep at least ~2 workgroups per CU, then grow the per-wave work
  while (Hkv * ((p.nbv + 8 * p.bpw - 1) / (8 * p.bpw)) >= 512) p.bpw *= 2;
  p.nchunk = (p.nbv + 4 * p.bpw - 1) / (4 * p.bpw);
  p.RT = static_cast<int>((R + 15) / 16);
  p.ws = static_cast<size_t>(Hkv) * p.nchunk * R * (kD + 2) * sizeof(float);
  return p;
}

template <int VIEW>
int launch_att(const AttArgs& a, const Plan& p, int Hkv, hipStream_t st) {
  dim3 grid(p.nchunk, Hkv);
  switch (p.RT) {
    case 1: attend_kernel<1, VIEW><<<grid, 256, 0, st>>>(a); break;
    case 2: attend_kernel<2, VIEW><<<grid, 256, 0, st>>>(a); break;
    case 3: attend_kernel<3, VIEW><<<grid, 256, 0, st>>>(a); break;
    default: attend_kernel<4, VIEW><<<grid, 256, 0, st>>>(a); break;
  }
  int rc = nest::check_launch("kv_nest_attend");
  if (rc) return rc;
  combine_kernel<<<dim3(a.R, Hkv), 256, 0, st>>>(a);
  return nest::check_launch("kv_nest_attend(combine)");
}

}  // namespace

extern "C" size_t kv_nest_attend_workspace_size(int64_t nq, int64_t n_q_heads, int64_t n_kv_heads,
                                                int64_t head_dim, int64_t ctx_len) {
  if (nq < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || head_dim != kD || ctx_len < 1) return 0;
  return make_plan(nq, n_q_heads, n_kv_heads, ctx_len).ws;
}

extern "C" int kv_nest_attend(const uint16_t* q, int64_t nq, int64_t n_q_heads, const nest_kv* kv,
                              int64_t ctx_len, int view, float* out, void* ws, size_t ws_bytes,
                              void* stream) {
  const char* what = "kv_nest_attend";
  if (!q || !kv || !out) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (!kv->k_base || !kv->v_base || !kv->k_scale || !kv->v_scale)
    return nest::fail(NEST_EINVAL, "%s: null cache pointer", what);
  if (view != 0 && view != 1) return nest::fail(NEST_EINVAL, "%s: view=%d", what, view);
  if (view == 1 && (!kv->k_refine || !kv->v_refine))
    return nest::fail(NEST_EINVAL, "%s: the full view needs both refinement planes", what);
  const int64_t Hkv = kv->n_kv_heads;
  if (Hkv < 1 || n_q_heads < 1 || nq < 1 || kv->capacity < 1)
    return nest::fail(NEST_EINVAL, "%s: empty shape", what);
  if (kv->head_dim != kD || kv->block != kBlk)
    return nest::fail(NEST_EUNSUPPORTED, "%s: head_dim and block must be 128", what);
  if (n_q_heads % Hkv) return nest::fail(NEST_ESHAPE, "%s: Hq %% Hkv != 0", what);
  if (kv->capacity % kBlk) return nest::fail(NEST_ESHAPE, "%s: capacity %% block != 0", what);
  if (ctx_len < nq || ctx_len > kv->capacity)
    return nest::fail(NEST_EINVAL, "%s: need nq <= ctx_len <= capacity (ctx_len=%lld)", what,
                      (long long)ctx_len);
  const int64_t R = nq * (n_q_heads / Hkv);
  if (R > 64) return nest::fail(NEST_EUNSUPPORTED, "%s: nq*(Hq/Hkv)=%lld > 64", what, (long long)R);
  if (kv->capacity > (1LL << 30) || Hkv > 65535)
    return nest::fail(NEST_EUNSUPPORTED, "%s: cache too large", what);
  if (!nest::aligned16(kv->k_base) || !nest::aligned16(kv->v_base) ||
      (view == 1 && (!nest::aligned16(kv->k_refine) || !nest::aligned16(kv->v_refine))))
    return nest::fail(NEST_EALIGN, "%s: planes must be 16-byte aligned", what);
  const Plan p = make_plan(nq, n_q_heads, Hkv, ctx_len);
  if (!ws || ws_bytes < p.ws) return nest::fail(NEST_EWORKSPACE, "%s: workspace needs %zu bytes", what, p.ws);
  AttArgs a{};
  a.q = q; a.nq = (int)nq; a.Hq = (int)n_q_heads; a.grp = (int)(n_q_heads / Hkv); a.R = (int)R;
  a.ctx = (int)ctx_len; a.nbv = p.nbv;
  a.kb = kv->k_base; a.kr = kv->k_refine; a.vb = kv->v_base; a.vr = kv->v_refine;
  a.ks = kv->k_scale; a.vs = kv->v_scale;
  a.cap = (int)kv->capacity; a.nb = (int)(kv->capacity / kBlk);
  a.bpw = p.bpw; a.nchunk = p.nchunk;
  a.part_ml = static_cast<float*>(ws);
  a.part_o = a.part_ml + static_cast<size_t>(Hkv) * p.nchunk * R * 2;
  a.out = out;
  hipStream_t st = nest::as_stream(stream);
  return view == 0 ? launch_att<0>(a, p, (int)Hkv, st) : launch_att<1>(a, p, (int)Hkv, st);
}

// Decode attention over the nested KV cache (BitNest, Figure 4). The draft
// attends the base view and reads only the base planes. Verification
// attends the full view, 16*q_b + q_r at s/16, reading both planes. Entries
// past ctx_len are never read, and the caller's length update discards a
// rejected suffix.
//
// gfx950 design (flash-decoding). Up to 16 query rows per kv head (the
// draft's one query over a GQA group): attend_wave_kernel, where each wave
// owns whole 128-token blocks and converts codes in registers. More rows
// (verification's k+1 queries): a workgroup of 4 waves walks a chunk of
// 128-token blocks of one kv head and shares converted operands. Per block:
//   phase A  all 256 threads read the block's codes once (K token-major, V
//            dim-major) and convert them to f16 MFMA operands in LDS
//            (32 KB K + 32 KB V). An 8-bit code u (16*q_b + 8 biased by 128
//            in the base view, 16*q_b + q_r biased by 136 in the full view)
//            is put under the f16 exponent byte 0x64 by v_perm_b32, giving
//            the exact f16 1024 + u. Both views thus carry codes at s/16
//            with a bias of about 18 times their typical size. The bias is
//            not subtracted per value: its contribution to a row's scores
//            is one MFMA with a constant operand (taken off inside the
//            exp2), and to O one more MFMA per 32 tokens (taken off at the
//            end).
//   phase B  waves split the query rows into 16-row tiles and, when rows
//            are few, the block's four 32-token k-steps. Each keeps an
//            online softmax (log2 domain, exp2f) and multiplies with
//            v_mfma_f32_16x16x32_f16:
//              S^T = K Q^T    (A = 16 tokens x 32 dims from LDS, B = Q^T)
//              O^T += V^T P^T (A = 16 dims x 32 tokens from LDS, B = P^T)
// Inside a block, token tile 2j+e row 4q+i holds token 32q + 8j + 4e + i.
// Then the S^T values a lane holds are exactly the P^T operand it needs.
// Waves that share a row tile merge in LDS in a fixed order, and each
// workgroup writes one partial (max, sum, O) per row. A second kernel
// merges the partials over chunks with log-sum-exp weights, also in a
// fixed order.
//
// Range. Only exact integers and values in [0, 1] pass through f16:
//   - each query row is multiplied by a power of two 2^e chosen from its
//     largest |value| (bf16 has fp32's exponent range, f16 does not), and
//     2^-e goes into the fp32 score scale;
//   - a block's softmax weights enter the PV product relative to the
//     block's own largest score (so the largest is 1), and the V block
//     scale together with the factor from the block's maximum to the
//     running maximum multiply the block's fp32 product.
// The result then does not depend on the magnitude of q, K or V beyond
// fp32's range.
#include "quant.h"

namespace {


constexpr int kD = 128;
constexpr int kBlk = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTargetBlocks = 512;  // LDS-table kernel: workgroups to aim for (two resident per CU)
constexpr int kTargetWaves = 2048;  // wave kernel: waves to aim for (eight per CU)

struct AttArgs {
  const uint16_t* q;
  int nq, Hq, grp, R;  // R = nq * grp query rows per kv head
  int ctx;             // visible length (an offset added to *ctx_dev when that is given)
  const int32_t* ctx_dev;  // device word holding the rest of the length, or null
  const uint8_t *kb, *kr, *vb, *vr;
  const float *ks, *vs;
  int cap, nb;         // capacity and blocks per head in the planes
  const float *shk, *shv;  // exact mode: fp32 shadows [Hkv][2][block][d] of the two newest blocks
  uint8_t* open;           // exact mode: [nq][Hkv] rebuilt open blocks, 4 planes each
  float* open_sc;          // exact mode: [nq][Hkv][2] their scales (K, V)
  // exact mode with the append folded in (kv_nest_append_attend_exact): the
  // pass's nq new tokens [Hkv][nq][d] (null otherwise), and what the append
  // writes: the touched blocks' planes and scales and the new tokens' shadow
  // rows. The first new position is ctx - nq; an append that would not fit
  // in the cache writes nothing (the pass then sees the planes and shadow as
  // they were), as kv_nest_append does.
  const float *knew, *vnew;
  uint8_t *w_kb, *w_kr, *w_vb, *w_vr;
  float *w_ks, *w_vs, *w_shk, *w_shv;
  int zbase;               // open_block_kernel: layer index of blockIdx.z = 0 (the append alone: nq)
  int qpack;               // exact mode: queries per workgroup (qpack * grp <= 16)
  int bpw, nchunk;     // blocks per workgroup, chunks (workgroups) per head
  float* part_ml;      // [Hkv][nchunk][R][2]  (max in log2 domain, sum)
  float* part_o;       // [Hkv][nchunk][R][128]
  float* out;          // [nq][Hq][128]
};

__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t x, uint32_t y) { return (x & m) | (y & ~m); }

// One 32-bit word of codes (8 elements e0..e7, e_{2b} in the low nibble of
// byte b) -> 8 biased f16 code values in the order [e0 e2 e4 e6 e1 e3 e5 e7]:
// f16 (1024 + u) with u the byte put under the exponent byte 0x64 by
// v_perm_b32, one permute per two values. View 0: u = 16*q_b + 128, i.e.
// the value 1152 + 16*q_b. View 1: u = c + 136 with c = 16*q_b + q_r, i.e.
// 1160 + c. Both are codes at s/16 plus a bias, removed afterwards from
// whole sums (kernels below).
template <int VIEW>
__device__ __forceinline__ uint4 codes_to_h8b(uint32_t wb, uint32_t wr) {
  const uint32_t xb = wb ^ 0x88888888u;
  uint32_t ev, od;
  if (VIEW == 0) {
    ev = (xb << 4) & 0xF0F0F0F0u;  // 16 (q_b + 8) of even elements
    od = xb & 0xF0F0F0F0u;         // 16 (q_b + 8) of odd elements
  } else {
    const uint32_t xr = wr ^ 0x88888888u;
    ev = bfi(0xF0F0F0F0u, xb << 4, xr);  // c + 136
    od = bfi(0xF0F0F0F0u, xb, xr >> 4);
  }
  const uint32_t c64 = 0x64646464u;
  uint4 r;
  r.x = __builtin_amdgcn_perm(c64, ev, 0x04010400u);
  r.y = __builtin_amdgcn_perm(c64, ev, 0x04030402u);
  r.z = __builtin_amdgcn_perm(c64, od, 0x04010400u);
  r.w = __builtin_amdgcn_perm(c64, od, 0x04030402u);
  return r;
}

// The bias of codes_to_h8b as an f16 operand (1152 for view 0, 1160 for
// view 1): its product with a partner operand is the amount to take off
// the biased product.
template <int VIEW>
__device__ __forceinline__ uint4 bias_h8() {
  return VIEW == 0 ? make_uint4(0x64806480u, 0x64806480u, 0x64806480u, 0x64806480u)
                   : make_uint4(0x64886488u, 0x64886488u, 0x64886488u, 0x64886488u);
}

__device__ __forceinline__ v4f mfma_h(uint4 a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Exponent e of a query row's power-of-two factor: the largest |value| of
// the row (its 128 bf16 values are spread over the four lanes c16 + 16*q4,
// 32 each in qraw) times 2^e lies in [2^14, 2^15), well inside f16's
// normal range, and every bf16 value of the row times 2^e is then exactly
// an f16 (8 significant bits) unless it is below 2^-28 of the largest.
// An all-zero row gives 0.
__device__ __forceinline__ int q_row_exp(const uint4 (&qraw)[4]) {
  uint32_t mx = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = max(mx, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
  mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), 16, 64)));
  mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), 32, 64)));
  if (mx == 0) return 0;
  return 15 - __builtin_amdgcn_frexp_expf(__uint_as_float(mx << 16));
}

// 8 bf16 query values (dims 8s .. 8s+7, two per word, even dim in the low
// half) times 2^e -> the f16 operand order [e0 e2 e4 e6 e1 e3 e5 e7] of
// codes_to_h8b
__device__ __forceinline__ v8h bf16x8_to_op(uint4 w, int e) {
  auto cv = [e](uint32_t bits) {
    return static_cast<_Float16>(__builtin_amdgcn_ldexpf(__uint_as_float(bits), e));
  };
  v8h v;
  v[0] = cv(w.x << 16);
  v[1] = cv(w.y << 16);
  v[2] = cv(w.z << 16);
  v[3] = cv(w.w << 16);
  v[4] = cv(w.x & 0xFFFF0000u);
  v[5] = cv(w.y & 0xFFFF0000u);
  v[6] = cv(w.z & 0xFFFF0000u);
  v[7] = cv(w.w & 0xFFFF0000u);
  return v;
}

__device__ __forceinline__ uint32_t word(uint4 v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The visible length of a call: the host value, plus the device word when
// one is given. A device length outside [nq, capacity] is clamped into it,
// so no read leaves the planes.
__device__ __forceinline__ int live_ctx(const AttArgs& a) {
  if (!a.ctx_dev) return a.ctx;
  const long long c = static_cast<long long>(a.ctx) + *a.ctx_dev;
  return static_cast<int>(c < a.nq ? a.nq : (c > a.cap ? a.cap : c));
}

// LDS operand tables (uint4 = 8 f16):
//   K: slot ((tt*4 + s)*4 + q)*16 + r: token tau(tt, r), dims 32q + 8s + [0 2 4 6 1 3 5 7]
//   V: slot ((dt*4 + j)*4 + q)*16 + r: dim dt*16 + r, tokens 32q + 8j + [0 2 4 6 1 3 5 7]
// with tau(tt, r) = 32*(r>>2) + 8*(tt>>1) + 4*(tt&1) + (r&3).
__device__ __forceinline__ int op_slot(int a, int b, int q, int r) { return ((a * 4 + b) * 4 + q) * 16 + r; }

template <int RT, int VIEW>
__global__ void __launch_bounds__(256) attend_kernel(AttArgs a) {
  __shared__ uint4 kf[2048];
  __shared__ uint4 vf[2048];
  // waves per row tile (TS) and 32-token k-steps per wave (JS)
  constexpr int TS = RT == 1 ? 4 : (RT == 2 ? 2 : 1);
  constexpr int JS = 4 / TS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int ctx = live_ctx(a), nbv = (ctx + kBlk - 1) / kBlk;
  const int rt = wave / TS, tp = wave % TS, j0 = tp * JS;
  const bool active = rt < RT;

  // Query operand of row rt*16 + c16, k-step s: dims 32*q4 + 8*s + [0 2 4 6 1 3 5 7].
  // Its raw bytes (four 16-byte loads) are requested with the first block's
  // codes, and converted while those are on the way.
  uint4 qraw[4];
  int pos = -1;
  {
    const int rho = rt * 16 + c16;
    if (active && rho < a.R) {
      const int i = rho / a.grp, g = rho % a.grp;
      pos = ctx - a.nq + i;
      const uint16_t* qr = a.q + (static_cast<size_t>(i) * a.Hq + h * a.grp + g) * kD + 32 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s) qraw[s] = ld16(qr + 8 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qraw[s] = make_uint4(0, 0, 0, 0);
    }
  }
  const int b_first = chunk * a.bpw;
  const int b_last = min(b_first + a.bpw, nbv);

  // Phase A items of this thread: it = threadIdx.x + 256*rep is (t, q, r) with
  // t = it >> 6 (K token tile / V dim tile), q = (it >> 4) & 3, r = it & 15.
  // The next block's codes are loaded into registers while the current block
  // is multiplied (software pipelining across blocks).
  uint4 ck_b[2], ck_r[2], cv_b[2], cv_r[2];
  auto load_codes = [&](int blk) {
    const int t0 = blk * kBlk;
    const size_t hb = static_cast<size_t>(h) * a.nb + blk;
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int it = threadIdx.x + rep * 256;
      const int t = it >> 6, q = (it >> 4) & 3, r = it & 15;
      const int tok = 32 * (r >> 2) + 8 * (t >> 1) + 4 * (t & 1) + (r & 3);
      const size_t koff = (static_cast<size_t>(h) * a.cap + t0 + tok) * (kD / 2) + 16 * q;
      const size_t voff = (hb * kD + t * 16 + r) * (kBlk / 2) + 16 * q;
      ck_b[rep] = nest::ldnt16(a.kb + koff);
      cv_b[rep] = nest::ldnt16(a.vb + voff);
      if (VIEW) {
        ck_r[rep] = nest::ldnt16(a.kr + koff);
        cv_r[rep] = nest::ldnt16(a.vr + voff);
      } else {
        ck_r[rep] = make_uint4(0, 0, 0, 0);
        cv_r[rep] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  if (b_first < b_last) load_codes(b_first);
  // the query operand of this lane's row, times the row's power of two
  const int qe = q_row_exp(qraw);
  v8h qop[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qop[s] = bf16x8_to_op(qraw[s], qe);

  // Biased codes in the tables (codes_to_h8b): the row's bias
  // sum(q * bias) is one product with the bias operand, taken off every
  // score of the row.
  float kbias;
  {
    v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_h(bias_h8<VIEW>(), qop[s], acc);
    kbias = acc[0];  // every row of the product is the same
  }

  float m = -INFINITY, l = 0.0f;
  float Ob = 0.0f;  // the bias part of O (the same for every dim)
  v4f O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = v4f{0, 0, 0, 0};

  // score scale in log2 units: codes at s/16, 1/sqrt(128), and the
  // query row's 2^-qe
  const float sm_scale = __builtin_amdgcn_ldexpf(0.0625f * 0.08838834764831845f * kLog2e, -qe);
  // blocks ending at or before the first query's position need no mask
  const int pos_min = ctx - a.nq;

  for (int blk = b_first; blk < b_last; ++blk) {
    const int t0 = blk * kBlk;
    const size_t hb = static_cast<size_t>(h) * a.nb + blk;

    // ---- phase A: codes -> f16 operands in LDS, then prefetch the next block ----
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int it = threadIdx.x + rep * 256;
      const int t = it >> 6, q = (it >> 4) & 3, r = it & 15;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[op_slot(t, s, q, r)] = codes_to_h8b<VIEW>(word(ck_b[rep], s), word(ck_r[rep], s));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vf[op_slot(t, j, q, r)] = codes_to_h8b<VIEW>(word(cv_b[rep], j), word(cv_r[rep], j));
    }
    if (blk + 1 < b_last) load_codes(blk + 1);
    __syncthreads();

    // ---- phase B: this wave's row tile over its k-steps ----
    if (active) {
      const float ck = a.ks[hb] * sm_scale;
      const float sv = a.vs[hb] * 0.0625f;
      v4f S[2 * JS];
#pragma unroll
      for (int jj = 0; jj < JS; ++jj)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tt = 2 * (j0 + jj) + e;
          v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma_h(kf[op_slot(tt, s, q4, c16)], qop[s], acc);
          S[2 * jj + e] = acc;
        }
      // maximum of the biased scores of this wave's tokens (the bias and
      // the scale ck >= 0 are applied after); the mask only near the end
      const bool masked = t0 + kBlk - 1 > pos_min;
      float mb = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < JS; ++jj)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (masked) {
              const int tok = t0 + 32 * q4 + 8 * (j0 + jj) + 4 * e + i;
              if (tok > pos) S[2 * jj + e][i] = -INFINITY;
            }
            mb = fmaxf(mb, S[2 * jj + e][i]);
          }
      mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
      mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
      // weights relative to this block's largest score (largest weight 1),
      // then beta = 2^(block max - running max) in fp32
      const bool live = mb != -INFINITY;
      const float mbs = live ? (mb - kbias) * ck : -INFINITY;
      const float c2 = live ? fmaf(kbias, ck, mbs) : 0.0f;
      const float mn = fmaxf(m, mbs);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m - mu);
      const float beta = live ? __builtin_amdgcn_exp2f(mbs - mu) : 0.0f;
      float ls = 0.0f;
#pragma unroll
      for (int k = 0; k < 2 * JS; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = __builtin_amdgcn_exp2f(fmaf(S[k][i], ck, -c2));
          if (masked) p = S[k][i] == -INFINITY ? 0.0f : p;
          S[k][i] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      l = fmaf(ls, beta, l * alpha);
      m = mn;
      // the block's product with weights in [0, 1], then the V scale and
      // beta applied to it in fp32
      v4f Ot[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) Ot[dt] = v4f{0, 0, 0, 0};
      v4f Obt = v4f{0, 0, 0, 0};
#pragma unroll
      for (int jj = 0; jj < JS; ++jj) {
        const v4f e0 = S[2 * jj], e1 = S[2 * jj + 1];
        v8h p;
        p[0] = (_Float16)e0[0]; p[1] = (_Float16)e0[2];
        p[2] = (_Float16)e1[0]; p[3] = (_Float16)e1[2];
        p[4] = (_Float16)e0[1]; p[5] = (_Float16)e0[3];
        p[6] = (_Float16)e1[1]; p[7] = (_Float16)e1[3];
        const int j = j0 + jj;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) Ot[dt] = mfma_h(vf[op_slot(dt, j, q4, c16)], p, Ot[dt]);
        Obt = mfma_h(bias_h8<VIEW>(), p, Obt);
      }
      const float w = sv * beta;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[dt][i] = fmaf(w, Ot[dt][i], O[dt][i] * alpha);
      Ob = fmaf(w, Obt[0], Ob * alpha);
    }
    __syncthreads();  // the next block's phase A overwrites the tables
  }

  // take the V bias off (every dim of a row has the same bias sum)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] -= Ob;

  // ---- write this workgroup's partial per row ----
  const size_t pbase = (static_cast<size_t>(h) * a.nchunk + chunk) * a.R;
  if (TS == 1) {
    const int rho = rt * 16 + c16;
    if (active && rho < a.R) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(&a.part_o[(pbase + rho) * kD + dt * 16 + 4 * q4]) =
            make_float4(O[dt][0], O[dt][1], O[dt][2], O[dt][3]);
      if (q4 == 0) {
        a.part_ml[(pbase + rho) * 2 + 0] = m;
        a.part_ml[(pbase + rho) * 2 + 1] = l;
      }
    }
    return;
  }
  // TS waves share a row tile: merge them in LDS, in the fixed order tp = TS-1 .. 0
  float* ml = reinterpret_cast<float*>(kf);      // [4 waves][16 rows][2]
  float* buf = reinterpret_cast<float*>(vf);     // [RT][16 rows][132]
  if (q4 == 0) {
    ml[(wave * 16 + c16) * 2 + 0] = m;
    ml[(wave * 16 + c16) * 2 + 1] = l;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int t = 0; t < TS; ++t) M = fmaxf(M, ml[((rt * TS + t) * 16 + c16) * 2]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  const float f = exp2f(m - Mu);
  for (int step = TS - 1; step >= 0; --step) {
    if (active && tp == step) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* p = &buf[(rt * 16 + c16) * (kD + 4) + dt * 16 + 4 * q4 + i];
          const float v = O[dt][i] * f;
          *p = (step == TS - 1) ? v : *p + v;
        }
    }
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < a.R * kD; idx += 256) {
    const int row = idx / kD, dim = idx % kD;
    if (row < RT * 16) a.part_o[(pbase + row) * kD + dim] = buf[row * (kD + 4) + dim];
  }
  if (threadIdx.x < a.R && static_cast<int>(threadIdx.x) < RT * 16) {
    const int row = threadIdx.x, r16 = row & 15, t_rt = row >> 4;
    float Mr = -INFINITY;
    for (int t = 0; t < TS; ++t) Mr = fmaxf(Mr, ml[((t_rt * TS + t) * 16 + r16) * 2]);
    const float Mru = Mr == -INFINITY ? 0.0f : Mr;
    float L = 0.0f;
    for (int t = 0; t < TS; ++t) {
      const int w = t_rt * TS + t;
      L += ml[(w * 16 + r16) * 2 + 1] * exp2f(ml[(w * 16 + r16) * 2] - Mru);
    }
    a.part_ml[(pbase + row) * 2 + 0] = Mr;
    a.part_ml[(pbase + row) * 2 + 1] = L;
  }
}

// Exact mode (kv_nest_attend_exact), first kernel: for every query z of the
// pass and kv head h, the block holding the query's position, rebuilt from
// its fp32 values in the shadow and quantized over its tokens up to that
// position alone, with the rule and the layouts kv_nest_append uses: the
// codes and scales a one-token append at that position would have
// written. Each goes to its own slot of the workspace, laid out as a block
// of the planes (K base, K refine: [token][64 B]; V base, V refine:
// [dim][64 B]), and its two scales (K, V) to open_sc.
//
// Grid (kOpenSplit, Hkv, 2 nq): workgroup (part, h, 2z + is_v) reduces the
// plane's max |x| over the valid tokens (every part reads the whole valid
// region, from L2 after the first) and writes part's eighth of the codes,
// one 32-bit word of each plane per thread (8 elements, element 2m in the
// low nibble of byte m).
constexpr int kOpenPlane = kBlk * kD / 2;  // bytes of one plane of one block
constexpr int kOpenSplit = 8;              // workgroups per (query, kv head, K or V)
static_assert(kOpenSplit * 256 * 8 == kBlk * kD, "one word of each plane per thread");

// With the append folded in (a.knew set), tokens at or past the first new
// position come from the new values rather than the shadow, and the grid
// carries four more workgroup layers (z = 2 nq .. 2 nq + 3): the append of
// the pass's tokens to the (at most two) blocks they touch, K or V, each
// workgroup the same eighth of the codes as above, quantized over the
// block's tokens up to the pass's last one, with the scale and its share of
// the new tokens' shadow rows. The rebuilds read only older tokens from the
// shadow, and no workgroup here reads the planes, so the layers are
// independent of one another.
__global__ void __launch_bounds__(256) open_block_kernel(AttArgs a) {
  __shared__ float red[4];
  const int part = blockIdx.x, h = blockIdx.y;
  const int zz = a.zbase + (static_cast<int>(blockIdx.z) >> 1);
  const bool is_v = (blockIdx.z & 1) != 0;
  const bool append = zz >= a.nq;  // an append layer (only when a.knew is set)
  const int Hkv = a.Hq / a.grp;
  const int ctx = live_ctx(a), pos0 = ctx - a.nq;  // the pass's first position
  // the append happened (or happens here) only if the tokens fit
  const bool fits = a.knew && (!a.ctx_dev || static_cast<long long>(a.ctx) + *a.ctx_dev == ctx);
  if (append && !fits) return;
  // the block and its last token: query zz's own position, or for an append
  // layer the pass's last token in the first or second block it touches
  int blk, pos;
  if (append) {
    blk = pos0 / kBlk + (zz - a.nq);
    if (blk * kBlk > ctx - 1) return;  // the second block, not touched
    pos = min(ctx - 1, blk * kBlk + kBlk - 1);
  } else {
    pos = pos0 + zz;
    blk = pos / kBlk;
  }
  const int t0 = blk * kBlk, valid = pos - t0 + 1;
  const float* sh = (is_v ? a.shv : a.shk) + (static_cast<size_t>(h) * 2 + (blk & 1)) * kBlk * kD;
  // tokens [0, old) of the block from the shadow, [old, valid) new (new
  // token t0 + t - pos0 of the pass)
  const int old = fits ? max(0, min(valid, pos0 - t0)) : valid;
  const float* nwh = fits ? (is_v ? a.vnew : a.knew) + static_cast<size_t>(h) * a.nq * kD : nullptr;
  auto row_ptr = [&](int t) {  // token t of the block
    return t < old ? sh + t * kD : nwh + static_cast<ptrdiff_t>(t0 + t - pos0) * kD;
  };
  // 1. max |x| over tokens [0, valid) (token-major); all loads are issued
  // together
  const int n4 = valid * (kD / 4);
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < kBlk * kD / 4 / 256; ++u) {
    const int i = static_cast<int>(threadIdx.x) + 256 * u;
    if (i < n4) {
      const float4 v = reinterpret_cast<const float4*>(row_ptr(i / (kD / 4)))[i % (kD / 4)];
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m / 7.0f, s16 = s * 0.0625f, rs = 1.0f / s, rs16 = 1.0f / s16;
  const size_t slot = static_cast<size_t>(zz) * Hkv + h;
  const size_t hb = static_cast<size_t>(h) * a.nb + blk;
  if (part == 0 && threadIdx.x == 0) {
    if (append)
      (is_v ? a.w_vs : a.w_ks)[hb] = s;
    else
      a.open_sc[slot * 2 + (is_v ? 1 : 0)] = s;
  }
  // 2. word w of each plane: elements 8w .. 8w + 7 in plane order (K: token
  // 8w / 128, dims 8w % 128 ..; V: dim 8w / 128, tokens 8w % 128 ..)
  const int w = part * 256 + static_cast<int>(threadIdx.x);
  const int row = (8 * w) / kD, c0 = (8 * w) % kD;
  float x[8];
  if (is_v) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = c0 + j < valid ? row_ptr(c0 + j)[row] : 0.0f;
  } else {
    const bool in = row < valid;
    const float* src = row_ptr(in ? row : 0) + c0;
    const float4 lo = reinterpret_cast<const float4*>(src)[0];
    const float4 hi = reinterpret_cast<const float4*>(src)[1];
    x[0] = in ? lo.x : 0.0f; x[1] = in ? lo.y : 0.0f; x[2] = in ? lo.z : 0.0f; x[3] = in ? lo.w : 0.0f;
    x[4] = in ? hi.x : 0.0f; x[5] = in ? hi.y : 0.0f; x[6] = in ? hi.z : 0.0f; x[7] = in ? hi.w : 0.0f;
  }
  uint32_t wb = 0, wr = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int qb, qr;
    nest::nest_codes_fast(x[j], s, s16, rs, rs16, qb, qr);
    wb |= static_cast<uint32_t>(qb & 15) << (4 * j);
    wr |= static_cast<uint32_t>(qr & 15) << (4 * j);
  }
  if (append) {
    // the cache's block: K planes [token][64 B] from (h cap + t0) * 64, V
    // planes [dim][64 B] from hb * 128 * 64 (the slot layout)
    const size_t off = is_v ? hb * kD * (kBlk / 2) : (static_cast<size_t>(h) * a.cap + t0) * (kD / 2);
    reinterpret_cast<uint32_t*>((is_v ? a.w_vb : a.w_kb) + off)[w] = wb;
    reinterpret_cast<uint32_t*>((is_v ? a.w_vr : a.w_kr) + off)[w] = wr;
    // this workgroup's share of the new tokens' shadow rows [old, valid)
    float* shw = (is_v ? a.w_shv : a.w_shk) + (static_cast<size_t>(h) * 2 + (blk & 1)) * kBlk * kD;
    for (int i = (old * kD) / 4 + w; i < (valid * kD) / 4; i += kOpenSplit * 256)
      reinterpret_cast<float4*>(shw)[i] = reinterpret_cast<const float4*>(row_ptr(i / (kD / 4)))[i % (kD / 4)];
    return;
  }
  uint8_t* base = a.open + (slot * 4 + (is_v ? 2 : 0)) * kOpenPlane;
  reinterpret_cast<uint32_t*>(base)[w] = wb;
  reinterpret_cast<uint32_t*>(base + kOpenPlane)[w] = wr;
}

// Few query rows (R <= 16, e.g. one draft query over a GQA group): every
// wave owns whole 128-token blocks. Lane (q4, c16) loads exactly the 16-byte
// code slices its MFMA operands need (K: token tau(tt, c16), dims
// 32*q4..32*q4+31, for the 8 token tiles; V: dim 16*dt + c16, tokens
// 32*q4..32*q4+31, for the 8 dim tiles) and converts them in registers, so
// the loop has no LDS tables and no barrier. Several resident waves per
// SIMD overlap one wave's loads with another's arithmetic. The 4 waves of a workgroup
// take interleaved blocks of its chunk and merge once at the end, in LDS,
// in the fixed order w = 3 .. 0. The grid holds about two waves per SIMD
// (one block per wave, kTargetWaves), so the register budget of two waves
// per SIMD is free: the MFMA accumulators then stay in VGPRs (no AGPR round
// trips per block).
//
// EXACT (kv_nest_attend_exact): each query of a verify pass is computed as
// the one-query call at its own position would compute it, in one launch.
// A workgroup serves one (chunk, kv head, group of qpack consecutive
// queries); its rows are those queries' GQA groups side by side (query
// z_lo + r / grp, head r % grp in row r; qpack * grp <= 16). A block that
// comes before every row's own block is processed once for all rows from
// the planes. A block that holds some rows' positions is processed once
// from the planes for the rows it is sealed for (their position lies in a
// later block), then once per query it holds, from that query's slot (the
// open block open_block_kernel rebuilt), each time with every other row
// masked. Every row therefore sees exactly the blocks, codes and order of
// the one-query call at its position, with the same split into chunks and
// the same merge; a call in which a row is masked leaves its running
// maximum, sum and output unchanged (or, as the wave's first call, at the
// state of an empty wave, from which the next call yields what a first
// call would), so the outputs are bit-identical to the one-query call.
// Workgroups are numbered so that the query groups of one (chunk, head)
// run one after another on one XCD and share its L2.
template <int VIEW, bool EXACT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
attend_wave_kernel(AttArgs a) {
  __shared__ float ml[4][16][2];
  __shared__ __align__(16) float buf[4][16][kD + 4];  // each wave's rescaled O
  // the wave index is uniform: block numbers, scale loads and branches on
  // them stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q4 = lane >> 4, c16 = lane & 15;
  int h = blockIdx.y, chunk = blockIdx.x, z_lo = 0, nz = 1;
  if (EXACT) {
    // item = (chunk, head, query group) with the group fastest; XCD x (=
    // block id mod 8) takes the contiguous items [x * per, (x + 1) * per),
    // so the groups of one (chunk, head) run together on one XCD and share
    // its L2
    const int ngrp = (a.nq + a.qpack - 1) / a.qpack;
    const int n_items = a.nchunk * (a.Hq / a.grp) * ngrp;
    const int per = (n_items + 7) / 8;
    const int item = (static_cast<int>(blockIdx.x) & 7) * per + (static_cast<int>(blockIdx.x) >> 3);
    if (item >= n_items) return;
    z_lo = (item % ngrp) * a.qpack;
    nz = min(a.qpack, a.nq - z_lo);
    chunk = (item / ngrp) % a.nchunk;
    h = item / ngrp / a.nchunk;
  }
  const int ctx = live_ctx(a);
  // exact: the group's first and last positions and the blocks holding them
  // (the group sees blocks up to the last one)
  const int pos_lo = ctx - a.nq + z_lo;
  const int b_open_lo = EXACT ? pos_lo / kBlk : -1;
  const int b_open_hi = EXACT ? (pos_lo + nz - 1) / kBlk : -1;
  const int nbv = EXACT ? b_open_hi + 1 : (ctx + kBlk - 1) / kBlk;

  const int b_first = chunk * a.bpw;
  const int b_last = min(b_first + a.bpw, nbv);
  const int b0 = b_first + wave;  // the wave's blocks are b0, b0 + 4, ...

  uint4 kb[8], kr[8], vb[8], vr[8];
  float ks, vs;
  // K codes first, then V: loads return in issue order, so the scores and
  // the softmax of a block start while its V codes are still on the way
  auto load = [&](int blk, int zs) {
    // the block's four planes (K [token][64 B], V [dim][64 B]) and scales:
    // from the cache, or, in exact mode with zs >= 0, query zs's rebuilt
    // open block (the same layout)
    const uint8_t *pkb, *pkr, *pvb, *pvr;
    if (EXACT && zs >= 0) {
      const size_t slot = static_cast<size_t>(zs) * (a.Hq / a.grp) + h;
      pkb = a.open + slot * 4 * kOpenPlane;
      pkr = pkb + kOpenPlane;
      pvb = pkb + 2 * kOpenPlane;
      pvr = pkb + 3 * kOpenPlane;
      ks = a.open_sc[slot * 2];
      vs = a.open_sc[slot * 2 + 1];
    } else {
      const size_t hb = static_cast<size_t>(h) * a.nb + blk;
      const size_t kblk = (static_cast<size_t>(h) * a.cap + static_cast<size_t>(blk) * kBlk) * (kD / 2);
      pkb = a.kb + kblk;
      pkr = a.kr + kblk;
      pvb = a.vb + hb * kD * (kBlk / 2);
      pvr = a.vr + hb * kD * (kBlk / 2);
      ks = a.ks[hb];
      vs = a.vs[hb];
    }
    auto ld = [](const uint8_t* p) { return nest::ldnt16(p); };
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int tok = 32 * (c16 >> 2) + 8 * (tt >> 1) + 4 * (tt & 1) + (c16 & 3);
      const int koff = tok * (kD / 2) + 16 * q4;
      kb[tt] = ld(pkb + koff);
      kr[tt] = VIEW ? ld(pkr + koff) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int voff = (tt * 16 + c16) * (kBlk / 2) + 16 * q4;
      vb[tt] = ld(pvb + voff);
      vr[tt] = VIEW ? ld(pvr + voff) : make_uint4(0, 0, 0, 0);
    }
  };

  // The query (dims 32*q4 .. 32*q4 + 31 of row c16: four 16-byte loads) and
  // the first block's codes are requested together; the query operand and
  // the bias product are formed while the codes are on the way.
  uint4 qraw[4];
  int pos = -1, zr = -1;
  // rows of this workgroup: its query group's GQA groups (exact), or all R
  // rows; row c16 is query c16 / grp (of the group) and head c16 % grp
  const int nrow = EXACT ? nz * a.grp : a.R;
  if (c16 < nrow) {
    const int i = (EXACT ? z_lo : 0) + c16 / a.grp, g = c16 % a.grp;
    zr = i;
    pos = ctx - a.nq + i;
    const uint16_t* qr = a.q + (static_cast<size_t>(i) * a.Hq + h * a.grp + g) * kD + 32 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = ld16(qr + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = make_uint4(0, 0, 0, 0);
  }
  // exact: the wave's calls (blk, zc) in order: per block, first the
  // planes (zc = z_lo - 1) when the block is sealed for some row, then each
  // query zc of the group whose position the block holds
  auto call_ok = [&](int blk, int zc) {
    return zc < z_lo ? blk < b_open_hi : (ctx - a.nq + zc) / kBlk == blk;
  };
  auto next_call = [&](int& blk, int& zc) {
    for (;;) {
      if (++zc >= z_lo + nz) {
        blk += 4;
        zc = z_lo - 1;
      }
      if (blk >= b_last) return false;
      if (call_ok(blk, zc)) return true;
    }
  };
  int cblk = b0, czc = z_lo - 1;
  bool have = b0 < b_last;
  if (EXACT && have && !call_ok(cblk, czc)) have = next_call(cblk, czc);
  // unconditional (a wave without a block of its own reads the chunk's first
  // block and discards it): a load under a branch makes the compiler copy
  // the codes at the join, which waits for all of them
  load(have ? cblk : b_first, (EXACT && have && czc >= z_lo) ? czc : -1);
  __builtin_amdgcn_sched_barrier(0);
  // the query operand of this lane's row, times the row's power of two
  const int qe = q_row_exp(qraw);
  v8h qop[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qop[s] = bf16x8_to_op(qraw[s], qe);

  // Biased codes (codes_to_h8b): the row's bias sum(q * bias) is one
  // product with the bias operand, taken off every score of the row.
  float kbias;
  {
    v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_h(bias_h8<VIEW>(), qop[s], acc);
    kbias = acc[0];  // every row of the product is the same
  }

  float m = -INFINITY, l = 0.0f;
  float Ob = 0.0f;  // the bias part of O (the same for every dim)
  v4f O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = v4f{0, 0, 0, 0};
  // score scale in log2 units: codes at s/16, 1/sqrt(128), and the query
  // row's 2^-qe
  const float sm_scale = __builtin_amdgcn_ldexpf(0.0625f * 0.08838834764831845f * kLog2e, -qe);

  // Rows whose position is at least pos_min see every token of a block that
  // ends at or before pos_min; only later blocks need the causal mask (and,
  // in exact mode, every call with masked rows: force). pc is this row's
  // position for the call, -1 for a masked row.
  const int pos_min = pos_lo;
  auto block = [&](int blk, bool first, int pc, bool force) {
    const uint4 *ck = kb, *cr = kr, *dk = vb, *dr = vr;
    const int t0 = blk * kBlk;
    const float sk = ks * sm_scale;
    const float sv = vs * 0.0625f;
    v4f S[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = mfma_h(codes_to_h8b<VIEW>(word(ck[tt], s), word(cr[tt], s)), qop[s], acc);
      S[tt] = acc;  // kbias + q . k
    }
    // block maximum of the biased scores (the bias and the scale sk >= 0
    // are applied after)
    const bool masked = force || t0 + kBlk - 1 > pos_min;
    float mb = -INFINITY;
    if (masked) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + 32 * q4 + 8 * (tt >> 1) + 4 * (tt & 1) + i;
          if (tok > pc) S[tt][i] = -INFINITY;
          mb = fmaxf(mb, S[tt][i]);
        }
    } else {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mb = fmaxf(mb, S[tt][i]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    // p = 2^(score - block max) in [0, 1] (up to rounding), the largest 1:
    // the hardware exp2 (flushing results below 2^-126 to zero, which no
    // sum here can notice); masked tokens give 0. beta = 2^(block max -
    // running max) carries the block to the running maximum in fp32.
    const bool live = mb != -INFINITY;
    const float mbs = live ? (mb - kbias) * sk : -INFINITY;
    const float c2 = live ? fmaf(kbias, sk, mbs) : 0.0f;
    const float mn = fmaxf(m, mbs);
    const float mu = mn == -INFINITY ? 0.0f : mn;
    const float beta = live ? __builtin_amdgcn_exp2f(mbs - mu) : 0.0f;
    float ls = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(fmaf(S[tt][i], sk, -c2));
        if (masked) p = S[tt][i] == -INFINITY ? 0.0f : p;
        S[tt][i] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    const float alpha = first ? 0.0f : __builtin_amdgcn_exp2f(m - mu);
    l = first ? ls * beta : fmaf(ls, beta, l * alpha);
    m = mn;
    // a scheduling fence: the V codes are converted only here, after the
    // softmax, so the scores never wait for them
    __builtin_amdgcn_sched_barrier(0);
    // the block's product with the weights in [0, 1]; the V scale and
    // beta are applied to it in fp32 (the first block accumulates straight
    // into O, which is still zero)
    v4f Ot[8];
    v4f Obt = v4f{0, 0, 0, 0};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) Ot[dt] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f e0 = S[2 * j], e1 = S[2 * j + 1];
      v8h p;
      p[0] = (_Float16)e0[0]; p[1] = (_Float16)e0[2];
      p[2] = (_Float16)e1[0]; p[3] = (_Float16)e1[2];
      p[4] = (_Float16)e0[1]; p[5] = (_Float16)e0[3];
      p[6] = (_Float16)e1[1]; p[7] = (_Float16)e1[3];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint4 vop = codes_to_h8b<VIEW>(word(dk[dt], j), word(dr[dt], j));
        if (first)
          O[dt] = mfma_h(vop, p, O[dt]);
        else
          Ot[dt] = mfma_h(vop, p, Ot[dt]);
      }
      Obt = mfma_h(bias_h8<VIEW>(), p, Obt);
    }
    const float w = sv * beta;
    if (first) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt] *= w;
      Ob = w * Obt[0];
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[dt][i] = fmaf(w, Ot[dt][i], O[dt][i] * alpha);
      Ob = fmaf(w, Obt[0], Ob * alpha);
    }
  };
  // the first block (already requested) starts the running max and sum, so
  // O needs no rescaling there; most waves own a single block
  if constexpr (EXACT) {
    const int b_row = pos >= 0 ? pos / kBlk : -1;  // the block holding this row's position
    bool first = true;
    while (have) {
      // planes: the rows for which the block is sealed; a query's slot: its rows
      const bool act = czc < z_lo ? (zr >= 0 && b_row > cblk) : zr == czc;
      block(cblk, first, act ? pos : -1, cblk >= b_open_lo);
      first = false;
      have = next_call(cblk, czc);
      if (have) {
        load(cblk, czc >= z_lo ? czc : -1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (b0 < b_last) {
    block(b0, true, pos, false);
    for (int blk = b0 + 4; blk < b_last; blk += 4) {
      load(blk, -1);
      __builtin_amdgcn_sched_barrier(0);
      block(blk, false, pos, false);
    }
  }
  // take the V bias off (every dim of a row has the same bias sum)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] -= Ob;

  // merge the 4 waves (fixed order w = 3 .. 0) and write the chunk's partial
  if (q4 == 0) {
    ml[wave][c16][0] = m;
    ml[wave][c16][1] = l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[w][c16][0]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  const float f = exp2f(m - Mu);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[wave][c16][dt * 16 + 4 * q4 + i] = O[dt][i] * f;
  __syncthreads();
  // the four waves' parts added in the fixed order w = 3 .. 0; in exact
  // mode this workgroup's rows are rows z_lo * grp .. of the call
  const size_t pbase = (static_cast<size_t>(h) * a.nchunk + chunk) * a.R + (EXACT ? z_lo * a.grp : 0);
  for (int idx = threadIdx.x; idx < nrow * (kD / 4); idx += 256) {
    const int row = idx / (kD / 4), d4 = idx % (kD / 4);
    float4 v = *reinterpret_cast<const float4*>(&buf[3][row][4 * d4]);
#pragma unroll
    for (int w = 2; w >= 0; --w) {
      const float4 u = *reinterpret_cast<const float4*>(&buf[w][row][4 * d4]);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    *reinterpret_cast<float4*>(&a.part_o[(pbase + row) * kD + 4 * d4]) = v;
  }
  if (static_cast<int>(threadIdx.x) < nrow) {
    const int row = threadIdx.x;
    float Mr = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mr = fmaxf(Mr, ml[w][row][0]);
    const float Mru = Mr == -INFINITY ? 0.0f : Mr;
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += ml[w][row][1] * exp2f(ml[w][row][0] - Mru);
    a.part_ml[(pbase + row) * 2 + 0] = Mr;
    a.part_ml[(pbase + row) * 2 + 1] = L;
  }
}

// Merge of the chunk partials: one block of 1024 threads per (row, kv head).
// Thread t sums the chunks c = t/128 (mod 8) of dim t % 128. Its first 16
// partial outputs are loaded before the chunk weights 2^(m_c - M) are
// known, so the kernel needs one round trip to memory for up to 128
// chunks. Each strand adds its chunks in ascending order, and the 8
// strands are then added in order (a fixed order overall).
constexpr int kStrands = 8;
constexpr int kBatch = 16;
constexpr int kMaxChunks = 4096;

__global__ void __launch_bounds__(1024) combine_kernel(AttArgs a) {
  __shared__ float wts[kMaxChunks];
  __shared__ float red_m[16], red_l[16];
  __shared__ float accs[kStrands][kD];
  const int row = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int dim = t & (kD - 1), strand = t >> 7, wave = t >> 6;
  const size_t base = static_cast<size_t>(h) * a.nchunk * a.R + row;  // partial of chunk c: base + c*R
  const size_t cstride = static_cast<size_t>(a.R) * kD;
  const float* po = a.part_o + base * kD + dim;
  float v[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int c = strand + i * kStrands;
    v[i] = c < a.nchunk ? po[static_cast<size_t>(c) * cstride] : 0.0f;
  }
  float M = -INFINITY;
  for (int c = t; c < a.nchunk; c += 1024) M = fmaxf(M, a.part_ml[(base + static_cast<size_t>(c) * a.R) * 2]);
  M = wave_max(M);
  if ((t & 63) == 0) red_m[wave] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) M = fmaxf(M, red_m[w]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float L = 0.0f;
  for (int c = t; c < a.nchunk; c += 1024) {
    const size_t pr = base + static_cast<size_t>(c) * a.R;
    const float mc = a.part_ml[pr * 2];
    const float w = mc == -INFINITY ? 0.0f : exp2f(mc - Mu);  // chunks with no visible token: O = 0
    wts[c] = w;
    L += w * a.part_ml[pr * 2 + 1];
  }
  L = wave_sum(L);
  if ((t & 63) == 0) red_l[wave] = L;
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int c = strand + i * kStrands;
    if (c < a.nchunk) acc = fmaf(v[i], wts[c], acc);
  }
  for (int c0 = kBatch * kStrands; c0 < a.nchunk; c0 += kBatch * kStrands) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + strand + i * kStrands;
      v[i] = c < a.nchunk ? po[static_cast<size_t>(c) * cstride] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + strand + i * kStrands;
      if (c < a.nchunk) acc = fmaf(v[i], wts[c], acc);
    }
  }
  accs[strand][dim] = acc;
  __syncthreads();
  if (strand == 0) {
    float o = accs[0][dim];
#pragma unroll
    for (int s2 = 1; s2 < kStrands; ++s2) o += accs[s2][dim];
    float Lt = red_l[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) Lt += red_l[w];
    const int i = row / a.grp, g = row % a.grp;
    a.out[(static_cast<size_t>(i) * a.Hq + h * a.grp + g) * kD + dim] = o / Lt;
  }
}

struct Plan {
  int nbv, bpw, nchunk, RT;
  size_t ws;
};

// Query rows per kv head one launch of kv_nest_attend holds (four 16-row
// tiles), and the queries per launch of a call that has more.
constexpr int kMaxRowsPerLaunch = 64;
int64_t chunk_queries(int64_t nq, int64_t grp) {
  const int64_t per = kMaxRowsPerLaunch / (grp > 0 ? grp : 1);
  return nq < per ? nq : (per > 0 ? per : 1);
}

// Work split. Up to 16 query rows: one 128-token block per wave while the
// chip has wave slots to spare (about kTargetWaves), 4 waves per workgroup.
// More rows: the LDS-table kernel with about kTargetBlocks workgroups.
Plan make_plan(int64_t nq, int64_t Hq, int64_t Hkv, int64_t ctx) {
  Plan p{};
  const int64_t R = nq * (Hq / Hkv);
  p.nbv = static_cast<int>((ctx + kBlk - 1) / kBlk);
  p.RT = static_cast<int>((R + 15) / 16);
  const int64_t blocks = Hkv * p.nbv;
  if (p.RT == 1) {
    const int64_t per_wave = (blocks + kTargetWaves - 1) / kTargetWaves;
    p.bpw = static_cast<int>(4 * per_wave);
  } else {
    p.bpw = static_cast<int>((blocks + kTargetBlocks - 1) / kTargetBlocks);
  }
  if (p.bpw < 1) p.bpw = 1;
  p.nchunk = (p.nbv + p.bpw - 1) / p.bpw;  // at most about max(kTargetWaves/4, kTargetBlocks)/Hkv + 1
  const size_t rows = static_cast<size_t>(Hkv) * p.nchunk * R;
  p.ws = (((rows * 2 + 3) & ~static_cast<size_t>(3)) + rows * kD) * sizeof(float);
  return p;
}

template <int VIEW>
int launch_att(const AttArgs& a, const Plan& p, int Hkv, hipStream_t st) {
  dim3 grid(p.nchunk, Hkv);
  switch (p.RT) {
    case 1: attend_wave_kernel<VIEW, false><<<grid, 256, 0, st>>>(a); break;
    case 2: attend_kernel<2, VIEW><<<grid, 256, 0, st>>>(a); break;
    case 3: attend_kernel<3, VIEW><<<grid, 256, 0, st>>>(a); break;
    default: attend_kernel<4, VIEW><<<grid, 256, 0, st>>>(a); break;
  }
  int rc = nest::check_launch("kv_nest_attend");
  if (rc) return rc;
  combine_kernel<<<dim3(a.R, Hkv), 1024, 0, st>>>(a);
  return nest::check_launch("kv_nest_attend(combine)");
}

// Exact mode's workspace: the partials of nq queries (R = nq * grp rows)
// under the one-query split, then, from a 256-byte boundary, the rebuilt
// open blocks [nq][Hkv][4 planes] and their scales [nq][Hkv][2].
struct ExactLayout {
  Plan p;
  size_t open_off, sc_off, bytes;
};

ExactLayout exact_layout(int64_t nq, int64_t Hq, int64_t Hkv, int64_t plan_len) {
  ExactLayout e{};
  e.p = make_plan(1, Hq, Hkv, plan_len);
  const size_t rows = static_cast<size_t>(Hkv) * e.p.nchunk * nq * (Hq / Hkv);
  const size_t part = (((rows * 2 + 3) & ~static_cast<size_t>(3)) + rows * kD) * sizeof(float);
  const size_t slots = static_cast<size_t>(nq) * Hkv;
  e.open_off = (part + 255) & ~static_cast<size_t>(255);
  e.sc_off = e.open_off + slots * 4 * kOpenPlane;
  e.bytes = e.sc_off + slots * 2 * sizeof(float);
  return e;
}

}  // namespace

extern "C" size_t kv_nest_attend_workspace_size(int64_t nq, int64_t n_q_heads, int64_t n_kv_heads,
                                                int64_t head_dim, int64_t ctx_len) {
  if (nq < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || head_dim != kD || ctx_len < 1) return 0;
  if (n_q_heads / n_kv_heads > kMaxRowsPerLaunch) return 0;
  // the largest launch: a full chunk of queries at the full length
  return make_plan(chunk_queries(nq, n_q_heads / n_kv_heads), n_q_heads, n_kv_heads, ctx_len).ws;
}

extern "C" size_t kv_nest_attend_exact_workspace_size(int64_t nq, int64_t n_q_heads, int64_t n_kv_heads,
                                                      int64_t head_dim, int64_t ctx_len) {
  if (nq < 1 || nq > kBlk || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads ||
      head_dim != kD || ctx_len < 1)
    return 0;
  if (nq == 1) return make_plan(1, n_q_heads, n_kv_heads, ctx_len).ws;
  return exact_layout(nq, n_q_heads, n_kv_heads, ctx_len).bytes;
}

namespace {

// Host checks shared by both attention entry points; fills the kernel
// arguments except the plan-dependent ones. max_rows bounds nq * (Hq/Hkv):
// 64 for kv_nest_attend (the LDS-table kernel's four row tiles); the exact
// pass attends one query's GQA group per workgroup and has no such bound.
int prepare_attend(const char* what, const uint16_t* q, int64_t nq, int64_t n_q_heads, const nest_kv* kv,
                   const int32_t* ctx_dev, int64_t ctx_len, int view, float* out, int64_t max_rows,
                   AttArgs& a) {
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
  if (ctx_dev ? (ctx_len < 0 || ctx_len > kv->capacity || nq > kv->capacity)
              : (ctx_len < nq || ctx_len > kv->capacity))
    return nest::fail(NEST_EINVAL, "%s: need nq <= ctx_len <= capacity (ctx_len=%lld)", what,
                      (long long)ctx_len);
  const int64_t R = nq * (n_q_heads / Hkv);
  if (R > max_rows)
    return nest::fail(NEST_EUNSUPPORTED, "%s: nq*(Hq/Hkv)=%lld > %lld", what, (long long)R, (long long)max_rows);
  if (kv->capacity > (1LL << 30) || Hkv > 65535)
    return nest::fail(NEST_EUNSUPPORTED, "%s: cache too large", what);
  if (!nest::aligned16(kv->k_base) || !nest::aligned16(kv->v_base) ||
      (view == 1 && (!nest::aligned16(kv->k_refine) || !nest::aligned16(kv->v_refine))))
    return nest::fail(NEST_EALIGN, "%s: planes must be 16-byte aligned", what);
  if (!nest::aligned16(q)) return nest::fail(NEST_EALIGN, "%s: q must be 16-byte aligned", what);
  a = AttArgs{};
  a.q = q; a.nq = (int)nq; a.Hq = (int)n_q_heads; a.grp = (int)(n_q_heads / Hkv); a.R = (int)R;
  a.ctx = (int)ctx_len; a.ctx_dev = ctx_dev;
  a.kb = kv->k_base; a.kr = kv->k_refine; a.vb = kv->v_base; a.vr = kv->v_refine;
  a.ks = kv->k_scale; a.vs = kv->v_scale;
  a.cap = (int)kv->capacity; a.nb = (int)(kv->capacity / kBlk);
  a.out = out;
  return NEST_OK;
}

int attach_workspace(const char* what, AttArgs& a, const Plan& p, int64_t Hkv, void* ws, size_t ws_bytes,
                     size_t need) {
  if (p.nchunk > kMaxChunks) return nest::fail(NEST_EUNSUPPORTED, "%s: too many chunks", what);
  if (!ws || ws_bytes < need) return nest::fail(NEST_EWORKSPACE, "%s: workspace needs %zu bytes", what, need);
  if (!nest::aligned16(ws)) return nest::fail(NEST_EALIGN, "%s: workspace must be 16-byte aligned", what);
  a.bpw = p.bpw; a.nchunk = p.nchunk;
  a.part_ml = static_cast<float*>(ws);
  // part_o starts 16-byte aligned after the (max, sum) pairs
  const size_t ml_floats = (static_cast<size_t>(Hkv) * p.nchunk * a.R * 2 + 3) & ~static_cast<size_t>(3);
  a.part_o = a.part_ml + ml_floats;
  return NEST_OK;
}

}  // namespace

extern "C" int kv_nest_attend(const uint16_t* q, int64_t nq, int64_t n_q_heads, const nest_kv* kv,
                              const int32_t* ctx_dev, int64_t ctx_len, int view, float* out, void* ws,
                              size_t ws_bytes, void* stream) {
  const char* what = "kv_nest_attend";
  AttArgs a;
  if (!kv) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (kv->n_kv_heads >= 1 && n_q_heads / kv->n_kv_heads > kMaxRowsPerLaunch)
    return nest::fail(NEST_EUNSUPPORTED, "%s: Hq/Hkv > %d", what, kMaxRowsPerLaunch);
  int rc = prepare_attend(what, q, nq, n_q_heads, kv, ctx_dev, ctx_len, view, out, 1LL << 40, a);
  if (rc) return rc;
  const int64_t Hkv = kv->n_kv_heads;
  // More query rows than one launch holds: the queries in chunks of
  // kMaxRowsPerLaunch / grp, each launched as the call of its queries alone
  // (its last query's position as the length), which is what each query
  // sees in any case; the chunks share the workspace in turn.
  const int64_t per = chunk_queries(nq, a.grp);
  hipStream_t st = nest::as_stream(stream);
  for (int64_t i0 = 0; i0 < nq; i0 += per) {
    const int64_t n = nq - i0 < per ? nq - i0 : per;
    const int64_t len = ctx_len - (nq - i0 - n);
    AttArgs c = a;
    c.q = q + static_cast<size_t>(i0) * n_q_heads * kD;
    c.out = out + static_cast<size_t>(i0) * n_q_heads * kD;
    c.nq = static_cast<int>(n);
    c.R = static_cast<int>(n * a.grp);
    c.ctx = static_cast<int>(len);
    // with the length on the device, the grid covers the whole capacity and
    // the workgroups past the live length write empty partials
    const Plan p = make_plan(n, n_q_heads, Hkv, ctx_dev ? kv->capacity : len);
    rc = attach_workspace(what, c, p, Hkv, ws, ws_bytes, p.ws);
    if (rc) return rc;
    rc = view == 0 ? launch_att<0>(c, p, (int)Hkv, st) : launch_att<1>(c, p, (int)Hkv, st);
    if (rc) return rc;
  }
  return NEST_OK;
}

namespace {

// Shared checks and arguments of the appends folded into an attention call.
int attach_append(const char* what, AttArgs& a, const nest_kv* kv, float* shadow_k, float* shadow_v,
                  const float* k_new, const float* v_new) {
  if (!shadow_k || !shadow_v || !k_new || !v_new) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (!kv->k_refine || !kv->v_refine)
    return nest::fail(NEST_EINVAL, "%s: the append writes both refinement planes", what);
  if (!nest::aligned16(k_new) || !nest::aligned16(v_new) || !nest::aligned16(shadow_k) ||
      !nest::aligned16(shadow_v) || !nest::aligned16(kv->k_refine) || !nest::aligned16(kv->v_refine))
    return nest::fail(NEST_EALIGN, "%s: new tokens, shadows and planes must be 16-byte aligned", what);
  a.knew = k_new;
  a.vnew = v_new;
  a.w_kb = const_cast<uint8_t*>(kv->k_base); a.w_kr = const_cast<uint8_t*>(kv->k_refine);
  a.w_vb = const_cast<uint8_t*>(kv->v_base); a.w_vr = const_cast<uint8_t*>(kv->v_refine);
  a.w_ks = const_cast<float*>(kv->k_scale); a.w_vs = const_cast<float*>(kv->v_scale);
  a.w_shk = shadow_k;
  a.w_shv = shadow_v;
  return NEST_OK;
}

int check_append_pos(const char* what, const nest_kv* kv, const int32_t* pos_dev, int64_t pos, int64_t n) {
  if (!kv) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  if (n < 1 || n > kBlk || (!pos_dev && (pos < 0 || pos + n > kv->capacity)) ||
      (pos_dev && (pos < -kv->capacity || pos > kv->capacity || pos + n < 0)))
    return nest::fail(NEST_EINVAL, "%s: need pos >= 0, 1 <= n <= block, pos + n <= capacity (pos=%lld n=%lld)",
                      what, (long long)pos, (long long)n);
  return NEST_OK;
}

// kv_nest_attend_exact, and with k_new set kv_nest_append_attend_exact: the
// append of the nq new tokens folded into the open-block kernel.
int attend_exact_impl(const char* what, const uint16_t* q, int64_t nq, int64_t n_q_heads, const nest_kv* kv,
                      float* shadow_k, float* shadow_v, const float* k_new, const float* v_new,
                      const int32_t* ctx_dev, int64_t ctx_len, int view, float* out, void* ws,
                      size_t ws_bytes, void* stream) {
  AttArgs a;
  int rc = prepare_attend(what, q, nq, n_q_heads, kv, ctx_dev, ctx_len, view, out, kBlk * 16, a);
  if (rc) return rc;
  if (!shadow_k || !shadow_v) return nest::fail(NEST_EINVAL, "%s: null shadow", what);
  if (a.grp > 16) return nest::fail(NEST_EUNSUPPORTED, "%s: Hq/Hkv=%d > 16", what, a.grp);
  if (nq > kBlk) return nest::fail(NEST_EUNSUPPORTED, "%s: nq=%lld > block", what, (long long)nq);
  a.shk = shadow_k;
  a.shv = shadow_v;
  const int64_t Hkv = kv->n_kv_heads;
  hipStream_t st = nest::as_stream(stream);
  if (k_new) {
    rc = attach_append(what, a, kv, shadow_k, shadow_v, k_new, v_new);
    if (rc) return rc;
  }
  if (nq == 1) {
    // one query: the append of its token leaves its block quantized over
    // exactly the tokens up to it, so the planes are what it must see (the
    // folded append runs alone first: the append layers of the open-block
    // kernel)
    if (k_new) {
      a.zbase = 1;
      open_block_kernel<<<dim3(kOpenSplit, static_cast<unsigned>(Hkv), 4), 256, 0, st>>>(a);
      rc = nest::check_launch("kv_nest_append_attend_exact(append)");
      if (rc) return rc;
    }
    const Plan p = make_plan(1, n_q_heads, Hkv, ctx_dev ? kv->capacity : ctx_len);
    rc = attach_workspace(what, a, p, Hkv, ws, ws_bytes, p.ws);
    if (rc) return rc;
    return view == 0 ? launch_att<0>(a, p, (int)Hkv, st) : launch_att<1>(a, p, (int)Hkv, st);
  }
  // every query takes the split of a one-query call (its workgroups write
  // rows z * grp .. of the partials); first the open blocks, one slot per
  // (query, kv head)
  const ExactLayout e = exact_layout(nq, n_q_heads, Hkv, ctx_dev ? kv->capacity : ctx_len);
  const Plan& p = e.p;
  rc = attach_workspace(what, a, p, Hkv, ws, ws_bytes, e.bytes);
  if (rc) return rc;
  a.open = static_cast<uint8_t*>(ws) + e.open_off;
  a.open_sc = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + e.sc_off);
  const unsigned layers = static_cast<unsigned>(2 * nq + (k_new ? 4 : 0));
  open_block_kernel<<<dim3(kOpenSplit, static_cast<unsigned>(Hkv), layers), 256, 0, st>>>(a);
  rc = nest::check_launch("kv_nest_attend_exact(open blocks)");
  if (rc) return rc;
  // as many queries per workgroup as their GQA groups fit in 16 rows
  a.qpack = static_cast<int>(16 / a.grp < nq ? 16 / a.grp : nq);
  if (a.qpack < 1) a.qpack = 1;
  const int64_t items = static_cast<int64_t>(p.nchunk) * Hkv * ((nq + a.qpack - 1) / a.qpack);
  const dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
  if (view == 0)
    attend_wave_kernel<0, true><<<grid, 256, 0, st>>>(a);
  else
    attend_wave_kernel<1, true><<<grid, 256, 0, st>>>(a);
  rc = nest::check_launch(what);
  if (rc) return rc;
  combine_kernel<<<dim3(a.R, Hkv), 1024, 0, st>>>(a);
  return nest::check_launch("kv_nest_attend_exact(combine)");
}

}  // namespace

extern "C" int kv_nest_attend_exact(const uint16_t* q, int64_t nq, int64_t n_q_heads, const nest_kv* kv,
                                    const float* shadow_k, const float* shadow_v, const int32_t* ctx_dev,
                                    int64_t ctx_len, int view, float* out, void* ws, size_t ws_bytes,
                                    void* stream) {
  return attend_exact_impl("kv_nest_attend_exact", q, nq, n_q_heads, kv, const_cast<float*>(shadow_k),
                           const_cast<float*>(shadow_v), nullptr, nullptr, ctx_dev, ctx_len, view, out, ws,
                           ws_bytes, stream);
}

extern "C" int kv_nest_append_attend_exact(const uint16_t* q, int64_t n, int64_t n_q_heads, const nest_kv* kv,
                                           float* shadow_k, float* shadow_v, const float* k_new,
                                           const float* v_new, const int32_t* pos_dev, int64_t pos, int view,
                                           float* out, void* ws, size_t ws_bytes, void* stream) {
  const char* what = "kv_nest_append_attend_exact";
  if (!k_new || !v_new) return nest::fail(NEST_EINVAL, "%s: null new tokens", what);
  const int rc = check_append_pos(what, kv, pos_dev, pos, n);
  if (rc) return rc;
  return attend_exact_impl(what, q, n, n_q_heads, kv, shadow_k, shadow_v, k_new, v_new, pos_dev, pos + n, view,
                           out, ws, ws_bytes, stream);
}

// Speculative sampling ("How Speculative Decoding Speeds Up Inference",
// section "The same output as the large model alone", and the method of
// Leviathan et al. and Chen et al. that it names): a draft token d is kept
// with probability min(1, p(d) / q(d)); at the first rejection the last
// token is drawn from max(0, p - q) normalized; when every draft is kept, a
// bonus token is drawn from the target's last position. Scores are
// softmax(logits / T). Draws are by inverse CDF with uniforms the caller
// passes in: the smallest id whose running weight exceeds u times the total.
//
// The logits stay in HBM in fp32 and are read in chunks of kChunk ids:
//   chunk_stats_kernel  per (row, chunk): max and sum of exp((y - max) / T);
//   sample_pick_kernel  per row: chunk weights from the statistics, a block
//                       scan that finds the chunk, then a scan of the chunk's
//                       ids that finds the token;
//   verify_decide_kernel per (sequence, chunk): every block redoes the accept
//                       test of the sequence from the row statistics (the
//                       same arithmetic, so every block reaches the same
//                       result) and sums its chunk of the final distribution;
//   verify_pick_kernel  per sequence: finds the token as above and writes the
//                       round's output.
// Arithmetic is fp32 with exp2 of (y - max) * log2(e) / T.
#include <climits>

#include "common.h"

namespace {

constexpr int kChunk = 2048;       // logits per chunk
constexpr int kStatThreads = 256;  // 8 logits of a chunk per thread
constexpr int kPer = kChunk / kStatThreads;
constexpr int kPickThreads = 1024;
constexpr int kPickWaves = kPickThreads / 64;
constexpr int kMaxChunks = 4096;  // 4 chunk weights per pick thread: V <= 8M
constexpr int kChunkPer = kMaxChunks / kPickThreads;
constexpr int kElemPer = kChunk / kPickThreads;
constexpr int kMaxK = 32;

int nchunks(int64_t V) { return static_cast<int>((V + kChunk - 1) / kChunk); }

// Weight of one logit relative to the row's max: exp((y - m) / T).
__device__ __forceinline__ float weight(float y, float m, float c) {
  return y == -INFINITY ? 0.0f : exp2f((y - m) * c);
}

template <int NW>
__device__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, sh[w]);
  __syncthreads();
  return r;
}

template <int NW>
__device__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += sh[w];
  __syncthreads();
  return r;
}

// Exclusive prefix of x over the block's threads in thread order, and the
// total (the same value in every thread).
template <int NW>
__device__ float block_excl_scan(float x, float& total, float* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  float off = 0.0f, tot = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float t = sh[w];
    if (w < wave) off += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + inc - x;
}

// Thread t holds items [t * PER, t * PER + PER) with weights v and the
// running weight excl before them. Returns the first item of positive
// weight whose running weight exceeds target; if none does (rounding), the
// last item of positive weight; -1 if no item has weight. *at gets the
// running weight before it. Only items of positive weight are returned, so
// padding items (weight 0) past the end never are.
template <int PER>
__device__ int block_find(const float (&v)[PER], float excl, float target, float* at, int* sh_i,
                          float* sh_f) {
  if (threadIdx.x == 0) {
    sh_i[0] = INT_MAX;
    sh_i[1] = -1;
  }
  __syncthreads();
  int cand = INT_MAX, last = -1;
  float cand_at = 0.0f, last_at = 0.0f, run = excl;
  const int first = threadIdx.x * PER;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (cand == INT_MAX && v[j] > 0.0f && run + v[j] > target) {
      cand = first + j;
      cand_at = run;
    }
    if (v[j] > 0.0f) {
      last = first + j;
      last_at = run;
    }
    run += v[j];
  }
  if (cand != INT_MAX) atomicMin(&sh_i[0], cand);
  if (last >= 0) atomicMax(&sh_i[1], last);
  __syncthreads();
  const bool hit = sh_i[0] != INT_MAX;
  const int idx = hit ? sh_i[0] : sh_i[1];
  if (hit ? cand == idx : (last == idx && idx >= 0)) sh_f[0] = hit ? cand_at : last_at;
  __syncthreads();
  *at = idx >= 0 ? sh_f[0] : 0.0f;
  __syncthreads();
  return idx;
}

// ---------------------------------------------------------------------------
// chunk statistics
// ---------------------------------------------------------------------------

struct StatArgs {
  const float* y0;  // rows [0, rows0)
  const float* y1;  // rows [rows0, rows)
  int rows0;
  int V, nchunk;
  float c;  // log2(e) / T
  float2* stats;  // [rows][nchunk]: (max, sum of exp((y - max) / T))
};

__global__ void __launch_bounds__(kStatThreads) chunk_stats_kernel(StatArgs a) {
  __shared__ float sh[kStatThreads / 64];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const float* y = row < a.rows0 ? a.y0 + static_cast<size_t>(row) * a.V
                                 : a.y1 + static_cast<size_t>(row - a.rows0) * a.V;
  const int base = chunk * kChunk + threadIdx.x;
  float v[kPer];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = base + j * kStatThreads;
    v[j] = i < a.V ? y[i] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  m = block_max<kStatThreads / 64>(m, sh);
  float s = 0.0f;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) s += weight(v[j], m, a.c);
  }
  s = block_sum<kStatThreads / 64>(s, sh);
  if (threadIdx.x == 0) a.stats[static_cast<size_t>(row) * a.nchunk + chunk] = make_float2(m, s);
}

// Row max and normalizer from a row's chunk statistics, by one wave (every
// lane ends with them).
__device__ void row_total(const float2* st, int nchunk, float c, float& M, float& Z) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
  for (int i = lane; i < nchunk; i += 64) m = fmaxf(m, st[i].x);
  m = wave_max(m);
  float z = 0.0f;
  for (int i = lane; i < nchunk; i += 64) {
    const float2 s = st[i];
    z += s.x == -INFINITY ? 0.0f : s.y * exp2f((s.x - m) * c);
  }
  M = m;
  Z = wave_sum(z);
}

// ---------------------------------------------------------------------------
// plain draws
// ---------------------------------------------------------------------------

struct SampleArgs {
  const float* y;
  const float2* stats;
  const float* u;
  int32_t* tokens;
  int V, nchunk;
  float c;
};

// Shared tail of both pick kernels: with chunk weights cw (thread t holds
// chunks [kChunkPer t, kChunkPer t + kChunkPer)) and the per-id weight
// function wfn, draw with the uniform u. Returns the id (-1 if no weight).
template <typename WFn>
__device__ int pick(const float (&cw)[kChunkPer], float u, int V, WFn wfn, float* shf, int* shi) {
  float local = 0.0f;
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j) local += cw[j];
  float total;
  const float excl = block_excl_scan<kPickWaves>(local, total, shf);
  float at;
  const int chunk = block_find<kChunkPer>(cw, excl, u * total, &at, shi, shf + kPickWaves);
  if (chunk < 0) return -1;
  const float rest = u * total - at;
  float w[kElemPer];
  const int id0 = chunk * kChunk + threadIdx.x * kElemPer;
  float lw = 0.0f;
#pragma unroll
  for (int j = 0; j < kElemPer; ++j) {
    w[j] = id0 + j < V ? wfn(id0 + j) : 0.0f;
    lw += w[j];
  }
  float ctot;
  const float cex = block_excl_scan<kPickWaves>(lw, ctot, shf);
  const int e = block_find<kElemPer>(w, cex, rest, &at, shi, shf + kPickWaves);
  return e < 0 ? -1 : chunk * kChunk + e;
}

__global__ void __launch_bounds__(kPickThreads) sample_pick_kernel(SampleArgs a) {
  __shared__ float shf[kPickWaves + 1];
  __shared__ int shi[2];
  const int row = blockIdx.x;
  const float2* st = a.stats + static_cast<size_t>(row) * a.nchunk;
  float2 s[kChunkPer];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j) {
    const int i = threadIdx.x * kChunkPer + j;
    s[j] = i < a.nchunk ? st[i] : make_float2(-INFINITY, 0.0f);
    m = fmaxf(m, s[j].x);
  }
  const float M = block_max<kPickWaves>(m, shf);
  float cw[kChunkPer];
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j) cw[j] = s[j].x == -INFINITY ? 0.0f : s[j].y * exp2f((s[j].x - M) * a.c);
  const float* y = a.y + static_cast<size_t>(row) * a.V;
  const float c = a.c;
  const int t = pick(cw, a.u[row], a.V, [&](int i) { return weight(y[i], M, c); }, shf, shi);
  if (threadIdx.x == 0) a.tokens[row] = t;
}

// ---------------------------------------------------------------------------
// the round's accept test and last draw
// ---------------------------------------------------------------------------

// What every decide block of a sequence concludes; written by its chunk-0
// block for the pick kernel.
struct Decision {
  int a;        // drafts kept
  int residual; // 1: last token from max(0, p - q); 0: from p
  float Mt, iZt, Md, iZd;  // max and 1/normalizer of the final rows
};

struct VerifyArgs {
  const float* yt;  // [B][k+1][V]
  const float* yd;  // [B][k][V]
  const int32_t* draft;  // [B][k]
  const float* u_acc;    // [B][k]
  const float* u_fin;    // [B]
  int B, k, V, nchunk;
  float c;
  const float2* stats;  // yt rows then yd rows, [row][nchunk]
  float* fsum;          // [B][nchunk]: chunk sums of the final weights
  Decision* dec;        // [B]
  int32_t* n_emitted;   // [B]
  int32_t* emitted;     // [B][k+1]
};

__device__ __forceinline__ float final_weight(const Decision& d, float yt, float yd, float c) {
  const float p = weight(yt, d.Mt, c) * d.iZt;
  return d.residual ? fmaxf(0.0f, p - weight(yd, d.Md, c) * d.iZd) : p;
}

__global__ void __launch_bounds__(kStatThreads) verify_decide_kernel(VerifyArgs a) {
  __shared__ float rowM[2 * kMaxK + 1], rowZ[2 * kMaxK + 1];
  __shared__ float sh[kStatThreads / 64];
  __shared__ Decision dsh;
  const int chunk = blockIdx.x, b = blockIdx.y, k = a.k, k1 = k + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // rows 0..k: target rows of b; rows k+1..2k: draft rows of b
  for (int r = wave; r < 2 * k + 1; r += kStatThreads / 64) {
    const size_t srow = r < k1 ? static_cast<size_t>(b) * k1 + r
                               : static_cast<size_t>(a.B) * k1 + static_cast<size_t>(b) * k + (r - k1);
    float M, Z;
    row_total(a.stats + srow * a.nchunk, a.nchunk, a.c, M, Z);
    if (lane == 0) {
      rowM[r] = M;
      rowZ[r] = Z;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // slot i (lane i) keeps its draft d when u * q(d) < p(d); an id outside
    // [0, V) is never kept
    bool keep = false;
    if (lane < k) {
      const int d = a.draft[b * k + lane];
      if (d >= 0 && d < a.V) {
        const float yt = a.yt[(static_cast<size_t>(b) * k1 + lane) * a.V + d];
        const float yd = a.yd[(static_cast<size_t>(b) * k + lane) * a.V + d];
        const float p = weight(yt, rowM[lane], a.c) / rowZ[lane];
        const float q = weight(yd, rowM[k1 + lane], a.c) / rowZ[k1 + lane];
        keep = a.u_acc[b * k + lane] * q < p;
      }
    }
    const unsigned long long rej = __ballot(lane < k && !keep);
    if (lane == 0) {
      Decision d;
      d.a = rej ? __ffsll(static_cast<long long>(rej)) - 1 : k;
      d.residual = d.a < k;
      d.Mt = rowM[d.a];
      d.iZt = 1.0f / rowZ[d.a];
      d.Md = d.residual ? rowM[k1 + d.a] : 0.0f;
      d.iZd = d.residual ? 1.0f / rowZ[k1 + d.a] : 0.0f;
      dsh = d;
      if (chunk == 0) a.dec[b] = d;
    }
  }
  __syncthreads();
  const Decision d = dsh;
  const float* yt = a.yt + (static_cast<size_t>(b) * k1 + d.a) * a.V;
  const float* yd = d.residual ? a.yd + (static_cast<size_t>(b) * k + d.a) * a.V : yt;
  float s = 0.0f;
  const int base = chunk * kChunk + threadIdx.x;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = base + j * kStatThreads;
    if (i < a.V) s += final_weight(d, yt[i], yd[i], a.c);
  }
  s = block_sum<kStatThreads / 64>(s, sh);
  if (threadIdx.x == 0) a.fsum[static_cast<size_t>(b) * a.nchunk + chunk] = s;
}

__global__ void __launch_bounds__(kPickThreads) verify_pick_kernel(VerifyArgs a) {
  __shared__ float shf[kPickWaves + 1];
  __shared__ int shi[2];
  const int b = blockIdx.x, k = a.k, k1 = k + 1;
  Decision d = a.dec[b];
  const float* fs = a.fsum + static_cast<size_t>(b) * a.nchunk;
  float cw[kChunkPer];
  float local = 0.0f;
#pragma unroll
  for (int j = 0; j < kChunkPer; ++j) {
    const int i = threadIdx.x * kChunkPer + j;
    cw[j] = i < a.nchunk ? fs[i] : 0.0f;
    local += cw[j];
  }
  if (d.residual && block_sum<kPickWaves>(local, shf) == 0.0f) {
    // the corrected weights rounded away entirely: draw from p itself
    d.residual = 0;
    const float2* st = a.stats + (static_cast<size_t>(b) * k1 + d.a) * a.nchunk;
#pragma unroll
    for (int j = 0; j < kChunkPer; ++j) {
      const int i = threadIdx.x * kChunkPer + j;
      const float2 s = i < a.nchunk ? st[i] : make_float2(-INFINITY, 0.0f);
      cw[j] = s.x == -INFINITY ? 0.0f : s.y * exp2f((s.x - d.Mt) * a.c) * d.iZt;
    }
  }
  const float* yt = a.yt + (static_cast<size_t>(b) * k1 + d.a) * a.V;
  const float* yd = d.residual ? a.yd + (static_cast<size_t>(b) * k + d.a) * a.V : yt;
  const float c = a.c;
  const int t = pick(cw, a.u_fin[b], a.V, [&](int i) { return final_weight(d, yt[i], yd[i], c); }, shf, shi);
  for (int j = threadIdx.x; j < k1; j += kPickThreads)
    a.emitted[static_cast<size_t>(b) * k1 + j] = j < d.a ? a.draft[b * k + j] : (j == d.a ? t : -1);
  if (threadIdx.x == 0) a.n_emitted[b] = d.a + 1;
}

size_t align16(size_t n) { return (n + 15) & ~static_cast<size_t>(15); }

int check_sampling(const char* what, int64_t rows, int64_t V, float T) {
  if (rows < 1 || V < 1) return nest::fail(NEST_EINVAL, "%s: empty shape", what);
  if (V > static_cast<int64_t>(kMaxChunks) * kChunk)
    return nest::fail(NEST_EUNSUPPORTED, "%s: V=%lld > %d", what, (long long)V, kMaxChunks * kChunk);
  if (rows > 65535) return nest::fail(NEST_EUNSUPPORTED, "%s: %lld rows > 65535", what, (long long)rows);
  if (!(T > 0.0f) || !(T < INFINITY)) return nest::fail(NEST_EINVAL, "%s: temperature must be > 0", what);
  const float c = 1.44269504088896340736f / T;
  if (!(c < INFINITY)) return nest::fail(NEST_EINVAL, "%s: temperature too small", what);
  return NEST_OK;
}

}  // namespace

extern "C" size_t nest_sample_workspace_size(int64_t M, int64_t V) {
  if (M < 1 || V < 1 || V > static_cast<int64_t>(kMaxChunks) * kChunk) return 0;
  return align16(static_cast<size_t>(M) * nchunks(V) * sizeof(float2));
}

extern "C" size_t verify_sample_workspace_size(int64_t B, int64_t k, int64_t V) {
  if (B < 1 || k < 0 || V < 1 || V > static_cast<int64_t>(kMaxChunks) * kChunk) return 0;
  const size_t nc = nchunks(V);
  return align16(static_cast<size_t>(B) * (2 * k + 1) * nc * sizeof(float2)) +
         align16(static_cast<size_t>(B) * nc * sizeof(float)) + align16(static_cast<size_t>(B) * sizeof(Decision));
}

extern "C" int nest_sample(const float* y, int64_t M, int64_t V, float temperature, const float* u,
                           int32_t* tokens, void* ws, size_t ws_bytes, void* stream) {
  const char* what = "nest_sample";
  int rc = check_sampling(what, M, V, temperature);
  if (rc) return rc;
  if (!y || !u || !tokens) return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  const size_t need = nest_sample_workspace_size(M, V);
  if (!ws || ws_bytes < need) return nest::fail(NEST_EWORKSPACE, "%s: workspace needs %zu bytes", what, need);
  if (!nest::aligned16(ws)) return nest::fail(NEST_EALIGN, "%s: workspace must be 16-byte aligned", what);
  hipStream_t st = nest::as_stream(stream);
  const int nc = nchunks(V);
  const float c = 1.44269504088896340736f / temperature;
  StatArgs sa{y, nullptr, static_cast<int>(M), static_cast<int>(V), nc, c, static_cast<float2*>(ws)};
  chunk_stats_kernel<<<dim3(nc, static_cast<unsigned>(M)), kStatThreads, 0, st>>>(sa);
  rc = nest::check_launch(what);
  if (rc) return rc;
  SampleArgs pa{y, static_cast<const float2*>(ws), u, tokens, static_cast<int>(V), nc, c};
  sample_pick_kernel<<<static_cast<unsigned>(M), kPickThreads, 0, st>>>(pa);
  return nest::check_launch(what);
}

extern "C" int verify_sample(const float* yt, const float* yd, int64_t B, int64_t k, int64_t V,
                             float temperature, const int32_t* draft, const float* u_acc,
                             const float* u_fin, int32_t* n_emitted, int32_t* emitted, void* ws,
                             size_t ws_bytes, void* stream) {
  const char* what = "verify_sample";
  if (B < 1 || k < 0) return nest::fail(NEST_EINVAL, "%s: B=%lld k=%lld", what, (long long)B, (long long)k);
  if (k > kMaxK) return nest::fail(NEST_EUNSUPPORTED, "%s: k=%lld > %d", what, (long long)k, kMaxK);
  int rc = check_sampling(what, B * (2 * k + 1), V, temperature);
  if (rc) return rc;
  if (!yt || !u_fin || !n_emitted || !emitted || (k > 0 && (!yd || !draft || !u_acc)))
    return nest::fail(NEST_EINVAL, "%s: null pointer", what);
  const size_t need = verify_sample_workspace_size(B, k, V);
  if (!ws || ws_bytes < need) return nest::fail(NEST_EWORKSPACE, "%s: workspace needs %zu bytes", what, need);
  if (!nest::aligned16(ws)) return nest::fail(NEST_EALIGN, "%s: workspace must be 16-byte aligned", what);
  hipStream_t st = nest::as_stream(stream);
  const int nc = nchunks(V);
  const float c = 1.44269504088896340736f / temperature;
  char* p = static_cast<char*>(ws);
  float2* stats = reinterpret_cast<float2*>(p);
  p += align16(static_cast<size_t>(B) * (2 * k + 1) * nc * sizeof(float2));
  float* fsum = reinterpret_cast<float*>(p);
  p += align16(static_cast<size_t>(B) * nc * sizeof(float));
  Decision* dec = reinterpret_cast<Decision*>(p);

  StatArgs sa{yt, yd, static_cast<int>(B * (k + 1)), static_cast<int>(V), nc, c, stats};
  chunk_stats_kernel<<<dim3(nc, static_cast<unsigned>(B * (2 * k + 1))), kStatThreads, 0, st>>>(sa);
  rc = nest::check_launch(what);
  if (rc) return rc;
  VerifyArgs va{yt, yd, draft, u_acc, u_fin, static_cast<int>(B), static_cast<int>(k), static_cast<int>(V),
                nc, c, stats, fsum, dec, n_emitted, emitted};
  verify_decide_kernel<<<dim3(nc, static_cast<unsigned>(B)), kStatThreads, 0, st>>>(va);
  rc = nest::check_launch(what);
  if (rc) return rc;
  verify_pick_kernel<<<static_cast<unsigned>(B), kPickThreads, 0, st>>>(va);
  return nest::check_launch(what);
}

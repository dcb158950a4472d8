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
constexpr int kIdPer = kChunk / 64;  // ids per lane when one wave scans a chunk
constexpr int kMaxChunks = 4096;     // V <= 8M
constexpr int kMaxK = 32;
constexpr int kRegChunks = 4;  // chunk values a lane holds in registers (nchunk <= 256)

int nchunks(int64_t V) { return static_cast<int>((V + kChunk - 1) / kChunk); }

// Weight of one logit relative to the row's max m (finite): exp((y - m) / T);
// a masked logit (-inf) weighs 0.
__device__ __forceinline__ float weight(float y, float m, float c) { return exp2f((y - m) * c); }

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

// Exclusive prefix of x over the wave's lanes in lane order; *total gets
// the sum over all lanes (the same in every lane).
__device__ float wave_excl_scan(float x, float* total) {
  const int lane = threadIdx.x & 63;
  float inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  *total = __shfl(inc, 63, 64);
  return inc - x;
}

// Lanes hold consecutive groups of items with group weight ls and running
// weight ex before the group. The lane whose group holds the first running
// weight above target; if none does (rounding), the last lane with weight;
// -1 if no lane has any.
__device__ int wave_find_lane(float ls, float ex, float target) {
  const unsigned long long hit = __ballot(ls > 0.0f && ex + ls > target);
  if (hit) return __ffsll(static_cast<long long>(hit)) - 1;
  const unsigned long long pos = __ballot(ls > 0.0f);
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : -1;
}

// LDS index of item i when lanes read runs of `run` consecutive items: one
// pad word after every run keeps a wave's lane-strided reads on distinct
// banks.
__device__ __forceinline__ int padded(int i, int run) { return i + i / run; }

// The first item of positive weight, among one lane's run of n items
// w(j) after running weight run0, whose running weight exceeds target; if
// none, the last item of positive weight. *at gets the running weight
// before it.
template <typename W>
__device__ int lane_find(int n, float run0, float target, W w, float* at) {
  int cand = -1, last = -1;
  float cand_at = 0.0f, last_at = 0.0f, run = run0;
  for (int j = 0; j < n; ++j) {
    const float x = w(j);
    if (cand < 0 && x > 0.0f && run + x > target) {
      cand = j;
      cand_at = run;
    }
    if (x > 0.0f) {
      last = j;
      last_at = run;
    }
    run += x;
  }
  *at = cand >= 0 ? cand_at : last_at;
  return cand >= 0 ? cand : last;
}

// One wave draws an id. cw_sh holds the nchunk chunk weights (chunk i at
// padded(i, cpl), zeros up to 64 * cpl); wfn(id) is the weight of one id
// (a chunk's weight is the sum of its ids', up to rounding); id_sh is
// scratch for one chunk. The draw takes the first id of positive weight
// whose running weight exceeds u times the total; where rounding leaves
// none inside the chosen lane or chunk, the last id of positive weight
// there. Returns -1 if nothing has weight.
template <typename WFn>
__device__ int wave_pick(const float* cw_sh, int nchunk, int V, float u, WFn wfn, float* id_sh) {
  const int lane = threadIdx.x & 63;
  const int cpl = (nchunk + 63) >> 6;  // lane l holds chunks [l * cpl, l * cpl + cpl)
  const float* mine = cw_sh + padded(lane * cpl, cpl);
  float ls = 0.0f;
  for (int j = 0; j < cpl; ++j) ls += mine[j];
  float total;
  const float ex = wave_excl_scan(ls, &total);
  const float target = u * total;
  const int L = wave_find_lane(ls, ex, target);
  if (L < 0) return -1;
  float at;
  const int j0 = lane_find(cpl, ex, target, [&](int j) { return mine[j]; }, &at);
  const int chunk = __shfl(lane * cpl + j0, L, 64);
  const float rest = target - __shfl(at, L, 64);
  // the chunk's id weights: coalesced loads, stored so that lane l then
  // reads ids [l * kIdPer, l * kIdPer + kIdPer) of the chunk
  const int base = chunk * kChunk;
  float v[kIdPer];
#pragma unroll
  for (int j = 0; j < kIdPer; ++j) {
    // clamped id: every load is issued without a branch, so all of them
    // are in flight together
    const int i = base + j * 64 + lane;
    const float x = wfn(min(i, V - 1));
    v[j] = i < V ? x : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kIdPer; ++j) id_sh[padded(j * 64 + lane, kIdPer)] = v[j];
  __syncthreads();
  const float* ids = id_sh + padded(lane * kIdPer, kIdPer);
  float w[kIdPer];
  float le = 0.0f;
#pragma unroll
  for (int j = 0; j < kIdPer; ++j) {
    w[j] = ids[j];
    le += w[j];
  }
  float ctot;
  const float cex = wave_excl_scan(le, &ctot);
  const int L2 = wave_find_lane(le, cex, rest);
  if (L2 < 0) return -1;
  const int e = lane_find(kIdPer, cex, rest, [&](int j) { return w[j]; }, &at);
  return base + __shfl(lane * kIdPer + e, L2, 64);
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
  for (int j = 0; j < kPer; ++j) v[j] = y[min(base + j * kStatThreads, a.V - 1)];  // branch-free loads
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (base + j * kStatThreads >= a.V) v[j] = -INFINITY;
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
// lane ends with both). The first 256 chunks are loaded together, without
// branches; later ones (V > 524288) in a loop.
__device__ void row_total(const float2* st, int nchunk, float c, float& M, float& Z) {
  const int lane = threadIdx.x & 63;
  float2 x[kRegChunks];
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) x[q] = st[min(lane + 64 * q, nchunk - 1)];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) {
    if (lane + 64 * q >= nchunk) x[q] = make_float2(-INFINITY, 0.0f);
    m = fmaxf(m, x[q].x);
  }
  for (int i = lane + 64 * kRegChunks; i < nchunk; i += 64) m = fmaxf(m, st[i].x);
  M = wave_max(m);
  float z = 0.0f;
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) z += x[q].x == -INFINITY ? 0.0f : x[q].y * exp2f((x[q].x - M) * c);
  for (int i = lane + 64 * kRegChunks; i < nchunk; i += 64) {
    const float2 xi = st[i];
    z += xi.x == -INFINITY ? 0.0f : xi.y * exp2f((xi.x - M) * c);
  }
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

// LDS of a pick: chunk weights (padded) and one chunk's id weights.
constexpr int kCwWords = kMaxChunks + 64;
constexpr int kIdWords = kChunk + kChunk / kIdPer;

// Store chunk weights for lane-run reading: cw_sh[padded(i, cpl)] = the
// weight of chunk i, zeros up to 64 * cpl. Chunk lane + 64 q (q < kRegChunks)
// comes from reg[q]; chunks from 256 on (V > 524288) from far(i).
template <typename Far>
__device__ void stage_chunks(float* cw_sh, int nchunk, const float (&reg)[kRegChunks], Far far) {
  const int cpl = (nchunk + 63) >> 6, lane = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) {
    const int i = lane + 64 * q;
    if (i < 64 * cpl) cw_sh[padded(i, cpl)] = i < nchunk ? reg[q] : 0.0f;
  }
  for (int i = lane + 64 * kRegChunks; i < 64 * cpl; i += 64) cw_sh[padded(i, cpl)] = i < nchunk ? far(i) : 0.0f;
  __syncthreads();
}

// One wave per row: row max and chunk weights from the chunk statistics
// (loaded once, coalesced), then the draw.
__global__ void __launch_bounds__(64) sample_pick_kernel(SampleArgs a) {
  __shared__ float cw_sh[kCwWords], id_sh[kIdWords];
  const int row = blockIdx.x, lane = threadIdx.x, nc = a.nchunk;
  const float2* st = a.stats + static_cast<size_t>(row) * nc;
  const float u = a.u[row];
  float2 sv[kRegChunks];
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) sv[q] = st[min(lane + 64 * q, nc - 1)];
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) {
    if (lane + 64 * q >= nc) sv[q] = make_float2(-INFINITY, 0.0f);
    m = fmaxf(m, sv[q].x);
  }
  for (int i = lane + 64 * kRegChunks; i < nc; i += 64) m = fmaxf(m, st[i].x);
  const float M = wave_max(m), c = a.c;
  auto cwf = [&](float2 x) { return x.x == -INFINITY ? 0.0f : x.y * exp2f((x.x - M) * c); };
  float cw[kRegChunks];
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) cw[q] = cwf(sv[q]);
  stage_chunks(cw_sh, nc, cw, [&](int i) { return cwf(st[i]); });
  const float* y = a.y + static_cast<size_t>(row) * a.V;
  const int t = wave_pick(cw_sh, nc, a.V, u, [&](int i) { return weight(y[i], M, c); }, id_sh);
  if (lane == 0) a.tokens[row] = t;
}

// ---------------------------------------------------------------------------
// the round's accept test and last draw
// ---------------------------------------------------------------------------

// What every decide block of a sequence concludes; written by its chunk-0
// block for the pick kernel.
struct Decision {
  int a;        // drafts kept
  int residual; // 1: last token from max(0, p - q); 0: from p
  float Mt, iZt, Md, iZd;  // max and 1/normalizer of the final rows; a draw
                           // from p has Md = Mt, iZd = 0 and reads the
                           // target row in place of the draft row
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

// max(0, p - q) of one id, or p when iZd = 0 (no branch: the loads of yt
// and yd stay unconditional, so the compiler issues a chunk's loads
// together).
__device__ __forceinline__ float final_weight(const Decision& d, float yt, float yd, float c) {
  return fmaxf(0.0f, weight(yt, d.Mt, c) * d.iZt - weight(yd, d.Md, c) * d.iZd);
}

constexpr int kDecideThreads = 1024;  // one wave per row of a sequence; 2 ids of the chunk per thread
constexpr int kDecideWaves = kDecideThreads / 64;
constexpr int kPrefetchRows = kDecideWaves - 1;  // 2k+1 rows when k <= 7

// PREFETCH (2k+1 <= 15): every row's two ids of this chunk are loaded with
// the statistics, before the decision says which rows the last draw uses.
template <bool PREFETCH>
__global__ void __launch_bounds__(kDecideThreads) verify_decide_kernel(VerifyArgs a) {
  __shared__ float rowM[2 * kMaxK + 1], rowZ[2 * kMaxK + 1];
  __shared__ float sh[kDecideWaves];
  __shared__ Decision dsh;
  const int chunk = blockIdx.x, b = blockIdx.y, k = a.k, k1 = k + 1, rows = 2 * k + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the accept test's inputs first (they do not depend on the statistics):
  // lane i of wave 0 takes slot i's draft id and both models' logits there
  bool live = false;
  float yt_d = 0.0f, yd_d = 0.0f, u = 0.0f;
  if (wave == 0 && lane < k) {
    const int d = a.draft[b * k + lane];
    live = d >= 0 && d < a.V;
    if (live) {
      yt_d = a.yt[(static_cast<size_t>(b) * k1 + lane) * a.V + d];
      yd_d = a.yd[(static_cast<size_t>(b) * k + lane) * a.V + d];
    }
    u = a.u_acc[b * k + lane];
  }
  // rows 0..k: target rows of b; rows k+1..2k: draft rows of b
  auto row_ptr = [&](int r) {
    return r < k1 ? a.yt + (static_cast<size_t>(b) * k1 + r) * a.V
                  : a.yd + (static_cast<size_t>(b) * k + (r - k1)) * a.V;
  };
  const int id0 = chunk * kChunk + threadIdx.x, id1 = id0 + kDecideThreads;
  float pre[PREFETCH ? kPrefetchRows : 1][2];
  if (PREFETCH) {
#pragma unroll
    for (int r = 0; r < kPrefetchRows; ++r) {
      if (r < rows) {
        const float* y = row_ptr(r);
        pre[r][0] = y[min(id0, a.V - 1)];  // clamped: no branch between the loads
        pre[r][1] = y[min(id1, a.V - 1)];
      }
    }
  }
  for (int r = wave; r < rows; r += kDecideWaves) {
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
    if (live) {
      const float p = weight(yt_d, rowM[lane], a.c) / rowZ[lane];
      const float q = weight(yd_d, rowM[k1 + lane], a.c) / rowZ[k1 + lane];
      keep = u * q < p;
    }
    const unsigned long long rej = __ballot(lane < k && !keep);
    if (lane == 0) {
      Decision d;
      d.a = rej ? __ffsll(static_cast<long long>(rej)) - 1 : k;
      d.residual = d.a < k;
      d.Mt = rowM[d.a];
      d.iZt = 1.0f / rowZ[d.a];
      d.Md = d.residual ? rowM[k1 + d.a] : d.Mt;
      d.iZd = d.residual ? 1.0f / rowZ[k1 + d.a] : 0.0f;
      dsh = d;
      if (chunk == 0) a.dec[b] = d;
    }
  }
  __syncthreads();
  const Decision d = dsh;
  float t0 = 0.0f, t1 = 0.0f, d0 = 0.0f, d1 = 0.0f;
  if (PREFETCH) {
    // pick the final rows out of the prefetched ones (static indices only)
#pragma unroll
    for (int r = 0; r < kPrefetchRows; ++r) {
      if (r == d.a) {
        t0 = pre[r][0];
        t1 = pre[r][1];
      }
      if (d.residual && r == k1 + d.a) {
        d0 = pre[r][0];
        d1 = pre[r][1];
      }
    }
    if (!d.residual) {
      d0 = t0;
      d1 = t1;
    }
  } else {
    const float* yt = row_ptr(d.a);
    const float* yd = d.residual ? row_ptr(k1 + d.a) : yt;
    t0 = yt[min(id0, a.V - 1)];
    t1 = yt[min(id1, a.V - 1)];
    d0 = yd[min(id0, a.V - 1)];
    d1 = yd[min(id1, a.V - 1)];
  }
  float s = 0.0f;
  if (id0 < a.V) s += final_weight(d, t0, d0, a.c);
  if (id1 < a.V) s += final_weight(d, t1, d1, a.c);
  s = block_sum<kDecideWaves>(s, sh);
  if (threadIdx.x == 0) a.fsum[static_cast<size_t>(b) * a.nchunk + chunk] = s;
}

// One wave per sequence: the draw from the decided distribution, then the
// round's output. The chunk sums of the final weights come from the decide
// kernel (residual or bonus alike); only when the residual's sums are all
// zero are p's chunk weights rebuilt from the statistics.
__global__ void __launch_bounds__(64) verify_pick_kernel(VerifyArgs a) {
  __shared__ float cw_sh[kCwWords], id_sh[kIdWords];
  const int b = blockIdx.x, k = a.k, k1 = k + 1, lane = threadIdx.x, nc = a.nchunk;
  const float* fs = a.fsum + static_cast<size_t>(b) * nc;
  Decision d = a.dec[b];
  const float u = a.u_fin[b];
  float fv[kRegChunks];
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) fv[q] = fs[min(lane + 64 * q, nc - 1)];
#pragma unroll
  for (int q = 0; q < kRegChunks; ++q) {
    if (lane + 64 * q >= nc) fv[q] = 0.0f;
    s += fv[q];
  }
  for (int i = lane + 64 * kRegChunks; i < nc; i += 64) s += fs[i];
  const float c = a.c;
  if (d.residual && wave_sum(s) == 0.0f) {
    // the corrected weights rounded away entirely: draw from p itself
    d.residual = 0;
    d.Md = d.Mt;
    d.iZd = 0.0f;
    const float2* st = a.stats + (static_cast<size_t>(b) * k1 + d.a) * nc;
    auto pw = [&](int i) {
      const float2 x = st[i];
      return x.x == -INFINITY ? 0.0f : x.y * exp2f((x.x - d.Mt) * c) * d.iZt;
    };
#pragma unroll
    for (int q = 0; q < kRegChunks; ++q) {
      const float x = pw(min(lane + 64 * q, nc - 1));
      fv[q] = lane + 64 * q < nc ? x : 0.0f;
    }
    stage_chunks(cw_sh, nc, fv, pw);
  } else {
    stage_chunks(cw_sh, nc, fv, [&](int i) { return fs[i]; });
  }
  const float* yt = a.yt + (static_cast<size_t>(b) * k1 + d.a) * a.V;
  const float* yd = d.residual ? a.yd + (static_cast<size_t>(b) * k + d.a) * a.V : yt;
  const int t = wave_pick(cw_sh, nc, a.V, u,
                          [&](int i) { return final_weight(d, yt[i], yd[i], c); }, id_sh);
  for (int j = lane; j < k1; j += 64)
    a.emitted[static_cast<size_t>(b) * k1 + j] = j < d.a ? a.draft[b * k + j] : (j == d.a ? t : -1);
  if (lane == 0) a.n_emitted[b] = d.a + 1;
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
  sample_pick_kernel<<<static_cast<unsigned>(M), 64, 0, st>>>(pa);
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
  if (2 * k + 1 <= kPrefetchRows)
    verify_decide_kernel<true><<<dim3(nc, static_cast<unsigned>(B)), kDecideThreads, 0, st>>>(va);
  else
    verify_decide_kernel<false><<<dim3(nc, static_cast<unsigned>(B)), kDecideThreads, 0, st>>>(va);
  rc = nest::check_launch(what);
  if (rc) return rc;
  verify_pick_kernel<<<static_cast<unsigned>(B), 64, 0, st>>>(va);
  return nest::check_launch(what);
}

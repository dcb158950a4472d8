// Batched verify over both planes (BitNest, Figure 3: the target reads the
// base and the refinement plane) for more than 16 activation rows, e.g. 16
// sequences x (k+1) = 144 rows: y = sa * fold_g s/16 * (sum q_a (16 q_b + q_r)).
// Given no refinement plane it computes the draft's base-plane product the
// same way (q_r = 0), for drafts of more than 16 rows.
//
// A block owns WR 16-row weight tiles (four, i.e. 64 rows; two to seven for
// some shapes), a range of the activation rows (CTP column tiles of 16) and all
// groups. Its last wave only copies int8 activation rows from HBM/L2 into an
// LDS ring (direct 16-byte loads to LDS, whole 128-byte rows of a group, two
// groups ahead). The WR WK compute waves (which hide each other's MFMA and
// LDS latencies) each own one weight tile and one of WK parts of the groups
// (WR waves per part) and stream their plane bytes with two groups of loads
// in flight beyond the current one. Per group the planes are merged into the
// 8-bit verify code of each weight,
//   c = 16 q_b + q_r = 16 (q_b - h) + (q_r mod 16),   h = [q_r < 0],
// an exact int8 (|c| <= 120): the base nibble less the refine sign goes to
// the high half of a byte (nibble arithmetic without borrows), the refine
// nibble to the low half, and the bytes are put back in element order. One
// v_mfma_i32_16x16x64_i8 pair per tile pair then gives the exact group sum
// of q_a c; the activation operand is 16 contiguous bytes of one row. The
// fp32 fold runs in registers in ascending group order within each half,
// and the halves are added in group order. Matrices with few rows split
// either the groups over S blocks (long rows: each block folds a
// contiguous slice of the groups for all activation rows, and the last of
// the S blocks to finish adds the slices' sums in slice order; it sees them
// by the same ordering argument as the argmax handoff in gemv.hip, agent-
// scope stores acknowledged before an agent-scope counter increment) or
// the activation rows over several blocks (each reads the same weights, on
// the same XCD, so the repeats come from its L2).
#include <algorithm>

#include "nibble.h"

namespace {

using nest::kGroup;
using nest::kMaxSplitRowBlocks;

constexpr int kRT = 1;                   // 16-row weight tiles per compute wave
// WR 16-row weight tiles per block (a template parameter, 2 and 4 to 7) and WK
// parts of the groups: WR WK compute waves, one per (tile, part), plus the
// copy wave
constexpr int threads_for(int wk, int wr) { return (wr * wk + 1) * 64; }
constexpr int kLdsBytes = 160 * 1024;    // LDS per workgroup on gfx950
// LDS ring slots per part of the groups: three (the copy wave runs two
// groups ahead) when they fit, else two
constexpr int ring_slots(int ctp, int wk) { return 3 * wk * ctp * 2048 <= kLdsBytes ? 3 : 2; }
constexpr int kSlots = 3;                // weight groups in flight per compute wave
constexpr int kMaxCT = 9;                // 144 activation rows per launch
constexpr int kXcds = 8;                 // blocks are dealt to the XCDs in turn
constexpr int kMaxSplit = 4;             // most slices of the groups (blocks per row block)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor: raw 32-bit data, bounds = num_records bytes
constexpr int kSC1 = 16;                // cache-policy bit sc1 of a buffer load / store

struct GemmArgs {
  const int8_t* qa;   // [M][K]
  const float* sa;    // [M]
  const uint8_t* base;
  const uint8_t* refine;
  const float* scales;
  float* y;           // [M][N]
  int32_t* acc_dbg;   // [M][N][G] (DBG)
  unsigned* done;     // split: [row_blocks] finished-slice counters (zero between launches)
  float* part;        // split: [row_blocks][S] per-block sums, lane-major
  int M, K, N, G, T;
  int row_blocks, parts, split;
};

struct WLoad {
  uint4 b, r;
  float s;
};

__device__ __forceinline__ void load_w(const GemmArgs& a, int t, int g, int kq, int idx, WLoad& w) {
  // tile layout: 16 bytes of row 16t + idx, k-quarter kq of group g at
  // ((t G + g) 4 + kq) 256 + 16 idx; the scale of that row and group at
  // ((t Gq + g/4) 16 + idx) 4 + g%4
  const size_t off = (static_cast<size_t>(t * a.G + g) * 4 + kq) * 256 + idx * 16;
  w.b = nest::ldnt16(a.base + off);
  // without a refinement plane (the draft over more than 16 rows) the codes
  // merge to 16 q_b: the product is 16 times the base plane's, folded at
  // s/16 as the verify's is
  w.r = a.refine ? nest::ldnt16(a.refine + off) : make_uint4(0, 0, 0, 0);
  const int Gq = (a.G + 3) >> 2;
  w.s = __builtin_nontemporal_load(a.scales + (static_cast<size_t>(t * Gq + (g >> 2)) * 16 + idx) * 4 + (g & 3));
}

// Eight elements (one word of each plane: nibble j is element 8t + j) ->
// their verify codes c = 16 q_b + q_r as eight bytes in element order.
__device__ __forceinline__ void merge_word(unsigned x, unsigned y, unsigned& lo, unsigned& hi) {
  constexpr unsigned H = 0x88888888u;
  const unsigned hv = (y >> 3) & 0x11111111u;    // refine sign -> bit 0 of its nibble
  const unsigned d = ((x | H) - hv) ^ (~x & H);  // per nibble (q_b - sign) mod 16, no borrows
  const unsigned e = ((d << 4) & 0xF0F0F0F0u) | (y & 0x0F0F0F0Fu);  // codes of elements 8t + 0, 2, 4, 6
  const unsigned o = (d & 0xF0F0F0F0u) | ((y >> 4) & 0x0F0F0F0Fu);  // and of 8t + 1, 3, 5, 7
  lo = __builtin_amdgcn_perm(o, e, 0x05010400u);  // elements 8t + 0..3
  hi = __builtin_amdgcn_perm(o, e, 0x07030602u);  // elements 8t + 4..7
}

// A weight slot's operands for one group: the codes of elements 0..15 and
// 16..31 of the lane's k-quarter for each tile, and the scales s/16.
struct WOps {
  v4i c0[kRT], c1[kRT];
  float sc[kRT];
};

__device__ __forceinline__ void build_ops(const WLoad (&w)[kRT], WOps& o) {
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    unsigned l, h;
    merge_word(w[rt].b.x, w[rt].r.x, l, h);
    o.c0[rt][0] = static_cast<int>(l);
    o.c0[rt][1] = static_cast<int>(h);
    merge_word(w[rt].b.y, w[rt].r.y, l, h);
    o.c0[rt][2] = static_cast<int>(l);
    o.c0[rt][3] = static_cast<int>(h);
    merge_word(w[rt].b.z, w[rt].r.z, l, h);
    o.c1[rt][0] = static_cast<int>(l);
    o.c1[rt][1] = static_cast<int>(h);
    merge_word(w[rt].b.w, w[rt].r.w, l, h);
    o.c1[rt][2] = static_cast<int>(l);
    o.c1[rt][3] = static_cast<int>(h);
    o.sc[rt] = w[rt].s * 0.0625f;
  }
}

// LDS slot of one group: per column tile ct, 16 rows of 128 bytes, the
// 16-byte piece q of row r stored at position q ^ swz(r) of that row, with
// swz(r) = (r & 7) ^ (r >> 3). A copy instruction then reads eight whole
// rows (full cache lines). A ds_read_b128 is served eight lanes at a time
// over 128 bytes of banks; lanes 0..7 (and 8..15) read one piece from eight
// consecutive rows, and swz gives those rows eight different positions, so
// no read has a bank conflict (measured: SQ_LDS_BANK_CONFLICT 0, against
// 3.7 cycles per read with the swizzle (r >> 1) & 7, which assumed
// 16-lane phases over 256 bytes).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int act_lds_off(int ct, int r, int q) { return ct * 2048 + r * 128 + ((q ^ swz(r)) << 4); }

// One group for the wave's weight tile(s) and the block's CTP column tiles:
// lane (kq, idx) takes pieces 2kq and 2kq + 1 (elements 32 kq .. +31) of
// row 16 ct + idx as its two A operands, and ends up with D[m][n] for
// m = 16 ct + 4 kq + i, n = 16 t + idx. Software-pipelined over the column
// tiles: operands are read two tiles ahead, products issued one tile ahead
// of their fold.
template <int CTP, bool DBG>
__device__ __forceinline__ void gemm_group(const GemmArgs& a, const uint8_t* slot, int lane, int kq, int idx,
                                           const int (&t)[kRT], int g, int ct0, const WOps& o,
                                           float (&run)[kRT][CTP][4]) {
  v4i la[3][2];
  v4i d[2][kRT];
  const v4i z = {0, 0, 0, 0};
  const int off0 = act_lds_off(0, idx, 2 * kq), off1 = act_lds_off(0, idx, 2 * kq + 1);
  auto lds = [&](int ct, int buf) {
    la[buf][0] = *reinterpret_cast<const v4i*>(slot + ct * 2048 + off0);
    la[buf][1] = *reinterpret_cast<const v4i*>(slot + ct * 2048 + off1);
  };
  auto mma = [&](int buf, int db) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      d[db][rt] = nest::mfma_i8(la[buf][0], o.c0[rt], z);
      d[db][rt] = nest::mfma_i8(la[buf][1], o.c1[rt], d[db][rt]);
    }
  };
  lds(0, 0);
  if (CTP > 1) lds(1, 1);
  mma(0, 0);
#pragma unroll
  for (int ct = 0; ct < CTP; ++ct) {
    if (ct + 2 < CTP) lds(ct + 2, (ct + 2) % 3);
    if (ct + 1 < CTP) mma((ct + 1) % 3, (ct + 1) % 2);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        run[rt][ct][i] = fmaf(o.sc[rt], static_cast<float>(d[ct % 2][rt][i]), run[rt][ct][i]);
      if (DBG) {
        const int n = t[rt] * 16 + idx;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = (ct0 + ct) * 16 + 4 * kq + i;
          if (m < a.M && n < a.N)  // the base plane's exact sum is the product / 16
            a.acc_dbg[(static_cast<size_t>(m) * a.N + n) * a.G + g] = a.refine ? d[ct % 2][rt][i] : d[ct % 2][rt][i] >> 4;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// LDS-only barrier for the compute waves (their weight loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The copy wave's barrier: it waits for its copies itself (vmcnt), so the
// compiler must neither add a wait nor move memory operations across.
__device__ __forceinline__ void copy_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int CTP, int WK, int WR, bool DBG>
__global__ void __launch_bounds__(threads_for(WK, WR)) gemm_kernel(GemmArgs a) {
  constexpr int kWK = WK, kWR = WR, kCW = kWR * WK;
  constexpr int SB = CTP * 2048;               // LDS bytes of one group's activations
  constexpr int kCopies = kWK * 2 * CTP;       // copy instructions per step
  constexpr int kNBuf = ring_slots(CTP, WK);   // ring slots per part
  constexpr int kAhead = kNBuf - 1;            // steps the copy wave runs ahead
  static_assert(kNBuf * kWK * SB <= kLdsBytes, "ring exceeds LDS");
  static_assert((kAhead - 1) * kCopies <= 63, "copies in flight exceed the vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kNBuf * kWK * SB];

  // blocks of one row block (its P activation-row parts or its S slices
  // of the groups) sit kXcds apart, i.e. on one XCD. (Giving each XCD one
  // slice instead, so that it reads only that slice's activation columns,
  // measured slower for 4096 x 14336: 28.5 against 26.5 us; the last
  // block's reads of sums written on other XCDs cost more than the saved
  // activation reads.)
  const int b = static_cast<int>(blockIdx.x), P = a.parts, S = a.split;
  const int rb = (b / (kXcds * P * S)) * kXcds + b % kXcds;
  const int ps = (b / kXcds) % (P * S);
  const int part = ps % P, slice = ps / P;
  if (rb >= a.row_blocks) return;
  const int ct0 = part * CTP;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int kq = lane >> 4, idx = lane & 15;
  // this block's groups: slice `slice` of S, [gs0, gs0 + Gs)
  const int gs0 = slice * a.G / S, Gs = (slice + 1) * a.G / S - gs0;
  const int steps = (Gs + kWK - 1) / kWK;
  auto h0 = [&](int wk) { return gs0 + wk * Gs / kWK; };  // half wk: groups [h0(wk), h0(wk + 1))

  if (wave == kCW) {
    // copy wave: group j of each half into slot j % kNBuf. Copy (ct, e)
    // fills rows 8e .. 8e + 7 of column tile ct: lane l writes position
    // l & 7 of row r = 8e + (l >> 3), i.e. piece (l & 7) ^ swz(r) of
    // activation row 16 ct + r (clamped to the last row). The group index is
    // clamped into the half (to group 0 for an empty half), so every step
    // issues kCopies copies.
    const int8_t* src_l[CTP][2];
#pragma unroll
    for (int c = 0; c < CTP; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 8 * e + (lane >> 3);
        src_l[c][e] = a.qa + static_cast<size_t>(min((ct0 + c) * 16 + r, a.M - 1)) * a.K +
                      (((lane & 7) ^ swz(r)) << 4);
      }
    auto copy_step = [&](int j) {
      uint8_t* slot0 = ring + (j % kNBuf) * kWK * SB;
#pragma unroll
      for (int wk = 0; wk < kWK; ++wk) {
        const int g = max(min(h0(wk) + j, h0(wk + 1) - 1), 0);
        uint8_t* dst = slot0 + wk * SB;
#pragma unroll
        for (int c = 0; c < CTP; ++c)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            __builtin_amdgcn_global_load_lds((glb_void*)(src_l[c][e] + static_cast<size_t>(g) * kGroup),
                                             (lds_void*)(dst + c * 2048 + e * 1024), 16, 0, 0);
      }
    };
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
      if (j < steps) copy_step(j);
    for (int j = 0; j < steps; ++j) {
      // step j's copies are done once at most the later step's are pending
      if (j + kAhead - 1 < steps) wait_vm<(kAhead - 1) * kCopies>();
      else wait_vm<0>();
      copy_barrier();
      if (j + kAhead < steps) copy_step(j + kAhead);
    }
    wait_vm<0>();
    copy_barrier();  // the ring is free: the parts' sums go through it
    copy_barrier();
    if (S > 1) {     // the compute waves' slice handoff
      copy_barrier();
      copy_barrier();
    }
    return;
  }

  const int wr = wave % kWR, wk = wave / kWR;
  const int t_first = (rb * kWR + wr) * kRT;
  int t[kRT];
  bool t_ok[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    t_ok[rt] = t_first + rt < a.T;
    t[rt] = min(t_first + rt, a.T - 1);
  }
  const int ga = h0(wk), gb = h0(wk + 1);
  float run[kRT][CTP][4];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CTP; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) run[rt][ct][i] = 0.0f;

  // weight loads: kSlots groups in flight, one register slot each; the
  // loop is unrolled by kSlots so that a slot's registers are only ever
  // refilled, never copied while their loads are in flight (group indices
  // clamped into the half, to group 0 for an empty half: branch-free and
  // in bounds), and every path through the loop issues the same loads
  auto gclamp = [&](int g) { return max(min(g, gb - 1), 0); };
  WLoad w[kSlots][kRT];
#pragma unroll
  for (int sl = 0; sl < kSlots; ++sl)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) load_w(a, t[rt], gclamp(ga + sl), kq, idx, w[sl][rt]);
  auto step = [&](int j, WLoad (&ws)[kRT]) {
    lds_barrier();  // step j's activations are in the ring
    WOps o;
    build_ops(ws, o);
    // the slot's registers are free again: request the group it serves next
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) load_w(a, t[rt], gclamp(ga + j + kSlots), kq, idx, ws[rt]);
    if (ga + j < gb)
      gemm_group<CTP, DBG>(a, ring + ((j % kNBuf) * kWK + wk) * SB, lane, kq, idx, t, ga + j, ct0, o, run);
  };
  const int full = steps - steps % kSlots;
  for (int j = 0; j < full; j += kSlots) {
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) step(j + sl, w[sl]);
  }
#pragma unroll
  for (int sl = 0; sl + 1 < kSlots; ++sl)
    if (full + sl < steps) step(full + sl, w[sl]);
  lds_barrier();  // all copies landed and every wave is past the ring

  // parts wk > 0 hand their sums to wk = 0 through LDS (ring reused), which
  // adds them in group order
  static_assert((kWK - 1) * kWR * kRT * CTP * 4 * 64 * 4 <= kNBuf * kWK * SB, "partial sums exceed the ring");
  float* comb = reinterpret_cast<float*>(ring);
  auto cidx = [&](int w, int rt, int ct, int i) {
    return ((((w - 1) * kWR + wr) * kRT + rt) * CTP * 4 + ct * 4 + i) * 64 + lane;
  };
  if (wk > 0) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTP; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) comb[cidx(wk, rt, ct, i)] = run[rt][ct][i];
  }
  lds_barrier();
  if (wk == 0) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTP; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int w = 1; w < kWK; ++w) run[rt][ct][i] += comb[cidx(w, rt, ct, i)];
  }
  if (S == 1) {
    if (wk > 0) return;
#pragma unroll
    for (int ct = 0; ct < CTP; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = (ct0 + ct) * 16 + 4 * kq + i;
        if (m >= a.M) continue;
        const float sm = a.sa[m];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const int n = t[rt] * 16 + idx;
          if (t_ok[rt] && n < a.N) a.y[static_cast<size_t>(m) * a.N + n] = run[rt][ct][i] * sm;
        }
      }
    return;
  }

  // Groups split over S blocks: this block's sums go to its slot, one
  // 16-byte piece per (tile, column tile, lane) holding its four rows i,
  // stored with the sc1 policy (what an agent-scope atomic store uses:
  // written through to the device's coherence point); once every store is
  // acknowledged the block counts itself in, and the last of the row
  // block's S blocks reads the S slots with the same policy (what an
  // agent-scope atomic load uses) and adds them in slice order.
  constexpr int kSlot = kWR * kRT * CTP * 4 * 64;  // floats per block slot
  const __amdgpu_buffer_rsrc_t slots = __builtin_amdgcn_make_buffer_rsrc(
      a.part + static_cast<size_t>(rb) * S * kSlot, 0, S * kSlot * static_cast<int>(sizeof(float)), kRsrcWord3);
  if (wk == 0) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CTP; ++ct) {
        const v4u v = {__float_as_uint(run[rt][ct][0]), __float_as_uint(run[rt][ct][1]),
                       __float_as_uint(run[rt][ct][2]), __float_as_uint(run[rt][ct][3])};
        const int piece = ((wr * kRT + rt) * CTP + ct) * 64 + lane;
        __builtin_amdgcn_raw_buffer_store_b128(v, slots, (slice * kSlot + 4 * piece) * 4, 0, kSC1);
      }
  }
  __shared__ int last_sh;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) last_sh = atomicAdd(a.done + rb, 1u) == static_cast<unsigned>(S - 1);
  __syncthreads();
  if (!last_sh) return;
  // the compute waves' threads take the pieces in turn; every load is
  // issued before the sums
  constexpr int kPieces = kSlot / 4, kNT = kCW * 64, kIter = (kPieces + kNT - 1) / kNT;
  const int tid = static_cast<int>(threadIdx.x);
  v4u v[kIter][kMaxSplit];
#pragma unroll
  for (int it = 0; it < kIter; ++it)
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      const int q = min(tid + it * kNT, kPieces - 1);
      v[it][s] = __builtin_amdgcn_raw_buffer_load_b128(slots, ((s < S ? s : 0) * kSlot + 4 * q) * 4, 0, kSC1);
    }
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int q = tid + it * kNT;
    if (q >= kPieces) continue;
    float tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] = __uint_as_float(v[it][0][i]);
#pragma unroll
    for (int s = 1; s < kMaxSplit; ++s)
      if (s < S) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] += __uint_as_float(v[it][s][i]);
      }
    // piece q: lane q % 64, column tile and tile from q / 64
    const int l = q & 63, ct = (q >> 6) % CTP, tr = (q >> 6) / CTP;  // tr = wr * kRT + rt
    const int tt = rb * kWR * kRT + tr, n = tt * 16 + (l & 15);
    if (tt >= a.T || n >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = (ct0 + ct) * 16 + 4 * (l >> 4) + i;
      if (m < a.M) a.y[static_cast<size_t>(m) * a.N + n] = tot[i] * a.sa[m];
    }
  }
  if (threadIdx.x == 0) atomicExch(a.done + rb, 0u);
}

template <int CTP, int WK, int WR, bool DBG>
int launch_gemm(const GemmArgs& a, int blocks, hipStream_t st) {
  gemm_kernel<CTP, WK, WR, DBG><<<dim3(blocks), dim3(threads_for(WK, WR)), 0, st>>>(a);
  return nest::check_launch("verify_gemm(batched)");
}

// Blocks carrying few column tiles have little work per group: their
// groups go to three parts (three compute waves per SIMD), which measured
// faster there (4096 x 14336: 43 -> 39 us); more column tiles keep two.
template <int WR, bool DBG>
int launch_ctp(const GemmArgs& a, int ctp, int blocks, hipStream_t st) {
  switch (ctp) {
    case 1: return launch_gemm<1, 3, WR, DBG>(a, blocks, st);
    case 2: return launch_gemm<2, 3, WR, DBG>(a, blocks, st);
    case 3: return launch_gemm<3, 3, WR, DBG>(a, blocks, st);
    case 4: return launch_gemm<4, 2, WR, DBG>(a, blocks, st);
    case 5: return launch_gemm<5, 2, WR, DBG>(a, blocks, st);
    case 6: return launch_gemm<6, 2, WR, DBG>(a, blocks, st);
    case 7: return launch_gemm<7, 2, WR, DBG>(a, blocks, st);
    case 8: return launch_gemm<8, 2, WR, DBG>(a, blocks, st);
    default: return launch_gemm<9, 2, WR, DBG>(a, blocks, st);
  }
}

// Wide blocks (five to seven tiles) always carry four or more column tiles,
// so two parts of the groups: 11 to 15 waves.
template <int WR, bool DBG>
int launch_ctp_wide(const GemmArgs& a, int ctp, int blocks, hipStream_t st) {
  switch (ctp) {
    case 4: return launch_gemm<4, 2, WR, DBG>(a, blocks, st);
    case 5: return launch_gemm<5, 2, WR, DBG>(a, blocks, st);
    case 6: return launch_gemm<6, 2, WR, DBG>(a, blocks, st);
    case 7: return launch_gemm<7, 2, WR, DBG>(a, blocks, st);
    case 8: return launch_gemm<8, 2, WR, DBG>(a, blocks, st);
    default: return launch_gemm<9, 2, WR, DBG>(a, blocks, st);
  }
}

template <bool DBG>
int launch_wr(const GemmArgs& a, int wr, int ctp, int blocks, hipStream_t st) {
  switch (wr) {
    case 2: return launch_ctp<2, DBG>(a, ctp, blocks, st);
    case 5: return launch_ctp_wide<5, DBG>(a, ctp, blocks, st);
    case 6: return launch_ctp_wide<6, DBG>(a, ctp, blocks, st);
    case 7: return launch_ctp_wide<7, DBG>(a, ctp, blocks, st);
    default: return launch_ctp<4, DBG>(a, ctp, blocks, st);
  }
}

int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// Work split: four weight tiles per block (five to seven when more tiles
// than four rounds' worth of CUs would need a second round: LLaMA-3-8B
// gate|up as one 28672 x 4096 matrix at 144 rows, 51.5 -> 39.9 us with
// seven-tile blocks in one round; seven for still more tiles). Few row blocks (under half the
// CUs) over long rows (64 groups or more) split the groups over S blocks
// per row block, each with all activation rows: every block stages a
// quarter (S = 4) of the activation bytes and streams a quarter of the
// row block's weights, where splitting the activation rows instead has each
// block read all the weights (LLaMA-3-8B down, 4096 x 14336 at 144 rows:
// 38.5 us as P = 3 against ~25 us for the same bytes in 256 one-slice
// blocks). Otherwise the activation rows are split evenly over P blocks per
// row block when the matrix alone would leave CUs idle (P divides the
// column tiles). When that needs more blocks than CUs (a partial second
// round of blocks on some CUs) and two-tile blocks over all activation rows
// fit in one round, those are taken (LLaMA-3-8B qkv, 6144 x 4096 at 144
// rows: 23.9 us as P = 3, 19.4-20.1 with two-tile blocks), with the other
// linears' splits measured best as they were. A group split needs one
// counter per row block in the workspace's counter zone, so it is taken
// only for at most kMaxSplitRowBlocks row blocks (with 256 CUs it never
// has more than 128).
struct Plan {
  int WR, P, S, row_blocks, CTP, blocks;
  size_t slot_bytes;  // the group split's partial sums (0 when S == 1)
};

Plan plan_batched(int M, int K, int N, int cus, bool split_ok = true) {
  Plan p{};
  const int T = (N + 15) / 16, CT = (M + 15) / 16, G = K / kGroup;
  p.WR = 4;
  p.P = 1;
  p.S = 1;
  int row_blocks = (T + 3) / 4;
  if (split_ok && 2 * row_blocks <= cus && G >= 64 && row_blocks <= kMaxSplitRowBlocks) {
    p.S = std::min(std::min(cus / row_blocks, G / 16), kMaxSplit);
  } else {
    for (int q = 1; q <= CT; ++q) {
      if (CT % q) continue;
      p.P = q;
      if (4 * row_blocks * q >= 3 * cus) break;
    }
    if (row_blocks * p.P > cus && (T + 1) / 2 <= cus) {
      p.WR = 2;
      p.P = 1;
    } else if (p.P == 1 && CT >= 4 && T > 4 * cus) {
      // more than one round of four-tile blocks: the fewest tiles per block
      // (five to seven) that fit one round, which also stages the
      // activations once per 80 to 112 weight rows instead of 64; seven
      // when even those need several rounds (the 152064-row LM head at 144
      // rows: 290-297 -> 248-261 us per verify_accept of 16 sequences)
      p.WR = std::min((T + cus - 1) / cus, 7);
    }
  }
  p.row_blocks = (T + p.WR - 1) / p.WR;
  p.CTP = CT / p.P;
  p.blocks = ((p.row_blocks + kXcds - 1) / kXcds) * kXcds * p.P * p.S;
  if (p.S > 1) {
    const size_t slot = static_cast<size_t>(p.WR) * kRT * p.CTP * 4 * 64 * sizeof(float);
    p.slot_bytes = static_cast<size_t>(p.row_blocks) * p.S * slot;
  }
  return p;
}

}  // namespace

namespace nest {

size_t verify_batched_slot_bytes(int M, int K, int N) {
  if (M < 1 || M > 16 * kMaxCT || K < kGroup || N < 1) return 0;
  return plan_batched(M, K, N, device_cus()).slot_bytes;
}

int launch_verify_batched(const int8_t* qa, const float* sa, int M, int K, const uint8_t* base,
                          const uint8_t* refine, const float* scales, int N, float* y, int32_t* acc_dbg,
                          unsigned* counters, void* slots, size_t slot_bytes, hipStream_t st) {
  if (M < 1 || M > 16 * kMaxCT)
    return fail(NEST_EINVAL, "verify_gemm(batched): %d rows per launch (1..%d)", M, 16 * kMaxCT);
  GemmArgs a{};
  a.qa = qa; a.sa = sa; a.base = base; a.refine = refine; a.scales = scales;
  a.y = y; a.acc_dbg = acc_dbg;
  a.M = M; a.K = K; a.N = N; a.G = K / kGroup; a.T = (N + 15) / 16;
  // without counters (a caller with no room for the partial sums) the
  // groups are not split
  const Plan p = plan_batched(M, K, N, device_cus(), counters != nullptr);
  if (p.S > 1) {
    if (!counters || !slots || slot_bytes < p.slot_bytes)
      return fail(NEST_EWORKSPACE, "verify_gemm: the group split needs %zu bytes of partial sums", p.slot_bytes);
    if (!aligned16(slots) || !aligned16(counters))
      return fail(NEST_EALIGN, "verify_gemm: workspace not 16-byte aligned");
    a.done = counters;
    a.part = static_cast<float*>(slots);
  }
  a.row_blocks = p.row_blocks;
  a.parts = p.P;
  a.split = p.S;
  return acc_dbg ? launch_wr<true>(a, p.WR, p.CTP, p.blocks, st) : launch_wr<false>(a, p.WR, p.CTP, p.blocks, st);
}

}  // namespace nest

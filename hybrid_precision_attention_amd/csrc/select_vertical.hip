// hq_select_vertical for gfx950: column-mass score and top-rho selection.
//
// The vertical-line score of a key position is the attention mass that the
// buffered FP16 queries put on it, accumulated over refreshes, and the lines
// are the top-rho positions of the non-window prefix (agihunt digest
// "HyQuant: Hybrid-Precision Quantization for LLM Attention", method
// paragraph; HyQuant README, Overview item 1).
//
// Rows of a unit are its R = G * nb buffered queries (row r = g * nb + jq, at
// position L - nb + jq).  Two streaming kernels read the unit's keys:
//   1. row_stats: per streaming workgroup, the (max, sum of exp) of every row
//      over the workgroup's causal keys (skipped when the caller passes the
//      rows' LSE);
//   2. col_mass: merges those into each row's LSE, then for every key of the
//      non-window prefix sums exp(tau q.k - lse) over the rows and adds it to
//      the running score.
// Both compute S = K Q^T with v_mfma_f32_16x16x32_f16 (A = 16 keys, B = 16
// rows).  A workgroup stages up to 256 rows of queries in LDS; each of its
// eight waves holds 64 keys in registers with the next 64 in flight, and the
// next row block's MFMAs are interleaved with the current block's
// exponentials.  More than 256 rows (G > 4) form row groups on the grid.
// Every sum has a fixed order (no float atomics): reruns are bit-identical.
//   3. topk: one workgroup per unit finds the n_vl-th largest score by a
//      radix select over order-preserving integer keys, then flags positions
//      in ascending order (ties at the threshold to the lower positions) and
//      compacts them into vl_idx.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <utility>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kSWaves = 8;            // waves per streaming workgroup
constexpr int kSThreads = 64 * kSWaves;
constexpr int kChunk = 64;            // keys a wave holds in registers at a time
constexpr int kRG = 256;              // rows per row group (queries staged in LDS)
constexpr int kRB = kRG / 16;         // 16-row blocks per row group
constexpr int kTopThreads = 1024;
constexpr int kSelCUs = 256;          // MI355X compute units

struct SelArgs {
  const uint16_t* qbuf;
  const uint16_t* k;
  const float* lse;                 // natural log, [B][Hq][nb]
  float2* stats;                    // [U][nwg1][R] (max raw score, sum exp2)
  float* colpart;                   // [nrg][U][n_nw] column mass per row group (nrg > 1)
  float* score;
  int32_t* vl_idx;
  uint8_t* vl_flag;
  int32_t Hq, Hkv, G, nb, L, W, R, n_nw, n_vl;
  int32_t C;                        // chunks per wave
  int32_t wg_keys;                  // keys per streaming workgroup = 64 * 8 * C
  int32_t nwg1, nrg, U;
  int32_t lse_from_stats;           // 1: rows' LSE merged from stats by col_mass
  float c2;                         // log2(e) / sqrt(d)
  float* cut;                       // [U] top-k cut-off value out (nullable)
  // decode-time refresh only: the hybrid cache at decode position t
  hq_cache c;
  int32_t t, cap_q, cap_vl, cap_stg;
  int32_t nwgr;                     // refresh workgroups per unit (its chunks split evenly)
  int32_t xcd_group;                // 1: a unit's workgroups are placed on one XCD
};

__device__ __forceinline__ half8_t as_half8(uint4 v) { return __builtin_bit_cast(half8_t, v); }

// float -> unsigned key with the same order (-0 folded onto +0)
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t bits = __builtin_bit_cast(uint32_t, f);
  if (bits == 0x80000000u) bits = 0;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// max / sum with lanes l^16 and l^32 (the four j-lanes of a row), through the
// VALU lane-swap instructions rather than the LDS crossbar
__device__ __forceinline__ float max_j(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_j(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Cross-lane moves inside the VALU (no LDS round trip).  DPP: lane ^ 1 and
// lane ^ 2 (quad permutes), the mirror inside each half-row of 8 (lane ^ 7)
// and inside each row of 16 (lane ^ 15); v_permlane16/32_swap exchange rows.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kCtrl, 0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ float dppf(float x) {
  return __uint_as_float(dpp<kCtrl>(__float_as_uint(x)));
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kRowMirror = 0x140;

// op over the 64 lanes of a wave; every lane gets the result
template <typename Op>
__device__ __forceinline__ uint32_t wave_all(uint32_t x, Op op) {
  x = op(x, dpp<kXor1>(x));
  x = op(x, dpp<kXor2>(x));
  x = op(x, dpp<kHalfMirror>(x));
  x = op(x, dpp<kRowMirror>(x));
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(b[0], b[1]);
}
__device__ __forceinline__ int wave_sum(int x) {
  return static_cast<int>(wave_all(static_cast<uint32_t>(x), [](uint32_t p, uint32_t q) { return p + q; }));
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return wave_all(x, [](uint32_t p, uint32_t q) { return min(p, q); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_all(x, [](uint32_t p, uint32_t q) { return max(p, q); });
}

// inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 (zero fill)
// inside each row of 16, then the totals of the earlier rows
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  x += static_cast<int>(dpp<0x111>(static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp<0x112>(static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp<0x114>(static_cast<uint32_t>(x)));
  x += static_cast<int>(dpp<0x118>(static_cast<uint32_t>(x)));
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

__device__ __forceinline__ float4_t mfma(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// K operand of the wave's 64 keys: lane (key t, j) holds dims 32j..32j+31 of
// key k0 + 16x + t for x = 0..3 (k-step kk = dims 32j+8kk..).  Keys past the
// last one are clamped to it, so the loads are unconditional.
__device__ __forceinline__ void load_keys(uint4 kr[4][4], const uint16_t* kunit, int k0, int L,
                                          int n, int j) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int key = min(k0 + 16 * x + n, L - 1);
    const uint16_t* p = kunit + static_cast<int64_t>(key) * kD + 32 * j;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kr[x][kk] = ld16(p + 8 * kk);
  }
}

// Rows [R rg, R rg + R) of the unit's buffered queries in LDS (R = 16 kNRB
// rows a group: 256 in the dense passes, 256 or 512 in the refresh), in the
// B-operand order of the MFMA: q[rb][kk][16 j + n] = dims 32j + 8kk .. +7 of
// row 16 rb + n.  Rows past the last one repeat it (their results are
// discarded).  Every lane of a wave then reads 16 consecutive bytes.
template <int kNRB>
using QStageT = uint4[kNRB][4][64];
using QStage = QStageT<kRB>;

constexpr int kStageIters = kRG * 16 / kSThreads;   // 16-byte pieces per thread (256 rows)

// The staging is split into loads and stores, so that other loads can be in
// flight with it: all of the thread's loads are issued before any is stored.
// Part `part` of a group of 16 kNRB rows covers its rows
// [256 part, 256 part + 256).
template <int kNRB = kRB>
__device__ __forceinline__ void stage_load(uint4 v[kStageIters], const SelArgs& a, int64_t b, int h0,
                                           int rg, int part = 0) {
#pragma unroll
  for (int i = 0; i < kStageIters; ++i) {
    const int idx = threadIdx.x + i * kSThreads;
    const int rr = kRG * part + (idx >> 4), ch = idx & 15;
    const int r = min(rg * 16 * kNRB + rr, a.R - 1);
    const int g = r / a.nb, jq = r - g * a.nb;
    v[i] = ld16(a.qbuf + ((b * a.Hq + h0 + g) * a.nb + jq) * kD + 8 * ch);
  }
}
template <int kNRB = kRB>
__device__ __forceinline__ void stage_store(QStageT<kNRB>& sq, const uint4 v[kStageIters], int part = 0) {
#pragma unroll
  for (int i = 0; i < kStageIters; ++i) {
    const int idx = threadIdx.x + i * kSThreads;
    const int rr = kRG * part + (idx >> 4), ch = idx & 15;
    sq[rr >> 4][ch & 3][16 * (ch >> 2) + (rr & 15)] = v[i];
  }
}
__device__ __forceinline__ void stage_rows(QStage& sq, const SelArgs& a, int64_t b, int h0, int rg) {
  uint4 v[kStageIters];
  stage_load(v, a, b, h0, rg);
  stage_store(sq, v);
}

template <int kNRB = kRB>
__device__ __forceinline__ void load_q(half8_t qb[4], const QStageT<kNRB>& sq, int rb, int lane) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qb[kk] = as_half8(sq[rb][kk][lane]);
}
// k-steps k0, k0 + 1 of row block rb
template <int kNRB = kRB>
__device__ __forceinline__ void load_q2(half8_t qb[2], const QStageT<kNRB>& sq, int rb, int k0, int lane) {
  qb[0] = as_half8(sq[rb][k0][lane]);
  qb[1] = as_half8(sq[rb][k0 + 1][lane]);
}

// S of the first kNX blocks of 16 keys (four independent accumulation
// chains when kNX = 4, interleaved)
template <int kNX = 4>
__device__ __forceinline__ void mfma_scores(float4_t s[4], const uint4 kr[4][4], const half8_t qb[4]) {
#pragma unroll
  for (int x = 0; x < kNX; ++x) s[x] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int x = 0; x < kNX; ++x) s[x] = mfma(as_half8(kr[x][kk]), qb[kk], s[x]);
}

// Every pass keeps its LDS operands ahead of use: the query operands of row
// block rb + 2 are read while row block rb is computed.

// Streaming workgroup (x, unit, row group): keys [x * wg_keys, ...), wave w
// taking 64-key chunks w, w + 8, ... with the next chunk's keys in flight
// while the current one is computed; the row group's queries sit in LDS.
// Inside a chunk the scores of row block rb + 1 are issued to the matrix
// cores before the exponentials of row block rb, so the two overlap.

// Pass 1 over one chunk: every lane keeps its own running (max, sum) per row
// block for the keys it holds (no cross-lane work inside the loop).
template <bool kMasked>
__device__ __forceinline__ void chunk_row_stats(float2 (*st)[64], const uint4 kr[4][4],
                                                const QStage& sq, const SelArgs& a, int rg, int k0,
                                                int lane, int n, int j) {
  float4_t sc[4];
  half8_t q1[4], q2[4];
  load_q(q1, sq, 0, lane);
  mfma_scores(sc, kr, q1);
  load_q(q1, sq, 1, lane);
  float2 old = st[0][lane];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float4_t sn[4];
    float2 old_n = old;
    if (rb + 2 < kRB) load_q(q2, sq, rb + 2, lane);
    if (rb + 1 < kRB) {
      old_n = st[rb + 1][lane];
      mfma_scores(sn, kr, q1);
    }
    float v[16];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * x + e] = sc[x][e];
    if (kMasked) {
      // keys past the prefix or after the row's own position do not count
      const int r = min(rg * kRG + rb * 16 + n, a.R - 1);
      const int prow = a.L - a.nb + (r - (r / a.nb) * a.nb);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 16 * x + 4 * j + e;
          if (!(key < a.L && key <= prow)) v[4 * x + e] = -INFINITY;
        }
    }
    // a tree of three-input maxima (v_max3_f32) over the 16 values and the old max
    const float m0 = fmaxf(fmaxf(v[0], v[1]), v[2]), m1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
    const float m2 = fmaxf(fmaxf(v[6], v[7]), v[8]), m3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
    const float m4 = fmaxf(fmaxf(v[12], v[13]), v[14]), m5 = fmaxf(fmaxf(v[15], old.x), m0);
    const float mx = fmaxf(fmaxf(m1, m2), fmaxf(fmaxf(m3, m4), m5));
    const float mu = (kMasked && mx == -INFINITY) ? 0.0f : mx;
    const float nmc = -mu * a.c2;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      s0 += __builtin_amdgcn_exp2f(fmaf(v[e], a.c2, nmc));
      s1 += __builtin_amdgcn_exp2f(fmaf(v[e + 1], a.c2, nmc));
    }
    st[rb][lane] = make_float2(mx, fmaf(old.y, __builtin_amdgcn_exp2f(fmaf(old.x, a.c2, nmc)), s0 + s1));
    if (!kMasked && rb + 1 < kRB) {
      // the LDS reads first, then the next row block's 16 MFMAs interleaved
      // with this block's VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
    if (rb + 1 < kRB) {
#pragma unroll
      for (int x = 0; x < 4; ++x) sc[x] = sn[x];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) q1[kk] = q2[kk];
      old = old_n;
    }
  }
}

// Pass 1: per (workgroup, row), (max raw score, sum exp2) over its keys.
__global__ __launch_bounds__(kSThreads) void row_stats_kernel(SelArgs a) {
  __shared__ QStage s_q;                                    // 64 KB
  // each lane's running (max, sum) of row 16 rb + n over the keys it held
  __shared__ float2 s_run[kSWaves][kRB][64];                // 64 KB
  __shared__ float2 s_st[kSWaves][kRG];                     // 16 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int64_t u = blockIdx.y;
  const int rg = blockIdx.z;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const int wg0 = blockIdx.x * a.wg_keys;
  const uint16_t* kunit = a.k + u * a.L * kD;
  uint4 kr[4][4];
  load_keys(kr, kunit, wg0 + kChunk * wave, a.L, n, j);
  stage_rows(s_q, a, b, h0, rg);
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) s_run[wave][rb][lane] = make_float2(-INFINITY, 0.0f);
  __syncthreads();

  for (int i = 0; i < a.C; ++i) {
    const int k0 = wg0 + kChunk * (wave + kSWaves * i);
    if (k0 >= a.L) break;
    // the next chunk's keys, only when this wave has one (a prefetch past
    // the workgroup's range would read keys no wave of it uses)
    const bool more = i + 1 < a.C && k0 + kChunk * kSWaves < a.L;
    uint4 kn[4][4];
    if (more) load_keys(kn, kunit, k0 + kChunk * kSWaves, a.L, n, j);
    __builtin_amdgcn_sched_barrier(0);                      // keep the prefetch ahead
    // every key of the chunk precedes every buffered query: no causal mask
    if (k0 + kChunk <= a.L - a.nb)
      chunk_row_stats<false>(s_run[wave], kr, s_q, a, rg, k0, lane, n, j);
    else
      chunk_row_stats<true>(s_run[wave], kr, s_q, a, rg, k0, lane, n, j);
    if (!more) break;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kr[x][kk] = kn[x][kk];
  }
  // merge the four j-lanes of each row, then the waves
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float2 v = s_run[wave][rb][lane];
    const float m = max_j(v.x);
    const float mu = (m == -INFINITY) ? 0.0f : m;
    const float sum = sum_j(v.y * __builtin_amdgcn_exp2f((v.x - mu) * a.c2));
    if (j == 0) s_st[wave][rb * 16 + n] = make_float2(m, sum);
  }
  __syncthreads();
  float2* out = a.stats + (u * a.nwg1 + blockIdx.x) * a.R + rg * kRG;
  const int nr = min(kRG, a.R - rg * kRG);
  for (int r = tid; r < nr; r += kSThreads) {
    float mx = s_st[0][r].x;
#pragma unroll
    for (int w = 1; w < kSWaves; ++w) mx = fmaxf(mx, s_st[w][r].x);
    float sum = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSWaves; ++w)
        sum = fmaf(s_st[w][r].y, __builtin_amdgcn_exp2f((s_st[w][r].x - mx) * a.c2), sum);
    }
    out[r] = make_float2(mx, sum);
  }
}

// Pass 2 over one chunk: acc[4x + e] += sum over the lane's rows of
// exp2(c2 s - lse log2 e) for key k0 + 16x + 4j + e.  The query operands and
// -lse of row block rb + 2 are read from LDS while row block rb is computed,
// so the MFMAs of rb + 1 never wait for an LDS round trip.
template <bool kMasked>
__device__ __forceinline__ void chunk_col_mass(float acc[16], const uint4 kr[4][4], const QStage& sq,
                                               const float* s_nl, const SelArgs& a, int rg, int k0,
                                               int lane, int n, int j) {
  float4_t sc[4];
  half8_t q0[4], q01[2], q23[2], n01[2];
  load_q(q0, sq, 0, lane);
  mfma_scores(sc, kr, q0);
  load_q2(q01, sq, 1, 0, lane);
  float nl_c = s_nl[n], nl_1 = s_nl[16 + n];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float4_t sn[4];
    float nl_2 = 0.0f;
    if (rb + 1 < kRB) load_q2(q23, sq, rb + 1, 2, lane);
    if (rb + 2 < kRB) {
      load_q2(n01, sq, rb + 2, 0, lane);
      nl_2 = s_nl[(rb + 2) * 16 + n];
    }
    if (rb + 1 < kRB) {
      const half8_t q1[4] = {q01[0], q01[1], q23[0], q23[1]};
      mfma_scores(sn, kr, q1);
    }
    if (!kMasked) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[4 * x + e] += __builtin_amdgcn_exp2f(fmaf(sc[x][e], a.c2, nl_c));
      if (rb + 1 < kRB) {
        // the LDS reads of rb + 2 first, then the next row block's 16 MFMAs
        // interleaved with this block's 48 VALU
        if (rb + 2 < kRB) __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
    } else {
      const int r = min(rg * kRG + rb * 16 + n, a.R - 1);
      const int prow = a.L - a.nb + (r - (r / a.nb) * a.nb);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 16 * x + 4 * j + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[x][e], a.c2, nl_c));
          acc[4 * x + e] += (key < a.n_nw && key <= prow) ? p : 0.0f;
        }
    }
    if (rb + 1 < kRB) {
#pragma unroll
      for (int x = 0; x < 4; ++x) sc[x] = sn[x];
      q01[0] = n01[0];
      q01[1] = n01[1];
      nl_c = nl_1;
      nl_1 = nl_2;
    }
    // one scheduling region a row block: the reads issued for rb + 2 are
    // not sunk to their use
    if (!kMasked) __builtin_amdgcn_sched_barrier(0);
  }
}

// Sum over the 16 row lanes of a wave: lane (n, j) ends with the total of
// acc[n], i.e. of entry 16 (n >> 2) + 4 j + (n & 3) of the chunk.  At the
// step for bit b the lane keeps the half of the values whose index bit b
// equals its own and adds the partner's copy of that half; any partner that
// differs in bit b and agrees in the higher bits will do, so the partners
// are the DPP row mirror (bit 3), half-row mirror (bit 2) and quad swaps.
__device__ __forceinline__ float reduce_scatter16(const float acc[16], int n) {
  float t8[8], t4[4], t2[2];
  {
    const bool hi = (n & 8) != 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float keep = hi ? acc[q + 8] : acc[q], send = hi ? acc[q] : acc[q + 8];
      t8[q] = keep + dppf<kRowMirror>(send);
    }
  }
  {
    const bool hi = (n & 4) != 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float keep = hi ? t8[q + 4] : t8[q], send = hi ? t8[q] : t8[q + 4];
      t4[q] = keep + dppf<kHalfMirror>(send);
    }
  }
  {
    const bool hi = (n & 2) != 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float keep = hi ? t4[q + 2] : t4[q], send = hi ? t4[q] : t4[q + 2];
      t2[q] = keep + dppf<kXor2>(send);
    }
  }
  const bool hi = (n & 1) != 0;
  const float keep = hi ? t2[1] : t2[0], send = hi ? t2[0] : t2[1];
  return keep + dppf<kXor1>(send);
}

// Pass 2: column mass of the non-window keys: per key, the sum over the row
// group's rows of exp(tau q.k - lse), added to the running score (one row
// group) or written as the group's part (several; top-k folds them in).
__global__ __launch_bounds__(kSThreads) void col_mass_kernel(SelArgs a) {
  __shared__ QStage s_q;                                    // 64 KB
  __shared__ float s_nl[kRG];                               // -lse * log2(e), -inf for padding
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int64_t u = blockIdx.y;
  const int rg = blockIdx.z;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const int wg0 = blockIdx.x * a.wg_keys;
  const uint16_t* kunit = a.k + u * a.L * kD;
  const int lim = a.n_nw;
  uint4 kr[4][4];
  load_keys(kr, kunit, wg0 + kChunk * wave, a.L, n, j);
  // keys, queries and the rows' statistics are all in flight before the first wait
  uint4 qv[kStageIters];
  stage_load(qv, a, b, h0, rg);
  if (a.lse_from_stats) {
    // merge each row's (max, sum exp2) over the pass-1 workgroups: thread
    // pair (row, half) takes every other workgroup, sixteen loads in flight
    // at a time, as running (max, sum) pairs; the halves then combine
    static_assert(kSThreads == 2 * kRG, "two threads per row");
    const int rr = tid >> 1, half = tid & 1;
    const int r = rg * kRG + rr;
    const float2* st = a.stats + u * a.nwg1 * a.R + min(r, a.R - 1);
    float mx = -INFINITY, sum = 0.0f;
    for (int t0 = half; t0 < a.nwg1; t0 += 32) {
      float2 v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        v[e] = st[static_cast<int64_t>(min(t0 + 2 * e, a.nwg1 - 1)) * a.R];
      float cm = mx;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (t0 + 2 * e < a.nwg1) cm = fmaxf(cm, v[e].x);
      if (cm != -INFINITY) {
        float s = sum * __builtin_amdgcn_exp2f((mx - cm) * a.c2);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (t0 + 2 * e < a.nwg1) s = fmaf(v[e].y, __builtin_amdgcn_exp2f((v[e].x - cm) * a.c2), s);
        sum = s;
        mx = cm;
      }
    }
    const float mo = dppf<kXor1>(mx), so = dppf<kXor1>(sum);
    const float m = fmaxf(mx, mo);
    float tot = 0.0f;
    if (m != -INFINITY)
      tot = sum * __builtin_amdgcn_exp2f((mx - m) * a.c2) + so * __builtin_amdgcn_exp2f((mo - m) * a.c2);
    if (half == 0) s_nl[rr] = (r < a.R) ? -(m * a.c2 + log2f(tot)) : -INFINITY;   // -lse * log2(e)
  } else {
    for (int rr = tid; rr < kRG; rr += kSThreads) {
      const int r = rg * kRG + rr;
      float nl = -INFINITY;                                 // padding rows add nothing
      if (r < a.R) {
        const int g = r / a.nb, jq = r - g * a.nb;
        nl = -a.lse[(b * a.Hq + h0 + g) * a.nb + jq] * 1.4426950408889634f;
      }
      s_nl[rr] = nl;
    }
  }
  stage_store(s_q, qv);
  __syncthreads();
  float* sc = a.score + u * a.L;
  float* part = a.colpart + (static_cast<int64_t>(rg) * a.U + u) * a.n_nw;
  // lane (n, j) owns key k0 + 16 (n >> 2) + 4 j + (n & 3) of each chunk: the
  // key whose total it ends with after the reduce-scatter below
  const int own = 16 * (n >> 2) + 4 * j + (n & 3);
  for (int i = 0; i < a.C; ++i) {
    const int k0 = wg0 + kChunk * (wave + kSWaves * i);
    if (k0 >= lim) break;
    // the running score of the owned key, loaded before the prefetch so that
    // waiting for it does not wait for the next chunk's keys
    const int key = k0 + own;
    const float prev = (a.nrg == 1) ? sc[min(key, lim - 1)] : 0.0f;
    const bool more = i + 1 < a.C && k0 + kChunk * kSWaves < lim;
    uint4 kn[4][4];
    if (more) load_keys(kn, kunit, k0 + kChunk * kSWaves, a.L, n, j);
    __builtin_amdgcn_sched_barrier(0);                      // keep the prefetch ahead
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    // all 64 keys are non-window and precede every buffered query
    if (k0 + kChunk <= min(lim, a.L - a.nb))
      chunk_col_mass<false>(acc, kr, s_q, s_nl, a, rg, k0, lane, n, j);
    else
      chunk_col_mass<true>(acc, kr, s_q, s_nl, a, rg, k0, lane, n, j);
    const float tot = reduce_scatter16(acc, n);
    if (key < lim) {
      if (a.nrg == 1) sc[key] = prev + tot;
      else part[key] = tot;
    }
    if (!more) break;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kr[x][kk] = kn[x][kk];
  }
}

// ---------------------------------------------------------------------------
// Decode-time refresh over the hybrid cache.  The unit's keys are its cache
// as stored at decode position t, in list order: the K4V4 slots, the
// vertical lines, the window positions t - nwin .. t - 1 (ring slot pos mod
// W) and the staged token (position t).  A K4V4 key's elements enter the
// matrix cores as fp16 roundings of code * scale + min (the fp16 operand
// type of the MFMA): each within 2^-11 relative (or half an fp16 subnormal
// step) of the cache's key, an error the scores' tolerance allows for.  Row
// r = g * nb + jq is the buffered query at position t - nb + 1 + jq; every
// cached key at a position up to the row's own gets exp(tau q.k - lse)
// added to the running score at that position.
//
// The products are v_mfma_f32_32x32x16_f16 tiles, S = K Q^T with 32 keys
// (A) by 32 rows (B), which on gfx950 deliver twice the rate of the
// 16x16x32 form.  A wave holds a chunk of 64 entries as two key tiles; lane
// (kl, h) = (lane % 32, lane / 32) holds dims 64 h + 8 ks .. + 7 of entry
// 32 kt + kl for k-steps ks = 0..7 (the contraction runs over the dims in
// that order on both operands, so a lane's dims are one contiguous half of
// the row: two groups of 32).  Output register r of tile (kt, row tile)
// holds entry 32 kt + 8 (r / 4) + 4 h + r % 4 against row lane % 32.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(half8_t a, half8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

struct HybridList {
  int nq, nvl, nwin, nst, n;
};

__device__ __forceinline__ HybridList hybrid_list(const SelArgs& a, int64_t u) {
  HybridList h;
  h.nq = min(max(a.c.n_q[u], 0), a.cap_q);
  h.nvl = min(max(a.c.n_vl[u], 0), a.cap_vl);
  h.nwin = min(a.W, a.t);
  h.nst = min(max(a.c.n_stg[u], 0), min(a.cap_stg, 1));
  h.n = h.nq + h.nvl + h.nwin + h.nst;
  return h;
}

constexpr int kNoPos = 0x7FFFFFFF;   // list entries past the last key

// Query rows in LDS in the B-operand order of the 32x32x16 tiles:
// q[rt][ks][lane] = dims 64 (lane / 32) + 8 ks .. + 7 of row 32 rt + lane % 32.
template <int kNRT>
using QStage32 = uint4[kNRT][8][64];
using QTile32 = uint4[8][64];                // one row tile

// Rows [rows rg + 256 part, ... + 256) of the group into their row tiles
template <int kNRT>
__device__ __forceinline__ void stage32_load(uint4 v[kStageIters], const SelArgs& a, int64_t b, int h0,
                                             int rg, int part) {
#pragma unroll
  for (int i = 0; i < kStageIters; ++i) {
    const int idx = threadIdx.x + i * kSThreads;
    const int rr = kRG * part + (idx >> 4), ch = idx & 15;
    const int r = min(rg * 32 * kNRT + rr, a.R - 1);
    const int g = r / a.nb, jq = r - g * a.nb;
    v[i] = ld16(a.qbuf + ((b * a.Hq + h0 + g) * a.nb + jq) * kD + 8 * ch);
  }
}
template <int kNRT>
__device__ __forceinline__ void stage32_store(QStage32<kNRT>& sq, const uint4 v[kStageIters], int part) {
#pragma unroll
  for (int i = 0; i < kStageIters; ++i) {
    const int idx = threadIdx.x + i * kSThreads;
    const int rr = kRG * part + (idx >> 4), ch = idx & 15;
    sq[rr >> 5][ch & 7][32 * (ch >> 3) + (rr & 31)] = v[i];
  }
}

// K4V4 entries k0 + 32 kt + kl (all below nq) for lane (kl, h): the codes of
// dims 64 h .. 64 h + 63 (2 kKB words), the {scale, min} words of groups
// 2h and 2h + 1, and the position, of both key tiles.
template <int kKB>
struct KRaw32 {
  uint32_t codes[2][2 * kKB];
  uint2 meta[2];
  int pos[2];
};

template <int kKB>
__device__ __forceinline__ void load_codes_half(uint32_t w[2 * kKB], const uint8_t* p) {
#pragma unroll
  for (int i = 0; i < 2 * kKB; i += 4) {
    const uint4 v = ld16(p + 4 * i);
    w[i] = v.x;
    w[i + 1] = v.y;
    w[i + 2] = v.z;
    w[i + 3] = v.w;
  }
}

template <int kKB>
__device__ __forceinline__ void load_k4raw32(KRaw32<kKB>& r, const SelArgs& a, int64_t u, int k0, int kl, int h) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int64_t sl = k4_slot(a.c.k4_pages, a.cap_q, u, k0 + 32 * kt + kl);
    load_codes_half<kKB>(r.codes[kt], a.c.kq + sl * (16 * kKB) + 8 * kKB * h);
    r.meta[kt] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint32_t*>(a.c.kq_meta) +
                                                 sl * kMetaWords + 2 * h);
    r.pos[kt] = a.c.q_pos[sl];
  }
}

// Eight 4-bit codes (element e in bits 4e .. 4e + 3) to eight fp16
// code * scale + min, each rounded once: the code goes into the mantissa of
// 1024 (giving exactly 1024 + code), 1024 is taken off (exact), then one
// fused multiply-add.
__device__ __forceinline__ uint4 dequant8(uint32_t w, half2_t s2, half2_t m2) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // byte i: element 2i
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // byte i: element 2i + 1
  const half2_t k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // low half: element 2i, high half: element 2i + 1
    const uint32_t pair = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * i) | 0x64006400u;
    const half2_t c = __builtin_bit_cast(half2_t, pair) - k1024;
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, s2, m2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Elements 8 ks .. 8 ks + 7 of the lane's 64 (kKB-bit codes, element e at
// bits kKB e of the words), dequantised with the group's {scale, min}.
template <int kKB>
__device__ __forceinline__ uint4 dequant_slice(const uint32_t w[2 * kKB], int ks, uint32_t meta) {
  const half2_t sm = __builtin_bit_cast(half2_t, meta);
  const half2_t s2 = {sm[0], sm[0]}, m2 = {sm[1], sm[1]};
  if constexpr (kKB == 4) {
    return dequant8(w[ks], s2, m2);
  } else {
    constexpr uint32_t kMask = (1u << kKB) - 1u;
    const half2_t k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = 8 * ks + 2 * p;
      const uint32_t c0 = (w[(kKB * e) >> 5] >> ((kKB * e) & 31)) & kMask;
      const uint32_t c1 = (w[(kKB * (e + 1)) >> 5] >> ((kKB * (e + 1)) & 31)) & kMask;
      const half2_t c = __builtin_bit_cast(half2_t, c0 | (c1 << 16) | 0x64006400u) - k1024;
      o[p] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, s2, m2));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <int kKB>
__device__ __forceinline__ void dequant_tile(uint4 kr[8], const uint32_t w[2 * kKB], uint2 meta) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kr[ks] = dequant_slice<kKB>(w, ks, ks < 4 ? meta.x : meta.y);
}

// fp16 operands of any 64 list entries (zeros past the list) and their
// positions (kNoPos past the list).  Used for the few chunks that are not
// all K4V4, so the loads are simply issued in order.
template <int kKB>
__device__ __forceinline__ void load_any32(uint4 kr[2][8], int pos[2], const SelArgs& a,
                                           const HybridList& h, int64_t u, int k0, int kl, int hh) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int ki = k0 + 32 * kt + kl;
    if (ki < h.nq) {
      const int64_t sl = k4_slot(a.c.k4_pages, a.cap_q, u, ki);
      uint32_t w[2 * kKB];
      load_codes_half<kKB>(w, a.c.kq + sl * (16 * kKB) + 8 * kKB * hh);
      const uint2 meta = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint32_t*>(a.c.kq_meta) +
                                                         sl * kMetaWords + 2 * hh);
      dequant_tile<kKB>(kr[kt], w, meta);
      pos[kt] = a.c.q_pos[sl];
    } else {
      int e = ki - h.nq;
      const uint16_t* row = nullptr;
      int p = kNoPos;
      if (e < h.nvl) {
        row = a.c.kvl + (u * a.cap_vl + e) * kD;
        p = a.c.vl_pos[u * a.cap_vl + e];
      } else if ((e -= h.nvl) < h.nwin) {
        p = a.t - h.nwin + e;
        row = a.c.kwin + (u * a.W + p % a.W) * kD;
      } else if (e - h.nwin < h.nst) {
        p = a.t;
        row = a.c.kstg + u * a.cap_stg * kD;
      }
      pos[kt] = p;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kr[kt][ks] = row ? ld16(row + 64 * hh + 8 * ks) : make_uint4(0, 0, 0, 0);
    }
  }
}

// S of row tile rt for the first kNT key tiles: two chains of eight k-steps
template <int kNT>
__device__ __forceinline__ void scores32(f32x16_t s[2], const uint4 kr[2][8], const half8_t q[8]) {
#pragma unroll
  for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt) s[kt] = mfma32(as_half8(kr[kt][ks]), q[ks], s[kt]);
}

__device__ __forceinline__ void load_q32(half8_t q[8], const QTile32& t, int lane) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) q[ks] = as_half8(t[ks][lane]);
}

// acc[kt][r] += sum over the 256 rows of the slice of exp2(c2 s - lse log2 e)
// for entry 32 kt + 8 (r / 4) + 4 h + r % 4 (this lane's share: its row
// lane % 32 of every row tile).  A software pipeline in steps: step ks of
// row tile rt issues the two MFMAs of k-step ks of tile rt + 1 (their query
// operand read from LDS two steps earlier), the read for two steps later,
// and the exponentials of four of tile rt's scores (key tile ks / 4, so the
// first key tile's chain, which ends first, is consumed first).  Each step
// is its own scheduling region, so the order holds.
__device__ __forceinline__ void chunk_refresh32(float acc[2][16], const uint4 kr[2][8], const QTile32* sq,
                                                const float* s_nl, float c2, int lane) {
  constexpr int kNRT = kRG / 32;               // row tiles of the 256-row slice
  const int rl = lane & 31;
  half8_t q[3];                                // query operands of steps s, s + 1, s + 2 (slot s mod 3)
  f32x16_t sc[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[kt][i] = 0.0f;
  q[0] = as_half8(sq[0][0][lane]);
  q[1] = as_half8(sq[0][1][lane]);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    q[(ks + 2) % 3] = as_half8(ks + 2 < 8 ? sq[0][ks + 2][lane] : sq[1][ks - 6][lane]);
    sc[0] = mfma32(as_half8(kr[0][ks]), q[ks % 3], sc[0]);
    sc[1] = mfma32(as_half8(kr[1][ks]), q[ks % 3], sc[1]);
  }
  float nl_c = s_nl[rl];
#pragma unroll
  for (int rt = 0; rt < kNRT; ++rt) {
    f32x16_t sn[2];
    const bool more = rt + 1 < kNRT;
    const float nl_n = more ? s_nl[32 * (rt + 1) + rl] : 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sn[kt][i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (more) {
        const int gs = 8 * (rt + 1) + ks;      // step index of tile rt + 1's k-step ks
        if (ks + 2 < 8) q[(gs + 2) % 3] = as_half8(sq[rt + 1][ks + 2][lane]);
        else if (rt + 2 < kNRT) q[(gs + 2) % 3] = as_half8(sq[rt + 2][ks - 6][lane]);
        sn[0] = mfma32(as_half8(kr[0][ks]), q[gs % 3], sn[0]);
        sn[1] = mfma32(as_half8(kr[1][ks]), q[gs % 3], sn[1]);
      }
      const int kt = ks >> 2, r0 = 4 * (ks & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[kt][r0 + e] += __builtin_amdgcn_exp2f(fmaf(sc[kt][r0 + e], c2, nl_c));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sc[kt] = sn[kt];
    nl_c = nl_n;
  }
}

// The masked form, for the few chunks holding entries that some rows must
// not see (positions past a row's own, and entries past the list, kNoPos):
// one row tile at a time, with the lane's 32 entry positions read from the
// wave's LDS list once.  Only the first kNT key tiles are computed (kNT = 1:
// the list's tail, at most 32 entries).
template <int kNT>
__device__ __forceinline__ void chunk_refresh32_masked(float acc[2][16], const uint4 kr[2][8], const QTile32* sq,
                                                       const float* s_nl, const int* s_prow, const int* kpos,
                                                       float c2, int lane) {
  constexpr int kNRT = kRG / 32;
  const int rl = lane & 31, hh = lane >> 5;
  int kp[2][16];
#pragma unroll
  for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) kp[kt][r] = kpos[32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3)];
#pragma unroll 1
  for (int rt = 0; rt < kNRT; ++rt) {
    f32x16_t sc[2];
    half8_t q[8];
    load_q32(q, sq[rt], lane);
    scores32<kNT>(sc, kr, q);
    const float nl = s_nl[32 * rt + rl];
    const int pr = s_prow[32 * rt + rl];
#pragma unroll
    for (int kt = 0; kt < kNT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kt][r], c2, nl));
        acc[kt][r] += (kp[kt][r] <= pr) ? p : 0.0f;
      }
  }
}

// Sum over the 32 row lanes of each half (lanes l, l ^ 16 by a row swap,
// then the 16 lanes of a row by DPP): lane l ends with the total of value
// v = l % 32 of the 32 acc[kt][r] (v = 16 kt + r).
__device__ __forceinline__ float reduce_scatter32(const float acc[2][16], int lane) {
  float t[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    // lanes with bit 4 clear keep kt = 0 and take the partner's kt = 0;
    // lanes with bit 4 set keep kt = 1 (the swap pairs the rows so that the
    // two results add to exactly that)
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[0][q]), __float_as_uint(acc[1][q]),
                                                    false, false);
    t[q] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  }
  return reduce_scatter16(t, lane & 15);
}

// Workgroup (x, unit) of the nwgr of a unit: its share of the unit's
// 64-entry chunks, [x nch / nwgr, (x + 1) nch / nwgr), wave w taking chunks
// w, w + 8, ... of it; while a chunk is computed, the next one's K4V4 codes
// are in flight (the other chunks, a few per unit, load in place).  The
// grid is one-dimensional: workgroup i runs on XCD i mod 8, so with
// xcd_group set the workgroups of a unit are numbered to share one XCD
// (its L2 then holds that unit's queries and codes only).  Row groups of
// 32 kNRT rows (256, or 512 when G * nb > 256, so that a chunk's codes are
// loaded and dequantised once per 512 rows) run one after another inside
// the workgroup, each adding its mass to the score entries it owns.
template <int kKB, int kNRT>
__global__ __launch_bounds__(kSThreads) void refresh_mass_kernel(SelArgs a) {
  constexpr int kRows = 32 * kNRT;
  __shared__ QStage32<kNRT> s_q;                            // 64 or 128 KB
  __shared__ float s_nl[kRows];                             // -lse * log2(e), -inf for padding
  __shared__ int s_prow[kRows];                             // row position, -1 for padding
  __shared__ int s_kpos[kSWaves][kChunk];                   // positions of the wave's chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kl = lane & 31, hh = lane >> 5;
  int idx = blockIdx.x;
  if (a.xcd_group) idx = (idx & 7) * (gridDim.x >> 3) + (idx >> 3);
  const int64_t u = idx / a.nwgr;
  const int xw = idx - static_cast<int>(u) * a.nwgr;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const HybridList h = hybrid_list(a, u);
  const int nch = (h.n + kChunk - 1) / kChunk;
  const int wg0 = static_cast<int>(static_cast<int64_t>(xw) * nch / a.nwgr) * kChunk;
  const int wg1 = min(h.n, static_cast<int>(static_cast<int64_t>(xw + 1) * nch / a.nwgr) * kChunk);
  if (wg0 >= wg1) return;                                   // the whole workgroup leaves
  // Entries every row sees (position at most t - nb + 1, the first row's):
  // when nb <= W + 1, the K4V4 slots and vertical lines (positions before
  // t - W) and the window's first nwin - nb + 2 positions (t - nwin + e).
  const int n_unmasked = (a.nb <= a.W + 1) ? h.nq + h.nvl + max(0, min(h.nwin, h.nwin - a.nb + 2)) : 0;
  float* sc_u = a.score + u * a.L;
  // the entry this lane owns after the reduction: v = lane % 32 of its half
  const int own = 32 * ((lane >> 4) & 1) + 8 * ((lane & 15) >> 2) + 4 * hh + (lane & 3);
  for (int rg = 0; rg < a.nrg; ++rg) {
    if (rg > 0) {
      // this workgroup's score updates of the last row group are visible to
      // its reloads below
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    KRaw32<kKB> raw;
    {
      const int k0 = wg0 + kChunk * wave;
      if (k0 < wg1 && k0 + kChunk <= h.nq) load_k4raw32(raw, a, u, k0, kl, hh);
    }
    uint4 qv[kStageIters];
    stage32_load<kNRT>(qv, a, b, h0, rg, 0);               // in flight with the LSE loads
    for (int rr = tid; rr < kRows; rr += kSThreads) {
      const int r = rg * kRows + rr;
      float nl = -INFINITY;
      int pr = -1;
      if (r < a.R) {
        const int g = r / a.nb, jq = r - g * a.nb;
        nl = -a.lse[(b * a.Hq + h0 + g) * a.nb + jq] * 1.4426950408889634f;
        pr = a.t - a.nb + 1 + jq;
      }
      s_nl[rr] = nl;
      s_prow[rr] = pr;
    }
    stage32_store<kNRT>(s_q, qv, 0);
#pragma unroll
    for (int part = 1; part < kRows / kRG; ++part) {
      stage32_load<kNRT>(qv, a, b, h0, rg, part);
      stage32_store<kNRT>(s_q, qv, part);
    }
    __syncthreads();
    for (int k0 = wg0 + kChunk * wave; k0 < wg1; k0 += kChunk * kSWaves) {
      uint4 kr[2][8];
      int kpos[2];
      if (k0 + kChunk <= h.nq) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          dequant_tile<kKB>(kr[kt], raw.codes[kt], raw.meta[kt]);
          kpos[kt] = raw.pos[kt];
        }
      } else {
        load_any32<kKB>(kr, kpos, a, h, u, k0, kl, hh);
      }
      // positions through LDS (both halves of a key tile hold the same entries)
      if (hh == 0) {
        s_kpos[wave][kl] = kpos[0];
        s_kpos[wave][32 + kl] = kpos[1];
      }
      const int op = s_kpos[wave][own];
      const bool owned = op >= 0 && op < a.L;
      // the running score of the owned position, loaded before the prefetch
      const float prev = owned ? sc_u[op] : 0.0f;
      const int k1 = k0 + kChunk * kSWaves;
      if (k1 < wg1 && k1 + kChunk <= h.nq) load_k4raw32(raw, a, u, k1, kl, hh);
      __builtin_amdgcn_sched_barrier(0);                    // keep the prefetch ahead
      float acc[2][16];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kt][r] = 0.0f;
      // the group's rows 256 at a time (one unrolled pass of 8 row tiles)
      if (k0 + kChunk <= n_unmasked) {
#pragma unroll 1
        for (int hf = 0; hf < kNRT / 8; ++hf)
          chunk_refresh32(acc, kr, &s_q[8 * hf], s_nl + kRG * hf, a.c2, lane);
      } else if (h.n - k0 <= 32) {
        // the list's tail: only the first key tile holds entries
#pragma unroll 1
        for (int hf = 0; hf < kNRT / 8; ++hf)
          chunk_refresh32_masked<1>(acc, kr, &s_q[8 * hf], s_nl + kRG * hf, s_prow + kRG * hf, s_kpos[wave],
                                    a.c2, lane);
      } else {
#pragma unroll 1
        for (int hf = 0; hf < kNRT / 8; ++hf)
          chunk_refresh32_masked<2>(acc, kr, &s_q[8 * hf], s_nl + kRG * hf, s_prow + kRG * hf, s_kpos[wave],
                                    a.c2, lane);
      }
      const float tot = reduce_scatter32(acc, lane);
      if (owned && k0 + own < h.n) sc_u[op] = prev + tot;
    }
  }
}

constexpr int kTopWaves = kTopThreads / 64;
constexpr int kKeysPerThread = 32;              // register-resident keys per thread
constexpr int kSeg = kKeysPerThread * kTopThreads;
constexpr int kSampleStride = 16;               // rows k = 0 and 16 form the sample

constexpr int kListMax = 4096;                  // keys of a confirmed bracket kept in LDS

constexpr int kSegWords = kSeg / 32;            // bitmap words of one segment (one per thread)

struct TopShared {
  int hist[256];
  int red[2][kTopWaves];
  uint32_t sel[4];
  uint64_t gt[kSegWords / 2];                   // bit p: position seg + p above the threshold
  uint64_t eq[kSegWords / 2];                   // bit p: equal to it; then: taken
  uint32_t list[kListMax];
};
static_assert(kSegWords == kTopThreads, "one bitmap word per thread");

// Sum of two ints over the workgroup (every thread gets both totals).
__device__ __forceinline__ void block_sum2(int& x, int& y, TopShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  y = wave_sum(y);
  if (lane == 0) {
    sh.red[0][wave] = x;
    sh.red[1][wave] = y;
  }
  __syncthreads();
  x = 0;
  y = 0;
#pragma unroll
  for (int w = 0; w < kTopWaves; ++w) {
    x += sh.red[0][w];
    y += sh.red[1][w];
  }
  __syncthreads();
}

// Exclusive prefix of x over the workgroup's threads, and the total.
__device__ __forceinline__ void block_excl_scan(int x, int& excl, int& total, TopShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x, lane);
  if (lane == 63) sh.red[1][wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopWaves; ++w) {
    const int v = sh.red[1][w];
    before += (w < wave) ? v : 0;
    tot += v;
  }
  excl = before + incl - x;
  total = tot;
  __syncthreads();
}

// Lane kLane of v takes the wave-uniform value x (v_writelane_b32 with an
// immediate lane select).  x is usually a ballot just written by a VALU
// compare; the wait states before the lane write let that SGPR write land
// (the compiler does not insert them for an asm statement).
template <int kLane>
__device__ __forceinline__ uint32_t write_lane(uint32_t v, uint32_t x) {
  asm volatile("s_nop 4\n\tv_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(x), "n"(kLane));
  return v;
}

// f(std::integral_constant<int, k>) for k = 0, 1, ..., in order.
template <typename F, int... K>
__device__ __forceinline__ void for_each_k(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}

// Add the wave's in-range lanes to an LDS histogram: the lanes that share
// the first in-range lane's bin add with one atomic (same-address LDS
// atomics serialise, and the bins crowd around the bulk of the scores); the
// others add one each (a loop over every distinct bin measured slower: the
// keys of a wave spread over many bins).
__device__ __forceinline__ void wave_hist_add(int* hist, uint32_t bin, bool in, int lane) {
  const uint64_t act = __ballot(in);
  if (act) {
    const int leader = __builtin_ctzll(act);
    const uint32_t lbin = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), leader));
    const uint64_t same = __ballot(in && bin == lbin);
    if (lane == leader) atomicAdd(&hist[lbin], __popcll(same));
    else if (in && bin != lbin) atomicAdd(&hist[bin], 1);
  }
}

// One histogram pass: keys in [lo, hi] counted into 256 bins of 2^shift keys
// in one LDS histogram.  Keys past the first segment are re-read.
__device__ __forceinline__ void hist_pass(const uint32_t keys[kKeysPerThread], const float* sc, int n,
                                          uint32_t lo, uint32_t hi, int shift, bool sample,
                                          TopShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 256) sh.hist[tid] = 0;
  __syncthreads();
  auto add = [&](uint32_t key, bool valid) {
    const bool in = valid && key >= lo && key <= hi;
    wave_hist_add(sh.hist, (key - lo) >> shift, in, lane);
  };
#pragma unroll
  for (int k = 0; k < kKeysPerThread; ++k) {
    if (sample && (k % kSampleStride) != 0) continue;
    add(keys[k], tid + k * kTopThreads < n);
  }
  if (!sample) {
    for (int i = kSeg + tid; i < n; i += kTopThreads) add(order_key(sc[i]), true);
  }
  __syncthreads();
}

// hist_pass over the compacted keys of a bracket (cnt <= kListMax).
__device__ __forceinline__ void hist_list(int cnt, uint32_t lo, uint32_t hi, int shift, TopShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 256) sh.hist[tid] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < cnt; i0 += kTopThreads) {
    const int i = i0 + tid;
    const uint32_t key = sh.list[max(min(i, cnt - 1), 0)];
    const bool in = i < cnt && key >= lo && key <= hi;
    wave_hist_add(sh.hist, (key - lo) >> shift, in, lane);
  }
  __syncthreads();
}

// Wave 0: the bin holding the kk-th largest counted key (bins scanned from
// the top): sel = {bin, rank inside the bin, count of the bin}.
__device__ __forceinline__ void find_bin(int kk, TopShared& sh) {
  const int lane = threadIdx.x & 63;
  int c[4], tot = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = sh.hist[255 - 4 * lane - e];        // lane l owns bins 255-4l .. 252-4l
    tot += c[e];
  }
  const int incl = wave_incl_scan(tot, lane);
  const int before = incl - tot;                  // keys in higher bins
  if (before < kk && incl >= kk) {
    int cum = before;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (cum + c[e] >= kk) {
        sh.sel[0] = static_cast<uint32_t>(255 - 4 * lane - e);
        sh.sel[1] = static_cast<uint32_t>(kk - cum);
        sh.sel[2] = static_cast<uint32_t>(c[e]);
        break;
      }
      cum += c[e];
    }
  }
}

__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
  return max(0, 32 - static_cast<int>(__clz(hi - lo)) - 8);
}

// One workgroup per unit: the n_vl-th largest score of the non-window prefix
// by a radix select over order-preserving integer keys, then flags and
// ascending indices, ties at the threshold taken from the lowest positions.
// Thread t holds the keys of positions t + 1024 k (k < 32) in registers.
// Before the radix passes, a 1/16 sample brackets the cut-off; one exact count
// checks the bracket (else the full range is used), so the passes then see
// a few hundred keys instead of all of them.
template <bool kCut>
__global__ __launch_bounds__(kTopThreads) void topk_kernel(SelArgs a) {
  __shared__ TopShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t u = blockIdx.x;
  float* sc = a.score + u * a.L;
  uint8_t* flag = a.vl_flag + u * a.L;
  int32_t* idx = a.vl_idx + u * a.n_vl;
  const int n = a.n_nw, k_want = a.n_vl;

  // The keys of the first segment (positions tid + 1024 k) into registers.
  // With several row groups their column-mass parts are folded into the
  // running score first (it is an output: the sums are written back), eight
  // positions at a time with every load of the eight in flight together;
  // positions past the first segment are folded in memory, by the thread
  // that reads them again below.  Loads use clamped indices, so they are
  // unconditional; only positions below n are written.
  uint32_t keys[kKeysPerThread];
  const bool fold = a.nrg > 1;
  if (n > 0) {
#pragma unroll
    for (int k0 = 0; k0 < kKeysPerThread; k0 += 8) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sc[min(tid + (k0 + e) * kTopThreads, n - 1)];
      if (fold) {
        for (int g = 0; g < a.nrg; ++g) {
          const float* cp = a.colpart + (static_cast<int64_t>(g) * a.U + u) * a.n_nw;
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = cp[min(tid + (k0 + e) * kTopThreads, n - 1)];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += p[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = tid + (k0 + e) * kTopThreads;
          if (i < n) sc[i] = v[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) keys[k0 + e] = order_key(v[e]);
    }
    if (fold) {
      for (int i = kSeg + tid; i < n; i += kTopThreads) {
        float v = sc[i];
        for (int g = 0; g < a.nrg; ++g) v += a.colpart[(static_cast<int64_t>(g) * a.U + u) * a.n_nw + i];
        sc[i] = v;
      }
    }
  }

  uint32_t thresh = 0;                 // keys > thresh are taken
  int take_eq = 0;                     // and this many keys == thresh, lowest positions first
  bool eq_all = true;                  // known: every key == thresh is taken, or none is
  if (k_want > 0) {
    uint32_t lo = 0, hi = 0;
    int kk = k_want;                   // rank of the target inside [lo, hi]
    int list_n = -1;                   // >= 0: the keys in [lo, hi] are in sh.list
    {
      // the key range [min, max]
      uint32_t kmin = 0xFFFFFFFFu, kmax = 0;
#pragma unroll
      for (int k = 0; k < kKeysPerThread; ++k) {
        if (tid + k * kTopThreads < n) {
          kmin = min(kmin, keys[k]);
          kmax = max(kmax, keys[k]);
        }
      }
      for (int i = kSeg + tid; i < n; i += kTopThreads) {
        const uint32_t key = order_key(sc[i]);
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
      kmin = wave_min(kmin);
      kmax = wave_max(kmax);
      if (lane == 0) {
        sh.red[0][wave] = static_cast<int>(kmin);
        sh.red[1][wave] = static_cast<int>(kmax);
      }
      __syncthreads();
      lo = 0xFFFFFFFFu;
      hi = 0;
      for (int w = 0; w < kTopWaves; ++w) {
        lo = min(lo, static_cast<uint32_t>(sh.red[0][w]));
        hi = max(hi, static_cast<uint32_t>(sh.red[1][w]));
      }
      __syncthreads();
    }

    // bracket from the sample (positions k = 0 mod 8 of the first segment)
    if (n <= kSeg && n >= 8192 && lo < hi) {
      const int shift = range_shift(lo, hi);
      hist_pass(keys, sc, n, lo, hi, shift, true, sh);
      // sampled positions: t + 1024 k with k % 8 == 0 and below n
      int ns = 0;
#pragma unroll
      for (int k = 0; k < kKeysPerThread; k += kSampleStride) ns += (k * kTopThreads < n) ? min(kTopThreads, n - k * kTopThreads) : 0;
      const float ts = static_cast<float>(k_want) * ns / n;
      const float dl = 4.0f * sqrtf(ts) + 16.0f;
      const int r_top = static_cast<int>(fmaxf(0.0f, ts - dl));            // sample keys surely above
      const int r_bot = static_cast<int>(fminf(static_cast<float>(ns), ts + dl));
      if (wave == 0) {
        // bins (from the top) where the cumulative sample count passes r_top and reaches r_bot
        int c[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = sh.hist[255 - 4 * lane - e];
          tot += c[e];
        }
        const int incl = wave_incl_scan(tot, lane);
        int cum = incl - tot;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b = 255 - 4 * lane - e;
          if (cum <= r_top && cum + c[e] > r_top) sh.sel[0] = static_cast<uint32_t>(b);
          if (cum < r_bot && cum + c[e] >= r_bot) sh.sel[1] = static_cast<uint32_t>(b);
          cum += c[e];
        }
      }
      __syncthreads();
      const uint32_t b_top = sh.sel[0], b_bot = sh.sel[1];
      __syncthreads();
      const uint32_t blo = (r_bot >= ns) ? lo : lo + (b_bot << shift);
      const uint32_t bhi = (r_top <= 0) ? hi : min(hi, lo + (b_top << shift) + ((1u << shift) - 1u));
      int c_above = 0;
      uint32_t inmask = 0;                         // bit k: key k lies in the bracket
#pragma unroll
      for (int k = 0; k < kKeysPerThread; ++k) {
        if (tid + k * kTopThreads < n) {
          c_above += keys[k] > bhi;
          inmask |= static_cast<uint32_t>(keys[k] >= blo && keys[k] <= bhi) << k;
        }
      }
      const int c_mine = __popc(inmask);
      int c_in = c_mine;
      block_sum2(c_above, c_in, sh);
      if (c_above < k_want && k_want <= c_above + c_in) {
        lo = blo;
        hi = bhi;
        kk = k_want - c_above;
        if (c_in <= kListMax) {
          // the bracket's keys into LDS, in thread order: the radix passes
          // below then read c_in keys instead of all n
          const int incl = wave_incl_scan(c_mine, lane);
          if (lane == 63) sh.red[0][wave] = incl;
          __syncthreads();
          int off = incl - c_mine;
          for (int w = 0; w < wave; ++w) off += sh.red[0][w];
#pragma unroll
          for (int k = 0; k < kKeysPerThread; ++k) {
            if ((inmask >> k) & 1u) sh.list[off++] = keys[k];
          }
          __syncthreads();
          list_n = c_in;
        }
      }
    }

    bool whole_bin = false;
    int eq_total = -1;                 // keys == lo once the range is one value
    while (lo < hi) {
      const int shift = range_shift(lo, hi);
      if (list_n >= 0) hist_list(list_n, lo, hi, shift, sh);
      else hist_pass(keys, sc, n, lo, hi, shift, false, sh);
      if (wave == 0) find_bin(kk, sh);
      __syncthreads();
      const uint32_t bin = sh.sel[0];
      kk = static_cast<int>(sh.sel[1]);
      const int cbin = static_cast<int>(sh.sel[2]);
      __syncthreads();
      const uint32_t nlo = lo + (bin << shift);
      const uint32_t nhi = min(hi, nlo + ((1u << shift) - 1u));
      if (kk == cbin && nlo > 0) {
        // every key of the bin is taken: the cut is just below it
        whole_bin = true;
        lo = nlo - 1;
        break;
      }
      lo = nlo;
      hi = nhi;
      if (lo == hi) eq_total = cbin;
    }
    thresh = lo;
    take_eq = whole_bin ? 0 : kk;
    eq_all = whole_bin || take_eq == eq_total;
  }

  // Flags and indices, segment by segment of kSeg positions.  The rows of the
  // coalesced layout (position seg + tid + 1024 k) leave their above- and
  // equal-to-threshold bits in LDS bitmaps, one 64-bit ballot per (row, wave)
  // covering 64 consecutive positions.  Thread t then owns bitmap word t
  // (positions seg + 32 t .. + 31): equal keys are ranked in position order
  // (only when some but not all of them are taken), and one scan of the
  // threads' taken counts gives each thread the index of its first taken
  // position.  Flags are written back in the coalesced layout.
  int base = 0;          // taken positions before the segment
  int eq_seen = 0;       // threshold-equal positions before the segment
  uint32_t tmin = 0xFFFFFFFFu;   // smallest taken key: the n_vl-th largest score
  // flags may go out four to a store when the unit's flag row is 4-byte aligned
  const bool flags4 = (reinterpret_cast<uintptr_t>(flag) & 3u) == 0;
  // segment 0 takes its keys from registers, later ones re-read them (the
  // first call is separate so that the register keys die with it)
  auto emit = [&](int seg, bool from_regs) {
    uint32_t* gt32 = reinterpret_cast<uint32_t*>(sh.gt);
    uint32_t* eq32 = reinterpret_cast<uint32_t*>(sh.eq);
    if (seg >= n) {
      // past the last candidate (window positions): nothing is taken
      const int end = min(seg + kSeg, a.L);
      if (flags4 && end == seg + kSeg) {
        for (int q = tid; q < kSeg / 4; q += kTopThreads) reinterpret_cast<uint32_t*>(flag + seg)[q] = 0u;
      } else {
        for (int i = seg + tid; i < end; i += kTopThreads) flag[i] = 0;
      }
      return;
    }
    if (k_want > 0) {
      // The ballot of row k (positions seg + 1024 k + 64 wave .. + 63, 64-bit
      // word 16 k + wave) goes into lanes 2k and 2k + 1 of one register, which
      // the wave then stores with one LDS write per lane.  When every
      // threshold-equal key is taken, or none is, one comparison per key
      // decides (key >= thresh, or key >= thresh + 1: finite scores never
      // reach the top key); otherwise the above and equal bitmaps are both
      // kept for the ranking of ties below.
      // v_writelane writes its lane whatever the exec mask, so the two forms
      // sit behind a branch on a wave-uniform (scalar) value: only the taken
      // side runs.
      const bool eq_all_u = __builtin_amdgcn_readfirstlane(eq_all ? 1 : 0) != 0;
      const uint32_t tcmp = thresh + (take_eq > 0 ? 0u : 1u);
      uint32_t wa = 0, wb = 0;
      if (eq_all_u) {
        for_each_k([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          const int i = seg + tid + k * kTopThreads;
          const uint32_t key = from_regs ? keys[k] : order_key(sc[min(i, n - 1)]);
          const bool t = i < n && key >= tcmp;
          if (kCut && t) tmin = min(tmin, key);
          // the flag is known here (no tie is ranked): one byte a key, 64
          // consecutive bytes a wave
          if (i < a.L) flag[i] = t ? 1 : 0;
          const uint64_t b = __ballot(t);
          wa = write_lane<2 * k>(wa, static_cast<uint32_t>(b));
          wa = write_lane<2 * k + 1>(wa, static_cast<uint32_t>(b >> 32));
        }, std::make_integer_sequence<int, kKeysPerThread>{});
      } else {
        for_each_k([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          const int i = seg + tid + k * kTopThreads;
          const uint32_t key = from_regs ? keys[k] : order_key(sc[min(i, n - 1)]);
          const bool valid = i < n;
          const bool g = valid && key > thresh, e = valid && key == thresh;
          if (kCut && g) tmin = min(tmin, key);
          const uint64_t bg = __ballot(g), be = __ballot(e);
          wa = write_lane<2 * k>(wa, static_cast<uint32_t>(bg));
          wa = write_lane<2 * k + 1>(wa, static_cast<uint32_t>(bg >> 32));
          wb = write_lane<2 * k>(wb, static_cast<uint32_t>(be));
          wb = write_lane<2 * k + 1>(wb, static_cast<uint32_t>(be >> 32));
        }, std::make_integer_sequence<int, kKeysPerThread>{});
      }
      const int w32 = 2 * (16 * (lane >> 1) + wave) + (lane & 1);
      gt32[w32] = wa;
      if (!eq_all_u) eq32[w32] = wb;
    } else if (tid < kSegWords / 2) {
      sh.gt[tid] = 0;
    }
    __syncthreads();
    // with eq_all the gt bitmap already holds every taken position
    uint32_t take = gt32[tid];
    if (!eq_all) {
      const uint32_t e = eq32[tid];
      // ties at the cut-off: the first take_eq equal keys in position order
      int ex_e, tot_e;
      block_excl_scan(__popc(e), ex_e, tot_e, sh);
      int want = take_eq - (eq_seen + ex_e);
      uint32_t m = e;
      while (want > 0 && m) {
        take |= m & (~m + 1u);
        m &= m - 1u;
        --want;
      }
      eq_seen += tot_e;
      if (kCut && (take & e)) tmin = min(tmin, thresh);
    }
    // this thread's taken positions, ascending, after those of the threads before it
    int ex_t, tot_t;
    block_excl_scan(__popc(take), ex_t, tot_t, sh);
    int o = base + ex_t;
    for (uint32_t m = take; m; m &= m - 1u) {
      if (o < k_want) idx[o] = seg + 32 * tid + __builtin_ctz(m);
      ++o;
    }
    base += tot_t;
    // the flags, unless the comparisons above already wrote them
    const bool flags_done = k_want > 0 && eq_all;
    if (!flags_done) {
      eq32[tid] = take;                    // the taken bitmap, for the flags
      __syncthreads();
      if (flags4 && seg + kSeg <= a.L) {
        // four positions a store: flag word q = positions seg + 4q .. + 3
#pragma unroll
        for (int k = 0; k < kKeysPerThread / 4; ++k) {
          const int q = tid + k * kTopThreads;
          const uint32_t x = (eq32[q >> 3] >> (4 * (q & 7))) & 0xFu;
          const uint32_t w = (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
          reinterpret_cast<uint32_t*>(flag + seg)[q] = w;
        }
      } else {
#pragma unroll 4
        for (int k = 0; k < kKeysPerThread; ++k) {
          const int pl = tid + k * kTopThreads;
          if (seg + pl < a.L) flag[seg + pl] = static_cast<uint8_t>((eq32[pl >> 5] >> (pl & 31)) & 1u);
        }
      }
    }
    __syncthreads();                     // before the next segment reuses the bitmaps
  };
  emit(0, true);
  for (int seg = kSeg; seg < a.L; seg += kSeg) emit(seg, false);
  if constexpr (kCut) {
    // the n_vl-th largest score: the smallest taken key (+inf when none)
    tmin = wave_min(tmin);
    if (lane == 0) sh.red[0][wave] = static_cast<int>(tmin);
    __syncthreads();
    if (tid == 0) {
      uint32_t m = 0xFFFFFFFFu;
      for (int w = 0; w < kTopWaves; ++w) m = min(m, static_cast<uint32_t>(sh.red[0][w]));
      a.cut[u] = (k_want > 0) ? key_value(m) : INFINITY;
    }
  }
}

}  // namespace

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t select_ws_bytes(const hq_dims& d, int32_t L_max) {
  const size_t units = static_cast<size_t>(d.B) * d.Hkv;
  const size_t R = static_cast<size_t>(d.Hq / d.Hkv) * 64;
  const size_t nrg = (R + kRG - 1) / kRG;
  // at least two chunks per wave: a streaming workgroup covers >= 1024 keys
  const size_t nwg = (static_cast<size_t>(L_max) + 2 * kChunk * kSWaves - 1) / (2 * kChunk * kSWaves);
  const size_t stats = units * nwg * R * sizeof(float2);
  const size_t part = nrg > 1 ? nrg * units * static_cast<size_t>(L_max) * sizeof(float) : 0;
  return round256(stats) + round256(part);
}

hipError_t launch_select(const hq_dims& d, const uint16_t* qbuf, int32_t nb, const uint16_t* k,
                         int32_t L, const float* lse_in, float* score, int32_t* vl_idx,
                         uint8_t* vl_flag, void* ws, hipStream_t s) {
  SelArgs a{};
  a.qbuf = qbuf;
  a.k = k;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.nb = nb;
  a.L = L;
  a.W = d.W;
  a.R = a.G * nb;
  a.n_nw = L > d.W ? L - d.W : 0;
  a.n_vl = n_vertical(d.rho, a.n_nw);
  a.c2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d.d)));
  const size_t units = static_cast<size_t>(d.B) * d.Hkv;
  a.U = static_cast<int32_t>(units);
  a.nrg = (a.R + kRG - 1) / kRG;
  // chunks per wave: 2 (one in flight while one is computed) up to 16, so
  // that large batches run a few workgroups per CU over time
  const int64_t chunks = static_cast<int64_t>(units) * ((L + kChunk - 1) / kChunk) * a.nrg;
  a.C = static_cast<int32_t>(std::min<int64_t>(16, std::max<int64_t>(2, (chunks + 8191) / 8192)));
  a.wg_keys = kChunk * kSWaves * a.C;
  a.nwg1 = (L + a.wg_keys - 1) / a.wg_keys;
  const size_t stats_bytes = units * a.nwg1 * a.R * sizeof(float2);
  char* w = reinterpret_cast<char*>(ws);
  a.stats = reinterpret_cast<float2*>(w);
  a.colpart = reinterpret_cast<float*>(w + round256(stats_bytes));
  a.score = score;
  a.vl_idx = vl_idx;
  a.vl_flag = vl_flag;
  const unsigned U = static_cast<unsigned>(units);
  const unsigned nrg = static_cast<unsigned>(a.nrg);
  if (lse_in) {
    a.lse = lse_in;
    a.lse_from_stats = 0;
  } else {
    hipLaunchKernelGGL(row_stats_kernel, dim3(a.nwg1, U, nrg), dim3(kSThreads), 0, s, a);
    a.lse = nullptr;
    a.lse_from_stats = 1;
  }
  if (a.n_nw > 0) {
    const unsigned nwg2 = static_cast<unsigned>((a.n_nw + a.wg_keys - 1) / a.wg_keys);
    hipLaunchKernelGGL(col_mass_kernel, dim3(nwg2, U, nrg), dim3(kSThreads), 0, s, a);
  }
  hipLaunchKernelGGL(topk_kernel<false>, dim3(U), dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_refresh(const hq_dims& d, const hq_cache& c, int32_t t, const uint16_t* qbuf,
                          int32_t nb, const float* lse, float* score, int32_t score_ld,
                          int32_t* vl_idx, uint8_t* vl_flag, float* cut, hipStream_t s) {
  SelArgs a{};
  a.qbuf = qbuf;
  a.lse = lse;
  a.score = score;
  a.vl_idx = vl_idx;
  a.vl_flag = vl_flag;
  a.cut = cut;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.nb = nb;
  a.L = score_ld;
  a.W = d.W;
  a.R = a.G * nb;
  a.n_nw = t > d.W ? t - d.W : 0;
  a.n_vl = n_vertical(d.rho, a.n_nw);
  a.c2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d.d)));
  a.c = c;
  a.t = t;
  a.cap_q = d.cap_q;
  a.cap_vl = d.cap_vl;
  a.cap_stg = d.cap_stg;
  const size_t units = static_cast<size_t>(d.B) * d.Hkv;
  a.U = static_cast<int32_t>(units);
  // 512 query rows a group when there are more than 256 (each chunk's codes
  // loaded and dequantised once per 512 rows)
  int rows = a.R > kRG ? 2 * kRG : kRG;
  a.nrg = (a.R + rows - 1) / rows;
  // a cache holding positions 0..t has t + 1 keys per unit: its chunks are
  // split evenly over nwgr workgroups, as many as fill one workgroup per CU
  // (the kernel's registers allow one), and at least eight chunks each
  const int64_t nk = static_cast<int64_t>(t) + 1;
  const int64_t nch = (nk + kChunk - 1) / kChunk;
  int64_t nwgr = std::max<int64_t>(1, std::min<int64_t>(kSelCUs / static_cast<int64_t>(units), nch / kSWaves));
  a.nwgr = static_cast<int32_t>(nwgr);
  const int64_t nwg_all = nwgr * static_cast<int64_t>(units);
  a.xcd_group = nwg_all % 8 == 0 ? 1 : 0;
  const unsigned nwg = static_cast<unsigned>(nwg_all);
  const int kb = kv_bits(d.k_bits);
  if (rows == kRG) {
    if (kb == 2) hipLaunchKernelGGL((refresh_mass_kernel<2, kRB / 2>), dim3(nwg), dim3(kSThreads), 0, s, a);
    else if (kb == 8) hipLaunchKernelGGL((refresh_mass_kernel<8, kRB / 2>), dim3(nwg), dim3(kSThreads), 0, s, a);
    else hipLaunchKernelGGL((refresh_mass_kernel<4, kRB / 2>), dim3(nwg), dim3(kSThreads), 0, s, a);
  } else {
    if (kb == 2) hipLaunchKernelGGL((refresh_mass_kernel<2, kRB>), dim3(nwg), dim3(kSThreads), 0, s, a);
    else if (kb == 8) hipLaunchKernelGGL((refresh_mass_kernel<8, kRB>), dim3(nwg), dim3(kSThreads), 0, s, a);
    else hipLaunchKernelGGL((refresh_mass_kernel<4, kRB>), dim3(nwg), dim3(kSThreads), 0, s, a);
  }
  const unsigned U = static_cast<unsigned>(units);
  a.nrg = 1;                       // the scores are complete: nothing to fold
  if (cut) hipLaunchKernelGGL(topk_kernel<true>, dim3(U), dim3(kTopThreads), 0, s, a);
  else hipLaunchKernelGGL(topk_kernel<false>, dim3(U), dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq

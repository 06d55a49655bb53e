// hq_select_vertical for gfx950: column-mass score and top-rho selection.
//
// The vertical-line score of a key position is the attention mass that the
// buffered FP16 queries put on it, accumulated over refreshes, and the lines
// are the top-rho positions of the non-window prefix (agihunt digest
// "HyQuant: Hybrid-Precision Quantization for LLM Attention", method
// paragraph; HyQuant README, Overview item 1).
//
// Rows of a unit are its R = G * nb buffered queries (row r = g * nb + jq, at
// position L - nb + jq).  Three kernels stream the unit's keys:
//   1. row_stats: per 256-key tile, the (max, sum of exp) of every row over
//      the tile's causal keys;  2. row_lse: merge the tiles -> natural-log
//      LSE per row (skipped when the caller passes it);  3. col_mass: per
//      256-key tile of the non-window prefix, sum over rows of
//      exp(tau q.k - lse) and add it to the running score.
// Both streaming passes compute S = K Q^T with v_mfma_f32_16x16x32_f16
// (A = 16 keys, B = 16 rows), each wave owning 64 keys for all row blocks.
// The sums use a fixed order (no float atomics) so reruns are bit-identical.
// 4. topk: one workgroup per unit finds the n_vl-th largest score by an
//    MSB-first radix select over order-preserving integer keys (per-wave LDS
//    histograms), then flags positions in ascending order (ties at the
//    threshold to the lower positions) and compacts them into vl_idx.
#include <hip/hip_runtime.h>
#include <math.h>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kTile = 256;          // keys per streaming workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 16 * 64;   // G <= 16, nb <= 64
constexpr int kTopThreads = 1024;

struct SelArgs {
  const uint16_t* qbuf;
  const uint16_t* k;
  const float* lse;                 // natural log, [B][Hq][nb]
  float* lse_out;                   // where row_lse writes
  float2* stats;                    // [U][ntiles][R] (max raw score, sum exp2)
  float* score;
  int32_t* vl_idx;
  uint8_t* vl_flag;
  int32_t Hq, Hkv, G, nb, L, W, R, ntiles, n_nw, n_vl;
  float c2;                         // log2(e) / sqrt(d)
};

__device__ __forceinline__ half8_t as_half8(uint4 v) { return __builtin_bit_cast(half8_t, v); }

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

__device__ __forceinline__ float4_t mfma(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// K operand of the wave's 64 keys: lane (key t, j) holds dims 32j..32j+31 of
// key k0 + 16x + t for x = 0..3, natural order (k-step kk = dims 32j+8kk..).
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

// B operand of one 16-row block: lane (row n, j) = row rb*16+n, dims 32j...
// Rows past the last one are clamped to it (their scores are masked), so the
// loads are unconditional and a prefetch stays in flight across the compute.
__device__ __forceinline__ void load_rows(half8_t qb[4], const SelArgs& a, int64_t b, int h0,
                                          int rb, int n, int j) {
  const int r = min(rb * 16 + n, a.R - 1);
  const int g = r / a.nb, jq = r - g * a.nb;
  const uint16_t* p = a.qbuf + ((b * a.Hq + h0 + g) * a.nb + jq) * kD + 32 * j;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qb[kk] = as_half8(ld16(p + 8 * kk));
}

__device__ __forceinline__ void scores(float4_t s[4], const uint4 kr[4][4], const half8_t qb[4]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    s[x] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s[x] = mfma(as_half8(kr[x][kk]), qb[kk], s[x]);
  }
}

// Pass 1: per (tile, unit), (max, sum exp2) of each row over the tile's keys.
__global__ __launch_bounds__(kThreads) void row_stats_kernel(SelArgs a) {
  __shared__ float2 s_st[kWaves][kMaxRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int64_t u = blockIdx.y;
  const int tile = blockIdx.x;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const int k0 = tile * kTile + 64 * wave;
  // every key of this wave precedes every buffered query: no causal mask
  const bool interior = k0 + 64 <= a.L - a.nb;
  const uint16_t* kunit = a.k + u * a.L * kD;
  uint4 kr[4][4];
  load_keys(kr, kunit, k0, a.L, n, j);
  const int nrb = (a.R + 15) / 16;
  half8_t qb[4];
  load_rows(qb, a, b, h0, 0, n, j);
  for (int rb = 0; rb < nrb; ++rb) {
    half8_t qn[4];                                   // next row block, loaded early
    load_rows(qn, a, b, h0, min(rb + 1, nrb - 1), n, j);
    __builtin_amdgcn_sched_barrier(0);               // keep the prefetch ahead of the compute
    float4_t s[4];
    scores(s, kr, qb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = qn[kk];
    const int r = rb * 16 + n;
    float v[16];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * x + e] = s[x][e];
    if (!interior) {
      // keys past the prefix or after the row's own position do not count
      const int prow = a.L - a.nb + (r - (r / a.nb) * a.nb);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 16 * x + 4 * j + e;
          if (!(key < a.L && key <= prow)) v[4 * x + e] = -INFINITY;
        }
    }
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, v[e]);
    mx = max_j(mx);
    float sum = 0.0f;
    if (mx != -INFINITY) {
      const float nmc = -mx * a.c2;
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f(fmaf(v[e], a.c2, nmc));
    }
    sum = sum_j(sum);
    if (j == 0 && r < a.R) s_st[wave][r] = make_float2(mx, sum);
  }
  __syncthreads();
  float2* out = a.stats + (u * a.ntiles + tile) * a.R;
  for (int r = tid; r < a.R; r += kThreads) {
    float mx = s_st[0][r].x;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_st[w][r].x);
    float sum = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        sum = fmaf(s_st[w][r].y, __builtin_amdgcn_exp2f((s_st[w][r].x - mx) * a.c2), sum);
    }
    out[r] = make_float2(mx, sum);
  }
}

// Merge the tiles' row statistics into the natural-log LSE of every row: one
// wave per row, lanes over tiles, a butterfly merge of (max, sum) pairs.
__global__ __launch_bounds__(kThreads) void row_lse_kernel(SelArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t u = blockIdx.y;
  if (r >= a.R) return;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const float2* st = a.stats + u * a.ntiles * a.R + r;
  float mx = -INFINITY, sum = 0.0f;
  for (int t = lane; t < a.ntiles; t += 64) {
    const float2 v = st[static_cast<int64_t>(t) * a.R];
    const float m2 = fmaxf(mx, v.x);
    if (m2 != -INFINITY)
      sum = sum * exp2f((mx - m2) * a.c2) + v.y * exp2f((v.x - m2) * a.c2);
    mx = m2;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(mx, o), os = __shfl_xor(sum, o);
    const float m2 = fmaxf(mx, om);
    if (m2 != -INFINITY) sum = sum * exp2f((mx - m2) * a.c2) + os * exp2f((om - m2) * a.c2);
    mx = m2;
  }
  if (lane == 0) {
    const int g = r / a.nb, jq = r - g * a.nb;
    a.lse_out[(b * a.Hq + h0 + g) * a.nb + jq] = (mx * a.c2 + log2f(sum)) * 0.69314718055994531f;
  }
}

// Pass 2: column mass of a 256-key tile of the non-window prefix.
__global__ __launch_bounds__(kThreads) void col_mass_kernel(SelArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int64_t u = blockIdx.y;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const int k0 = blockIdx.x * kTile + 64 * wave;
  if (k0 >= a.n_nw) return;
  // all 64 keys are non-window and precede every buffered query
  const bool interior = k0 + 64 <= min(a.n_nw, a.L - a.nb);
  const uint16_t* kunit = a.k + u * a.L * kD;
  uint4 kr[4][4];
  load_keys(kr, kunit, k0, a.L, n, j);
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  const float log2e = 1.4426950408889634f;
  const int nrb = (a.R + 15) / 16;
  auto row_lse = [&](int rb) {
    const int rc = min(rb * 16 + n, a.R - 1);
    const int g = rc / a.nb, jq = rc - g * a.nb;
    return a.lse[(b * a.Hq + h0 + g) * a.nb + jq];
  };
  half8_t qb[4];
  load_rows(qb, a, b, h0, 0, n, j);
  float lse_cur = row_lse(0);
  for (int rb = 0; rb < nrb; ++rb) {
    half8_t qn[4];                                   // next row block, loaded early
    const int rn = min(rb + 1, nrb - 1);
    load_rows(qn, a, b, h0, rn, n, j);
    const float lse_nxt = row_lse(rn);
    __builtin_amdgcn_sched_barrier(0);               // keep the prefetch ahead of the compute
    const int r = rb * 16 + n;
    const float nl2 = (r < a.R) ? -lse_cur * log2e : -INFINITY;   // padded rows add 0
    float4_t s[4];
    scores(s, kr, qb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = qn[kk];
    lse_cur = lse_nxt;
    if (interior) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[4 * x + e] += __builtin_amdgcn_exp2f(fmaf(s[x][e], a.c2, nl2));
    } else {
      const int rc = min(r, a.R - 1);
      const int prow = a.L - a.nb + (rc - (rc / a.nb) * a.nb);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = k0 + 16 * x + 4 * j + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(s[x][e], a.c2, nl2));
          acc[4 * x + e] += (key < a.n_nw && key <= prow) ? p : 0.0f;
        }
    }
  }
  // sum over the 16 row lanes of each key (butterfly: every lane gets the total)
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float v = acc[e];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    acc[e] = v;
  }
  if (n < 4) {
    float* sc = a.score + u * a.L;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (x != n) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + 16 * x + 4 * j + e;
        if (key < a.n_nw) sc[key] += acc[4 * x + e];
      }
    }
  }
}

// float -> unsigned key with the same order (-0 folded onto +0)
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t bits = __builtin_bit_cast(uint32_t, f);
  if (bits == 0x80000000u) bits = 0;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

constexpr int kTopWaves = kTopThreads / 64;
constexpr int kKeysPerThread = 32;              // register-resident keys per thread

// Block-wide exclusive prefix sum of one count per thread; the total goes to
// *total.  Two barriers.
__device__ __forceinline__ int block_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopWaves; ++w) {
    const int c = s_w[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// One workgroup per unit.  Radix select of the n_vl-th largest key over the
// unit's non-window scores (MSB first, 8-bit digits; each wave has its own
// LDS histogram so atomics only contend inside a wave), then a pass in which
// each thread owns 32 consecutive positions: flags, and ascending indices,
// with ties at the threshold taken from the lowest positions.
__global__ __launch_bounds__(kTopThreads) void topk_kernel(SelArgs a) {
  __shared__ int s_hist[kTopWaves][256];
  __shared__ int s_w[kTopWaves];
  __shared__ uint32_t s_sel[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t u = blockIdx.x;
  const float* sc = a.score + u * a.L;
  uint8_t* flag = a.vl_flag + u * a.L;
  int32_t* idx = a.vl_idx + u * a.n_vl;
  const int n = a.n_nw, k_want = a.n_vl;

  // The k_want-th largest key lies in [lo, hi]; each pass splits the range
  // into 256 bins of 2^shift keys, so the bins follow the keys' actual
  // spread (scores share their leading bits, fixed 8-bit digits would put
  // nearly all of them in one bin and serialise the LDS atomics).
  uint32_t thresh = 0;
  int take_eq = 0;
  uint32_t keys_first[kKeysPerThread];   // keys of the first 32 rows of 1024
#pragma unroll
  for (int k = 0; k < kKeysPerThread; ++k) keys_first[k] = 0;
  if (k_want > 0) {
    uint32_t* keys = keys_first;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0;
#pragma unroll
    for (int k = 0; k < kKeysPerThread; ++k) {
      const int i = tid + k * kTopThreads;
      keys[k] = i < n ? order_key(sc[i]) : 0u;
      if (i < n) {
        kmin = min(kmin, keys[k]);
        kmax = max(kmax, keys[k]);
      }
    }
    for (int i = kKeysPerThread * kTopThreads + tid; i < n; i += kTopThreads) {
      const uint32_t key = order_key(sc[i]);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o)));
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o)));
    }
    if (lane == 0) {
      s_hist[0][wave] = static_cast<int>(kmin);
      s_hist[1][wave] = static_cast<int>(kmax);
    }
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0;
    for (int w = 0; w < kTopWaves; ++w) {
      lo = min(lo, static_cast<uint32_t>(s_hist[0][w]));
      hi = max(hi, static_cast<uint32_t>(s_hist[1][w]));
    }
    __syncthreads();
    int kk = k_want;                      // rank of the target inside [lo, hi]
    while (lo < hi) {
      const uint32_t span = hi - lo;
      const int shift = max(0, 32 - __clz(span) - 8);
      for (int i = tid; i < kTopWaves * 256; i += kTopThreads) (&s_hist[0][0])[i] = 0;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kKeysPerThread; ++k) {
        const int i = tid + k * kTopThreads;
        if (i < n && keys[k] >= lo && keys[k] <= hi)
          atomicAdd(&s_hist[wave][(keys[k] - lo) >> shift], 1);
      }
      for (int i = kKeysPerThread * kTopThreads + tid; i < n; i += kTopThreads) {
        const uint32_t key = order_key(sc[i]);
        if (key >= lo && key <= hi) atomicAdd(&s_hist[wave][(key - lo) >> shift], 1);
      }
      __syncthreads();
      if (tid < 256) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kTopWaves; ++w) c += s_hist[w][tid];
        s_hist[0][tid] = c;
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 255-4l .. 252-4l (highest bins in lane 0)
        int c[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = s_hist[0][255 - 4 * lane - e];
          tot += c[e];
        }
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        const int before = incl - tot;           // keys in higher bins
        if (before < kk && incl >= kk) {
          int cum = before;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (cum + c[e] >= kk) {
              s_sel[0] = static_cast<uint32_t>(255 - 4 * lane - e);
              s_sel[1] = static_cast<uint32_t>(kk - cum);
              break;
            }
            cum += c[e];
          }
        }
      }
      __syncthreads();
      const uint32_t bin = s_sel[0];
      kk = static_cast<int>(s_sel[1]);
      __syncthreads();
      const uint32_t nlo = lo + (bin << shift);
      const uint32_t nhi = min(hi, nlo + ((1u << shift) - 1u));
      lo = nlo;
      hi = nhi;
    }
    thresh = lo;
    take_eq = kk;
  }

  // Flags and indices.  Positions are handled in segments of 32 rows of
  // 1024 (position seg + 1024 k + tid), so loads and flag stores coalesce.
  // Keys equal to the threshold are taken lowest position first; when all of
  // them are taken (no tie at the cut-off, the usual case) no ranking is
  // needed.  Indices are compacted with per-(row, wave) ballot counts and one
  // scan over them.
  __shared__ int s_cnt[kKeysPerThread * kTopWaves];
  __shared__ int s_tot;
  int base = 0;          // taken positions before the segment
  int eq_seen = 0;       // threshold-equal positions before the segment
  for (int seg = 0; seg < a.L; seg += kKeysPerThread * kTopThreads) {
    uint32_t gt = 0, eq = 0;            // bit k: row k of this thread
    if (k_want > 0) {
#pragma unroll
      for (int k = 0; k < kKeysPerThread; ++k) {
        const int i = seg + tid + k * kTopThreads;
        if (i < n) {
          const uint32_t key = seg == 0 ? keys_first[k] : order_key(sc[i]);
          gt |= static_cast<uint32_t>(key > thresh) << k;
          eq |= static_cast<uint32_t>(key == thresh) << k;
        }
      }
    }
    // how many threshold-equal keys the segment holds, in total
    int eq_tot;
    (void)block_scan(__popc(eq), s_w, &eq_tot);
    uint32_t take = gt;
    if (eq_seen + eq_tot <= take_eq) {
      take |= eq;                        // every equal key of the segment is taken
    } else {
      // ties at the cut-off: rank the equal keys in position order, row by row
      int seen = eq_seen;
      for (int k = 0; k < kKeysPerThread; ++k) {
        const uint64_t bal = __ballot((eq >> k) & 1u);
        if (lane == 0) s_w[wave] = __popcll(bal);
        __syncthreads();
        int off = 0, tot = 0;
        for (int w = 0; w < kTopWaves; ++w) {
          off += (w < wave) ? s_w[w] : 0;
          tot += s_w[w];
        }
        __syncthreads();
        const int rank = seen + off + __popcll(bal & ((1ull << lane) - 1ull));
        if (((eq >> k) & 1u) && rank < take_eq) take |= 1u << k;
        seen += tot;
      }
    }
    eq_seen += eq_tot;
    // per (row, wave) counts of taken positions, then their exclusive prefix
#pragma unroll
    for (int k = 0; k < kKeysPerThread; ++k) {
      const uint64_t bal = __ballot((take >> k) & 1u);
      if (lane == 0) s_cnt[k * kTopWaves + wave] = __popcll(bal);
    }
    __syncthreads();
    if (wave == 0) {
      // 512 counts in (row, wave) order = position order; 8 per lane
      int c[8], run = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        c[e] = s_cnt[8 * lane + e];
        run += c[e];
      }
      int incl = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      int acc = incl - run;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = c[e];
        s_cnt[8 * lane + e] = acc;
        acc += v;
      }
      if (lane == 63) s_tot = incl;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKeysPerThread; ++k) {
      const int i = seg + tid + k * kTopThreads;
      const bool t = (take >> k) & 1u;
      if (i < a.L) flag[i] = static_cast<uint8_t>(t);
      const uint64_t bal = __ballot(t);
      if (t) idx[base + s_cnt[k * kTopWaves + wave] + __popcll(bal & ((1ull << lane) - 1ull))] = i;
    }
    base += s_tot;
    __syncthreads();
  }
}

}  // namespace

size_t select_ws_bytes(const hq_dims& d, int32_t L_max) {
  const size_t units = static_cast<size_t>(d.B) * d.Hkv;
  const size_t R = static_cast<size_t>(d.Hq / d.Hkv) * 64;
  const size_t ntiles = (static_cast<size_t>(L_max) + kTile - 1) / kTile;
  const size_t stats = units * ntiles * R * sizeof(float2);
  const size_t lse = static_cast<size_t>(d.B) * d.Hq * 64 * sizeof(float);
  return (stats + 255) / 256 * 256 + lse;
}

hipError_t launch_select(const hq_dims& d, const uint16_t* qbuf, int32_t nb, const uint16_t* k,
                         int32_t L, const float* lse_in, float* score, int32_t* vl_idx,
                         uint8_t* vl_flag, void* ws, hipStream_t s) {
  SelArgs a;
  a.qbuf = qbuf;
  a.k = k;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.nb = nb;
  a.L = L;
  a.W = d.W;
  a.R = a.G * nb;
  a.ntiles = (L + kTile - 1) / kTile;
  a.n_nw = L > d.W ? L - d.W : 0;
  a.n_vl = n_vertical(d.rho, a.n_nw);
  a.c2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d.d)));
  const size_t units = static_cast<size_t>(d.B) * d.Hkv;
  const size_t stats_bytes = units * a.ntiles * a.R * sizeof(float2);
  a.stats = reinterpret_cast<float2*>(ws);
  a.lse_out = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (stats_bytes + 255) / 256 * 256);
  a.score = score;
  a.vl_idx = vl_idx;
  a.vl_flag = vl_flag;
  const unsigned U = static_cast<unsigned>(units);
  if (lse_in) {
    a.lse = lse_in;
  } else {
    hipLaunchKernelGGL(row_stats_kernel, dim3(a.ntiles, U), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(row_lse_kernel, dim3((a.R + kWaves - 1) / kWaves, U), dim3(kThreads), 0, s, a);
    a.lse = a.lse_out;
  }
  if (a.n_nw > 0) {
    const unsigned t2 = static_cast<unsigned>((a.n_nw + kTile - 1) / kTile);
    hipLaunchKernelGGL(col_mass_kernel, dim3(t2, U), dim3(kThreads), 0, s, a);
  }
  hipLaunchKernelGGL(topk_kernel, dim3(U), dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq

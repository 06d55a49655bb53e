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
//    MSB-first radix select over order-preserving integer keys in LDS
//    histograms, then flags positions in ascending order (ties at the
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
__device__ __forceinline__ void load_rows(half8_t qb[4], const SelArgs& a, int64_t b, int h0,
                                          int rb, int n, int j) {
  const int r = rb * 16 + n;
  if (r < a.R) {
    const int g = r / a.nb, jq = r - g * a.nb;
    const uint16_t* p = a.qbuf + ((b * a.Hq + h0 + g) * a.nb + jq) * kD + 32 * j;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = as_half8(ld16(p + 8 * kk));
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[kk] = as_half8(make_uint4(0, 0, 0, 0));
  }
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
  const uint16_t* kunit = a.k + u * a.L * kD;
  uint4 kr[4][4];
  load_keys(kr, kunit, k0, a.L, n, j);
  const int nrb = (a.R + 15) / 16;
  for (int rb = 0; rb < nrb; ++rb) {
    half8_t qb[4];
    load_rows(qb, a, b, h0, rb, n, j);
    float4_t s[4];
    scores(s, kr, qb);
    const int r = rb * 16 + n;
    const int prow = a.L - a.nb + (r % a.nb);
    float v[16];
    float mx = -INFINITY;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + 16 * x + 4 * j + e;
        const bool ok = key < a.L && key <= prow;
        v[4 * x + e] = ok ? s[x][e] : -INFINITY;
        mx = fmaxf(mx, v[4 * x + e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.0f;
    if (mx != -INFINITY) {
      const float nmc = -mx * a.c2;
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += exp2f(fmaf(v[e], a.c2, nmc));
    }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
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
      for (int w = 0; w < kWaves; ++w) sum = fmaf(s_st[w][r].y, exp2f((s_st[w][r].x - mx) * a.c2), sum);
    }
    out[r] = make_float2(mx, sum);
  }
}

// Merge the tiles' row statistics into the natural-log LSE of every row.
__global__ __launch_bounds__(kThreads) void row_lse_kernel(SelArgs a) {
  const int64_t u = blockIdx.x;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * a.G;
  const float2* st = a.stats + u * a.ntiles * a.R;
  for (int r = threadIdx.x; r < a.R; r += kThreads) {
    float mx = -INFINITY;
    for (int t = 0; t < a.ntiles; ++t) mx = fmaxf(mx, st[static_cast<int64_t>(t) * a.R + r].x);
    float sum = 0.0f;
    for (int t = 0; t < a.ntiles; ++t) {
      const float2 v = st[static_cast<int64_t>(t) * a.R + r];
      if (v.x != -INFINITY) sum = fmaf(v.y, exp2f((v.x - mx) * a.c2), sum);
    }
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
  const uint16_t* kunit = a.k + u * a.L * kD;
  uint4 kr[4][4];
  load_keys(kr, kunit, k0, a.L, n, j);
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  const float log2e = 1.4426950408889634f;
  const int nrb = (a.R + 15) / 16;
  for (int rb = 0; rb < nrb; ++rb) {
    half8_t qb[4];
    load_rows(qb, a, b, h0, rb, n, j);
    const int r = rb * 16 + n;
    const bool row_ok = r < a.R;
    const int g = row_ok ? r / a.nb : 0, jq = row_ok ? r - g * a.nb : 0;
    const float lse2 = row_ok ? a.lse[(b * a.Hq + h0 + g) * a.nb + jq] * log2e : 0.0f;
    const int prow = a.L - a.nb + jq;
    float4_t s[4];
    scores(s, kr, qb);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + 16 * x + 4 * j + e;
        const bool ok = row_ok && key < a.n_nw && key <= prow;
        const float p = exp2f(fmaf(s[x][e], a.c2, -lse2));
        acc[4 * x + e] += ok ? p : 0.0f;
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

// Block-wide exclusive prefix of a 0/1 flag (kTopThreads threads); returns
// the rank and writes the block total to *total.
__device__ __forceinline__ int block_rank(int f, int* s_w, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t bal = __ballot(f);
  const int in_w = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_w[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < kTopThreads / 64; ++w) {
    const int c = s_w[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + in_w;
}

__global__ __launch_bounds__(kTopThreads) void topk_kernel(SelArgs a) {
  __shared__ int s_hist[256];
  __shared__ int s_w[kTopThreads / 64];
  __shared__ uint32_t s_sel[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t u = blockIdx.x;
  const float* sc = a.score + u * a.L;
  uint8_t* flag = a.vl_flag + u * a.L;
  int32_t* idx = a.vl_idx + u * a.n_vl;
  const int n = a.n_nw, k_want = a.n_vl;

  uint32_t thresh = 0;          // key of the k_want-th largest (0: take nothing by key)
  int take_eq = 0;              // how many keys equal to thresh to take
  if (k_want > 0) {
    uint32_t prefix = 0, mask = 0;
    int k = k_want;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kTopThreads) s_hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kTopThreads) {
        const uint32_t key = order_key(sc[i]);
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 0xFFu], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns digits 252-4l .. 255-4l (highest digits in lane 0)
        int c[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = s_hist[255 - 4 * lane - e];
          tot += c[e];
        }
        int incl = tot;                       // inclusive prefix over lanes 0..l
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        const int before = incl - tot;        // keys with a higher digit than this lane's
        if (before < k && incl >= k) {
          int cum = before;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (cum + c[e] >= k) {
              s_sel[0] = static_cast<uint32_t>(255 - 4 * lane - e);
              s_sel[1] = static_cast<uint32_t>(k - cum);
              break;
            }
            cum += c[e];
          }
        }
      }
      __syncthreads();
      prefix |= s_sel[0] << shift;
      mask |= 0xFFu << shift;
      k = static_cast<int>(s_sel[1]);
      __syncthreads();
    }
    thresh = prefix;
    take_eq = k;
  }

  // flag positions in ascending order; equal keys: the lowest positions first
  int eq_seen = 0, taken = 0;
  for (int base = 0; base < a.L; base += kTopThreads) {
    const int i = base + tid;
    int gt = 0, eq = 0;
    if (k_want > 0 && i < n) {
      const uint32_t key = order_key(sc[i]);
      gt = key > thresh;
      eq = key == thresh;
    }
    int eq_tot;
    const int eq_rank = block_rank(eq, s_w, &eq_tot);
    const int take = gt || (eq && eq_seen + eq_rank < take_eq);
    int take_tot;
    const int t_rank = block_rank(take, s_w, &take_tot);
    if (i < a.L) flag[i] = static_cast<uint8_t>(take);
    if (take) idx[taken + t_rank] = i;
    eq_seen += eq_tot;
    taken += take_tot;
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
    hipLaunchKernelGGL(row_lse_kernel, dim3(U), dim3(kThreads), 0, s, a);
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

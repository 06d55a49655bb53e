// hq_quant_int8 and hq_prefill_attn kernels for gfx950.
//
// The prefill's fused hybrid-precision attention (agihunt digest "HyQuant:
// Hybrid-Precision Quantization for LLM Attention", method paragraph, the
// prefill sentences; HyQuant README, Overview item 2 and the ops listing of
// the repository layout, INT8-QK + FP16-PV prefill attention with window and
// vertical variants): causal attention of every prefix query in one online
// softmax.  A logit comes from symmetric per-token INT8 codes of q and k,
// except for the vertical lines and the query's own W-window, which use the
// FP16 values; P V is FP16 for every key.
//
// Layout of the work: one workgroup of four waves takes four (query head,
// 32-position block) pairs of one KV unit -- four heads of the GQA group at
// the same positions when G >= 4 -- so that every 64-key tile staged in LDS
// serves all of them.  Per wave S^T = K Q^T (keys as MFMA rows, the wave's 32
// queries as two 16-column blocks): v_mfma_i32_16x16x64_i8 on the codes (an
// exact int32 dot product, scaled by s_q s_k afterwards) or
// v_mfma_f32_16x16x32_f16 on the FP16 values; then O^T += V^T P^T with the
// FP16 instruction.  The INT8 operands of A and B take the same bytes of the
// same lane groups, so the dot product does not depend on the order in which
// the instruction walks them.  Tiles come in three kinds:
//   far   (every key at least W before every query of the workgroup): INT8
//         logits, vertical lines masked out (their FP16 turn comes below);
//   near  (the rest, up to the diagonal): FP16 and INT8 products both, the
//         choice made per (query, key); causal mask;
//   lines (the unit's vertical lines at least W before some query, gathered
//         from their ascending list): FP16 logits where key <= query - W.
#include <hip/hip_runtime.h>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kTile = 64;          // keys per tile
constexpr int kKP = kD + 8;        // K tile row pitch in halves (272-byte rows)
constexpr int kVP = kTile + 8;     // V^T row pitch in halves (144-byte rows, 16-byte aligned)
constexpr int kQW = 32;            // query positions per wave
constexpr int kPThreads = 256;

__device__ __forceinline__ half8_t as_h8(uint4 v) { return __builtin_bit_cast(half8_t, v); }

__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Symmetric INT8 of 128-element fp16 rows: scale = fp32(amax / 127), code =
// round-half-even(127 x / amax), decided in fp64 (127 x is exact there, and
// one correctly rounded division cannot cross a half-integer: the exact
// quotient is a ratio of 18- and 11-bit integers).  16 lanes per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void int8_rows_kernel(const uint16_t* x, int64_t rows,
                                                        int8_t* codes, float* scales) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  const bool ok = row < rows;
  const uint4 v = ok ? ld16(x + row * kD + 8 * part) : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax = fmaxf(amax, fabsf(h2f(static_cast<uint16_t>(w[i] & 0xFFFFu))));
    amax = fmaxf(amax, fabsf(h2f(static_cast<uint16_t>(w[i] >> 16))));
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  uint32_t c[2] = {0u, 0u};
  if (amax > 0.0f) {
    const double a = static_cast<double>(amax);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double xv = static_cast<double>(h2f(static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)))));
      const int q = static_cast<int>(rint(xv * 127.0 / a));
      c[j >> 2] |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * (j & 3));
    }
  }
  if (ok) {
    *reinterpret_cast<uint2*>(codes + row * kD + 8 * part) = make_uint2(c[0], c[1]);
    if (part == 0) scales[row] = static_cast<float>(static_cast<double>(amax) / 127.0);
  }
}

// ---------------------------------------------------------------------------
// The flagged positions of each unit, ascending, and their count.  One
// 1024-thread workgroup per unit; thread t takes a run of consecutive
// positions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void vl_list_kernel(const uint8_t* flag, int32_t L, int32_t* list,
                                                       int32_t* count) {
  __shared__ int s_w[16];
  const int64_t u = blockIdx.x;
  const uint8_t* f = flag + u * L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (L + 1023) / 1024;
  const int a0 = min(L, tid * per), a1 = min(L, a0 + per);
  int c = 0;
  for (int i = a0; i < a1; ++i) c += f[i] != 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  int off = incl - c;
  for (int w = 0; w < wave; ++w) off += s_w[w];
  int32_t* out = list + u * L;
  for (int i = a0; i < a1; ++i)
    if (f[i] != 0) out[off++] = i;
  if (tid == 1023) {
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += s_w[w];
    count[u] = tot;
  }
}

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------
typedef int32_t int4_t __attribute__((ext_vector_type(4)));

struct PrefillArgs {
  const uint16_t* q;       // [B][Hq][L][d]
  const uint16_t* k;       // [B][Hkv][L][d]
  const uint16_t* v;
  const int8_t* q8;        // [B][Hq][L][d]
  const float* sq;         // [B][Hq][L]
  const int8_t* k8;        // [B][Hkv][L][d]
  const float* sk;         // [B][Hkv][L]
  const uint8_t* flag;     // [B][Hkv][L] or null
  const int32_t* vl_list;  // [B][Hkv][L] ascending, or null
  const int32_t* vl_cnt;   // [B][Hkv]
  uint16_t* out;           // [B][Hq][L][d]
  float* lse;              // [B][Hq][L] or null
  int32_t L, W, Hq, Hkv, G, gw, pos_wg, n_qblk;
  float c2;                // log2(e) / sqrt(d)
};

constexpr int kCP = kD + 16;       // INT8 code tile row pitch in bytes

// Column of key k of a tile in the V^T rows: within each 32-key half kk the
// keys 4 g + r and 16 + 4 g + r (r = 0..3) sit side by side at 8 g + r and
// 8 g + 4 + r, which is the key order of one lane's P^T operand, so the
// matching V^T operand is a single 16-byte read.  Four consecutive keys 4 q
// .. 4 q + 3 stay consecutive, at vslot(4 q).
__host__ __device__ constexpr int vslot(int k) {
  return ((k >> 5) << 5) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// 16-byte aligned, so that 16-byte LDS accesses reach every field with the
// instruction's own offset (a 4-byte read pair can only reach 1 KiB)
struct alignas(16) TileBuf {
  uint16_t vt[kD][kVP];      // values, transposed: vt[dim][vslot(key)]
  int8_t kc[kTile][kCP];     // INT8 key codes
  alignas(16) float sk[kTile];     // key scales
  alignas(16) float bias[kTile];   // -inf at a vertical line (its FP16 turn comes later), else 0
  int32_t pos[kTile];        // key positions (-1: no key)
  uint8_t vl[kTile];         // vertical-line flags of the tile's keys
};

// Two tile buffers (the far tiles alternate between them, one barrier a
// tile) and the FP16 keys of the near and line tiles.
struct alignas(16) PrefillShared {
  TileBuf tb[2];
  uint16_t kf[kTile][kKP];
};

enum TileKind { kFar = 0, kNear = 1, kLines = 2 };

__device__ __forceinline__ float4_t mfma_i8(uint4 a, uint4 b, float4_t c_as_int) {
  const int4_t r = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(int4_t, a),
                                                         __builtin_bit_cast(int4_t, b),
                                                         __builtin_bit_cast(int4_t, c_as_int), 0, 0, 0);
  return __builtin_bit_cast(float4_t, r);
}

// The global half of staging a tile, into registers: thread t takes key t / 4
// (a quarter row: 32 dims of K, 32 codes) and, for V, keys 4 (t % 16) .. + 3
// at dims 8 (t / 16) .. + 7 (so the 16 lanes of one LDS store cycle write one
// V^T row's 16 four-key groups).
struct TileRegs {
  uint4 kf[4];
  uint4 kc[2];
  uint4 v[4];
  int32_t pos;       // threads < 64: key position of slot t (or -1)
  float sk;
  uint8_t vl;
};

__device__ __forceinline__ int slot_pos(int kind, int base, int n, int j, const int32_t* list) {
  if (j >= n) return -1;
  return kind == kLines ? list[base + j] : base + j;
}

__device__ __forceinline__ void load_tile(TileRegs& r, const PrefillArgs& a, int64_t u, int kind, int base,
                                          int n, const int32_t* list) {
  const int tid = threadIdx.x;
  if (tid < kTile) {
    const int p = slot_pos(kind, base, n, tid, list);
    r.pos = p;
    r.sk = (p >= 0 && kind != kLines) ? a.sk[u * a.L + p] : 0.0f;
    r.vl = (p >= 0 && a.flag && kind != kLines) ? a.flag[u * a.L + p] : 0;
  }
  const int j = tid >> 2, qt = tid & 3;
  const int p = slot_pos(kind, base, n, j, list);
  if (kind != kFar) {
    const uint16_t* src = a.k + (u * a.L + max(p, 0)) * kD + 32 * qt;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.kf[i] = p >= 0 ? ld16(src + 8 * i) : make_uint4(0, 0, 0, 0);
  }
  if (kind != kLines) {
    const int8_t* src = a.k8 + (u * a.L + max(p, 0)) * kD + 32 * qt;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      r.kc[i] = p >= 0 ? *reinterpret_cast<const uint4*>(src + 16 * i) : make_uint4(0, 0, 0, 0);
  }
  const int kq = tid & 15, oct = tid >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pe = slot_pos(kind, base, n, 4 * kq + e, list);
    r.v[e] = pe >= 0 ? ld16(a.v + (u * a.L + pe) * kD + 8 * oct) : make_uint4(0, 0, 0, 0);
  }
}

// A far tile holds 64 keys that all exist (it ends before the workgroup's
// first query), so its loads need no position test: each thread keeps its
// byte offsets inside a tile for the whole loop, and only the tile's base
// address, the same for every lane, moves from one tile to the next.
struct FarOffsets {
  uint32_t kc;   // INT8 codes: key tid / 4, bytes 32 (tid % 4) ..
  uint32_t v;    // values: key 4 (tid % 16), dims 8 (tid / 16) .. (3 more keys at +256 B)
};

__device__ __forceinline__ FarOffsets far_offsets() {
  const uint32_t tid = threadIdx.x;
  return {(tid >> 2) * kD + 32 * (tid & 3), ((tid & 15) * 4 * kD + 8 * (tid >> 4)) * 2};
}

__device__ __forceinline__ void load_far(TileRegs& r, const PrefillArgs& a, int64_t u, int base,
                                         const FarOffsets& o) {
  const int64_t row0 = u * a.L + base;
  const int tid = threadIdx.x;
  if (tid < kTile) {
    r.pos = base + tid;
    r.sk = a.sk[row0 + tid];
    r.vl = a.flag ? a.flag[row0 + tid] : 0;
  }
  const char* kc = reinterpret_cast<const char*>(a.k8 + row0 * kD) + o.kc;
  r.kc[0] = ld16(kc);
  r.kc[1] = ld16(kc + 16);
  const char* v = reinterpret_cast<const char*>(a.v + row0 * kD) + o.v;
#pragma unroll
  for (int e = 0; e < 4; ++e) r.v[e] = ld16(v + 2 * kD * e);
}

__device__ __forceinline__ void store_tile(TileBuf& sh, uint16_t (*kf)[kKP], const TileRegs& r, int kind) {
  const int tid = threadIdx.x;
  if (tid < kTile) {
    sh.pos[tid] = r.pos;
    sh.sk[tid] = r.sk;
    sh.vl[tid] = r.vl;
    sh.bias[tid] = r.vl ? -INFINITY : 0.0f;
  }
  const int j = tid >> 2, qt = tid & 3;
  if (kind != kFar) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&kf[j][32 * qt + 8 * i]) = r.kf[i];
  }
  if (kind != kLines) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&sh.kc[j][32 * qt + 16 * i]) = r.kc[i];
  }
  const int kq = tid & 15, oct = tid >> 4, c0 = vslot(4 * kq);
  const uint32_t w[4][4] = {{r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w}, {r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w},
                            {r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w}, {r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w}};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint2 lo = make_uint2(__builtin_amdgcn_perm(w[1][m], w[0][m], 0x05040100u),
                                __builtin_amdgcn_perm(w[3][m], w[2][m], 0x05040100u));
    const uint2 hi = make_uint2(__builtin_amdgcn_perm(w[1][m], w[0][m], 0x07060302u),
                                __builtin_amdgcn_perm(w[3][m], w[2][m], 0x07060302u));
    *reinterpret_cast<uint2*>(&sh.vt[8 * oct + 2 * m][c0]) = lo;
    *reinterpret_cast<uint2*>(&sh.vt[8 * oct + 2 * m + 1][c0]) = hi;
  }
}

struct WaveState {
  uint4 q8[2][2];       // INT8 query operand: column block cb, 64-dim step
  float qs2[2];         // query scale * c2 of this lane's query, per column block
  float4_t o[2][8];     // O^T: rows = dims 16 db + 4 g + r, column = query
  float m[2], l[2];     // running max (log2 units) and this lane's partial sum
};

// the maximum / sum over the four lanes g = 0..3 that share a query column
__device__ __forceinline__ float max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Online softmax of one column block's 16 values per lane (keys 16 kb + 4 g
// + r), whose logits in log2 units are scale * y (scale > 0, one per lane:
// the maximum is taken over y and each exponent is one fma), then its P^T
// operands for the two 32-key steps.
__device__ __forceinline__ void softmax_block(WaveState& ws, int cb, float (&y)[4][4], float scale,
                                              uint4 (&pb)[2]) {
  // a chain of three-operand maxima (v_max3): two new values per instruction
  float mx = fmaxf(y[0][0], y[0][1]);
#pragma unroll
  for (int e = 2; e < 16; e += 2) mx = fmaxf(fmaxf(mx, y[e / 4][e % 4]), y[e / 4][e % 4 + 1]);
  mx = max4(mx) * scale;
  const float m_new = fmaxf(ws.m[cb], mx);
  const float mu = m_new == -INFINITY ? 0.0f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(ws.m[cb] - mu);
  float ps = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      y[kb][r] = __builtin_amdgcn_exp2f(fmaf(y[kb][r], scale, -mu));
      ps += y[kb][r];
    }
  ws.l[cb] = ws.l[cb] * alpha + ps;
  ws.m[cb] = m_new;
  // rescale only when some query of the wave got a larger maximum
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int db = 0; db < 8; ++db) ws.o[cb][db] *= alpha;
  }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    half8_t h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = static_cast<_Float16>(y[2 * kk][r]);
      h[4 + r] = static_cast<_Float16>(y[2 * kk + 1][r]);
    }
    pb[kk] = __builtin_bit_cast(uint4, h);
  }
}

// O^T += V^T P^T; the V^T operand of dims 16 db + lane % 16 holds the same
// key order as the P^T operand (keys 32 kk + 4 g + r, then 32 kk + 16 + 4 g +
// r), 16 bytes at vslot(32 kk + 4 g) = 32 kk + 8 g
__device__ __forceinline__ void pv_tile(WaveState& ws, const TileBuf& sh, const uint4 (&pb)[2][2],
                                        int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const half8_t va = as_h8(*reinterpret_cast<const uint4*>(sh.vt[16 * db + (lane & 15)] + 32 * kk + 8 * g));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) ws.o[cb][db] = mfma16(va, as_h8(pb[cb][kk]), ws.o[cb][db]);
    }
}

// INT8 S^T of the tile for both column blocks: rows = keys 16 kb + lane % 16
__device__ __forceinline__ void s_int8(float4_t (&si)[2][4], const WaveState& ws, const TileBuf& sh,
                                       int lane) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int8_t* row = sh.kc[16 * kb + (lane & 15)] + 16 * (lane >> 4);
    const uint4 a0 = *reinterpret_cast<const uint4*>(row);
    const uint4 a1 = *reinterpret_cast<const uint4*>(row + 64);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_i8(a0, ws.q8[cb][0], acc);
      si[cb][kb] = mfma_i8(a1, ws.q8[cb][1], acc);
    }
  }
}

// FP16 S^T of the tile for both column blocks
__device__ __forceinline__ void s_fp16(float4_t (&sf)[2][4], const half8_t (&qf)[2][4],
                                       const uint16_t (*kf)[kKP], int lane) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint16_t* row = kf[16 * kb + (lane & 15)] + 8 * (lane >> 4);
    half8_t ar[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ar[kk] = as_h8(*reinterpret_cast<const uint4*>(row + 32 * kk));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma16(ar[kk], qf[cb][kk], acc);
      sf[cb][kb] = acc;
    }
  }
}

// A far tile: INT8 logits, vertical lines masked (bias), no causal mask.
__device__ __forceinline__ void far_tile(WaveState& ws, const TileBuf& sh, int lane) {
  const int g = lane >> 4;
  float4_t si[2][4];
  s_int8(si, ws, sh, lane);
  uint4 pb[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    float z[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float4_t s4 = *reinterpret_cast<const float4_t*>(&sh.sk[16 * kb + 4 * g]);
      const float4_t b4 = *reinterpret_cast<const float4_t*>(&sh.bias[16 * kb + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float acc = static_cast<float>(__builtin_bit_cast(int4_t, si[cb][kb])[r]);
        z[kb][r] = fmaf(acc, s4[r], b4[r]);      // logit / qs2 of key 16 kb + 4 g + r
      }
    }
    softmax_block(ws, cb, z, ws.qs2[cb], pb[cb]);
  }
  pv_tile(ws, sh, pb, lane);
}

// A near-diagonal tile (INT8 and FP16 logits chosen per element, causal) or
// a tile of gathered vertical lines (FP16, key <= query - W).
__device__ __forceinline__ void mixed_tile(WaveState& ws, const half8_t (&qf)[2][4], const TileBuf& sh,
                                           const uint16_t (*kf)[kKP], const PrefillArgs& a, int kind,
                                           int pos0, int lane) {
  const int g = lane >> 4;
  float4_t si[2][4], sf[2][4];
  if (kind == kNear) s_int8(si, ws, sh, lane);
  s_fp16(sf, qf, kf, lane);
  uint4 pb[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int p = pos0 + 16 * cb + (lane & 15);
    float z[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * kb + 4 * g + r;
        const int i = sh.pos[j];
        float zz;
        if (kind == kNear) {
          const float zi = sh.vl[j] ? -INFINITY
                                    : static_cast<float>(__builtin_bit_cast(int4_t, si[cb][kb])[r]) *
                                          ws.qs2[cb] * sh.sk[j];
          zz = (i < 0 || i > p) ? -INFINITY : (p - i < a.W ? sf[cb][kb][r] * a.c2 : zi);
        } else {
          zz = (i < 0 || i > p - a.W) ? -INFINITY : sf[cb][kb][r] * a.c2;
        }
        z[kb][r] = zz;
      }
    softmax_block(ws, cb, z, 1.0f, pb[cb]);
  }
  pv_tile(ws, sh, pb, lane);
}

__global__ __launch_bounds__(kPThreads, 2) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ PrefillShared sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hgroups = a.G / a.gw;
  const int64_t u = blockIdx.x / hgroups;            // unit (b, kv head): fastest, one XCD each
  const int hg = blockIdx.x % hgroups;
  const int64_t b = u / a.Hkv;
  const int h = static_cast<int>(u % a.Hkv) * a.G + hg * a.gw + wave % a.gw;
  const int qblk = a.n_qblk - 1 - static_cast<int>(blockIdx.y);   // the longest rows first
  const int m0 = qblk * a.pos_wg;
  const int pos0 = m0 + (wave / a.gw) * kQW;                      // this wave's first query
  const int pmax = min(a.L, m0 + a.pos_wg) - 1;                   // the workgroup's last query
  const int64_t bh = b * a.Hq + h;

  WaveState ws;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int p = pos0 + 16 * cb + (lane & 15);
    const bool ok = p < a.L;
    const int8_t* row = a.q8 + (bh * a.L + min(p, a.L - 1)) * kD + 16 * (lane >> 4);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      ws.q8[cb][c] = ok ? *reinterpret_cast<const uint4*>(row + 64 * c) : make_uint4(0, 0, 0, 0);
    // kept positive: an all-zero query row has all-zero codes, so its INT8
    // logits stay 0 = 0 * anything finite, and -inf stays -inf
    ws.qs2[cb] = fmaxf(ok ? a.sq[bh * a.L + p] * a.c2 : 0.0f, 1e-30f);
    ws.m[cb] = -INFINITY;
    ws.l[cb] = 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db) ws.o[cb][db] = (float4_t){0.f, 0.f, 0.f, 0.f};
  }

  // far tiles: every key at least W before every query of the workgroup;
  // the next tile's loads are in flight while this one is computed
  const int n_tiles = pmax / kTile + 1;
  const int n_far = min(n_tiles, max(0, (m0 - a.W + 1) / kTile));
  // (buffer t % 2 is read while buffer (t + 1) % 2 is filled: it was last
  // read in the previous iteration, before that iteration's barrier)
  TileRegs tr;
  const FarOffsets fo = far_offsets();
  if (n_far > 0) {
    load_far(tr, a, u, 0, fo);
    store_tile(sh.tb[0], sh.kf, tr, kFar);
  }
  __syncthreads();
  // (two tiles an iteration, so that each buffer's LDS addresses are the
  // instructions' constant offsets)
  auto far_step = [&](int t, const TileBuf& cur, TileBuf& nxt) {
    const bool more = t + 1 < n_far;
    if (more) load_far(tr, a, u, (t + 1) * kTile, fo);
    far_tile(ws, cur, lane);
    if (more) store_tile(nxt, sh.kf, tr, kFar);
    __syncthreads();
  };
  for (int t = 0; t < n_far; t += 2) {
    far_step(t, sh.tb[0], sh.tb[1]);
    if (t + 1 < n_far) far_step(t + 1, sh.tb[1], sh.tb[0]);
  }

  // near-diagonal tiles and the vertical lines, with the FP16 queries
  half8_t qf[2][4];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int p = pos0 + 16 * cb + (lane & 15);
    const bool ok = p < a.L;
    const uint16_t* row = a.q + (bh * a.L + min(p, a.L - 1)) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[cb][kk] = as_h8(ok ? ld16(row + 32 * kk) : make_uint4(0, 0, 0, 0));
  }
  for (int t = n_far; t < n_tiles; ++t) {
    const int base = t * kTile;
    load_tile(tr, a, u, kNear, base, min(kTile, a.L - base), nullptr);
    store_tile(sh.tb[0], sh.kf, tr, kNear);
    __syncthreads();
    if (base <= pos0 + kQW - 1) mixed_tile(ws, qf, sh.tb[0], sh.kf, a, kNear, pos0, lane);
    __syncthreads();
  }
  if (a.vl_list) {
    const int32_t* list = a.vl_list + u * a.L;
    const int cnt = a.vl_cnt[u];
    for (int base = 0; base < cnt; base += kTile) {
      const int first = list[base];
      if (first > pmax - a.W) break;      // ascending: nothing further is W before a query
      load_tile(tr, a, u, kLines, base, min(kTile, cnt - base), list);
      store_tile(sh.tb[0], sh.kf, tr, kLines);
      __syncthreads();
      if (first <= pos0 + kQW - 1 - a.W) mixed_tile(ws, qf, sh.tb[0], sh.kf, a, kLines, pos0, lane);
      __syncthreads();
    }
  }

  // normalise and store: lane holds dims 16 db + 4 g + r of query 16 cb + lane % 16
  const int g = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float lt = sum4(ws.l[cb]);
    const int p = pos0 + 16 * cb + (lane & 15);
    if (p < a.L) {
      const float inv = 1.0f / lt;
      uint16_t* dst = a.out + (bh * a.L + p) * kD + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        half2_t h01 = {static_cast<_Float16>(ws.o[cb][db][0] * inv), static_cast<_Float16>(ws.o[cb][db][1] * inv)};
        half2_t h23 = {static_cast<_Float16>(ws.o[cb][db][2] * inv), static_cast<_Float16>(ws.o[cb][db][3] * inv)};
        *reinterpret_cast<uint2*>(dst + 16 * db) =
            make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
      }
      if (a.lse && g == 0) a.lse[bh * a.L + p] = (ws.m[cb] + __log2f(lt)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

static size_t round256p(size_t x) { return (x + 255) / 256 * 256; }

size_t prefill_ws_bytes(const hq_dims& d, int32_t L_max) {
  const size_t L = static_cast<size_t>(L_max);
  const size_t rq = static_cast<size_t>(d.B) * d.Hq * L, rk = static_cast<size_t>(d.B) * d.Hkv * L;
  return round256p(rq * kD) + round256p(rq * 4) + round256p(rk * kD) + round256p(rk * 4) +
         round256p(rk * 4) + round256p(static_cast<size_t>(d.B) * d.Hkv * 4);
}

hipError_t launch_quant_int8(const uint16_t* x, int64_t rows, int8_t* codes, float* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(int8_rows_kernel, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, s, x,
                     rows, codes, scales);
  return hipGetLastError();
}

hipError_t launch_prefill(const hq_dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int32_t L, const uint8_t* vl_flag, uint16_t* out, float* lse, void* ws,
                          hipStream_t s) {
  if (L <= 0) return hipSuccess;
  const size_t Ls = static_cast<size_t>(L);
  const size_t rq = static_cast<size_t>(d.B) * d.Hq * Ls, rk = static_cast<size_t>(d.B) * d.Hkv * Ls;
  char* p = static_cast<char*>(ws);
  int8_t* q8 = reinterpret_cast<int8_t*>(p);
  p += round256p(rq * kD);
  float* sq = reinterpret_cast<float*>(p);
  p += round256p(rq * 4);
  int8_t* k8 = reinterpret_cast<int8_t*>(p);
  p += round256p(rk * kD);
  float* sk = reinterpret_cast<float*>(p);
  p += round256p(rk * 4);
  int32_t* list = reinterpret_cast<int32_t*>(p);
  p += round256p(rk * 4);
  int32_t* cnt = reinterpret_cast<int32_t*>(p);

  hipError_t e = launch_quant_int8(q, static_cast<int64_t>(rq), q8, sq, s);
  if (e != hipSuccess) return e;
  if ((e = launch_quant_int8(k, static_cast<int64_t>(rk), k8, sk, s)) != hipSuccess) return e;
  const int units = d.B * d.Hkv;
  if (vl_flag) {
    hipLaunchKernelGGL(vl_list_kernel, dim3(units), dim3(1024), 0, s, vl_flag, L, list, cnt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q8 = q8;
  a.sq = sq;
  a.k8 = k8;
  a.sk = sk;
  a.flag = vl_flag;
  a.vl_list = vl_flag ? list : nullptr;
  a.vl_cnt = vl_flag ? cnt : nullptr;
  a.out = out;
  a.lse = lse;
  a.L = L;
  a.W = d.W;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.gw = a.G % 4 == 0 ? 4 : (a.G % 2 == 0 ? 2 : 1);   // heads per workgroup, a divisor of G
  a.pos_wg = kQW * (4 / a.gw);
  a.n_qblk = (L + a.pos_wg - 1) / a.pos_wg;
  a.c2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(kD)));
  dim3 grid(static_cast<unsigned>(units * (a.G / a.gw)), static_cast<unsigned>(a.n_qblk));
  hipLaunchKernelGGL(prefill_attn_kernel, grid, dim3(kPThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq

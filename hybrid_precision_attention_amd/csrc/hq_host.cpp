// Host side of libhq: the extern "C" entry points declared in include/hq.h.
//
// Every check runs here, before anything is launched, so that a bad call
// returns an error without touching device memory (and can be exercised on a
// machine without a GPU).  Launch configuration and workspace sizing also
// live here; the kernels themselves are in the *.hip files.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "hq.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kMaxGroup = 16;      // query heads per KV head handled by one MFMA tile
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kDecodeWaves = 4;    // waves per decode workgroup
constexpr int kBlk = 32;           // tokens per decode block
constexpr int kMaxWG = 8 * kCUs;   // decode workgroups per launch, at most (short prefixes)
constexpr int kMaxPerCU = 1;       // decode workgroups per CU the byte plan aims at, at most (G <= 4, 4/8-bit)
constexpr int kMaxPerCUGen = 2;    // the same for the G > 4 scan and the 2-bit widths
constexpr int kMaxSplit = 128;     // decode workgroups per unit, at most (LDS of the final merge)
constexpr int kPartFloats = kPartFloatsPerRecord;
constexpr double kWgBytes = 384.0 * 1024;  // bytes one decode workgroup streams at small batch

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const hq_dims* d) {
  if (!d) return HQ_ERR_ARG;
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv != 0) return HQ_ERR_ARG;
  if (d->W < 0 || d->cap_q < 0 || d->cap_vl < 0 || d->cap_stg < 0) return HQ_ERR_ARG;
  if (!(d->rho >= 0.0 && d->rho <= 1.0)) return HQ_ERR_ARG;
  if (d->d != 128) return HQ_ERR_UNSUPPORTED;
  for (const int32_t b : {d->k_bits, d->v_bits})
    if (b != 0 && b != 2 && b != 4 && b != 8) return HQ_ERR_UNSUPPORTED;
  if (d->Hq / d->Hkv > kMaxGroup) return HQ_ERR_UNSUPPORTED;
  // several launches put the (sequence, KV head) units on a grid dimension
  // limited to 65535
  const int64_t units = static_cast<int64_t>(d->B) * d->Hkv;
  if (units > 65535) return HQ_ERR_ARG;
  return HQ_OK;
}

int check_cache(const hq_dims& d, const hq_cache* c) {
  if (!c) return HQ_ERR_ARG;
  const void* must[] = {c->kq, c->vq, c->kq_meta, c->vq_meta, c->q_pos, c->kvl, c->vvl,
                        c->vl_pos, c->kstg, c->vstg, c->n_q, c->n_vl, c->n_stg};
  for (const void* p : must)
    if (!p) return HQ_ERR_ARG;
  if (d.W > 0 && (!c->kwin || !c->vwin)) return HQ_ERR_ARG;
  // rows are read with 16-byte loads; positions and counters one int32 at a time
  const void* rows[] = {c->kq, c->vq, c->kq_meta, c->vq_meta, c->kvl, c->vvl, c->kstg, c->vstg};
  for (const void* p : rows)
    if (!aligned16(p)) return HQ_ERR_ALIGN;
  const void* words[] = {c->q_pos, c->vl_pos, c->n_q, c->n_vl, c->n_stg, c->k4_pages};
  for (const void* p : words)
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return HQ_ERR_ALIGN;
  // paged K4V4 slots come in whole 32-slot blocks
  if (c->k4_pages && d.cap_q % 32 != 0) return HQ_ERR_ARG;
  if (d.W > 0 && (!aligned16(c->kwin) || !aligned16(c->vwin))) return HQ_ERR_ALIGN;
  return HQ_OK;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int32_t n_vertical(double rho, int32_t n_nw) {
  if (n_nw <= 0 || !(rho >= 0.0 && rho <= 1.0)) return 0;
  return static_cast<int32_t>(floor(rho * static_cast<double>(n_nw) + 1e-6));
}

// Splits per unit for the decode: workgroups carry about equal bytes (160 per
// K4V4 token, 16 (k_bits + v_bits) + 32 at other widths, 512 per FP16 token).
// The launch is one round of long workgroups: each workgroup's start-up
// loads and its merge then come once per CU slot, not once per 384 KB (B = 32
// at L = 32K: 268 us against 283 us with up to eight workgroups per CU).  The
// G <= 4 scan at 4- and 8-bit widths keeps one workgroup per CU at every
// batch (side by side on one box: B = 16 133-134 against 137-138 us with two,
// K8V8 at B = 32 438 against 450 us, K4V4 at B = 32 the same); the G > 4 scan
// and the 2-bit widths go up to two (Qwen3-32B-shaped B = 32: 268 against
// 275 us with one).
static int64_t max_splits(int64_t units) {
  return std::min<int64_t>(kMaxSplit, cdiv(kMaxWG, units) + 3);
}

DecodePlan plan_decode(const hq_dims& d, int32_t L) {
  // Workgroups per unit: the whole launch carries about kWgBytes per
  // workgroup with one to eight workgroups per CU, and no workgroup has
  // fewer than one 32-token block per wave.  (The host estimates n_q and
  // n_vl from L and rho; the kernel reads the true counts.)
  const int64_t units = static_cast<int64_t>(d.B) * d.Hkv;
  const int32_t n_nw = std::max<int32_t>(0, L - d.W);
  const int32_t n_vl = std::min(n_vertical(d.rho, n_nw), d.cap_vl);
  const int64_t n_q = std::max<int32_t>(0, n_nw - n_vl);
  const int32_t n_win = std::min(d.W, L);
  const int64_t n_f = static_cast<int64_t>(n_vl) + n_win + d.cap_stg;
  const double q_tok = 16.0 * (kv_bits(d.k_bits) + kv_bits(d.v_bits)) + 32.0;
  const double per_unit = q_tok * static_cast<double>(n_q) + 512.0 * static_cast<double>(n_f);
  const double total = static_cast<double>(units) * per_unit;
  const bool one_per_cu = d.Hq / d.Hkv <= 4 && kv_bits(d.k_bits) != 2 && kv_bits(d.v_bits) != 2;
  const int cap_cu = one_per_cu ? kMaxPerCU : kMaxPerCUGen;
  const double per_cu = std::min<double>(cap_cu, std::max(1.0, std::floor(total / (kCUs * kWgBytes))));
  const double wg_bytes = std::max(total / (kCUs * per_cu), 1.0);
  const int64_t items = cdiv(n_q, kBlk) + cdiv(n_f, kBlk);
  int64_t ns = std::max<int64_t>(1, std::llround(per_unit / wg_bytes));
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, cdiv(items, kDecodeWaves)));
  ns = std::min<int64_t>(ns, max_splits(units));
  DecodePlan p;
  p.nsplit = static_cast<int>(ns);
  p.n_win = n_win;
  return p;
}

size_t decode_counter_bytes(const hq_dims& d) {
  const size_t units = static_cast<size_t>(d.B) * d.Hkv;
  return (units * 4 * kCounterStride + 255) / 256 * 256;
}

size_t decode_ws_bytes(const hq_dims& d, int32_t /*L_max*/) {
  // plan_decode never exceeds max_splits(units) splits per unit, whatever L is
  const int64_t units = static_cast<int64_t>(d.B) * d.Hkv;
  const size_t G = static_cast<size_t>(d.Hq / d.Hkv);
  return decode_counter_bytes(d) +
         static_cast<size_t>(units) * static_cast<size_t>(max_splits(units)) * G * kPartFloats *
             sizeof(float);
}

}  // namespace hq

using namespace hq;

extern "C" {

int hq_abi_version(void) { return 10; }

int32_t hq_n_vertical(double rho, int32_t n_nw) { return n_vertical(rho, n_nw); }

const char* hq_status_string(int status) {
  switch (status) {
    case HQ_OK: return "ok";
    case HQ_ERR_ARG: return "invalid argument (null pointer, shape or range)";
    case HQ_ERR_UNSUPPORTED: return "unsupported shape (head_dim 128, Hq/Hkv <= 16, code widths 2/4/8)";
    case HQ_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case HQ_ERR_CAPACITY: return "cache region capacity too small";
    case HQ_ERR_WORKSPACE: return "workspace missing or too small";
    case HQ_ERR_HIP: return "HIP launch or runtime error";
    case HQ_ERR_SCRATCH: return "request exceeds the static decode scratch (hq_decode_attn_noalloc)";
    default: return "unknown status";
  }
}

size_t hq_workspace_bytes(const hq_dims* dims, int op, int32_t L_max) {
  if (check_dims(dims) != HQ_OK || L_max < 0) return 0;
  if (op == HQ_OP_DECODE) return decode_ws_bytes(*dims, L_max);
  if (op == HQ_OP_SELECT) return L_max >= 1 ? select_ws_bytes(*dims, L_max) : 0;
  if (op == HQ_OP_PREFILL) return prefill_ws_bytes(*dims, L_max);
  return 0;
}

int hq_quant_pack(const hq_dims* dims, const uint16_t* k, const uint16_t* v, int32_t L,
                  const uint8_t* vl_flag, const hq_cache* cache, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (L < 0) return HQ_ERR_ARG;
  if (L > 0 && (!k || !v || !vl_flag)) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (L > 0 && (!aligned16(k) || !aligned16(v) || !aligned16(vl_flag))) return HQ_ERR_ALIGN;
  if (dims->cap_q < std::max(0, L - dims->W)) return HQ_ERR_CAPACITY;
  if (launch_quant_pack(*dims, k, v, L, vl_flag, *cache, stream) != hipSuccess) return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_append_merge(const hq_dims* dims, const hq_cache* cache, int32_t t,
                    const uint16_t* k_new, const uint16_t* v_new,
                    const uint8_t* evict_is_vl_or_null, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (t < 0 || !k_new || !v_new) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(k_new) || !aligned16(v_new)) return HQ_ERR_ALIGN;
  if (evict_is_vl_or_null && !aligned16(evict_is_vl_or_null)) return HQ_ERR_ALIGN;
  if (dims->cap_stg < 1) return HQ_ERR_CAPACITY;
  if (dims->cap_q < std::max(0, t - dims->W)) return HQ_ERR_CAPACITY;
  if (launch_append_merge(*dims, *cache, t, k_new, v_new, evict_is_vl_or_null, stream) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_decode_attn(const hq_dims* dims, const hq_cache* cache, int32_t L, const uint16_t* q,
                   uint16_t* out, float* lse_or_null, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (L < 0 || !q || !out) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(q) || !aligned16(out)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  if (!ws || ws_bytes < decode_ws_bytes(*dims, L)) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  const DecodePlan plan = plan_decode(*dims, L);
  if (launch_decode(*dims, *cache, L, plan, q, out, lse_or_null, ws, stream) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_decode_attn_noalloc(const hq_dims* dims, const hq_cache* cache, int32_t L, const uint16_t* q,
                           uint16_t* out, float* lse_or_null, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (L < 0 || !q || !out) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(q) || !aligned16(out)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  // the request must fit the static scratch: its counter area and the
  // records of this call's split plan
  const DecodePlan plan = plan_decode(*dims, L);
  const int64_t units = static_cast<int64_t>(dims->B) * dims->Hkv;
  const int64_t G = dims->Hq / dims->Hkv;
  const int64_t rec_bytes = units * plan.nsplit * G * kPartFloats * static_cast<int64_t>(sizeof(float));
  if (units > kScratchUnits || rec_bytes > static_cast<int64_t>(kScratchRecordBytes)) return HQ_ERR_SCRATCH;
  void* base = nullptr;
  if (decode_scratch(&base, stream) != hipSuccess) return HQ_ERR_HIP;
  if (launch_decode_at(*dims, *cache, L, plan, q, out, lse_or_null, static_cast<int32_t*>(base),
                       reinterpret_cast<float*>(static_cast<char*>(base) + kScratchCounterBytes),
                       stream) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_select_vertical(const hq_dims* dims, const uint16_t* qbuf, int32_t nb, const uint16_t* k,
                       int32_t L, const float* lse_or_null, float* score_inout,
                       int32_t* vl_idx, uint8_t* vl_flag, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (L < 1 || nb < 1 || nb > 64 || nb > L) return HQ_ERR_ARG;
  if (!qbuf || !k || !score_inout || !vl_flag) return HQ_ERR_ARG;
  const int32_t n_vl = n_vertical(dims->rho, std::max(0, L - dims->W));
  if (n_vl > 0 && !vl_idx) return HQ_ERR_ARG;
  if (!aligned16(qbuf) || !aligned16(k) || !aligned16(score_inout) || !aligned16(vl_flag))
    return HQ_ERR_ALIGN;
  if (vl_idx && !aligned16(vl_idx)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  if (!ws || ws_bytes < select_ws_bytes(*dims, L)) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  if (launch_select(*dims, qbuf, nb, k, L, lse_or_null, score_inout, vl_idx, vl_flag, ws,
                    stream) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_refresh_hybrid(const hq_dims* dims, const hq_cache* cache, int32_t t,
                      const uint16_t* qbuf, int32_t nb, const float* lse, float* score_inout,
                      int32_t score_ld, int32_t* vl_idx, uint8_t* vl_flag, float* cut_out,
                      hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (t < 0 || nb < 1 || nb > 64 || nb > t + 1 || score_ld < t + 1) return HQ_ERR_ARG;
  if (!qbuf || !lse || !score_inout || !vl_flag || !cut_out) return HQ_ERR_ARG;
  const int32_t n_vl = n_vertical(dims->rho, std::max(0, t - dims->W));
  if (n_vl > 0 && !vl_idx) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(qbuf) || !aligned16(lse) || !aligned16(score_inout) || !aligned16(vl_flag) ||
      !aligned16(cut_out))
    return HQ_ERR_ALIGN;
  if (vl_idx && !aligned16(vl_idx)) return HQ_ERR_ALIGN;
  if (launch_refresh(*dims, *cache, t, qbuf, nb, lse, score_inout, score_ld, vl_idx, vl_flag,
                     cut_out, stream) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_append_merge_scored(const hq_dims* dims, const hq_cache* cache, int32_t t,
                           const uint16_t* k_new, const uint16_t* v_new, const float* score,
                           int32_t score_ld, const float* cut, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (t < 0 || !k_new || !v_new || !score || !cut || score_ld < std::max(t, 1)) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(score) || !aligned16(cut))
    return HQ_ERR_ALIGN;
  if (dims->cap_stg < 1) return HQ_ERR_CAPACITY;
  if (dims->cap_q < std::max(0, t - dims->W)) return HQ_ERR_CAPACITY;
  if (launch_append_merge_scored(*dims, *cache, t, k_new, v_new, score, score_ld, cut, stream) !=
      hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_append_merge_ragged(const hq_dims* dims, const hq_cache* cache, const int32_t* t_seq,
                           int32_t t_max, const uint16_t* k_new, const uint16_t* v_new,
                           const uint8_t* evict_is_vl_or_null, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (t_max < 0 || !t_seq || !k_new || !v_new) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(t_seq) || !aligned16(k_new) || !aligned16(v_new)) return HQ_ERR_ALIGN;
  if (evict_is_vl_or_null && !aligned16(evict_is_vl_or_null)) return HQ_ERR_ALIGN;
  if (dims->cap_stg < 1) return HQ_ERR_CAPACITY;
  if (dims->cap_q < std::max(0, t_max - dims->W)) return HQ_ERR_CAPACITY;
  if (launch_append_merge(*dims, *cache, t_max, k_new, v_new, evict_is_vl_or_null, stream, t_seq) !=
      hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_decode_attn_ragged(const hq_dims* dims, const hq_cache* cache, const int32_t* L_seq,
                          int32_t L_max, const uint16_t* q, uint16_t* out, float* lse_or_null,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (L_max < 0 || !L_seq || !q || !out) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(L_seq) || !aligned16(q) || !aligned16(out)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  if (!ws || ws_bytes < decode_ws_bytes(*dims, L_max)) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  const DecodePlan plan = plan_decode(*dims, L_max);
  if (launch_decode(*dims, *cache, L_max, plan, q, out, lse_or_null, ws, stream, L_seq) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_decode_step(const hq_dims* dims, const hq_cache* cache, int32_t t, const uint16_t* k_new,
                   const uint16_t* v_new, const uint8_t* evict_is_vl_or_null, const uint16_t* q,
                   uint16_t* out, float* lse_or_null, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (t < 0 || !k_new || !v_new || !q || !out) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out)) return HQ_ERR_ALIGN;
  if (evict_is_vl_or_null && !aligned16(evict_is_vl_or_null)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  // after the step the K4V4 region may hold every position up to t - W
  if (static_cast<int64_t>(dims->cap_q) < static_cast<int64_t>(t) + 1 - dims->W) return HQ_ERR_CAPACITY;
  if (!ws || ws_bytes < decode_ws_bytes(*dims, t)) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  const DecodePlan plan = plan_decode(*dims, t);
  if (launch_decode(*dims, *cache, t, plan, q, out, lse_or_null, ws, stream, nullptr, k_new, v_new,
                    evict_is_vl_or_null) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_decode_step_ragged(const hq_dims* dims, const hq_cache* cache, const int32_t* t_seq,
                          int32_t t_max, const uint16_t* k_new, const uint16_t* v_new,
                          const uint8_t* evict_is_vl_or_null, const uint16_t* q, uint16_t* out,
                          float* lse_or_null, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (t_max < 0 || !t_seq || !k_new || !v_new || !q || !out) return HQ_ERR_ARG;
  if ((st = check_cache(*dims, cache))) return st;
  if (!aligned16(t_seq) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out))
    return HQ_ERR_ALIGN;
  if (evict_is_vl_or_null && !aligned16(evict_is_vl_or_null)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  if (static_cast<int64_t>(dims->cap_q) < static_cast<int64_t>(t_max) + 1 - dims->W) return HQ_ERR_CAPACITY;
  if (!ws || ws_bytes < decode_ws_bytes(*dims, t_max)) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  const DecodePlan plan = plan_decode(*dims, t_max);
  if (launch_decode(*dims, *cache, t_max, plan, q, out, lse_or_null, ws, stream, t_seq, k_new, v_new,
                    evict_is_vl_or_null) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_quant_int8(const uint16_t* x, int64_t rows, int8_t* codes, float* scales, hipStream_t stream) {
  if (rows < 0 || (rows > 0 && (!x || !codes || !scales))) return HQ_ERR_ARG;
  if (rows > (int64_t{1} << 36)) return HQ_ERR_ARG;
  if (rows > 0 && (!aligned16(x) || !aligned16(codes) || !aligned16(scales))) return HQ_ERR_ALIGN;
  if (launch_quant_int8(x, rows, codes, scales, stream) != hipSuccess) return HQ_ERR_HIP;
  return HQ_OK;
}

int hq_prefill_attn(const hq_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    int32_t L, const uint8_t* vl_flag_or_null, uint16_t* out, float* lse_or_null,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (L < 0) return HQ_ERR_ARG;
  if (L == 0) return HQ_OK;
  if (!q || !k || !v || !out) return HQ_ERR_ARG;
  // positions, and rows of one unit, stay inside int32 in the kernels
  if (static_cast<int64_t>(L) * 128 > (int64_t{1} << 31) - 1) return HQ_ERR_ARG;
  {
    // the query blocks (32, 64 or 128 positions by the GQA group) are a grid
    // dimension limited to 65535
    const int G = dims->Hq / dims->Hkv;
    const int gw = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
    const int64_t pos_wg = 32 * (4 / gw);
    if ((static_cast<int64_t>(L) + pos_wg - 1) / pos_wg > 65535) return HQ_ERR_UNSUPPORTED;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HQ_ERR_ALIGN;
  if (vl_flag_or_null && !aligned16(vl_flag_or_null)) return HQ_ERR_ALIGN;
  if (lse_or_null && !aligned16(lse_or_null)) return HQ_ERR_ALIGN;
  if (!ws || ws_bytes < prefill_ws_bytes(*dims, L)) return HQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return HQ_ERR_ALIGN;
  if (launch_prefill(*dims, q, k, v, L, vl_flag_or_null, out, lse_or_null, ws, stream) != hipSuccess)
    return HQ_ERR_HIP;
  return HQ_OK;
}

}  // extern "C"

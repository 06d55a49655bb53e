// Internal interface between the host entry points (hq_host.cpp) and the
// kernel launchers (*.hip).  Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "hq.h"

namespace hq {

// Decode split plan: how many workgroups scan the K4V4 region and the FP16
// region (vertical lines + window + staging) of each unit.
struct DecodePlan {
  int nsplit;         // workgroups per unit
  int n_win;          // valid window slots: min(W, L)
};

// Decode arrival counters: one int32 per unit, each on its own 128-byte line
// (the atomics of a unit's workgroups then do not queue behind those of the
// other units on one line).
constexpr int kCounterStride = 32;

DecodePlan plan_decode(const hq_dims& d, int32_t L);
size_t decode_ws_bytes(const hq_dims& d, int32_t L_max);
size_t decode_counter_bytes(const hq_dims& d);

size_t select_ws_bytes(const hq_dims& d, int32_t L_max);

hipError_t launch_quant_pack(const hq_dims& d, const uint16_t* k, const uint16_t* v,
                             int32_t L, const uint8_t* vl_flag, const hq_cache& c,
                             hipStream_t s);

hipError_t launch_append_merge(const hq_dims& d, const hq_cache& c, int32_t t,
                               const uint16_t* k_new, const uint16_t* v_new,
                               const uint8_t* evict_is_vl, hipStream_t s,
                               const int32_t* t_seq = nullptr);

hipError_t launch_decode(const hq_dims& d, const hq_cache& c, int32_t L,
                         const DecodePlan& plan, const uint16_t* q, uint16_t* out,
                         float* lse, void* ws, hipStream_t s, const int32_t* L_seq = nullptr,
                         const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr,
                         const uint8_t* evict_is_vl = nullptr);

// The decode with its arrival counters (one per unit, kCounterStride words
// apart, zero before the call, zero again after it) and partial records at
// the given device addresses.
hipError_t launch_decode_at(const hq_dims& d, const hq_cache& c, int32_t L, const DecodePlan& plan,
                            const uint16_t* q, uint16_t* out, float* lse, int32_t* counters,
                            float* part, hipStream_t s, const int32_t* L_seq = nullptr,
                            const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr,
                            const uint8_t* evict_is_vl = nullptr);

// Static scratch of hq_decode_attn_noalloc: one copy per GPU of
// kDecodeScratchBytes, the arrival counters of up to kScratchUnits units in
// its first kScratchCounterBytes and the partial records after them.
constexpr size_t kDecodeScratchBytes = size_t{8} << 20;
constexpr int kScratchUnits = 4096;
constexpr size_t kScratchCounterBytes = size_t{kScratchUnits} * 4 * kCounterStride;
constexpr size_t kScratchRecordBytes = kDecodeScratchBytes - kScratchCounterBytes;
constexpr int kPartFloatsPerRecord = 132;     // m, l, 2 pad, o[128]

// Device address of the current GPU's scratch: looked up once per device
// (with that device current) and its counter area cleared then, by a fill
// kernel on `s`; later calls return the kept address.
hipError_t decode_scratch(void** ptr, hipStream_t s);

hipError_t launch_select(const hq_dims& d, const uint16_t* qbuf, int32_t nb,
                         const uint16_t* k, int32_t L, const float* lse_in,
                         float* score, int32_t* vl_idx, uint8_t* vl_flag, void* ws,
                         hipStream_t s);

hipError_t launch_refresh(const hq_dims& d, const hq_cache& c, int32_t t, const uint16_t* qbuf,
                          int32_t nb, const float* lse, float* score, int32_t score_ld,
                          int32_t* vl_idx, uint8_t* vl_flag, float* cut, hipStream_t s);

hipError_t launch_append_merge_scored(const hq_dims& d, const hq_cache& c, int32_t t,
                                      const uint16_t* k_new, const uint16_t* v_new,
                                      const float* score, int32_t score_ld, const float* cut,
                                      hipStream_t s);

// Code width of a quantised region: 0 (unset) means 4.
size_t prefill_ws_bytes(const hq_dims& d, int32_t L_max);
hipError_t launch_quant_int8(const uint16_t* x, int64_t rows, int8_t* codes, float* scales,
                             hipStream_t s);
hipError_t launch_prefill(const hq_dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int32_t L, const uint8_t* vl_flag, uint16_t* out, float* lse, void* ws,
                          hipStream_t s);

inline int kv_bits(int32_t b) { return b == 0 ? 4 : b; }

// floor(rho * n_nw + 1e-6): size of the vertical-line set of n_nw candidates.
int32_t n_vertical(double rho, int32_t n_nw);

}  // namespace hq

// hq_quant_pack and hq_append_merge kernels for gfx950.
//
// Building the hybrid cache of a prefix (agihunt digest "HyQuant: Hybrid-
// Precision Quantization for LLM Attention", method and decode paragraphs;
// HyQuant README, Overview item 3): vertical-line tokens and the recent
// window stay FP16, every other non-window token is quantised to K4V4 and
// stored in ascending position.  New decode tokens are staged and then merged
// into the hybrid layout, the token leaving the window being quantised.
#include <hip/hip_runtime.h>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kChunk = 256;     // prefix positions per pack workgroup
constexpr int kPackThreads = 256;

struct PackArgs {
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* flag;
  hq_cache c;
  int32_t L, W, cap_q, cap_vl;
  int32_t k_bits, v_bits;           // code widths of the quantised region
};

// Number of nonzero bytes of w: bit 7 of each byte ends up set iff the byte
// is nonzero (its low seven bits carry into bit 7, or bit 7 was set).
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return __popc((((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u);
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// One workgroup per (chunk of 256 positions, unit).  Each workgroup counts the
// flagged non-window positions before its chunk, ranks its own positions, and
// then quantises (K4V4) or copies (vertical line, window) its tokens with
// eight threads per token: {K, V} x four groups of 32 elements.
__global__ __launch_bounds__(kPackThreads) void quant_pack_kernel(PackArgs a) {
  __shared__ int s_wave[4];
  __shared__ int s_kind[kChunk];
  __shared__ int s_slot[kChunk];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t u = blockIdx.y;
  const int L = a.L, W = a.W;
  const int n_nw = max(0, L - W);
  const int p0 = blockIdx.x * kChunk;
  const int p1 = min(L, p0 + kChunk);
  const uint8_t* flag = a.flag + u * L;

  // flagged non-window positions before this chunk: sixteen flags a load over
  // the 16-byte-aligned body of the row, single bytes for its head and tail
  int cnt = 0;
  const int lim = min(p0, n_nw);
  const int head = min(lim, static_cast<int>((16u - (reinterpret_cast<uintptr_t>(flag) & 15u)) & 15u));
  if (tid < head) cnt += flag[tid] != 0;
  const uint4* body = reinterpret_cast<const uint4*>(flag + head);
  const int nbody = (lim - head) >> 4;
  for (int i = tid; i < nbody; i += kPackThreads) {
    const uint4 w = body[i];
    cnt += nonzero_bytes(w.x) + nonzero_bytes(w.y) + nonzero_bytes(w.z) + nonzero_bytes(w.w);
  }
  for (int i = head + 16 * nbody + tid; i < lim; i += kPackThreads) cnt += flag[i] != 0;
  cnt = wave_sum(cnt);
  if (lane == 0) s_wave[wave] = cnt;
  __syncthreads();
  const int before = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
  __syncthreads();

  // rank of each flagged position inside the chunk
  const int p = p0 + tid;
  const int f = (p < p1 && p < n_nw && flag[p] != 0) ? 1 : 0;
  const uint64_t bal = __ballot(f);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(bal);
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < wave; ++w) wave_off += s_wave[w];
  const int chunk_total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
  const int flagged_before = before + wave_off + in_wave;   // raw, before p
  const int vl_before = min(flagged_before, a.cap_vl);      // stored VL tokens before p

  int kind = 0, slot = 0;                                   // 0 none, 1 K4, 2 VL, 3 window
  if (p < p1) {
    if (p >= n_nw) {
      kind = 3;
      slot = p % W;
    } else if (f && flagged_before < a.cap_vl) {
      kind = 2;
      slot = flagged_before;
      a.c.vl_pos[u * a.cap_vl + slot] = p;
    } else {
      kind = 1;
      slot = p - vl_before;
      a.c.q_pos[k4_slot(a.c.k4_pages, a.cap_q, u, slot)] = p;
    }
  }
  s_kind[tid] = kind;
  s_slot[tid] = slot;
  if (p1 == L && tid == 0) {          // the last chunk of the unit sets the counters
    const int n_vl = min(before + chunk_total, a.cap_vl);
    a.c.n_vl[u] = n_vl;
    a.c.n_q[u] = n_nw - n_vl;
    a.c.n_stg[u] = 0;
  }
  __syncthreads();

  const int sub = tid & 7;            // {K,V} x group
  const int kv = sub >> 2, g = sub & 3;
  const int ntok = p1 - p0;
  constexpr int kStride = kPackThreads / 8;   // tokens per pass
  // the group of token t of the chunk (64 bytes), as 16 words
  auto load = [&](int t, uint32_t (&x)[16]) {
    const uint16_t* src = (kv ? a.v : a.k) + (u * L + p0 + t) * kD + g * kGroup;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w4 = ld16(src + 8 * i);
      x[4 * i + 0] = w4.x; x[4 * i + 1] = w4.y; x[4 * i + 2] = w4.z; x[4 * i + 3] = w4.w;
    }
  };
  uint32_t xn[16];
  if ((tid >> 3) < ntok) load(tid >> 3, xn);
  for (int tl = tid >> 3; tl < ntok; tl += kStride) {
    // this pass's group, and the next pass's in flight while it is stored
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = xn[i];
    if (tl + kStride < ntok) load(tl + kStride, xn);
    const int knd = s_kind[tl], sl = s_slot[tl];
    if (knd == 1) {
      const int bits = kv ? a.v_bits : a.k_bits;
      const int64_t fs = k4_slot(a.c.k4_pages, a.cap_q, u, sl);
      uint8_t* dst = (kv ? a.c.vq : a.c.kq) + fs * (kD * bits / 8) + g * (4 * bits);
      uint32_t* md = reinterpret_cast<uint32_t*>(kv ? a.c.vq_meta : a.c.kq_meta);
      quant_store_group_bits(bits, x, dst, &md[fs * kMetaWords + g]);
    } else {
      uint16_t* dst;
      if (knd == 2) dst = (kv ? a.c.vvl : a.c.kvl) + (u * a.cap_vl + sl) * kD + g * kGroup;
      else dst = (kv ? a.c.vwin : a.c.kwin) + (u * W + sl) * kD + g * kGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st16(dst + 8 * i, make_uint4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]));
    }
  }
}

struct MergeArgs {
  hq_cache c;
  int32_t k_bits, v_bits;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint8_t* evict_is_vl;
  // scored promotion (when score is set): the leaving token becomes a
  // vertical line when its running score reaches the unit's cut-off
  const float* score;               // [U][score_ld]
  const float* cut;                 // [U]
  int32_t score_ld;
  int32_t t, W, cap_q, cap_vl, cap_stg;
  const int32_t* t_seq;             // [B] per-sequence positions (ragged batch), or null
  int32_t Hkv;
};

// One wave per unit.  Lanes 0-15 carry the K row, lanes 16-31 the V row, 16
// bytes each.  The token leaving the window is either copied to the
// vertical-line region or quantised in place, four lanes per group.
__global__ __launch_bounds__(64) void append_merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x;
  const int64_t u = blockIdx.x;
  const bool mover = lane < 32;
  const int kv = (lane >> 4) & 1, part = lane & 15;
  const int W = a.W;
  // the new token's position: its sequence's own in a ragged batch (clamped
  // to [0, t_max]), else the batch's common one
  const int t = a.t_seq ? min(max(a.t_seq[u / a.Hkv], 0), a.t) : a.t;
  // Every address is known from the arguments, so all loads are issued
  // before any is used: the counters, the staged row, the ring slot the
  // staged token goes to (its old token is the evictee) and the new token.
  uint16_t* stg = (kv ? a.c.vstg : a.c.kstg) + u * a.cap_stg * kD + 8 * part;
  uint16_t* win = W > 0 ? (kv ? a.c.vwin : a.c.kwin) + (u * W + (t - 1 + W) % W) * kD + 8 * part
                        : nullptr;
  const uint16_t* src = (kv ? a.v_new : a.k_new) + u * kD + 8 * part;
  const int nstg = a.c.n_stg[u];
  const int nq = a.c.n_q[u];
  const int nvl = a.c.n_vl[u];
  const int ev = W > 0 ? t - 1 - W : t - 1;   // position of the token that would leave
  bool flag_vl = a.evict_is_vl && a.evict_is_vl[u] != 0;
  if (a.score && ev >= 0) flag_vl = a.score[u * a.score_ld + ev] >= a.cut[u];
  const uint4 staged = mover ? ld16(stg) : make_uint4(0, 0, 0, 0);
  const uint4 old = (mover && win) ? ld16(win) : make_uint4(0, 0, 0, 0);
  const uint4 fresh = mover ? ld16(src) : make_uint4(0, 0, 0, 0);

  if (nstg > 0) {
    // the staged token (position t - 1) enters the ring; the token it
    // replaces (t - 1 - W) leaves the window; with no window it leaves itself
    const uint4 evv = W > 0 ? old : staged;
    if (ev >= 0) {
      const bool to_vl = flag_vl && nvl < a.cap_vl;
      if (to_vl) {
        if (mover) st16((kv ? a.c.vvl : a.c.kvl) + (u * a.cap_vl + nvl) * kD + 8 * part, evv);
        if (lane == 0) {
          a.c.vl_pos[u * a.cap_vl + nvl] = ev;
          a.c.n_vl[u] = nvl + 1;
        }
      } else if (nq < a.cap_q) {
        // the row is already spread 8 values per lane, so a group is the
        // four lanes of a quad: K groups in lanes 0-15, V groups in 16-31
        // (lanes 32-63 quantise zeros and store nothing)
        const int bits = kv ? a.v_bits : a.k_bits;
        uint32_t meta;
        const uint64_t codes = quant_quad8(evv, bits, &meta);
        const int64_t slot = k4_slot(a.c.k4_pages, a.cap_q, u, nq);
        if (mover) {
          store_codes8((kv ? a.c.vq : a.c.kq) + slot * (kD * bits / 8) + bits * part, codes, bits);
          if ((part & 3) == 0)
            reinterpret_cast<uint32_t*>(kv ? a.c.vq_meta : a.c.kq_meta)[slot * kMetaWords + (part >> 2)] = meta;
        }
        if (lane == 0) {
          a.c.q_pos[slot] = ev;
          a.c.n_q[u] = nq + 1;
        }
      }
    }
    if (W > 0 && mover) st16(win, staged);
  }
  if (mover) st16(stg, fresh);
  if (lane == 0) a.c.n_stg[u] = 1;
}

}  // namespace

hipError_t launch_quant_pack(const hq_dims& d, const uint16_t* k, const uint16_t* v, int32_t L,
                             const uint8_t* vl_flag, const hq_cache& c, hipStream_t s) {
  PackArgs a{k, v, vl_flag, c, L, d.W, d.cap_q, d.cap_vl, kv_bits(d.k_bits), kv_bits(d.v_bits)};
  const int chunks = L > 0 ? (L + kChunk - 1) / kChunk : 1;
  dim3 grid(chunks, d.B * d.Hkv);
  hipLaunchKernelGGL(quant_pack_kernel, grid, dim3(kPackThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_merge(const hq_dims& d, const hq_cache& c, int32_t t,
                               const uint16_t* k_new, const uint16_t* v_new,
                               const uint8_t* evict_is_vl, hipStream_t s, const int32_t* t_seq) {
  MergeArgs a{c, kv_bits(d.k_bits), kv_bits(d.v_bits), k_new, v_new, evict_is_vl, nullptr, nullptr, 0,
              t, d.W, d.cap_q, d.cap_vl, d.cap_stg, t_seq, d.Hkv};
  hipLaunchKernelGGL(append_merge_kernel, dim3(d.B * d.Hkv), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_merge_scored(const hq_dims& d, const hq_cache& c, int32_t t,
                                      const uint16_t* k_new, const uint16_t* v_new,
                                      const float* score, int32_t score_ld, const float* cut,
                                      hipStream_t s) {
  MergeArgs a{c, kv_bits(d.k_bits), kv_bits(d.v_bits), k_new, v_new, nullptr, score, cut, score_ld,
              t, d.W, d.cap_q, d.cap_vl, d.cap_stg, nullptr, d.Hkv};
  hipLaunchKernelGGL(append_merge_kernel, dim3(d.B * d.Hkv), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq

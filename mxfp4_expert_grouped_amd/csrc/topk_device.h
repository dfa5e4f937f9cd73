// Top-k of a token by one wavefront, and the whole top-k + permutation of a
// few tokens by one 256-thread workgroup (device code shared by the routing
// kernels and the fused top-k / shared-expert gate_up launch).
//
// Router and top-k follow "Kimi K3 Tech Intro", section 4.3 ("Router (Top-16,
// ...)") and the 16-of-896 routing of the section 1 architecture table; the
// sigmoid score with renormalisation over the selected experts is the reading
// taken for the unspecified score function.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "mx_device.h"

namespace mxmoe {

constexpr int kMaxSlots = 16;

// k-th largest of one key per lane (keys of 0 never count): the threshold is
// built bit by bit from the top, counting candidates with a ballot.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t key, int k) {
  uint32_t th = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    th = __popcll(__ballot(key >= cand)) >= k ? cand : th;
  }
  return th;
}

__device__ __forceinline__ float order_key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

// Top-k of token t by one wave: ids ascending, w = sigmoid / sum sigmoid.
// Keys are order-preserving 32-bit images of the logits; slot i of lane l
// holds expert l + 64 i (slots past E hold key 0, which never counts).
// 1. The k-th largest of the 64 per-lane maxima is a lower bound L of the
//    k-th largest key (at least k lanes hold a key >= L).
// 2. Keys >= L are compacted in (slot, lane) = ascending expert order into
//    `cand` (LDS, 64 entries per wave); if more than 64 qualify, the full
//    16-slot search runs instead.
// 3. With one candidate per lane, the k-th largest key th is found by a
//    one-slot radix select; keys > th are taken and keys == th fill the
//    remaining places in ascending expert order (ties -> lower index).
// With s_ids non-null the chosen ids are also stored there (LDS, [t*k + j]).
static __device__ void topk_token(const FwdArgs& a, int t, int lane, uint2* cand, int* s_ids = nullptr) {
  // t is the same in every lane: saying so keeps the buffer resource in
  // scalar registers, so the 16 loads below go out together (a lane-varying
  // resource would get one waterfall loop with a full wait per load)
  t = __builtin_amdgcn_readfirstlane(t);
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc(a.logits + int64_t(t) * a.E, static_cast<short>(0), a.E * 4, 0x00020000);
  // every load is issued before any is used (offsets past the row read 0
  // through the resource's bound); slots past E get key 0
  uint32_t key[kMaxSlots];
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) key[i] = __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * (lane + 64 * i), 0, 0);
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i)
    key[i] = float_order_key(__builtin_bit_cast(float, key[i])) & (lane + 64 * i < a.E ? ~0u : 0u);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t lmax = 0;
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) lmax = max(lmax, key[i]);
  const uint32_t lo = wave_kth_largest(lmax, a.k);
  int ncand = 0;
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) ncand += __popcll(__ballot(key[i] >= lo));

  uint32_t ck;   // this lane's candidate key (0: none)
  int cidx;      // its expert index
  if (ncand <= 64) {
    int base = 0;
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i) {
      const bool c = key[i] >= lo;
      const uint64_t m = __ballot(c);
      if (c) cand[base + __popcll(m & lt_mask)] = make_uint2(key[i], uint32_t(lane + 64 * i));
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint2 cv = lane < ncand ? cand[lane] : make_uint2(0u, 0u);
    ck = cv.x;
    cidx = static_cast<int>(cv.y);
  } else {
    // many equal or clustered keys: radix select over all slots, then keep the
    // selected keys as candidates (at most k <= 32 of them)
    uint32_t th = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = th | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < kMaxSlots; ++i) cnt += __popcll(__ballot(key[i] >= c));
      th = cnt >= a.k ? c : th;
    }
    int need = a.k;
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i) need -= __popcll(__ballot(key[i] > th));
    int base = 0;
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i) {
      const uint64_t eq = __ballot(key[i] == th);
      const bool take = key[i] > th || (key[i] == th && __popcll(eq & lt_mask) < need);
      need -= min(need, __popcll(eq));
      const uint64_t m = __ballot(take);
      if (take) cand[base + __popcll(m & lt_mask)] = make_uint2(key[i], uint32_t(lane + 64 * i));
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint2 cv = lane < a.k ? cand[lane] : make_uint2(0u, 0u);
    ck = cv.x;
    cidx = static_cast<int>(cv.y);
  }
  const uint32_t th = wave_kth_largest(ck, a.k);
  const int need = a.k - __popcll(__ballot(ck > th));
  const uint64_t eq = __ballot(ck == th && ck != 0u);
  const bool take = ck > th || (ck == th && ck != 0u && __popcll(eq & lt_mask) < need);
  const uint64_t m = __ballot(take);
  const float sig = 1.0f / (1.0f + expf(-order_key_to_float(ck)));
  const float inv = 1.0f / group_sum<64>(take ? sig : 0.f);
  if (take) {
    const int pos = __popcll(m & lt_mask);  // candidates are in ascending expert order
    a.topk_ids[int64_t(t) * a.k + pos] = cidx;
    a.topk_w[int64_t(t) * a.k + pos] = sig * inv;
    if (s_ids) s_ids[t * a.k + pos] = cidx;
  }
}


// Exclusive scan of n <= 1024 ints held in LDS `v` (in place) by a 256-thread
// workgroup, four consecutive entries per thread; returns the total.  Every
// thread of the workgroup calls it.
__device__ __forceinline__ int block_exclusive_scan_256(int* v, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int x[4];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * tid + q;
    x[q] = i < n ? v[i] : 0;
    sum += x[q];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int woff = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = wave_tot[w];
    woff += w < wv ? t : 0;
    total += t;
  }
  int run = woff + incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * tid + q;
    if (i < n) v[i] = run;
    run += x[q];
  }
  __syncthreads();
  return total;
}

// Top-k of every token (T <= 32; one wave per token) and the permutation, by
// one 256-thread workgroup whose LDS scratch is `lds` (>= 14.5 KB): choices
// kept in LDS, per-expert token bitmasks by LDS atomics, one scan of the
// packed (rows | tiles << 16) per expert for row and tile starts, each pair's
// row = expert start + number of earlier tokens with that expert.  The tile
// list holds the routed experts' tiles of a.bm rows, then the shared experts'.
// x must already be quantised (the few-token router does it).
__device__ __forceinline__ void topk_permute_block256(const FwdArgs& a, uint8_t* lds) {
  uint2* cand = reinterpret_cast<uint2*>(lds);                 // [4][64]
  int* s_ids = reinterpret_cast<int*>(lds + 2048);             // [32 * 32]
  int* cnt = reinterpret_cast<int*>(lds + 2048 + 4096);        // [1024]
  uint32_t* mask = reinterpret_cast<uint32_t*>(lds + 2048 + 8192);  // [1024]
  int* wave_tot = reinterpret_cast<int*>(lds + 2048 + 12288);  // [8]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < a.E; e += 256) mask[e] = 0u;
  for (int t = wv; t < a.T; t += 4) topk_token(a, t, lane, cand + 64 * wv, s_ids);
  __syncthreads();
  const int npairs = a.T * a.k;
  for (int p = tid; p < npairs; p += 256) atomicOr(&mask[s_ids[p]], 1u << (p / a.k));
  __syncthreads();
  for (int e = tid; e < a.E; e += 256) {
    const int c = __popc(mask[e]);  // each token takes an expert at most once
    cnt[e] = c | (((c + a.bm - 1) / a.bm) << 16);
  }
  __syncthreads();
  const int total = block_exclusive_scan_256(cnt, a.E, wave_tot);  // ends with a barrier
  const int rtiles = total >> 16;
  const int nts = (a.T + a.bm - 1) / a.bm;  // tiles per shared expert
  for (int e = tid; e < a.E; e += 256) {
    const int c = __popc(mask[e]);
    const int ntile = (c + a.bm - 1) / a.bm;
    const int row0 = cnt[e] & 0xFFFF, tile0 = cnt[e] >> 16;
    a.offsets[e] = row0;
    a.counts[e] = c;
    a.ex_tiles[e] = tile0;
    for (int i = 0; i < ntile; ++i) {
      Tile tl;
      tl.ex = e;
      tl.row_begin = row0 + i * a.bm;
      tl.row_end = min(row0 + (i + 1) * a.bm, row0 + c);
      tl.pad = 0;
      a.tiles[tile0 + i] = tl;
    }
  }
  for (int i = tid; i < a.S * nts; i += 256) {
    const int sx = i / nts, j = i % nts;
    const int rb = a.Rr + sx * a.T;
    Tile tl;
    tl.ex = a.E + sx;
    tl.row_begin = rb + j * a.bm;
    tl.row_end = min(rb + (j + 1) * a.bm, rb + a.T);
    tl.pad = 0;
    a.tiles[rtiles + i] = tl;
  }
  for (int i = tid; i <= a.S; i += 256) a.ex_tiles[a.E + i] = rtiles + i * nts;
  if (tid == 0) {
    a.offsets[a.E] = a.Rr;
    *a.tile_count = rtiles + a.S * nts;
  }
  for (int p = tid; p < npairs; p += 256) {
    const int t = p / a.k, e = s_ids[p];
    const int row = (cnt[e] & 0xFFFF) + __popc(mask[e] & ((1u << t) - 1u));
    a.row_src[row] = p;
    a.row_token[row] = t;
    a.token_row[p] = row;
  }
}

}  // namespace mxmoe

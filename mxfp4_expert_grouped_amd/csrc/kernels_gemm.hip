// Grouped expert GEMMs on the gfx950 scaled MFMA (MXFP8 activations x MXFP4
// weights, fp32 accumulate): gate_up with a fused SwiGLU + MXFP8 re-quantise
// epilogue, and down.  "Kimi K3 Tech Intro", section 4.3 names the routed +
// shared experts and the A8W4 fused operators on MI355X; SwiGLU stands in for
// the SiTU activation the pages name without defining.
//
// Operand layout of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (established by probes
// in the exact-arithmetic regime):
//   * an FP4 operand lane (row r = lane%16, group g = lane/16) holds 32
//     consecutive logical k = 32g .. 32g+31 (16 bytes, element 2i in the low
//     nibble of byte i);
//   * an FP8 operand lane holds bytes j = 0..31 at logical k = 64(j/16) + 16g
//     + j%16, i.e. two 16-byte halves from logical blocks g/2 and 2 + g/2;
//   * the scale byte of lane (r, g) applies to logical block g (k = 32g..32g+31)
//     of row r; the result of lane l, register i is D[4(l/16)+i][l%16].
// MFMA step s covers K = 128s .. 128s+127 in natural order.  Weights arrive
// packed (moe_pack_mx4): the FP4 operands of the four 16-row blocks of a
// 64-row group and one step are 4 KB contiguous in lane order (1 KB per
// block), and their block scales one dword per lane, byte j holding the scale
// of block j for that lane's row and 32-wide K group.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "mx_device.h"
#include "topk_device.h"

namespace mxmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, v4f c, uint32_t sa, uint32_t sb) {
  // A: FP8 E4M3 (format 0), B: FP4 E2M1 (format 4); scale in byte 0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, static_cast<int>(sa), 0,
                                                          static_cast<int>(sb));
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ v8i make_a(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}
__device__ __forceinline__ v8i make_b(uint4 v) {
  v8i r;
  r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct-to-LDS copy of 16 (or 4) bytes per lane to LDS byte address
// lds + lane*16 (lane*4).  Issued as inline assembly so that the compiler's
// wait insertion does not guard later LDS reads against it: the kernel waits
// for its own copies with explicit counts.  M0 holds the LDS base; one wait
// state separates its write from the copy.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
// The same with the non-temporal hint, for data read exactly once (streamed
// expert weights): such loads sustain a higher HBM read rate on this part
// (about 7.1 against 6.2-6.3 TB/s for the plain form over an 8 GB buffer).
__device__ __forceinline__ void lds_copy16_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4_nt(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

// s_waitcnt with vmcnt = n, lgkmcnt and expcnt left unconstrained
#define PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

// ---------------------------------------------------------------------------
// Decode variant (tiles of at most 8 rows: a few tokens per expert), weight
// streaming.  A persistent grid of one 4-wave workgroup per CU walks the
// items (tile, 64-row packed weight group) round-robin, so at any time the
// grid streams neighbouring groups of a few experts (DRAM-page friendly;
// per-workgroup contiguous item ranges measured slower).  For gate_up a group
// is the gate and up rows of 32 h columns (interleaved packing), for down 64
// output columns.  With the K split (gate_up when there are fewer than 16
// items per wave, so that whole items would leave a long tail) wave w takes
// the K steps w, w+4, w+8, ... of every item of its workgroup (the four
// waves' current elements are 16 KB of contiguous weights); otherwise every
// wave takes whole items of its own, round-robin over all waves of the grid,
// and needs no cross-wave reduction.  A wave streams its steps through a
// private ring of kDsS LDS slots filled by direct-to-LDS copies,
// kDsS - 1 elements (one K step of one item) ahead, across item boundaries;
// the stream itself has no workgroup barrier.  After its last step of an
// item of gate_up a wave parks its partial sums in the slot it just consumed;
// between two barriers every wave sums the four quarters in wave order for a
// quarter of the output lanes and writes that part of the epilogue.  The
// MFMA's rows 8-15 repeat rows 0-7 and are discarded.  With many items (16+
// per wave) a down item covers two groups (128 output columns): one A copy
// then feeds eight MFMAs and the per-item work halves, through a shallower
// ring of larger slots.  With bf16 activations (twice the activation bytes
// per K step) a gate_up item covers two groups (64 h columns) as well.
// Slot (5632 bytes; 9984 for two-group items): weights 4 KB per group (the
// group's step, as packed) | A 8 rows x 128 B (16-byte chunks XOR-swizzled by
// (row/2)%4; only the tile's rows are copied) | A scales (dword per row, lanes
// 0-7) | weight scales per group (the packed dword of each lane, byte = block).
// ---------------------------------------------------------------------------
constexpr int kDsS = 7;                        // ring slots per wave (5632-byte slots)
constexpr int kDsSWide = 4;                    // ring slots per wave of wide items (9984 bytes)
constexpr int kDsS16 = 6;                      // ring slots per wave with bf16 activations (6400 bytes)
constexpr int kDsS16Wide = 3;                  // ... of wide items with bf16 activations (10752 bytes)
// LDS: four waves' rings, then per wave 8 x {ex, row_begin, row_end, group}
constexpr int kDsLds = 4 * kDsSWide * 9984 + 4 * 8 * 16;   // 160256 bytes (the larger ring)
__shared__ __attribute__((aligned(1024))) uint8_t ds_lds[kDsLds];

typedef int v4i_s __attribute__((ext_vector_type(4)));
typedef int v8i_s __attribute__((ext_vector_type(8)));

// Scalar loads of wave-uniform metadata, waited for inside the statement so
// that no vector-memory count is involved (the copies own vmcnt).
__device__ __forceinline__ v4i_s sload4(const void* p) {
  v4i_s v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ v8i_s sload8(const void* p) {
  v8i_s v;
  asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ int sload1(const void* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// A16 (the A16W4 variant: bf16 activations): the activation rows are bf16
// (8 rows x 256 bytes per K step, two copies, no activation scales), the
// weights are expanded in registers from FP4 to bf16 with their block scale
// (V_CVT_SCALEF32_PK_BF16_FP4) and multiplied on the bf16 MFMA
// (16x16x32: four per 16-row block and K step); h leaves the gate_up
// epilogue as bf16.  Six ring slots of 6400 bytes (three of 10752 bytes for
// two-group items).
// PH (phase) splits a few-token gate_up in two launches: PH = 1 is the top-k
// and permutation (workgroup 0, topk_permute_block256) together with the
// shared experts' items (every other workgroup: their tiles need no
// routing, only x, which the router launch has quantised), so the GPU
// streams the shared experts' weights while one workgroup routes; PH = 2 is
// then the routed experts' items alone.  PH = 0: every item of the tile list.
// Canonical (unpacked) weights [N][K/2] codes, [N][K/32] scales: the row
// offset of 16-row block jb of a packed group from the group's first row --
// gate_up groups pair the gate rows 32G .. 32G+31 with the up rows of the
// same h columns (d_ff further), down groups are 64 consecutive rows.
template <bool GU>
__device__ __forceinline__ int canon_row_off(int jb, int dff) {
  return GU ? (jb >> 1) * dff + 16 * (jb & 1) : 16 * jb;
}

template <bool GU, bool KSPLIT, bool WIDE, bool A16 = false, int PH = 0, bool CANON = false>
__global__ void __launch_bounds__(256, 1) k_gemm_stream(FwdArgs a) {
  static_assert(PH == 0 || GU, "the phases split the gate_up GEMM");
  if constexpr (PH == 1) {
    if (blockIdx.x == 0) {
      topk_permute_block256(a, ds_lds);
      return;
    }
  }
  // workgroups that walk items (all of them, or all but the routing one)
  const int wg_id = PH == 1 ? static_cast<int>(blockIdx.x) - 1 : static_cast<int>(blockIdx.x);
  const int wg_n = PH == 1 ? static_cast<int>(gridDim.x) - 1 : static_cast<int>(gridDim.x);
  // ring geometry: WIDE items (down only) cover two 64-row groups
  constexpr int GPI = WIDE ? 2 : 1;                 // packed groups per item
  constexpr int S = A16 ? (WIDE ? kDsS16Wide : kDsS16) : (WIDE ? kDsSWide : kDsS);  // ring slots per wave
  constexpr int NC = 4 * GPI + 2 + GPI;             // copies per element
  constexpr int SW = 0, SA = 4096 * GPI, SAS = SA + (A16 ? 2048 : 1024), SBS = A16 ? SAS : SAS + 256,
                SLOT = SBS + 256 * GPI;
  constexpr int WAVE = S * SLOT, FIFO = 4 * WAVE;
  static_assert(FIFO + 4 * 8 * 16 <= kDsLds, "ring does not fit");
  static_assert(!(WIDE && KSPLIT), "wide items take whole K");
  static_assert(GU || !KSPLIT, "the K split is for the gate_up GEMM");
  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane >> 4, r16 = lane & 15;
  const int K = GU ? a.d : a.dff;
  const int ns = K / 128;
  // K steps per item of wave w: w, w+4, ... (split) or all of them
  auto wsteps = [&](int w) { return KSPLIT ? (ns - w + 3) / 4 : ns; };
  const int nsw = wsteps(wu);
  const int ngrp = (GU ? a.dff / 32 : a.d / 64) / GPI;   // items per tile
  // shared experts' tiles (T rows each, in tiles of a.bm), last in the list
  const int nts_sh = (a.T + a.bm - 1) / a.bm;
  const int nitems = PH == 1 ? a.S * nts_sh * ngrp
                   : PH == 2 ? (sload1(a.tile_count) - a.S * nts_sh) * ngrp
                             : sload1(a.tile_count) * ngrp;
  // item walkers: workgroups (split) or single waves, round-robin.  With
  // many items per walker (16+) the items are first cut into 8 contiguous
  // ranges, one per XCD (workgroups go to the XCDs round-robin), and an
  // XCD's walkers take its range round-robin: the column groups of a tile
  // then share its activation rows in one L2 while every XCD streams
  // neighbouring weight groups.  With few items plain round-robin keeps the
  // whole grid on one contiguous stretch of weights, which measured faster.
  const int walkers = KSPLIT ? wg_n : wg_n * 4;
  const bool by_xcd = PH == 0 && nitems >= 16 * walkers;
  const int xcd = by_xcd ? wg_id & 7 : 0;
  const int xw = by_xcd ? wg_id >> 3 : wg_id;
  const int nxw = by_xcd ? wg_n >> 3 : wg_n;
  const int bid = KSPLIT ? xw : xw * 4 + wu;
  const int nwg = KSPLIT ? nxw : nxw * 4;
  const int per_xcd = by_xcd ? (nitems + 7) / 8 : nitems;
  const int xbase = xcd * per_xcd, xn = max(0, min(per_xcd, nitems - xbase));
  const int my_items = xn > bid ? (xn - bid + nwg - 1) / nwg : 0;
  const int nel = my_items * nsw;
  const int64_t wrows = GU ? 2 * a.dff : a.d;
  const int64_t wc_stride = wrows * (K / 2), ws_stride = packed_scale_bytes(wrows, K);
  const uint32_t wbase = lds_addr(ds_lds) + wu * WAVE;
  const uint8_t* wlds = ds_lds + wu * WAVE;
  // item metadata, issue side -> epilogue: every wave writes its own queue;
  // with the K split the epilogue reads wave 0's, the one wave with K steps
  // whenever K >= 128
  int* fifo = reinterpret_cast<int*>(ds_lds + FIFO) + wu * 32;
  const int* fifo_ep = reinterpret_cast<const int*>(ds_lds + FIFO) + (KSPLIT ? 0 : wu * 32);

  // ---- issue side: copy sources of the item being issued
  const uint8_t* w_src = nullptr;
  const uint8_t* bs_src = nullptr;
  const uint8_t* a_src = nullptr;
  const uint8_t* as_src = nullptr;
  const uint8_t* a16_src[2] = {nullptr, nullptr};
  const int ar = lane >> 3;                           // A row of this lane's copy
  const int achunk = (lane & 7) ^ ((ar >> 1) & 3);    // global chunk landing at chunk lane&7
  int cur_tile = -1, ex = 0, rb = 0, nr = 0;
  auto item_setup = [&](int il) {
    const int item = xbase + bid + il * nwg;
    const int tidx = item / ngrp, G = item - tidx * ngrp;
    const bool new_tile = tidx != cur_tile;
    if (new_tile) {
      cur_tile = tidx;
      if constexpr (PH == 1) {
        // shared tile tidx: expert tidx / nts_sh, its rows in tiles of a.bm
        const int sx = tidx / nts_sh, i = tidx - sx * nts_sh;
        ex = a.E + sx;
        rb = a.Rr + sx * a.T + i * a.bm;
        nr = min(a.bm, a.T - i * a.bm);
      } else {
        const v4i_s tl = sload4(a.tiles + tidx);      // ex, row_begin, row_end
        ex = tl.x;
        rb = tl.y;
        nr = tl.z - tl.y;
      }
    }
    if (lane < 4) fifo[(il & 7) * 4 + lane] = lane == 0 ? ex : lane == 1 ? rb : lane == 2 ? rb + nr : G;
    const bool shared = ex >= a.E;
    const int sidx = ex - a.E;
    const uint8_t* wc = GU ? (shared ? a.sgu_c + sidx * wc_stride : a.gu_c + ex * wc_stride)
                           : (shared ? a.sdn_c + sidx * wc_stride : a.dn_c + ex * wc_stride);
    const uint8_t* ws = GU ? (shared ? a.sgu_s + sidx * ws_stride : a.gu_s + ex * ws_stride)
                           : (shared ? a.sdn_s + sidx * ws_stride : a.dn_s + ex * ws_stride);
    if constexpr (CANON) {
      // canonical weights: lane 16g + r of a block's copy reads the 16 bytes
      // of its row that the packed order would hold (row r of the block, K
      // bytes 64 st + 16g ..), and lane 16jb + r of the scale copy the
      // dword of blocks 4st .. 4st+3 of row r of block jb
      const int64_t row0 = (GU ? 32 : 64) * int64_t(G) * GPI;
      w_src = wc + (row0 + r16) * (K / 2) + 16 * g;
      bs_src = ws + (row0 + canon_row_off<GU>(lane >> 4, a.dff) + r16) * (K / 32);
    } else {
      w_src = wc + int64_t(G) * GPI * ns * 4096 + 16 * lane;
      bs_src = ws + int64_t(G) * GPI * ns * 256 + 4 * lane;
    }
    if (!new_tile) return;
    // activation row of tile row r (rows past the end repeat the first); a
    // routed gate_up tile reads its eight row-token entries with one scalar
    // load (the workspace pads row_token by eight past the last routed row;
    // only rows < nr are used)
    v8i_s rt = {};
    if (GU && !shared) rt = sload8(a.row_token + rb);
    auto act_row = [&](int r) -> int {
      const int rr = r < nr ? r : 0;
      if (!GU) return rb + rr;
      if (shared) return rb - a.Rr - sidx * a.T + rr;
      int v = rt[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) v = rr == j ? rt[j] : v;
      return v;
    };
    if constexpr (A16) {
      // copy q moves rows 4q .. 4q+3 (lane -> row 4q + lane/16, 16-byte chunk
      // lane%16 ^ row%16, landing at chunk lane%16), so both copies always go out
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rr = 4 * q + (lane >> 4);
        a16_src[q] = reinterpret_cast<const uint8_t*>(GU ? a.x : a.h16) + int64_t(act_row(rr)) * K * 2 +
                     16 * ((lane & 15) ^ (rr & 15));
      }
      return;
    }
    a_src = (GU ? a.x_codes : a.h_codes) + int64_t(act_row(ar)) * K + 16 * achunk;
    as_src = (GU ? a.x_scales : a.h_scales) + int64_t(act_row(lane & 7)) * (K / 32);
  };
  auto issue = [&](int el) {
    const int il = el / nsw, si = el - il * nsw;
    if (si == 0) item_setup(il);
    const int st = KSPLIT ? wu + 4 * si : si;
    const uint32_t slot = wbase + (el % S) * SLOT;
    // weights and their scales are read once: non-temporal, except for the
    // two-group down items, which measured slower with it (activation rows
    // are shared by the column groups of a tile and stay plain)
#pragma unroll
    for (int g2 = 0; g2 < GPI; ++g2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* src = CANON ? w_src + (int64_t(g2) * (GU ? 32 : 64) + canon_row_off<GU>(j, a.dff)) * (K / 2) + st * 64
                                   : w_src + int64_t(g2) * ns * 4096 + st * 4096 + j * 1024;
        if (WIDE && !GU) lds_copy16(src, slot + SW + g2 * 4096 + j * 1024);
        else lds_copy16_nt(src, slot + SW + g2 * 4096 + j * 1024);
      }
    // only the tile's rows (tiles are never empty, so the copy is always
    // issued and every element counts NC copies)
    if constexpr (A16) {
      // only the tile's rows (lane 0's row 0 or 4 always goes, so both
      // copies are issued and every element counts NC copies)
      if ((lane >> 4) < nr || lane == 0) lds_copy16(a16_src[0] + 256 * st, slot + SA);
      if (4 + (lane >> 4) < nr || lane == 0) lds_copy16(a16_src[1] + 256 * st, slot + SA + 1024);
    } else {
      if (lane < 8 * nr) lds_copy16(a_src + 128 * st, slot + SA);
      lds_copy4(as_src + 4 * st, slot + SAS);
    }
#pragma unroll
    for (int g2 = 0; g2 < GPI; ++g2) {
      const uint8_t* src = CANON ? bs_src + int64_t(g2) * (GU ? 32 : 64) * (K / 32) + st * 4
                                 : bs_src + int64_t(g2) * ns * 256 + st * 256;
      if (WIDE && !GU) lds_copy4(src, slot + SBS + g2 * 256);
      else lds_copy4_nt(src, slot + SBS + g2 * 256);
    }
  };

  // ---- consume side
  const int arow = r16 & 7;
  const int a_off0 = arow * 128 + 16 * (g ^ ((arow >> 1) & 3));
  const int a_off1 = arow * 128 + 16 * ((4 + g) ^ ((arow >> 1) & 3));
  v4f acc[4 * GPI];
#pragma unroll
  for (int j = 0; j < 4 * GPI; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  // bf16 operands: lane (row i = lane%16, group kg = lane/16) supplies, for
  // MFMA c of a step, the 8 values k = 32 kg + 8c .. +7: its A row's 16
  // bytes at chunk 4 kg + c, and 8 of the 32 FP4 weights it holds (block kg
  // of its weight row), expanded with that block's scale.  Any assignment of
  // k to (lane group, element) gives the same sum as long as A and B agree.
  const int a16_row = r16 & 7;
  auto compute16 = [&](int el) {
    const uint8_t* sl = wlds + (el % S) * SLOT;
    v8bf16 av[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      av[c] = *reinterpret_cast<const v8bf16*>(sl + SA + a16_row * 256 + 16 * ((4 * g + c) ^ a16_row));
#pragma unroll
    for (int g2 = 0; g2 < GPI; ++g2) {
      const uint32_t sbw = *reinterpret_cast<const uint32_t*>(sl + SBS + g2 * 256 + 4 * lane);
      uint32_t wd[4][4];
      float scl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 wv = ld16(sl + SW + g2 * 4096 + j * 1024 + 16 * lane);
        wd[j][0] = wv.x; wd[j][1] = wv.y; wd[j][2] = wv.z; wd[j][3] = wv.w;
        // scale of block j of this lane's row, K block 4st + g: byte j of the
        // packed dword, or byte g of the row's dword (canonical)
        const uint32_t sb =
            CANON ? (*reinterpret_cast<const uint32_t*>(sl + SBS + g2 * 256 + 4 * (16 * j + r16)) >> (8 * g)) & 0xFFu
                  : (sbw >> (8 * j)) & 0xFFu;
        scl[j] = __uint_as_float(sb ? sb << 23 : 0x00400000u);  // 2^(sb-127)
      }
      // K chunk outer, block inner: consecutive MFMAs use different accumulators
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v2bf16 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[j][c], scl[j], 0);
          const v2bf16 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[j][c], scl[j], 1);
          const v2bf16 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[j][c], scl[j], 2);
          const v2bf16 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[j][c], scl[j], 3);
          const v8bf16 bv = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          acc[4 * g2 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[c], bv, acc[4 * g2 + j], 0, 0, 0);
        }
    }
  };
  auto compute = [&](int el) {
    if constexpr (A16) {
      compute16(el);
      return;
    }
    const uint8_t* sl = wlds + (el % S) * SLOT;
    const v8i av = make_a(ld16(sl + SA + a_off0), ld16(sl + SA + a_off1));
    const uint32_t sa = *reinterpret_cast<const uint32_t*>(sl + SAS + 4 * arow) >> (8 * g);
#pragma unroll
    for (int g2 = 0; g2 < GPI; ++g2) {
      const uint32_t sbw = *reinterpret_cast<const uint32_t*>(sl + SBS + g2 * 256 + 4 * lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8i bv = make_b(ld16(sl + SW + g2 * 4096 + j * 1024 + 16 * lane));
        const uint32_t sb = CANON ? *reinterpret_cast<const uint32_t*>(sl + SBS + g2 * 256 + 4 * (16 * j + r16)) >> (8 * g)
                                  : sbw >> (8 * j);
        acc[4 * g2 + j] = mfma_mx(av, bv, acc[4 * g2 + j], sa, sb);
      }
    }
  };
  // end of item il: partial sums into the slot just consumed (a wave without
  // K steps uses slot 0 of its idle ring), then wave w reduces output lanes
  // 16w .. 16w+15 (tile rows 4w .. 4w+3) in wave order and writes them
  auto part_slot = [&](int w, int il) -> const v4f* {
    const int n = wsteps(w);
    const int sl = n > 0 ? ((il + 1) * n - 1) % S : 0;
    return reinterpret_cast<const v4f*>(ds_lds + w * WAVE + sl * SLOT);
  };
  // gate_up epilogue of one output row: v[0..1] gate and v[2..3] up sums of h
  // columns 32G + col and 32G + 16 + col (the 16 lanes with equal lane/16
  // hold the row's 32 columns: one MXFP8 block)
  auto gu_epilogue = [&](const float* v, int row, bool valid, int G, int col) {
    float h[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      h[j] = v[j] / (1.0f + __expf(-v[j])) * v[2 + j];
      if (valid && a.gu_acc) {
        const int c = 32 * G + 16 * j + col;
        a.gu_acc[int64_t(row) * 2 * a.dff + c] = v[j];
        a.gu_acc[int64_t(row) * 2 * a.dff + a.dff + c] = v[2 + j];
      }
    }
    if constexpr (A16) {
      if (valid) {
        uint16_t* hb = a.h16 + int64_t(row) * a.dff + 32 * G + col;
        hb[0] = f32_to_bf16_rne(h[0]);
        hb[16] = f32_to_bf16_rne(h[1]);
      }
      return;
    }
    const int e = mx8_block_exp(group_max<16>(fmaxf(fabsf(h[0]), fabsf(h[1]))));
    const float sc = exp2_int(-e);
    const uint32_t codes = e4m3_cvt2(h[0] * sc, h[1] * sc);
    if (valid) {
      uint8_t* hc = a.h_codes + int64_t(row) * a.dff + 32 * G + col;
      hc[0] = static_cast<uint8_t>(codes & 0xFFu);
      hc[16] = static_cast<uint8_t>(codes >> 8);
      if (col == 0) a.h_scales[int64_t(row) * (a.dff / 32) + G] = static_cast<uint8_t>(e + 127);
    }
  };
  auto item_end = [&](int il, int el_last) {
    if (!KSPLIT) {
      // whole item in this wave: lane l holds rows 4(l/16) + i, column l%16
      const int* md = fifo_ep + (il & 7) * 4;
      const int t_rb = md[1], t_re = md[2], G = md[3];
      if (GU) {
        // group g2 of the item: h columns 32 (GPI G + g2) ..
#pragma unroll
        for (int g2 = 0; g2 < GPI; ++g2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = t_rb + 4 * g + i;
            float v[4] = {acc[4 * g2][i], acc[4 * g2 + 1][i], acc[4 * g2 + 2][i], acc[4 * g2 + 3][i]};
            gu_epilogue(v, row, row < t_re, GPI * G + g2, r16);
          }
      } else {
        // o rows [8][64*GPI] as bf16 (RNE), staged in the slot of the item's
        // last element (no copy lands there before the next element is
        // issued) and written in 16-byte chunks of 8 columns
        constexpr int OC = 64 * GPI;
        uint16_t* stg = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(wlds) + (el_last % S) * SLOT);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4 * GPI; ++j) stg[(4 * g + i) * OC + 16 * j + r16] = f32_to_bf16_rne(acc[j][i]);
#pragma unroll
        for (int q = 0; q < GPI; ++q) {
          const int ch = 64 * q + lane;             // chunk: row ch / (OC/8), columns 8 (ch % (OC/8))
          const int rl = ch / (OC / 8), c8 = ch - rl * (OC / 8);
          const uint4 v = *reinterpret_cast<const uint4*>(stg + rl * OC + 8 * c8);
          if (t_rb + rl < t_re)
            *reinterpret_cast<uint4*>(a.o16 + int64_t(t_rb + rl) * a.d + OC * G + 8 * c8) = v;
        }
      }
#pragma unroll
      for (int j = 0; j < 4 * GPI; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
      return;
    }
    v4f* mine = const_cast<v4f*>(part_slot(wu, il));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mine[j * 64 + lane] = acc[j];
      acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    const int* md = fifo_ep + (il & 7) * 4;
    const int t_rb = md[1], t_re = md[2], G = md[3];
    const int i = lane >> 4, col = lane & 15;
    const int row = t_rb + 4 * wu + i;
    if (4 * wu < t_re - t_rb) {                       // else this wave's rows are all padding
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += part_slot(w, il)[j * 64 + 16 * wu + col][i];
        v[j] = sum;
      }
      gu_epilogue(v, row, row < t_re, G, col);
    }
    __syncthreads();  // the parked partials are read: their slots may be refilled
  };

  int iss = 0;
  for (; iss < nel && iss < S - 1; ++iss) issue(iss);
  int el = 0;
  for (int il = 0; il < my_items; ++il) {
    for (int k = 0; k < nsw; ++k, ++el) {
      if (iss < nel) issue(iss++);
      // copies issued after element el are still allowed in flight
      switch (iss - 1 - el) {
        case 0: PF_WAIT_VM(0); break;
        case 1: PF_WAIT_VM(NC); break;
        case 2: PF_WAIT_VM(2 * NC); break;
        case 3: PF_WAIT_VM(3 * NC); break;
        case 4: PF_WAIT_VM(4 * NC); break;
        case 5: PF_WAIT_VM(5 * NC); break;
        default: PF_WAIT_VM(6 * NC); break;
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      compute(el);
    }
    item_end(il, el - 1);
  }
}

template <bool GU, bool C>
static hipError_t launch_stream_w(const FwdArgs& a, hipStream_t st) {
  // the item count is known on the device only; max_tiles bounds it
  const int64_t max_items = int64_t(a.max_tiles) * (GU ? a.dff / 32 : a.d / 64);
  // persistent: one workgroup per CU, a multiple of 8 (one share per XCD)
  const unsigned grid = 8u * static_cast<unsigned>(a.num_cus >= 16 ? a.num_cus / 8 : 1);
  // few items per wave (< 16): gate_up splits K across a workgroup's waves,
  // down keeps one-group items and the deeper ring; many: whole items per
  // wave, two groups per down item and, with bf16 activations, per gate_up
  // item
  const bool few = max_items < 16 * 4 * int64_t(a.num_cus);
  // few-token routing in one workgroup: the shared experts' items already ran
  // in the routing launch (stream_topk_shared), only the routed ones here
  const bool routed_only = GU && stream_split_phases(a);
  if (a.a16) {
    if (!GU && !few)
      hipLaunchKernelGGL((k_gemm_stream<false, false, true, true, 0, C>), dim3(grid), dim3(256), 0, st, a);
    else if (!GU)
      hipLaunchKernelGGL((k_gemm_stream<false, false, false, true, 0, C>), dim3(grid), dim3(256), 0, st, a);
    else if (routed_only && few)
      hipLaunchKernelGGL((k_gemm_stream<true, true, false, true, 2, C>), dim3(grid), dim3(256), 0, st, a);
    else if (routed_only)
      hipLaunchKernelGGL((k_gemm_stream<true, false, true, true, 2, C>), dim3(grid), dim3(256), 0, st, a);
    else if (few)
      hipLaunchKernelGGL((k_gemm_stream<true, true, false, true, 0, C>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_gemm_stream<true, false, true, true, 0, C>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (routed_only) {
    if (few)
      hipLaunchKernelGGL((k_gemm_stream<true, true, false, false, 2, C>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_gemm_stream<true, false, false, false, 2, C>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (!GU && !few)
    hipLaunchKernelGGL((k_gemm_stream<false, false, true, false, 0, C>), dim3(grid), dim3(256), 0, st, a);
  else if (!GU)
    hipLaunchKernelGGL((k_gemm_stream<false, false, false, false, 0, C>), dim3(grid), dim3(256), 0, st, a);
  else if (few)
    hipLaunchKernelGGL((k_gemm_stream<true, true, false, false, 0, C>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_stream<true, false, false, false, 0, C>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <bool GU>
static hipError_t launch_stream(const FwdArgs& a, hipStream_t st) {
  return a.wcanon ? launch_stream_w<GU, true>(a, st) : launch_stream_w<GU, false>(a, st);
}

// ---------------------------------------------------------------------------
// Prefill variant: 256-row x 256-weight-row workgroup tiles, four waves (one
// per SIMD), each computing 128 rows x 128 weight rows on the 32x32x64
// scaled MFMA (sixteen 32x32 fp32 accumulators per wave).
//
// Operands move global -> LDS with direct-to-LDS copies (no registers stage
// them) through a ring of three K-step slots.  A slot holds
//   * A codes, 32 KB: row-major, 128 bytes per row, with the 16-byte chunks
//     of row r XOR-swizzled by (r/2)%8.  One copy moves 8 whole rows (8
//     lanes per row, each 128-byte line read once) and the MFMA fragment
//     reads (32 rows x one chunk) hit every bank once per 16 lanes;
//   * B codes, 16 KB: the tile's four packed 64-row groups (4 KB each: four
//     1 KB chunks of 16 rows x 128 K); the FP4 operand of 32 rows x 64 K is a
//     per-lane gather over two chunks that touches 16 consecutive bytes per
//     lane group (conflict free);
//   * A scales, 1 KB: one dword (the step's four block scales) per row -- only
//     when K is not a multiple of 512.  Otherwise the activation scales of
//     four steps (16 bytes per row) come once per group into 4 KB of the
//     (then unused) A-scale areas of slots 0 and 1, and every wave keeps its
//     rows' 16 bytes in registers for the group;
//   * B scales, 1 KB: the step's packed scale dwords of the four groups (one
//     byte per 16-row block).
// The two waves of a row half (w%2 == wm) copy the activation rows of that
// half's 32-row blocks between them (8-row copies, alternating; two per
// block), wave w the packed group w of the weights and its scales, and the
// activation scales of rows 64w .. 64w+63.
//
// Step st (K = 128) runs in two K halves of 64 with two register sets:
//   LDS reads of half 1 into set 1;   MFMAs of half 0 from set 0;
//   wait for those reads and for this wave's copies of step st+1; barrier
//     (every wave is then done with slot st, and step st+1 is in LDS);
//   copies of step st+3 into slot st%3;
//   LDS reads of half 0 of step st+1 (and its scales) into set 0;
//   MFMAs of half 1 from set 1.
// The LDS reads always run under the other half's MFMAs, and every copy has
// two steps to land.  Row blocks past the tile's end skip their reads and
// MFMAs.  Scale bytes are picked by the MFMA's operand selects.
//
// The two waves with the same w/2 split the tile's 32-row blocks evenly
// (up to four each, the first ones to w%2 == 0) and compute them against
// 128 of the 256 weight rows (w/2 picks them): gate and up rows of the same
// 64 h columns for gate_up, 128 output columns for down.
// ---------------------------------------------------------------------------

typedef float v16f __attribute__((ext_vector_type(16)));

// A: FP8 E4M3 with its scale in byte SA of sa; B: FP4 E2M1 with its scale in
// byte SB of sb
template <int SA, int SB>
__device__ __forceinline__ v16f mfma32_mx(const v8i& a, const v8i& b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, SA, static_cast<int>(sa), SB,
                                                         static_cast<int>(sb));
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// f(IntC<B>{}), f(IntC<B+1>{}), ..., f(IntC<E-1>{})
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kPfSlot = 52224;                 // A 32 KB | B 16 KB | A scales 2 KB | B scales 1 KB
constexpr int kPfA = 0, kPfB = 32768, kPfAS = 49152, kPfBS = 51200;
constexpr int kPfRowTab = 3 * kPfSlot;         // the ring: 156672 bytes; then 256 row entries
constexpr int kPfLds = kPfRowTab + 1024;
__shared__ __attribute__((aligned(1024))) uint8_t pf_lds[kPfLds];


// Work order of the prefill GEMMs.  Items (tile, column block) run in groups
// of G consecutive tiles (tiles are expert-major; G is chosen by the launch),
// column block next and tile fastest, so the workgroups an XCD runs at once cover a few
// tiles x several column blocks: every activation window and every weight
// window they read in the same K step is shared by several of them and comes
// from that XCD's L2.  Whole groups are dealt to the XCDs round-robin in list
// order (workgroups go to the XCDs round-robin by linear id), so at any time
// the eight XCDs work on neighbouring groups -- mostly the same expert, whose
// weight tiles they then share through the memory-side cache -- and the
// sparse tiles of lightly loaded experts are spread over all XCDs instead of
// piling up on the last ones (measured faster than cutting the list into
// eight contiguous ranges, and than taking groups alternately from its two
// ends).  The mapping needs only the tile count.  Returns false for a
// workgroup with no item.
constexpr int kPfGroupTiles = 4;
__device__ __forceinline__ bool pf_work_item(const FwdArgs& a, int nblocks, int G, int* tile_out, int* blk_out) {
  const int ntiles = *a.tile_count;
  const int ngroups = (ntiles + G - 1) / G;
  if (ngroups < 8) {
    // fewer groups than XCDs: items one by one, tile fastest, so that every
    // XCD gets a share (the grid holds at least 32 items per group)
    const int i = blockIdx.x;
    if (i >= ntiles * nblocks) return false;
    *tile_out = i % ntiles;
    *blk_out = i / ntiles;
    return true;
  }
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int gitems = G * nblocks;                              // items of a full group
  const int j = i / gitems, rem = i - j * gitems;
  const int tg = 8 * j + xcd;                                  // tile group
  if (tg >= ngroups) return false;
  const int gsize = min(G, ntiles - tg * G);
  if (rem >= gsize * nblocks) return false;
  *blk_out = rem / gsize;
  *tile_out = tg * G + rem % gsize;
  return true;
}

typedef float v2f __attribute__((ext_vector_type(2)));

// lane l reads lane l^1's (l^2's) x
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
// In every quad of lanes (4m .. 4m+3), with lane q holding v[j] = M[q][j]:
// afterwards lane q holds v[j] = M[j][q].  Two exchanges, between lanes q and
// q^2 then q and q^1, each of the two entries that sit in the other half.
__device__ __forceinline__ void quad_transpose4(float (&v)[4], int q) {
  const bool h2 = (q & 2) != 0, h1 = (q & 1) != 0;
  float r0 = dpp_xor2(h2 ? v[0] : v[2]), r1 = dpp_xor2(h2 ? v[1] : v[3]);
  if (h2) { v[0] = r0; v[1] = r1; } else { v[2] = r0; v[3] = r1; }
  r0 = dpp_xor1(h1 ? v[0] : v[1]);
  r1 = dpp_xor1(h1 ? v[2] : v[3]);
  if (h1) { v[0] = r0; v[2] = r1; } else { v[1] = r0; v[3] = r1; }
}

// LDS address of the A-scale group area written by wave w (0..3)
__device__ __forceinline__ int pf_asg_off(int w) { return (w >> 1) * kPfSlot + kPfAS + (w & 1) * 1024; }

template <bool GU, bool AG, bool CANON>
__global__ void __launch_bounds__(256, 1) k_gemm_pf(FwdArgs a, int group) {
  int tile_idx, nblk;
  // down with a K split: the slices of a column block are further blocks
  const int kspl = GU || a.ksplit <= 1 ? 1 : a.ksplit;
  if (!pf_work_item(a, GU ? a.dff / 128 : ((a.d + 255) / 256) * kspl, group, &tile_idx, &nblk)) return;
  const int kslice = nblk % kspl;
  nblk /= kspl;
  const Tile tile = a.tiles[tile_idx];
  // the tile's expert has no other tile: its weights are read once
  const bool w_once = a.ex_tiles[tile.ex + 1] - a.ex_tiles[tile.ex] == 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g32 = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy of the wave index
  const int wm = wu & 1, wn = wu >> 1;
  const int K = GU ? a.d : a.dff;
  const int nsteps_all = K / 128;
  // K steps of this item (the whole K, or one slice of it: a multiple of 4
  // steps, so the grouped activation scales stay aligned)
  const int nsteps = nsteps_all / kspl;
  const int k0 = kslice * nsteps;

  const bool shared = tile.ex >= a.E;
  const int sidx = tile.ex - a.E;
  const int64_t wrows = GU ? 2 * a.dff : a.d;
  const int64_t wc_stride = wrows * (K / 2), ws_stride = packed_scale_bytes(wrows, K);
  const uint8_t* wc = GU ? (shared ? a.sgu_c + sidx * wc_stride : a.gu_c + tile.ex * wc_stride)
                         : (shared ? a.sdn_c + sidx * wc_stride : a.dn_c + tile.ex * wc_stride);
  const uint8_t* ws = GU ? (shared ? a.sgu_s + sidx * ws_stride : a.gu_s + tile.ex * ws_stride)
                         : (shared ? a.sdn_s + sidx * ws_stride : a.dn_s + tile.ex * ws_stride);

  // the tile's four packed 64-row groups 4*nblk .. 4*nblk+3: gate and up rows
  // of h columns 32 apiece (gate_up, interleaved packing), or 256 consecutive
  // output rows (down)
  const int c0 = GU ? nblk * 128 : nblk * 256;
  const int64_t grp0 = 4 * int64_t(nblk);
  const uint32_t lds0 = lds_addr(pf_lds);
  // A routed tile's row indirections come to LDS ahead of everything else,
  // one direct copy per wave (tile rows 64 wu .. 64 wu + 63, rows past the
  // tile's end reading its first row): the row-to-token entries of gate_up,
  // which the activation copies' addresses need (so the weight copies of the
  // first steps can go out while they travel), and the row-to-pair entries
  // of down, which only its epilogue's stores need.
  const int* const row_tab = reinterpret_cast<const int*>(pf_lds + kPfRowTab);
  const bool routed = tile.row_begin < a.Rr;   // (a tile never mixes routed and shared rows)
  if (routed) {
    const int r = 64 * wu + lane;
    const int row = tile.row_begin + (tile.row_begin + r < tile.row_end ? r : 0);
    lds_copy4((GU ? a.row_token : a.row_src) + row, lds0 + kPfRowTab + wu * 256);
  }
  // activation row of tile row r; padding rows read the tile's first row
  // (gate_up: only once the row table has landed)
  auto src_row = [&](int r) -> int64_t {
    if (GU && routed) return row_tab[r];
    int row = tile.row_begin + r;
    if (row >= tile.row_end) row = tile.row_begin;
    return GU ? row - a.Rr - sidx * a.T : row;
  };

  // the tile's 32-row blocks split evenly between the two row halves (a
  // step lasts as long as its busiest wave): wave half wm takes blocks
  // rb0 .. rb0 + nact - 1
  const int nb = (tile.row_end - tile.row_begin + 31) >> 5;
  const int rb0 = wm ? (nb + 1) >> 1 : 0;
  const int nact = wm ? nb >> 1 : (nb + 1) >> 1;                        // active row blocks
  // ---- copy sources of this wave.  The two waves of a row half copy the
  // activation rows of its nact blocks between them: copy q of wave (wm, wn)
  // covers the 8-row group ag(q) = 4 rb0 + 2q + wn (q < 2 nact); lane l
  // reads chunk (l%8) ^ swz(row) of row 8 ag(q) + l/8 and lands at LDS
  // row*128 + 16(l%8).  (Set once the rows are known: for gate_up after a
  // barrier that follows every wave's wait for its own row-table copy, as a
  // wave looks up rows that another wave copied.)
  auto ag = [&](int q) -> int { return 4 * rb0 + 2 * q + wn; };
  const uint8_t* a_src[8];
  const uint8_t* as_src = nullptr;
  auto set_act_sources = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rl = 8 * ag(q) + (lane >> 3);
      a_src[q] = (GU ? a.x_codes : a.h_codes) + src_row(rl) * K + 128 * k0 + 16 * ((lane & 7) ^ ((rl >> 1) & 7));
    }
    as_src = (GU ? a.x_scales : a.h_scales) + src_row(64 * wu + lane) * (K / 32) + (AG ? 16 * (k0 / 4) : 4 * k0);
  };
  // down with d an odd multiple of 128: the last column block has two
  // groups; the waves of the missing half copy group grp0 instead (the
  // same number of copies, data never stored) and store nothing
  const int64_t gw = GU || grp0 + wu < a.d / 64 ? grp0 + wu : grp0;
  const bool cols_live = GU || c0 + 128 * wn < a.d;
  // canonical weights: the same LDS image as the packed order for the codes
  // (lane 16g + r of block m's copy reads row r of the block, K bytes
  // 64 st + 16g ..), and per row a dword of four block scales (lane 16jb + r
  // of the scale copy: row r of block jb, blocks 4st .. 4st+3)
  const int64_t crow0 = GU ? 32 * gw : 64 * gw;
  const uint8_t* b_src = CANON ? wc + (crow0 + (lane & 15)) * (K / 2) + 16 * (lane >> 4) + int64_t(k0) * 64
                               : wc + gw * nsteps_all * 4096 + int64_t(k0) * 4096 + 16 * lane;
  const uint8_t* bs_src = CANON ? ws + (crow0 + canon_row_off<GU>(lane >> 4, a.dff) + (lane & 15)) * (K / 32) + int64_t(k0) * 4
                                : ws + gw * nsteps_all * 256 + int64_t(k0) * 256 + 4 * lane;
  // per-step strides of the two
  constexpr int kBStep = CANON ? 64 : 4096, kBSStep = CANON ? 4 : 256;

  // Copies of step st into slot st % 3 (and of the activation scales of
  // group st / 4 when st starts a group).  Their number per step is fixed --
  // an 8-row copy past the tile's end reads the tile's first row, and a step
  // past K re-reads step 0 into a slot that is not read again -- so that every
  // wait on them is a constant and a step has no branches.  They come in two
  // parts: the 2 nact activation copies (copy_a) and the weights, weight
  // scales and activation scales (copy_w, items 0-5).  ncop(NA, st): the
  // copies of step st for NA activation copies.
  constexpr auto ncop = [](int na, int st) -> int { return na + 5 + (AG ? ((st & 3) == 0 ? 1 : 0) : 1); };
  auto copy_a = [&](int st, auto qc) {
    constexpr int q = decltype(qc)::value;
    const int ss = st < nsteps ? st : 0;
    lds_copy16(a_src[q] + 128 * ss, lds0 + (st % 3) * kPfSlot + kPfA + (8 * ag(q)) * 128);
  };
  // item m of step st; GS: st starts a group of four steps
  // WNT: the weights are read by this tile only (its expert has one tile),
  // so their copies carry the non-temporal hint; an expert with several tiles
  // keeps its weight tiles cacheable for the others
  auto copy_w = [&](int st, auto mc, auto gsc, auto wntc) {
    constexpr bool WNT = decltype(wntc)::value != 0;
    constexpr int m = decltype(mc)::value;
    constexpr bool GS = decltype(gsc)::value != 0;
    const int ss = st < nsteps ? st : 0;
    const uint32_t slot = lds0 + (st % 3) * kPfSlot;
    constexpr int64_t kBlk = 1024;   // packed: block m of the group's step is 1 KB further
    const uint8_t* bsrc = CANON ? b_src + ss * kBStep + int64_t(canon_row_off<GU>(m < 4 ? m : 0, a.dff)) * (K / 2)
                                : b_src + ss * kBStep + m * kBlk;
    if constexpr (m < 4 && WNT) lds_copy16_nt(bsrc, slot + kPfB + (4 * wu + m) * 1024);
    if constexpr (m < 4 && !WNT) lds_copy16(bsrc, slot + kPfB + (4 * wu + m) * 1024);
    if constexpr (m == 4 && WNT) lds_copy4_nt(bs_src + ss * kBSStep, slot + kPfBS + wu * 256);
    if constexpr (m == 4 && !WNT) lds_copy4(bs_src + ss * kBSStep, slot + kPfBS + wu * 256);
    if constexpr (m == 5 && !AG) lds_copy4(as_src + 4 * ss, slot + kPfAS + wu * 256);
    if constexpr (m == 5 && AG && GS) lds_copy16(as_src + 16 * (ss >> 2), lds0 + pf_asg_off(wu));
  };

  // ---- per-lane LDS read offsets
  // weight fragment p (32 rows) starts at chunk j0(p) of the tile's 16: for
  // gate_up, gate rows of h columns c0 + 64wn + 32p (p < 2; group 2wn + p,
  // blocks 0-1) and the up rows of the same columns (blocks 2-3).  Its scale
  // dword lies in group 2wn + pg(p), byte j0(p)%4 (+1 for rows 16-31).
  auto j0 = [&](int p) -> int { return GU ? (p < 2 ? 8 * wn + 4 * p : 8 * wn + 4 * (p - 2) + 2) : 8 * wn + 2 * p; };
  const int b_lane = ((l32 >> 4) << 10) + 16 * (16 * g32 + (lane & 15));  // + j0*1024 + 512h
  // A fragment (row l32 of a 32-row block, K half h, piece c): chunk 4h+2c+g32
  int a_lane[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) a_lane[h][c] = l32 * 128 + 16 * ((4 * h + 2 * c + g32) ^ ((l32 >> 1) & 7));
  const int bs_lane = 4 * (16 * g32 + (lane & 15)) + (2 * wn) * 256;  // + 256*group + 128h
  const int wrow0 = 32 * rb0;                                            // first tile row of this wave

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[i][p] = v16f{};

  auto main_loop = [&](auto nact_c, auto wnt_c) {
    constexpr int NACT = decltype(nact_c)::value;
    constexpr int NA = 2 * NACT;                 // this wave's activation copies per step
    uint4 asg[4];               // grouped activation scales of this lane's rows
    uint32_t asr[2][4];         // A scale dwords (shifted by 8*g32) of the current / next step
    uint32_t bsd[2][2][2];      // B scale dwords [buffer][group 2wn+gi][half] (shifted by 8*(l32/16))
    v8i av[2][4], bv[2][4];     // operand sets of K half 0 and 1

    // operand reads (slot byte offset so): A fragment of row block I_, B
    // fragment P, K half H
    auto read_a = [&](int so, auto hc, auto ic_) {
      constexpr int H = decltype(hc)::value, I_ = decltype(ic_)::value;
      if (I_ >= NACT) return;
      const uint8_t* pa = pf_lds + so + kPfA + (rb0 + I_) * 4096;
      av[H][I_] = make_a(ld16(pa + a_lane[H][0]), ld16(pa + a_lane[H][1]));
    };
    auto read_b = [&](int so, auto hc, auto pc) {
      constexpr int H = decltype(hc)::value, P = decltype(pc)::value;
      if (NACT == 0) return;
      bv[H][P] = make_b(ld16(pf_lds + so + kPfB + j0(P) * 1024 + 512 * H + b_lane));
    };
    // scales of step st (st % 4 == I): raw loads, then (once later LDS reads
    // are in flight) the shifts into buffer B
    uint32_t bs_raw[2][2], as_raw[4];
    auto load_scales = [&](int st, auto ic) {
      constexpr int I = decltype(ic)::value;
      if (NACT == 0) return;
      const uint8_t* sb = pf_lds + (st % 3) * kPfSlot;
      if constexpr (CANON) {
        // fragment P = 2a + b in bs_raw[a][b]: the dword of its row l32
        // (block SB(P) + l32/16 of group 2wn + GI(P)); both K halves in it
#pragma unroll
        for (int P = 0; P < 4; ++P) {
          const int gi = GU ? (P & 1) : (P >> 1), sbk = GU ? (P >= 2 ? 2 : 0) : ((P & 1) ? 2 : 0);
          bs_raw[P >> 1][P & 1] =
              *reinterpret_cast<const uint32_t*>(sb + kPfBS + (2 * wn + gi) * 256 + 4 * (16 * sbk + l32));
        }
      } else {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            bs_raw[gi][h] = *reinterpret_cast<const uint32_t*>(sb + kPfBS + gi * 256 + 128 * h + bs_lane);
      }
      if (AG) {
        if (I == 0) {
#pragma unroll
          for (int i = 0; i < NACT; ++i)
            asg[i] = *reinterpret_cast<const uint4*>(pf_lds + pf_asg_off((rb0 + i) >> 1) + (32 * ((rb0 + i) & 1) + l32) * 16);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NACT; ++i)
          as_raw[i] = *reinterpret_cast<const uint32_t*>(sb + kPfAS + (wrow0 + 32 * i + l32) * 4);
      }
    };
    auto shift_scales = [&](auto ic, auto bc) {
      constexpr int I = decltype(ic)::value, B = decltype(bc)::value;
      if (NACT == 0) return;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int h = 0; h < 2; ++h) bsd[B][gi][h] = bs_raw[gi][h] >> (CANON ? 8 * g32 : 8 * (l32 >> 4));
#pragma unroll
      for (int i = 0; i < NACT; ++i) {
        const uint32_t v = AG ? (I == 0 ? asg[i].x : I == 1 ? asg[i].y : I == 2 ? asg[i].z : asg[i].w) : as_raw[i];
        asr[B][i] = v >> (8 * g32);
      }
    };
    // MFMA k of K half H (row block k/4, fragment k%4) with scale buffer B;
    // fragment p's weight scale: group 2wn + gi, byte sel
    auto mf = [&](auto hc, auto bc, auto kc) {
      constexpr int H = decltype(hc)::value, B = decltype(bc)::value, Kk = decltype(kc)::value;
      constexpr int I_ = Kk >> 2, P = Kk & 3;
      constexpr int GI = GU ? (P & 1) : (P >> 1);
      constexpr int SB = GU ? (P >= 2 ? 2 : 0) : ((P & 1) ? 2 : 0);
      // canonical: byte 2H + g32 of the row's dword (shifted by 8 g32 already)
      if constexpr (CANON) {
        if (I_ < NACT)
          acc[I_][P] = mfma32_mx<2 * H, 2 * H>(av[H][I_], bv[H][P], acc[I_][P], asr[B][I_], bsd[B][P >> 1][P & 1]);
      } else {
        if (I_ < NACT)
          acc[I_][P] = mfma32_mx<2 * H, SB>(av[H][I_], bv[H][P], acc[I_][P], asr[B][I_], bsd[B][GI][H]);
      }
    };

    // step st: the memory work of the step sits between its MFMAs in a fixed
    // order (one scheduling region per MFMA), so the copies and LDS reads
    // issue while the matrix core is busy, spread over the step so the four
    // waves do not queue their copies at once
    auto step = [&](int st, auto ic) {
      constexpr int I = decltype(ic)::value;   // st % 4
      constexpr int B = I & 1;                 // scale buffer of step st
      const int s0 = (st % 3) * kPfSlot;
      // half 0 from set 0; between the MFMAs: reads of half 1 into set 1 and
      // the weight copies of step st+2 (its slot was freed in step st-1)
      static_for<0, 16>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        mf(IntC<0>{}, IntC<B>{}, kc);
        if constexpr (k % 2 == 1) {
          if constexpr (k / 2 < 4) read_a(s0, IntC<1>{}, IntC<k / 2>{});
          else read_b(s0, IntC<1>{}, IntC<k / 2 - 4>{});
        } else if constexpr (k / 2 < 6) {
          copy_w(st + 2, IntC<k / 2>{}, IntC<((I + 2) & 3) == 0>{}, wnt_c);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // (after the last step the reads below fetch a stale slot whose values
      // go unused: one code path keeps the accumulators in place)
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave is done reading slot st
      PF_WAIT_VM(ncop(NA, I + 2));             // its copies of step st+1 have landed
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const int s1 = ((st + 1) % 3) * kPfSlot;
      // half 1 from set 1; between the MFMAs: the scales and half 0 of step
      // st+1 (into set 0), then the activation copies of step st+3 into slot st
      static_for<0, 16>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        mf(IntC<1>{}, IntC<B>{}, kc);
        if constexpr (k == 0) { load_scales(st + 1, IntC<(I + 1) & 3>{}); read_a(s1, IntC<0>{}, IntC<0>{}); }
        if constexpr (k == 1) { read_b(s1, IntC<0>{}, IntC<0>{}); read_b(s1, IntC<0>{}, IntC<1>{}); }
        if constexpr (k == 2) read_a(s1, IntC<0>{}, IntC<1>{});
        if constexpr (k == 3) { read_b(s1, IntC<0>{}, IntC<2>{}); read_b(s1, IntC<0>{}, IntC<3>{}); }
        if constexpr (k == 4) read_a(s1, IntC<0>{}, IntC<2>{});
        if constexpr (k == 5) read_a(s1, IntC<0>{}, IntC<3>{});
        if constexpr (k >= 6 && k - 6 < NA) copy_a(st + 3, IntC<k - 6>{});
        if constexpr (k == 8) shift_scales(IntC<(I + 1) & 3>{}, IntC<B ^ 1>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: steps 0 and 1, and the activation copies of step 2 (its
    // weight copies come in step 0)
    if constexpr (GU) {
      // the weights and weight scales of steps 0 and 1 while the row table
      // travels; then, with the rows known, the activation scales of steps 0
      // and 1 and the activations of steps 0-2
      static_for<0, 5>([&](auto mc) { copy_w(0, mc, IntC<1>{}, wnt_c); });
      static_for<0, 5>([&](auto mc) { copy_w(1, mc, IntC<0>{}, wnt_c); });
      PF_WAIT_VM(10);                          // this wave's row-table copy (the oldest) has landed
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();            // and every wave's: a wave looks up rows others copied
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      set_act_sources();
      copy_w(0, IntC<5>{}, IntC<1>{}, wnt_c);
      copy_w(1, IntC<5>{}, IntC<0>{}, wnt_c);
      static_for<0, NA>([&](auto qc) { copy_a(0, qc); });
      static_for<0, NA>([&](auto qc) { copy_a(1, qc); });
      static_for<0, NA>([&](auto qc) { copy_a(2, qc); });
      PF_WAIT_VM(2 * NA);                      // step 0 (and 1 but its last activations) has landed
    } else {
      set_act_sources();
      static_for<0, NA>([&](auto qc) { copy_a(0, qc); });
      static_for<0, 6>([&](auto mc) { copy_w(0, mc, IntC<1>{}, wnt_c); });
      static_for<0, NA>([&](auto qc) { copy_a(1, qc); });
      static_for<0, 6>([&](auto mc) { copy_w(1, mc, IntC<0>{}, wnt_c); });
      static_for<0, NA>([&](auto qc) { copy_a(2, qc); });
      PF_WAIT_VM(ncop(NA, 1) + NA);            // step 0 has landed
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_scales(0, IntC<0>{});
    shift_scales(IntC<0>{}, IntC<0>{});
    static_for<0, 4>([&](auto ic_) { read_a(0, IntC<0>{}, ic_); read_b(0, IntC<0>{}, ic_); });
    // one branch-free block per loop body (K % 512 == 0 with grouped scales)
    if (AG) {
      for (int st0 = 0; st0 < nsteps; st0 += 4) {
        step(st0, IntC<0>{});
        step(st0 + 1, IntC<1>{});
        step(st0 + 2, IntC<2>{});
        step(st0 + 3, IntC<3>{});
      }
    } else {
      int st0 = 0;
      for (; st0 + 1 < nsteps; st0 += 2) {
        step(st0, IntC<0>{});
        step(st0 + 1, IntC<1>{});
      }
      if (st0 < nsteps) step(st0, IntC<0>{});
    }
  };
  switch (nact) {
    case 4: w_once ? main_loop(IntC<4>{}, IntC<1>{}) : main_loop(IntC<4>{}, IntC<0>{}); break;
    case 3: w_once ? main_loop(IntC<3>{}, IntC<1>{}) : main_loop(IntC<3>{}, IntC<0>{}); break;
    case 2: w_once ? main_loop(IntC<2>{}, IntC<1>{}) : main_loop(IntC<2>{}, IntC<0>{}); break;
    case 1: w_once ? main_loop(IntC<1>{}, IntC<1>{}) : main_loop(IntC<1>{}, IntC<0>{}); break;
    default: main_loop(IntC<0>{}, IntC<0>{}); break;
  }

  // ---- epilogue through LDS: after this wave's last copies have landed and
  // the barrier, every wave is past its last operand read and each wave then
  // owns a private stage region.
  // acc[i][p] register r holds tile row wrow0 + 32i + 8(r/4) + 4 g32 + r%4
  // and column l32 of weight fragment p.
  PF_WAIT_VM(0);
  __syncthreads();
  if (nact == 0 || !cols_live) return;
  if (GU) {
    // h = silu(gate) * up as fp32 [128 rows][64 h columns] (row stride 68)
    float* hs = reinterpret_cast<float*>(pf_lds) + wu * (128 * 68);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nact) break;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * i + 8 * (r / 4) + 4 * g32 + (r % 4);
          const float gt = acc[i][pp][r], up = acc[i][pp + 2][r];
          hs[rl * 68 + 32 * pp + l32] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
        }
    }
    // (the optional accumulator tap in a loop of its own: a branch inside the
    // loop above would cut it into one basic block per value and serialise
    // the exponential / reciprocal chains)
    if (a.gu_acc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nact) break;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = 32 * i + 8 * (r / 4) + 4 * g32 + (r % 4);
            const int row = tile.row_begin + wrow0 + rl;
            if (row < tile.row_end) {
              const int col = c0 + 64 * wn + 32 * pp + l32;
              a.gu_acc[int64_t(row) * 2 * a.dff + col] = acc[i][pp][r];
              a.gu_acc[int64_t(row) * 2 * a.dff + a.dff + col] = acc[i][pp + 2][r];
            }
          }
      }
    }
    // lane l quantises rows l and l + 64: two MXFP8 blocks of 32 h values each
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int rl = 64 * half + lane;
      const int row = tile.row_begin + wrow0 + rl;
      if (rl < 32 * nact && row < tile.row_end) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const float4* src = reinterpret_cast<const float4*>(hs + rl * 68 + 32 * blk);
          float v[32];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float4 t = src[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
          }
          float amax = 0.0f;
#pragma unroll
          for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
          const int e = mx8_block_exp(amax);
          const float sc = exp2_int(-e);
          uint32_t w[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            w[q] = e4m3_cvt4(v[4 * q] * sc, v[4 * q + 1] * sc, v[4 * q + 2] * sc, v[4 * q + 3] * sc);
          const int col = c0 + 64 * wn + 32 * blk;
          uint4* dst = reinterpret_cast<uint4*>(a.h_codes + int64_t(row) * a.dff + col);
          dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
          dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
          a.h_scales[int64_t(row) * (a.dff / 32) + (col >> 5)] = static_cast<uint8_t>(e + 127);
        }
      }
    }
  } else {
    if (kspl > 1) {
      // K slice: fp32 partials of this slice, rows in tile order, 16 bytes
      // per lane after a 4x4 transpose inside each lane quad (lane q of a
      // quad then holds one row and the quad's four columns)
      float* const pbase = a.kpart + int64_t(kslice) * a.R * a.d + c0 + 128 * wn + (l32 & ~3);
      const int q4 = lane & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nact) break;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int row = tile.row_begin + wrow0 + 32 * i + 8 * rb + 4 * g32 + q4;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            float v[4] = {acc[i][pp][4 * rb], acc[i][pp][4 * rb + 1], acc[i][pp][4 * rb + 2], acc[i][pp][4 * rb + 3]};
            quad_transpose4(v, q4);
            if (row < tile.row_end)
              *reinterpret_cast<float4*>(pbase + int64_t(row) * a.d + 32 * pp) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
      return;
    }
    // o rows are stored in (token, slot) order: routed row r goes to its pair
    // index row_src[r] (token-major, so the combine reads a token's rows
    // back to back), shared rows keep their place.  The routed rows'
    // destinations are in the row table, copied ahead of the operands and
    // landed before the barrier above.
    // bf16 outputs [128 rows][128 columns] staged in LDS, then 16-byte row
    // chunks to HBM: 16 per row, 2048 per wave, 32 per lane.  Staging: the
    // registers r, r+1 of a lane hold rows R, R+1 of one column; one exchange
    // with the neighbouring lane gives the even lane row R and the odd lane
    // row R+1, each for two adjacent columns, written as one packed dword.
    // Rows are 256 bytes apart, with their four 32-column chunks permuted by
    // bits 0 and 2 of the row, so that the four rows one write instruction
    // touches fall on distinct banks (and a row read touches every bank once).
    uint16_t* os = reinterpret_cast<uint16_t*>(pf_lds) + wu * (128 * 128);
    auto chunk_of = [](int rl, int c32) { return c32 ^ ((rl & 1) | (((rl >> 2) & 1) << 1)); };
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nact) break;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float v0 = acc[i][pp][r], v1 = acc[i][pp][r + 1];
          const float rv = dpp_xor1(odd ? v0 : v1);
          const v2bf16 pk = __builtin_convertvector((v2f){odd ? rv : v0, odd ? v1 : rv}, v2bf16);
          const int rl = 32 * i + 8 * (r / 4) + 4 * g32 + (r % 4) + (odd ? 1 : 0);
          *reinterpret_cast<uint32_t*>(os + rl * 128 + chunk_of(rl, pp) * 32 + (l32 & ~1)) =
              __builtin_bit_cast(uint32_t, pk);
        }
    }
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int ch = q * 64 + lane;          // chunk: row ch / 16, 8 columns at 8 (ch % 16)
      const int rl = ch >> 4, cc = 8 * (ch & 15);
      const int row = tile.row_begin + wrow0 + rl;
      if (rl < 32 * nact && row < tile.row_end) {
        const uint4 t = *reinterpret_cast<const uint4*>(os + rl * 128 + chunk_of(rl, cc >> 5) * 32 + (cc & 31));
        const int dst = routed ? row_tab[wrow0 + rl] : row;
        *reinterpret_cast<uint4*>(a.o16 + int64_t(dst) * a.d + c0 + 128 * wn + cc) = t;
      }
    }
  }
}

template <bool GU>
static hipError_t launch_pf(const FwdArgs& a, hipStream_t st) {
  const int64_t N = GU ? a.dff / 128 : int64_t((a.d + 255) / 256) * (a.ksplit > 1 ? a.ksplit : 1);
  // tile groups of four when experts have several tiles (they then share
  // each weight window in L2); of one when experts have 256 rows or fewer
  // on average, so most have one tile and only the activation windows are
  // shared (prefill8k 7.70-7.72 -> 7.63-7.64 ms; at prefill32k_skew groups of
  // one re-read the hot experts' weights: 44 against 36 GB per gate_up)
  const int group = a.Rr < int64_t(256) * a.E ? 1 : kPfGroupTiles;
  // room for the most groups one XCD can get (the tile count is known on the
  // device only; max_tiles bounds it)
  const int64_t max_groups = (int64_t(a.max_tiles) + group - 1) / group;
  const int64_t per_xcd = (max_groups + 7) / 8 * group * N;
  const int K = GU ? a.d : a.dff;
  const dim3 grid(static_cast<unsigned>(8 * per_xcd));
  if (K % 512 == 0 && a.wcanon)
    hipLaunchKernelGGL((k_gemm_pf<GU, true, true>), grid, dim3(256), 0, st, a, group);
  else if (K % 512 == 0)
    hipLaunchKernelGGL((k_gemm_pf<GU, true, false>), grid, dim3(256), 0, st, a, group);
  else if (a.wcanon)
    hipLaunchKernelGGL((k_gemm_pf<GU, false, true>), grid, dim3(256), 0, st, a, group);
  else
    hipLaunchKernelGGL((k_gemm_pf<GU, false, false>), grid, dim3(256), 0, st, a, group);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Prefill variant with bf16 activations (A16W4): the tiles of k_gemm_pf (256
// rows x 256 weight rows per workgroup, four waves of 128 x 128, the XCD
// round-robin of tile groups, here of one tile each), on the bf16 MFMA
// 32x32x16 with every FP4 weight fragment
// expanded to bf16 with its block scale in registers
// (V_CVT_SCALEF32_PK_BF16_FP4).  K steps of 64: a bf16 activation row is then
// 128 bytes per step, so the A slot is the MXFP8 kernel's (row-major, 16-byte
// chunks XOR-swizzled by (row/2)%8).  A slot of the three-slot ring holds
//   * A 32 KB;
//   * B 8 KB: per packed 64-row group 2 KB, per 16-row block the 512 bytes of
//     its packed 1 KB step that hold this K half (lanes 16g'+r, g' = 0, 1:
//     row r, K group g' of the half);
//   * B scales 1 KB: per group 256 bytes -- packed: the 32 scale dwords of
//     this half (lane 16g'+r, byte = block); canonical: a dword per row
//     (lane 16 block + r) holding the scales of the row's four K groups of
//     the 128-wide step, of which this half uses bytes 2h, 2h+1.
// Wave w copies the 8-row activation groups w, w+4, .. of the tile's nb
// 32-row blocks (nb copies; rows past the tile's end read its first row),
// packed group w's weights (two copies) and their scales (one): nb + 3
// copies per step.  Per step each wave waits for
// its own copies of the step, then a barrier (every wave's copies have
// landed, every wave is done with the slot of the step before); the LDS
// reads, the expansion and the MFMAs follow, with the copies of step st+2
// (into that slot) spread between them.  MFMA slice q of a step takes, in
// lane (row or column l%32, half kh = l/32), the 8 values 32 kh + 8q .. +7
// of the step: four consecutive bytes of the lane's 16-byte weight
// fragment, and the matching 16 bytes of its activation row.  The 32-row
// blocks of a tile are split evenly between the two row-half waves (an odd
// block shared by column halves).  The epilogues stage bf16 h (SwiGLU) or
// o in LDS and store 16-byte row chunks.
// ---------------------------------------------------------------------------
constexpr int kP16Slot = 32768 + 8192 + 1024;  // A | B | B scales
constexpr int kP16A = 0, kP16B = 32768, kP16BS = 40960;
// the ring (125952 bytes), reused by the epilogue's staging (four waves x 128
// rows x 128 bf16 columns)
constexpr int kP16Lds = 3 * kP16Slot > 4 * 128 * 128 * 2 ? 3 * kP16Slot : 4 * 128 * 128 * 2;
// Work order: groups of one tile (all column blocks of a tile, then the
// next), so an XCD's workgroups at any time cover two tiles of gate_up (one
// of down) and share their bf16 activation windows through its L2.  A bf16
// row is twice an MXFP8 one, and groups of four tiles (the MXFP8 kernel's
// order) re-read the windows of each tile from beyond the L2 for every
// second half of its column blocks (prefill8k gate_up 8.91 -> 8.43 ms, down
// 5.17 -> 4.96 ms against groups of four; groups of two in between).
constexpr int kP16GroupTiles = 1;
__shared__ __attribute__((aligned(1024))) uint8_t p16_lds[kP16Lds];

typedef float v16f_t __attribute__((ext_vector_type(16)));

template <bool GU, bool CANON>
__global__ void __launch_bounds__(256, 1) k_gemm_pf16(FwdArgs a) {
  int tile_idx, nblk;
  if (!pf_work_item(a, GU ? a.dff / 128 : (a.d + 255) / 256, kP16GroupTiles, &tile_idx, &nblk)) return;
  const Tile tile = a.tiles[tile_idx];
  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wu & 1, wn = wu >> 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int K = GU ? a.d : a.dff;
  const int nst = K / 64;                          // K steps of 64
  const int ns128 = K / 128;                       // packed steps of 128
  const bool shared = tile.ex >= a.E;
  const int sidx = tile.ex - a.E;
  const int64_t wrows = GU ? 2 * a.dff : a.d;
  const int64_t wc_stride = wrows * (K / 2), ws_stride = packed_scale_bytes(wrows, K);
  const uint8_t* wc = GU ? (shared ? a.sgu_c + sidx * wc_stride : a.gu_c + tile.ex * wc_stride)
                         : (shared ? a.sdn_c + sidx * wc_stride : a.dn_c + tile.ex * wc_stride);
  const uint8_t* ws = GU ? (shared ? a.sgu_s + sidx * ws_stride : a.gu_s + tile.ex * ws_stride)
                         : (shared ? a.sdn_s + sidx * ws_stride : a.dn_s + tile.ex * ws_stride);
  // the tile's four packed groups 4 nblk .. 4 nblk + 3 (gate_up: the gate
  // and up rows of h columns c0 .. c0+127; down: output columns c0 ..
  // c0+255); wave w copies group w.  Down with d an odd multiple of 128:
  // the waves of the missing half of the last block copy group grp0 again
  // and store nothing
  const int grp0 = 4 * nblk;
  const int c0 = GU ? 128 * nblk : 256 * nblk;
  const int64_t gw = GU || grp0 + wu < a.d / 64 ? grp0 + wu : grp0;
  const bool cols_live = GU || c0 + 128 * wn < a.d;
  const bool routed = tile.row_begin < a.Rr;
  const int nrows = tile.row_end - tile.row_begin;

  // activation source rows of this wave's copies: copy j moves the 8-row
  // group wu + 4j (rows past the tile's end read its first row), and a tile of
  // nb 32-row blocks takes copies j < nb, so the four waves copy exactly its
  // 4 nb groups; gate_up x rows (routed: through row -> token), down h rows
  // (contiguous)
  const uint16_t* act = GU ? a.x : a.h16;
  const uint8_t* a_src[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rl = 8 * wu + 32 * q + (lane >> 3);
    const int row = tile.row_begin + (rl < nrows ? rl : 0);
    int64_t srow = row;
    if (GU) srow = routed ? a.row_token[row] : row - a.Rr - int64_t(sidx) * a.T;
    a_src[q] = reinterpret_cast<const uint8_t*>(act) + srow * (2 * int64_t(K)) + 16 * ((lane & 7) ^ ((rl >> 1) & 7));
  }
  // weight copies: copy c (0, 1) moves blocks 2c (lanes 0-31) and 2c+1
  // (lanes 32-63) of group gw, 16 bytes a lane
  const uint8_t* b_src[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int jb = 2 * c + (lane >> 5), l = lane & 31;
    if (CANON) {
      const int64_t crow = (GU ? 32 * gw : 64 * gw) + canon_row_off<GU>(jb, a.dff) + (l & 15);
      b_src[c] = wc + crow * (K / 2) + 16 * (l >> 4);
    } else {
      b_src[c] = wc + gw * ns128 * 4096 + jb * 1024 + 16 * l;
    }
  }
  // their scales: packed, lanes 0-31 take the half's 32 dwords; canonical,
  // every lane the dword of row (lane/16 block, lane%16)
  const uint8_t* bs_src =
      CANON ? ws + ((GU ? 32 * gw : 64 * gw) + canon_row_off<GU>(lane >> 4, a.dff) + (lane & 15)) * (K / 32)
            : ws + gw * ns128 * 256 + 4 * (lane & 31);
  const uint32_t lds0 = lds_addr(p16_lds);
  // copy c of step st for a tile of NB row blocks: activations (c < NB),
  // weights (NB, NB+1), weight scales (NB+2).  Steps past K re-read the last
  // step into a slot that is not read again, so that every step issues the
  // same NB + 3 copies and every wait on them is a constant.
  auto issue_one = [&](int st, auto cc, auto nbc) {
    constexpr int c = decltype(cc)::value, NB = decltype(nbc)::value;
    const int ss = st < nst ? st : nst - 1;
    const uint32_t slot = lds0 + (st % 3) * kP16Slot;
    const int h = ss & 1, s128 = ss >> 1;
    if constexpr (c < NB) {
      lds_copy16(a_src[c] + 128 * int64_t(ss), slot + kP16A + (8 * wu + 32 * c) * 128);
    } else if constexpr (c < NB + 2) {
      const uint8_t* src = CANON ? b_src[c - NB] + 32 * int64_t(ss) : b_src[c - NB] + int64_t(s128) * 4096 + 512 * h;
      lds_copy16(src, slot + kP16B + wu * 2048 + (c - NB) * 1024);
    } else if constexpr (CANON) {
      lds_copy4(bs_src + 4 * s128, slot + kP16BS + wu * 256);
    } else {
      if (lane < 32) lds_copy4(bs_src + int64_t(s128) * 256 + 128 * h, slot + kP16BS + wu * 256);
    }
  };

  // row blocks: nb / 2 whole ones per wave (the first half of the tile's
  // blocks for wm = 0, the last for wm = 1) and, for odd nb, the middle
  // block hb shared by both, each taking half of its weight fragments
  // (gate_up: the gate and up fragments of h columns 32 wm .. of the wave's
  // 64; down: output columns 64 wm .. of its 128).  Accumulator set i < nfull
  // is block rb0 + i, set nfull the shared block.
  const int nb = (nrows + 31) >> 5;
  const int nfull = nb >> 1, hb = nb >> 1;
  const int rb0 = wm ? (nb + 1) >> 1 : 0;
  // accumulator p holds weight fragment pc(p): numbered per wave so that the
  // shared block's half is p = 0, 2 (gate_up) or p = 0, 1 (down) in both
  // row-half waves
  auto pc = [&](int p) -> int { return GU ? (((p & 1) ^ wm) | (p & 2)) : p ^ (2 * wm); };
  // operand offsets: weight fragment f (32 rows): 16-row chunk j0(f) of the
  // tile's sixteen (gate_up: gate rows of h columns 32f .. of groups 2wn,
  // 2wn+1 for f < 2, their up rows for f >= 2; down: 32 output columns each)
  auto j0 = [&](int f) -> int { return GU ? (f < 2 ? 8 * wn + 4 * f : 8 * wn + 4 * (f - 2) + 2) : 8 * wn + 2 * f; };
  int b_off[4], bs_off[4], bs_sh[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int jc = j0(pc(p)) + (l32 >> 4), grp = jc >> 2, jb = jc & 3, r = l32 & 15;
    b_off[p] = kP16B + grp * 2048 + jb * 512 + 16 * (16 * kh + r);
    bs_off[p] = kP16BS + grp * 256 + 4 * (CANON ? 16 * jb + r : 16 * kh + r);
    bs_sh[p] = CANON ? 8 * kh : 8 * jb;              // + 16 h for canonical
  }

  v16f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[i][p] = v16f_t{};

  // A step: after the barrier, the weight fragments and their scales, and the
  // activation fragments of slice 0; then per slice q the activation reads of
  // slice q+1 go out first, and each fragment's expansion, MFMAs and one of
  // the eleven copies of step st+2 follow in a fixed order (one scheduling
  // region per fragment), so the copies spread over the step's MFMAs.
  auto main_loop = [&](auto nact_c, auto half_c) {
    constexpr int NACT = decltype(nact_c)::value;
    constexpr bool HALF = decltype(half_c)::value != 0;
    constexpr int NSET = NACT + (HALF ? 1 : 0);   // accumulator sets in use
    constexpr int NB = 2 * NACT + (HALF ? 1 : 0);  // the tile's row blocks
    constexpr int NCOP = NB + 3;                   // copies per wave and step
    static_for<0, NCOP>([&](auto cc) { issue_one(0, cc, IntC<NB>{}); });
    static_for<0, NCOP>([&](auto cc) { issue_one(1, cc, IntC<NB>{}); });
    for (int st = 0; st < nst; ++st) {
      PF_WAIT_VM(NCOP);                       // this wave's copies of step st have landed
      __syncthreads();
      if constexpr (NSET == 0) {
        static_for<0, NCOP>([&](auto cc) { issue_one(st + 2, cc, IntC<NB>{}); });
      } else {
        const uint8_t* sl = p16_lds + (st % 3) * kP16Slot;
        const int h = st & 1;
        uint4 bw[4];
        float bscl[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          bw[p] = *reinterpret_cast<const uint4*>(sl + b_off[p]);
          const uint32_t sb = (*reinterpret_cast<const uint32_t*>(sl + bs_off[p]) >> (bs_sh[p] + (CANON ? 16 * h : 0))) & 0xFFu;
          bscl[p] = __uint_as_float(sb ? sb << 23 : 0x00400000u);   // 2^(sb-127)
        }
        v8bf16 av[2][NSET];
        auto read_a = [&](auto qc) {
          constexpr int q = decltype(qc)::value;
#pragma unroll
          for (int i = 0; i < NSET; ++i) {
            const int row = 32 * (i < NACT ? rb0 + i : hb) + l32;
            av[q & 1][i] = *reinterpret_cast<const v8bf16*>(sl + kP16A + row * 128 + 16 * ((4 * kh + q) ^ ((row >> 1) & 7)));
          }
        };
        read_a(IntC<0>{});
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, 4>([&](auto qc) {
          constexpr int q = decltype(qc)::value;
          if constexpr (q < 3) read_a(IntC<q + 1>{});
          __builtin_amdgcn_sched_barrier(0);
          static_for<0, 4>([&](auto pcc) {
            constexpr int p = decltype(pcc)::value;
            const uint32_t w = q == 0 ? bw[p].x : q == 1 ? bw[p].y : q == 2 ? bw[p].z : bw[p].w;
            const v2bf16 e0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bscl[p], 0);
            const v2bf16 e1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bscl[p], 1);
            const v2bf16 e2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bscl[p], 2);
            const v2bf16 e3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, bscl[p], 3);
            const v8bf16 bv = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
            for (int i = 0; i < NACT; ++i)
              acc[i][p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[q & 1][i], bv, acc[i][p], 0, 0, 0);
            if constexpr (HALF && (GU ? (p & 1) == 0 : p < 2))
              acc[NACT][p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[q & 1][NACT], bv, acc[NACT][p], 0, 0, 0);
            constexpr int c = 4 * q + p - 2;       // copies in regions 2 .. NCOP + 1
            if constexpr (c >= 0 && c < NCOP) issue_one(st + 2, IntC<c>{}, IntC<NB>{});
            __builtin_amdgcn_sched_barrier(0);
          });
        });
      }
    }
  };
  switch (nb) {
    case 8: main_loop(IntC<4>{}, IntC<0>{}); break;
    case 7: main_loop(IntC<3>{}, IntC<1>{}); break;
    case 6: main_loop(IntC<3>{}, IntC<0>{}); break;
    case 5: main_loop(IntC<2>{}, IntC<1>{}); break;
    case 4: main_loop(IntC<2>{}, IntC<0>{}); break;
    case 3: main_loop(IntC<1>{}, IntC<1>{}); break;
    case 2: main_loop(IntC<1>{}, IntC<0>{}); break;
    case 1: main_loop(IntC<0>{}, IntC<1>{}); break;
    default: main_loop(IntC<0>{}, IntC<0>{}); break;
  }
  // every copy has landed and every wave is past its last operand read: the
  // ring becomes the epilogue's staging area, a private region per wave
  PF_WAIT_VM(0);
  __syncthreads();
  const int nset = nfull + (nb & 1);
  if (nset == 0 || !cols_live) return;

  // Epilogue: register r of acc[i][p] is tile row 32 rb(i) + 8(r/4) + 4 kh +
  // r%4, column l32 of fragment pc(p); it becomes staged row 32i + .. of the
  // wave.  The bf16 outputs (h after SwiGLU: 64 columns; o: 128 columns) are
  // staged in LDS, then leave as 16-byte row chunks.  Staging: registers r,
  // r+1 of a lane hold rows R, R+1 of one column; one exchange with the
  // neighbouring lane gives the even lane row R and the odd lane row R+1, each
  // for two adjacent columns, written as one packed dword.  A staged row's
  // 32-column chunks are permuted by bits 0 and 2 of the row (gate_up: bit 2)
  // so that the four rows one write instruction touches fall on distinct
  // banks.
  constexpr int SC = GU ? 64 : 128;                        // staged columns
  uint16_t* os = reinterpret_cast<uint16_t*>(p16_lds) + wu * (128 * SC);
  auto chunk_of = [](int rl, int c32) {
    return GU ? c32 ^ ((rl >> 2) & 1) : c32 ^ ((rl & 1) | (((rl >> 2) & 1) << 1));
  };
  const bool odd = (lane & 1) != 0;
  auto stage_pair = [&](int i, int r, int f, float v0, float v1) {
    const float rv = dpp_xor1(odd ? v0 : v1);
    const v2bf16 pk = __builtin_convertvector((v2f){odd ? rv : v0, odd ? v1 : rv}, v2bf16);
    const int rl = 32 * i + 8 * (r / 4) + 4 * kh + (r % 4) + (odd ? 1 : 0);
    *reinterpret_cast<uint32_t*>(os + rl * SC + chunk_of(rl, f) * 32 + (l32 & ~1)) = __builtin_bit_cast(uint32_t, pk);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= nset) break;
    const bool shared_blk = i == nfull;
    if (GU) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (shared_blk && pp != 0) continue;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float g0 = acc[i][pp][r], u0 = acc[i][pp + 2][r];
          const float g1 = acc[i][pp][r + 1], u1 = acc[i][pp + 2][r + 1];
          stage_pair(i, r, pc(pp), g0 / (1.0f + __expf(-g0)) * u0, g1 / (1.0f + __expf(-g1)) * u1);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (shared_blk && p >= 2) continue;
#pragma unroll
        for (int r = 0; r < 16; r += 2) stage_pair(i, r, pc(p), acc[i][p][r], acc[i][p][r + 1]);
      }
    }
  }
  // (the optional accumulator tap straight from the registers)
  if (GU && a.gu_acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nset) break;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        if (i == nfull && pp != 0) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * (i < nfull ? rb0 + i : hb) + 8 * (r / 4) + 4 * kh + (r % 4);
          if (rl < nrows) {
            const int64_t row = tile.row_begin + rl;
            const int col = c0 + 64 * wn + 32 * pc(pp) + l32;
            a.gu_acc[row * 2 * a.dff + col] = acc[i][pp][r];
            a.gu_acc[row * 2 * a.dff + a.dff + col] = acc[i][pp + 2][r];
          }
        }
      }
    }
  }
  // stores: a wave's staged rows in 16-byte chunks, SC / 8 chunks per row;
  // the shared block's rows hold columns 32 wm .. (gate_up) or 64 wm ..
  // (down) of the wave's only
  constexpr int CPR = SC / 8;                              // chunks per row
#pragma unroll 4
  for (int q = 0; q < 128 * CPR / 64; ++q) {
    const int ch = q * 64 + lane;
    const int rl = ch / CPR, cc = 8 * (ch % CPR);
    const int ib = rl >> 5;
    const int trow = 32 * (ib < nfull ? rb0 + ib : hb) + (rl & 31);   // tile row
    const bool col_ok = ib != nfull || (GU ? (cc >> 5) == wm : (cc >> 6) == wm);
    if (ib < nset && trow < nrows && col_ok) {
      const uint4 t = *reinterpret_cast<const uint4*>(os + rl * SC + chunk_of(rl, cc >> 5) * 32 + (cc & 31));
      const int64_t row = tile.row_begin + trow;
      if (GU) {
        *reinterpret_cast<uint4*>(a.h16 + row * a.dff + c0 + 64 * wn + cc) = t;
      } else {
        const int64_t dst = routed ? a.row_src[row] : row;
        *reinterpret_cast<uint4*>(a.o16 + dst * a.d + c0 + 128 * wn + cc) = t;
      }
    }
  }
}

template <bool GU>
static hipError_t launch_pf16(const FwdArgs& a, hipStream_t st) {
  const int64_t N = GU ? a.dff / 128 : (a.d + 255) / 256;
  const int64_t max_groups = (int64_t(a.max_tiles) + kP16GroupTiles - 1) / kP16GroupTiles;
  const int64_t per_xcd = (max_groups + 7) / 8 * kP16GroupTiles * N;
  const dim3 grid(static_cast<unsigned>(8 * per_xcd));
  if (a.wcanon)
    hipLaunchKernelGGL((k_gemm_pf16<GU, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_pf16<GU, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// The routing launch of a few tokens: top-k and permutation in workgroup 0,
// the shared experts' gate_up items in the others (PH = 1).
hipError_t launch_topk_shared_gate_up(const FwdArgs& a, hipStream_t st) {
  const unsigned grid = 8u * static_cast<unsigned>(a.num_cus >= 16 ? a.num_cus / 8 : 1);
  if (a.a16 && a.wcanon)
    hipLaunchKernelGGL((k_gemm_stream<true, true, false, true, 1, true>), dim3(grid), dim3(256), 0, st, a);
  else if (a.a16)
    hipLaunchKernelGGL((k_gemm_stream<true, true, false, true, 1>), dim3(grid), dim3(256), 0, st, a);
  else if (a.wcanon)
    hipLaunchKernelGGL((k_gemm_stream<true, true, false, false, 1, true>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_stream<true, true, false, false, 1>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const FwdArgs& a, hipStream_t st) {
  if (a.bm <= kDecodeMaxRows) return launch_stream<true>(a, st);
  if (a.a16) return launch_pf16<true>(a, st);
  return launch_pf<true>(a, st);
}

hipError_t launch_gemm_down(const FwdArgs& a, hipStream_t st) {
  if (a.bm <= kDecodeMaxRows) return launch_stream<false>(a, st);
  if (a.a16) return launch_pf16<false>(a, st);
  return launch_pf<false>(a, st);
}

}  // namespace mxmoe

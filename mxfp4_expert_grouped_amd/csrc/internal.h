// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

// One unit of grouped-GEMM work: rows [row_begin, row_end) of expert `ex`
// (ex < E: routed expert; ex >= E: shared expert ex - E).
struct Tile {
  int32_t ex, row_begin, row_end, pad;
};

// Everything the kernels of one forward need; all pointers are device memory.
struct FwdArgs {
  // shape
  int T, d, dff, E, k, S;
  int R;         // permuted rows: T*k routed + S*T shared
  int Rr;        // routed rows T*k
  // inputs
  const uint16_t* x;    // bf16 [T][d]
  const float* wr;      // [E][d]
  const float* br;      // [E] or null
  const uint8_t *gu_c, *gu_s, *dn_c, *dn_s;      // routed weights
  const uint8_t *sgu_c, *sgu_s, *sdn_c, *sdn_s;  // shared weights
  // outputs
  uint16_t* y;  // bf16 [T][d]
  // workspace buffers (or caller taps substituted for them)
  float* logits;        // [T][E]
  float* router_part;   // [router_ks][T][E] split-K partial logits (router_ks > 1)
  int32_t* topk_ids;    // [T][k]
  float* topk_w;        // [T][k]
  uint8_t* x_codes;     // [T][d]
  uint8_t* x_scales;    // [T][d/32]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* row_src;     // [Rr]   pair index
  int32_t* row_token;   // [Rr]   token of each routed row
  int32_t* token_row;   // [T][k]
  uint64_t* chunk_mask; // [nchunks][E]
  int32_t* chunk_base;  // [E][nchunks]
  Tile* tiles;          // [max_tiles], grouped by expert (routed ascending, then shared)
  int32_t* tile_count;  // [1]
  int32_t* ex_tiles;    // [E+S+1] first tile of each expert (prefix over tile counts)
  uint8_t* h_codes;     // [R][dff]
  uint8_t* h_scales;    // [R][dff/32]
  uint16_t* h16;        // [R][dff] bf16 h (A16W4 variant), else unused
  int a16;              // 1: A16W4 variant (bf16 x and h, no MXFP8 activations)
  uint16_t* o16;        // [R][d] bf16 down outputs: permuted-row order after the
                        // decode kernels, (token, slot) order after the prefill ones
  // optional taps (null = skip)
  float* gu_acc;        // [R][2*dff]
  float* y_routed;      // [T][d]
  float* y_shared;      // [T][d]
  // launch-time choices
  int router_ks;        // K slices of the MFMA router (1: no partials)
  int bm;               // rows per tile: 8 (decode kernels) or 256 (prefill kernels)
  int num_cus;          // compute units of the device (persistent decode grid)
  int max_tiles;
  int nchunks;          // 64-token chunks
  // the prefill down GEMM's K split (LatentMoE tail only): > 1 cuts K into
  // ksplit equal slices (multiples of 512) and writes fp32 partials
  // kpart[slice][R][d] in row order instead of bf16 o rows
  int ksplit;
  float* kpart;
  // 1: expert weights in the canonical layout ([N][K/2] codes, [N][K/32]
  // scales) instead of the packed one
  int wcanon;
};

// Everything the kernels of one LatentMoE tail call need (device pointers).
struct TailArgs {
  int T, latent, hidden, bm;
  float eps;
  const float* z;        // [T][latent] routed experts' weighted sum
  const float* gamma;    // [latent]
  const float* s;        // [T][hidden] shared experts' output, or null
  const uint8_t *up_c, *up_s;  // MXFP4 W_up [hidden][latent], packed or canonical
  int wcanon;                  // 1: canonical layout
  uint16_t* y;           // bf16 [T][hidden]
  uint8_t* codes;        // [T][latent] MXFP8 of the normalised rows
  uint8_t* scales;       // [T][latent/32]
  float* inv_rms;        // [T] tap, or null
  uint16_t* o16;         // [T][hidden] projection (y itself when s is null)
  int32_t* row_src;      // [T] identity
  Tile* tiles;           // [ceil(T/bm)]
  int32_t* tile_count;   // [1]
  int32_t* ex_tiles;     // [2]
  float* part;           // [slices][T][hidden] split-K partials (T <= kTailGemvMaxT)
};

// The tail's projection for at most kTailGemvMaxT rows runs split along K:
// each wave takes at most kTailGemvSteps of the 128-wide K steps.
constexpr int kTailGemvMaxT = 16;
constexpr int kTailGemvSteps = 4;
inline int tail_gemv_slices(int latent) {
  const int ns = latent / 128;
  return (ns + 4 * kTailGemvSteps - 1) / (4 * kTailGemvSteps);
}

// Rows per tile of the decode (weight-streaming) kernels; larger tiles go to
// the prefill kernels.
constexpr int kDecodeMaxRows = 8;

// Rows per tile of the LatentMoE tail's projection: the weight-streaming
// kernel for a few rows; from 24 rows on the prefill kernel, on 64-row tiles
// up to 512 rows (more tiles per column block, so fewer K slices and fp32
// partials are needed to fill the chip) and 256-row tiles above.
inline int tail_tile_rows(int64_t T) { return T < 24 ? kDecodeMaxRows : T <= 512 ? 64 : 256; }
// K slices of the tail's projection on those tiles, when its tiles x
// 256-column blocks alone would give fewer workgroups than three quarters of
// the 256 CUs: the smallest divisor of latent/512 (at most 8) that reaches
// 192 workgroups, else the largest.  Each slice adds one fp32 partial of the
// output, summed in order (with s) by the tail's reduction.
inline int tail_ksplit(int64_t T, int64_t latent, int64_t hidden, int64_t bm) {
  if (T < 24 || latent % 512 != 0) return 1;
  const int64_t base = ((T + bm - 1) / bm) * ((hidden + 255) / 256);
  const int64_t g = latent / 512;
  int best = 1;
  for (int d = 1; d <= 8 && d <= g; ++d) {
    if (g % d != 0) continue;
    best = d;
    if (base * d >= 192) break;
  }
  return best;
}

// Launchers (kernels_*.hip).  Each returns hipSuccess or the launch error.
hipError_t launch_tail(const TailArgs& a, int num_cus, hipStream_t st);
hipError_t launch_quantize(const void* src, int src_fp32, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t* codes, uint8_t* scales, hipStream_t st);

// Tokens up to which the per-expert GEMV router (with the x quantisation
// fused) runs; above it, the bf16 MFMA router.
constexpr int kRouterSmallMaxT = 32;
inline bool router_small(int64_t T, int64_t d, int64_t E) { return T <= kRouterSmallMaxT && T * (d / 32) <= 32 * E; }

// K slices of the MFMA router for T tokens: few 128x128 output tiles are
// spread over the GPU by cutting d into up to 16 slices of at least 512.
inline int router_splits(int64_t T, int64_t E, int64_t d) {
  const int64_t tiles = ((T + 127) / 128) * ((E + 127) / 128);
  if (tiles >= 256) return 1;
  int64_t ks = (256 + tiles - 1) / tiles;
  if (ks > d / 512) ks = d / 512;
  if (ks > 16) ks = 16;
  return ks < 1 ? 1 : static_cast<int>(ks);
}

// The few-token forward splits its gate_up in two launches (top-k +
// permutation + shared experts, then the routed experts) when routing runs in
// one workgroup and every tile is a weight-streaming one, with the K split.
inline bool stream_split_phases(const FwdArgs& a) {
  return router_small(a.T, a.d, a.E) && a.bm <= kDecodeMaxRows && a.S > 0;
}

hipError_t launch_router_bias_update(const int32_t* offsets, int E, int64_t tk, float rate, float* b,
                                     hipStream_t st);
hipError_t launch_router(const FwdArgs& a, hipStream_t st);
hipError_t launch_topk_shared_gate_up(const FwdArgs& a, hipStream_t st);
hipError_t launch_topk_quant(const FwdArgs& a, hipStream_t st);
hipError_t launch_permute(const FwdArgs& a, hipStream_t st);
hipError_t launch_gemm_gate_up(const FwdArgs& a, hipStream_t st);
hipError_t launch_gemm_down(const FwdArgs& a, hipStream_t st);
hipError_t launch_combine(const FwdArgs& a, hipStream_t st);
hipError_t launch_pack_mx4(const uint8_t* codes, const uint8_t* scales, int64_t mats, int64_t rows,
                           int64_t k, int interleave, uint8_t* codes_p, uint8_t* scales_p, hipStream_t st);

// bytes of one packed scale matrix [rows/16][ceil(k/512)][64][4]
__host__ __device__ inline int64_t packed_scale_bytes(int64_t rows, int64_t k) { return rows * (k / 32); }

// token counts at or below which the single-workgroup permutation is used
constexpr int kPermSmallMaxTokens = 1024;

}  // namespace mxmoe

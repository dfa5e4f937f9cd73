// C ABI of the MoE layer: argument checks, plan, workspace layout and the
// launch sequence router -> top-k/quantise -> permute -> gate_up -> down ->
// combine on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mxmoe.h"
#include "internal.h"

using namespace mxmoe;

struct moe_plan_s {
  moe_config cfg;
  // optional per-stage timing (moe_profile_begin / moe_profile_end)
  uint32_t prof_mask = 0;
  int prof_cap = 0, prof_n = 0;
  std::vector<hipEvent_t> prof_ev;  // [prof_cap][MOE_NUM_STAGES][2]
};

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checked once per device: a visible gfx950 device is current.  Also gives
// its compute-unit count.  The per-device cache holds the compute-unit count
// (0 = not yet checked) in one atomic word, so threads that check the same
// device at once at worst both query it and store the same value.
moe_status check_device(int* num_cus = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "no HIP device available");
  }
  static std::atomic<int> cus[64];  // zero-initialised (static storage)
  if (dev < 64) {
    const int c = cus[dev].load(std::memory_order_acquire);
    if (c > 0) {
      if (num_cus) *num_cus = c;
      return MOE_OK;
    }
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_DEVICE, "device %d is %s, the kernels are built for gfx950", dev,
                prop.gcnArchName);
  const int c = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  if (dev < 64) cus[dev].store(c, std::memory_order_release);
  if (num_cus) *num_cus = c;
  return MOE_OK;
}

// rows per grouped-GEMM tile: 8 when experts see few rows (weight-streaming
// decode kernels), else 256 (LDS-staged prefill kernels)
int choose_bm(const moe_config& c, int64_t T) {
  int64_t avg = (T * c.top_k) / c.num_experts;
  return avg >= 24 ? 256 : kDecodeMaxRows;
}

struct Layout {
  size_t logits, router_part, topk_ids, topk_w, x_codes, x_scales, counts, offsets, row_src, row_token,
      token_row, chunk_mask, chunk_base, tiles, tile_count, ex_tiles, h_codes, h_scales, o, total;
  int bm, max_tiles, nchunks, router_ks;
};

Layout make_layout(const moe_config& c, int64_t T) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  const int64_t E = c.num_experts, k = c.top_k, S = c.num_shared, d = c.d_model, f = c.d_ff;
  const int64_t Rr = T * k, R = Rr + S * T;
  L.bm = choose_bm(c, T);
  L.nchunks = static_cast<int>((T + 63) / 64);
  L.max_tiles = static_cast<int>((Rr + L.bm - 1) / L.bm + std::min<int64_t>(E, Rr) +
                                 S * ((T + L.bm - 1) / L.bm));
  L.logits = take(T * E * 4);
  L.router_ks = router_small(T, d, E) ? 1 : router_splits(T, E, d);
  L.router_part = take(L.router_ks > 1 ? size_t(L.router_ks) * T * E * 4 : 0);
  L.topk_ids = take(T * k * 4);
  L.topk_w = take(T * k * 4);
  L.x_codes = take(T * d);
  L.x_scales = take(T * d / 32);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.row_src = take(Rr * 4);
  // eight spare entries: the decode GEMM loads a tile's eight row-token
  // entries with one scalar load, past the last routed row for the last tile
  L.row_token = take((Rr + 8) * 4);
  L.token_row = take(T * k * 4);
  L.chunk_mask = take(size_t(L.nchunks) * E * 8);
  L.chunk_base = take(size_t(L.nchunks) * E * 4);
  L.tiles = take(size_t(std::max(L.max_tiles, 1)) * sizeof(Tile));
  L.tile_count = take(4);
  L.ex_tiles = take((E + S + 1) * 4);
  if (c.flags & MOE_FLAG_A16W4) {
    L.h_codes = take(R * f * 2);   // bf16 h
    L.h_scales = take(0);
  } else {
    L.h_codes = take(R * f);
    L.h_scales = take(R * f / 32);
  }
  L.o = take(R * d * 2);
  L.total = off;
  return L;
}

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->d_model <= 0 || c->d_ff <= 0 || c->num_experts <= 0 || c->top_k <= 0 ||
      c->num_shared < 0 || c->max_tokens <= 0)
    return fail(MOE_ERR_INVALID_ARG, "non-positive size in config");
  if (c->flags & ~MOE_FLAG_A16W4) return fail(MOE_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
  if (c->d_model % 128 || c->d_ff % 128)
    return fail(MOE_ERR_UNSUPPORTED, "d_model (%d) and d_ff (%d) must be multiples of 128",
                c->d_model, c->d_ff);
  if (c->d_model > 65536 || c->d_ff > 65536)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be <= 65536");
  if (c->num_experts > 1024) return fail(MOE_ERR_UNSUPPORTED, "num_experts must be <= 1024");
  if (c->top_k > 32 || c->top_k > c->num_experts)
    return fail(MOE_ERR_UNSUPPORTED, "top_k must be <= min(32, num_experts)");
  if (c->num_shared > 8) return fail(MOE_ERR_UNSUPPORTED, "num_shared must be <= 8");
  if (c->max_tokens > (1 << 20)) return fail(MOE_ERR_UNSUPPORTED, "max_tokens must be <= 2^20");
  // permuted-row indices and element offsets must fit the kernels' int32 row math
  if ((c->max_tokens * (c->top_k + c->num_shared)) > (int64_t(1) << 30))
    return fail(MOE_ERR_UNSUPPORTED, "max_tokens * (top_k + num_shared) too large");
  // MXFP8 activation buffers are addressed with 31-bit byte offsets
  if (c->max_tokens * c->d_model >= (int64_t(1) << 31) ||
      c->max_tokens * (c->top_k + c->num_shared) * c->d_ff >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "activation buffers exceed 2^31 bytes");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_plan(const moe_config* cfg, moe_plan_t** out_plan) {
  if (!out_plan) return fail(MOE_ERR_INVALID_ARG, "out_plan is NULL");
  *out_plan = nullptr;
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  moe_plan_t* p = new (std::nothrow) moe_plan_t;
  if (!p) return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  p->cfg = *cfg;
  *out_plan = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan_t* plan) {
  if (!plan) return;
  for (hipEvent_t x : plan->prof_ev)
    if (x) (void)hipEventDestroy(x);
  delete plan;
}

moe_status moe_workspace_bytes(const moe_plan_t* plan, int64_t num_tokens, size_t* out_bytes) {
  if (!plan || !out_bytes) return fail(MOE_ERR_INVALID_ARG, "plan or out_bytes is NULL");
  if (num_tokens < 0 || num_tokens > plan->cfg.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "num_tokens %lld outside [0, max_tokens]",
                static_cast<long long>(num_tokens));
  *out_bytes = num_tokens == 0 ? 0 : make_layout(plan->cfg, num_tokens).total;
  return MOE_OK;
}

moe_status moe_quantize_act(const void* src, moe_src_dtype dt, int64_t rows, int64_t cols,
                            int64_t ld_src, uint8_t* codes, uint8_t* scales, void* stream) {
  if (dt != MOE_SRC_BF16 && dt != MOE_SRC_FP32) return fail(MOE_ERR_INVALID_ARG, "bad dtype");
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "negative size");
  if (cols % 32) return fail(MOE_ERR_UNSUPPORTED, "cols (%lld) must be a multiple of 32",
                             static_cast<long long>(cols));
  if (ld_src < cols) return fail(MOE_ERR_INVALID_ARG, "ld_src < cols");
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!src || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL buffer");
  const int esz = dt == MOE_SRC_FP32 ? 4 : 2;
  if (!aligned(src, 16) || (ld_src * esz) % 16 || !aligned(codes, 16))
    return fail(MOE_ERR_UNSUPPORTED, "src/codes must be 16-byte aligned and rows 16-byte strided");
  moe_status s = check_device();
  if (s != MOE_OK) return s;
  hipError_t e = launch_quantize(src, dt == MOE_SRC_FP32, rows, cols, ld_src, codes, scales,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

size_t moe_packed_scale_bytes(int64_t rows, int64_t k) {
  if (rows <= 0 || k <= 0 || rows % 64 || k % 128) return 0;
  return static_cast<size_t>(packed_scale_bytes(rows, k));
}

moe_status moe_pack_mx4(const uint8_t* codes, const uint8_t* scales, int64_t mats, int64_t rows,
                        int64_t k, int interleave, uint8_t* codes_p, uint8_t* scales_p,
                        void* stream) {
  if (mats < 0 || rows < 0 || k < 0) return fail(MOE_ERR_INVALID_ARG, "negative size");
  if (interleave != 0 && interleave != 1) return fail(MOE_ERR_INVALID_ARG, "interleave must be 0 or 1");
  if (rows % 64 || k % 128)
    return fail(MOE_ERR_UNSUPPORTED, "rows must be a multiple of 64 and k of 128");
  if (mats == 0 || rows == 0 || k == 0) return MOE_OK;
  if (!codes || !scales || !codes_p || !scales_p) return fail(MOE_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(codes, 16) || !aligned(codes_p, 16) || !aligned(scales_p, 4))
    return fail(MOE_ERR_INVALID_ARG, "codes/codes_p need 16-byte, scales_p 4-byte alignment");
  moe_status s = check_device();
  if (s != MOE_OK) return s;
  hipError_t e = launch_pack_mx4(codes, scales, mats, rows, k, interleave, codes_p, scales_p,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // extern "C"

namespace {

// Scratch memory of moe_forward_noalloc: one array per GPU in the library's
// code object, allocated when the code object is loaded on that device and
// held until the process ends.  In host code `noalloc_scratch` names a
// host-side stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t noalloc_scratch[kNoAllocScratchBytes];

// Device address of this device's scratch array (looked up once per device;
// concurrent first calls look it up twice and store the same address).
moe_status noalloc_scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "no usable HIP device (index %d)", dev);
  }
  static std::atomic<void*> ptrs[64];
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (!p) {
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress of the scratch array failed on device %d: %s",
                  dev, hipGetErrorString(e));
    }
    ptrs[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

// workspace == nullptr with noalloc: the per-device scratch array
moe_status forward_impl(const moe_plan_t* plan, const moe_weights* w, const void* x_bf16,
                        int64_t num_tokens, void* y_bf16, void* workspace, size_t workspace_bytes,
                        const moe_taps* taps, void* stream, bool noalloc) {
  if (!plan) return fail(MOE_ERR_INVALID_ARG, "plan is NULL");
  const moe_config& c = plan->cfg;
  if (num_tokens < 0 || num_tokens > c.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "num_tokens %lld outside [0, %lld]",
                static_cast<long long>(num_tokens), static_cast<long long>(c.max_tokens));
  if (num_tokens == 0) return MOE_OK;
  if (!w || !x_bf16 || !y_bf16) return fail(MOE_ERR_INVALID_ARG, "weights, x or y is NULL");
  if (w->layout != MOE_WEIGHTS_PACKED && w->layout != MOE_WEIGHTS_CANONICAL)
    return fail(MOE_ERR_INVALID_ARG,
                "weights.layout is 0x%x: expected MOE_WEIGHTS_PACKED (0x%x, matrices made by "
                "moe_pack_mx4) or MOE_WEIGHTS_CANONICAL (0x%x)",
                w->layout, MOE_WEIGHTS_PACKED, MOE_WEIGHTS_CANONICAL);
  if (!w->gu_codes || !w->gu_scales || !w->dn_codes || !w->dn_scales || !w->router_w)
    return fail(MOE_ERR_INVALID_ARG, "routed-expert or router weight pointer is NULL");
  if (c.num_shared > 0 && (!w->sgu_codes || !w->sgu_scales || !w->sdn_codes || !w->sdn_scales))
    return fail(MOE_ERR_INVALID_ARG, "shared-expert weight pointer is NULL");
  if (!aligned(x_bf16, 16) || !aligned(y_bf16, 16) || !aligned(w->router_w, 16) ||
      !aligned(w->gu_codes, 16) || !aligned(w->dn_codes, 16) || !aligned(w->gu_scales, 4) ||
      !aligned(w->dn_scales, 4) || (w->router_b && !aligned(w->router_b, 4)) ||
      (c.num_shared > 0 && (!aligned(w->sgu_codes, 16) || !aligned(w->sdn_codes, 16) ||
                            !aligned(w->sgu_scales, 4) || !aligned(w->sdn_scales, 4))))
    return fail(MOE_ERR_INVALID_ARG,
                "misaligned buffer (x, y, codes, router_w: 16 bytes; scales, bias: 4 bytes)");
  const bool a16 = (c.flags & MOE_FLAG_A16W4) != 0;
  if (taps && a16 && (taps->x_codes || taps->x_scales || taps->h_codes || taps->h_scales))
    return fail(MOE_ERR_INVALID_ARG, "A16W4 has no MXFP8 activations: x/h code and scale taps must be NULL");
  if (taps && !a16 && taps->h_bf16)
    return fail(MOE_ERR_INVALID_ARG, "the h_bf16 tap exists only in the A16W4 variant");
  const Layout L = make_layout(c, num_tokens);
  if (noalloc) {
    if (L.total > kNoAllocScratchBytes)
      return fail(MOE_ERR_WORKSPACE,
                  "moe_forward_noalloc: %lld tokens need %zu bytes of scratch, above its fixed %zu "
                  "bytes; use moe_forward with a workspace",
                  static_cast<long long>(num_tokens), L.total, kNoAllocScratchBytes);
  } else {
    if (!workspace || workspace_bytes < L.total)
      return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", L.total,
                  workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 256)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (taps) {
    if ((taps->x_codes && !aligned(taps->x_codes, 16)) ||
        (taps->h_codes && !aligned(taps->h_codes, 16)) ||
        (taps->x_scales && !aligned(taps->x_scales, 16)) ||
        (taps->h_scales && !aligned(taps->h_scales, 16)) ||
        (taps->y_routed && !aligned(taps->y_routed, 16)) ||
        (taps->y_shared && !aligned(taps->y_shared, 16)) ||
        (taps->logits && !aligned(taps->logits, 4)) || (taps->topk_w && !aligned(taps->topk_w, 4)) ||
        (taps->topk_ids && !aligned(taps->topk_ids, 4)) ||
        (taps->expert_offsets && !aligned(taps->expert_offsets, 4)) ||
        (taps->row_src && !aligned(taps->row_src, 4)) ||
        (taps->token_row && !aligned(taps->token_row, 4)) || (taps->gu_acc && !aligned(taps->gu_acc, 4)) ||
        (taps->h_bf16 && !aligned(taps->h_bf16, 16)))
      return fail(MOE_ERR_INVALID_ARG, "misaligned tap buffer");
  }
  int num_cus = 0;
  moe_status s = check_device(&num_cus);
  if (s != MOE_OK) return s;
  if (noalloc) {
    s = noalloc_scratch_ptr(&workspace);
    if (s != MOE_OK) return s;
  }

  char* ws = static_cast<char*>(workspace);
  FwdArgs a{};
  a.num_cus = num_cus > 0 ? num_cus : 256;
  a.T = static_cast<int>(num_tokens);
  a.d = c.d_model; a.dff = c.d_ff; a.E = c.num_experts; a.k = c.top_k; a.S = c.num_shared;
  a.Rr = a.T * a.k;
  a.R = a.Rr + a.S * a.T;
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.wr = w->router_w; a.br = w->router_b;
  a.gu_c = w->gu_codes; a.gu_s = w->gu_scales; a.dn_c = w->dn_codes; a.dn_s = w->dn_scales;
  a.sgu_c = w->sgu_codes; a.sgu_s = w->sgu_scales; a.sdn_c = w->sdn_codes; a.sdn_s = w->sdn_scales;
  a.y = static_cast<uint16_t*>(y_bf16);
  auto pick = [&](auto* tap, size_t off, auto* type_tag) {
    using P = decltype(type_tag);
    return tap ? reinterpret_cast<P>(tap) : reinterpret_cast<P>(ws + off);
  };
  const moe_taps none{};
  const moe_taps& tp = taps ? *taps : none;
  a.logits = pick(tp.logits, L.logits, static_cast<float*>(nullptr));
  a.topk_ids = pick(tp.topk_ids, L.topk_ids, static_cast<int32_t*>(nullptr));
  a.topk_w = pick(tp.topk_w, L.topk_w, static_cast<float*>(nullptr));
  a.x_codes = pick(tp.x_codes, L.x_codes, static_cast<uint8_t*>(nullptr));
  a.x_scales = pick(tp.x_scales, L.x_scales, static_cast<uint8_t*>(nullptr));
  a.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  a.offsets = pick(tp.expert_offsets, L.offsets, static_cast<int32_t*>(nullptr));
  a.row_src = pick(tp.row_src, L.row_src, static_cast<int32_t*>(nullptr));
  a.row_token = reinterpret_cast<int32_t*>(ws + L.row_token);
  a.token_row = pick(tp.token_row, L.token_row, static_cast<int32_t*>(nullptr));
  a.chunk_mask = reinterpret_cast<uint64_t*>(ws + L.chunk_mask);
  a.chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  a.tiles = reinterpret_cast<Tile*>(ws + L.tiles);
  a.tile_count = reinterpret_cast<int32_t*>(ws + L.tile_count);
  a.ex_tiles = reinterpret_cast<int32_t*>(ws + L.ex_tiles);
  a.a16 = a16 ? 1 : 0;
  a.wcanon = w->layout == MOE_WEIGHTS_CANONICAL ? 1 : 0;
  if (a16) {
    a.h16 = pick(tp.h_bf16, L.h_codes, static_cast<uint16_t*>(nullptr));
  } else {
    a.h_codes = pick(tp.h_codes, L.h_codes, static_cast<uint8_t*>(nullptr));
    a.h_scales = pick(tp.h_scales, L.h_scales, static_cast<uint8_t*>(nullptr));
  }
  a.o16 = reinterpret_cast<uint16_t*>(ws + L.o);
  a.gu_acc = tp.gu_acc;
  a.y_routed = tp.y_routed;
  a.y_shared = tp.y_shared;
  a.bm = L.bm;
  a.router_ks = L.router_ks;
  a.router_part = reinterpret_cast<float*>(ws + L.router_part);
  a.max_tiles = L.max_tiles;
  a.nchunks = L.nchunks;

  hipStream_t st = static_cast<hipStream_t>(stream);
  moe_plan_t* pl = const_cast<moe_plan_t*>(plan);
  const bool prof = pl->prof_mask && pl->prof_n < pl->prof_cap;
  hipEvent_t* ev = prof ? &pl->prof_ev[size_t(pl->prof_n) * MOE_NUM_STAGES * 2] : nullptr;
  auto stage = [&](int i, hipError_t (*launch)(const FwdArgs&, hipStream_t), const FwdArgs& args) -> bool {
    const bool rec = prof && ((pl->prof_mask >> i) & 1u);
    if (rec) (void)hipEventRecord(ev[2 * i], st);
    if (launch(args, st) != hipSuccess) return false;
    if (rec) (void)hipEventRecord(ev[2 * i + 1], st);
    return true;
  };

  static hipError_t (*const stages[MOE_NUM_STAGES])(const FwdArgs&, hipStream_t) = {
      launch_router, launch_topk_quant, launch_permute, launch_gemm_gate_up, launch_gemm_down, launch_combine};
  for (int i = 0; i < MOE_NUM_STAGES; ++i)
    if (!stage(i, stages[i], a))
      return fail(MOE_ERR_DEVICE, "launch failed: %s", hipGetErrorString(hipGetLastError()));
  if (prof) pl->prof_n++;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_plan_t* plan, const moe_weights* w, const void* x_bf16,
                       int64_t num_tokens, void* y_bf16, void* workspace, size_t workspace_bytes,
                       const moe_taps* taps, void* stream) {
  return forward_impl(plan, w, x_bf16, num_tokens, y_bf16, workspace, workspace_bytes, taps, stream,
                      false);
}

moe_status moe_forward_noalloc(const moe_plan_t* plan, const moe_weights* w, const void* x_bf16,
                               int64_t num_tokens, void* y_bf16, const moe_taps* taps, void* stream) {
  return forward_impl(plan, w, x_bf16, num_tokens, y_bf16, nullptr, 0, taps, stream, true);
}

}  // extern "C"

namespace {

struct TailLayout {
  size_t codes, scales, o16, row_src, tiles, tile_count, ex_tiles, part, total;
  int bm;
};

TailLayout tail_layout(int64_t T, int64_t latent, int64_t hidden, bool with_s) {
  TailLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  // rows per projection tile (tail_tile_rows)
  L.bm = tail_tile_rows(T);
  L.codes = take(T * latent);
  L.scales = take(T * latent / 32);
  L.o16 = take(with_s ? T * hidden * 2 : 0);
  L.row_src = take(T * 4);
  L.tiles = take(((T + L.bm - 1) / L.bm) * sizeof(Tile));
  L.tile_count = take(4);
  L.ex_tiles = take(8);
  // fp32 partials: of the K slices of the few-row projection, or of the
  // K slices of few 256-row tiles
  const int64_t ks = T <= kTailGemvMaxT ? tail_gemv_slices(static_cast<int>(latent))
                   : L.bm > kDecodeMaxRows ? tail_ksplit(T, latent, hidden, L.bm) : 1;
  L.part = take(ks > 1 ? size_t(ks) * T * hidden * 4 : 0);
  L.total = off;
  return L;
}

moe_status check_tail_shape(int64_t T, int32_t latent, int32_t hidden) {
  if (T < 0 || T > (int64_t(1) << 20)) return fail(MOE_ERR_INVALID_ARG, "num_tokens outside [0, 2^20]");
  if (latent <= 0 || hidden <= 0) return fail(MOE_ERR_INVALID_ARG, "non-positive width");
  if (latent % 128 || hidden % 128 || latent > 65536 || hidden > 65536)
    return fail(MOE_ERR_UNSUPPORTED,
                "latent (%d) and hidden (%d) must be multiples of 128, both <= 65536", latent,
                hidden);
  if (T * latent >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "num_tokens * latent must be below 2^31");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_latent_tail_workspace_bytes(int64_t num_tokens, int32_t latent, int32_t hidden,
                                           size_t* out_bytes) {
  if (!out_bytes) return fail(MOE_ERR_INVALID_ARG, "out_bytes is NULL");
  moe_status s = check_tail_shape(num_tokens, latent, hidden);
  if (s != MOE_OK) return s;
  // sized for a call with s (the projection then has rows of its own)
  *out_bytes = num_tokens == 0 ? 0 : tail_layout(num_tokens, latent, hidden, true).total;
  return MOE_OK;
}

moe_status moe_latent_tail(int64_t num_tokens, int32_t latent, int32_t hidden, float eps,
                           const moe_tail_weights* w, const float* z, const float* s, void* y_bf16,
                           void* workspace, size_t workspace_bytes, const moe_tail_taps* taps,
                           void* stream) {
  moe_status st = check_tail_shape(num_tokens, latent, hidden);
  if (st != MOE_OK) return st;
  if (!(eps >= 0.0f) || eps > 3.4e38f) return fail(MOE_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (num_tokens == 0) return MOE_OK;
  if (!w || !z || !y_bf16) return fail(MOE_ERR_INVALID_ARG, "weights, z or y is NULL");
  if (w->layout != MOE_WEIGHTS_PACKED && w->layout != MOE_WEIGHTS_CANONICAL)
    return fail(MOE_ERR_INVALID_ARG,
                "tail weights.layout is 0x%x: expected MOE_WEIGHTS_PACKED or MOE_WEIGHTS_CANONICAL",
                w->layout);
  if (!w->up_codes || !w->up_scales || !w->gamma) return fail(MOE_ERR_INVALID_ARG, "tail weight pointer is NULL");
  if (!aligned(z, 16) || (s && !aligned(s, 16)) || !aligned(y_bf16, 16) || !aligned(w->gamma, 16) ||
      !aligned(w->up_codes, 16) || !aligned(w->up_scales, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "misaligned buffer (z, s, y, gamma, up_codes: 16 bytes; up_scales: 4 bytes)");
  if (taps && ((taps->inv_rms && !aligned(taps->inv_rms, 4)) ||
               (taps->a_codes && !aligned(taps->a_codes, 16)) ||
               (taps->a_scales && !aligned(taps->a_scales, 16))))
    return fail(MOE_ERR_INVALID_ARG, "misaligned tap buffer");
  const TailLayout L = tail_layout(num_tokens, latent, hidden, s != nullptr);
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu%s", L.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned(workspace, 256)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  int num_cus = 0;
  st = check_device(&num_cus);
  if (st != MOE_OK) return st;
  char* ws = static_cast<char*>(workspace);
  TailArgs a{};
  a.T = static_cast<int>(num_tokens);
  a.latent = latent;
  a.hidden = hidden;
  a.bm = L.bm;
  a.eps = eps;
  a.z = z;
  a.gamma = w->gamma;
  a.s = s;
  a.up_c = w->up_codes;
  a.wcanon = w->layout == MOE_WEIGHTS_CANONICAL ? 1 : 0;
  a.up_s = w->up_scales;
  a.y = static_cast<uint16_t*>(y_bf16);
  a.codes = (taps && taps->a_codes) ? taps->a_codes : reinterpret_cast<uint8_t*>(ws + L.codes);
  a.scales = (taps && taps->a_scales) ? taps->a_scales : reinterpret_cast<uint8_t*>(ws + L.scales);
  a.inv_rms = taps ? taps->inv_rms : nullptr;
  a.o16 = s ? reinterpret_cast<uint16_t*>(ws + L.o16) : a.y;
  a.row_src = reinterpret_cast<int32_t*>(ws + L.row_src);
  a.tiles = reinterpret_cast<Tile*>(ws + L.tiles);
  a.tile_count = reinterpret_cast<int32_t*>(ws + L.tile_count);
  a.ex_tiles = reinterpret_cast<int32_t*>(ws + L.ex_tiles);
  a.part = reinterpret_cast<float*>(ws + L.part);
  hipError_t e = launch_tail(a, num_cus > 0 ? num_cus : 256, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_router_bias_update(const moe_plan_t* plan, const int32_t* expert_offsets,
                                  int64_t num_tokens, float rate, float* router_b, void* stream) {
  if (!plan) return fail(MOE_ERR_INVALID_ARG, "plan is NULL");
  const moe_config& c = plan->cfg;
  if (num_tokens < 0 || num_tokens > c.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "num_tokens %lld outside [0, %lld]",
                static_cast<long long>(num_tokens), static_cast<long long>(c.max_tokens));
  if (!(rate >= 0.0f) || rate > 3.4e38f) return fail(MOE_ERR_INVALID_ARG, "rate must be finite and >= 0");
  if (num_tokens == 0) return MOE_OK;
  if (!expert_offsets || !router_b) return fail(MOE_ERR_INVALID_ARG, "expert_offsets or router_b is NULL");
  if (!aligned(expert_offsets, 4) || !aligned(router_b, 4))
    return fail(MOE_ERR_INVALID_ARG, "expert_offsets and router_b need 4-byte alignment");
  moe_status s = check_device();
  if (s != MOE_OK) return s;
  hipError_t e = launch_router_bias_update(expert_offsets, c.num_experts, num_tokens * c.top_k, rate,
                                           router_b, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_profile_begin(moe_plan_t* plan, uint32_t stage_mask, int32_t max_calls) {
  if (!plan) return fail(MOE_ERR_INVALID_ARG, "plan is NULL");
  if (max_calls < 1 || max_calls > 65536) return fail(MOE_ERR_INVALID_ARG, "max_calls outside [1, 65536]");
  if (stage_mask == 0 || stage_mask >= (1u << MOE_NUM_STAGES))
    return fail(MOE_ERR_INVALID_ARG, "bad stage mask 0x%x", stage_mask);
  if (plan->prof_mask) return fail(MOE_ERR_INVALID_ARG, "profiling already active on this plan");
  moe_status s = check_device();
  if (s != MOE_OK) return s;
  plan->prof_ev.assign(size_t(max_calls) * MOE_NUM_STAGES * 2, nullptr);
  for (int n = 0; n < max_calls; ++n)
    for (int i = 0; i < MOE_NUM_STAGES; ++i) {
      if (!((stage_mask >> i) & 1u)) continue;
      for (int j = 0; j < 2; ++j) {
        hipEvent_t& e = plan->prof_ev[(size_t(n) * MOE_NUM_STAGES + i) * 2 + j];
        if (hipEventCreate(&e) != hipSuccess) {
          (void)hipGetLastError();
          for (hipEvent_t x : plan->prof_ev)
            if (x) (void)hipEventDestroy(x);
          plan->prof_ev.clear();
          return fail(MOE_ERR_DEVICE, "hipEventCreate failed");
        }
      }
    }
  plan->prof_cap = max_calls;
  plan->prof_n = 0;
  plan->prof_mask = stage_mask;
  return MOE_OK;
}

moe_status moe_profile_end(moe_plan_t* plan, double* stage_ms, int32_t* calls) {
  if (!plan || !stage_ms || !calls) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
  if (!plan->prof_mask) return fail(MOE_ERR_INVALID_ARG, "profiling is not active on this plan");
  moe_status st = MOE_OK;
  for (int i = 0; i < MOE_NUM_STAGES; ++i) stage_ms[i] = 0.0;
  for (int n = 0; n < plan->prof_n; ++n)
    for (int i = 0; i < MOE_NUM_STAGES; ++i) {
      if (!((plan->prof_mask >> i) & 1u)) continue;
      hipEvent_t a = plan->prof_ev[(size_t(n) * MOE_NUM_STAGES + i) * 2];
      hipEvent_t b = plan->prof_ev[(size_t(n) * MOE_NUM_STAGES + i) * 2 + 1];
      float ms = 0.f;
      if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess) {
        (void)hipGetLastError();
        st = fail(MOE_ERR_DEVICE, "reading profiling events failed");
      }
      stage_ms[i] += ms;
    }
  *calls = plan->prof_n;
  for (hipEvent_t x : plan->prof_ev)
    if (x) (void)hipEventDestroy(x);
  plan->prof_ev.clear();
  plan->prof_mask = 0;
  plan->prof_cap = plan->prof_n = 0;
  return st;
}

}  // extern "C"

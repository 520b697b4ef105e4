// Host side of the C ABI declared in include/moe_lp.h: argument validation,
// workspace carving and the fixed launch sequence of the MoE expert forward.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "kernels.h"
#include "moe_lp.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Byte layout of the forward workspace; offsets relative to its base.
struct WsLayout {
  size_t ids, wts, offsets, sorted_rows, row_of, active, num_active, tile_a, tile_16, tiles, queue, hist;
  size_t act, act_scale, h, h_scale, y;
  size_t total;
};

struct Dims {
  int T, H, I, E, k, fmt;  // fmt: the kernel family (the pow2 FP8 variant runs the FP8 kernels)
  bool pow2;               // FP8 with power-of-two scales
  bool oft;
  bool oft_shared;         // one R for all experts (adapter_expert_stride = 0)
  bool kblocked;           // weights in 16 x 128 tiles (MOE_WL_KBLOCKED)
  int64_t R;
  int nblk;
  int tile_rows;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Validates the descriptor (pointer checks are done by each entry point).
moe_status check_layer(const moe_layer* L, Dims* d) {
  if (L == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (L->num_tokens < 0 || L->hidden <= 0 || L->inter <= 0 || L->num_experts <= 0 || L->top_k <= 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (L->top_k > L->num_experts) return MOE_ERR_INVALID_ARGUMENT;
  if (L->wformat != MOE_W_INT4_G32_BF16 && L->wformat != MOE_W_FP8_E4M3_B128 && L->wformat != MOE_W_MXFP4 &&
      L->wformat != MOE_W_FP8_E4M3_B128_POW2 && L->wformat != MOE_W_NVFP4)
    return MOE_ERR_INVALID_ARGUMENT;
  if (L->oft_block != 0 && L->oft_block != 32) return MOE_ERR_UNSUPPORTED;
  if (L->adapter_expert_stride < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (L->hidden % 256 != 0 || L->inter % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (L->num_experts > MAX_EXPERTS || L->top_k > MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)L->num_tokens * L->top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (L->weight_layout != MOE_WL_ROWS && L->weight_layout != MOE_WL_KBLOCKED) return MOE_ERR_INVALID_ARGUMENT;
  if (L->tile_rows != 0 && L->tile_rows != 16 && L->tile_rows != 32 && L->tile_rows != 48 && L->tile_rows != 64 &&
      L->tile_rows != 96 && L->tile_rows != 128 && L->tile_rows != 160 && L->tile_rows != 192)
    return MOE_ERR_UNSUPPORTED;
  // the GEMMs address activation rows with 32-bit byte offsets
  if ((int64_t)L->num_tokens * L->top_k * (int64_t)(L->hidden > L->inter ? L->hidden : L->inter) * 2 >= (1ll << 32))
    return MOE_ERR_UNSUPPORTED;
  d->T = L->num_tokens;
  d->H = L->hidden;
  d->I = L->inter;
  d->E = L->num_experts;
  d->k = L->top_k;
  d->fmt = L->wformat;
  d->pow2 = L->wformat == MOE_W_FP8_E4M3_B128_POW2;
  if (d->pow2) d->fmt = MOE_W_FP8_E4M3_B128;  // same layouts and kernels, power-of-two scale path
  d->oft = L->oft_block != 0;
  d->oft_shared = d->oft && L->adapter_expert_stride == 0;
  d->R = (int64_t)d->T * d->k;
  d->nblk = (int)((d->R + PAIRS_PER_BLOCK - 1) / PAIRS_PER_BLOCK);
  d->tile_rows = L->tile_rows;
  d->kblocked = L->weight_layout == MOE_WL_KBLOCKED;
  return MOE_OK;
}

// Per-XCD work-queue counters of the grouped-GEMM pair launches: 8 per launch, at most
// num_experts + 1 launches (chunk_experts >= 1).
int queue_ints(const Dims& d) { return 8 * (d.E + 1); }

// The OFT rotation's output format for the layer's GEMM1 input (launch_oft).
int oft_out_format(const Dims& d) {
  if (d.fmt == MOE_W_INT4_G32_BF16) return 0;
  if (d.fmt == MOE_W_NVFP4) return 2;
  if (d.fmt == MOE_W_FP8_E4M3_B128) return d.pow2 ? 4 : 3;
  return 5;
}

WsLayout layout(const Dims& d) {
  WsLayout w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t R = (size_t)d.R, T = (size_t)d.T, H = (size_t)d.H, I = (size_t)d.I, E = (size_t)d.E;
  w.ids = take(R * 4);
  w.wts = take(R * 4);
  w.offsets = take((E + 1) * 4);
  w.sorted_rows = take(R * 4);
  w.row_of = take(R * 4);
  w.active = take(E * 4);
  w.num_active = take(16);
  w.tile_a = take((E + 1) * 4);
  w.tile_16 = take((E + 1) * 4);
  w.tiles = take((size_t)max_row_tiles(d.R, d.E) * 16);
  w.queue = take((size_t)queue_ints(d) * 4);
  w.hist = take((size_t)(d.nblk > 0 ? d.nblk : 1) * E * 4);
  const size_t arows = d.oft ? R : T;
  if (d.fmt == MOE_W_INT4_G32_BF16 || d.fmt == MOE_W_NVFP4) {
    w.act = take(arows * H * 2);
    w.act_scale = take(0);
    w.h = take(R * I * 2);
    w.h_scale = take(0);
  } else if (d.fmt == MOE_W_FP8_E4M3_B128) {
    w.act = take(arows * H);
    w.act_scale = take(arows * scale_row_bytes((int)H));
    w.h = take(R * I);
    w.h_scale = take(R * scale_row_bytes((int)I));
  } else {
    w.act = take(arows * H);
    w.act_scale = take(arows * scale_row_bytes((int)H));
    w.h = take(R * I);
    w.h_scale = take(R * scale_row_bytes((int)I));
  }
  w.y = take(R * H * 2);
  w.total = o;
  return w;
}

// Rows per GEMM tile from the mean rows per expert and the weight format
// (measured on MI355X: the INT4 unpack favours two workgroups per CU at 64
// rows, and at 96 rows with 64-K stages, which cost about 8% less per row,
// where those pad an expert's rows less than 64-row tiles do; NVFP4 takes
// the 96-row, 64-K tiles above 64 rows (the DeepSeek-V3 Zipf shape: 4%
// faster than 64); FP8 and MXFP4 favour 128-row tiles once experts have that many rows,
// and FP8 160-row tiles above that: experts of ~256 rows then take two tiles
// instead of two full ones and a nearly empty third).  A kernel without a
// 160-row instantiation runs such tiles in its 192-row one.
int choose_bm(const Dims& d) {
  if (d.tile_rows) return d.tile_rows;
  const int64_t mean = d.R / d.E;
  if (mean <= 16) return 16;
  if (mean <= 32) return 32;
  if (d.fmt == MOE_W_INT4_G32_BF16) {
    const int64_t p64 = (mean + 63) / 64 * 64, p96 = (mean + 95) / 96 * 96;  // padded rows
    return p96 * 12 < p64 * 13 ? 96 : 64;
  }
  if (d.fmt == MOE_W_NVFP4) return mean > 64 ? 96 : 64;
  if (mean <= 96) return 64;
  if (d.fmt == MOE_W_FP8_E4M3_B128 && mean > 128) return 160;
  return 128;
}

int gemm_grid(const Dims& d, int bm, int chunk, int nblk_n) {
  int64_t tiles = d.R / bm + chunk;
  if (tiles > (int64_t)d.E + d.R / bm) tiles = (int64_t)d.E + d.R / bm;
  int64_t g = tiles * nblk_n;
  if (g > 1024) g = 1024;
  if (g < 8) g = 8;
  return (int)((g + 7) / 8 * 8);
}

moe_status launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// Optional per-stage timing: a HIP event is recorded on the stream before and
// after every launch group; durations are read after one stream sync.
struct StageTimer {
  hipStream_t s;
  std::vector<hipEvent_t> ev;  // start/stop pairs
  std::vector<int> stage_of;
  bool ok = true;
  void begin(int stage) {
    hipEvent_t a = nullptr, b = nullptr;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) ok = false;
    ev.push_back(a);
    ev.push_back(b);
    stage_of.push_back(stage);
    if (ok && hipEventRecord(a, s) != hipSuccess) ok = false;
  }
  void end() {
    if (ok && hipEventRecord(ev.back(), s) != hipSuccess) ok = false;
  }
  void finish(float* ms, int32_t* counts) {
    for (int i = 0; i < MOE_NUM_STAGES; ++i) { ms[i] = 0.0f; counts[i] = 0; }
    if (ok && hipStreamSynchronize(s) != hipSuccess) ok = false;
    for (size_t i = 0; i < stage_of.size(); ++i) {
      float t = 0.0f;
      if (ok && hipEventElapsedTime(&t, ev[2 * i], ev[2 * i + 1]) == hipSuccess) {
        ms[stage_of[i]] += t;
        counts[stage_of[i]] += 1;
      }
      if (ev[2 * i]) (void)hipEventDestroy(ev[2 * i]);
      if (ev[2 * i + 1]) (void)hipEventDestroy(ev[2 * i + 1]);
    }
  }
};

struct Scope {
  StageTimer* t;
  Scope(StageTimer* tm, int stage) : t(tm) { if (t) t->begin(stage); }
  ~Scope() { if (t) t->end(); }
};

moe_status forward_impl(const moe_layer* layer, const void* x_bf16, const float* logits, const moe_qweights* qw,
                        const moe_scales* sc, const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                        void* ws, size_t ws_bytes, void* stream, StageTimer* tm);

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_LP_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, format or limit";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_DEVICE: return "device launch error";
  }
  return "unknown status";
}

moe_status moe_pack_weights_kblocked(const moe_layer* layer, const moe_qweights* qw, void* w13_out, void* w2_out,
                                     void* stream) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (qw == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {qw->w13, qw->w2, w13_out, w2_out};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bytes = d.fmt == MOE_W_FP8_E4M3_B128;
  launch_pack_kblocked(static_cast<const uint8_t*>(qw->w13), d.E, 2 * d.I, d.H, bytes,
                       static_cast<uint8_t*>(w13_out), s);
  launch_pack_kblocked(static_cast<const uint8_t*>(qw->w2), d.E, d.H, d.I, bytes, static_cast<uint8_t*>(w2_out), s);
  return launch_status();
}

moe_status moe_quantize_activations(const moe_layer* layer, const void* x_bf16, void* codes, void* scales,
                                    void* stream) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (d.fmt != MOE_W_FP8_E4M3_B128 && d.fmt != MOE_W_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (d.T == 0) return MOE_OK;
  if (x_bf16 == nullptr || codes == nullptr || scales == nullptr || !aligned16(x_bf16) || !aligned16(codes) ||
      !aligned4(scales))
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  if (d.fmt == MOE_W_FP8_E4M3_B128)
    launch_act_fp8(x, d.T, d.H, static_cast<uint8_t*>(codes), static_cast<float*>(scales), (d.H / 128) * 4, d.pow2,
                   s);
  else
    launch_act_mxfp8(x, d.T, d.H, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), d.H / 32, s);
  return launch_status();
}

size_t moe_workspace_bytes(const moe_layer* layer, int32_t chunk_experts) {
  Dims d;
  if (check_layer(layer, &d) != MOE_OK || chunk_experts < 1) return 0;
  return layout(d).total;
}

int32_t moe_tile_rows(const moe_layer* layer) {
  Dims d;
  if (check_layer(layer, &d) != MOE_OK) return 0;
  return choose_bm(d);
}

size_t moe_route_workspace_bytes(const moe_layer* layer) {
  Dims d;
  if (check_layer(layer, &d) != MOE_OK) return 0;
  return align_up((size_t)(d.E + 1) * 4) * 2 + align_up((size_t)max_row_tiles(d.R, d.E) * 16) +
         align_up((size_t)(d.nblk > 0 ? d.nblk : 1) * d.E * 4);
}

moe_status moe_route_permute(const moe_layer* layer, const float* logits, const moe_route_out* out, void* ws,
                             size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (d.T == 0) return MOE_OK;
  const void* ptrs[] = {logits, out->topk_ids, out->topk_w, out->expert_offsets, out->sorted_rows,
                        out->row_of, out->active_experts, out->num_active, ws};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < moe_route_workspace_bytes(layer)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  int32_t* tile_a = reinterpret_cast<int32_t*>(base);
  int32_t* tile_16 = reinterpret_cast<int32_t*>(base + align_up((size_t)(d.E + 1) * 4));
  int32_t* tiles = reinterpret_cast<int32_t*>(base + 2 * align_up((size_t)(d.E + 1) * 4));
  int32_t* hist = reinterpret_cast<int32_t*>(base + 2 * align_up((size_t)(d.E + 1) * 4) +
                                             align_up((size_t)max_row_tiles(d.R, d.E) * 16));
  launch_route(logits, d.T, d.E, d.k, out->topk_ids, out->topk_w, s);
  launch_permute(out->topk_ids, (int)d.R, d.E, choose_bm(d), hist, out->expert_offsets, out->sorted_rows,
                 out->row_of, out->active_experts, out->num_active, tile_a, tile_16, tiles, nullptr, 0, s);
  return launch_status();
}

moe_status moe_expert_forward(const moe_layer* layer, const void* x_bf16, const float* logits,
                              const moe_qweights* qw, const moe_scales* sc, const void* adapter_bf16,
                              int32_t chunk_experts, void* out_bf16, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(layer, x_bf16, logits, qw, sc, adapter_bf16, chunk_experts, out_bf16, ws, ws_bytes, stream,
                      nullptr);
}

moe_status moe_expert_forward_timed(const moe_layer* layer, const void* x_bf16, const float* logits,
                                    const moe_qweights* qw, const moe_scales* sc, const void* adapter_bf16,
                                    int32_t chunk_experts, void* out_bf16, void* ws, size_t ws_bytes, void* stream,
                                    float* stage_ms, int32_t* stage_launches) {
  if (stage_ms == nullptr || stage_launches == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  StageTimer* tm = new StageTimer();
  tm->s = static_cast<hipStream_t>(stream);
  moe_status st = forward_impl(layer, x_bf16, logits, qw, sc, adapter_bf16, chunk_experts, out_bf16, ws, ws_bytes,
                               stream, tm);
  tm->finish(stage_ms, stage_launches);
  const bool ok = tm->ok;
  delete tm;
  if (st == MOE_OK && !ok) st = MOE_ERR_DEVICE;
  return st;
}

}  // extern "C"

namespace {
moe_status forward_impl(const moe_layer* layer, const void* x_bf16, const float* logits, const moe_qweights* qw,
                        const moe_scales* sc, const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                        void* ws, size_t ws_bytes, void* stream, StageTimer* tm) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (chunk_experts < 1 || qw == nullptr || sc == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((adapter_bf16 != nullptr) != d.oft) return MOE_ERR_INVALID_ARGUMENT;
  if (d.T == 0) return MOE_OK;
  const void* ptrs[] = {x_bf16, logits, qw->w13, qw->w2, sc->s13, sc->s2, out_bf16, ws};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (d.fmt == MOE_W_NVFP4 && (sc->g13 == nullptr || sc->g2 == nullptr || !aligned4(sc->g13) || !aligned4(sc->g2)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (d.oft && !aligned16(adapter_bf16)) return MOE_ERR_INVALID_ARGUMENT;
  if (d.oft && (layer->adapter_expert_stride % 8) != 0) return MOE_ERR_INVALID_ARGUMENT;
  const WsLayout wl = layout(d);
  if (ws_bytes < wl.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
  int32_t* ids = I32(wl.ids);
  float* wts = reinterpret_cast<float*>(base + wl.wts);
  int32_t* offsets = I32(wl.offsets);
  int32_t* sorted_rows = I32(wl.sorted_rows);
  int32_t* row_of = I32(wl.row_of);
  int32_t* active = I32(wl.active);
  int32_t* num_active = I32(wl.num_active);
  int32_t* tile_a = I32(wl.tile_a);
  int32_t* tile_16 = I32(wl.tile_16);
  int32_t* tiles = I32(wl.tiles);
  int32_t* queue = I32(wl.queue);
  int32_t* hist = I32(wl.hist);
  void* act = base + wl.act;
  void* act_scale = base + wl.act_scale;
  void* h = base + wl.h;
  void* h_scale = base + wl.h_scale;
  uint16_t* y = reinterpret_cast<uint16_t*>(base + wl.y);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int bm = choose_bm(d);

  // 1-2. route and permute
  { Scope sc_(tm, MOE_STAGE_ROUTE); launch_route(logits, d.T, d.E, d.k, ids, wts, s); }
  { Scope sc_(tm, MOE_STAGE_PERMUTE);
    launch_permute(ids, (int)d.R, d.E, bm, hist, offsets, sorted_rows, row_of, active, num_active, tile_a, tile_16,
                   tiles, queue, queue_ints(d), s); }

  // 3. the GEMM1 input: per token, or per permuted row when the adapter rotates it
  {
  Scope sc_(tm, MOE_STAGE_ACT);
  if (d.oft) {
    // with 16-row GEMM tiles the tile descriptors are the rotation's row groups
    launch_oft(oft_out_format(d), x, static_cast<const uint16_t*>(adapter_bf16), layer->adapter_expert_stride, d.H,
               d.k, offsets, sorted_rows, active, num_active, tile_16, bm == 16 ? tiles : nullptr, act, act_scale,
               scale_row_bytes(d.H), s);
  } else if (d.fmt == MOE_W_INT4_G32_BF16) {
    launch_act_f16(x, d.T, d.H, static_cast<uint16_t*>(act), s);
  } else if (d.fmt == MOE_W_NVFP4) {
    launch_act_f16_natural(x, d.T, d.H, static_cast<uint16_t*>(act), s);
  } else if (d.fmt == MOE_W_FP8_E4M3_B128) {
    launch_act_fp8(x, d.T, d.H, static_cast<uint8_t*>(act), static_cast<float*>(act_scale), scale_row_bytes(d.H),
                   d.pow2, s);
  } else {
    launch_act_mxfp8(x, d.T, d.H, static_cast<uint8_t*>(act), static_cast<uint8_t*>(act_scale), scale_row_bytes(d.H),
                     s);
  }
  }

  // 4. chunk loop over the active experts: GEMM1 (+SwiGLU) then GEMM2 per chunk
  const int nchunks = (d.E + chunk_experts - 1) / chunk_experts;
  GemmArgs g1{}, g2{};
  g1.a = act;
  g1.a_scale = act_scale;
  g1.a_scale_stride = scale_row_bytes(d.H);
  g1.out_scale_stride = scale_row_bytes(d.I);
  g1.a_per_token = d.oft ? 0 : 1;
  g1.w = static_cast<const uint8_t*>(qw->w13);
  g1.w_scale = sc->s13;
  g1.N = 2 * d.I;
  g1.K = d.H;
  g1.inter = d.I;
  g1.out = h;
  g1.out_scale = h_scale;
  g2.a = h;
  g2.a_scale = h_scale;
  g2.a_scale_stride = scale_row_bytes(d.I);
  g2.a_per_token = 0;
  g2.w = static_cast<const uint8_t*>(qw->w2);
  g2.w_scale = sc->s2;
  g2.N = d.H;
  g2.K = d.I;
  g2.inter = d.I;
  g2.out = y;
  g2.out_scale = nullptr;
  const int64_t n13 = (int64_t)2 * d.I * d.H, n2 = (int64_t)d.H * d.I;
  if (d.fmt == MOE_W_INT4_G32_BF16) {
    g1.w_expert_bytes = n13 / 2; g1.ws_expert_elems = n13 / 32;
    g2.w_expert_bytes = n2 / 2;  g2.ws_expert_elems = n2 / 32;
  } else if (d.fmt == MOE_W_NVFP4) {
    g1.w_expert_bytes = n13 / 2; g1.ws_expert_elems = n13 / 16;
    g2.w_expert_bytes = n2 / 2;  g2.ws_expert_elems = n2 / 16;
    g1.gscale = sc->g13;
    g2.gscale = sc->g2;
  } else if (d.fmt == MOE_W_FP8_E4M3_B128) {
    g1.w_expert_bytes = n13; g1.ws_expert_elems = n13 / (128 * 128);
    g2.w_expert_bytes = n2;  g2.ws_expert_elems = n2 / (128 * 128);
  } else {
    g1.w_expert_bytes = n13 / 2; g1.ws_expert_elems = n13 / 32;
    g2.w_expert_bytes = n2 / 2;  g2.ws_expert_elems = n2 / 32;
  }
  for (GemmArgs* g : {&g1, &g2}) {
    g->offsets = offsets;
    g->sorted_rows = sorted_rows;
    g->active = active;
    g->num_active = num_active;
    g->tile_start = tile_a;
    g->tiles = tiles;
    g->top_k = d.k;
    g->chunk_experts = chunk_experts;
    g->w_kblocked = d.kblocked ? 1 : 0;
  }
  // expert-major item order (N blocks fastest, an expert's tiles adjacent):
  // an XCD then works on all items of one or two experts at once, so both
  // the expert's weight slices and its activation tiles stay in that L2
  g1.nb_fastest = 1;
  g2.nb_fastest = 1;
  const int grid1 = gemm_grid(d, bm, chunk_experts, d.I / 128);
  const int grid2 = gemm_grid(d, bm, chunk_experts, d.H / 256);
  // launch c runs chunk c's GEMM1 together with chunk c-1's GEMM2
  const int grid = grid1 > grid2 ? grid1 : grid2;
  auto pair = d.fmt == MOE_W_INT4_G32_BF16 ? launch_gemm_int4_pair
            : d.fmt == MOE_W_NVFP4         ? launch_gemm_nvfp4_pair
            : d.fmt == MOE_W_FP8_E4M3_B128 ? (d.pow2 ? launch_gemm_fp8_pow2_pair : launch_gemm_fp8_pair)
                                           : launch_gemm_mxfp4_pair;
  for (int c = 0; c <= nchunks; ++c) {
    g1.chunk = c < nchunks ? c : -1;
    g2.chunk = c - 1;
    Scope sc_(tm, c < nchunks ? MOE_STAGE_GEMM1 : MOE_STAGE_GEMM2);
    pair(g1, g2, queue + 8 * c, bm, grid, s);
  }

  // 5. weighted combine back to token order
  { Scope sc_(tm, MOE_STAGE_COMBINE);
    launch_combine(y, wts, row_of, d.T, d.k, d.H, static_cast<uint16_t*>(out_bf16), s); }
  return launch_status();
}

// ---------------------------------------------------------------------------
// Materialized-chunk scheme: per chunk, dequantize its experts into a BF16
// copy in the workspace, then BF16 GEMM1 and GEMM2 over that copy.

// Workspace of the materialized scheme: the routing arrays, the bf16 GEMM1
// input (OFT only; otherwise x is read directly), h and y in bf16, work
// counters for two launches per chunk, and one chunk's BF16 weight copy.
struct MatLayout {
  size_t ids, wts, offsets, sorted_rows, row_of, active, num_active, tile_a, tile_16, tiles, queue, hist;
  size_t act, h, y, copy;
  size_t total;
};

int mat_queue_ints(const Dims& d) { return 16 * (d.E + 1); }
int64_t mat_copy_elems(const Dims& d) { return (int64_t)3 * d.H * d.I; }  // W13 + W2 of one expert

MatLayout mat_layout(const Dims& d, int chunk) {
  MatLayout w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t R = (size_t)d.R, H = (size_t)d.H, I = (size_t)d.I, E = (size_t)d.E;
  w.ids = take(R * 4);
  w.wts = take(R * 4);
  w.offsets = take((E + 1) * 4);
  w.sorted_rows = take(R * 4);
  w.row_of = take(R * 4);
  w.active = take(E * 4);
  w.num_active = take(16);
  w.tile_a = take((E + 1) * 4);
  w.tile_16 = take((E + 1) * 4);
  w.tiles = take((size_t)max_row_tiles(d.R, d.E) * 16);
  w.queue = take((size_t)mat_queue_ints(d) * 4);
  w.hist = take((size_t)(d.nblk > 0 ? d.nblk : 1) * E * 4);
  w.act = take(d.oft ? R * H * 2 : 0);
  w.h = take(R * I * 2);
  w.y = take(R * H * 2);
  w.copy = take((size_t)chunk * (size_t)mat_copy_elems(d) * 2);
  w.total = o;
  return w;
}

// BF16 GEMM tile rows: 16, 32, 64 or 128 (layer->tile_rows if one of these).
int choose_bm_mat(const Dims& d) {
  if (d.tile_rows == 16 || d.tile_rows == 32 || d.tile_rows == 64 || d.tile_rows == 128) return d.tile_rows;
  const int64_t mean = d.R / d.E;
  if (mean <= 16) return 16;
  if (mean <= 32) return 32;
  if (mean <= 96) return 64;
  return 128;
}

moe_status forward_materialized_impl(const moe_layer* layer, const void* x_bf16, const float* logits,
                                     const moe_qweights* qw, const moe_scales* sc, const void* adapter_bf16,
                                     int32_t chunk_experts, void* out_bf16, void* ws, size_t ws_bytes, void* stream,
                                     StageTimer* tm) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (chunk_experts < 1 || qw == nullptr || sc == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((adapter_bf16 != nullptr) != d.oft) return MOE_ERR_INVALID_ARGUMENT;
  if (d.T == 0) return MOE_OK;
  const void* ptrs[] = {x_bf16, logits, qw->w13, qw->w2, sc->s13, sc->s2, out_bf16, ws};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (d.fmt == MOE_W_NVFP4 && (sc->g13 == nullptr || sc->g2 == nullptr || !aligned4(sc->g13) || !aligned4(sc->g2)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (d.oft && !aligned16(adapter_bf16)) return MOE_ERR_INVALID_ARGUMENT;
  if (d.oft && (layer->adapter_expert_stride % 8) != 0) return MOE_ERR_INVALID_ARGUMENT;
  const int C = chunk_experts < d.E ? chunk_experts : d.E;  // a chunk never holds more than E experts
  const MatLayout wl = mat_layout(d, C);
  if (ws_bytes < wl.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
  int32_t* ids = I32(wl.ids);
  float* wts = reinterpret_cast<float*>(base + wl.wts);
  int32_t* offsets = I32(wl.offsets);
  int32_t* sorted_rows = I32(wl.sorted_rows);
  int32_t* row_of = I32(wl.row_of);
  int32_t* active = I32(wl.active);
  int32_t* num_active = I32(wl.num_active);
  int32_t* tile_a = I32(wl.tile_a);
  int32_t* tile_16 = I32(wl.tile_16);
  int32_t* tiles = I32(wl.tiles);
  int32_t* queue = I32(wl.queue);
  int32_t* hist = I32(wl.hist);
  uint16_t* act = reinterpret_cast<uint16_t*>(base + wl.act);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + wl.h);
  uint16_t* y = reinterpret_cast<uint16_t*>(base + wl.y);
  uint16_t* copy = reinterpret_cast<uint16_t*>(base + wl.copy);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int bm = choose_bm_mat(d);

  { Scope sc_(tm, MOE_STAGE_ROUTE); launch_route(logits, d.T, d.E, d.k, ids, wts, s); }
  { Scope sc_(tm, MOE_STAGE_PERMUTE);
    launch_permute(ids, (int)d.R, d.E, bm, hist, offsets, sorted_rows, row_of, active, num_active, tile_a, tile_16,
                   tiles, queue, mat_queue_ints(d), s); }
  if (d.oft) {
    Scope sc_(tm, MOE_STAGE_ACT);
    launch_oft_bf16(x, static_cast<const uint16_t*>(adapter_bf16), layer->adapter_expert_stride, d.H, d.k, offsets,
                    sorted_rows, active, num_active, tile_16, act, s);
  }

  const int64_t copy_bytes = mat_copy_elems(d) * 2;
  GemmArgs g1{}, g2{};
  g1.a = d.oft ? static_cast<const void*>(act) : static_cast<const void*>(x);
  g1.a_per_token = d.oft ? 0 : 1;
  g1.w = reinterpret_cast<const uint8_t*>(copy);
  g1.w_expert_bytes = copy_bytes;
  g1.N = 2 * d.I;
  g1.K = d.H;
  g1.inter = d.I;
  g1.out = h;
  g2.a = h;
  g2.a_per_token = 0;
  g2.w = reinterpret_cast<const uint8_t*>(copy + (int64_t)2 * d.I * d.H);
  g2.w_expert_bytes = copy_bytes;
  g2.N = d.H;
  g2.K = d.I;
  g2.inter = d.I;
  g2.out = y;
  for (GemmArgs* g : {&g1, &g2}) {
    g->offsets = offsets;
    g->sorted_rows = sorted_rows;
    g->active = active;
    g->num_active = num_active;
    g->tile_start = tile_a;
    g->tiles = tiles;
    g->top_k = d.k;
    g->chunk_experts = C;
    g->nb_fastest = 1;
  }
  const int grid1 = gemm_grid(d, bm, C, d.I / 128);
  const int grid2 = gemm_grid(d, bm, C, d.H / 256);
  const int nchunks = (d.E + C - 1) / C;
  for (int c = 0; c < nchunks; ++c) {
    { Scope sc_(tm, MOE_STAGE_DEQUANT);
      launch_dequant_chunk(d.fmt, static_cast<const uint8_t*>(qw->w13), sc->s13,
                           static_cast<const uint8_t*>(qw->w2), sc->s2, active, num_active, c, C, d.H, d.I, sc->g13,
                           sc->g2, d.kblocked, copy, s); }
    g1.chunk = c;
    g2.chunk = -1;
    { Scope sc_(tm, MOE_STAGE_GEMM1); launch_gemm_bf16_pair(g1, g2, queue + 16 * c, bm, grid1, s); }
    g1.chunk = -1;
    g2.chunk = c;
    { Scope sc_(tm, MOE_STAGE_GEMM2); launch_gemm_bf16_pair(g1, g2, queue + 16 * c + 8, bm, grid2, s); }
  }
  { Scope sc_(tm, MOE_STAGE_COMBINE);
    launch_combine(y, wts, row_of, d.T, d.k, d.H, static_cast<uint16_t*>(out_bf16), s); }
  return launch_status();
}
// ---------------------------------------------------------------------------
// Frozen-base backward (every weight format).

// The transposed weight copy made by moe_prepare_backward_weights.
struct BwdWeights {
  size_t w13t, w2t, s13, s2, total;
};

// INT4 / MXFP4: nibbles + fp16 scales (2 bytes per 32 weights; NVFP4 per 16);
// FP8: bytes + fp32 block scales (the forward sizes).
BwdWeights bwd_weights_layout(const Dims& d) {
  BwdWeights b{};
  const size_t H = (size_t)d.H, I = (size_t)d.I, E = (size_t)d.E;
  const bool fp8 = d.fmt == MOE_W_FP8_E4M3_B128;
  const size_t gk = d.fmt == MOE_W_NVFP4 ? 16 : 32;
  size_t o = 0;
  b.w13t = o; o = align_up(o + E * H * 2 * I / (fp8 ? 1 : 2));
  b.w2t = o;  o = align_up(o + E * I * H / (fp8 ? 1 : 2));
  b.s13 = o;  o = align_up(o + (fp8 ? E * (H / 128) * (2 * I / 128) * 4 : E * (H / gk) * 2 * I * 2));
  b.s2 = o;   o = align_up(o + (fp8 ? E * (I / 128) * (H / 128) * 4 : E * (I / gk) * H * 2));
  b.total = o;
  return b;
}

moe_status check_backward(const moe_layer* L, Dims* d) {
  moe_status st = check_layer(L, d);
  if (st != MOE_OK) return st;
  if (d->I % 256 != 0) return MOE_ERR_UNSUPPORTED;
  // FP8 backward keeps one K run of block scales per item (at most 64 K blocks)
  if (d->fmt == MOE_W_FP8_E4M3_B128 && (d->H > 64 * 128 || 2 * d->I > 64 * 128)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Tile heights of the backward: the recompute of GEMM1 uses the forward's;
// the backward GEMMs at most 64 rows (measured on MI355X: their fp16 operand
// tiles are twice the forward's FP8 / MXFP8 bytes, and 64-row tiles keep
// three stages in flight).
int bwd_bm(const Dims& d) {
  const int bm = choose_bm(d);
  return bm > 64 ? 64 : bm;
}

struct BwdLayout {
  size_t ids, wts, offsets, sorted_rows, row_of, active, num_active, tile_a, tile_16, tiles, queue, hist;
  size_t tile_a_r, tiles_r;  // tiles of the recompute's height
  size_t act, act_scale, h, h_scale, gact, ab, dab, gpart, dxt, dxr, drp;
  size_t total;
};

int bwd_queue_ints(const Dims& d) { return 16 * (d.E + 1); }

BwdLayout bwd_layout(const Dims& d) {
  BwdLayout w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t R = (size_t)d.R, T = (size_t)d.T, H = (size_t)d.H, I = (size_t)d.I, E = (size_t)d.E;
  w.ids = take(R * 4);
  w.wts = take(R * 4);
  w.offsets = take((E + 1) * 4);
  w.sorted_rows = take(R * 4);
  w.row_of = take(R * 4);
  w.active = take(E * 4);
  w.num_active = take(16);
  w.tile_a = take((E + 1) * 4);
  w.tile_16 = take((E + 1) * 4);
  w.tiles = take((size_t)max_row_tiles(d.R, d.E) * 16);
  w.queue = take((size_t)bwd_queue_ints(d) * 4);
  w.hist = take((size_t)(d.nblk > 0 ? d.nblk : 1) * E * 4);
  w.tile_a_r = take((E + 1) * 4);
  w.tiles_r = take((size_t)max_row_tiles(d.R, d.E) * 16);
  if (d.fmt == MOE_W_INT4_G32_BF16 || d.fmt == MOE_W_NVFP4) {
    w.act = take((d.oft ? R : T) * H * 2);
    w.act_scale = take(0);
    w.h = take(0);
    w.h_scale = take(0);
  } else {
    // the forward's GEMM1 input (per token, or per permuted row with an
    // adapter) and its quantized h, as the recompute writes them
    w.act = take((d.oft ? R : T) * H);
    w.act_scale = take((d.oft ? R : T) * scale_row_bytes((int)H));
    w.h = take(R * I);
    w.h_scale = take(R * scale_row_bytes((int)I));
  }
  w.gact = take(T * H * 2);
  w.ab = take(R * 2 * I * 4);
  w.dab = take(R * 2 * I * 2);
  w.gpart = take(R * (I / 256) * 4);
  w.dxt = take(R * H * 4);
  w.dxr = take(d.oft ? R * H * 4 : 0);
  // one shared R: the adapter gradient's per-active-expert partials
  w.drp = take(d.oft && d.oft_shared ? E * H * 32 * 4 : 0);
  w.total = o;
  return w;
}
}  // namespace

extern "C" {

size_t moe_backward_weights_bytes(const moe_layer* layer) {
  Dims d;
  if (check_backward(layer, &d) != MOE_OK) return 0;
  return bwd_weights_layout(d).total;
}

moe_status moe_prepare_backward_weights(const moe_layer* layer, const moe_qweights* qw, const moe_scales* sc,
                                        void* bwd_weights, size_t bwd_bytes, void* stream) {
  Dims d;
  moe_status st = check_backward(layer, &d);
  if (st != MOE_OK) return st;
  if (qw == nullptr || sc == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {qw->w13, qw->w2, sc->s13, sc->s2, bwd_weights};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  const BwdWeights b = bwd_weights_layout(d);
  if (bwd_bytes < b.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(bwd_weights);
  launch_repack_bwd(d.fmt, static_cast<const uint8_t*>(qw->w13), sc->s13, d.E, 2 * d.I, d.H, d.kblocked,
                    reinterpret_cast<uint8_t*>(base + b.w13t), base + b.s13, s);
  launch_repack_bwd(d.fmt, static_cast<const uint8_t*>(qw->w2), sc->s2, d.E, d.H, d.I, d.kblocked,
                    reinterpret_cast<uint8_t*>(base + b.w2t), base + b.s2, s);
  return launch_status();
}

size_t moe_backward_workspace_bytes(const moe_layer* layer, int32_t chunk_experts) {
  Dims d;
  if (check_backward(layer, &d) != MOE_OK || chunk_experts < 1) return 0;
  return bwd_layout(d).total;
}

}  // extern "C"

namespace {
moe_status backward_impl(const moe_layer* layer, const void* x_bf16, const float* logits, const moe_qweights* qw,
                         const moe_scales* sc, const void* bwd_weights, const void* adapter_bf16,
                         const void* d_out_bf16, int32_t chunk_experts, void* d_x_bf16, float* d_logits,
                         float* d_adapter, void* ws, size_t ws_bytes, void* stream, StageTimer* tm) {
  Dims d;
  moe_status st = check_backward(layer, &d);
  if (st != MOE_OK) return st;
  if (chunk_experts < 1 || qw == nullptr || sc == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((adapter_bf16 != nullptr) != d.oft || (d_adapter != nullptr) != d.oft) return MOE_ERR_INVALID_ARGUMENT;
  if (d.T == 0) return MOE_OK;
  const void* ptrs[] = {x_bf16, logits, qw->w13, qw->w2, sc->s13, sc->s2, bwd_weights, d_out_bf16, d_x_bf16,
                        d_logits, ws};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (d.oft && (!aligned16(adapter_bf16) || !aligned16(d_adapter) || (layer->adapter_expert_stride % 8) != 0))
    return MOE_ERR_INVALID_ARGUMENT;
  if (d.fmt == MOE_W_NVFP4 && (sc->g13 == nullptr || sc->g2 == nullptr || !aligned4(sc->g13) || !aligned4(sc->g2)))
    return MOE_ERR_INVALID_ARGUMENT;
  const BwdLayout wl = bwd_layout(d);
  if (ws_bytes < wl.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const BwdWeights bw = bwd_weights_layout(d);

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  auto I32 = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
  int32_t* ids = I32(wl.ids);
  float* wts = reinterpret_cast<float*>(base + wl.wts);
  int32_t* offsets = I32(wl.offsets);
  int32_t* sorted_rows = I32(wl.sorted_rows);
  int32_t* row_of = I32(wl.row_of);
  int32_t* active = I32(wl.active);
  int32_t* num_active = I32(wl.num_active);
  int32_t* tile_a = I32(wl.tile_a);
  int32_t* tile_16 = I32(wl.tile_16);
  int32_t* tiles = I32(wl.tiles);
  int32_t* queue = I32(wl.queue);
  int32_t* hist = I32(wl.hist);
  void* act = base + wl.act;
  void* act_scale = base + wl.act_scale;
  uint8_t* hq = reinterpret_cast<uint8_t*>(base + wl.h);
  void* h_scale = base + wl.h_scale;
  uint16_t* gact = reinterpret_cast<uint16_t*>(base + wl.gact);
  float* ab = reinterpret_cast<float*>(base + wl.ab);
  uint16_t* dab = reinterpret_cast<uint16_t*>(base + wl.dab);
  float* gpart = reinterpret_cast<float*>(base + wl.gpart);
  float* dxt = reinterpret_cast<float*>(base + wl.dxt);
  float* dxr = reinterpret_cast<float*>(base + wl.dxr);
  const char* bwb = static_cast<const char*>(bwd_weights);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  const int bm = bwd_bm(d), bm_r = choose_bm(d);
  int32_t* tile_a_r = bm_r == bm ? tile_a : I32(wl.tile_a_r);
  int32_t* tiles_r = bm_r == bm ? tiles : I32(wl.tiles_r);

  { Scope sc_(tm, MOE_STAGE_ROUTE); launch_route(logits, d.T, d.E, d.k, ids, wts, s); }
  { Scope sc_(tm, MOE_STAGE_PERMUTE);
    // second pass (same permutation) for the recompute's tile list when its height differs
    if (bm_r != bm)
      launch_permute(ids, (int)d.R, d.E, bm_r, hist, offsets, sorted_rows, row_of, active, num_active, tile_a_r,
                     tile_16, tiles_r, queue, bwd_queue_ints(d), s);
    launch_permute(ids, (int)d.R, d.E, bm, hist, offsets, sorted_rows, row_of, active, num_active, tile_a, tile_16,
                   tiles, queue, bwd_queue_ints(d), s); }
  {
  Scope sc_(tm, MOE_STAGE_ACT);
  // the forward's GEMM1 input
  if (d.oft)
    launch_oft(oft_out_format(d), x, static_cast<const uint16_t*>(adapter_bf16), layer->adapter_expert_stride, d.H,
               d.k, offsets, sorted_rows, active, num_active, tile_16, nullptr, act, act_scale, scale_row_bytes(d.H),
               s);
  else if (d.fmt == MOE_W_FP8_E4M3_B128)
    launch_act_fp8(x, d.T, d.H, static_cast<uint8_t*>(act), static_cast<float*>(act_scale), scale_row_bytes(d.H),
                   d.pow2, s);
  else if (d.fmt == MOE_W_MXFP4)
    launch_act_mxfp8(x, d.T, d.H, static_cast<uint8_t*>(act), static_cast<uint8_t*>(act_scale), scale_row_bytes(d.H),
                     s);
  else if (d.fmt == MOE_W_NVFP4)
    launch_act_f16_natural(x, d.T, d.H, static_cast<uint16_t*>(act), s);
  else
    launch_act_f16(x, d.T, d.H, static_cast<uint16_t*>(act), s);
  launch_act_f16(static_cast<const uint16_t*>(d_out_bf16), d.T, d.H, gact, s);
  if (d.oft) launch_zero_f32(d_adapter, (int64_t)d.E * layer->adapter_expert_stride, s);
  }

  GemmArgs r1{}, none{}, bh{}, bx{};
  const int64_t n13 = (int64_t)2 * d.I * d.H, n2 = (int64_t)d.H * d.I;
  // recompute of GEMM1 (gate/up pre-activations; FP8 / MXFP4 also the quantized h)
  r1.a = act;
  r1.a_per_token = d.oft ? 0 : 1;
  r1.w = static_cast<const uint8_t*>(qw->w13);
  r1.w_scale = sc->s13;
  r1.N = 2 * d.I;
  r1.K = d.H;
  r1.inter = d.I;
  if (d.fmt == MOE_W_INT4_G32_BF16 || d.fmt == MOE_W_NVFP4) {
    const bool nv = d.fmt == MOE_W_NVFP4;
    r1.w_expert_bytes = n13 / 2;
    r1.ws_expert_elems = n13 / (nv ? 16 : 32);
    r1.gscale = nv ? sc->g13 : nullptr;
    r1.out = ab;
    r1.save_ab = 1;
  } else {
    const bool fp8 = d.fmt == MOE_W_FP8_E4M3_B128;
    r1.w_expert_bytes = fp8 ? n13 : n13 / 2;
    r1.ws_expert_elems = fp8 ? n13 / (128 * 128) : n13 / 32;
    r1.a_scale = act_scale;
    r1.a_scale_stride = scale_row_bytes(d.H);
    r1.out = hq;
    r1.out_scale = h_scale;
    r1.out_scale_stride = scale_row_bytes(d.I);
    r1.ab_out = ab;
  }
  // u = dout W2 with the SwiGLU backward in the epilogue
  bh.a = gact;
  bh.a_per_token = 1;
  const bool fp8 = d.fmt == MOE_W_FP8_E4M3_B128;
  const int64_t gk = d.fmt == MOE_W_NVFP4 ? 16 : 32;  // weights per fp16 scale of the transposed copy
  bh.w = reinterpret_cast<const uint8_t*>(bwb + bw.w2t);
  bh.w_scale = bwb + bw.s2;
  bh.gscale = sc->g2;
  bh.w_expert_bytes = fp8 ? n2 : n2 / 2;
  bh.ws_expert_elems = fp8 ? n2 / (128 * 128) : n2 / gk;
  bh.N = d.I;
  bh.K = d.H;
  bh.inter = d.I;
  bh.out = dab;
  bh.ab = ab;
  bh.topk_w = wts;
  bh.gpart = gpart;
  bh.hq = hq;
  bh.hsc = h_scale;
  bh.hsc_stride = scale_row_bytes(d.I);
  // dx' = [da | db] W13
  bx.a = dab;
  bx.a_per_token = 0;
  bx.w = reinterpret_cast<const uint8_t*>(bwb + bw.w13t);
  bx.w_scale = bwb + bw.s13;
  bx.gscale = sc->g13;
  bx.w_expert_bytes = fp8 ? n13 : n13 / 2;
  bx.ws_expert_elems = fp8 ? n13 / (128 * 128) : n13 / gk;
  bx.N = d.H;
  bx.K = 2 * d.I;
  bx.inter = d.I;
  bx.out = dxt;
  for (GemmArgs* g : {&r1, &none, &bh, &bx}) {
    g->offsets = offsets;
    g->sorted_rows = sorted_rows;
    g->active = active;
    g->num_active = num_active;
    g->tile_start = tile_a;
    g->tiles = tiles;
    g->top_k = d.k;
    g->chunk_experts = chunk_experts;
    g->nb_fastest = 1;
  }
  none.chunk = -1;
  r1.w_kblocked = d.kblocked ? 1 : 0;  // the recompute reads the forward's codes as given
  r1.tile_start = tile_a_r;
  r1.tiles = tiles_r;
  const int gridr = gemm_grid(d, bm_r, chunk_experts, d.I / 128);
  const int gh = gemm_grid(d, bm, chunk_experts, d.I / 256), gx = gemm_grid(d, bm, chunk_experts, d.H / 256);
  const int gridb = gh > gx ? gh : gx;
  const int nchunks = (d.E + chunk_experts - 1) / chunk_experts;
  // launch pair c: recompute chunk c, then chunk c's dh items with chunk c-1's dx' items
  for (int c = 0; c <= nchunks; ++c) {
    if (c < nchunks) {
      r1.chunk = c;
      Scope sc_(tm, MOE_STAGE_GEMM1);
      if (d.fmt == MOE_W_INT4_G32_BF16) launch_gemm_int4_pair(r1, none, queue + 16 * c, bm_r, gridr, s);
      else if (d.fmt == MOE_W_NVFP4) launch_gemm_nvfp4_pair(r1, none, queue + 16 * c, bm_r, gridr, s);
      else if (fp8)
        (d.pow2 ? launch_gemm_fp8_pow2_pair : launch_gemm_fp8_pair)(r1, none, queue + 16 * c, bm_r, gridr, s);
      else launch_gemm_mxfp4_pair(r1, none, queue + 16 * c, bm_r, gridr, s);
    }
    bh.chunk = c < nchunks ? c : -1;
    bx.chunk = c - 1;
    Scope sc_(tm, MOE_STAGE_GEMM2);
    launch_gemm_bwd_pair(d.fmt, bh, bx, queue + 16 * c + 8, bm, gridb, s);
  }
  {
  Scope sc_(tm, MOE_STAGE_COMBINE);
  const float* dx_rows = dxt;
  if (d.oft) {
    launch_oft_bwd(x, static_cast<const uint16_t*>(adapter_bf16), layer->adapter_expert_stride, dxt, d.H, d.k,
                   offsets, sorted_rows, active, num_active, d.E, dxr, d_adapter,
                   reinterpret_cast<float*>(base + wl.drp), s);
    dx_rows = dxr;
  }
  launch_unpermute_sum(dx_rows, row_of, d.T, d.k, d.H, static_cast<uint16_t*>(d_x_bf16), s);
  launch_router_grad(ids, wts, row_of, gpart, d.I / 256, d.T, d.k, d.E, d_logits, s);
  }
  return launch_status();
}
}  // namespace


extern "C" {

moe_status moe_expert_backward(const moe_layer* layer, const void* x_bf16, const float* logits,
                               const moe_qweights* qw, const moe_scales* sc, const void* bwd_weights,
                               const void* adapter_bf16, const void* d_out_bf16, int32_t chunk_experts,
                               void* d_x_bf16, float* d_logits, float* d_adapter, void* ws, size_t ws_bytes,
                               void* stream, float* stage_ms, int32_t* stage_launches) {
  if ((stage_ms == nullptr) != (stage_launches == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (stage_ms == nullptr)
    return backward_impl(layer, x_bf16, logits, qw, sc, bwd_weights, adapter_bf16, d_out_bf16, chunk_experts,
                         d_x_bf16, d_logits, d_adapter, ws, ws_bytes, stream, nullptr);
  StageTimer* tm = new StageTimer();
  tm->s = static_cast<hipStream_t>(stream);
  moe_status st = backward_impl(layer, x_bf16, logits, qw, sc, bwd_weights, adapter_bf16, d_out_bf16,
                                chunk_experts, d_x_bf16, d_logits, d_adapter, ws, ws_bytes, stream, tm);
  tm->finish(stage_ms, stage_launches);
  const bool ok = tm->ok;
  delete tm;
  if (st == MOE_OK && !ok) st = MOE_ERR_DEVICE;
  return st;
}

moe_status moe_combine(const moe_layer* layer, const void* y_perm_bf16, const float* topk_w, const int32_t* row_of,
                       void* out_bf16, void* stream) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  const void* ptrs[] = {y_perm_bf16, topk_w, row_of, out_bf16};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  launch_combine(static_cast<const uint16_t*>(y_perm_bf16), topk_w, row_of, d.T, d.k, d.H,
                 static_cast<uint16_t*>(out_bf16), static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t moe_lm_head_workspace_bytes(int32_t T, int32_t V) {
  if (T < 0 || V <= 0) return 0;
  // per (token, vocabulary block) maximum and sum of exponentials, then the target logits
  return align_up((size_t)T * lm_head_blocks(V) * 2 * 4) + align_up((size_t)T * 4);
}


moe_status moe_lm_head_logprob(int32_t T, int32_t H, int32_t V, const void* h_bf16, const void* w_lm_bf16,
                               const int32_t* targets, float* logprob, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || H <= 0 || V <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128 != 0 || T > 4096) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {h_bf16, w_lm_bf16, targets, logprob, ws};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < moe_lm_head_workspace_bytes(T, V)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  char* base = static_cast<char*>(ws);
  float* stats = reinterpret_cast<float*>(base);
  float* tz = reinterpret_cast<float*>(base + align_up((size_t)T * lm_head_blocks(V) * 2 * 4));
  launch_lm_head(static_cast<const uint16_t*>(h_bf16), static_cast<const uint16_t*>(w_lm_bf16), targets, T, H, V,
                 stats, tz, logprob, static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t moe_materialized_workspace_bytes(const moe_layer* layer, int32_t chunk_experts) {
  Dims d;
  if (check_layer(layer, &d) != MOE_OK || chunk_experts < 1) return 0;
  return mat_layout(d, chunk_experts < d.E ? chunk_experts : d.E).total;
}

moe_status moe_expert_forward_materialized(const moe_layer* layer, const void* x_bf16, const float* logits,
                                           const moe_qweights* qw, const moe_scales* sc, const void* adapter_bf16,
                                           int32_t chunk_experts, void* out_bf16, void* ws, size_t ws_bytes,
                                           void* stream, float* stage_ms, int32_t* stage_launches) {
  if ((stage_ms == nullptr) != (stage_launches == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (stage_ms == nullptr)
    return forward_materialized_impl(layer, x_bf16, logits, qw, sc, adapter_bf16, chunk_experts, out_bf16, ws,
                                     ws_bytes, stream, nullptr);
  StageTimer* tm = new StageTimer();
  tm->s = static_cast<hipStream_t>(stream);
  moe_status st = forward_materialized_impl(layer, x_bf16, logits, qw, sc, adapter_bf16, chunk_experts, out_bf16,
                                            ws, ws_bytes, stream, tm);
  tm->finish(stage_ms, stage_launches);
  const bool ok = tm->ok;
  delete tm;
  if (st == MOE_OK && !ok) st = MOE_ERR_DEVICE;
  return st;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is a file-scope device array, one
// copy per GPU the library runs on, alive until the process ends.

namespace {
// In host code `scratch` names a host-side stand-in, not a device address:
// its device address is taken once per device with hipGetSymbolAddress and
// kept in g_scratch; only that pointer is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch (set-up on the first call per device).
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_expert_forward_noalloc(const moe_layer* layer, const void* x_bf16, const float* logits,
                                                 const moe_qweights* qweights, const moe_scales* scales,
                                                 const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                                                 void* stream) {
  Dims d;
  moe_status st = check_layer(layer, &d);
  if (st != MOE_OK) return st;
  if (chunk_experts < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (layout(d).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MOE_OK) return st;
  return forward_impl(layer, x_bf16, logits, qweights, scales, adapter_bf16, chunk_experts, out_bf16, ws,
                      (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

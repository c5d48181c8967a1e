// Host side of the C ABI declared in include/moe_fp4.h: validation, workspace layout,
// path choice and the launch sequence. Nothing here waits on the device except
// moe_get_device_error.
//
// Validation follows the MoE constructor page (spark_model/layers/moe/init.rs):
// top_k must lie in 1..=num_experts with num_experts > 0, and the routing kernels'
// own capacity bounds are checked up front rather than overrun. Here those bounds
// are this library's (MOE_MAX_EXPERTS, MOE_MAX_TOP_K), set by the top-K kernel's
// register and LDS budget. A weight whose format tag does not match its scale
// layout is an error, never a silent decode in the other format (MoE module page,
// MoeLayer::e8m0_or).
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "moe_fp4.h"
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct Layout {
  size_t partial, logits, ids, w, errtok, xn, row_token, inv, tiles, ntiles, h, y, wcnt,
      errpart, part, part_bytes, x8, xs8, h8, hs8, total;
  int ks, hsplit;
  int rows;        // R
  int h_stride;
  int tile_bound_dec, tile_bound_pre;
};

// Tiles of at most h rows over S rows in at most min(S, E) groups: at most S / h + one
// partial tile per group, and at most S (a tile holds a row). The decode grids have this
// many tile columns; the ones past the device's count exit at once (Qwen3-like decode at
// 8 tokens: 64 columns instead of 81; measured within noise, at most ~0.5 us per kernel).
int tile_bound(int S, int E, int h) {
  const int b = S / h + (S < E ? S : E) + 1;
  const int m = b < S ? b : S;
  return m > 1 ? m : 1;
}

// The shared expert on the MFMA kernels: from this many tokens a decode layer runs it as
// one group over all its tokens (its weights read once per 32-64-128 rows) instead of the
// GEMV's tiles of kDecodeTile tokens (its weights streamed once per 4 tokens).
constexpr int kSharedMfmaMinTokens = 8;

// From this many tokens the shared expert's MFMA launches keep K whole: beside the routed
// experts on the side stream its few long blocks cost the layer less than split-K's short
// blocks with their fp32 partial sums (hash layer, 512 tokens: 0.810 against 0.836 ms). Below
// it, K is split: a DeepSeek-V3-like decode layer's 16 blocks of 112 stages would be on the
// critical path whenever the two streams do not overlap (graph replays: 0.651 against
// 0.610 ms). The choice depends on the configuration alone, so every entry and every replay
// of a configuration rounds the same way.
constexpr int kSharedNoSplitTokens = 256;

// Tile height of the shared expert: its one group holds every token. (Choosing 32-row tiles
// whenever taller ones leave the chip's block slots unfilled, and splitting their K, was
// slower: hash layer shared stage 88.7 us against 71.7 us with 128-row tiles.)
int shared_mt(int T) { return T < 48 ? 32 : (T < 96 ? 64 : 128); }

// Prefill M-tile height from the mean rows per routed expert.
int prefill_mt(const moe_config& c) {
  const int S = c.tokens * c.top_k;
  const int groups = S < c.num_experts ? S : c.num_experts;
  const int rpe = groups > 0 ? S / groups : 0;
  if (rpe < 48) return 32;
  if (rpe < 96) return 64;
  return 128;
}

Layout make_layout(const moe_config& c) {
  Layout L{};
  const int T = c.tokens, E = c.num_experts, K = c.top_k, H = c.hidden;
  const int NE = E + c.zero_experts;  // router outputs
  const int S = T * K;
  L.rows = S + (c.has_shared ? T : 0);
  const RouterPlan rp = plan_router(T, NE, H);
  L.ks = rp.ks;
  L.hsplit = rp.hsplit;
  int imax = c.inter;
  if (c.has_shared && c.shared_inter > imax) imax = c.shared_inter;
  L.h_stride = ceil_div(imax, 8) * 8;
  L.tile_bound_dec = tile_bound(S, E, kDecodeTile);
  L.tile_bound_pre = tile_bound(S, E, prefill_mt(c));
  const int tb = L.tile_bound_dec > L.tile_bound_pre ? L.tile_bound_dec : L.tile_bound_pre;
  size_t off = kAlign;  // header: device error word
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.partial = take((size_t)L.ks * T * NE * sizeof(double));
  L.logits = take((size_t)T * NE * 4);
  L.ids = take((size_t)S * 4);
  L.w = take((size_t)S * 4);
  L.errtok = take((size_t)T * 4);
  L.xn = take(c.pre_norm ? (size_t)T * H * 2 : 0);
  L.row_token = take((size_t)L.rows * 4);
  L.inv = take((size_t)S * 4);
  L.tiles = take((size_t)tb * sizeof(Tile));
  L.ntiles = take(kTileCountBytes);  // the tile count and the GEMMs' work counters
  L.h = take((size_t)L.rows * L.h_stride * 2);
  L.y = take((size_t)L.rows * H * 4);
  // multi-block dispatch (many slots): per-wave expert counts and per-block error bits
  const int dblocks = S >= kDispMultiMinSlots ? dispatch_blocks(S) : 0;
  L.wcnt = take((size_t)dblocks * E * 4);
  L.errpart = take((size_t)dblocks * 4);
  // K-split partial sums of the shared expert's MFMA launches
  L.part_bytes = 0;
  if (c.has_shared && c.tokens < kSharedNoSplitTokens) {
    const int nout = 2 * c.shared_inter > H ? 2 * c.shared_inter : H;
    L.part_bytes = (size_t)kMaxKsplit * T * nout * sizeof(float);
    if (L.part_bytes > kSplitPartMax) L.part_bytes = kSplitPartMax;
  }
  L.part = take(L.part_bytes);
#if MOE_PRE_MX8
  L.x8 = take((size_t)T * H * 2);
  L.xs8 = take((size_t)T * (H / 32) * 2);
  L.h8 = take((size_t)L.rows * L.h_stride * 2);
  L.hs8 = take((size_t)L.rows * (imax / 32) * 2);
#endif
  L.total = off;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->tokens < 0 || c->hidden <= 0 || c->hidden % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (c->num_experts <= 0 || c->zero_experts < 0) return MOE_ERR_INVALID_ARG;
  const int64_t ntot = (int64_t)c->num_experts + c->zero_experts;  // router outputs
  if (c->top_k < 1 || c->top_k > ntot) return MOE_ERR_INVALID_ARG;
  if (ntot > MOE_MAX_EXPERTS || c->top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
  if (c->inter <= 0 || c->inter % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (c->score_mode != MOE_SCORE_SOFTMAX && c->score_mode != MOE_SCORE_SIGMOID &&
      c->score_mode != MOE_SCORE_SQRT_SOFTPLUS && c->score_mode != MOE_SCORE_SOFTMAX_BIAS)
    return MOE_ERR_INVALID_ARG;
  if (c->select_mode != MOE_SELECT_TOPK && c->select_mode != MOE_SELECT_HASH)
    return MOE_ERR_INVALID_ARG;
  if (c->select_mode == MOE_SELECT_HASH && c->vocab <= 0) return MOE_ERR_INVALID_ARG;
  if (c->has_shared && (c->shared_inter <= 0 || c->shared_inter % 32 != 0))
    return MOE_ERR_INVALID_ARG;
  if (c->path < MOE_PATH_AUTO || c->path > MOE_PATH_PREFILL) return MOE_ERR_INVALID_ARG;
  if (!(c->routed_scaling == c->routed_scaling)) return MOE_ERR_INVALID_ARG;
  if (c->pre_norm && !(c->norm_eps >= 0.f)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)c->tokens * c->top_k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_weight(const moe_fp4_weight& w, int experts, int n, int k) {
  switch (w.format) {
    case MOE_FMT_NVFP4:
      if (!w.global_scale) return MOE_ERR_FORMAT;
      break;
    case MOE_FMT_MXFP4:
    case MOE_FMT_FP8:
      if (w.global_scale) return MOE_ERR_FORMAT;
      break;
    case MOE_FMT_BF16:
      if (w.global_scale || w.scales) return MOE_ERR_FORMAT;
      break;
    default:
      return MOE_ERR_FORMAT;
  }
  if (!w.packed || (w.format != MOE_FMT_BF16 && !w.scales)) return MOE_ERR_INVALID_ARG;
  if (w.format == MOE_FMT_FP8 && k > 16384) return MOE_ERR_UNSUPPORTED;
  if (w.experts != experts || w.n != n || w.k != k) return MOE_ERR_INVALID_ARG;
  if (k % 32 != 0 || n <= 0) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w.packed) || (w.scales && !aligned16(w.scales))) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_group(const moe_expert_weights* g, int experts, int H, int I) {
  if (!g) return MOE_ERR_INVALID_ARG;
  int r;
  if ((r = check_weight(g->gate, experts, I, H)) != MOE_OK) return r;
  if ((r = check_weight(g->up, experts, I, H)) != MOE_OK) return r;
  if ((r = check_weight(g->down, experts, H, I)) != MOE_OK) return r;
  if (g->gate.format != g->up.format) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

WeightDesc desc(const moe_fp4_weight& w) {
  WeightDesc d;
  d.packed = w.packed;
  d.scales = w.scales;
  d.global = w.global_scale;
  d.fmt = w.format;
  d.n = w.n;
  d.k = w.k;
  return d;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(ws) + off);
}

// Which expert path runs, or an error when a forced path cannot take the shapes.
int choose_path(const moe_config& c, int* path) {
  const bool pre_ok = c.hidden % 64 == 0 && c.inter % 64 == 0 &&
                      (!c.has_shared || c.shared_inter % 64 == 0);
  // decode stages a tile's activation rows in LDS: kTileTok rows of K bf16 in 160 KB
  int kmax = c.hidden > c.inter ? c.hidden : c.inter;
  if (c.has_shared && c.shared_inter > kmax) kmax = c.shared_inter;
  const bool dec_ok = (long long)kTileTok * kmax * 2 <= kDecodeMaxLds;
  if (c.path == MOE_PATH_DECODE) {
    if (!dec_ok) return MOE_ERR_UNSUPPORTED;
    *path = MOE_PATH_DECODE;
    return MOE_OK;
  }
  if (c.path == MOE_PATH_PREFILL) {
    if (!pre_ok) return MOE_ERR_UNSUPPORTED;
    *path = MOE_PATH_PREFILL;
    return MOE_OK;
  }
  const int S = c.tokens * c.top_k;
  const int groups = S < c.num_experts ? S : c.num_experts;
  const bool many_rows = groups > 0 && S >= 4 * groups;
  if ((many_rows || !dec_ok) && pre_ok) {
    *path = MOE_PATH_PREFILL;
    return MOE_OK;
  }
  if (!dec_ok) return MOE_ERR_UNSUPPORTED;
  *path = MOE_PATH_DECODE;
  return MOE_OK;
}

// Whether the shared expert runs on the MFMA kernels: always on the prefill path; on the
// decode path from kSharedMfmaMinTokens tokens when its sizes suit the MFMA tiles.
bool shared_on_mfma(const moe_config& c, bool pre) {
  if (pre) return true;
  return c.tokens >= kSharedMfmaMinTokens && c.hidden % 64 == 0 && c.shared_inter % 64 == 0;
}

#define MOE_HIP(call)                          \
  do {                                         \
    if ((call) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// One-shot stage-event request of this host thread (moe_set_stage_events).
thread_local hipEvent_t* t_stage_events = nullptr;
thread_local int t_stage_count = 0;

// The shared expert on a secondary stream (MoE constructor page: the shared expert overlaps
// the routed experts on a second stream, joined by an event pair before the blend). Each
// caller stream gets its own side stream and fork / join events, created on first use
// (never while the caller's stream is being captured into a graph) and kept until the
// process ends; the side stream is non-blocking and of default priority. Calls on one
// caller stream are ordered by the caller, so its side stream and events are never used by
// two calls at once.
#ifndef MOE_SHARED_SIDE_STREAM
#define MOE_SHARED_SIDE_STREAM 1
#endif
struct SideStream {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::map<std::pair<int, hipStream_t>, SideStream> g_side;

// The side stream of `s`, or nullptr (run the shared expert on `s` itself) when it cannot be
// had without creating it during a capture, or when creating it fails.
const SideStream* side_stream(hipStream_t s) {
  if (!MOE_SHARED_SIDE_STREAM) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_side_mu);
  auto it = g_side.find({dev, s});
  if (it != g_side.end()) return &it->second;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return nullptr;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  SideStream ss;
  bool ok = hipStreamCreateWithFlags(&ss.side, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
  if (cur != dev) ok = (hipSetDevice(cur) == hipSuccess) && ok;
  if (!ok) {
    if (ss.join) (void)hipEventDestroy(ss.join);
    if (ss.fork) (void)hipEventDestroy(ss.fork);
    if (ss.side) (void)hipStreamDestroy(ss.side);
    return nullptr;
  }
  return &(g_side[{dev, s}] = ss);
}

struct StageMarks {
  hipEvent_t* ev = nullptr;
  int n = 0;
  hipStream_t s = nullptr;
  hipError_t mark(int i) const {
    return (ev && i < n && ev[i]) ? hipEventRecord(ev[i], s) : hipSuccess;
  }
};

DispatchArgs make_dispatch_args(const moe_config& c, const Layout& L, const int32_t* ids,
                                const int32_t* err_tok, void* ws) {
  int path = MOE_PATH_DECODE;
  choose_path(c, &path);
  DispatchArgs d{};
  d.ids = ids;
  d.err_tok = err_tok;
  d.row_token = at<int32_t>(ws, L.row_token);
  d.inv = at<int32_t>(ws, L.inv);
  d.tiles = at<Tile>(ws, L.tiles);
  d.ntiles = at<int32_t>(ws, L.ntiles);
  d.err_word = at<int32_t>(ws, 0);
  d.T = c.tokens;
  d.K = c.top_k;
  d.E = c.num_experts;
  d.zero = c.zero_experts;
  d.shared_rows = c.has_shared ? c.tokens : 0;
  d.tile_h = path == MOE_PATH_PREFILL ? prefill_mt(c) : kDecodeTile;
  d.wcnt = at<int32_t>(ws, L.wcnt);
  d.err_part = at<int32_t>(ws, L.errpart);
  return d;
}

// Dispatch (unless the caller already built it) + experts + blend on a validated config.
// The shared expert: one group over rows [0, T) (implicit tile list), on the MFMA kernels
// (with K split over blocks when its tiles are few) unless a decode layer has too few
// tokens for them to pay. `base` carries the input, h, y and sizes of the call.
int launch_shared(const moe_config& c, const Layout& L, const ExpertGemmArgs& base,
                  const moe_expert_weights* shared, bool pre, void* ws, hipStream_t s) {
  const bool sh_pre = shared_on_mfma(c, pre);
  const int smt = sh_pre ? shared_mt(c.tokens) : kDecodeTile;
  ExpertGemmArgs b = base;
  b.src.tiles = nullptr;
  b.src.ntiles = nullptr;
  b.work = nullptr;
  b.src.implicit_row0 = 0;
  b.src.implicit_rows = c.tokens;
  b.src.implicit_height = smt;
  b.tile_bound = ceil_div(c.tokens, smt);
  b.gate = desc(shared->gate);
  b.up = desc(shared->up);
  b.down = desc(shared->down);
  b.I = c.shared_inter;
  b.y_half = 0;  // the shared expert's rows stay fp32
  b.err_word = nullptr;
  b.part = L.part_bytes ? at<float>(ws, L.part) : nullptr;
  b.part_bytes = L.part_bytes;
  if (sh_pre) {
    MOE_HIP(launch_prefill_gate_up(b, smt, s));
    MOE_HIP(launch_prefill_down(b, smt, s));
  } else {
    MOE_HIP(launch_decode_gate_up(b, s));
    MOE_HIP(launch_decode_down(b, s));
  }
  return MOE_OK;
}

int run_experts(const moe_config& c, const Layout& L, const uint16_t* xe, const int32_t* ids,
                const float* w, const int32_t* err_tok, const moe_expert_weights* routed,
                const moe_expert_weights* shared, const uint16_t* residual, uint16_t* out,
                void* ws, hipStream_t s, const StageMarks& marks = StageMarks(),
                bool dispatched = false, const TopkArgs* fused_topk = nullptr,
                bool allow_side = true) {
  int path;
  int r = choose_path(c, &path);
  if (r != MOE_OK) return r;
  const bool pre = path == MOE_PATH_PREFILL;
  const int mt = pre ? prefill_mt(c) : kDecodeTile;

  ExpertGemmArgs a{};
  a.x = xe;
  a.h = at<uint16_t>(ws, L.h);
  a.h_stride = L.h_stride;
  a.y = at<void>(ws, L.y);
  a.T = c.tokens;
  a.H = c.hidden;
  a.I = c.inter;
  a.rows = L.rows;
  // the shared expert needs only the input: with a side stream it starts now and runs
  // beside the dispatch and the routed experts, joined before the blend. Only where its
  // launches leave most of the chip idle (the GEMV's few tiles at few tokens, or unsplit
  // MFMA blocks from kSharedNoSplitTokens tokens): MFMA launches whose K is split over
  // blocks fill the chip themselves, and beside the routed experts they only slow those
  // (DeepSeek-V3-like decode at 32 tokens: layer 0.557 ms either way, routed gate+up 339
  // against 324 us).
  const bool shared_fills = c.has_shared && shared_on_mfma(c, pre) && L.part_bytes > 0;
  const SideStream* side = c.has_shared && allow_side && !shared_fills ? side_stream(s) : nullptr;
  if (side) {
    MOE_HIP(hipEventRecord(side->fork, s));
    MOE_HIP(hipStreamWaitEvent(side->side, side->fork, 0));
    if ((r = launch_shared(c, L, a, shared, pre, ws, side->side)) != MOE_OK) return r;
    MOE_HIP(hipEventRecord(side->join, side->side));
  }

  const DispatchArgs d = make_dispatch_args(c, L, ids, err_tok, ws);
  if (!dispatched) MOE_HIP(launch_dispatch(d, s));
  MOE_HIP(marks.mark(MOE_STAGE_DISPATCHED));

  a.row_token = d.row_token;
  a.src.tiles = d.tiles;
  a.src.ntiles = d.ntiles;
  a.tile_bound = pre ? L.tile_bound_pre : L.tile_bound_dec;
  a.gate = desc(routed->gate);
  a.up = desc(routed->up);
  a.down = desc(routed->down);
  CombineArgs cb{};
  cb.y = reinterpret_cast<const float*>(a.y);
  // routed prefill rows of y as fp16, after the shared expert's fp32 rows: row r >=
  // shared_rows at byte 2 * H * (shared_rows + r) of the y region (past the 4 * H *
  // shared_rows bytes of fp32 rows; the last row ends within the region's 4 * H * rows bytes)
  ExpertGemmArgs ad = a;
  if (pre) {
    uint16_t* y16 = at<uint16_t>(ws, L.y) + (size_t)d.shared_rows * c.hidden;
    cb.y16 = y16;
    ad.y = y16;
    ad.y_half = 1;
    ad.err_word = d.err_word;
  }
  cb.xe = xe;
  cb.w = w;
  cb.inv = d.inv;
  cb.shared = c.has_shared;
  cb.residual = residual;
  cb.out = out;
  cb.T = c.tokens;
  cb.K = c.top_k;
  cb.H = c.hidden;
  // one token without a shared expert: the blend runs inside the down kernel
  const bool blend_in_down = !pre && decode_blend_fusable(a, cb);
  if (pre) {
    a.work = d.ntiles + kWorkCtrOffset;
#if MOE_PRE_MX8
    const bool mx8 = routed->gate.format == MOE_FMT_MXFP4 && mt == 128;
    if (mx8) {
      MOE_HIP(launch_quant_mx8(xe, c.tokens, c.hidden, c.hidden, at<uint8_t>(ws, L.x8),
                               at<uint16_t>(ws, L.xs8), s));
      a.a8 = at<uint8_t>(ws, L.x8);
      a.a8s = at<uint16_t>(ws, L.xs8);
    }
#endif
    MOE_HIP(launch_prefill_gate_up(a, mt, s));
    MOE_HIP(marks.mark(MOE_STAGE_GATE_UP));
    a.work = d.ntiles + kWorkCtrOffset + kXcds * kWorkCtrStride;
#if MOE_PRE_MX8
    if (mx8) {
      MOE_HIP(launch_quant_mx8(a.h, L.rows, c.inter, L.h_stride, at<uint8_t>(ws, L.h8),
                               at<uint16_t>(ws, L.hs8), s));
      a.a8 = at<uint8_t>(ws, L.h8);
      a.a8s = at<uint16_t>(ws, L.hs8);
    }
#endif
    ad.work = a.work;
#if MOE_PRE_MX8
    ad.a8 = a.a8;
    ad.a8s = a.a8s;
#endif
    MOE_HIP(launch_prefill_down(ad, mt, s));
  } else {
    if (fused_topk) {  // one token: selection and dispatch inside the gate+up kernel
      FusedRoute fr{};
      fr.row_token = d.row_token;
      fr.inv = d.inv;
      fr.tiles = d.tiles;
      fr.ntiles = d.ntiles;
      fr.err_word = d.err_word;
      fr.shared_rows = d.shared_rows;
      MOE_HIP(launch_decode_gate_up_topk(a, *fused_topk, fr, s));
    } else {
      MOE_HIP(launch_decode_gate_up(a, s));
    }
    MOE_HIP(marks.mark(MOE_STAGE_GATE_UP));
    if (blend_in_down) {
      MOE_HIP(launch_decode_down_blend(a, cb, s));
    } else {
      MOE_HIP(launch_decode_down(a, s));
    }
  }
  MOE_HIP(marks.mark(MOE_STAGE_DOWN));
  if (side) {
    MOE_HIP(hipStreamWaitEvent(s, side->join, 0));
  } else if (c.has_shared) {
    if ((r = launch_shared(c, L, a, shared, pre, ws, s)) != MOE_OK) return r;
  }
  MOE_HIP(marks.mark(MOE_STAGE_SHARED));
  if (!blend_in_down) MOE_HIP(launch_combine(cb, s));
  MOE_HIP(marks.mark(MOE_STAGE_COMBINED));
  return MOE_OK;
}

int check_ws(const Layout& L, const void* ws, size_t bytes) {
  if (!ws || bytes < L.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

TopkArgs make_topk_args(const moe_config& c, const Layout& L, const float* logit_bias,
                        const float* corr, const int32_t* token_ids, const int64_t* tid2eid,
                        const float* logits_in, float* logits_out, int32_t* ids, float* w,
                        void* ws) {
  TopkArgs t{};
  t.partial = logits_in ? nullptr : at<double>(ws, L.partial);
  t.ks = L.ks;
  t.logits_in = logits_in;
  t.logit_bias = logit_bias;
  t.correction_bias = c.score_mode != MOE_SCORE_SOFTMAX ? corr : nullptr;
  t.token_ids = token_ids;
  t.tid2eid = tid2eid;
  t.vocab = c.vocab;
  t.logits_out = logits_out;
  t.ids = ids;
  t.w = w;
  t.err_tok = at<int32_t>(ws, L.errtok);
  t.T = c.tokens;
  t.E = c.num_experts + c.zero_experts;  // selection runs over the zero experts too
  t.K = c.top_k;
  t.score = c.score_mode;
  t.select = c.select_mode;
  t.renorm = c.renormalize;
  t.scaling = c.routed_scaling;
  return t;
}

// Router GEMM (unless logits_in) + top-K. With fuse_dispatch and few tokens, the top-K
// runs fused with the dispatch build and *dispatched is set; the stage mark ROUTED is
// then recorded between the router GEMM and that kernel.
int launch_route(const moe_config& c, const Layout& L, const uint16_t* x,
                 const uint16_t* router_w, const float* logit_bias, const float* corr,
                 const int32_t* token_ids, const int64_t* tid2eid, const float* logits_in,
                 float* logits_out, int32_t* ids, float* w, void* ws, hipStream_t s,
                 const StageMarks* marks = nullptr, bool* dispatched = nullptr) {
  const int NE = c.num_experts + c.zero_experts;
  const TopkArgs t = make_topk_args(c, L, logit_bias, corr, token_ids, tid2eid, logits_in,
                                    logits_out, ids, w, ws);
  // hash routing whose weights need only the selected experts' logits, none asked for: no
  // router GEMM (unless the top-K runs fused with the dispatch)
  const bool fuse_dispatch = dispatched && fused_topk_dispatch_fits(c.tokens, NE, c.top_k);
  if (!fuse_dispatch && hash_gather_fits(t, c.hidden)) {
    MOE_HIP(launch_hash_gather(t, x, router_w, c.hidden, s));
    if (marks) MOE_HIP(marks->mark(MOE_STAGE_ROUTED));
    return MOE_OK;
  }
  if (!logits_in)
    MOE_HIP(launch_router_partial(x, router_w, at<double>(ws, L.partial), c.tokens, NE,
                                  c.hidden, L.ks, L.hsplit, s));
  if (fuse_dispatch) {
    if (marks) MOE_HIP(marks->mark(MOE_STAGE_ROUTED));
    const DispatchArgs d = make_dispatch_args(c, L, ids, t.err_tok, ws);
    MOE_HIP(launch_topk_dispatch(t, d, s));
    *dispatched = true;
    return MOE_OK;
  }
  MOE_HIP(launch_topk(t, s));
  if (marks) MOE_HIP(marks->mark(MOE_STAGE_ROUTED));
  return MOE_OK;
}

// One token with top-K selection over at most 128 experts on the one-step decode GEMV: the
// selection and the dispatch run inside the gate+up kernel (one launch fewer).
bool topk_in_gate_up(const moe_config& c, const moe_expert_weights& routed) {
  int path;
  if (choose_path(c, &path) != MOE_OK || path != MOE_PATH_DECODE) return false;
  return c.tokens == 1 && c.select_mode == MOE_SELECT_TOPK && c.zero_experts == 0 &&
         decode_topk_fusable(routed.gate.format, c.hidden, c.num_experts);
}

int check_route_ptrs(const moe_config& c, const uint16_t* x, const uint16_t* router_w,
                     const int32_t* token_ids, const int64_t* tid2eid, const float* logits_in) {
  if (!logits_in && (!x || !router_w)) return MOE_ERR_INVALID_ARG;
  if (c.select_mode == MOE_SELECT_HASH && (!token_ids || !tid2eid)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ------------------------------------------------------------ no-allocation entry point
// The workspace of moe_layer_forward_noalloc: a fixed array of device memory. Every GPU the
// library runs on holds its own copy (at its own address) until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: kernels and copies
// only ever get the address hipGetSymbolAddress returns for the device in question.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of the scratch array on the device of `stream`, looked up once per device
// with that device current.
int scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
    if (e != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the library's limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime or launch failure";
    case MOE_ERR_FORMAT: return "MOE_ERR_FORMAT: weight format tag inconsistent with its scales";
    default: return "unknown moe_status";
  }
}

int moe_workspace_size(const moe_config* cfg, size_t* bytes_out) {
  int r = check_config(cfg);
  if (r != MOE_OK) return r;
  if (!bytes_out) return MOE_ERR_INVALID_ARG;
  *bytes_out = make_layout(*cfg).total;
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const uint16_t* x, const uint16_t* router_w,
              const float* logit_bias, const float* correction_bias, const int32_t* token_ids,
              const int64_t* tid2eid, const float* logits_in, float* logits_out,
              int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  int r = check_config(cfg);
  if (r != MOE_OK) return r;
  const moe_config& c = *cfg;
  if (c.tokens == 0) return MOE_OK;  // no-op: no pointer is touched
  if ((r = check_route_ptrs(c, x, router_w, token_ids, tid2eid, logits_in)) != MOE_OK) return r;
  if (!topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(c);
  if ((r = check_ws(L, workspace, workspace_bytes)) != MOE_OK) return r;
  if (c.tokens == 0) return MOE_OK;
  return launch_route(c, L, x, router_w, logit_bias, correction_bias, token_ids, tid2eid,
                      logits_in, logits_out, topk_ids, topk_w, workspace, stream);
}

int moe_experts_forward(const moe_config* cfg, const uint16_t* x_experts,
                        const int32_t* topk_ids, const float* topk_w,
                        const moe_expert_weights* routed, const moe_expert_weights* shared,
                        const uint16_t* residual, uint16_t* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int r = check_config(cfg);
  if (r != MOE_OK) return r;
  const moe_config& c = *cfg;
  if (c.tokens == 0) return MOE_OK;  // no-op: no pointer is touched
  if (!x_experts || !topk_ids || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_experts) || !aligned16(out) || (residual && !aligned16(residual)))
    return MOE_ERR_INVALID_ARG;
  if (out == x_experts) return MOE_ERR_INVALID_ARG;
  if ((r = check_group(routed, c.num_experts, c.hidden, c.inter)) != MOE_OK) return r;
  if (c.has_shared) {
    if ((r = check_group(shared, 1, c.hidden, c.shared_inter)) != MOE_OK) return r;
  }
  int path;
  if ((r = choose_path(c, &path)) != MOE_OK) return r;
  const Layout L = make_layout(c);
  if ((r = check_ws(L, workspace, workspace_bytes)) != MOE_OK) return r;
  if (c.tokens == 0) return MOE_OK;
  return run_experts(c, L, x_experts, topk_ids, topk_w, nullptr, routed,
                     c.has_shared ? shared : nullptr, residual, out, workspace, stream);
}

// moe_layer_forward; allow_side = false keeps the shared expert on `stream` (the
// no-allocation entry creates no side stream).
static int layer_forward_impl(const moe_config* cfg, const uint16_t* x,
                              const uint16_t* norm_gamma, const uint16_t* router_w,
                              const float* logit_bias, const float* correction_bias,
                              const int32_t* token_ids, const int64_t* tid2eid,
                              const moe_expert_weights* routed, const moe_expert_weights* shared,
                              const uint16_t* residual, uint16_t* out, float* dbg_logits,
                              int32_t* dbg_ids, float* dbg_w, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, bool allow_side) {
  int r = check_config(cfg);
  if (r != MOE_OK) return r;
  const moe_config& c = *cfg;
  if (c.tokens == 0) return MOE_OK;  // no-op: no pointer is touched
  if (!x || !router_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out) || (residual && !aligned16(residual)))
    return MOE_ERR_INVALID_ARG;
  if (out == x) return MOE_ERR_INVALID_ARG;
  if (c.pre_norm && (!norm_gamma || !aligned16(norm_gamma))) return MOE_ERR_INVALID_ARG;
  if ((r = check_route_ptrs(c, x, router_w, token_ids, tid2eid, nullptr)) != MOE_OK) return r;
  if ((r = check_group(routed, c.num_experts, c.hidden, c.inter)) != MOE_OK) return r;
  if (c.has_shared) {
    if ((r = check_group(shared, 1, c.hidden, c.shared_inter)) != MOE_OK) return r;
  }
  int path;
  if ((r = choose_path(c, &path)) != MOE_OK) return r;
  const Layout L = make_layout(c);
  if ((r = check_ws(L, workspace, workspace_bytes)) != MOE_OK) return r;
  if (c.tokens == 0) return MOE_OK;
  StageMarks marks;
  marks.ev = t_stage_events;
  marks.n = t_stage_count;
  marks.s = stream;
  t_stage_events = nullptr;
  t_stage_count = 0;
  MOE_HIP(marks.mark(MOE_STAGE_BEGIN));
  const uint16_t* xe = x;
  if (c.pre_norm) {
    uint16_t* xn = at<uint16_t>(workspace, L.xn);
    MOE_HIP(launch_rmsnorm(x, norm_gamma, xn, c.tokens, c.hidden, c.norm_eps, stream));
    xe = xn;
  }
  int32_t* ids = at<int32_t>(workspace, L.ids);
  float* w = at<float>(workspace, L.w);
  bool dispatched = false;
  TopkArgs fused{};
  const bool fuse = topk_in_gate_up(c, *routed);
  if (fuse) {
    // one token, top-K: the router GEMM here, the selection inside the gate+up kernel
    MOE_HIP(launch_router_partial(x, router_w, at<double>(workspace, L.partial), c.tokens,
                                  c.num_experts, c.hidden, L.ks, L.hsplit, stream));
    MOE_HIP(marks.mark(MOE_STAGE_ROUTED));
    fused = make_topk_args(c, L, logit_bias, correction_bias, token_ids, tid2eid, nullptr,
                           dbg_logits, ids, w, workspace);
    dispatched = true;
  } else {
    r = launch_route(c, L, x, router_w, logit_bias, correction_bias, token_ids, tid2eid, nullptr,
                     dbg_logits, ids, w, workspace, stream, &marks, &dispatched);
    if (r != MOE_OK) return r;
  }
  r = run_experts(c, L, xe, ids, w, at<int32_t>(workspace, L.errtok), routed,
                  c.has_shared ? shared : nullptr, residual, out, workspace, stream, marks,
                  dispatched, fuse ? &fused : nullptr, allow_side);
  if (r != MOE_OK) return r;
  const size_t slots = (size_t)c.tokens * c.top_k;
  if (dbg_ids) MOE_HIP(hipMemcpyAsync(dbg_ids, ids, slots * 4, hipMemcpyDeviceToDevice, stream));
  if (dbg_w) MOE_HIP(hipMemcpyAsync(dbg_w, w, slots * 4, hipMemcpyDeviceToDevice, stream));
  return MOE_OK;
}

int moe_layer_forward(const moe_config* cfg, const uint16_t* x, const uint16_t* norm_gamma,
                      const uint16_t* router_w, const float* logit_bias,
                      const float* correction_bias, const int32_t* token_ids,
                      const int64_t* tid2eid, const moe_expert_weights* routed,
                      const moe_expert_weights* shared, const uint16_t* residual,
                      uint16_t* out, float* dbg_logits, int32_t* dbg_ids, float* dbg_w,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return layer_forward_impl(cfg, x, norm_gamma, router_w, logit_bias, correction_bias,
                            token_ids, tid2eid, routed, shared, residual, out, dbg_logits,
                            dbg_ids, dbg_w, workspace, workspace_bytes, stream, true);
}

int moe_layer_forward_noalloc(const moe_config* cfg, const uint16_t* x,
                              const uint16_t* norm_gamma, const uint16_t* router_w,
                              const float* logit_bias, const float* correction_bias,
                              const int32_t* token_ids, const int64_t* tid2eid,
                              const moe_expert_weights* routed, const moe_expert_weights* shared,
                              const uint16_t* residual, uint16_t* out, float* dbg_logits,
                              int32_t* dbg_ids, float* dbg_w, hipStream_t stream) {
  int r = check_config(cfg);
  if (r != MOE_OK) return r;
  if (cfg->tokens == 0) return MOE_OK;  // no-op: no pointer is touched
  if (make_layout(*cfg).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((r = scratch_address(stream, &ws)) != MOE_OK) return r;
  return layer_forward_impl(cfg, x, norm_gamma, router_w, logit_bias, correction_bias,
                            token_ids, tid2eid, routed, shared, residual, out, dbg_logits,
                            dbg_ids, dbg_w, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, false);
}

int moe_debug_dequant_fp4(const moe_fp4_weight* w, int32_t expert, int32_t path, float* out,
                          hipStream_t stream) {
  if (!w || !out) return MOE_ERR_INVALID_ARG;
  int r = check_weight(*w, w->experts, w->n, w->k);
  if (r != MOE_OK) return r;
  if (expert < 0 || expert >= w->experts) return MOE_ERR_INVALID_ARG;
  if (path != MOE_PATH_DECODE && path != MOE_PATH_PREFILL) return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_debug_dequant(desc(*w), expert, path, out, stream));
  return MOE_OK;
}

int moe_set_stage_events(hipEvent_t* events, int32_t count) {
  if (events && count < 0) return MOE_ERR_INVALID_ARG;
  t_stage_events = events;
  t_stage_count = events ? count : 0;
  return MOE_OK;
}

int moe_get_device_error(const void* workspace, size_t workspace_bytes, int32_t* host_err,
                         hipStream_t stream) {
  if (!workspace || workspace_bytes < kAlign || !host_err) return MOE_ERR_INVALID_ARG;
  MOE_HIP(hipMemcpyAsync(host_err, workspace, 4, hipMemcpyDeviceToHost, stream));
  MOE_HIP(hipStreamSynchronize(stream));
  return MOE_OK;
}

}  // extern "C"

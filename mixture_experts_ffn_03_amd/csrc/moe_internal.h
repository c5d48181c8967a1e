// Internal interface between the host side of the library (moe_api.hip) and the
// kernel translation units: argument structs and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One projection of an expert group, with device pointers. Expert e's matrix is
// packed + e * n * (k/2) bytes, scales + e * n * (k/blk) bytes (blk = 16 NVFP4, 32 MXFP4).
struct WeightDesc {
  const uint8_t* packed;
  const uint8_t* scales;
  const float* global;  // NVFP4 only
  int32_t fmt;          // 0 NVFP4, 1 MXFP4
  int32_t n;
  int32_t k;
};

// A run of rows of one expert group in the expert-sorted row space. Tiles of at most
// kTileTok rows also carry the tokens of their rows (saves a dependent load in decode).
constexpr int kTileTok = 4;
struct Tile {
  int32_t group;
  int32_t row0;
  int32_t count;
  int32_t pad;
  int32_t tok[kTileTok];
};

// Where the rows a kernel processes come from: either the device tile list written by
// the dispatch kernel, or an implicit list of fixed-height tiles over a known row range
// (the shared expert, whose rows are [0, T) of the row space). Row r of an implicit list
// holds token r - implicit_row0, so its kernels read no dispatch output and may run
// before or beside the dispatch.
struct TileSource {
  const Tile* tiles;       // device list, or nullptr for the implicit list
  const int32_t* ntiles;   // device count of the list
  int32_t implicit_row0;   // implicit list: first row
  int32_t implicit_rows;   // implicit list: number of rows
  int32_t implicit_height; // implicit list: rows per tile
};

// Work counters of the persistent prefill GEMMs, beside the tile count: one per XCD and
// launch (gate+up, down), each on its own 64-byte line, after the count's 256-byte line.
// Every writer of the tile count zeroes them (publish_tile_count), so each call's GEMMs
// start from zero without a memset.
constexpr int kXcds = 8;             // XCDs of the chip; block ids go round-robin over them
constexpr int kWorkCtrOffset = 64;   // int32 index of the first counter
constexpr int kWorkCtrStride = 16;   // int32s between counters
constexpr int kWorkCtrSets = 2;      // gate+up, down
constexpr size_t kTileCountBytes = (size_t)(kWorkCtrOffset + kWorkCtrSets * kXcds * kWorkCtrStride) * 4;

constexpr int kMaxExperts = 1024;  // MOE_MAX_EXPERTS
constexpr int kMaxTopK = 32;       // MOE_MAX_TOP_K
constexpr int kDecodeTile = 4;     // rows (tokens) per decode tile
constexpr int kDecodeMaxLds = 160 * 1024;  // staged activations of a decode tile

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, uint16_t* out, int T, int H,
                          float eps, hipStream_t s);

// Router GEMM split: H is summed in ks slices of hsplit columns (fp64 partials from the
// fp64-MFMA kernel, added in slice order by the top-K kernel).
constexpr int kRouterMaxSplit = 8;  // H slices of the router sum
struct RouterPlan {
  int ks, hsplit;
};
RouterPlan plan_router(int T, int E, int H);

hipError_t launch_router_partial(const uint16_t* x, const uint16_t* w, double* partial, int T,
                                 int E, int H, int ks, int hsplit, hipStream_t s);

struct TopkArgs {
  const double* partial;  // [ks, T, E] or nullptr when logits_in is used
  int ks;
  const float* logits_in;
  const float* logit_bias;
  const float* correction_bias;
  const int32_t* token_ids;
  const int64_t* tid2eid;
  int64_t vocab;
  float* logits_out;
  int32_t* ids;
  float* w;
  int32_t* err_tok;
  int T, E, K;
  int score, select, renorm;
  float scaling;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Hash routing from the selected experts' logits only (no router GEMM), where the scores
// allow it and no logits are asked for.
bool hash_gather_fits(const TopkArgs& a, int H);
hipError_t launch_hash_gather(const TopkArgs& a, const uint16_t* x, const uint16_t* w, int H,
                              hipStream_t s);

struct DispatchArgs {
  const int32_t* ids;     // [T, K]
  const int32_t* err_tok; // [T] or nullptr
  int32_t* row_token;     // [R]
  int32_t* inv;           // [T*K]
  Tile* tiles;
  int32_t* ntiles;
  int32_t* err_word;
  int T, K, E, shared_rows, tile_h;
  int zero;               // ids in [E, E + zero): zero-computation experts (inv = -2)
  int32_t* wcnt;          // multi-block dispatch: [E, blocks] slot counts
  int32_t* err_part;      // multi-block dispatch: [blocks] error bits
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
// Many slots with prefill tiles: the dispatch runs as two multi-block launches (per-wave
// expert counts, then scatter) over chunks of kDispChunk slots.
constexpr int kDispChunk = 1024;  // slots per block (16 waves x 64)
constexpr int kDispMultiMinSlots = 8192;
inline bool dispatch_multi_block(int S, int tile_h) {
  return S >= kDispMultiMinSlots && tile_h > kTileTok;
}
// blocks of the multi-block dispatch, a multiple of 4 (16-byte count rows)
inline int dispatch_blocks(int S) { return ((S + kDispChunk - 1) / kDispChunk + 3) / 4 * 4; }

// Top-K and dispatch fused in one block (few tokens: decode).
constexpr int kFusedMaxTokens = 16;  // one block: beyond this, separate kernels are faster
constexpr int kFusedMaxExperts = 256;
constexpr int kFusedMaxSlots = 1024;
bool fused_topk_dispatch_fits(int T, int E, int K);
hipError_t launch_topk_dispatch(const TopkArgs& ta, const DispatchArgs& da, hipStream_t s);


struct ExpertGemmArgs {
  const uint16_t* x;          // bf16 [T, H] expert input
  const int32_t* row_token;   // [R]
  TileSource src;
  int tile_bound;             // grid rows (>= number of tiles)
  WeightDesc gate, up, down;
  uint16_t* h;                // bf16 [R, h_stride]
  int h_stride;
  void* y;                    // [R, H] fp32
  int T, H, I;
  int rows;                   // R: rows of the row space (h and y)
  // prefill over an implicit row list (the shared expert) may split K over blocks:
  // fp32 partial sums [ksplit][implicit_rows][2*I (gate+up) or H (down)] in `part`
  // (at most part_bytes), added in split order by a reduce kernel
  float* part;
  size_t part_bytes;
  int ksplit;                 // set by the launcher
  // per-XCD work counters of a persistent launch over the device tile list (zeroed by the
  // dispatch), or nullptr: one block per tile
  int32_t* work;
  // prefill down over the device tile list: store y as fp16 (uint16_t rows [R, H], row r at
  // y + r * H), saturating at +-65504 and setting MOE_DEVERR_Y_RANGE in *err_word; else fp32
  int y_half;
  int32_t* err_word;
#if MOE_PRE_MX8
  // block-scaled MFMA variant (build flag, off by default; see moe_prefill.hip): activations
  // as MXFP8 hi + lo pairs ([rows][K/32][32 hi bytes, 32 lo bytes], same row bytes as bf16)
  // with E8M0 scales [rows][K/32] (hi | lo << 8)
  const uint8_t* a8;
  const uint16_t* a8s;
#endif
};
#if MOE_PRE_MX8
hipError_t launch_quant_mx8(const uint16_t* src, int rows, int K, int stride, uint8_t* dst,
                            uint16_t* scales, hipStream_t s);
#endif
// Largest K split of a shared-expert GEMM and the cap on its partial sums.
constexpr int kMaxKsplit = 16;
constexpr size_t kSplitPartMax = (size_t)32 << 20;
hipError_t launch_decode_gate_up(const ExpertGemmArgs& a, hipStream_t s);
// One token, top-K selection: the selection and the dispatch run inside the gate+up kernel.
struct FusedRoute {
  int32_t* row_token;
  int32_t* inv;
  Tile* tiles;
  int32_t* ntiles;
  int32_t* err_word;
  int shared_rows;
};
bool decode_topk_fusable(int fmt, int H, int E);
hipError_t launch_decode_gate_up_topk(const ExpertGemmArgs& a, const TopkArgs& ta,
                                      const FusedRoute& fr, hipStream_t s);
hipError_t launch_decode_down(const ExpertGemmArgs& a, hipStream_t s);
hipError_t launch_prefill_gate_up(const ExpertGemmArgs& a, int mt, hipStream_t s);
hipError_t launch_prefill_down(const ExpertGemmArgs& a, int mt, hipStream_t s);

struct CombineArgs {
  const float* y;         // [R, H] fp32 (with y16: the shared expert's rows [0, T) only)
  const uint16_t* y16;    // routed rows as fp16 (row r at y16 + r * H), or nullptr
  const float* w;         // [T, K]
  const int32_t* inv;     // [T, K] row of slot (t, j), -1 (dropped) or -2 (zero expert)
  const uint16_t* xe;     // [T, H] expert input (the identity of a zero expert)
  int shared;             // shared rows are [0, T)
  const uint16_t* residual;
  uint16_t* out;
  int T, K, H;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// One token without a shared expert on the one-step down GEMV: down and blend in one launch.
bool decode_blend_fusable(const ExpertGemmArgs& a, const CombineArgs& cb);
hipError_t launch_decode_down_blend(const ExpertGemmArgs& a, const CombineArgs& cb,
                                    hipStream_t s);

hipError_t launch_debug_dequant(const WeightDesc& w, int expert, int path, float* out,
                                hipStream_t s);

}  // namespace moe

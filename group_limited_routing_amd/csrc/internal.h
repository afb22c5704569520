// Internal launchers and workspace layout of the Beam MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace beam {

// Row tile (tokens per M-tile) of the two expert-GEMM variants.
constexpr int kStreamBM = 16;   // decode: weight streaming, one MFMA row block (or two: stream_bm)
constexpr int kTiledBM = 128;   // prefill, row-major weights: LDS-staged MFMA tiles
// M-tile list of the mixed-height DMA GEMMs: 256-row slots, and 512-row tiles
// (two slots each) for experts with more than 256 rows.
constexpr int kMixedBM = 512;

struct Shape {
  int T, H, I, E, n_group, topk_group, top_k;
  float rsf;
  int x_f32;   // 1: x/out fp32, 0: bf16
  int w_fp8;   // 1: fp8 e4m3 weights with per-row scales
  int w_packed;  // 1: weights in the MFMA fragment layout
  int w_mx4;     // 1: MXFP4 weights (w_fp8 is set too: E4M3 activations)
  int n_run;     // experts whose GEMMs run (E, or an expert shard's count)
};

// Byte offsets of each workspace region (all 256-byte aligned).
struct Layout {
  size_t z, idx, w, chist, cbase, counts, offsets, meta, tile_e, tile_r, e_tstart, e_ntiles;
  size_t stok, sw, inv, xq, xs, hamax, h, hq, hs, y, total;
  size_t wsplit, zpart;  // split router weights (bf16 tokens, many), partial logits
  int nchunks, max_mtiles;
  int router_ks;         // K ranges of the partial logits (0: logits straight into z)
  int router_x3;         // 1: partials from the split-weight bf16 kernel, 0: fp32 kernel
};

// Up to this many tokens the router runs the fp32 kernel with its reduction
// split over workgroups (partial logits summed by the selection).
constexpr int kRouterSplitMaxT = 256;

Layout make_layout(const Shape& s);
bool use_stream_gemm(const Shape& s);
// M-tile height of the streaming variants: kStreamBM, or 2 kStreamBM above 8
// rows per expert on average
int stream_bm(const Shape& s);
// prefill with packed weights: M-tile of 128 or 256 rows, from the rows per expert
int wide_bm(const Shape& s);
// Row height of the forward's M-tile list (shared by the gate/up and down
// passes): kStreamBM or 2 kStreamBM, kTiledBM, 128, 256, or kMixedBM (256-row slots, 512-row
// tiles for experts with more than 256 rows).
int forward_list_bm(const Shape& s);
int mtile_bound(const Shape& s, int BM);

hipError_t launch_router_logits(const void* x, int x_f32, const float* W, float* z, int T, int H,
                                hipStream_t st);
// Few tokens: partial logits zp[kz, t, e] over nz = router_small_split(H)
// ranges of the hidden dimension, from the fp32 kernel.
int router_small_split(int H);
hipError_t launch_router_logits_split(const void* x, int x_f32, const float* W, float* zp, int T,
                                      int H, int nz, hipStream_t st);
// bf16 tokens: router weights split into three bf16 parts, partial logits
// over router_ksplit(T, H) ranges of the hidden dimension.
int router_ksplit(int T, int H);
hipError_t launch_router_x3(const uint16_t* x, const float* W, uint16_t* wsplit, float* zp, int T,
                            int H, int ks, hipStream_t st);
// s_sel (nullable): [T, top_k] sigmoid scores of the chosen experts
hipError_t launch_select(const float* z, int nparts, size_t pstride, float* zout, const float* bias,
                         int T, int n_group, int topk_group, int top_k, int32_t* idx, float* w,
                         float* s_sel, hipStream_t st);
hipError_t launch_perm_hist(const int32_t* idx, int T, int k, int32_t* chist, hipStream_t st);
// Tiles only for experts in [e0, e1) (all experts by default).
hipError_t launch_perm_scan(const int32_t* chist, int nchunks, int BM, int32_t* cbase,
                            int32_t* counts, int32_t* offsets, int32_t* meta, int32_t* tile_e,
                            int32_t* tile_r, int32_t* e_tstart, int32_t* e_ntiles,
                            int32_t* counts_out, hipStream_t st, int e0 = 0, int e1 = kExperts);
hipError_t launch_perm_scatter(const int32_t* idx, const float* w, int T, int k, float rsf,
                               const int32_t* cbase, const int32_t* offsets, int32_t* stok,
                               float* sw, int32_t* inv, hipStream_t st);
// One chunk (T <= 256): hist, scan and scatter in one launch, same results.
hipError_t launch_perm_single(const int32_t* idx, const float* w, int T, int k, float rsf, int BM,
                              int32_t* counts, int32_t* offsets, int32_t* meta, int32_t* tile_e,
                              int32_t* tile_r, int32_t* e_tstart, int32_t* e_ntiles,
                              int32_t* counts_out, int32_t* stok, float* sw, int32_t* inv,
                              hipStream_t st, int e0 = 0, int e1 = kExperts);

struct GemmArgs {
  const void* a;            // gate/up: x [T, H]; down: h_perm [T*k, I]
  const void* w0;           // gate/up: w_gate; down: w_down
  const void* w1;           // gate/up: w_up; down: unused
  const float* ws0;         // fp8 per-row weight scales matching w0 (or null)
  const float* ws1;         // fp8 per-row weight scales matching w1 (or null)
  const float* a_scale;     // fp8: per-row activation scales (x: [T], h: [T*k])
  const int32_t* tile_e;
  const int32_t* tile_r;
  const int32_t* e_tstart;  // first M-tile of each expert
  const int32_t* e_ntiles;  // M-tiles of each expert
  const int32_t* meta;
  const int32_t* offsets;
  const int32_t* stok;
  const float* sw;          // rsf * routing weight per sorted row
  void* out;                // gate/up: h_perm; down: y_perm
  uint32_t* hamax;          // fp8 gate/up: per-row running max |h| (float bits)
  int K, N;                 // reduction length and output width
  int max_mtiles;
  // backward pass only
  const void* a2;           // g | u rows of the recomputed gate/up pass
  void* tout0;              // transposed outputs [N, pcols] in 32-column blocks (null: none)
  void* tout1;
  const int32_t* pcol;      // first column of each expert's segment in them
  float* part;              // per-row partial sums of h . q, nparts per row
  int nparts;
};

hipError_t launch_gateup(const Shape& s, const GemmArgs& g, hipStream_t st);
// Backward-pass GEMMs (bf16 tokens, packed bf16 weights; modes 2-4 of the DMA
// variant) with M-tiles of BM rows; the grid covers mtile_bound(s, BM) tiles.
hipError_t launch_backward_gemm(int mode, const Shape& s, int BM, const GemmArgs& g,
                                hipStream_t st);
hipError_t launch_down(const Shape& s, const GemmArgs& g, hipStream_t st);
hipError_t launch_pack(const void* src, void* dst, int E, int rows, int cols, int fp8,
                       hipStream_t st);
// rows of row_bytes bytes, SB bytes per row per matrix-core step
hipError_t launch_pack_bytes(const void* src, void* dst, int E, int rows, int row_bytes, int SB,
                             hipStream_t st);
hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int E, int rows, int cols,
                                 hipStream_t st);
hipError_t launch_combine(const void* y, const int32_t* inv, int T, int k, int H, int out_f32,
                          void* out, hipStream_t st);
// an expert shard's share of the output (slots with experts in [e0, e1))
hipError_t launch_combine_shard(const void* y, const int32_t* inv, const int32_t* idx, int T,
                                int k, int H, int e0, int e1, int out_f32, void* out,
                                hipStream_t st);
// Largest hidden size of the fused combine + residual step (a token's row is
// held in the registers of one workgroup).
constexpr int kResidualMaxH = 16384;
hipError_t launch_combine_residual(const void* y, const int32_t* inv, int T, int k, int H,
                                   int x_f32, const void* stream_in, const float* gain, float eps,
                                   float keep, float add, void* stream_out, hipStream_t st);
// backward pass (backward.hip)
hipError_t launch_segment_cols(const int32_t* counts, int32_t* pcol, hipStream_t st);
// Transposed copies [R, pcols] are stored in 32-column blocks: element (n, c)
// at ((c / 32) R + n) 32 + c % 32.
hipError_t launch_gather_t(const uint16_t* src, int H, bool scaled, const int32_t* stok,
                           const float* sw, const int32_t* offsets, const int32_t* pcol,
                           uint16_t* out, int max_blocks, hipStream_t st);
hipError_t launch_zero_pads(uint16_t* a, uint16_t* b, uint16_t* c, int N, const int32_t* offsets,
                            const int32_t* pcol, hipStream_t st);
hipError_t launch_token_grad(const uint16_t* dxr, const int32_t* inv, const int32_t* idx,
                             const float* w, const float* s_sel, const float* part, int nparts,
                             float rsf, const float* router_w, int T, int k, int H,
                             float* dz_sorted, uint16_t* dx, hipStream_t st);
hipError_t launch_router_grad(const uint16_t* x, int H, const int32_t* stok,
                              const int32_t* offsets, const float* dz, float* drw, hipStream_t st);
hipError_t launch_wgrad(const uint16_t* A, const uint16_t* B, int M, int N, const int32_t* pcol,
                        uint16_t* C, hipStream_t st);
hipError_t launch_pack_t(const void* src, void* dst, int E, int rows, int cols, hipStream_t st);
hipError_t launch_bias_step(float* bias, const int32_t* counts, float gamma, hipStream_t st);
hipError_t launch_quant_x(const void* x, int x_f32, int T, int H, int k, uint8_t* xq, float* xs,
                          uint32_t* hamax, hipStream_t st);
hipError_t launch_quant_h(const uint16_t* hb, const uint32_t* hamax, int rows, int I, uint8_t* hq,
                          float* hs, hipStream_t st);

}  // namespace beam

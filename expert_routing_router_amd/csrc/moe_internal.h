// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/moe_rocm.h"

namespace moe {

// ---------------------------------------------------------------- router
enum RouterFront { kFrontScoresIn = 0, kFrontPartials = 1, kFrontF64 = 3 };
struct RouteArgs {
  const void* u; const void* E; const float* b; const float* scores_in;
  float* scores_out; int32_t* idx; float* gate;
  int32_t* counts;   // nullable: per-expert loads, counted after the selection by a separate kernel
  int T, d, n_routed, top_k, n_groups, topk_groups, group_topk, group_score_biased;
  int in_dtype, router_dtype;
  const float* partials = nullptr;   // kFrontPartials: [n_slices][T][n_routed] fp32 slice sums of the logits
  int n_slices = 0;
};
hipError_t launch_route(const RouteArgs& a, int front, hipStream_t s);
// The router every entry point uses: the selection alone when scores_in is
// set, else the split-K router (bf16 u and centroids, 256 experts), the tiled
// two-phase router (N_r % 64 == 0), or the fp64 front end, by shape. Needs
// router_scratch_bytes of device scratch (0 for the fp64 front end).
size_t router_scratch_bytes(const RouteArgs& a);
hipError_t run_router(const RouteArgs& a, void* scratch, hipStream_t s);
bool route_splitk_ok(const RouteArgs& a);
size_t route_splitk_bytes(int T, int d);
hipError_t launch_route_splitk(const RouteArgs& a, void* scratch, hipStream_t s);
bool route_two_phase_ok(const RouteArgs& a);
size_t route_two_phase_bytes(int T, int N, int d, int router_dtype);
hipError_t launch_route_two_phase(const RouteArgs& a, void* scratch, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, long n, hipStream_t s);
// counts[e] = number of the n entries of idx equal to e (zeroed first)
hipError_t launch_count_loads(const int32_t* idx, long n, int N, int32_t* counts, hipStream_t s);

// ---------------------------------------------------------------- permute
// Workspace pieces: bitmap [N_r][W] u64 (W = ceil(T/64)), wprefix [N_r][W] i32.
struct PermuteArgs {
  const int32_t* idx; int T, K, n_routed;
  uint64_t* bitmap; int32_t* wprefix; int32_t* counts_ws;   // counts_ws [N_r] scratch
  int32_t* offsets;       // [n_seg+1], n_seg = n_routed + n_extra_seg
  int32_t* row_token;     // [T*K + n_extra_seg*T]
  int32_t* slot_row;      // [T*K]
  int32_t* counts_out;    // nullable [N_r]
  int n_extra_seg;        // shared-expert segments appended after the routed rows (identity rows)
  int32_t* mtile_prefix;  // nullable [n_seg+1]: prefix of ceil(n_e/bm)
  int bm;
  const int32_t* keep = nullptr;   // nullable [T*K]: 0 = dropped selection (slot_row -1, no row)
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// diagnostics: streaming read of `bytes` (multiple of 16); kCalMfmaWaves waves of iters x 8 bf16 MFMAs
constexpr int kCalMfmaWaves = 8192;
hipError_t launch_cal_read(const void* buf, size_t bytes, int32_t* sink, hipStream_t s);
hipError_t launch_cal_mfma(int iters, float* sink, hipStream_t s);
// capacity limit: keep [T*K] (1 kept, 0 dropped) from the no-drop layout; dropped: total count
hipError_t launch_capacity(const int32_t* offsets, const int32_t* row_token, const int32_t* idx,
                           const float* scores, int T, int N, int K, int cap, int32_t* keep, int32_t* dropped,
                           hipStream_t s);
hipError_t launch_gather_rows(const void* src, long src_rows, const int32_t* row_token, const int32_t* n_valid,
                              void* dst, long rows, int row_bytes, hipStream_t s);
hipError_t launch_mtile_prefix(const int32_t* offsets, int n_seg, int bm, int32_t* out,
                               hipStream_t s);

// ---------------------------------------------------------------- grouped GEMMs
// Segment e uses weights (e < n_first ? w0 + e*stride0 : w1 + (e-n_first)*stride1).
struct GemmArgs {
  const void* x;              // A source rows (through row_index when not null)
  long x_rows;                // rows of x (for the buffer-load range check)
  const float* x_scale;       // FP8: [.., K/128] per source row
  const int32_t* row_index;   // nullable
  const int32_t* offsets;     // [n_seg+1]
  const int32_t* mtile_prefix;// [n_seg+1]
  int n_seg;
  const void* w0; const void* w1; long wstride0, wstride1;       // elements
  const float* ws0; const float* ws1; long sstride0, sstride1;   // FP8 block scales
  int n_first;
  void* out;                  // [rows, N]
  int N;                      // output columns (I for the SwiGLU GEMM, d for down)
  int K;                      // reduction length
  int rows_bound;             // upper bound on total rows (grid sizing)
  // K-blocked operands (bf16 LDS-DMA kernel only): a tile's rows are stored per 32-element
  // step as [step][tile rows][64 B] with the kernel's LDS chunk swizzle applied, so each
  // 1 KB load instruction reads one contiguous kilobyte.
  int w_blocked = 0;          // w0/w1: moe_pack_expert_weights layout
  int x_blocked = 0;          // x: per m-tile (mtile_prefix numbering) blocks of BM rows, K = this GEMM's K
  int out_blocked = 0;        // SwiGLU output H written in the x_blocked layout of the down GEMM
  // FP8 SwiGLU GEMM: when out_q is set, H goes out as E4M3 codes out_q [rows][N] with 1x128
  // scales out_qs [rows][N/128], quantised exactly as launch_quant_act does from fp32 H
  uint8_t* out_q = nullptr;
  float* out_qs = nullptr;
};
// bf16 weights [n_mat][rows][K] -> K-blocked tiles of 256 rows; swiglu_i > 0: rows = 2*swiglu_i and
// tile t holds gate rows t*128.. and up rows swiglu_i + t*128..
hipError_t launch_pack_blocked(const uint16_t* src, uint16_t* dst, int n_mat, int rows, int K, int swiglu_i,
                               hipStream_t s);
// FP8 codes: tiles of 256 rows, 128-element blocks (the FP8 LDS-DMA kernel's stage)
hipError_t launch_pack_blocked_f8(const uint8_t* src, uint8_t* dst, int n_mat, int rows, int K, int swiglu_i,
                                  hipStream_t s);
int gemm_bm(int dtype, int mean_rows, int dmodel, int inter);
hipError_t launch_gemm_swiglu(const GemmArgs& a, int dtype, int bm, hipStream_t s);
hipError_t launch_gemm_down(const GemmArgs& a, int dtype, int bm, hipStream_t s);

// ---------------------------------------------------------------- combine / bias / quant
struct CombineArgs {
  const void* u; const void* y; const void* y_shared; const int32_t* slot_row;
  const float* gate; void* out; int T, d, K, n_shared; long shared_stride;  // rows
  int io_dtype;   // MOE_F32 or MOE_BF16 (u/out)
  int y_dtype;    // MOE_F32 or MOE_BF16
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_update_bias(const int32_t* counts, float* b, int n_routed, long total,
                              float gamma, hipStream_t s);

// ---------------------------------------------------------------- backward
struct WgradArgs {
  const uint16_t* P;          // [R, M] bf16 permuted rows
  const uint16_t* Q;          // rows [*, Nn] bf16
  const int32_t* q_row;       // nullable: Q row of permuted row r
  long q_rows;                // rows of Q (range of the buffer loads)
  const int32_t* offsets;     // [n_seg+1]
  int n_seg, M, Nn;           // M, Nn multiples of 128
  float* out0; float* out1; long ostride0, ostride1;   // [M, Nn] per segment
  int n_first;                // segments below: out0, others: out1
  // nullable scratch for the transposed-operand path (M, Nn multiples of 256): pt [M][pitch],
  // qt [Nn][pitch] bf16, kofs [n_seg+1]; pitch = wgrad_pitch(rows of P, n_seg)
  uint16_t* pt = nullptr; uint16_t* qt = nullptr; int32_t* kofs = nullptr; long pitch = 0;
};
long wgrad_pitch(long rows, int n_seg, int pad = 64);
hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s);
// FP8 weight gradients (E4M3 operands in 128-row tiles along each segment's rows): needs the
// WgradArgs' pt/qt/kofs with pitch = wgrad_pitch(rows, n_seg, 128) and these E4M3 copies and
// transposed scales: pt8 [M][pitch], qt8 [Nn][pitch], spt [pitch/128][M], sqt [pitch/128][Nn]
struct WgradF8Scratch { uint8_t* pt8; uint8_t* qt8; float* spt; float* sqt; };
hipError_t launch_wgrad_f8(const WgradArgs& a, const WgradF8Scratch& f, hipStream_t s);
// fp32 layers: P, Q fp32 (the args' P/Q/pt/qt are ignored)
hipError_t launch_wgrad_f32(const WgradArgs& a, const float* P, const float* Q, hipStream_t s);
// element-wise backward pieces; dtype MOE_BF16 or MOE_F32 for the activations they read and write
hipError_t launch_swiglu_fwd(const void* ab, void* h, long rows, int I, int dtype, hipStream_t s);
hipError_t launch_swiglu_bwd(const void* dh, const void* ab, void* dab, long rows, int I, int dtype, hipStream_t s);
hipError_t launch_dgate_dy(const void* dout, const void* y, const int32_t* slot_row, const float* gate, int T, int d,
                           int K, int n_shared, long shared_base, long shared_stride, float* dg, void* dy, int dtype,
                           hipStream_t s);
hipError_t launch_router_bwd(const float* scores, const int32_t* idx, const float* dg, const void* dout,
                             const void* dx, const int32_t* slot_row, const void* E, int e_dtype, const void* u,
                             const int32_t* offsets, const int32_t* row_token, int T, int N, int d, int K,
                             int n_shared, long shared_base, long shared_stride, float* dz, float* du, float* dE,
                             int dtype, hipStream_t s);
hipError_t launch_transpose(const void* src, void* dst, int batch, int rows, int cols, int dtype, hipStream_t s);

// sequence-wise balance loss (forward value)
size_t seq_balance_ws_bytes(int T, int N, int seq_len);
hipError_t launch_seq_balance(const float* s, const int32_t* idx, int T, int N, int K, int seq_len, float alpha,
                              float* f, float* P, float* loss, void* ws, hipStream_t st);
hipError_t launch_quant_act(const void* src, int src_dtype, long rows, int cols,
                            const int32_t* row_index, uint8_t* q, float* scale, hipStream_t s);
// bf16 rows [rows][cols] in 1x128 tiles, scales stored transposed: scale_t [cols/128][rows]
hipError_t launch_quant_act_tscale(const uint16_t* src, long rows, int cols, uint8_t* q, float* scale_t,
                                   hipStream_t s);
hipError_t launch_quant_w(const void* src, int src_dtype, long rows, int cols, uint8_t* q,
                          float* scale, hipStream_t s);

}  // namespace moe

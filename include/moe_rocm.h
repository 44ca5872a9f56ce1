/*
 * moe_rocm.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer with
 * auxiliary-loss-free load balancing.
 *
 * What the layer computes (DeepSeek-V3 Technical Report; the xyznot.com
 * reading guides, "Metodo"/"al-tariqa" section 2, and the pwwt.cn study note):
 *   s_{i,t} = sigmoid(u_t . e_i)                               (affinity)
 *   g'_{i,t} = s_{i,t} if s_{i,t}+b_i is among the top K_r of
 *              {s_{j,t}+b_j}, else 0                            (gating equation)
 *   g_{i,t}  = g'_{i,t} / sum_j g'_{j,t}                        (normalised gate)
 *   h'_t     = u_t + sum_s FFN^(s)(u_t) + sum_i g_{i,t} FFN^(r)_i(u_t)
 *   b_i     <- b_i - gamma if expert i is overloaded, + gamma if underloaded
 * with top-K_r restricted to the M expert groups whose top K_r/M scores sum
 * highest (pwwt.cn note section 1.3) and no token dropped (note section 1.4).
 *
 * Conventions
 *   - Every tensor argument is a DEVICE pointer owned by the caller, 16-byte
 *     aligned, row-major and dense. The library never allocates, frees or
 *     synchronises; scratch memory comes from the caller's workspace.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *     Results are valid once the stream has reached the end of the call.
 *   - Each call validates every argument before enqueueing anything: a call
 *     that returns an error has enqueued nothing (MOE_EHIP aside, which
 *     reports a failed launch; moe_last_hip_error() gives the HIP code).
 *   - The library holds no state between calls; calls on different streams
 *     are independent provided they use different workspaces and outputs.
 *   - Ties are broken deterministically and every result is reproducible
 *     bit-for-bit from run to run (integer atomics only; fixed-order sums).
 */
#ifndef MOE_ROCM_H
#define MOE_ROCM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

/* status codes */
#define MOE_OK          0
#define MOE_EINVAL     -1  /* bad dimension, NULL required pointer, misaligned pointer */
#define MOE_ENOTSUP    -2  /* dtype / shape combination the library does not implement */
#define MOE_EWORKSPACE -3  /* workspace smaller than the call needs */
#define MOE_EHIP       -4  /* a HIP launch or runtime call failed */

/* element types */
#define MOE_F32       0
#define MOE_BF16      1
#define MOE_FP8_E4M3  2    /* OCP E4M3FN: bias 7, max 448, no infinities */

/* moe_quantize_fp8 kinds */
#define MOE_QUANT_ACT_1x128   0   /* one fp32 scale per row per 128 columns */
#define MOE_QUANT_W_128x128   1   /* one fp32 scale per 128x128 block */

typedef void* moe_stream_t;      /* hipStream_t */

/* Layer description. Groups are contiguous blocks of n_routed/n_groups
 * experts (the pages' nodes); n_groups = topk_groups = 1 disables the limit. */
typedef struct moe_desc {
  int32_t abi_version;        /* MOE_ABI_VERSION */
  int32_t T;                  /* tokens in the batch */
  int32_t d;                  /* hidden size */
  int32_t n_routed;           /* N_r, 1..256 */
  int32_t top_k;              /* K_r, 1..min(N_r, 32) */
  int32_t n_groups;           /* G, divides N_r, <= 64 */
  int32_t topk_groups;        /* M, 1..G */
  int32_t group_topk;         /* q: scores summed per group (K_r/M on the pages), 1..N_r/G */
  int32_t n_shared;           /* N_s >= 0 */
  int32_t inter;              /* I, routed expert intermediate size */
  int32_t inter_shared;       /* I_s, shared expert intermediate size */
  int32_t in_dtype;           /* u and out: MOE_F32 | MOE_BF16 */
  int32_t router_dtype;       /* centroids: MOE_F32 | MOE_BF16 */
  int32_t expert_dtype;       /* expert weights: MOE_F32 | MOE_BF16 | MOE_FP8_E4M3 */
  int32_t group_score_biased; /* 1: group scores from s+b (default); 0: from s */
  float   gamma;              /* bias update speed, 0.001 on the pages */
} moe_desc_t;

/* Weights for moe_forward. Layouts:
 *   centroids   [N_r, d]        router_dtype
 *   w13         [N_r, 2I, d]    rows 0..I-1: W1 (gate, goes through SiLU); I..2I-1: W3 (up)
 *   w2          [N_r, d, I]
 *   w13_shared  [N_s, 2I_s, d], w2_shared [N_s, d, I_s]
 *   FP8 only: E4M3 codes in w13/w2/..., and fp32 block scales
 *   w13_scale [N_r, 2I/128, d/128], w2_scale [N_r, d/128, I/128] (same for shared). */
typedef struct moe_weights {
  const void*  centroids;
  const void*  w13;
  const void*  w2;
  const void*  w13_shared;
  const void*  w2_shared;
  const float* w13_scale;
  const float* w2_scale;
  const float* w13_shared_scale;
  const float* w2_shared_scale;
  /* Optional K-blocked copies of w13, w2, w13_shared, w2_shared made by
   * moe_pack_expert_weights (bf16 or FP8 codes). When the routed ones (and,
   * with N_s > 0, the shared ones) are all set, moe_forward and
   * moe_forward_capacity read them instead of the row-major arrays (bf16:
   * and keep their intermediate H K-blocked too); the results are
   * bit-identical. NULL: the row-major arrays are used. */
  const void*  w13_blk;
  const void*  w2_blk;
  const void*  w13_shared_blk;
  const void*  w2_shared_blk;
} moe_weights_t;

/* Optional routing outputs of moe_forward (any member may be NULL). */
typedef struct moe_route_out {
  int32_t* topk_idx;   /* [T, K] */
  float*   topk_gate;  /* [T, K] */
  int32_t* counts;     /* [N_r] */
} moe_route_out_t;

int         moe_abi_version(void);
const char* moe_strerror(int status);
int         moe_last_hip_error(void);

/* Checks a descriptor alone (dims, dtypes, group rule). MOE_OK or MOE_EINVAL/ENOTSUP. */
int moe_validate(const moe_desc_t* desc);

/* Workspace bytes moe_forward needs for this descriptor (0 on invalid desc). */
size_t moe_workspace_bytes(const moe_desc_t* desc);

/* Router: affinities, biased group-limited top-K, normalised gates, loads.
 * (xyznot.com guides section 2, gating equation; pwwt.cn note 1.1.2, 1.3.)
 *   u [T,d] in_dtype and E [N_r,d] router_dtype; or scores_in [T,N_r] fp32
 *   (exactly one of the two sources). With scores_in the affinities are taken
 *   as given and the selection runs on the same code path.
 *   b [N_r] fp32 (read only).
 *   scores_out [T,N_r] fp32, nullable: the fp32 affinities used.
 *   topk_idx [T,K] int32: selected experts in rank order (key desc, index asc).
 *   topk_gate [T,K] fp32: s / sum(s) over the selected experts (unbiased s;
 *     1/K if the sum is 0).
 *   counts [N_r] int32: overwritten with the number of tokens per expert.
 *   ws: scratch of moe_route_workspace_bytes(desc) bytes (the router's
 *     partial logits); nullable when that is 0 or with
 *     scores_in. MOE_EWORKSPACE when it is missing or smaller.
 * moe_forward and moe_backward route with the same kernels, so their
 * selections equal this call's bit for bit. */
size_t moe_route_workspace_bytes(const moe_desc_t* desc);
int moe_route(const moe_desc_t* desc, const void* u, const void* E, const float* b,
              const float* scores_in, float* scores_out, int32_t* topk_idx,
              float* topk_gate, int32_t* counts, void* ws, size_t ws_bytes,
              moe_stream_t stream);

/* Dispatch layout (single-GPU analog of the pwwt.cn note's section 4
 * dispatch; no capacity, note 1.4).
 *   offsets [N_r+1]: rows of expert e are [offsets[e], offsets[e+1]).
 *   row_token [T*K]: token of each permuted row, ascending within an expert.
 *   slot_row [T*K]: permuted row of (t, topk_idx[t,k]) at index t*K+k.
 *   counts [N_r], nullable: loads recomputed from topk_idx.
 *   u [T,d] and x_perm [T*K,d] (in_dtype), nullable together: gathered rows.
 *   ws: at least moe_workspace_bytes(desc) bytes.
 * An expert id outside [0, N_r) in topk_idx gets no row: its slot_row is -1,
 * it is not counted, and the rows it would have had are not written. */
int moe_permute(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* offsets,
                int32_t* row_token, int32_t* slot_row, int32_t* counts,
                const void* u, void* x_perm, void* ws, size_t ws_bytes,
                moe_stream_t stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results as moe_permute without the workspace. Its
 * bitmap and word-prefix scratch, 12 * ceil(T/64) * N_r bytes (plus
 * alignment), lives in a device array of MOE_NOALLOC_SCRATCH_BYTES held by
 * the library on each GPU it runs on until the process ends; the call neither
 * allocates nor frees anything. MOE_EWORKSPACE when the scratch would not fit
 * (T above about 174k tokens at N_r = 256). Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (on different streams, or from
 * different host threads before the first finishes) race, and must be
 * serialised by the caller. Nothing in the scratch needs to start at zero. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_permute_noalloc(const moe_desc_t* desc, const int32_t* topk_idx, int32_t* offsets,
                        int32_t* row_token, int32_t* slot_row, int32_t* counts,
                        const void* u, void* x_perm, moe_stream_t stream);

/* Grouped SwiGLU experts over `rows` permuted rows in n_experts segments:
 *   y[r] = W2_e (SiLU(W1_e x_r) * (W3_e x_r)) for offsets[e] <= r < offsets[e+1].
 * (xyznot.com guides section 2, output equation; the SwiGLU form is a
 *  reading, the pages do not state the FFN's inner form.)
 *   x: [T,d] read through row_token (x_r = x[row_token[r]]) or, with
 *      row_token NULL, [rows,d] read directly. Type: in_dtype for F32/BF16
 *      experts; E4M3 codes for FP8 experts, with x_scale [.., d/128] fp32.
 *   w13 [n_experts, 2*inter, d], w2 [n_experts, d, inter] expert_dtype; FP8
 *      scales w13_scale/w2_scale as in moe_weights_t.
 *   y [rows, d]: fp32 for F32 experts, bf16 otherwise.
 *   ws: at least moe_expert_ffn_workspace_bytes(...) bytes.
 * offsets must be non-decreasing with offsets[0] >= 0 and offsets[n_experts]
 * <= rows (the kernels keep every row index they form inside [0, rows)). */
size_t moe_expert_ffn_workspace_bytes(const moe_desc_t* desc, int32_t n_experts,
                                      int32_t inter, int32_t rows);
int moe_expert_ffn(const moe_desc_t* desc, int32_t n_experts, int32_t inter, int32_t rows,
                   const void* x, const float* x_scale, const int32_t* row_token,
                   const int32_t* offsets, const void* w13, const float* w13_scale,
                   const void* w2, const float* w2_scale, void* y, void* ws,
                   size_t ws_bytes, moe_stream_t stream);

/* Combine: out_t = u_t + sum_s y_shared[s,t] + sum_k gate[t,k] * y[slot_row[t*K+k]]
 * accumulated in fp32 in that fixed order (output equation; the pwwt.cn
 * note's section 4 combine).  u, out [T,d] in_dtype; y [T*K,d] and
 * y_shared [N_s,T,d] (nullable when N_s = 0) fp32 for F32 experts, bf16 otherwise.
 * A slot_row entry outside [0, T*K) (-1 for a dropped selection) adds nothing. */
int moe_combine(const moe_desc_t* desc, const void* u, const void* y, const void* y_shared,
                const int32_t* slot_row, const float* topk_gate, void* out,
                moe_stream_t stream);

/* End-of-step bias update (pwwt.cn note 1.1.3; guides section 2):
 *   b_i <- fl32(b_i - gamma) if N_r*c_i > T*K (overloaded),
 *          fl32(b_i + gamma) if N_r*c_i < T*K (underloaded), unchanged otherwise. */
int moe_update_bias(const moe_desc_t* desc, const int32_t* counts, float* b,
                    moe_stream_t stream);

/* Gradients of the layer (moe_backward). fp32, caller-owned, row-major:
 *   du [T, d]; dE [N_r, d]; dw13 [N_r, 2I, d]; dw2 [N_r, d, I];
 *   dw13_shared [N_s, 2I, d], dw2_shared [N_s, d, I] (unused when N_s = 0). */
typedef struct moe_grads {
  float* du;
  float* dE;
  float* dw13;
  float* dw2;
  float* dw13_shared;
  float* dw2_shared;
} moe_grads_t;

/* Transposed expert weights for moe_backward: fills wt->w13 [N_r, d, 2I] and
 * wt->w2 [N_r, I, d] (and the shared ones) from the weights in w, in the
 * experts' dtype (bf16, fp32 or E4M3 codes). FP8 layers: also the block
 * scales, transposed: wt->w13_scale [N_r, d/128, 2I/128], wt->w2_scale
 * [N_r, I/128, d/128] (and the shared ones), so wt holds exactly the values
 * of the transposed E4M3 matrices. Other members of wt are ignored. */
int moe_transpose_expert_weights(const moe_desc_t* desc, const moe_weights_t* w, moe_weights_t* wt,
                                 moe_stream_t stream);

/* K-blocked copies of the expert weights, the layout the grouped GEMMs' LDS
 * rings consume: for each matrix, tiles of 256 rows (SwiGLU w13: W1 rows
 * 128t..128t+127 then W3 rows I+128t..), then steps of the reduction, then
 * the tile's 256 rows of one step each. Steps are 64 bytes of a row: 32
 * bf16 elements or 64 FP8 codes, a row's four 16-byte chunks c stored at
 * slot c ^ ((row >> 2) & 3); FP8 block scales keep their layout. A tile's
 * step is then one contiguous block, so every 1 KB load instruction of the
 * kernels reads one contiguous kilobyte instead of pieces of 16 different
 * rows (a layout choice for gfx950's load path; the products are
 * unchanged). Fills wb->w13, wb->w2 (and wb->w13_shared, wb->w2_shared when
 * N_s > 0), each the size of its source, from w; other members of wb are
 * ignored; the caller then passes them as w13_blk ... in moe_weights_t.
 * bf16 or FP8 experts with I % 128 == 0, I_s % 128 == 0 and d % 256 == 0;
 * MOE_ENOTSUP otherwise. */
int moe_pack_expert_weights(const moe_desc_t* desc, const moe_weights_t* w, moe_weights_t* wb,
                            moe_stream_t stream);

/* Backward of moe_forward for the routing it chooses (same u, b, weights):
 * given dout = dL/dout [T, d] (in_dtype), writes dL/du, dL/dE and the expert
 * weight gradients. The selection and the bias are piecewise constant (b only
 * routes: pwwt.cn note 1.1.2-1.1.3), so gradients flow through the gates'
 * dependence on the affinities, g = s_sel / sum(s_sel), and the SwiGLU
 * experts (output equation of the xyznot.com guides, section 2):
 *   dg = <dout, Y>, dY = g dout, dH = dY W2, dA|dB from SwiGLU, dX = [dA dB] W13,
 *   ds = (dg - sum g dg) / sum s, dz = ds s (1 - s), dE = dz^T u.
 * The forward is recomputed inside (intermediates in the experts' dtype,
 * bf16 for FP8 layers; fp32 accumulation). Supported: bf16 u and experts
 * with I % 128 == 0; fp32 u and experts with I % 8 == 0; bf16 u and FP8
 * experts with d % 256 == 0 and I % 256 == 0 (and the padded weight-gradient
 * operands under 2^31 bytes); N_s == 0 or I_s == I; MOE_ENOTSUP otherwise.
 * FP8 layers run Fprop, Dgrad and Wgrad as E4M3 GEMMs (pwwt.cn note section
 * 3): each activation operand quantised per 1x128 tile along the product's
 * reduction dimension (for Wgrad: 128-row tiles starting at each expert's
 * first row), the layer's 128x128-block weights; gradients with respect to
 * the E4M3 weight values. wt: moe_transpose_expert_weights of w.
 * ws: moe_backward_workspace_bytes(desc) bytes (0 when unsupported). */
size_t moe_backward_workspace_bytes(const moe_desc_t* desc);
int moe_backward(const moe_desc_t* desc, const moe_weights_t* w, const moe_weights_t* wt, const void* u,
                 const float* b, const void* dout, moe_grads_t* grads, void* ws, size_t ws_bytes,
                 moe_stream_t stream);

/* Complementary sequence-wise balance loss, forward value (pwwt.cn note
 * section 1.2; alpha = 0.0001 on the xyznot.com guides, section 2). The T
 * tokens are T/seq_len consecutive sequences; for sequence q
 *   f_i = #{(t,k) in q : topk_idx[t,k] = i} / (K * seq_len)
 *   P_i = mean over t in q of scores[t,i] / sum_j scores[t,j]
 *         (1/N_r for a token whose affinities sum to 0)
 *   loss[q] = alpha * sum_i f_i * P_i
 * (the page's formula is missing; these normalisations are the reading taken).
 *   scores [T, N_r] fp32: the router's affinities (moe_route's scores_out);
 *   topk_idx [T, K] int32: its selections. f, P [T/seq_len, N_r] fp32 (each
 *   nullable), loss [T/seq_len] fp32. Sums are fp64 in a fixed order.
 *   ws: moe_seq_balance_workspace_bytes(desc, seq_len) bytes (0 on bad args).
 * MOE_EINVAL when seq_len < 1 or T % seq_len != 0. */
size_t moe_seq_balance_workspace_bytes(const moe_desc_t* desc, int32_t seq_len);
int moe_seq_balance_loss(const moe_desc_t* desc, int32_t seq_len, float alpha, const float* scores,
                         const int32_t* topk_idx, float* f, float* P, float* loss, void* ws,
                         size_t ws_bytes, moe_stream_t stream);

/* Whole layer, the output equation of the xyznot.com guides ("Método" §2):
 *   out_t = u_t + sum_s FFN_s(u_t) + sum_k g_{k,t} FFN_{idx_k}(u_t)
 * with the gates of the gating equation (same section; pwwt.cn note 1.1.2,
 * 1.3) and, when update_bias != 0, the end-of-step bias update (pwwt.cn note
 * 1.1.3). The steps run as route -> permute -> grouped experts (routed +
 * shared) -> combine -> bias update, with the kernels of the calls above.
 * b is read by the router and, if update_bias, updated in place after the
 * loads are known.
 *   u, out [T,d] in_dtype. dbg nullable. ws: moe_workspace_bytes(desc). */
int moe_forward(const moe_desc_t* desc, const moe_weights_t* w, const void* u, float* b,
                void* out, moe_route_out_t* dbg, int32_t update_bias, void* ws,
                size_t ws_bytes, moe_stream_t stream);

/* Capacity-limited dispatch with token dropping: the DeepSeek-V2-style
 * baseline that DeepSeek-V3 does without (pwwt.cn note on the report,
 * section 1.4: V2 caps what a device receives and drops the lowest-affinity
 * tokens, which then skip the layer's experts; V3 drops none). On one GPU the
 * cap is per expert:
 *   keep [T*K] int32 (row-major over (t, k), 1 = kept, 0 = dropped): an
 *   expert with more than `capacity` selections keeps the `capacity` with the
 *   largest affinity scores[t, e] (ties: lower t) and drops the rest; every
 *   selection of an expert at or under the cap is kept. The caller picks
 *   capacity, e.g. ceil(cf * T * K / N_r) for a capacity factor cf; capacity
 *   0 drops every routed selection. n_dropped [1] (nullable): total dropped.
 *
 * moe_capacity_mask: the mask alone, from given affinities scores [T, N_r]
 *   fp32 and selections topk_idx [T, K]. ws: moe_workspace_bytes(desc).
 * moe_forward_capacity: moe_forward with the cap applied between routing and
 *   the experts. A dropped selection skips its expert and adds nothing to the
 *   token's output; the token's other gates are not renormalised. The bias
 *   update (update_bias != 0) uses the router's loads before dropping. keep
 *   nullable (workspace-internal when null). ws:
 *   moe_capacity_workspace_bytes(desc) (0 on bad desc).
 * Both: MOE_EINVAL for capacity < 0 or misaligned pointers. */
size_t moe_capacity_workspace_bytes(const moe_desc_t* desc);
int moe_capacity_mask(const moe_desc_t* desc, int32_t capacity, const float* scores,
                      const int32_t* topk_idx, int32_t* keep, int32_t* n_dropped, void* ws,
                      size_t ws_bytes, moe_stream_t stream);
int moe_forward_capacity(const moe_desc_t* desc, const moe_weights_t* w, const void* u, float* b,
                         void* out, moe_route_out_t* dbg, int32_t update_bias, int32_t capacity,
                         int32_t* keep, int32_t* n_dropped, void* ws, size_t ws_bytes,
                         moe_stream_t stream);

/* FP8 quantiser (xyznot.com guides, FP8 key idea; pwwt.cn note section 3):
 *   scale = fl32(amax/448) per 1x128 tile (ACT) or 128x128 block (W), 1 when
 *   amax = 0; q = E4M3(fl32(x/scale)), round to nearest even, saturated.
 *   src [rows, cols] fp32 or bf16 (src_dtype); cols % 128 == 0, and for W
 *   rows % 128 == 0. q [rows, cols] uint8; scale [rows, cols/128] (ACT) or
 *   [rows/128, cols/128] (W). */
int moe_quantize_fp8(int32_t kind, const void* src, int32_t src_dtype, int32_t rows,
                     int32_t cols, uint8_t* q, float* scale, moe_stream_t stream);

/* Stage timing (diagnostics, for benchmarks; not thread-safe). While enabled,
 * moe_forward records a hipEvent on its stream at every stage boundary (a
 * pool of events created by moe_profile_enable; recording stops when the pool
 * is used up). moe_profile_read waits for the recorded events, writes the
 * summed milliseconds of each stage into ms[MOE_N_STAGES] and the number of
 * recorded moe_forward calls into *calls, and with reset != 0 starts over.
 * Stage intervals are measured between consecutive events on the caller's
 * stream, so each covers exactly the kernels of that stage. */
#define MOE_STAGE_ROUTE    0   /* counts fill + router kernel */
#define MOE_STAGE_PERMUTE  1   /* bitmap, scan, scatter */
#define MOE_STAGE_QUANT_X  2   /* FP8 only: 1x128 quantiser of u */
#define MOE_STAGE_GEMM1    3   /* grouped gate/up GEMM with SwiGLU epilogue */
#define MOE_STAGE_GEMM2    4   /* (FP8: quantiser of H +) grouped down GEMM */
#define MOE_STAGE_COMBINE  5
#define MOE_STAGE_BIAS     6
#define MOE_N_STAGES       7
int moe_profile_enable(int on);
int moe_profile_read(double* ms, int64_t* calls, int reset);

/* Calibration (diagnostics, for benchmarks): the ceilings a roofline fraction
 * can be quoted against besides the published peaks.
 * moe_calibrate_read: one streaming read of buf [bytes] (bytes % 16 == 0,
 *   16-byte aligned), non-temporal 16-byte loads over a 4096-workgroup grid;
 *   sink (16-byte aligned int32, device) is written only in a case that does
 *   not occur in practice. Time it with events on `stream`: bytes / time.
 * moe_calibrate_mfma_bf16: MOE_CAL_MFMA_WAVES waves each issue iters x 8
 *   independent v_mfma_f32_32x32x16_bf16 (32768 flops each), no memory
 *   traffic: MOE_CAL_MFMA_WAVES * iters * 8 * 32768 flops per call.
 * Both: MOE_EINVAL on bad arguments. */
#define MOE_CAL_MFMA_WAVES 8192
int moe_calibrate_read(const void* buf, size_t bytes, int32_t* sink, moe_stream_t stream);
int moe_calibrate_mfma_bf16(int32_t iters, float* sink, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ROCM_H */

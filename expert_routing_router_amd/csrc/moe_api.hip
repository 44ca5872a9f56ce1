// C ABI of the MoE layer: argument validation (before anything is enqueued),
// workspace layout, and the launch sequence of each call.
#include <cmath>
#include <cstring>
#include <mutex>
#include "common.h"
#include "moe_internal.h"

using namespace moe;

static thread_local int g_last_hip = 0;

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = (int)e;
  return MOE_EHIP;
}
#define MOE_TRY(x)                           \
  do {                                       \
    hipError_t _e = (x);                     \
    if (_e != hipSuccess) return hip_status(_e); \
  } while (0)

// ---------------------------------------------------------------- stage timing
namespace {
constexpr int kProfPool = 4096;
struct Prof {
  bool on = false;
  hipEvent_t ev[kProfPool];
  int stage[kProfPool];      // stage that ends at this event; -1 marks the start of a call
  int used = 0;
  int created = 0;
  long calls = 0;
} g_prof;

void prof_mark(int stage, hipStream_t s) {
  if (!g_prof.on || g_prof.used >= g_prof.created) return;
  if (stage < 0 && g_prof.used + 2 * MOE_N_STAGES + 2 > g_prof.created) {
    g_prof.created = g_prof.used;          // not enough room for a whole call: stop here
    return;
  }
  if (stage < 0) g_prof.calls++;
  g_prof.stage[g_prof.used] = stage;
  (void)hipEventRecord(g_prof.ev[g_prof.used], s);
  g_prof.used++;
}
}  // namespace

extern "C" int moe_profile_enable(int on) {
  if (on && !g_prof.created) {
    for (int i = 0; i < kProfPool; i++) {
      hipError_t e = hipEventCreate(&g_prof.ev[i]);
      if (e != hipSuccess) { g_last_hip = (int)e; return MOE_EHIP; }
    }
    g_prof.created = kProfPool;
  }
  g_prof.on = on != 0;
  return MOE_OK;
}

extern "C" int moe_profile_read(double* ms, int64_t* calls, int reset) {
  if (!ms || !calls) return MOE_EINVAL;
  for (int i = 0; i < MOE_N_STAGES; i++) ms[i] = 0.0;
  if (g_prof.used > 0) {
    hipError_t e = hipEventSynchronize(g_prof.ev[g_prof.used - 1]);
    if (e != hipSuccess) { g_last_hip = (int)e; return MOE_EHIP; }
  }
  for (int i = 1; i < g_prof.used; i++) {
    if (g_prof.stage[i] < 0) continue;
    float t = 0.f;
    hipError_t e = hipEventElapsedTime(&t, g_prof.ev[i - 1], g_prof.ev[i]);
    if (e != hipSuccess) { g_last_hip = (int)e; return MOE_EHIP; }
    ms[g_prof.stage[i]] += t;
  }
  *calls = g_prof.calls;
  if (reset) {
    g_prof.used = 0;
    g_prof.calls = 0;
    if (g_prof.created) g_prof.created = kProfPool;
  }
  return MOE_OK;
}

static bool aligned(const void* p) { return p && (((uintptr_t)p) & 15u) == 0; }
static bool aligned_or_null(const void* p) { return !p || (((uintptr_t)p) & 15u) == 0; }
static size_t esize(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

static_assert(kCalMfmaWaves == MOE_CAL_MFMA_WAVES, "calibration grid and header disagree");

extern "C" int moe_calibrate_read(const void* buf, size_t bytes, int32_t* sink, moe_stream_t stream) {
  if (!aligned(buf) || !aligned(sink) || bytes % 16) return MOE_EINVAL;
  if (bytes == 0) return MOE_OK;
  return hip_status(launch_cal_read(buf, bytes, sink, (hipStream_t)stream));
}

extern "C" int moe_calibrate_mfma_bf16(int32_t iters, float* sink, moe_stream_t stream) {
  if (iters < 1 || !aligned(sink)) return MOE_EINVAL;
  return hip_status(launch_cal_mfma(iters, sink, (hipStream_t)stream));
}
extern "C" int moe_last_hip_error(void) { return g_last_hip; }
extern "C" const char* moe_strerror(int st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (dimension, NULL or misaligned pointer)";
    case MOE_ENOTSUP: return "unsupported dtype or shape combination";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error (see moe_last_hip_error)";
    default: return "unknown status";
  }
}

extern "C" int moe_validate(const moe_desc_t* d) {
  if (!d || d->abi_version != MOE_ABI_VERSION) return MOE_EINVAL;
  if (d->T < 0 || d->d < 8 || d->d % 8) return MOE_EINVAL;
  if (d->n_routed < 1 || d->n_routed > 256) return MOE_EINVAL;
  if (d->top_k < 1 || d->top_k > d->n_routed || d->top_k > 32) return MOE_EINVAL;
  if (d->n_groups < 1 || d->n_groups > 64 || d->n_routed % d->n_groups) return MOE_EINVAL;
  if (d->topk_groups < 1 || d->topk_groups > d->n_groups) return MOE_EINVAL;
  const int S = d->n_routed / d->n_groups;
  if (d->n_groups > 1) {
    if (d->group_topk < 1 || d->group_topk > S || d->group_topk > 8) return MOE_EINVAL;
    if (d->topk_groups * S < d->top_k) return MOE_EINVAL;
  }
  if (d->n_shared < 0 || d->n_shared > 64) return MOE_EINVAL;
  if (d->inter < 1 || (d->n_shared > 0 && d->inter_shared < 1)) return MOE_EINVAL;
  if (d->group_score_biased != 0 && d->group_score_biased != 1) return MOE_EINVAL;
  if (!std::isfinite(d->gamma)) return MOE_EINVAL;
  if (d->in_dtype != MOE_F32 && d->in_dtype != MOE_BF16) return MOE_ENOTSUP;
  if (d->router_dtype != MOE_F32 && d->router_dtype != MOE_BF16) return MOE_ENOTSUP;
  if (d->expert_dtype != MOE_F32 && d->expert_dtype != MOE_BF16 && d->expert_dtype != MOE_FP8_E4M3)
    return MOE_ENOTSUP;
  if (d->expert_dtype == MOE_F32 && d->in_dtype != MOE_F32) return MOE_ENOTSUP;
  if (d->expert_dtype == MOE_BF16) {
    if (d->in_dtype != MOE_BF16) return MOE_ENOTSUP;
    if (d->d % 128 || d->inter % 64 || (d->n_shared && d->inter_shared % 64)) return MOE_ENOTSUP;
  }
  if (d->expert_dtype == MOE_FP8_E4M3) {
    if (d->d % 128 || d->inter % 128 || (d->n_shared && d->inter_shared % 128)) return MOE_ENOTSUP;
  }
  const long rows = (long)d->T * d->top_k + (long)d->n_shared * d->T;
  const long wide = d->d > d->inter ? d->d : d->inter;
  const long wide2 = d->inter_shared > wide ? d->inter_shared : wide;
  // byte offsets of 2-byte rows stay below 2^31 (buffer-load range and int offsets)
  if (rows * wide2 >= (1L << 30) || (long)d->T * d->d >= (1L << 30)) return MOE_ENOTSUP;
  // the router addresses the centroids (as three bf16 planes for fp32 centroids)
  // with 32-bit byte offsets
  if (3L * d->n_routed * d->d * 2 >= (1L << 31)) return MOE_ENOTSUP;
  return MOE_OK;
}

// ---------------------------------------------------------------- workspace layout
struct Ws {
  size_t idx, gate, counts, bitmap, wprefix, offsets, mtile, row_token, slot_row, H, Y;
  size_t qu, su, qh, sh, offs_s, mtile_s, rscratch, total;
  size_t keep, dropped, scores;   // capacity-limited forward only
};

static RouteArgs route_args(const moe_desc_t* d, const void* u, const void* E, const float* b,
                            const float* scores_in, float* scores_out, int32_t* idx, float* gate, int32_t* counts);

// device scratch of the router for this descriptor (shape-dependent path)
static size_t route_scratch(const moe_desc_t* d) {
  return router_scratch_bytes(route_args(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr));
}

static bool fused_shared(const moe_desc_t* d) { return d->n_shared == 0 || d->inter == d->inter_shared; }

// rows of H: bf16 experts may store H K-blocked (each m-tile padded to its tile
// height, at most kMaxTileRows), for the routed and shared passes together; FP8
// experts store H's codes that way (qh_rows) and H itself row-major
constexpr size_t kMaxTileRows = 320;
static size_t h_rows(const moe_desc_t* d, size_t rows, size_t n_seg) {
  return d->expert_dtype == MOE_BF16 ? rows + (n_seg + 1) * kMaxTileRows : rows;
}
static size_t qh_rows(size_t rows, size_t n_seg) { return rows + (n_seg + 1) * kMaxTileRows; }

// K-blocked weights apply to bf16 and FP8 experts whose products all take the LDS-DMA kernels
// (FP8: 256- or 320-row tiles, which gemm_bm picks when d % 256 == 0)
static bool blocked_ok(const moe_desc_t* d) {
  const bool shared_ok = d->n_shared == 0 || d->inter_shared % 128 == 0;
  const bool dt_ok = d->expert_dtype == MOE_BF16 || d->expert_dtype == MOE_FP8_E4M3;
  return dt_ok && d->inter % 128 == 0 && d->d % 256 == 0 && shared_ok;
}
static bool use_blocked(const moe_desc_t* d, const moe_weights_t* w) {
  return blocked_ok(d) && w->w13_blk && w->w2_blk && (d->n_shared == 0 || (w->w13_shared_blk && w->w2_shared_blk));
}

static Ws layout(const moe_desc_t* d, bool capacity = false) {
  Ws w;
  const size_t T = d->T, K = d->top_k, N = d->n_routed, Ns = d->n_shared;
  const size_t W = (T + 63) / 64;
  const size_t n_seg = N + Ns;
  const size_t R = T * K + Ns * T;
  const size_t Imax = d->inter > d->inter_shared || Ns == 0 ? d->inter : d->inter_shared;
  const size_t hy = d->expert_dtype == MOE_BF16 ? 2 : 4;   // H: fp32 for F32 and FP8 experts
  const size_t yy = d->expert_dtype == MOE_F32 ? 4 : 2;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += al256(bytes); return at; };
  w.idx = take(T * K * 4);
  w.gate = take(T * K * 4);
  w.counts = take(N * 4);
  w.bitmap = take(W * N * 8);
  w.wprefix = take(W * N * 4);
  w.offsets = take((n_seg + 1) * 4);
  w.mtile = take((n_seg + 1) * 4);
  w.row_token = take(R * 4);
  w.slot_row = take(T * K * 4);
  w.offs_s = take((Ns + 1) * 4);
  w.mtile_s = take((Ns + 1) * 4);
  w.H = take(h_rows(d, R, n_seg) * Imax * hy);
  w.Y = take(R * (size_t)d->d * yy);
  if (d->expert_dtype == MOE_FP8_E4M3) {
    w.qu = take(T * d->d);
    w.su = take(T * (d->d / 128) * 4);
    w.qh = take(qh_rows(R, n_seg) * Imax);
    w.sh = take(R * (Imax / 128) * 4);
  } else {
    w.qu = w.su = w.qh = w.sh = 0;
  }
  w.rscratch = take(route_scratch(d));
  w.keep = w.dropped = w.scores = 0;
  if (capacity) {
    w.keep = take(T * K * 4);
    w.dropped = take(4);
    w.scores = take(T * N * 4);      // the router's fp32 affinities, which the cap ranks by
  }
  w.total = o;
  return w;
}

extern "C" size_t moe_workspace_bytes(const moe_desc_t* d) {
  if (moe_validate(d) != MOE_OK) return 0;
  return layout(d).total;
}

extern "C" size_t moe_expert_ffn_workspace_bytes(const moe_desc_t* d, int32_t n_experts, int32_t inter,
                                                 int32_t rows) {
  if (moe_validate(d) != MOE_OK || n_experts < 1 || inter < 1 || rows < 0) return 0;
  const size_t hy = d->expert_dtype == MOE_BF16 ? 2 : 4;
  size_t o = al256((size_t)(n_experts + 1) * 4);                 // m-tile prefix
  o += al256((size_t)rows * inter * hy);                         // H
  if (d->expert_dtype == MOE_FP8_E4M3) {
    o += al256((size_t)rows * inter);                            // H codes
    o += al256((size_t)rows * (inter / 128) * 4);                // H scales
  }
  return o;
}

static RouteArgs route_args(const moe_desc_t* d, const void* u, const void* E, const float* b,
                            const float* scores_in, float* scores_out, int32_t* idx, float* gate,
                            int32_t* counts) {
  RouteArgs a;
  a.u = u; a.E = E; a.b = b; a.scores_in = scores_in; a.scores_out = scores_out;
  a.idx = idx; a.gate = gate; a.counts = counts;
  a.T = d->T; a.d = d->d; a.n_routed = d->n_routed; a.top_k = d->top_k;
  a.n_groups = d->n_groups; a.topk_groups = d->topk_groups;
  a.group_topk = d->n_groups > 1 ? d->group_topk : 1;
  a.group_score_biased = d->group_score_biased;
  a.in_dtype = d->in_dtype; a.router_dtype = d->router_dtype;
  return a;
}

extern "C" size_t moe_route_workspace_bytes(const moe_desc_t* d) {
  if (moe_validate(d) != MOE_OK) return 0;
  return route_scratch(d);
}

extern "C" int moe_route(const moe_desc_t* d, const void* u, const void* E, const float* b,
                         const float* scores_in, float* scores_out, int32_t* topk_idx, float* topk_gate,
                         int32_t* counts, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  const bool have_ue = u || E;
  if (have_ue == (scores_in != nullptr)) return MOE_EINVAL;            // exactly one source
  if (have_ue && (!aligned(u) || !aligned(E))) return MOE_EINVAL;
  if (scores_in && !aligned(scores_in)) return MOE_EINVAL;
  if (!aligned(b) || !aligned(topk_idx) || !aligned(topk_gate) || !aligned(counts)) return MOE_EINVAL;
  if (!aligned_or_null(scores_out) || !aligned_or_null(ws)) return MOE_EINVAL;
  const size_t need = scores_in ? 0 : route_scratch(d);
  if (need && (!ws || ws_bytes < need)) return MOE_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (d->T == 0) return hip_status(launch_fill_i32(counts, 0, d->n_routed, s));
  RouteArgs a = route_args(d, u, E, b, scores_in, scores_out, topk_idx, topk_gate, counts);
  return hip_status(run_router(a, ws, s));
}

// The dispatch layout from topk_idx into caller buffers, with the bitmap and
// word-prefix scratch at `bitmap` / `wprefix` (sized for ceil(T/64) x N_r words).
static int permute_into(const moe_desc_t* d, const int32_t* topk_idx, int32_t* offsets, int32_t* row_token,
                        int32_t* slot_row, int32_t* counts, const void* u, void* x_perm, uint64_t* bitmap,
                        int32_t* wprefix, hipStream_t s) {
  if (d->T == 0) {
    MOE_TRY(launch_fill_i32(offsets, 0, d->n_routed + 1, s));
    if (counts) MOE_TRY(launch_fill_i32(counts, 0, d->n_routed, s));
    return MOE_OK;
  }
  PermuteArgs p;
  p.idx = topk_idx; p.T = d->T; p.K = d->top_k; p.n_routed = d->n_routed;
  p.bitmap = bitmap; p.wprefix = wprefix; p.counts_ws = nullptr;
  p.offsets = offsets; p.row_token = row_token; p.slot_row = slot_row; p.counts_out = counts;
  p.n_extra_seg = 0; p.mtile_prefix = nullptr; p.bm = 0;
  MOE_TRY(launch_permute(p, s));
  if (x_perm)
    MOE_TRY(launch_gather_rows(u, d->T, row_token, offsets + d->n_routed, x_perm, (long)d->T * d->top_k,
                               d->d * (int)esize(d->in_dtype), s));
  return MOE_OK;
}

static int permute_args_ok(const moe_desc_t* d, const int32_t* topk_idx, const int32_t* offsets,
                           const int32_t* row_token, const int32_t* slot_row, const int32_t* counts,
                           const void* u, const void* x_perm) {
  int st = moe_validate(d);
  if (st) return st;
  if (!aligned(topk_idx) || !aligned(offsets) || !aligned(row_token) || !aligned(slot_row)) return MOE_EINVAL;
  if (!aligned_or_null(counts) || !aligned_or_null(u) || !aligned_or_null(x_perm)) return MOE_EINVAL;
  if ((u == nullptr) != (x_perm == nullptr)) return MOE_EINVAL;
  return MOE_OK;
}

extern "C" int moe_permute(const moe_desc_t* d, const int32_t* topk_idx, int32_t* offsets, int32_t* row_token,
                           int32_t* slot_row, int32_t* counts, const void* u, void* x_perm, void* ws,
                           size_t ws_bytes, moe_stream_t stream) {
  int st = permute_args_ok(d, topk_idx, offsets, row_token, slot_row, counts, u, x_perm);
  if (st) return st;
  if (!aligned(ws)) return MOE_EINVAL;
  const Ws w = layout(d);
  if (ws_bytes < w.total) return MOE_EWORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  return permute_into(d, topk_idx, offsets, row_token, slot_row, counts, u, x_perm,
                      (uint64_t*)(base + w.bitmap), (int32_t*)(base + w.wprefix), (hipStream_t)stream);
}

// ---------------------------------------------------------------- permute without allocation
// The scratch of moe_permute_noalloc lives in this file-scope device array.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is ever handed to kernels. Each GPU holds its own copy
// until the process ends.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];
}  // namespace

// Device address of `scratch` on the current device (looked up on first use).
static int scratch_address(void** out) {
  int dev = 0;
  MOE_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    MOE_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return MOE_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

extern "C" int moe_permute_noalloc(const moe_desc_t* d, const int32_t* topk_idx, int32_t* offsets,
                                   int32_t* row_token, int32_t* slot_row, int32_t* counts, const void* u,
                                   void* x_perm, moe_stream_t stream) {
  int st = permute_args_ok(d, topk_idx, offsets, row_token, slot_row, counts, u, x_perm);
  if (st) return st;
  const size_t words = (size_t)((d->T + 63) / 64) * d->n_routed;
  const size_t bitmap_bytes = al256(words * 8);
  if (bitmap_bytes + al256(words * 4) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  void* base = nullptr;
  if ((st = scratch_address(&base))) return st;
  // every bitmap word and word prefix in range is written before it is read: nothing to clear
  return permute_into(d, topk_idx, offsets, row_token, slot_row, counts, u, x_perm, (uint64_t*)base,
                      (int32_t*)((uint8_t*)base + bitmap_bytes), (hipStream_t)stream);
}

static GemmArgs gemm_args(const void* x, long x_rows, const float* xs, const int32_t* ridx,
                          const int32_t* offsets, const int32_t* mtile, int n_seg, const void* w0,
                          const float* s0, long ws0, long ss0, void* out, int N, int K, int rows_bound) {
  GemmArgs g;
  g.x = x; g.x_rows = x_rows; g.x_scale = xs; g.row_index = ridx; g.offsets = offsets; g.mtile_prefix = mtile;
  g.n_seg = n_seg; g.w0 = w0; g.w1 = w0; g.wstride0 = ws0; g.wstride1 = ws0;
  g.ws0 = s0; g.ws1 = s0; g.sstride0 = ss0; g.sstride1 = ss0; g.n_first = n_seg;
  g.out = out; g.N = N; g.K = K; g.rows_bound = rows_bound;
  return g;
}

// GEMM1 + (FP8: quantise H) + GEMM2 over one set of segments.
// blocked: w13/w13b/w2/w2b are K-blocked copies (bf16, or FP8 codes); for bf16, H is then
// written and read K-blocked too.
static int run_ffn(const moe_desc_t* d, int inter, const void* x, long x_rows, const float* xs, const int32_t* ridx,
                   const int32_t* offsets, const int32_t* mtile, int n_seg, int rows_bound,
                   const void* w13, const float* s13, const void* w13b, const float* s13b,
                   const void* w2, const float* s2, const void* w2b, const float* s2b, int n_first,
                   void* H, uint8_t* qh, float* sh, void* Y, int bm, hipStream_t s, bool blocked = false) {
  const int dt = d->expert_dtype;
  const bool f8 = dt == MOE_FP8_E4M3;
  const long ws13 = 2L * inter * d->d, ws2 = (long)d->d * inter;
  const long ss13 = f8 ? (2L * inter / 128) * (d->d / 128) : 0, ss2 = f8 ? (long)(d->d / 128) * (inter / 128) : 0;
  GemmArgs g1 = gemm_args(x, x_rows, xs, ridx, offsets, mtile, n_seg, w13, s13, ws13, ss13, H, inter, d->d,
                          rows_bound);
  g1.w1 = w13b; g1.ws1 = s13b; g1.n_first = n_first;
  g1.w_blocked = blocked;
  g1.out_blocked = blocked;
  if (f8) {                                    // FP8: H comes out quantised (codes, 1x128 scales)
    g1.out_q = qh;
    g1.out_qs = sh;
  }
  MOE_TRY(launch_gemm_swiglu(g1, dt, bm, s));
  prof_mark(MOE_STAGE_GEMM1, s);
  const void* x2 = f8 ? (const void*)qh : H;
  const float* xs2 = f8 ? sh : nullptr;
  GemmArgs g2 = gemm_args(x2, rows_bound, xs2, nullptr, offsets, mtile, n_seg, w2, s2, ws2, ss2, Y, d->d, inter,
                          rows_bound);
  g2.w1 = w2b; g2.ws1 = s2b; g2.n_first = n_first;
  g2.w_blocked = blocked;
  g2.x_blocked = blocked;
  MOE_TRY(launch_gemm_down(g2, dt, bm, s));
  prof_mark(MOE_STAGE_GEMM2, s);
  return MOE_OK;
}

extern "C" int moe_expert_ffn(const moe_desc_t* d, int32_t n_experts, int32_t inter, int32_t rows,
                              const void* x, const float* x_scale, const int32_t* row_token,
                              const int32_t* offsets, const void* w13, const float* w13_scale,
                              const void* w2, const float* w2_scale, void* y, void* ws, size_t ws_bytes,
                              moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if (n_experts < 1 || n_experts > 320 || inter < 1 || rows < 0) return MOE_EINVAL;
  const bool f8 = d->expert_dtype == MOE_FP8_E4M3;
  if (d->expert_dtype == MOE_BF16 && inter % 64) return MOE_ENOTSUP;
  if (f8 && inter % 128) return MOE_ENOTSUP;
  if ((long)rows * (d->d > inter ? d->d : inter) >= (1L << 30)) return MOE_ENOTSUP;
  if (!aligned(x) || !aligned(offsets) || !aligned(w13) || !aligned(w2) || !aligned(y) || !aligned(ws))
    return MOE_EINVAL;
  if (!aligned_or_null(row_token)) return MOE_EINVAL;
  if (f8 && (!aligned(x_scale) || !aligned(w13_scale) || !aligned(w2_scale))) return MOE_EINVAL;
  if (ws_bytes < moe_expert_ffn_workspace_bytes(d, n_experts, inter, rows)) return MOE_EWORKSPACE;
  if (rows == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const size_t hy = d->expert_dtype == MOE_BF16 ? 2 : 4;
  uint8_t* base = (uint8_t*)ws;
  int32_t* mtile = (int32_t*)base;
  size_t o = al256((size_t)(n_experts + 1) * 4);
  void* H = base + o;
  o += al256((size_t)rows * inter * hy);
  uint8_t* qh = f8 ? base + o : nullptr;
  if (f8) o += al256((size_t)rows * inter);
  float* sh = f8 ? (float*)(base + o) : nullptr;
  const int bm = gemm_bm(d->expert_dtype, rows / n_experts, d->d, inter);
  if (d->expert_dtype != MOE_F32) MOE_TRY(launch_mtile_prefix(offsets, n_experts, bm, mtile, s));
  return run_ffn(d, inter, x, row_token ? (long)d->T : (long)rows, x_scale, row_token, offsets, mtile, n_experts,
                 rows, w13, w13_scale, w13,
                 w13_scale, w2, w2_scale, w2, w2_scale, n_experts, H, qh, sh, y, bm, s);
}

extern "C" int moe_combine(const moe_desc_t* d, const void* u, const void* y, const void* y_shared,
                           const int32_t* slot_row, const float* topk_gate, void* out, moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if (!aligned(u) || !aligned(y) || !aligned(slot_row) || !aligned(topk_gate) || !aligned(out)) return MOE_EINVAL;
  if (d->n_shared > 0 ? !aligned(y_shared) : !aligned_or_null(y_shared)) return MOE_EINVAL;
  CombineArgs c;
  c.u = u; c.y = y; c.y_shared = y_shared; c.slot_row = slot_row; c.gate = topk_gate; c.out = out;
  c.T = d->T; c.d = d->d; c.K = d->top_k; c.n_shared = y_shared ? d->n_shared : 0; c.shared_stride = d->T;
  c.io_dtype = d->in_dtype; c.y_dtype = d->expert_dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
  return hip_status(launch_combine(c, (hipStream_t)stream));
}

extern "C" int moe_update_bias(const moe_desc_t* d, const int32_t* counts, float* b, moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if (!aligned(counts) || !aligned(b)) return MOE_EINVAL;
  return hip_status(launch_update_bias(counts, b, d->n_routed, (long)d->T * d->top_k, d->gamma,
                                       (hipStream_t)stream));
}

extern "C" size_t moe_seq_balance_workspace_bytes(const moe_desc_t* d, int32_t seq_len) {
  if (moe_validate(d) != MOE_OK || seq_len < 1 || d->T % seq_len) return 0;
  return seq_balance_ws_bytes(d->T, d->n_routed, seq_len);
}

extern "C" int moe_seq_balance_loss(const moe_desc_t* d, int32_t seq_len, float alpha, const float* scores,
                                    const int32_t* topk_idx, float* f, float* P, float* loss, void* ws,
                                    size_t ws_bytes, moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if (seq_len < 1 || d->T % seq_len) return MOE_EINVAL;
  if (!aligned(scores) || !aligned(topk_idx) || !aligned(loss) || !aligned(ws)) return MOE_EINVAL;
  if (!aligned_or_null(f) || !aligned_or_null(P)) return MOE_EINVAL;
  if (d->T == 0) return MOE_OK;
  if (ws_bytes < seq_balance_ws_bytes(d->T, d->n_routed, seq_len)) return MOE_EWORKSPACE;
  return hip_status(launch_seq_balance(scores, topk_idx, d->T, d->n_routed, d->top_k, seq_len, alpha, f, P, loss,
                                       ws, (hipStream_t)stream));
}

__global__ void iota_kernel(int32_t* p, int n, int step) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i <= n) p[i] = i * step;
}

// cap < 0: no capacity limit (the layer as the method defines it); cap >= 0: each expert keeps at
// most cap selections (the dropping baseline), keep_out/n_dropped report what was kept.
static int forward_impl(const moe_desc_t* d, const moe_weights_t* w, const void* u, float* b, void* out,
                        moe_route_out_t* dbg, int32_t update_bias, void* ws, size_t ws_bytes, hipStream_t s,
                        int cap, int32_t* keep_out, int32_t* n_dropped) {
  int st = moe_validate(d);
  if (st) return st;
  if (!w || !aligned(u) || !aligned(b) || !aligned(out) || !aligned(ws)) return MOE_EINVAL;
  if (!aligned(w->centroids) || !aligned(w->w13) || !aligned(w->w2)) return MOE_EINVAL;
  const bool f8 = d->expert_dtype == MOE_FP8_E4M3;
  if (d->n_shared > 0) {
    if (!aligned(w->w13_shared) || !aligned(w->w2_shared)) return MOE_EINVAL;
    if (f8 && (!aligned(w->w13_shared_scale) || !aligned(w->w2_shared_scale))) return MOE_EINVAL;
  }
  if (f8 && (!aligned(w->w13_scale) || !aligned(w->w2_scale))) return MOE_EINVAL;
  if (dbg && (!aligned_or_null(dbg->topk_idx) || !aligned_or_null(dbg->topk_gate) ||
              !aligned_or_null(dbg->counts)))
    return MOE_EINVAL;
  const bool capped = cap >= 0;
  if (!aligned_or_null(keep_out) || !aligned_or_null(n_dropped)) return MOE_EINVAL;
  const Ws L = layout(d, capped);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (d->T == 0) {
    if (dbg && dbg->counts) MOE_TRY(launch_fill_i32(dbg->counts, 0, d->n_routed, s));
    if (n_dropped) MOE_TRY(launch_fill_i32(n_dropped, 0, 1, s));
    return MOE_OK;
  }
  uint8_t* base = (uint8_t*)ws;
  const int T = d->T, K = d->top_k, N = d->n_routed, Ns = d->n_shared;
  int32_t* idx = dbg && dbg->topk_idx ? dbg->topk_idx : (int32_t*)(base + L.idx);
  float* gate = dbg && dbg->topk_gate ? dbg->topk_gate : (float*)(base + L.gate);
  int32_t* counts = dbg && dbg->counts ? dbg->counts : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* mtile = (int32_t*)(base + L.mtile);
  int32_t* row_token = (int32_t*)(base + L.row_token);
  int32_t* slot_row = (int32_t*)(base + L.slot_row);
  const size_t hy = d->expert_dtype == MOE_BF16 ? 2 : 4;
  const size_t yy = d->expert_dtype == MOE_F32 ? 4 : 2;
  uint8_t* H = base + L.H;
  uint8_t* Y = base + L.Y;

  // 1. router
  prof_mark(-1, s);
  float* scores = capped ? (float*)(base + L.scores) : nullptr;
  // the loads come from the dispatch's bitmaps below, not from the router
  RouteArgs ra = route_args(d, u, w->centroids, b, nullptr, scores, idx, gate, nullptr);
  MOE_TRY(run_router(ra, base + L.rscratch, s));
  prof_mark(MOE_STAGE_ROUTE, s);

  // 2. dispatch layout; shared experts become extra identity segments
  const long TK = (long)T * K;
  const int bm = gemm_bm(d->expert_dtype, (int)(TK / N), d->d, d->inter);
  PermuteArgs p;
  p.idx = idx; p.T = T; p.K = K; p.n_routed = N;
  p.bitmap = (uint64_t*)(base + L.bitmap); p.wprefix = (int32_t*)(base + L.wprefix);
  p.counts_ws = nullptr; p.offsets = offsets; p.row_token = row_token; p.slot_row = slot_row;
  p.counts_out = counts;                 // every selection's load (before any dropping)
  int32_t* keep = nullptr;
  if (capped) {
    // no-drop layout first (rows of each expert in token order), then the kept subset
    p.n_extra_seg = 0; p.mtile_prefix = nullptr; p.bm = 0;
    MOE_TRY(launch_permute(p, s));
    p.counts_out = nullptr;
    keep = keep_out ? keep_out : (int32_t*)(base + L.keep);
    MOE_TRY(launch_capacity(offsets, row_token, idx, scores, T, N, K, cap, keep,
                            n_dropped ? n_dropped : (int32_t*)(base + L.dropped), s));
    p.keep = keep;
  }
  p.n_extra_seg = Ns;
  p.mtile_prefix = d->expert_dtype == MOE_F32 ? nullptr : mtile;
  p.bm = bm;
  MOE_TRY(launch_permute(p, s));
  prof_mark(MOE_STAGE_PERMUTE, s);
  // with dropping, the shared experts' rows sit at a fixed place (row T*K on) only in the
  // separate shared pass, so that pass is used
  const bool fused = fused_shared(d) && !capped;

  // 3. FP8: quantise u once per 1x128 tile
  const void* x = u;
  const float* xs = nullptr;
  if (f8) {
    MOE_TRY(launch_quant_act(u, d->in_dtype, T, d->d, nullptr, base + L.qu, (float*)(base + L.su), s));
    x = base + L.qu;
    xs = (const float*)(base + L.su);
    prof_mark(MOE_STAGE_QUANT_X, s);
  }
  uint8_t* qh = f8 ? base + L.qh : nullptr;
  float* shs = f8 ? (float*)(base + L.sh) : nullptr;

  // 4. experts
  const void* y_shared = nullptr;
  const bool blk = use_blocked(d, w);
  const void* w13r = blk ? w->w13_blk : w->w13;
  const void* w2r = blk ? w->w2_blk : w->w2;
  const void* w13s = blk ? w->w13_shared_blk : w->w13_shared;
  const void* w2s = blk ? w->w2_shared_blk : w->w2_shared;
  if (fused) {
    int st2 = run_ffn(d, d->inter, x, T, xs, row_token, offsets, mtile, N + Ns, (int)(TK + (long)Ns * T),
                      w13r, w->w13_scale, Ns ? w13s : w13r, Ns ? w->w13_shared_scale : w->w13_scale,
                      w2r, w->w2_scale, Ns ? w2s : w2r, Ns ? w->w2_shared_scale : w->w2_scale, N,
                      H, qh, shs, Y, bm, s, blk);
    if (st2) return st2;
    if (Ns) y_shared = Y + (size_t)TK * d->d * yy;
  } else {
    int st2 = run_ffn(d, d->inter, x, T, xs, row_token, offsets, mtile, N, (int)TK, w13r, w->w13_scale, w13r,
                      w->w13_scale, w2r, w->w2_scale, w2r, w->w2_scale, N, H, qh, shs, Y, bm, s, blk);
    if (st2) return st2;
  }
  if (!fused && Ns > 0) {
    int32_t* offs_s = (int32_t*)(base + L.offs_s);
    int32_t* mtile_s = (int32_t*)(base + L.mtile_s);
    iota_kernel<<<cdiv(Ns + 1, 64), 64, 0, s>>>(offs_s, Ns, T);
    MOE_TRY(hipGetLastError());
    const int bms = gemm_bm(d->expert_dtype, T, d->d, d->inter_shared);
    if (d->expert_dtype != MOE_F32) MOE_TRY(launch_mtile_prefix(offs_s, Ns, bms, mtile_s, s));
    uint8_t* Hs = H + h_rows(d, TK, N) * (d->inter > d->inter_shared ? d->inter : d->inter_shared) * hy;
    uint8_t* Ys = Y + (size_t)TK * d->d * yy;
    uint8_t* qhs = f8 ? qh + qh_rows(TK, N) * (d->inter > d->inter_shared ? d->inter : d->inter_shared) : nullptr;
    float* shss = f8 ? shs + (size_t)TK * (d->inter / 128) : nullptr;
    int st2 = run_ffn(d, d->inter_shared, x, T, xs, row_token + TK, offs_s, mtile_s, Ns, Ns * T, w13s,
                      w->w13_shared_scale, w13s, w->w13_shared_scale, w2s, w->w2_shared_scale,
                      w2s, w->w2_shared_scale, Ns, Hs, qhs, shss, Ys, bms, s, blk);
    if (st2) return st2;
    y_shared = Ys;
  }

  // 5. combine
  CombineArgs c;
  c.u = u; c.y = Y; c.y_shared = y_shared; c.slot_row = slot_row; c.gate = gate; c.out = out;
  c.T = T; c.d = d->d; c.K = K; c.n_shared = Ns; c.shared_stride = T;
  c.io_dtype = d->in_dtype; c.y_dtype = d->expert_dtype == MOE_F32 ? MOE_F32 : MOE_BF16;
  MOE_TRY(launch_combine(c, s));
  prof_mark(MOE_STAGE_COMBINE, s);

  // 6. end-of-step bias update from this batch's loads
  if (update_bias) MOE_TRY(launch_update_bias(counts, b, N, TK, d->gamma, s));
  prof_mark(MOE_STAGE_BIAS, s);
  return MOE_OK;
}

extern "C" int moe_forward(const moe_desc_t* d, const moe_weights_t* w, const void* u, float* b, void* out,
                           moe_route_out_t* dbg, int32_t update_bias, void* ws, size_t ws_bytes,
                           moe_stream_t stream) {
  return forward_impl(d, w, u, b, out, dbg, update_bias, ws, ws_bytes, (hipStream_t)stream, -1, nullptr, nullptr);
}

extern "C" size_t moe_capacity_workspace_bytes(const moe_desc_t* d) {
  if (moe_validate(d) != MOE_OK) return 0;
  return layout(d, true).total;
}

extern "C" int moe_forward_capacity(const moe_desc_t* d, const moe_weights_t* w, const void* u, float* b,
                                    void* out, moe_route_out_t* dbg, int32_t update_bias, int32_t capacity,
                                    int32_t* keep, int32_t* n_dropped, void* ws, size_t ws_bytes,
                                    moe_stream_t stream) {
  if (capacity < 0) return MOE_EINVAL;
  return forward_impl(d, w, u, b, out, dbg, update_bias, ws, ws_bytes, (hipStream_t)stream, capacity, keep,
                      n_dropped);
}

extern "C" int moe_capacity_mask(const moe_desc_t* d, int32_t capacity, const float* scores,
                                 const int32_t* topk_idx, int32_t* keep, int32_t* n_dropped, void* ws,
                                 size_t ws_bytes, moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if (capacity < 0) return MOE_EINVAL;
  if (!aligned(scores) || !aligned(topk_idx) || !aligned(keep) || !aligned_or_null(n_dropped) || !aligned(ws))
    return MOE_EINVAL;
  const Ws L = layout(d);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (d->T == 0) return n_dropped ? hip_status(launch_fill_i32(n_dropped, 0, 1, s)) : MOE_OK;
  uint8_t* base = (uint8_t*)ws;
  PermuteArgs p;
  p.idx = topk_idx; p.T = d->T; p.K = d->top_k; p.n_routed = d->n_routed;
  p.bitmap = (uint64_t*)(base + L.bitmap); p.wprefix = (int32_t*)(base + L.wprefix);
  p.counts_ws = nullptr; p.offsets = (int32_t*)(base + L.offsets); p.row_token = (int32_t*)(base + L.row_token);
  p.slot_row = (int32_t*)(base + L.slot_row); p.counts_out = nullptr;
  p.n_extra_seg = 0; p.mtile_prefix = nullptr; p.bm = 0;
  MOE_TRY(launch_permute(p, s));
  return hip_status(launch_capacity(p.offsets, p.row_token, topk_idx, scores, d->T, d->n_routed, d->top_k,
                                    capacity, keep, n_dropped, s));
}

extern "C" int moe_quantize_fp8(int32_t kind, const void* src, int32_t src_dtype, int32_t rows, int32_t cols,
                                uint8_t* q, float* scale, moe_stream_t stream) {
  if (kind != MOE_QUANT_ACT_1x128 && kind != MOE_QUANT_W_128x128) return MOE_EINVAL;
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_ENOTSUP;
  if (rows < 0 || cols < 128 || cols % 128) return MOE_EINVAL;
  if (kind == MOE_QUANT_W_128x128 && rows % 128) return MOE_EINVAL;
  if (!aligned(src) || !aligned(q) || !aligned(scale)) return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (kind == MOE_QUANT_ACT_1x128) return hip_status(launch_quant_act(src, src_dtype, rows, cols, nullptr, q, scale, s));
  return hip_status(launch_quant_w(src, src_dtype, rows, cols, q, scale, s));
}

// ---------------------------------------------------------------- backward
// Supported, with shared experts of the routed experts' size (or none); T == 0 is a no-op:
//   bf16 layers (I % 128 == 0), fp32 layers (I % 8 == 0), and FP8 layers with bf16 u,
//   d % 256 == 0 and I % 256 == 0 (every product of the FP8 backward on the 256-row
//   LDS-DMA kernels) whose padded weight-gradient operands stay under 2^31 bytes.
static long bwd_rows(const moe_desc_t* d) { return (long)d->T * d->top_k + (long)d->n_shared * d->T; }
static long bwd_f8_pitch(const moe_desc_t* d) {
  return wgrad_pitch(bwd_rows(d), d->n_routed + d->n_shared, 128);
}
static int backward_shape_ok(const moe_desc_t* d) {
  const bool bf = d->in_dtype == MOE_BF16 && d->expert_dtype == MOE_BF16;
  const bool f32 = d->in_dtype == MOE_F32 && d->expert_dtype == MOE_F32;
  const bool f8 = d->in_dtype == MOE_BF16 && d->expert_dtype == MOE_FP8_E4M3;
  if (!bf && !f32 && !f8) return MOE_ENOTSUP;
  if (bf && d->inter % 128) return MOE_ENOTSUP;
  if (f32 && d->inter % 8) return MOE_ENOTSUP;
  if (f8) {
    if (d->d % 256 || d->inter % 256) return MOE_ENOTSUP;
    const long wide = std::max<long>(d->d, 2L * d->inter);
    if (wide * bwd_f8_pitch(d) >= (1L << 31) || bwd_rows(d) * wide >= (1L << 31)) return MOE_ENOTSUP;
  }
  if (d->n_shared && d->inter_shared != d->inter) return MOE_ENOTSUP;
  return MOE_OK;
}

struct BwdWs {
  size_t idx, gate, scores, rscratch, bitmap, wprefix, offsets, mtile, row_token, slot_row;
  size_t ab, h, y, dy, dh, dab, dg, dz, pt, qt, kofs, q8, qs, pt8, qt8, spt, sqt, total;
  long pitch;
};

static BwdWs bwd_layout(const moe_desc_t* d) {
  BwdWs w;
  const size_t T = d->T, K = d->top_k, N = d->n_routed, Ns = d->n_shared, I = d->inter, D = d->d;
  const size_t W = (T + 63) / 64, n_seg = N + Ns, R = T * K + Ns * T;
  const bool f8 = d->expert_dtype == MOE_FP8_E4M3;
  const size_t es = d->expert_dtype == MOE_F32 ? 4 : 2;     // activations A|B, H, Y, dY, dH, dA|dB
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += al256(bytes); return at; };
  w.idx = take(T * K * 4);
  w.gate = take(T * K * 4);
  w.scores = take(T * N * 4);
  w.rscratch = take(route_scratch(d));
  w.bitmap = take(W * N * 8);
  w.wprefix = take(W * N * 4);
  w.offsets = take((n_seg + 1) * 4);
  w.mtile = take((n_seg + 1) * 4);
  w.row_token = take(R * 4);
  w.slot_row = take(T * K * 4);
  w.ab = take(R * 2 * I * es);
  w.h = take(R * I * es);
  w.y = take(R * D * es);          // Y, then dX
  w.dy = take(R * D * es);
  w.dh = take(R * I * es);
  w.dab = take(R * 2 * I * es);
  w.dg = take(T * K * 4);
  w.dz = take(T * K * 4);
  // transposed, padded operands of the weight-gradient GEMMs (d a multiple of 256; FP8:
  // segments padded to 128 rows, one scale tile)
  w.pitch = f8 ? bwd_f8_pitch(d) : D % 256 == 0 && es == 2 ? wgrad_pitch((long)R, (int)n_seg) : 0;
  const size_t wide = D > 2 * I ? D : 2 * I;
  w.pt = w.pitch ? take(wide * (size_t)w.pitch * 2) : 0;
  w.qt = w.pitch ? take(wide * (size_t)w.pitch * 2) : 0;
  w.kofs = w.pitch ? take((n_seg + 1) * 4) : 0;
  // FP8: E4M3 copy of the activation each product reads (u, H, dY, dA|dB in turn) and its
  // 1x128 scales; the weight-gradient operands' codes and transposed scales
  w.q8 = f8 ? take(R * wide) : 0;
  w.qs = f8 ? take(R * (wide / 128) * 4) : 0;
  w.pt8 = f8 ? take(wide * (size_t)w.pitch) : 0;
  w.qt8 = f8 ? take(wide * (size_t)w.pitch) : 0;
  w.spt = f8 ? take((size_t)w.pitch / 128 * wide * 4) : 0;
  w.sqt = f8 ? take((size_t)w.pitch / 128 * wide * 4) : 0;
  w.total = o;
  return w;
}

extern "C" size_t moe_backward_workspace_bytes(const moe_desc_t* d) {
  if (moe_validate(d) != MOE_OK || backward_shape_ok(d) != MOE_OK) return 0;
  return bwd_layout(d).total;
}

extern "C" int moe_transpose_expert_weights(const moe_desc_t* d, const moe_weights_t* w, moe_weights_t* wt,
                                            moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if ((st = backward_shape_ok(d))) return st;
  if (!w || !wt || !aligned(w->w13) || !aligned(w->w2) || !aligned(wt->w13) || !aligned(wt->w2)) return MOE_EINVAL;
  if (d->n_shared && (!aligned(w->w13_shared) || !aligned(w->w2_shared) || !aligned(wt->w13_shared) ||
                      !aligned(wt->w2_shared)))
    return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const int I = d->inter, D = d->d, dt = d->expert_dtype;
  if (dt == MOE_FP8_E4M3) {
    // the transpose of an E4M3 matrix with 128x128 block scales is its codes and its scale grid
    // transposed: exactly the same values
    if (!aligned(w->w13_scale) || !aligned(w->w2_scale) || !aligned(wt->w13_scale) || !aligned(wt->w2_scale))
      return MOE_EINVAL;
    if (d->n_shared && (!aligned(w->w13_shared_scale) || !aligned(w->w2_shared_scale) ||
                        !aligned(wt->w13_shared_scale) || !aligned(wt->w2_shared_scale)))
      return MOE_EINVAL;
    MOE_TRY(launch_transpose(w->w13_scale, (void*)wt->w13_scale, d->n_routed, 2 * I / 128, D / 128, MOE_F32, s));
    MOE_TRY(launch_transpose(w->w2_scale, (void*)wt->w2_scale, d->n_routed, D / 128, I / 128, MOE_F32, s));
    if (d->n_shared) {
      MOE_TRY(launch_transpose(w->w13_shared_scale, (void*)wt->w13_shared_scale, d->n_shared, 2 * I / 128, D / 128,
                               MOE_F32, s));
      MOE_TRY(launch_transpose(w->w2_shared_scale, (void*)wt->w2_shared_scale, d->n_shared, D / 128, I / 128,
                               MOE_F32, s));
    }
  }
  MOE_TRY(launch_transpose(w->w13, (void*)wt->w13, d->n_routed, 2 * I, D, dt, s));
  MOE_TRY(launch_transpose(w->w2, (void*)wt->w2, d->n_routed, D, I, dt, s));
  if (d->n_shared) {
    MOE_TRY(launch_transpose(w->w13_shared, (void*)wt->w13_shared, d->n_shared, 2 * I, D, dt, s));
    MOE_TRY(launch_transpose(w->w2_shared, (void*)wt->w2_shared, d->n_shared, D, I, dt, s));
  }
  return MOE_OK;
}

extern "C" int moe_pack_expert_weights(const moe_desc_t* d, const moe_weights_t* w, moe_weights_t* wb,
                                       moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if (!blocked_ok(d)) return MOE_ENOTSUP;
  if (!w || !wb || !aligned(w->w13) || !aligned(w->w2) || !aligned(wb->w13) || !aligned(wb->w2)) return MOE_EINVAL;
  if (d->n_shared && (!aligned(w->w13_shared) || !aligned(w->w2_shared) || !aligned(wb->w13_shared) ||
                      !aligned(wb->w2_shared)))
    return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const int I = d->inter, Is = d->inter_shared, D = d->d;
  auto pack = [&](const void* src, const void* dst, int n_mat, int rows, int K, int swiglu_i) {
    return d->expert_dtype == MOE_BF16
        ? launch_pack_blocked((const uint16_t*)src, (uint16_t*)dst, n_mat, rows, K, swiglu_i, s)
        : launch_pack_blocked_f8((const uint8_t*)src, (uint8_t*)dst, n_mat, rows, K, swiglu_i, s);
  };
  MOE_TRY(pack(w->w13, wb->w13, d->n_routed, 2 * I, D, I));
  MOE_TRY(pack(w->w2, wb->w2, d->n_routed, D, I, 0));
  if (d->n_shared) {
    MOE_TRY(pack(w->w13_shared, wb->w13_shared, d->n_shared, 2 * Is, D, Is));
    MOE_TRY(pack(w->w2_shared, wb->w2_shared, d->n_shared, D, Is, 0));
  }
  return MOE_OK;
}

extern "C" int moe_backward(const moe_desc_t* d, const moe_weights_t* w, const moe_weights_t* wt, const void* u,
                            const float* b, const void* dout, moe_grads_t* g, void* ws, size_t ws_bytes,
                            moe_stream_t stream) {
  int st = moe_validate(d);
  if (st) return st;
  if ((st = backward_shape_ok(d))) return st;
  if (!w || !wt || !g) return MOE_EINVAL;
  if (!aligned(u) || !aligned(b) || !aligned(dout) || !aligned(ws) || !aligned(w->centroids)) return MOE_EINVAL;
  if (!aligned(w->w13) || !aligned(w->w2) || !aligned(wt->w13) || !aligned(wt->w2)) return MOE_EINVAL;
  if (!aligned(g->du) || !aligned(g->dE) || !aligned(g->dw13) || !aligned(g->dw2)) return MOE_EINVAL;
  if (d->n_shared && (!aligned(w->w13_shared) || !aligned(w->w2_shared) || !aligned(wt->w13_shared) ||
                      !aligned(wt->w2_shared) || !aligned(g->dw13_shared) || !aligned(g->dw2_shared)))
    return MOE_EINVAL;
  const bool f8 = d->expert_dtype == MOE_FP8_E4M3;
  if (f8 && (!aligned(w->w13_scale) || !aligned(w->w2_scale) || !aligned(wt->w13_scale) || !aligned(wt->w2_scale)))
    return MOE_EINVAL;
  if (f8 && d->n_shared && (!aligned(w->w13_shared_scale) || !aligned(w->w2_shared_scale) ||
                            !aligned(wt->w13_shared_scale) || !aligned(wt->w2_shared_scale)))
    return MOE_EINVAL;
  const BwdWs L = bwd_layout(d);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  const int T = d->T, K = d->top_k, N = d->n_routed, Ns = d->n_shared, I = d->inter, D = d->d;
  const long TK = (long)T * K, R = TK + (long)Ns * T;
  const int n_seg = N + Ns;
  const int wdt = d->expert_dtype;
  const int dt = f8 ? MOE_BF16 : wdt;                // activations: bf16 (bf16 and FP8 layers) or fp32
  int32_t* idx = (int32_t*)(base + L.idx);
  float* gate = (float*)(base + L.gate);
  float* scores = (float*)(base + L.scores);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* mtile = (int32_t*)(base + L.mtile);
  int32_t* row_token = (int32_t*)(base + L.row_token);
  int32_t* slot_row = (int32_t*)(base + L.slot_row);
  void* AB = base + L.ab;
  void* H = base + L.h;
  void* Y = base + L.y;
  void* dY = base + L.dy;
  void* dH = base + L.dh;
  void* dAB = base + L.dab;
  float* dg = (float*)(base + L.dg);
  float* dz = (float*)(base + L.dz);

  // forward recompute: the same routing and dispatch as moe_forward (the same router,
  // which also keeps the affinities for the gate gradients), then A|B, H, Y
  RouteArgs ra = route_args(d, u, w->centroids, b, nullptr, scores, idx, gate, nullptr);   // loads not needed
  MOE_TRY(run_router(ra, base + L.rscratch, s));
  // the forward's tile height (FP8: 256 or 320 rows by the mean load; every product's width
  // is a multiple of 256 here, as the LDS-DMA kernels need)
  const int bm = gemm_bm(d->expert_dtype, (int)(TK / N), d->d, d->inter);
  PermuteArgs p;
  p.idx = idx; p.T = T; p.K = K; p.n_routed = N;
  p.bitmap = (uint64_t*)(base + L.bitmap); p.wprefix = (int32_t*)(base + L.wprefix);
  p.counts_ws = nullptr; p.offsets = offsets; p.row_token = row_token; p.slot_row = slot_row;
  p.counts_out = nullptr; p.n_extra_seg = Ns; p.mtile_prefix = mtile; p.bm = bm;
  MOE_TRY(launch_permute(p, s));
  // out = x W^T per segment (W = w0[e], or w1[e - N] for the shared segments); FP8 layers
  // first quantise x per 1x128 tile (the activation operand of each FP8 product) and
  // multiply E4M3 by E4M3 with both scales applied per 128-long block of the reduction
  uint8_t* q8 = f8 ? base + L.q8 : nullptr;
  float* qs = f8 ? (float*)(base + L.qs) : nullptr;
  auto grouped = [&](const void* x, long x_rows, const int32_t* ridx, const void* w0, const void* w1,
                     const float* sc0, const float* sc1, long wstride, void* out, int Nout,
                     int Kred) -> hipError_t {
    const long sstride = f8 ? wstride / (128L * 128) : 0;
    if (f8) {
      hipError_t e = launch_quant_act(x, MOE_BF16, x_rows, Kred, nullptr, q8, qs, s);
      if (e != hipSuccess) return e;
    }
    GemmArgs ga = gemm_args(f8 ? q8 : x, x_rows, qs, ridx, offsets, mtile, n_seg, w0, sc0, wstride, sstride, out,
                            Nout, Kred, (int)R);
    ga.w1 = Ns ? w1 : w0;
    ga.ws1 = Ns ? sc1 : sc0;
    ga.n_first = N;
    return launch_gemm_down(ga, wdt, bm, s);
  };
  const long s13 = 2L * I * D, s2 = (long)D * I;
  MOE_TRY(grouped(u, T, row_token, w->w13, w->w13_shared, w->w13_scale, w->w13_shared_scale, s13, AB, 2 * I,
                  D));                                                                // [A|B] = X W13^T
  MOE_TRY(launch_swiglu_fwd(AB, H, R, I, dt, s));                                     // H = SiLU(A) B
  MOE_TRY(grouped(H, R, nullptr, w->w2, w->w2_shared, w->w2_scale, w->w2_shared_scale, s2, Y, D,
                  I));                                                                // Y = H W2^T

  // backward
  MOE_TRY(launch_dgate_dy(dout, Y, slot_row, gate, T, D, K, Ns, TK, T, dg, dY, dt, s));   // dg, dY
  MOE_TRY(grouped(dY, R, nullptr, wt->w2, wt->w2_shared, wt->w2_scale, wt->w2_shared_scale, s2, dH, I,
                  D));                                                                // dH = dY W2
  MOE_TRY(launch_swiglu_bwd(dH, AB, dAB, R, I, dt, s));                               // dA | dB
  void* dX = Y;                                                                       // Y is no longer needed
  MOE_TRY(grouped(dAB, R, nullptr, wt->w13, wt->w13_shared, wt->w13_scale, wt->w13_shared_scale, s13, dX, D,
                  2 * I));                                                            // dX = [dA dB] W13
  MOE_TRY(launch_router_bwd(scores, idx, dg, dout, dX, slot_row, w->centroids, d->router_dtype, u, offsets,
                            row_token, T, N, D, K, Ns, TK, T, dz, g->du, g->dE, dt, s));  // dz, du, dE
  WgradArgs wa;
  wa.offsets = offsets; wa.n_seg = n_seg; wa.n_first = N;
  if (L.pitch) {
    wa.pt = (uint16_t*)(base + L.pt); wa.qt = (uint16_t*)(base + L.qt); wa.kofs = (int32_t*)(base + L.kofs);
    wa.pitch = L.pitch;
  }
  // FP8: both operands quantised in 128-row tiles along each expert's rows
  WgradF8Scratch f8s{f8 ? base + L.pt8 : nullptr, f8 ? base + L.qt8 : nullptr,
                     f8 ? (float*)(base + L.spt) : nullptr, f8 ? (float*)(base + L.sqt) : nullptr};
  auto wgrad = [&](const void* P, const void* Q) -> hipError_t {
    if (dt == MOE_F32) return launch_wgrad_f32(wa, (const float*)P, (const float*)Q, s);
    return f8 ? launch_wgrad_f8(wa, f8s, s) : launch_wgrad(wa, s);
  };
  wa.P = (const uint16_t*)dY; wa.Q = (const uint16_t*)H; wa.q_row = nullptr; wa.q_rows = R; wa.M = D; wa.Nn = I;
  wa.out0 = g->dw2; wa.ostride0 = s2; wa.out1 = Ns ? g->dw2_shared : g->dw2; wa.ostride1 = s2;
  MOE_TRY(wgrad(dY, H));                                                              // dW2 = dY^T H
  wa.P = (const uint16_t*)dAB; wa.Q = (const uint16_t*)u; wa.q_row = row_token; wa.q_rows = T; wa.M = 2 * I;
  wa.Nn = D;
  wa.out0 = g->dw13; wa.ostride0 = s13; wa.out1 = Ns ? g->dw13_shared : g->dw13; wa.ostride1 = s13;
  MOE_TRY(wgrad(dAB, u));                                                             // dW13 = [dA dB]^T X
  return MOE_OK;
}

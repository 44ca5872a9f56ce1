"""ctypes binding of libmoe_rocm.so: argument marshalling only.

Every function here has the name of the C entry point it calls and forwards
torch tensors as device pointers plus torch's current HIP stream. No step of
the layer runs in Python: if the library is missing the import-time loader
raises, and there is no CPU fallback.
"""

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ROCM_LIB names another build of the same library (e.g. the host-sanitizer build)
LIB_PATH = os.environ.get("MOE_ROCM_LIB") or os.path.join(HERE, "libmoe_rocm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe_rocm.h")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_QUANT_ACT_1x128, MOE_QUANT_W_128x128 = 0, 1
ABI_VERSION = 3
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}


class MoeError(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.moe_strerror(status).decode()
        if status == MOE_EHIP:
            msg += " (hip error %d)" % lib.moe_last_hip_error()
        super().__init__("%s: %s [%d]" % (fn, msg, status))
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "T", "d", "n_routed", "top_k", "n_groups", "topk_groups", "group_topk",
        "n_shared", "inter", "inter_shared", "in_dtype", "router_dtype", "expert_dtype",
        "group_score_biased")] + [("gamma", ctypes.c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "centroids", "w13", "w2", "w13_shared", "w2_shared", "w13_scale", "w2_scale",
        "w13_shared_scale", "w2_shared_scale", "w13_blk", "w2_blk", "w13_shared_blk", "w2_shared_blk")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("du", "dE", "dw13", "dw2", "dw13_shared", "dw2_shared")]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_gate", ctypes.c_void_p), ("counts", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the in-tree library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_rocm.so is not built (python -m expert_routing_router_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(MoeDesc)
        sig = {
            "moe_abi_version": ([], I32),
            "moe_strerror": ([I32], ctypes.c_char_p),
            "moe_last_hip_error": ([], I32),
            "moe_validate": ([D], I32),
            "moe_workspace_bytes": ([D], SZ),
            "moe_route_workspace_bytes": ([D], SZ),
            "moe_route": ([D, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_permute": ([D, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_permute_noalloc": ([D, P, P, P, P, P, P, P, P], I32),
            "moe_expert_ffn_workspace_bytes": ([D, I32, I32, I32], SZ),
            "moe_expert_ffn": ([D, I32, I32, I32, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_combine": ([D, P, P, P, P, P, P, P], I32),
            "moe_update_bias": ([D, P, P, P], I32),
            "moe_forward": ([D, ctypes.POINTER(MoeWeights), P, P, P, ctypes.POINTER(MoeRouteOut),
                             I32, P, SZ, P], I32),
            "moe_quantize_fp8": ([I32, P, I32, I32, I32, P, P, P], I32),
            "moe_seq_balance_workspace_bytes": ([D, I32], SZ),
            "moe_transpose_expert_weights": ([D, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeights), P], I32),
            "moe_pack_expert_weights": ([D, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeights), P], I32),
            "moe_backward_workspace_bytes": ([D], SZ),
            "moe_backward": ([D, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeights), P, P, P,
                              ctypes.POINTER(MoeGrads), P, SZ, P], I32),
            "moe_seq_balance_loss": ([D, I32, ctypes.c_float, P, P, P, P, P, P, SZ, P], I32),
            "moe_capacity_workspace_bytes": ([D], SZ),
            "moe_capacity_mask": ([D, I32, P, P, P, P, P, SZ, P], I32),
            "moe_forward_capacity": ([D, ctypes.POINTER(MoeWeights), P, P, P, ctypes.POINTER(MoeRouteOut),
                                      I32, I32, P, P, P, SZ, P], I32),
            "moe_calibrate_read": ([P, SZ, P, P], I32),
            "moe_calibrate_mfma_bf16": ([I32, P, P], I32),
            "moe_profile_enable": ([I32], I32),
            "moe_profile_read": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), I32], I32),
        }
        for name, (argt, rest) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = argt, rest
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError("libmoe_rocm ABI mismatch")
        _lib = L
    return _lib


def header_symbols():
    """Entry points declared in include/moe_rocm.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\(", text, re.M)))


# ---------------------------------------------------------------- marshalling helpers
def make_desc(T, d, n_routed, top_k, n_groups=1, topk_groups=1, group_topk=None, n_shared=0,
              inter=128, inter_shared=None, in_dtype="bf16", router_dtype="bf16",
              expert_dtype="bf16", group_score_biased=1, gamma=0.001) -> MoeDesc:
    if group_topk is None:
        group_topk = max(1, top_k // topk_groups)
    return MoeDesc(ABI_VERSION, T, d, n_routed, top_k, n_groups, topk_groups, group_topk,
                   n_shared, inter, inter if inter_shared is None else inter_shared,
                   DTYPES.get(in_dtype, in_dtype), DTYPES.get(router_dtype, router_dtype),
                   DTYPES.get(expert_dtype, expert_dtype), group_score_biased, gamma)


def desc_from_config(cfg, T=None) -> MoeDesc:
    return make_desc(cfg.T if T is None else T, cfg.d, cfg.n_routed, cfg.top_k, cfg.n_groups,
                     cfg.topk_groups, cfg.group_topk, cfg.n_shared, cfg.inter, cfg.inter_shared,
                     cfg.in_dtype, cfg.router_dtype, cfg.expert_dtype, cfg.group_score_biased,
                     cfg.gamma)


def _ptr(t, name, required=True):
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st, lib())


# ---------------------------------------------------------------- entry points
def moe_validate(desc: MoeDesc) -> int:
    return lib().moe_validate(ctypes.byref(desc))


def moe_workspace_bytes(desc: MoeDesc) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(desc))


def moe_expert_ffn_workspace_bytes(desc, n_experts, inter, rows) -> int:
    return lib().moe_expert_ffn_workspace_bytes(ctypes.byref(desc), n_experts, inter, rows)


def moe_route_workspace_bytes(desc) -> int:
    return lib().moe_route_workspace_bytes(ctypes.byref(desc))


def moe_route(desc, b, topk_idx, topk_gate, counts, u=None, E=None, scores_in=None,
              scores_out=None, ws=None, stream=None):
    """ws: the router's scratch (moe_route_workspace_bytes); allocated here when not given."""
    if ws is None and scores_in is None:
        n = moe_route_workspace_bytes(desc)
        if n:
            ws = torch.empty(n, dtype=torch.uint8, device=b.device)
    _check("moe_route", lib().moe_route(
        ctypes.byref(desc), _ptr(u, "u", False), _ptr(E, "E", False), _ptr(b, "b"),
        _ptr(scores_in, "scores_in", False), _ptr(scores_out, "scores_out", False),
        _ptr(topk_idx, "topk_idx"), _ptr(topk_gate, "topk_gate"), _ptr(counts, "counts"),
        _ptr(ws, "ws", False), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute(desc, topk_idx, offsets, row_token, slot_row, ws, counts=None, u=None,
                x_perm=None, stream=None):
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(desc), _ptr(topk_idx, "topk_idx"), _ptr(offsets, "offsets"),
        _ptr(row_token, "row_token"), _ptr(slot_row, "slot_row"), _ptr(counts, "counts", False),
        _ptr(u, "u", False), _ptr(x_perm, "x_perm", False), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute_noalloc(desc, topk_idx, offsets, row_token, slot_row, counts=None, u=None,
                        x_perm=None, stream=None):
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        ctypes.byref(desc), _ptr(topk_idx, "topk_idx"), _ptr(offsets, "offsets"),
        _ptr(row_token, "row_token"), _ptr(slot_row, "slot_row"), _ptr(counts, "counts", False),
        _ptr(u, "u", False), _ptr(x_perm, "x_perm", False), _stream(stream)))


def moe_expert_ffn(desc, n_experts, inter, rows, x, offsets, w13, w2, y, ws, row_token=None,
                   x_scale=None, w13_scale=None, w2_scale=None, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(desc), n_experts, inter, rows, _ptr(x, "x"), _ptr(x_scale, "x_scale", False),
        _ptr(row_token, "row_token", False), _ptr(offsets, "offsets"), _ptr(w13, "w13"),
        _ptr(w13_scale, "w13_scale", False), _ptr(w2, "w2"), _ptr(w2_scale, "w2_scale", False),
        _ptr(y, "y"), _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def moe_combine(desc, u, y, slot_row, topk_gate, out, y_shared=None, stream=None):
    _check("moe_combine", lib().moe_combine(
        ctypes.byref(desc), _ptr(u, "u"), _ptr(y, "y"), _ptr(y_shared, "y_shared", False),
        _ptr(slot_row, "slot_row"), _ptr(topk_gate, "topk_gate"), _ptr(out, "out"),
        _stream(stream)))


def moe_update_bias(desc, counts, b, stream=None):
    _check("moe_update_bias", lib().moe_update_bias(
        ctypes.byref(desc), _ptr(counts, "counts"), _ptr(b, "b"), _stream(stream)))


def moe_forward(desc, weights: MoeWeights, u, b, out, ws, update_bias=True, topk_idx=None,
                topk_gate=None, counts=None, stream=None):
    dbg = None
    if topk_idx is not None or topk_gate is not None or counts is not None:
        dbg = MoeRouteOut(_ptr(topk_idx, "topk_idx", False), _ptr(topk_gate, "topk_gate", False),
                          _ptr(counts, "counts", False))
    _check("moe_forward", lib().moe_forward(
        ctypes.byref(desc), ctypes.byref(weights), _ptr(u, "u"), _ptr(b, "b"), _ptr(out, "out"),
        ctypes.byref(dbg) if dbg is not None else None, int(bool(update_bias)), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_capacity_workspace_bytes(desc) -> int:
    return lib().moe_capacity_workspace_bytes(ctypes.byref(desc))


def moe_capacity_mask(desc, capacity, scores, topk_idx, keep, ws, n_dropped=None, stream=None):
    _check("moe_capacity_mask", lib().moe_capacity_mask(
        ctypes.byref(desc), capacity, _ptr(scores, "scores"), _ptr(topk_idx, "topk_idx"), _ptr(keep, "keep"),
        _ptr(n_dropped, "n_dropped", False), _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def moe_forward_capacity(desc, weights: MoeWeights, u, b, out, ws, capacity, update_bias=True, keep=None,
                         n_dropped=None, topk_idx=None, topk_gate=None, counts=None, stream=None):
    dbg = None
    if topk_idx is not None or topk_gate is not None or counts is not None:
        dbg = MoeRouteOut(_ptr(topk_idx, "topk_idx", False), _ptr(topk_gate, "topk_gate", False),
                          _ptr(counts, "counts", False))
    _check("moe_forward_capacity", lib().moe_forward_capacity(
        ctypes.byref(desc), ctypes.byref(weights), _ptr(u, "u"), _ptr(b, "b"), _ptr(out, "out"),
        ctypes.byref(dbg) if dbg is not None else None, int(bool(update_bias)), capacity,
        _ptr(keep, "keep", False), _ptr(n_dropped, "n_dropped", False), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_quantize_fp8(kind, src, rows, cols, q, scale, stream=None):
    sdt = MOE_BF16 if src.dtype == torch.bfloat16 else MOE_F32
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(
        kind, _ptr(src, "src"), sdt, rows, cols, _ptr(q, "q"), _ptr(scale, "scale"),
        _stream(stream)))


def moe_seq_balance_workspace_bytes(desc, seq_len) -> int:
    return lib().moe_seq_balance_workspace_bytes(ctypes.byref(desc), seq_len)


def moe_seq_balance_loss(desc, seq_len, alpha, scores, topk_idx, loss, ws, f=None, P=None, stream=None):
    _check("moe_seq_balance_loss", lib().moe_seq_balance_loss(
        ctypes.byref(desc), seq_len, alpha, _ptr(scores, "scores"), _ptr(topk_idx, "topk_idx"),
        _ptr(f, "f", False), _ptr(P, "P", False), _ptr(loss, "loss"), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_transpose_expert_weights(desc, weights: MoeWeights, wt: MoeWeights, stream=None):
    _check("moe_transpose_expert_weights", lib().moe_transpose_expert_weights(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(wt), _stream(stream)))


def moe_pack_expert_weights(desc, weights: MoeWeights, wb: MoeWeights, stream=None):
    _check("moe_pack_expert_weights", lib().moe_pack_expert_weights(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(wb), _stream(stream)))


def moe_backward_workspace_bytes(desc) -> int:
    return lib().moe_backward_workspace_bytes(ctypes.byref(desc))


def make_grads(du, dE, dw13, dw2, dw13_shared=None, dw2_shared=None) -> MoeGrads:
    return MoeGrads(*[_ptr(t, n, n in ("du", "dE", "dw13", "dw2")) for t, n in (
        (du, "du"), (dE, "dE"), (dw13, "dw13"), (dw2, "dw2"), (dw13_shared, "dw13_shared"),
        (dw2_shared, "dw2_shared"))])


def moe_backward(desc, weights: MoeWeights, wt: MoeWeights, u, b, dout, grads: MoeGrads, ws, stream=None):
    _check("moe_backward", lib().moe_backward(
        ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(wt), _ptr(u, "u"), _ptr(b, "b"),
        _ptr(dout, "dout"), ctypes.byref(grads), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)))


MOE_CAL_MFMA_WAVES = 8192


def moe_calibrate_read(buf, sink, stream=None):
    _check("moe_calibrate_read", lib().moe_calibrate_read(
        _ptr(buf, "buf"), buf.numel() * buf.element_size(), _ptr(sink, "sink"), _stream(stream)))


def moe_calibrate_mfma_bf16(iters, sink, stream=None):
    _check("moe_calibrate_mfma_bf16", lib().moe_calibrate_mfma_bf16(iters, _ptr(sink, "sink"), _stream(stream)))


STAGES = ("route", "permute", "quant_x", "gemm1", "gemm2", "combine", "bias")


def moe_profile_enable(on=True):
    _check("moe_profile_enable", lib().moe_profile_enable(int(bool(on))))


def moe_profile_read(reset=True):
    """Summed milliseconds per stage of the recorded moe_forward calls, and the call count."""
    ms = (ctypes.c_double * len(STAGES))()
    calls = ctypes.c_int64(0)
    _check("moe_profile_read", lib().moe_profile_read(ms, ctypes.byref(calls), int(bool(reset))))
    return dict(zip(STAGES, list(ms))), calls.value


def make_weights(centroids, w13, w2, w13_shared=None, w2_shared=None, w13_scale=None,
                 w2_scale=None, w13_shared_scale=None, w2_shared_scale=None, w13_blk=None, w2_blk=None,
                 w13_shared_blk=None, w2_shared_blk=None) -> MoeWeights:
    return MoeWeights(*[_ptr(t, n, False) for t, n in (
        (centroids, "centroids"), (w13, "w13"), (w2, "w2"), (w13_shared, "w13_shared"),
        (w2_shared, "w2_shared"), (w13_scale, "w13_scale"), (w2_scale, "w2_scale"),
        (w13_shared_scale, "w13_shared_scale"), (w2_shared_scale, "w2_shared_scale"),
        (w13_blk, "w13_blk"), (w2_blk, "w2_blk"), (w13_shared_blk, "w13_shared_blk"),
        (w2_shared_blk, "w2_shared_blk"))])

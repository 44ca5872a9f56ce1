"""Device-side plumbing around the C ABI: weight upload, workspace, one call.

`MoELayer` owns device tensors (centroids, expert weights, FP8 codes and
scales, the workspace) and calls `moe_forward`. Weights arrive as numpy arrays
from a generator callback, one expert at a time, so a 22.5 GB bf16 stack never
needs a second full host copy. All arithmetic happens in libmoe_rocm.so.
"""

from concurrent.futures import ThreadPoolExecutor
import ctypes
import os

import numpy as np
import torch

from . import _lib as L


def np_to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Canonical numpy input (bf16 bits as uint16, or fp32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


class MoELayer:
    def __init__(self, cfg, gen, device="cuda", threads=0, blocked_weights=True):
        """cfg: layer configuration (T, d, N_r, ... dtypes); gen: the input source, an object
        with centroids(cfg), expert_w13(cfg, e), expert_w2(cfg, e), shared_w13(cfg, s),
        shared_w2(cfg, s) returning numpy arrays (bf16 bits as uint16, or fp32).
        blocked_weights: also keep K-blocked copies of bf16 / FP8 expert weights (moe_pack_expert_weights)
        for the forward, where the shapes allow it; self.blocked says whether they are in use."""
        self.cfg = cfg
        self.device = torch.device(device)
        self.desc = L.desc_from_config(cfg)
        st = L.moe_validate(self.desc)
        if st != L.MOE_OK:
            raise L.MoeError("moe_validate", st, L.lib())
        self.E = np_to_device(gen.centroids(cfg), cfg.router_dtype, self.device)
        threads = threads or min(16, os.cpu_count() or 1)
        fp8 = cfg.expert_dtype == "fp8"
        wdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[cfg.expert_dtype]
        I, Is, d = cfg.inter, cfg.inter_shared, cfg.d
        dev = self.device
        self.w13 = torch.empty((cfg.n_routed, 2 * I, d), dtype=wdt, device=dev)
        self.w2 = torch.empty((cfg.n_routed, d, I), dtype=wdt, device=dev)
        ns = max(cfg.n_shared, 1)
        self.w13s = torch.empty((ns, 2 * Is, d), dtype=wdt, device=dev)
        self.w2s = torch.empty((ns, d, Is), dtype=wdt, device=dev)
        self.s13 = self.s2 = self.s13s = self.s2s = None
        if fp8:
            self.s13 = torch.empty((cfg.n_routed, 2 * I // 128, d // 128), dtype=torch.float32, device=dev)
            self.s2 = torch.empty((cfg.n_routed, d // 128, I // 128), dtype=torch.float32, device=dev)
            self.s13s = torch.empty((ns, 2 * Is // 128, d // 128), dtype=torch.float32, device=dev)
            self.s2s = torch.empty((ns, d // 128, Is // 128), dtype=torch.float32, device=dev)
        src_dt = "bf16" if cfg.expert_dtype == "bf16" else "f32"

        def put(dst, sc, i, arr):
            if not fp8:
                dst[i].copy_(np_to_device(arr, src_dt, "cpu"))
                return
            master = np_to_device(arr, "f32", dev)
            L.moe_quantize_fp8(L.MOE_QUANT_W_128x128, master, master.shape[0], master.shape[1],
                               dst[i], sc[i])

        jobs = [(e, False) for e in range(cfg.n_routed)] + [(s, True) for s in range(cfg.n_shared)]

        def make(job):
            i, shared = job
            if shared:
                return job, gen.shared_w13(cfg, i), gen.shared_w2(cfg, i)
            return job, gen.expert_w13(cfg, i), gen.expert_w2(cfg, i)

        with ThreadPoolExecutor(threads) as ex:
            for (i, shared), a13, a2 in ex.map(make, jobs):
                if shared:
                    put(self.w13s, self.s13s, i, a13)
                    put(self.w2s, self.s2s, i, a2)
                else:
                    put(self.w13, self.s13, i, a13)
                    put(self.w2, self.s2, i, a2)
        torch.cuda.synchronize(dev)
        self.weights = L.make_weights(self.E, self.w13, self.w2,
                                      self.w13s if cfg.n_shared else None,
                                      self.w2s if cfg.n_shared else None,
                                      self.s13, self.s2,
                                      self.s13s if cfg.n_shared else None,
                                      self.s2s if cfg.n_shared else None)
        self.blocked = False
        if blocked_weights and cfg.expert_dtype in ("bf16", "fp8"):
            self._pack_weights()
        self.ws = torch.empty(L.moe_workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
        T, K = cfg.T, cfg.top_k
        self.idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty(cfg.n_routed, dtype=torch.int32, device=dev)
        iodt = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
        self.out = torch.empty((T, d), dtype=iodt, device=dev)

    def _pack_weights(self):
        sh = self.cfg.n_shared > 0
        blk = [torch.empty_like(t) for t in (self.w13, self.w2)] + \
              ([torch.empty_like(t) for t in (self.w13s, self.w2s)] if sh else [None, None])
        wb = L.make_weights(None, *blk)
        st = L.lib().moe_pack_expert_weights(ctypes.byref(self.desc), ctypes.byref(self.weights),
                                             ctypes.byref(wb), None)
        if st == L.MOE_ENOTSUP:
            return
        if st != L.MOE_OK:
            raise L.MoeError("moe_pack_expert_weights", st, L.lib())
        torch.cuda.synchronize(self.device)
        self._blk = blk
        w = self.weights
        w.w13_blk, w.w2_blk = blk[0].data_ptr(), blk[1].data_ptr()
        if sh:
            w.w13_shared_blk, w.w2_shared_blk = blk[2].data_ptr(), blk[3].data_ptr()
        self.blocked = True

    def forward(self, u: torch.Tensor, b: torch.Tensor, update_bias=True, stream=None):
        L.moe_forward(self.desc, self.weights, u, b, self.out, self.ws, update_bias,
                      self.idx, self.gate, self.counts, stream=stream)
        return self.out

    def forward_capacity(self, u: torch.Tensor, b: torch.Tensor, capacity: int, update_bias=True, stream=None):
        """forward() with each expert capped at `capacity` selections (the token-dropping baseline);
        self.keep [T, K] int32 and self.n_dropped [1] say what was kept."""
        if getattr(self, "_cap_ws", None) is None:
            dev = self.device
            self._cap_ws = torch.empty(L.moe_capacity_workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
            self.keep = torch.empty((self.cfg.T, self.cfg.top_k), dtype=torch.int32, device=dev)
            self.n_dropped = torch.empty(1, dtype=torch.int32, device=dev)
        L.moe_forward_capacity(self.desc, self.weights, u, b, self.out, self._cap_ws, capacity, update_bias,
                               self.keep, self.n_dropped, self.idx, self.gate, self.counts, stream=stream)
        return self.out

    def backward(self, u: torch.Tensor, b: torch.Tensor, dout: torch.Tensor, stream=None):
        """Gradients of forward(u, b) for the upstream gradient dout [T, d] (in_dtype), for the routing
        the forward chooses with this b: a dict of fp32 device tensors du [T, d], dE [N_r, d],
        dw13 [N_r, 2I, d], dw2 [N_r, d, I] (and dw13s, dw2s for the shared experts). The
        transposed weight copies and the gradient buffers are allocated on the first call."""
        cfg, dev = self.cfg, self.device
        if getattr(self, "_wt", None) is None:
            I, d, N, ns = cfg.inter, cfg.d, cfg.n_routed, max(cfg.n_shared, 1)
            wdt = self.w13.dtype                          # bf16, fp32 or E4M3 codes, as the experts
            self._w13t = torch.empty((N, d, 2 * I), dtype=wdt, device=dev)
            self._w2t = torch.empty((N, I, d), dtype=wdt, device=dev)
            self._w13st = torch.empty((ns, d, 2 * I), dtype=wdt, device=dev)
            self._w2st = torch.empty((ns, I, d), dtype=wdt, device=dev)
            sh = cfg.n_shared > 0
            sc = [None] * 4
            if cfg.expert_dtype == "fp8":                 # the block-scale grids, transposed with the codes
                f32 = torch.float32
                sc = [torch.empty((N, d // 128, 2 * I // 128), dtype=f32, device=dev),
                      torch.empty((N, I // 128, d // 128), dtype=f32, device=dev),
                      torch.empty((ns, d // 128, 2 * I // 128), dtype=f32, device=dev),
                      torch.empty((ns, I // 128, d // 128), dtype=f32, device=dev)]
                self._wt_scales = sc
            self._wt = L.make_weights(None, self._w13t, self._w2t, self._w13st if sh else None,
                                      self._w2st if sh else None, sc[0], sc[1],
                                      sc[2] if sh else None, sc[3] if sh else None)
            L.moe_transpose_expert_weights(self.desc, self.weights, self._wt, stream=stream)
            f32 = torch.float32
            self.grads = {
                "du": torch.empty((cfg.T, d), dtype=f32, device=dev),
                "dE": torch.empty((N, d), dtype=f32, device=dev),
                "dw13": torch.empty((N, 2 * I, d), dtype=f32, device=dev),
                "dw2": torch.empty((N, d, I), dtype=f32, device=dev),
                "dw13s": torch.empty((ns, 2 * I, d), dtype=f32, device=dev),
                "dw2s": torch.empty((ns, d, I), dtype=f32, device=dev),
            }
            g = self.grads
            self._grads = L.make_grads(g["du"], g["dE"], g["dw13"], g["dw2"], g["dw13s"] if sh else None,
                                       g["dw2s"] if sh else None)
            self._bws = torch.empty(L.moe_backward_workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
        L.moe_backward(self.desc, self.weights, self._wt, u, b, dout, self._grads, self._bws, stream=stream)
        return self.grads

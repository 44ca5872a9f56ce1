"""Device-side plumbing around the C ABI: weight upload, workspace, one call.

`MoELayer` owns device tensors (centroids, expert weights, FP8 codes and
scales, the workspace) and calls `moe_forward`. Weights arrive as numpy arrays
from a generator callback, one expert at a time, so a 22.5 GB bf16 stack never
needs a second full host copy. All arithmetic happens in libmoe_rocm.so.
"""

from concurrent.futures import ThreadPoolExecutor
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
    def __init__(self, cfg, gen, device="cuda", threads=0):
        """cfg: layer configuration (T, d, N_r, ... dtypes); gen: the input source, an object
        with centroids(cfg), expert_w13(cfg, e), expert_w2(cfg, e), shared_w13(cfg, s),
        shared_w2(cfg, s) returning numpy arrays (bf16 bits as uint16, or fp32)."""
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
        self.ws = torch.empty(L.moe_workspace_bytes(self.desc), dtype=torch.uint8, device=dev)
        T, K = cfg.T, cfg.top_k
        self.idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty(cfg.n_routed, dtype=torch.int32, device=dev)
        iodt = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
        self.out = torch.empty((T, d), dtype=iodt, device=dev)

    def forward(self, u: torch.Tensor, b: torch.Tensor, update_bias=True, stream=None):
        L.moe_forward(self.desc, self.weights, u, b, self.out, self.ws, update_bias,
                      self.idx, self.gate, self.counts, stream=stream)
        return self.out

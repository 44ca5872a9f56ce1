"""Layer configurations of the DeepSeekMoE FFN used by tests and the bench.

Shapes come from the DeepSeek-V3 Technical Report pages:
  * d = 7168 (zeeklog.com page, §3 "注意力机制参数");
  * 1 shared + 256 routed experts, 8 active (xyznot.com guides, key-ideas list);
  * 8 expert groups standing for the 8 nodes, at most M = 4 of them per token
    (zeeklog.com page §4 "节点受限路由"; pwwt.cn note §1.3 and §5);
  * each group ranked by the sum of its top K_r/M scores (pwwt.cn note §1.3);
  * gamma = 0.001 (xyznot.com guides, Método §2).
T, the intermediate sizes and the smaller configurations are workload choices
of this repository, named for what they are.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int          # first word of every seed of this workload
    T: int               # tokens per batch
    d: int               # hidden size
    n_routed: int        # N_r
    top_k: int           # K_r
    n_groups: int        # G (groups of n_routed/G contiguous experts); 1 = no limit
    topk_groups: int     # M, groups kept per token
    group_topk: int      # q = K_r/M, scores summed per group
    n_shared: int        # N_s
    inter: int           # I, routed expert intermediate size
    inter_shared: int    # I_s, shared expert intermediate size
    in_dtype: str        # dtype of u:  "f32" | "bf16"
    router_dtype: str    # dtype of the centroids: "f32" | "bf16"
    expert_dtype: str    # dtype of expert weights: "f32" | "bf16" | "fp8"
    gamma: float = 0.001
    group_score_biased: int = 1
    steps: int = 1
    bias_kind: str = "zero"        # "zero" | "uniform"  (U(-0.01, 0.01))
    centroid_kind: str = "normal"  # "normal" | "zipf"
    zipf_alpha: float = 2.0
    zipf_exponent: float = 1.1
    outlier_frac: float = 0.0      # fraction of u entries set to +-outlier_value
    outlier_value: float = 50.0
    weights_cfg_id: int = 0        # seed id of weights/centroids (0 = cfg_id)

    @property
    def wid(self) -> int:
        return self.weights_cfg_id or self.cfg_id

    @property
    def rows(self) -> int:
        return self.T * self.top_k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    # algorithmic work, per forward (SwiGLU = 3 matmuls per expert row)
    def flops(self) -> dict:
        router = 2.0 * self.T * self.d * self.n_routed
        routed = 2.0 * self.rows * self.d * self.inter * 3
        shared = 2.0 * self.T * self.d * self.inter_shared * 3 * self.n_shared
        return {"router": router, "routed": routed, "shared": shared,
                "total": router + routed + shared}


_V3 = dict(T=8192, d=7168, n_routed=256, top_k=8, n_groups=8, topk_groups=4,
           group_topk=2, n_shared=1, inter=2048, inter_shared=2048)

CONFIGS = {
    "tiny": MoEConfig("tiny", 1, T=64, d=256, n_routed=16, top_k=4, n_groups=4,
                      topk_groups=2, group_topk=2, n_shared=1, inter=128,
                      inter_shared=128, in_dtype="f32", router_dtype="f32",
                      expert_dtype="f32"),
    "mid": MoEConfig("mid", 2, T=4096, d=2048, n_routed=64, top_k=6, n_groups=1,
                     topk_groups=1, group_topk=6, n_shared=2, inter=1408,
                     inter_shared=1408, in_dtype="bf16", router_dtype="bf16",
                     expert_dtype="bf16", bias_kind="uniform"),
    "v3": MoEConfig("v3", 3, **_V3, in_dtype="bf16", router_dtype="bf16",
                    expert_dtype="bf16", steps=10),
    "skew": MoEConfig("skew", 4, **_V3, in_dtype="bf16", router_dtype="bf16",
                      expert_dtype="bf16", steps=200, centroid_kind="zipf"),
    "fp8": MoEConfig("fp8", 5, **_V3, in_dtype="bf16", router_dtype="f32",
                     expert_dtype="fp8", steps=10, outlier_frac=0.001),
    # decode-sized batches at the V3 shape, V3 weights and centroids
    "decode": MoEConfig("decode", 6, **{**_V3, "T": 256}, in_dtype="bf16",
                        router_dtype="bf16", expert_dtype="bf16", steps=20,
                        weights_cfg_id=3),
    # one GPU's share of the V3 layer under 8-way expert parallelism:
    # 32 experts (one group), every routed row of 8192 tokens x 8 lands here
    "ep_share": MoEConfig("ep_share", 7, T=8192, d=7168, n_routed=32, top_k=8,
                          n_groups=1, topk_groups=1, group_topk=8, n_shared=0,
                          inter=2048, inter_shared=2048, in_dtype="bf16",
                          router_dtype="bf16", expert_dtype="bf16"),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg

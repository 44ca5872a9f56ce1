"""CPU oracle for the DeepSeekMoE layer with auxiliary-loss-free balancing.

TEST INFRASTRUCTURE ONLY. Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import anything from this package. The
product path (the HIP library and its Python binding) never imports it, and
this package never imports the product path: they share no code, no tables and
no helpers. The only module both read is `workloads` (seeded input draws).

What it computes, and where the pages fix it (DeepSeek-V3 Technical Report
reading guides on xyznot.com, "Método"/"الطريقة" §2, and the pwwt.cn study
note, §1.1.2, §1.1.3, §1.3, §1.4, §3):
  * s = sigmoid(u . e_i)                          -- affinity, §2 of the guides
  * key = fl32(s + b)                             -- biased routing key, gating eq.
  * group-limited top-K on key                    -- note §1.3 (top K_r/M sum)
  * g = s_sel / sum(s_sel) from the unbiased s    -- note §1.1.2 step 3, guides §2
  * h' = u + sum shared FFN + sum_k g_k FFN_k(u)  -- output equation, guides §2
  * b <- b -/+ gamma from batch load              -- note §1.1.3, guides §2
Floating point is fp64 throughout, rounded to fp32 only at the points the
selection needs bit-for-bit (keys, group sums, bias). Readings of the points the
pages leave open are listed with each function.

Parity status: every function here is pinned by a `-m "not gpu"` test against
values fixed outside this package (hand cases with exact rationals, brute-force
enumeration, library routines, closed forms). The end-to-end FFN values have no
printed reference on the pages; they are pinned by special cases (dense
SwiGLU, zero weights, linearity in W2) only.
"""

from . import numerics, routing, ffn, permute, brute, balance, backward, capacity  # noqa: F401

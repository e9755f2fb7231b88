"""Writes tests/golden/lm_head_argmax.txt from the CPU oracle alone.

The NVFP4 language-model head over a 16-node verification tree (M=16,
K=5120, N=151936; weights N(0, 0.02^2), bf16 activations N(0, 1), seed 0):
the head is NVFP4 on the page "TensorRT Edge-LLM Completes the MLPerf Edge
Agentic Benchmark 6.4x Faster on Jetson AGX Thor" (section "Using NVFP4
quantization to accelerate Qwen3.6-27B inference"), and the 16 rows are one
verification pass over the candidate tree (section "Using tree-based
multi-token prediction to accelerate LLM inference").  At temperature 0 the
tree is accepted by comparing each node's argmax token, so the argmax must
match exactly.

For each row the file stores the oracle's argmax, the best and second-best
logits and the tolerance 1e-3 * sum_k |a_hat * w_hat| at the best column.
A second file, lm_head_admissible.txt, lists per row every column whose exact
logit lies within the two columns' tolerances of the exact maximum
(oracle.tree.admissible_argmax): the argmax a correct fp32 product may return.
Inputs come from the seeded generator; everything else from oracle/.

    python tests/golden/make_lm_head_golden.py      (about 3-4 minutes, ~8 GB RAM)
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from nvfp4_w4a4_block_amd import workloads as WL  # noqa: E402
from oracle import gemm as G  # noqa: E402
from oracle import quant as Q  # noqa: E402
from oracle import tree as TR  # noqa: E402

CHUNK = 2048


def main() -> None:
    wl = WL.get("lm_head")
    inp = WL.generate(wl)
    a = inp.a_f32()
    g_a = Q.global_scale(a)
    ap, asc = Q.quantize_packed(a, g_a)
    g_w = Q.global_scale(inp.W)
    C = np.empty((wl.M, wl.N))
    T = np.empty((wl.M, wl.N))
    for n0 in range(0, wl.N, CHUNK):
        wp, wsc = Q.quantize_packed(inp.W[n0:n0 + CHUNK], g_w)
        C[:, n0:n0 + CHUNK], T[:, n0:n0 + CHUNK] = G.gemm_ref(ap, asc, g_a, wp, wsc, g_w)
    top = G.argmax_rows(C)
    lines = [
        "# Oracle argmax of the NVFP4 LM head, M=16 K=5120 N=151936, seed 0 (see make_lm_head_golden.py).",
        f"# g_a = {float(g_a).hex()}  g_w = {float(g_w).hex()}",
        "# row ; argmax ; best logit ; second-best column ; second-best logit ; tol at best",
    ]
    for m in range(wl.M):
        row = C[m].copy()
        best = int(top[m])
        row[best] = -np.inf
        second = int(np.argmax(row))
        lines.append(f"{m} ; {best} ; {float(C[m, best])!r} ; {second} ; {float(C[m, second])!r} ; {float(T[m, best])!r}")
    with open(os.path.join(HERE, "lm_head_argmax.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    adm = TR.admissible_argmax(C, T)
    alines = [
        "# Admissible argmax columns of the NVFP4 LM head (M=16 K=5120 N=151936, seed 0): every column",
        "# whose oracle logit is within tol[column] + tol[argmax] of the row maximum (make_lm_head_golden.py).",
        "# row ; columns",
    ] + [f"{m} ; {' '.join(str(c) for c in sorted(adm[m]))}" for m in range(wl.M)]
    with open(os.path.join(HERE, "lm_head_admissible.txt"), "w") as f:
        f.write("\n".join(alines) + "\n")
    print("\n".join(alines))


if __name__ == "__main__":
    main()

"""Writes the hand-derived golden fixtures in this folder.

The expected values are closed forms worked out below from the definitions (no
library, oracle or GPU output is involved).  Run: python tests/golden/make_golden.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def dense_two_token():
    return {
        "source": "SkipKV Sec. 4.1 token importance score: softmax(q k^T / sqrt(d)); "
                  "output = weights applied to V",
        "derivation": "d=4 so scale=1/2. q=(1,0,0,0). k0=0 gives z0=0. k1=(2 ln 3,0,0,0) "
                      "gives z1=ln 3. weights = (1,3)/4, lse = ln 4. v0=(4,0,0,0), "
                      "v1=(0,4,0,0) so out=(1,3,0,0).",
        "d": 4, "q": [1.0, 0.0, 0.0, 0.0],
        "k": [[0.0, 0.0, 0.0, 0.0], [2.0 * math.log(3.0), 0.0, 0.0, 0.0]],
        "v": [[4.0, 0.0, 0.0, 0.0], [0.0, 4.0, 0.0, 0.0]],
        "expected_logits": [0.0, math.log(3.0)], "expected_lse": math.log(4.0),
        "expected_out": [1.0, 3.0, 0.0, 0.0],
        "tolerance": 1e-6,
        "tolerance_reason": "k1 is stored in fp32, so z1 carries a relative rounding "
                            "error near 6e-8",
    }


def select_lse_j():
    n_sink, n_recent, N = 4, 4, 18          # J = [4, 14), |J| = 10
    a, b = 6, 9
    e5, e1 = math.exp(5.0), math.exp(1.0)
    f_a = 0.5 * (e5 / (e5 + 9) + 1.0 / (e1 + 9))
    f_b = 0.5 * (1.0 / (e5 + 9) + e1 / (e1 + 9))
    f_other = 0.5 * (1.0 / (e5 + 9) + 1.0 / (e1 + 9))
    z0 = [30.0] * 4 + [0.0] * 10 + [30.0] * 4
    z0[a] = 5.0
    z1 = [0.0] * 18
    z1[b] = 1.0
    return {
        "source": "Slow-Fast Inference Sec. 3.2 (evidence: a per-head distribution over "
                  "the allowed positions J) and Sec. 3.3 (Top-K per KV head)",
        "derivation": "G=2, J=[4,14). Head 0: z=30 on sinks and recent, z=5 at j=6, 0 "
                      "elsewhere in J. Head 1: z=0 everywhere except z=1 at j=9. "
                      "Normalising each head over J: p0(6)=e^5/(e^5+9), p1(9)=e/(e+9); "
                      "f(j)=mean of the two. f(6)>f(9) so k_sel=1 keeps 6. Normalising "
                      "over all positions would give head 0 almost no mass on J and keep "
                      "9 instead.",
        "N": N, "n_sink": n_sink, "n_recent": n_recent, "k_sel": 1,
        "z_head0": z0, "z_head1": z1,
        "expected_idx": [0, 1, 2, 3, a],
        "expected_f_at": {str(a): f_a, str(b): f_b, "4": f_other},
        "tolerance": 1e-12,
    }


if __name__ == "__main__":
    for name, fn in [("dense_two_token", dense_two_token), ("select_lse_j", select_lse_j)]:
        with open(os.path.join(HERE, name + ".json"), "w") as fh:
            json.dump(fn(), fh, indent=1)

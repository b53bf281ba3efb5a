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


def select_soft_nms():
    # one KV head, G = 1, no sinks or recent window: J = [0, 6) and f = softmax(z) over J.
    # With z = ln f for an f that sums to one, the evidence is f itself.
    f = [0.30, 0.25, 0.05, 0.20, 0.05, 0.15]
    return {
        "source": "Slow-Fast Inference Sec. 3.3 (Soft-NMS within a head keeps the local maximum "
                  "of a neighbourhood and decays the lower-scoring candidates next to it, in "
                  "log-score space; Top-K per KV head)",
        "derivation": "f = (0.30, 0.25, 0.05, 0.20, 0.05, 0.15) on J = [0, 6), k_sel = 2, "
                      "no prior (lambda = 0), alpha_soft = 0.5, neighbourhood j-1 and j+1. "
                      "Local maxima: 0 (0.30 > 0.25), 3 (0.20 > 0.05, 0.05), 5 (0.15 > 0.05). "
                      "Position 1 has the higher neighbour 0 and drops to 0.125, positions 2 "
                      "and 4 drop to 0.025. Without Soft-NMS the two largest are {0, 1}; with "
                      "it they are {0, 3} (0.30, 0.20 > 0.15 > 0.125).",
        "N": 6, "n_sink": 0, "n_recent": 0, "k_sel": 2, "alpha_soft": 0.5,
        "z": [math.log(x) for x in f],
        "expected_idx_plain": [0, 1],
        "expected_idx": [0, 3],
        "expected_refined": [math.log(0.30), math.log(0.125), math.log(0.025),
                             math.log(0.20), math.log(0.025), math.log(0.15)],
        "tolerance": 1e-12,
    }


def select_cross_head():
    # two KV heads with one query head each (G = 1), J = [0, 4), f_h = softmax(z_h) = f_h
    fa = [0.35, 0.32, 0.23, 0.10]
    fb = [0.36, 0.31, 0.05, 0.28]
    keep = 1.0 - 0.35
    ra = [fa[0] * keep, fa[1], fa[2], fa[3] * keep]
    rb = [fb[0], fb[1] * keep, fb[2] * keep, fb[3]]
    return {
        "source": "Slow-Fast Inference Sec. 3.3 (cross-head exclusivity: a soft competition "
                  "across heads at each fixed position, in log-score space, before Top-K)",
        "derivation": "f_A = (0.35, 0.32, 0.23, 0.10), f_B = (0.36, 0.31, 0.05, 0.28), "
                      "k_sel = 2, lambda = alpha_soft = 0, alpha_cross = 0.35. At j = 0 head B "
                      "is larger, so A's score is multiplied by 0.65; at j = 1 and j = 2 head A "
                      "is larger, so B's are; at j = 3 B is larger. Refined A = (0.2275, 0.32, "
                      "0.23, 0.065), B = (0.36, 0.2015, 0.0325, 0.28). Without exclusivity "
                      "both heads keep {0, 1}; with it A keeps {1, 2} and B keeps {0, 3}.",
        "N": 4, "n_sink": 0, "n_recent": 0, "k_sel": 2, "alpha_cross": 0.35,
        "z_head0": [math.log(x) for x in fa], "z_head1": [math.log(x) for x in fb],
        "expected_idx_plain": [[0, 1], [0, 1]],
        "expected_idx": [[1, 2], [0, 3]],
        "expected_refined": [[math.log(x) for x in ra], [math.log(x) for x in rb]],
        "tolerance": 1e-12,
    }


if __name__ == "__main__":
    for name, fn in [("dense_two_token", dense_two_token), ("select_lse_j", select_lse_j),
                     ("select_soft_nms", select_soft_nms), ("select_cross_head", select_cross_head)]:
        with open(os.path.join(HERE, name + ".json"), "w") as fh:
            json.dump(fn(), fh, indent=1)

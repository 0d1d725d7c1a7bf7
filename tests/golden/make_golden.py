"""Write the closed-form fixtures of tests/golden/ (run: python make_golden.py).

Every expected value here comes from the mathematics of a small hand-worked
case, evaluated with Python's math module: nothing is imported from the
oracle or the HIP library, so the fixtures pin both from the outside.  All
inputs are exact in bf16 (a few significant bits), so both sides read the
same numbers.  Each fixture names the page and section its operation comes
from and states its derivation.
"""
from __future__ import annotations

import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _dump(name, obj):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(obj, f, indent=1)
        f.write("\n")


def rmsnorm_constant():
    D, c, eps = 8, 0.5, 1e-6
    w = [1.0, 2.0, 0.5, -1.0, 0.25, 1.5, 3.0, -0.75]
    r = 1.0 / math.sqrt(c * c + eps)            # mean(x^2) = c^2 for x = c * 1
    _dump("rmsnorm_constant.json", {
        "source": "cutileGPT README, Why tiles (RMSNorm figure: rstd = 1/sqrt(sum(x*x)/N + eps), y = x*rstd*w)",
        "derivation": "x = c*1 over D elements: mean(x^2) = c^2, so y_i = c * w_i / sqrt(c^2 + eps)",
        "D": D, "x": [c] * D, "w": w, "eps": eps,
        "y": [c * r * wi for wi in w],
    })


def rope_neox_d4():
    x, theta, pos = [1.0, 2.0, 3.0, 4.0], 4.0, 3
    f = [1.0, 4.0 ** -0.5]                      # theta^(-2i/D), i = 0, 1, D = 4
    a = [pos * fi for fi in f]
    y = [x[0] * math.cos(a[0]) - x[2] * math.sin(a[0]),
         x[1] * math.cos(a[1]) - x[3] * math.sin(a[1]),
         x[2] * math.cos(a[0]) + x[0] * math.sin(a[0]),
         x[3] * math.cos(a[1]) + x[1] * math.sin(a[1])]
    _dump("rope_neox_d4.json", {
        "source": "fusedtok 1.0.1 README, Operators (RoPE: NeoX layout) and Usage (rope with pos_offset, neox=True)",
        "derivation": "NeoX pairs (i, i + D/2) rotate by pos * theta^(-2i/D); D = 4, theta = 4 gives frequencies 1 and 1/2",
        "reading": "the pages name the layout but print no frequency schedule (parity unpinned beyond this standard reading)",
        "x": x, "theta": theta, "pos": pos, "y": y,
    })


def attention_two_keys():
    # D = 64 so that the HIP kernels (D in {64, 128}) run the same case.
    D, a, b = 64, 1.5, -0.25
    q = [0.0] * D
    q[0] = 1.0
    K = [[0.0] * D for _ in range(2)]
    K[0][0], K[1][0] = a, b
    V = [[((j % 7) - 3) * 0.25 + (0.5 if r else 0.0) for j in range(D)] for r in range(2)]
    ea, eb = math.exp(a), math.exp(b)
    out = [(ea * V[0][j] + eb * V[1][j]) / (ea + eb) for j in range(D)]
    _dump("attention_two_keys.json", {
        "source": "fusedtok 1.0.1 README, Operators (attention_decode: single-token attention, online softmax)",
        "derivation": "q = e_0 and scale = 1 give scores a and b; softmax weights e^a/(e^a+e^b), e^b/(e^a+e^b); lse = ln(e^a + e^b)",
        "D": D, "scale": 1.0, "q": q, "K": K, "V": V,
        "out": out, "lse": math.log(ea + eb),
    })


def attention_identical_keys():
    D, n = 64, 5
    q = [((j % 5) - 2) * 0.5 for j in range(D)]
    k = [((j % 3) - 1) * 0.25 for j in range(D)]
    V = [[(((r * 13 + j) % 9) - 4) * 0.125 for j in range(D)] for r in range(n)]
    s = sum(qi * ki for qi, ki in zip(q, k)) / math.sqrt(D)
    _dump("attention_identical_keys.json", {
        "source": "fusedtok 1.0.1 README, Operators (attention_decode); softmax scale 1/sqrt(D), the reading of the unstated scale",
        "derivation": "n identical keys give equal weights 1/n: out = mean of the V rows, lse = s + ln n with s = <q,k>/sqrt(D)",
        "D": D, "n": n, "q": q, "k": k, "V": V,
        "out": [sum(V[r][j] for r in range(n)) / n for j in range(D)],
        "lse": s + math.log(n),
    })


def split_merge_two_parts():
    # Two partitions with known (o_k, lse_k); the merge is the weighted mean.
    o1, l1 = [1.0, -2.0, 0.5, 4.0], 0.75
    o2, l2 = [3.0, 0.0, -1.0, 2.0], -1.25
    m = max(l1, l2)
    w1, w2 = math.exp(l1 - m), math.exp(l2 - m)
    _dump("split_merge_two_parts.json", {
        "source": "fusedtok 1.0.1 README, Operators (attention_decode: flash-decoding split over long caches)",
        "derivation": "out = (e^l1 o1 + e^l2 o2)/(e^l1 + e^l2), lse = ln(e^l1 + e^l2), with the larger lse factored out",
        "o": [o1, o2], "lse_parts": [l1, l2],
        "out": [(w1 * a + w2 * b) / (w1 + w2) for a, b in zip(o1, o2)],
        "lse": m + math.log(w1 + w2),
    })


if __name__ == "__main__":
    rmsnorm_constant()
    rope_neox_d4()
    attention_two_keys()
    attention_identical_keys()
    split_merge_two_parts()

"""Write ``geometric_weights.json``: closed-form attention cases with exact answers.

The expected outputs come from the mathematics alone (Python ``fractions``),
not from the oracle or the GPU path.

Construction (definition: "Hand-written Masked Multi-Head Attention CUDA
kernel" page, section 2; causal visibility j <= i: same page, section 2.2):
with D = 4 the scale is 1/sqrt(4) = 1/2. Take every query of head h equal to
[2 (h+1) ln 2, 0, 0, 0] and key j equal to [j, 0, 0, 0]. Then the scaled
score is s_ij = (h+1) j ln 2, so exp(s_ij) = r^j with r = 2^(h+1), and the
softmax weight of key j among the visible keys J_i is r^j / sum_{t in J_i} r^t:
a ratio of integers. With value rows v_j = c_b * [1, j, (-1)^j, 2^-j]
(c_b = b + 1) every output is a rational number, stored here exactly. The
log-sum-exp of row i is ln(sum_{t in J_i} r^t), the log of an integer,
stored to double precision (-inf for a row that sees no key).

KV-cache cases give entry b only its first len_b keys (k, v then hold S_cap
rows); query i of entry b sits at position len_b - S_q + i, and a query that
sees no key has an all-zero output row.

Run from the repository root: ``python tests/golden/make_golden.py``.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def value_row(b: int, j: int):
    c = Fraction(b + 1)
    return [c, c * j, c * (-1) ** j, c * Fraction(1, 2 ** j)]


def case(name, B, H, S_q, S_kv, causal, seqlens=None):
    D = 4
    q = [[[[2.0 * (h + 1) * math.log(2.0), 0.0, 0.0, 0.0] for h in range(H)]
          for _ in range(S_q)] for _ in range(B)]
    k = [[[[float(j), 0.0, 0.0, 0.0] for _ in range(H)] for j in range(S_kv)] for _ in range(B)]
    v = [[[[float(x) for x in value_row(b, j)] for _ in range(H)] for j in range(S_kv)]
         for b in range(B)]
    o = []
    lse = [[[None] * S_q for _ in range(H)] for _ in range(B)]
    for b in range(B):
        n = S_kv if seqlens is None else seqlens[b]   # valid keys of entry b
        off = n - S_q
        rows = []
        for i in range(S_q):
            heads = []
            for h in range(H):
                r = Fraction(2) ** (h + 1)
                vis = [j for j in range(n) if (not causal) or j <= i + off]
                if not vis:
                    heads.append(["0"] * D)
                    lse[b][h][i] = "-inf"
                    continue
                den = sum(r ** j for j in vis)   # an integer
                lse[b][h][i] = repr(math.log(den.numerator))
                out = []
                for d in range(D):
                    num = sum(r ** j * value_row(b, j)[d] for j in vis)
                    out.append(str(num / den))
                heads.append(out)
            rows.append(heads)
        o.append(rows)
    doc = {"name": name, "B": B, "H": H, "S_q": S_q, "S_kv": S_kv, "D": D,
           "causal": causal, "q": q, "k": k, "v": v, "o_exact": o, "lse_exact": lse}
    if seqlens is not None:
        doc["seqlens"] = list(seqlens)
    return doc


def main():
    doc = {
        "citation": "Masked MHA page section 2 (A = softmax(QK^T/sqrt(d_k) + M), O = A.V) "
                    "and section 2.2 (key j visible to query i iff j <= i); "
                    "bottom-right alignment for S_q < S_kv is this project's reading.",
        "derivation": __doc__,
        "cases": [
            case("causal_square", 1, 1, 6, 6, True),
            case("causal_bottom_right", 1, 1, 2, 6, True),
            case("non_causal", 1, 1, 2, 6, False),
            case("causal_two_batches_two_heads", 2, 2, 5, 5, True),
            case("kvcache_causal_lengths", 3, 2, 3, 7, True, seqlens=[7, 4, 2]),
            case("kvcache_non_causal_lengths", 2, 1, 2, 5, False, seqlens=[5, 3]),
            case("kvcache_empty_entry", 2, 1, 2, 4, True, seqlens=[0, 4]),
        ],
    }
    with open(os.path.join(HERE, "geometric_weights.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()

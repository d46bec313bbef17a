"""Writes uniform_attention.json: exact closed-form values of one step under
uniform attention, computed with rational arithmetic only (no oracle code).

With every key equal to zero all logits are 0, so query row i of the chunk
spreads weight 1/(n + i + 1) over its n cache slots and chunk tokens 0..i
(causal GQA attention over cache + chunk, as in "Learning how to Forget:
Fine-tuning for Long-Context Sparse Attention", Chinese translation page,
§1 contributions: the kernel returns the summed attention weights).
With H(x) = sum_{k=1..x} 1/k the summed weights of a KV head with G query
heads are

    cache slot j < n      : G * (H(n + S) - H(n))
    empty slot n <= j < C : 0
    chunk token t         : G * (H(n + S) - H(n + t))

and the log-sum-exp of row i is ln(n + i + 1).
Run:  python tests/golden/make_uniform_golden.py
"""
import json
import os
from fractions import Fraction


def harmonic(x):
    return sum((Fraction(1, k) for k in range(1, x + 1)), Fraction(0))


def case(n, S, G, C):
    full = harmonic(n + S)
    cache = G * (full - harmonic(n))
    chunk = [G * (full - harmonic(n + t)) for t in range(S)]
    return {
        "n_valid": n, "chunk_len": S, "group": G, "cache_len": C,
        "cache_slot_wsum": [cache.numerator, cache.denominator],
        "chunk_wsum": [[c.numerator, c.denominator] for c in chunk],
        "lse_exp": [n + i + 1 for i in range(S)],
    }


def main():
    cases = [case(0, 8, 2, 32), case(8, 8, 2, 32), case(24, 8, 4, 32),
             case(32, 8, 4, 32), case(100, 5, 3, 128)]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "uniform_attention.json")
    with open(path, "w") as f:
        json.dump({"source": "closed form, exact rationals; see module docstring "
                             "of make_uniform_golden.py",
                   "cases": cases}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

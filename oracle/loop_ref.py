"""Pure-Python loop version of the decode step, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.sparse_decode``).  It is a
second, independent write-up of the same definitions -- exact rationals
for the int8 codes, plain integer loops for scores, an explicit sort for
the selection and a sum over a Python set for the attention -- used to
cross-check the vectorised oracle on small random cases.  Sources are the
same passages cited in ``oracle.sparse_decode``.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction
from typing import List, Sequence, Tuple


def bf16_value(bits: int) -> float:
    """Exact value of a bf16 bit pattern (as a Python float)."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def round_half_even(x: Fraction) -> int:
    f = math.floor(x)
    r = x - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def code(x_bits: int, scale: float) -> int:
    """Exact rational symmetric int8 code of one bf16 value."""
    if scale == 0:
        return 0
    return round_half_even(Fraction(127) * Fraction(bf16_value(x_bits)) / Fraction(scale))


def step(q_bits, k_bits, v_bits, length: int, G: int,
         stages: Sequence[Tuple[int, int, int]], sink: int, window: int,
         scale: float):
    """One request, all KV heads.  q_bits [Hq][d], k_bits/v_bits [Hkv][>=L][d]
    as nested lists or arrays of ints.  Returns (codes, kept, T, out)."""
    Hq, d = len(q_bits), len(q_bits[0])
    Hkv = Hq // G
    # query codes
    q8 = []
    for h in range(Hq):
        amax = max(abs(bf16_value(x)) for x in q_bits[h])
        q8.append([code(x, amax) for x in q_bits[h]])
    kept_all, T_all, k8_all = [], [], []
    out = [[0.0] * d for _ in range(Hq)]
    for j in range(Hkv):
        amax = 0.0
        for t in range(length):
            for c in range(d):
                amax = max(amax, abs(bf16_value(k_bits[j][t][c])))
        k8 = [[code(k_bits[j][t][c], amax) for c in range(d)] for t in range(length)]
        k8_all.append(k8)

        def S(t):
            return sum(q8[h][c] * k8[t][c] for h in range(j * G, (j + 1) * G) for c in range(d))

        cands = list(range(0, length, stages[0][0]))
        kept_stages = []
        for s, (c_s, r_s, keep) in enumerate(stages):
            scored = []
            for x in cands:
                best = None
                t = x
                while t < x + c_s and t < length:
                    v = S(t)
                    best = v if best is None or v > best else best
                    t += r_s
                scored.append((best, x))
            scored.sort(key=lambda p: (-p[0], p[1]))
            kept = sorted(x for _, x in scored[:keep])
            kept_stages.append(kept)
            if s + 1 < len(stages):
                c_n = stages[s + 1][0]
                cands = [x + i * c_n for x in kept for i in range(c_s // c_n) if x + i * c_n < length]
        T = set()
        for x in kept_stages[-1]:
            T.update(range(x, min(x + stages[-1][0], length)))
        T.update(range(0, min(sink, length)))
        T.update(range(max(0, length - window), length))
        T = sorted(T)
        kept_all.append(kept_stages)
        T_all.append(T)
        for h in range(j * G, (j + 1) * G):
            qv = [bf16_value(x) for x in q_bits[h]]
            z = {t: scale * sum(qv[c] * bf16_value(k_bits[j][t][c]) for c in range(d)) for t in T}
            m = max(z.values())
            w = {t: math.exp(z[t] - m) for t in T}
            tot = sum(w.values())
            for c in range(d):
                out[h][c] = sum(w[t] * bf16_value(v_bits[j][t][c]) for t in T) / tot
    return dict(q8=q8, k8=k8_all, kept=kept_all, T=T_all, out=out)

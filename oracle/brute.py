"""Pure-Python brute force for tiny MLA shapes (TEST INFRASTRUCTURE ONLY).

Loops over lists of Python floats, no numpy, so that the vectorised oracle in
``mla_oracle.py`` can be checked against an independent transcription of the
same definitions:

* [V3-src] "深度解读DeepSeek：源码解读 DeepSeek-V3", section "MLA",
  subsection "(a) Naive实现": per head, key = (W_UK c_t) followed by k_pe_t,
  value = W_UV c_t; softmax over positions of q.k * scale; output sum p v.
* [V2L] "DeepSeek-V2-Lite 模型结构详解" §四 RMSNorm: row rule
  x / sqrt(mean(x^2) + eps) * w.

Inputs are already plain floats (the caller widens bf16 exactly).
"""
from __future__ import annotations

import math


def decode_brute(q, kv_b, rows, length, q_len, nope, rope, v_dim, scale):
    """q[i][h][d] (nope+rope), kv_b[row][c] with row = h*(nope+v_dim)+d,
    rows[t][c] (latent+rope) in logical order.  Returns out[i][h][d]."""
    n_heads = len(q[0])
    latent = len(kv_b[0])
    out = []
    for i in range(q_len):
        out_i = []
        for h in range(n_heads):
            base = h * (nope + v_dim)
            scores = []
            for t in range(length):
                if t > length - q_len + i:
                    scores.append(None)
                    continue
                key = []
                for d in range(nope):
                    key.append(sum(kv_b[base + d][c] * rows[t][c] for c in range(latent)))
                for d in range(rope):
                    key.append(rows[t][latent + d])
                scores.append(sum(q[i][h][d] * key[d] for d in range(nope + rope)) * scale)
            mx = max(s for s in scores if s is not None)
            ex = [0.0 if s is None else math.exp(s - mx) for s in scores]
            den = sum(ex)
            o = []
            for d in range(v_dim):
                acc = 0.0
                for t in range(length):
                    if ex[t] == 0.0:
                        continue
                    val = sum(kv_b[base + nope + d][c] * rows[t][c] for c in range(latent))
                    acc += ex[t] / den * val
                o.append(acc)
            out_i.append(o)
        out.append(out_i)
    return out


def rmsnorm_brute(x, w, eps):
    """One row: x / sqrt(mean(x^2) + eps) * w, in Python floats."""
    ms = sum(v * v for v in x) / len(x)
    r = math.sqrt(ms + eps)
    return [x[j] / r * w[j] for j in range(len(x))]

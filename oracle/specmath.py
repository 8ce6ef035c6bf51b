"""A fully specified float32 exp / sigmoid used to take routing decisions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Routing with sigmoid scores ranks experts by sigmoid(logit) + bias
(vLLM PR 65207, Purpose, commit 1 names AITER's biased grouped top-k).  The
chosen expert indices must agree bit for bit between this oracle and the GPU,
so the score is computed by a routine whose every step is an IEEE-754 float32
operation with a single correct rounding, written from this recipe (both sides
implement it independently):

1. clamp x to [-80, 80] (keeps every intermediate and the sigmoid normal);
2. n = rint(x * log2(e))  (float32 multiply, round-half-even);
3. Cody & Waite (1980) two-constant reduction r = (x - n*LN2_HI) - n*LN2_LO,
   LN2_HI = 45426 / 2^16 (16 significant bits, so n*LN2_HI is exact for
   |n| < 2^8) and LN2_LO = float32(ln 2 - LN2_HI);
4. p = degree-7 Taylor polynomial of e^r, coefficients float32(1/j!),
   evaluated by Horner with a separate multiply and add per step (no fused
   multiply-add);
5. exp = p * 2^n (exact);
6. sigmoid(x) = 1 / (1 + exp(-x)) with float32 add and correctly rounded
   float32 division.

|r| <= ln(2)/2 so the truncated series term is below 2^-27 relative; the
routine is within a few ulp of the true exponential (checked by the tests).
"""

import numpy as np

_F = np.float32
CLAMP = _F(80.0)
LOG2E = _F(1.4426950408889634)
LN2_HI = _F(45426.0 / 65536.0)
LN2_LO = _F(0.6931471805599453 - 45426.0 / 65536.0)
# 1/j! for j = 0..7
_COEF = [_F(1.0), _F(1.0), _F(1.0 / 2), _F(1.0 / 6), _F(1.0 / 24), _F(1.0 / 120),
         _F(1.0 / 720), _F(1.0 / 5040)]


def spec_exp(x):
    """float32 exp by the recipe above; returns float32."""
    x = np.clip(np.asarray(x, dtype=np.float32), -CLAMP, CLAMP).astype(np.float32)
    n = np.rint(x * LOG2E).astype(np.float32)
    r = ((x - n * LN2_HI) - n * LN2_LO).astype(np.float32)
    p = _COEF[7]
    for j in range(6, -1, -1):
        p = (p * r).astype(np.float32)
        p = (p + _COEF[j]).astype(np.float32)
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def spec_sigmoid(x):
    """float32 logistic function 1 / (1 + spec_exp(-x)); returns float32."""
    x = np.asarray(x, dtype=np.float32)
    d = (_F(1.0) + spec_exp(-x)).astype(np.float32)
    return (_F(1.0) / d).astype(np.float32)

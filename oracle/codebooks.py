"""Value tables of the two 4-bit formats (oracle; test infrastructure only).

NF4: the pages name a 16-entry codebook decoded through a LUT
("grouped-nf4-gemm 0.33.1", opening description) but never print its values.
The values are the NF4 data type of the QLoRA paper (Dettmers et al. 2023,
appendix E), the same table bitsandbytes stores; the fp32 bit patterns below
are the authority. `nf4_table_closed_form` restates the paper's construction
(normal quantiles, asymmetric so that zero is exact) as an independent pin: it
agrees with the table to about 2e-7, not bit for bit.

MXFP4: OCP Microscaling Formats v1.0. An e2m1 element has 1 sign, 2 exponent
bits (bias 1) and 1 mantissa bit; exponent field 0 is subnormal (value m/2).
An e8m0 scale byte x means 2^(x-127); x = 255 is NaN.
"""
from __future__ import annotations

import math
import numpy as np

# NF4 table, index 0..15, as fp32 bit patterns.
NF4_TABLE_BITS = np.array([
    0xBF800000, 0xBF3239B1, 0xBF066B30, 0xBECA32A0,
    0xBE91A24D, 0xBE3D353F, 0xBDBA7871, 0x00000000,
    0x3DA2FAFF, 0x3E24CAE3, 0x3E7C04DD, 0x3EAD033A,
    0x3EE1A4B8, 0x3F1007AB, 0x3F3913B3, 0x3F800000,
], dtype=np.uint32)
NF4_TABLE_F32 = NF4_TABLE_BITS.view(np.float32)


def nf4_table_closed_form() -> np.ndarray:
    """NF4 construction from QLoRA appendix E, in fp64.

    Offset delta = 1 - (1/32 + 1/30)/2. Positive half: standard-normal quantiles
    of 9 points evenly spaced from delta down to 0.5, the last (zero) dropped.
    Negative half: negated quantiles of 8 such points, last dropped. Add an
    exact 0, sort, and divide by the largest value.
    """
    from scipy.stats import norm
    delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    return v / v.max()


def e2m1_value(code: int) -> float:
    """OCP e2m1 element value of a 4-bit code (sign bit 3, exponent bits 2..1,
    mantissa bit 0, exponent bias 1; exponent 0 encodes m * 0.5)."""
    code = int(code) & 0xF
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return math.copysign(mag, s)  # code 8 is -0.0


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(x) -> np.ndarray:
    """OCP e8m0 scale: 2^(x-127), NaN for x = 255. Exact in fp64."""
    x = np.asarray(x, dtype=np.int64)
    out = np.ldexp(np.ones(x.shape, dtype=np.float64), (x - 127).astype(np.int32))
    return np.where(x == 255, np.nan, out)

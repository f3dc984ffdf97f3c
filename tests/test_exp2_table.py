"""The constant table 2^(j/256) read by the acceptance kernels' fp64 exp:
256 entries, each within half an ulp of the exact value (checked in decimal
arithmetic at 80 digits, independent of how the table was written)."""

import math
import os
import re
from decimal import Decimal, getcontext

HDR = os.path.join(os.path.dirname(__file__), '..', 'block_draft_verification_spec_amd', 'csrc',
                   'exp2_table.h')


def _entries():
    body = open(HDR).read().split('{', 1)[1].split('}', 1)[0]
    return [float.fromhex(t) for t in re.findall(r'0x[0-9a-fA-Fp.+-]+', body)]


def test_table_is_correctly_rounded():
    vals = _entries()
    assert len(vals) == 256
    getcontext().prec = 80
    for j, d in enumerate(vals):
        exact = Decimal(2) ** (Decimal(j) / 256)
        half_ulp = Decimal(math.ulp(d)) / 2
        assert abs(Decimal(d) - exact) <= half_ulp, j
    assert vals[0] == 1.0 and vals[128] == float.fromhex('0x1.6a09e667f3bcdp+0')  # sqrt(2)

"""Compiled-code checks (CPU only: hipcc cross-compiles for gfx950).

Every kernel of the library keeps its working set in registers: the
compiler's resource-usage remarks must report no scratch memory and no
spilled vector registers for any of them (scalar registers spilled into
vector-register lanes are not memory traffic and are allowed).  The list of
kernels is also pinned against the variants the C ABI dispatches to: the
vector-ALU decode is built for 1, 2 and 4 heads per group (16-bit types)
and 1 (fp32) only, the sizes that fit without spilling; the matrix-core
decode for 1-16 heads and for 32 and 64 (column-split groups); other
groups run as virtual groups of those."""
import re

import pytest

from paged_kv_cache_196_amd import build


@pytest.fixture(scope="module")
def usage():
    return build.resource_usage()


def _decode(usage):
    out = {}
    for sym, u in usage.items():
        m = re.match(r"_ZN2pa13decode_kernelINS_\d(F32|F16|BF16)ELi(\d+)ELi(\d+)ELb([01])E", sym)
        if m:
            out[(m.group(1), int(m.group(2)), int(m.group(3)), m.group(4) == "1")] = u
    return out


def test_no_kernel_spills(usage):
    assert len(usage) > 50
    bad = {sym: (u.get("ScratchSize"), u.get("VGPRSpill")) for sym, u in usage.items()
           if u.get("ScratchSize", -1) != 0 or u.get("VGPRSpill", -1) != 0}
    assert not bad, bad
    assert all(u["VGPRs"] <= 256 for u in usage.values())


def test_decode_variants_built(usage):
    dec = _decode(usage)
    want = set()
    for B in (16, 32):
        for t in ("F16", "BF16"):
            want |= {(t, B, G, True) for G in (1, 2, 4, 8, 16, 32, 64)}
            want |= {(t, B, G, False) for G in (1, 2, 4)}
        want.add(("F32", B, 1, False))
    assert set(dec) == want
    shared = [s for s in usage if s.startswith("_ZN2pa20decode_shared_kernel")]
    prefill = [s for s in usage if s.startswith("_ZN2pa14prefill_kernel")]
    assert len(shared) == 2 * 2 * 4 and len(prefill) == 2 * 2 * 5

"""Which merge paths of the stream-form combine the attention parity cases
reach on a 256-CU part (MI355X), worked out on the host with the kernel's cut
rule (harness.stream_plan / stream_grid / stream_units):

* a unit cut once: its two pieces are loaded together with the range's record;
* a unit over three or more ranges: its other pieces are listed from the record;
* one sequence on a whole number of ranges per unit, every range holding tiles
  of its unit: the pieces are taken without a record;
* the same grid with some ranges holding no tile of their unit: the unit's
  first cut range is found among its ranges' records;
* more than 64 sequences: the range search over the LDS table instead of the
  wave-ballot search.

Every parity case runs with the stream form forced (and with the automatic
choice), so this pins that a change of the cases, or of the cut rule, cannot
leave one of these paths untested on the GPU."""
import numpy as np

import harness as H
import test_gpu_parity as P

CUS = 256


def _bf16_cases():
    cases = [(name, over, np.asarray(lens, np.int64)) for name, over, lens in P.ATTN_CASES]
    for name, over, lmax in P.MANY_CASES:
        cases.append((name, over, None))  # lengths drawn in the test; only B matters here
    return [(n, o, l) for n, o, l in cases if o.get("dtype") == "bf16"]


def _paths(over, lens):
    B, T, Hq, Hkv = over["B"], over["M"] + 1, over["Hq"], over["Hkv"]
    found = set()
    if B > 64:
        found.add("lds-search")
    if lens is None:
        return found
    nqb, _, _, pc = H.stream_plan(B, T, Hq, Hkv, CUS, int(lens.max()), over["D"])
    units = Hkv * nqb
    if B == 1 and units <= CUS and 10 * units * (CUS // units) >= 9 * CUS:
        rpu = CUS // units
        ntl = (int(lens[0]) + H.KT - 1) // H.KT + (T + H.KT - 1) // H.KT
        found.add("whole-ranges" if (ntl + pc) // rpu >= pc + 2 else "whole-ranges-fallback")
        return found
    for u in H.stream_units(B, T, Hq, Hkv, lens, CUS, D=over["D"]):
        if len(u.cuts) == 1:
            found.add("cut-once")
        elif len(u.cuts) >= 2:
            found.add("three-or-more-ranges")
    return found


def test_parity_cases_reach_every_combine_path():
    reached = {}
    for name, over, lens in _bf16_cases():
        for p in _paths(over, lens):
            reached.setdefault(p, []).append(name)
    for p in ["cut-once", "three-or-more-ranges", "whole-ranges", "whole-ranges-fallback", "lds-search"]:
        assert p in reached, f"no attention parity case reaches the stream combine's {p} path"

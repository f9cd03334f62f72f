"""Writes nf4_codebook.txt: the fixed 16-entry NF4 table both sides take as input.

Run from the repository root: ``python tests/golden/make_codebook.py``.
The table comes from ``synth.nf4_codebook`` (normal quantiles, P_MAX = 0.97);
the file freezes it so that a change of the generator is caught by the tests.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

cb = synth.nf4_codebook()
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "nf4_codebook.txt"), "w") as f:
    f.write("# NF4 codebook (fp32, exact hex), index 0..15; normal quantiles, P_MAX = %r\n" % synth.P_MAX)
    for i, c in enumerate(cb):
        f.write("%s  # %d  %.9g\n" % (float(c).hex(), i, float(c)))

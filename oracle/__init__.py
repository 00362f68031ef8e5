"""CPU float64 oracle for Windowed-MTP draft and verify attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it. It shares no code with the HIP library
(no kernels, headers, helpers, tables or pre/post-processing) and does not
import it.

Sources (the three web pages on arXiv 2607.21535, cited by title and part):

* [VERDICT] pith.science review page "Windowed-MTP" (arXiv 2607.21535):
  fields *key machinery*, *core discovery*, *referee report* (major comment on
  App. B / Table 7 / Eq. 1, minor comments on Eq. 3 / Table 1 and on the
  App. A pseudocode), *forward implications*, *falsifier*.
* [NOTES] "Weekly Paper Notes" TL;DR page on Windowed-MTP (sparsenotes).
* [ABSTRACT] field-notes entry "Windowed-MTP: Removing the Full-Context
  Draft-KV Tax at Million-Token Context", section *English abstract*.

Modules
-------
``attention``   plain attention (two-pass softmax) over an explicit key set:
                full draft, windowed draft (sink + recent), causal verify,
                split combine.
``ring``        the draft-KV ring buffer slot mapping and its state after
                any sequence of appends (pure Python).
``fp8``         OCP e4m3 storage of the draft KV: the quantizer and the values
                of the 8-bit codes.
``accounting``  the per-step cost identity (Eq. 1), the two readings of the
                cost reduction, the dropped-entry and reclaimed-KV fractions.

Every function states which passage it follows.  Where the pages leave a step
open, the reading taken is stated in the function's docstring.
"""

from . import accounting, attention, ring  # noqa: F401

"""Plain, slow, fp64 CPU oracle for grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library in ``gqa_flashattention_amd/``; the two meet only
through the seeded input generator, which holds none of the method's
arithmetic.

Sources.  The pages are five revisions of one design record, "ADR-0060: AHBM
GQA Fused Attention Kernel (Llama3-70B)" of the kernbench2 project.  They are
cited as ``ADR-0060@<commit>`` plus a section; ``@5a76ed4`` is the newest
revision and the one followed where revisions differ; ``ADR-001@1897945`` is
the oldest draft.

Every function here is pinned by ``tests/test_oracle_pins.py`` to something
other than itself (brute force, closed forms, a library routine, algebraic
invariants); none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attend_rows,
    decode,
    decode_multi,
    decode_multi_visible_len,
    decode_paged,
    paged_gather,
    prefill,
    prefill_varlen,
    prefill_paged,
    prefill_visible_len,
    kv_head_of,
    partial,
    merge,
    merge_normalized,
    finalize,
    online_sweep,
)

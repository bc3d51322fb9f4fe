"""CPU oracle for the DDTree tree-verify path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this code:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it.  It shares no code with the HIP path; both
sides take their inputs from the seeded generators in ``workloads``.

Each function is a plain, slow, obviously-correct statement of one stage:

* ``tree.build_tree``            best-first draft-tree growth (heapq), plus a
                                 brute-force enumerator used to pin it;
* ``visibility``                 ancestor-or-self visibility, full
                                 ``[q_len, prefix+q_len]`` mask and positions;
* ``attention.verify_request``   fp64 masked softmax over the absorbed-MLA
                                 576-d latents, output = weighted c_kv;
* ``accept.accept``              greedy root walk along the target argmax,
                                 plus a brute-force path enumerator;
* ``commit.batch``               committing the accepted path into the paged
                                 cache (new slot lists; optional compaction
                                 of the accepted latent rows);
* ``drafter.batch``              per-depth top-k log-probabilities of the
                                 drafter's logits (fp64 log-softmax);
* ``sample.batch``               stochastic acceptance along the tree
                                 (rejection sampling against the target
                                 distribution, fixed-order fp32 sums).

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against brute force, closed forms, hand-derived fixtures or an independent
library routine (see each test module's docstring).  No function is
"parity unpinned".
"""
from . import accept, attention, commit, drafter, sample, tree, visibility  # noqa: F401

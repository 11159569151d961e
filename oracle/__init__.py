"""CPU oracle for block-sparse attention over a 3D video token grid.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library (no kernels, headers, tables
or layout formulas); the only thing both sides consume is the seeded input
generator module ``workloads``, which holds none of the method's arithmetic.

Everything here is plain numpy in float64 and written for a reader to check by
eye against the pages' description of the method:

* ``layout``    token orders of the grid (frame-major, 3D cubes) and permutations
* ``masks``     block masks from token patterns (spatial / temporal windows)
* ``attention`` masked softmax attention, the exact result block skipping computes
* ``scores``    block mean-pooling and pooled query-key scores
* ``select``    forced + top-k / top-p block selection
* ``profile``   per-head pattern choice from a sample of query rows
* ``pipeline``  the three end-to-end flows, in natural token coordinates
* ``semantic``  k-means clustering, cluster-major order and size-weighted top-p
* ``attention_bwd`` gradients of masked attention
* ``fp8``       the e4m3 codec, quantisers and attention on quantised inputs
* ``skiparse``  the Skiparse-2D token-wise and group-wise spatial patterns

Pins (see tests/test_oracle_*.py) tie every function to something other than
itself: a library special case, closed forms, invariants, hand-worked values,
or brute force on tiny inputs. Functions without such a pin say so in their
docstring ("parity unpinned").
"""
from . import layout, masks, attention, scores, select, profile, pipeline, skiparse  # noqa: F401

"""CPU oracle for the scaled narrow-format (FP8) cast.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code, table or constant generator with
the HIP kernels and imports nothing from them.

Two tiers implement the same definitions:

* ``oracle.formats`` / ``oracle.cast`` / ``oracle.policy`` -- tier 0, the
  specification, in exact rational arithmetic (``fractions.Fraction``) with an
  explicit sign bit on every value, zero included.
* ``oracle.bulk`` -- tier 1, the same definitions vectorised with numpy in
  binary64, where every step used is exact for the inputs it is given (fp32 and
  bf16 values times powers of two, rounding to an integer with ``np.rint``).
  Sums are formed exactly and rounded once.
* ``oracle.swamp`` -- the update/step-ratio ("swamping") monitor and its
  promotion window, tier 0 and tier 1.
* ``oracle.rng`` -- Philox4x32-10, the counter-based generator whose words the
  stochastic-rounding cast draws, written from its published definition.

Sources, cited by page title and section throughout:

* [MP-card]  "Mixed Precision FP16/BF16/FP8" (talentme.airsota.com mind-map
  card), items (1) FP16, (2) BF16, (3) FP8.
* [Drift]    "what actually breaks low precision training"
  (aarohigandhi.vercel.app/writing/drift), sections "First, catching myself",
  "What the measurements said", "The part I would rather not write".
* [E3]       practice exercise c06/E3, "Worked solution"
  (deeper.gabrielebattimelli.com).
* [MaxWin]   "Max-Window Scale Estimation for Near-Lossless HiF8 W8A8
  Quantization-Aware Training" (gist.science explainer), sections
  "Experimental Variables" and "Key Contributions".
* [SP]       "Which parts of a mixed-precision training step must stay in
  single precision, and why?" (katajob.com).

Pinning: every function here is checked by ``tests/test_oracle_*.py`` against
facts fixed independently of this code (constants printed on the pages, closed
forms, library routines such as numpy's float16 and torch's float8 casts,
brute force and invariants; the generator against rocRAND's Philox4x32-10
run on the host).  The error statistics and the value a code stands for
(``stats``, ``stats_terms``, ``represented``, ``dequant_bf16`` and their
tier-1 forms) are pinned by hand-worked elements and sums
(``tests/golden/stats_hand.json``, ``tests/golden/dequant_hand.json``), the
half-step bound, and a closed form of the tanh workload's bias and kept
fraction; ``tests/test_oracle_stats_pins.py`` also plants mistakes in them
and checks that the pins fail.  The scale-update state machine
(``oracle.policy``) follows a reading of an ambiguous hysteresis rule; it is
pinned by brute-force properties and by traces worked by hand from that
reading (``tests/golden/scale_update_hand.json``), which planted mistakes in
the machine fail.
"""

from .formats import BF16, E4M3, E5M2, FP16, FP32, FORMATS, Fmt, Val  # noqa: F401

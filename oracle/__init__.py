"""CPU oracle for entropy-coded weights decoded inside a batch-1 GEMV.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code with the
HIP library (entropy_coded_weight_amd) and imports nothing from it.

What it computes, and the passage each part follows:

* ``coding``   -- histograms, Shannon entropy (DFloat11 page, Eq. 2), the
                  cross-entropy size bound (MINE page, Section 4.2 "Compressed Size
                  Prediction") and the frequency normaliser that minimises it.
* ``rans``     -- interleaved rANS over independent 64-lane tiles: 32-bit states,
                  16-bit payload words, at most one word per symbol (EntroPack page,
                  Sections 3.6 and C.3; ANS background on the MINE page, Section 3).
* ``symbols``  -- logical tensor <-> symbol streams: integer codes packed k per
                  symbol (MINE page, Section 4.1 "Data Types"), BF16 exponent coded
                  with sign+mantissa kept as a raw byte (DFloat11 page, Eq. 1 and
                  Algorithm 1's bit join; MINE page Section 4.1), FP8 E4M3 bytes.
* ``corrections`` -- the sparse correction stream of escaped weights that lets
                  BF16 exponents be coded in pairs over a table of the 16 most
                  frequent exponents, and 4-bit codes in quads over a table of the
                  most frequent 4-tuples (MINE page, Section 4.1 "Escapes",
                  Section 4.2 "Tuning t").
* ``e8``       -- E8 lattice fields with coset-conditioned tables and parity
                  reduction (EntroPack page, Sections 3.2, 3.3 and A.3).
* ``gemv``     -- y = W x in float64 and the per-row error bound.

Every function is plain numpy (vectorised only across independent tiles and
lanes, which the method itself treats as independent); nothing is blocked, fused
or reordered beyond the definitions.
"""

"""CPU oracle for the 1-bit sign GEMV, the +-1 popcount product and the XOR row patch.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or run anything in this package.  The product library
(``bit_packed_sign_amd``) never imports it, and this package never imports the product.

Contents:
  bin1_oracle.c  plain C: fp64 dequantise-and-dot (binary and ternary weights), +-1 product,
                 XOR row patch, bit-granular XOR patch, exact scale ranking (built with gcc)
  oracle.py      ctypes loader and numpy-facing wrappers of bin1_oracle.c
  exact.py       exact-rational (fractions.Fraction) evaluation used to pin the fp64 rounding
  build.py       gcc build of liboracle.so

Parity status per function (what pins it is in tests/test_oracle.py; every function is pinned):
  half_to_double  pinned: all 65536 fp16 patterns against numpy's decode.
  gemv            pinned: closed form (all-ones / all-zeros rows), one-hot bit order, dense
                  numpy expansion (unpackbits + BLAS), exact rationals, exhaustive tiny K,
                  power-of-two scaling, zero / subnormal / negative scales; planted mistakes
                  (MSB-first order, inverted sign, reversed groups, dropped term, transposed
                  output) each fail a pin.
  gemv_t2         pinned: term-for-term equality with gemv on binary-valued rows, zero and
                  code-10 slots, one-hot slots, all 3^8 rows of K = 8 against exact rationals,
                  page byte figures for 2-bit slots; planted mistakes fail.
  pm1             pinned: K - 2*popcount(a xor w) computed with numpy.bitwise_count.
  xor_patch       pinned: involution, bitwise-NOT definition on listed rows, negation of y,
                  out-of-range rows skipped and counted.
  xor_bits        pinned: rank-one closed form, equivalence with row patches, multiset
                  cancellation; planted mistakes fail.
  rank_rows       pinned: brute-force sort and hand-worked examples; planted mistakes fail.
"""

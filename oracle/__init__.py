"""CPU oracle for the 1-bit sign GEMV, the +-1 popcount product and the XOR row patch.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or run anything in this package.  The product library
(``bit_packed_sign_amd``) never imports it, and this package never imports the product.

Contents:
  bin1_oracle.c  plain C, fp64 dequantise-and-dot, +-1 product, XOR patch (built with gcc)
  oracle.py      ctypes loader and numpy-facing wrappers of bin1_oracle.c
  exact.py       exact-rational (fractions.Fraction) evaluation used to pin the fp64 rounding
  build.py       gcc build of liboracle.so

Parity status per function (what pins it is in tests/test_oracle.py):
  gemv      pinned: closed form (all-ones / all-zeros rows), one-hot bit order, dense
            numpy expansion (unpackbits + BLAS), exact rationals, exhaustive tiny K,
            power-of-two scaling, +-1 popcount identity.
  pm1       pinned: K - 2*popcount(a xor w) computed with numpy.bitwise_count.
  xor_patch pinned: involution, bitwise-NOT definition on listed rows, negation of y.
"""

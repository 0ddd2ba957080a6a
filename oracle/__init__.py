"""CPU oracle for the one-shot signal-pad reduction — test infrastructure.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product library never imports, links or runs anything
here, and this package imports nothing from the product.

Modules:
  reduce    the rank-ordered binary32 sum of bf16 partials, rounded once to
            bf16 (plain C in arx_oracle.c, loaded with ctypes)
  protocol  the sequential single-GPU protocol model and the brute-force
            interleaving checkers for the parity protocol and the pad barrier
  build     compiles arx_oracle.c with gcc
"""

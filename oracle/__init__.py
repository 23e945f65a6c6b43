"""CPU oracle for the FibQuant KV-cache codec — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct fp64 (NumPy/SciPy) statement
of what the codec computes.  It exists to check the HIP library; it is not part
of the product.  Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it.  It shares no code with the HIP path and never
takes an input or expected value from it.

Source ("the FibQuant summary"): the technical summary of "FibQuant: universal
vector quantisation for random-access KV-cache compression", published on
gist.science as paper 2605.11478 in a Korean and a Dutch version with the same
section numbering.  Sections cited below:

    §1    Problem statement (fixed-address random access; normalise-rotate-quantise)
    §2.1  The canonical source (normalise + Haar rotation -> spherical-Beta blocks)
    §2.2  Codebook construction (companded radii, Fibonacci / Roberts-Kronecker
          directions, multi-restart Lloyd-Max refinement)
    §2.3  Encoding and decoding (norm, rotation, d/k blocks, nearest codeword;
          gather, concatenate, inverse rotation, rescale; rate b = log2(N)/k)
    §3.1  Theorem 1 (every nonzero input law maps to the same block law f_{d,k})
    §3.2  Theorem 2 (an optimal k-vector code strictly beats the scalar k=1 code)
    §3.3  Dense rate axis (fractional and sub-one-bit rates, e.g. b ~ 0.19)
    §5    Significance (fixed addresses allow decompression fused into attention)

Where the pages leave a step open the module that implements it says which
reading it takes ("Reading:").

Modules
    rotation   Haar rotation Π (seeded QR with sign fix)
    source     the canonical spherical-Beta block source and its density
    codebook   radii, directions, Lloyd-Max, fp16-grid rounding, build_codebook
    codec      norm, rotation, brute-force nearest codeword, pack/unpack, decode
    attention  dense decode attention over a decoded cache
"""

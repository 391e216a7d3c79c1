"""CPU oracle for the fused channelwise tensor-product convolution and the
symmetric contraction.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The product path (``segmented_polynomials_amd``) never
imports it, and it imports nothing from the product path: the two share no
kernels, tables, constants or helpers.  Only the seeded input generators in
``workloads/`` (which hold none of the method's arithmetic) serve both.

Everything here is plain float64 NumPy (complex128 where the complex basis is
needed), written for a reader to check against the pages by eye, with no
blocking, fusion or reordering beyond what a definition states.  Library
routines (``numpy.einsum``, ``numpy.add.at``, ``numpy.linalg.lstsq``,
``scipy.linalg.expm``, ``numpy.polynomial.legendre``) serve as single steps.

Modules
-------
irreps   O(3) irreps strings, dimensions, output ordering.
layout   ``mul_ir`` / ``ir_mul`` block layouts and the blockwise transpose.
sh       real spherical harmonics, component normalisation.
cg       complex Clebsch-Gordan by Racah's formula, the real-basis coupling
         tensor with its sign rule and "component" scaling.
wigner   real Wigner-D two ways (least squares on the harmonics; matrix
         exponential of the angular-momentum generators).
tp       channelwise (uvu) tensor product with gather / sum-scatter.
symcon   symmetric-contraction coupling basis and evaluation.
metrics  the absolute-sum-scaled error used by every parity test.

Pins (what fixes each part other than itself; see ``tests/test_oracle_*.py``):
irreps dims and layouts against the values the pages print; SH against
textbook closed forms and norms; complex CG against ``sympy``'s routine;
real CG by orthogonality, closed forms, equivariance and the SH-coupling
identity with the 3j closed form; Wigner-D by two independent constructions
and the l=1 closed form; TP counts against the descriptor the pages print,
TP values by a dense brute force, the gather/scatter worked example and
equivariance; symmetric-contraction counts against the page's descriptor,
coupling multiplicities by the character formula, the basis-free projector,
the degree-1 and degree-2 closed forms, and equivariance.
"""

from . import irreps, layout, sh, cg, wigner, tp, symcon, metrics  # noqa: F401

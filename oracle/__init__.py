"""Reference oracle for the FlashCart edge convolution and correlation ladder.

TEST INFRASTRUCTURE ONLY.  This package is a slow, plain, fp64 CPU
implementation of what the method computes, written from the FlashCart paper
("FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic
Potentials", arXiv 2610.06409).  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product
library (``cartesian_tensor_product_amd``) never imports it and shares no code
with it: the oracle builds full 3^l tensors, symmetrises by averaging over
index permutations and removes traces by an orthogonal projection, while the
GPU path uses exact rational tables produced by its own generator.

Modules
-------
tensors   STF machinery, direction tensors T_l, Cartesian couplings (paths).
conv      edge convolution forward, VJP and VJP-of-VJP.
ladder    node-local correlation ladder (full and path-reduced) and its VJP.

Parity status of every function is listed in each module's header.
"""


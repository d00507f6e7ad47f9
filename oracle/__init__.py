"""CPU float64 oracle for the equivariant interaction convolution.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library: its harmonics come from Legendre polynomials (not Cartesian
polynomials), its coupling coefficients from numerical quadrature of Gaunt
integrals (not the Racah formula), its neighbour list from brute force (or a
plain binned search that is itself checked against brute force).

Modules
-------
paths   admissible coupling paths and the feature/output layouts
sh      real spherical harmonics (component normalised) and their gradients
cg      real coupling coefficients from Gaunt integrals
nbr     periodic neighbour list, receiver-sorted CSR and reverse-edge index
radial  Bessel basis, polynomial envelope, radial MLP and its input gradient
conv    edge geometry, the convolution forward, its backward, and forces
fd      finite-difference forces of the surrogate scalar L = sum(G * out)
autograd_check  a torch-CPU float64 forward whose autograd cross-checks conv

Every function cites the passage of the pages it follows: the FlashCart paper
("FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic
Potentials"), the FastMACE page "Rewrites and precision options", the pet-jax
README and the Frost model card.  Readings where the pages are silent are
listed in the design notes of the repository.
"""

from . import paths, sh, cg, nbr, radial, conv, fd  # noqa: F401

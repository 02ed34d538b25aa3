"""fp64 CPU oracle for the IPA forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` and by nothing on the product
path. Independent of the HIP library: no shared kernels, headers, helpers or
constants.

Pinning status of each function (see the tests under ``tests/``):
  ipa_forward     pinned: textbook-attention reduction (library SDPA), MEET
                  lifting identity through library SDPA, SE(3) invariance,
                  L = 1 and two-residue closed forms, uniform-attention pair
                  closed form, permutation equivariance, mask semantics
                  (prefix and scattered masks: a masked batch element
                  equals the oracle on its valid residues alone).
  to_global       pinned by a closed form (a quarter turn about z plus a
                  shift) and through the pins of ipa_forward.
  ipa_bruteforce  pinned against the same closed forms on tiny inputs.
  ipa_lifted      pinned to ipa_forward (exact algebra, 1e-12 relative).
  frames_from_atoms  pinned: orthonormal right-handed frames, local atom
                  coordinates, SE(3) equivariance, hand-worked closed forms.
  meet_attention  pinned: textbook attention (library SDPA) at s = 0, the
                  MEET lifting identity through library SDPA, rigid
                  invariance, two-residue closed form, mask rules, agreement
                  with ipa_forward configured to the same logit.
  dirdist_attention  pinned: scalar-loop brute force, textbook attention
                  (library SDPA) when the distance term vanishes, closed forms
                  for the unsquared distance and the value transport, rigid
                  invariance, permutation equivariance, mask and readout rules.
  dirdist_bruteforce pinned by the same closed forms on tiny inputs.
  ipa_backward    pinned: central finite differences of ipa_forward along
                  random directions for every input, its restated forward
                  equals ipa_forward, rigid-motion identities of the frame
                  gradients, masked rows and keys; its row-restricted form
                  (rows=) against the full gradient, and its sum over a
                  partition of the rows into blocks equals the full
                  gradient for every input.
  ipa_layer       pinned: reduces to ipa_forward plus the readout with
                  selection weights, readout order by one-hot rows, the
                  affine maps against a scalar loop, masked rows; its
                  row-restricted form against the full layer.
"""

from .ipa_oracle import ipa_forward, to_global
from .bruteforce import ipa_bruteforce, dirdist_bruteforce
from .lifted import ipa_lifted, block_centres
from .geometry import frames_from_atoms, meet_attention
from .dirdist import dirdist_attention
from .ipa_grad import ipa_backward
from .layer import ipa_layer

__all__ = ["ipa_forward", "to_global", "ipa_bruteforce",
           "ipa_lifted", "block_centres", "frames_from_atoms", "meet_attention",
           "dirdist_attention", "dirdist_bruteforce", "ipa_backward", "ipa_layer"]

"""Plain fp64 CPU oracle for the Muon optimizer step and its AdamW fallback.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers or
constant tables) and imports nothing from it.

Every function is a slow, literal statement of what the method computes, in
numpy float64, with matrix products through the host BLAS and no blocking,
fusion or reordering beyond the steps the sources give.  Citations name the
web page and the section on it:

* "About Muon: Why Not Adam" (kiungsong.github.io) -- sections "Why Muon?",
  "Making It Actually Run" (the odd-polynomial lemma, the Frobenius
  normalisation, the quintic coefficients and their scalar map), "How Do We
  Turn It Into a Real Optimizer?" (parameter routing, the shape multipliers,
  decoupled weight decay) and "The whole thing, in about forty lines" (the
  order of the optimizer's steps).
* "The Optimizer Wars: How Muon Is Replacing Adam in Frontier AI Training"
  (ai.info) -- section "What is Muon? Momentum orthogonalized by
  Newton-Schulz" (five quintic iterations, coefficients (3.4445, -4.7750,
  2.0315)) and section "What is MuonClip?" (QK-Clip after the update).
* "Por qué AdamW para entrenar modelos de lenguaje, y qué está cambiando"
  (gustavoai.dev) -- sections "Momentum: recordar el paso anterior",
  "Adam: las dos ideas juntas", "La W: un error de regularización que duró
  tres años" and "Por qué AdamW, y por qué con esos números".
* "Why Muon Works" (r00kie-liu.github.io) -- section 7.1 (parameter routing),
  7.3 (QKV split) and 7.6 (starter configuration).

``storage.round_to_bf16`` rounds a result to bfloat16 for parameters kept in
that format (round to nearest, ties to even), from the format's definition.

Pins: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms (the SVD form of the odd polynomial, momentum and Adam
recurrences), numbers the pages print (tests/golden/) and invariants
(transpose symmetry, orthogonal equivariance, convergence of the textbook
coefficients to the polar factor).
"""

from .muon import (
    MUON_COEFFS,
    momentum_update,
    nesterov_blend,
    newton_schulz,
    shape_scale,
    muon_matrix_step,
    muon_step,
    qk_clip,
)
from .adamw import adamw_tensor_step, adamw_step, clip_by_global_norm
from .storage import round_to_bf16, store

__all__ = [
    "MUON_COEFFS",
    "momentum_update",
    "nesterov_blend",
    "newton_schulz",
    "shape_scale",
    "muon_matrix_step",
    "muon_step",
    "qk_clip",
    "adamw_tensor_step",
    "adamw_step",
    "clip_by_global_norm",
    "round_to_bf16",
    "store",
]

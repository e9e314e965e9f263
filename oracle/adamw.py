"""fp64 oracle of AdamW with bias correction and decoupled weight decay.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

"Por qué AdamW para entrenar modelos de lenguaje, y qué está cambiando"
(gustavoai.dev).  The page's display formulas did not survive extraction;
this follows its prose:

* section "Adam: las dos ideas juntas": a moving average of the gradient
  (``m``, rate ``beta1``) and of its square (``v``, rate ``beta2``), each
  divided by ``1 - beta^t`` so that the first step already has the right
  scale; the step is the coordinate-wise quotient ``m_hat / sqrt(v_hat)`` with
  a tiny ``eps`` that only prevents division by zero (introduced in
  "AdaGrad y RMSProp"; read here as added to the square root);
* section "La W: ...": the decay ``eta * lambda * theta`` is taken out of the
  quotient and multiplied by the learning rate;
* section "Por qué AdamW, y por qué con esos números": the usual values
  ``beta1 = 0.9``, ``beta2 = 0.95``, ``lambda = 0.1``, ``eps = 1e-8``.
"""

import numpy as np

from .storage import store


def adamw_tensor_step(theta, g, m, v, *, step, lr, beta1=0.9, beta2=0.95,
                      eps=1e-8, weight_decay=0.1, param_dtype="fp32"):
    """One AdamW update of one tensor.  ``step`` is t >= 1 (already counted).

    Returns ``(theta_new, m_new, v_new)``; every operation is elementwise:

    ``m = b1 m + (1-b1) g``; ``v = b2 v + (1-b2) g^2``;
    ``m_hat = m / (1-b1^t)``; ``v_hat = v / (1-b2^t)``;
    ``theta = theta - lr * (m_hat / (sqrt(v_hat) + eps) + wd * theta_old)``;
    a ``param_dtype="bf16"`` parameter stores theta rounded once to bfloat16
    (:func:`oracle.storage.store`); the moments are fp32 state.
    """
    if step < 1:
        raise ValueError("AdamW step count starts at 1")
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * (g * g)
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    direction = m_hat / (np.sqrt(v_hat) + eps)
    theta_new = theta - lr * (direction + weight_decay * theta)
    return store(theta_new, param_dtype), m_new, v_new


def clip_by_global_norm(grads, max_norm):
    """Gradient clipping to a global norm ("Por qué AdamW ...", section "Por
    qué AdamW, y por qué con esos números": before the gradient enters m and
    v, if its norm exceeds 1 it is rescaled to 1; the threshold is a
    parameter here).  The norm is the Euclidean norm of all the given
    tensors together.  Returns ``(clipped_grads, norm)``."""
    gs = [np.asarray(g, dtype=np.float64) for g in grads]
    norm = np.sqrt(sum(float(np.sum(g * g)) for g in gs))
    if norm > max_norm:
        gs = [g * (max_norm / norm) for g in gs]
    return gs, norm


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, max_grad_norm=None, **hparams):
    """AdamW over a list of tensors (each independent).  Returns three lists.
    With ``max_grad_norm``, the gradients are first clipped together to that
    global norm."""
    if max_grad_norm is not None:
        grads, _ = clip_by_global_norm(grads, max_grad_norm)
    ts, ms, vs = [], [], []
    for p, g, m, v in zip(params, grads, exp_avgs, exp_avg_sqs):
        t, mm, vv = adamw_tensor_step(p, g, m, v, **hparams)
        ts.append(t)
        ms.append(mm)
        vs.append(vv)
    return ts, ms, vs

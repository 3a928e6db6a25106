"""Oracle: the canvas embedding with the self-conditioning vector injected (float64).

Test infrastructure only (see the package docstring).

What is computed, and where the pages state it: between denoising steps the model
conditions on its previous full softmax distribution; that distribution becomes the
probability-weighted average of the token embeddings (oracle.selfcond), which is
added to the canvas embedding through a gated MLP - [P1] section "안정성을 위한 셀프
컨디셔닝"; the canvas embedding and the self-conditioning are the prepare_inputs hook's
work - [P1] section "ModelState 인터페이스".

Reading taken where the pages leave the step open: the gated MLP is a GeGLU with the
tanh-approximated GELU and no bias or normalisation, weights applied as x . W:
    out_i = E[token_i] + (gelu(s_i . Wg) * (s_i . Wu)) . Wd
    gelu(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))).
"""
from __future__ import annotations

import numpy as np


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def selfcond_inject(tokens: np.ndarray, embed: np.ndarray, s: np.ndarray, w_gate_up: np.ndarray,
                    w_down: np.ndarray, round_to=None) -> np.ndarray:
    """out [M, d] for canvas tokens [M], embed [V, d], s [M, d], w_gate_up [d, 2h] (gate
    columns first), w_down [h, d]. `round_to`, if given, rounds the two intermediates the
    way the stored dtype does (it is applied to gate/up and to the GeGLU output)."""
    r = (lambda x: x) if round_to is None else round_to
    h = w_down.shape[0]
    gu = r(np.asarray(s, np.float64) @ np.asarray(w_gate_up, np.float64))
    hid = r(gelu_tanh(gu[:, :h]) * gu[:, h:])
    return np.asarray(embed, np.float64)[np.asarray(tokens)] + hid @ np.asarray(w_down, np.float64)

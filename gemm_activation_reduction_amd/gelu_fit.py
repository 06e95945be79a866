"""Fits the polynomial behind the device erf-GELU (``gelu_erf`` in csrc/device_math.h).

The exact-form GELU is v Phi(v) (the Kimi-K2.6 l2_p67 page: PyTorch's default
approximate='none'). With a = |v| it equals max(v, 0) - a Phi(-a) for either sign of v,
so the device needs only the normal tail Phi(-a). It evaluates that tail as 2^Q(a), Q a
polynomial of degree 5, with one v_exp_f32.

The fit minimizes the largest GELU error over a in [0, A]. An error dQ in Q moves the GELU
by a Phi(-a) (2^dQ - 1), about a Phi(-a) ln 2 dQ, so Q is fitted to log2 Phi(-a) in the
weighted minimax sense, as one linear program on a dense grid. The weight vanishes at a = 0
and decays like e^(-a^2/2), so the fit concentrates where the tail matters for the GELU.

Run ``python -m gemm_activation_reduction_amd.gelu_fit`` to print the coefficients as C
literals; they are copied into device_math.h.
"""
from __future__ import annotations

import numpy as np

DEGREE = 5
A_MAX = 6.5


def fit(degree: int = DEGREE, a_max: float = A_MAX, n: int = 3000):
    """Returns (coefficients c_0..c_degree of Q in increasing order, minimax weighted error)."""
    from scipy.optimize import linprog
    from scipy.special import log_ndtr, ndtr

    # uniform points plus a set that is denser near a = 0
    a = np.unique(np.concatenate([np.linspace(0.0, a_max, n),
                                  a_max * (1.0 - np.cos(np.linspace(0.0, np.pi / 2, n)))]))
    target = log_ndtr(-a) / np.log(2.0)
    w = a * ndtr(-a) * np.log(2.0)
    nv = degree + 1
    scale = a_max ** np.arange(nv)  # the columns are scaled for conditioning
    V = (a[:, None] / a_max) ** np.arange(nv)
    # variables (d_0..d_degree, t) with c_k = d_k / a_max^k: minimize t subject to
    # -t <= w (V d - target) <= t
    A_ub = np.vstack([np.hstack([w[:, None] * V, -np.ones((a.size, 1))]),
                      np.hstack([-w[:, None] * V, -np.ones((a.size, 1))])])
    b_ub = np.concatenate([w * target, -w * target])
    cost = np.zeros(nv + 1)
    cost[-1] = 1.0
    res = linprog(cost, A_ub=A_ub, b_ub=b_ub, bounds=[(None, None)] * nv + [(0.0, None)], method="highs")
    if not res.success:
        raise RuntimeError(res.message)
    return res.x[:nv] / scale, float(res.x[-1])


def main() -> None:
    c, err = fit()
    print(f"// degree {DEGREE} on [0, {A_MAX}], weighted minimax error {err:.3e}")
    for k in range(DEGREE, -1, -1):
        print(f"c{k} = {float(np.float32(c[k])):.17g}f")


if __name__ == "__main__":
    main()

"""Hand-built MoE inputs whose exact outputs are known in closed form.

Codes are produced with torch's own float8_e4m3fn cast of values that are
exactly representable, so these inputs do not depend on any oracle code.
"""

import numpy as np
import torch


def code(v):
    t = torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn)
    assert float(t.float()[0]) == v, f"{v} is not representable in e4m3"
    return int(t.view(torch.uint8)[0])


def crafted_exact_case():
    """Every stage exact: gate in {0} U [18, 64] (sigmoid rounds to 1 in fp32),
    activations fp8-representable with each 128-block max = 448 * 4^t, power-of-
    two routing weights.  Returns (inputs tuple of numpy arrays, expected fp32
    values of the bf16 output, derived by hand)."""
    T, H, I, E, K = 3, 128, 128, 2, 2
    x_q = np.full((T, H), code(1.0), np.uint8)
    x_s = np.array([[2.0 ** t] for t in range(T)], np.float32)
    G = [np.zeros(I), np.zeros(I)]
    U = [np.zeros(I), np.zeros(I)]
    G[0][:4] = [56, 24, 18, 0];  U[0][:4] = [8, 2, -1, 5]        # acts 448, 48, -18, 0
    G[1][:3] = [32, 20, 64];     U[1][:3] = [0.25, -0.5, 7]      # acts 8, -10, 448
    w13_q = np.zeros((E, 2 * I, H), np.uint8)
    for e in range(E):
        for c in range(I):
            w13_q[e, c, :] = code(G[e][c] / H)
            w13_q[e, I + c, :] = code(U[e][c] / H)
    w13_s = np.ones((E, 2, 1), np.float32)
    w2_q = np.zeros((E, H, I), np.uint8)
    for n in range(H):
        w2_q[0, n, n % 4] = code(1.0)
        w2_q[1, n, n % 3] = code(2.0)
    w2_s = np.ones((E, 1, 1), np.float32)
    ids = np.array([[0, 1], [1, 0], [0, 0]], np.int32)
    wts = np.array([[0.75, 0.25], [0.5, 0.5], [0.5, 0.25]], np.float32)
    # h = 2^t (G, U); act = 4^t G U; block amax = 448 * 4^t -> s = 4^t, q = G U;
    # Y0[n] = act0[n % 4], Y1[n] = 2 * act1[n % 3]; out = sum_j w_j Y_j, one bf16 rounding
    act0 = np.array([448, 48, -18, 0], float)
    act1 = np.array([8, -10, 448], float)
    expect = np.zeros((T, H))
    for t in range(T):
        for j in range(K):
            for n in range(H):
                y = 4.0 ** t * (act0[n % 4] if ids[t, j] == 0 else 2 * act1[n % 3])
                expect[t, n] += float(wts[t, j]) * y
    assert np.all(expect.astype(np.float32) == expect)
    expect_bf16 = torch.from_numpy(expect.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return (x_q, x_s, w13_q, w13_s, w2_q, w2_s, ids, wts), expect_bf16

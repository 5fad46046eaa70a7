"""Hand-derived cases shared by the oracle pins and the GPU parity tests.

Each case states its inputs and the exact expected output, derived in its
docstring from the definitions on the pages, so that both the oracle and the
kernels are checked against the same closed form rather than against each
other.
"""
import numpy as np

K = V = 128


def gated_rounding_case():
    """A one-token, one-head case whose gated output depends on the stage's
    BF16 rounding of o at both places it is used (fused page, KdaFused.kernel,
    the output stage: o is rounded to BF16, then squared and summed, then
    multiplied by rstd, the weight and the gate's sigmoid).

    Inputs: lb = 0, so every decay is exactly 1; a zero key, whose normalised
    value k / sqrt(0 + 1e-6) is exactly 0, so the update adds nothing; q = e_0.
    Then o[v] = S_0[v][0] exactly. S_0[0][0] = a = 1 + 2^-8 - 2^-15, which is
    not a BF16 value and rounds down to 1 (it lies below the midpoint
    1 + 2^-8); S_0[1][0] = 2^-4; every other row is 0. The gate is BF16(100),
    whose sigmoid is 1 in FP64, and eps = 0. So

        sum of o_bf^2 = 1 + 2^-8,  rstd = sqrt(128 / (1 + 2^-8)),

    and the weights are chosen so that row 0 lands at o_bf * rstd * w_0 =
    1 + 0.3 * 2^-7 and row 1 at 2^-4 * rstd * w_1 = 1 - 0.3 * 2^-8: both
    round to 1.0 (BF16 0x3F80), 0.2 ulp inside the rounding interval.

    Without the rounding in the sum of squares, rstd falls by the factor
    sqrt((1 + 2^-8) / (a^2 + 2^-8)) = 0.99615, and row 1 becomes
    0.99499 -> 0.99609375 (0x3F7F). Without the rounding in the product, row 0
    becomes (1 + 0.3 * 2^-7) * a = 1.00623 -> 1.0078125 (0x3F81). Rows 2.. are 0.
    Returns the inputs as keyword arguments of a verify call and the expected
    output row."""
    H, B, T, RQ = 1, 1, 1, 1
    a = 1.0 + 2.0 ** -8 - 2.0 ** -15
    state = np.zeros((2, H, V, K), np.float32)
    state[1, 0, 0, 0] = a
    state[1, 0, 1, 0] = 2.0 ** -4
    q = np.zeros((B * T, H, K), np.uint16)
    q[0, 0, 0] = 0x3F80  # 1.0
    zeros = np.zeros((B * T, H, K), np.uint16)
    rstd = np.sqrt(128.0 / (1.0 + 2.0 ** -8))
    w = np.ones(V, np.float32)
    w[0] = np.float32((1.0 + 0.3 * 2.0 ** -7) / rstd)
    w[1] = np.float32((1.0 - 0.3 * 2.0 ** -8) / (2.0 ** -4 * rstd))
    args = dict(heads=H, tokens=T, batch=B, q=q, k=zeros, v=zeros, raw_g=zeros,
                raw_beta=np.zeros((B * T, H), np.uint16), a_log=np.zeros(H, np.float32),
                dt_bias=np.zeros((H, K), np.float32), lower_bound=0.0, state=state.reshape(-1),
                state_slot_stride=H * V * K, state_indices=np.array([1], np.int32),
                corr=np.zeros((B, H, RQ, V), np.float32),
                kg=np.zeros((B, H, RQ, 2 * K), np.uint16), record_tokens=RQ,
                record_rows=np.array([0], np.int32),
                gate=np.full((B * T, H * V), 0x42C8, np.uint16),  # BF16 100.0
                norm_weight=w, norm_eps=0.0)
    want = np.zeros(V, np.uint16)
    want[:2] = 0x3F80
    return args, want, a

"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the value it checks.  ``tests/test_oracle_pins.py`` runs every pin against the
real oracle; ``tests/test_oracle_mutations.py`` runs them against deliberately
broken copies of ``oracle/oracle.c`` and requires every copy to fail at least
one pin, which shows the battery catches dropped terms, wrong exponents, swapped
operands and read-before-write mistakes.

None of these checks re-types the oracle's own loop: expected values come from
the worked examples printed on the pages (``tests/golden``), from closed forms,
or from textbook library routines (numpy matmul / tril) applied to the special
cases in which the operator reduces to them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from retention_chunkwise_amd import metrics

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * scale, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def _rand(rng, shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- P-1
def pin_hand_example_elu1():
    """The three-token elu+1 example: o = (1,0), (5/9,4/9), (7/12,2/3).

    "Linear attention", worked example "Linear attention by hand on three
    tokens".  With eps = 0 the fp64 result must equal the printed fractions;
    the final S and z must equal the printed S_3 and z_3.
    """
    g = _golden("linattn_hand_example.json")
    q = np.array(g["q"], float)[None, None]
    k = np.array(g["k"], float)[None, None]
    v = np.array(g["v"], float)[None, None]
    out, S, z = oracle.linattn_recurrent(q, k, v, eps=0.0)
    _close(out[0, 0], g["o"], 1e-15, "hand example outputs (recurrent)")
    _close(S[0, 0], g["S"][-1], 1e-15, "hand example S_3")
    _close(z[0, 0], g["z"][-1], 1e-15, "hand example z_3")
    outp = oracle.linattn_parallel(q, k, v, eps=0.0)
    _close(outp[0, 0], g["o"], 1e-15, "hand example outputs (parallel)")
    rows = oracle.linattn_rows(q, k, v, [(0, 0, t) for t in range(3)], eps=0.0)
    _close(rows, g["o"], 1e-15, "hand example outputs (rows)")
    # the prefix states of the example, one token at a time
    for t in range(3):
        _, St, zt = oracle.linattn_recurrent(q[:, :, :t + 1], k[:, :, :t + 1],
                                             v[:, :, :t + 1], eps=0.0)
        _close(St[0, 0], g["S"][t], 1e-15, f"hand example S_{t + 1}")
        _close(zt[0, 0], g["z"][t], 1e-15, f"hand example z_{t + 1}")


def pin_eps_placement():
    """eps sits in the denominator only: o_t = num_t / (den_t + eps).

    Hand example with eps = 1: o_1 = (3, 0) / (3 + 1), o_2 = (5, 4) / (9 + 1),
    o_3 = (7, 8) / (12 + 1), from the printed numerators and denominators.
    """
    g = _golden("linattn_hand_example.json")
    q = np.array(g["q"], float)[None, None]
    k = np.array(g["k"], float)[None, None]
    v = np.array(g["v"], float)[None, None]
    num = np.array(g["numerator"], float)
    den = np.array(g["denominator"], float)
    expect = num / (den[:, None] + 1.0)
    out, _, _ = oracle.linattn_recurrent(q, k, v, eps=1.0)
    _close(out[0, 0], expect, 1e-15, "eps = 1 (recurrent)")
    _close(oracle.linattn_parallel(q, k, v, eps=1.0)[0, 0], expect, 1e-15,
           "eps = 1 (parallel)")
    _close(oracle.linattn_rows(q, k, v, [(0, 0, 2)], eps=1.0)[0], expect[2], 1e-15,
           "eps = 1 (rows)")
    # and the default eps moves the exact answer by less than 1e-6
    out6, _, _ = oracle.linattn_recurrent(q, k, v)
    _close(out6[0, 0], g["o"], 1e-6, "default eps")


def pin_phi_negative_branch():
    """phi(x) = e^x for x < 0 (elu(x) + 1 with elu(x) = e^x - 1).

    Two tokens, d = 1: q_2 = -1, k_1 = -2, k_2 = 0.5, v = (1, 3).
    w_1 = e^-1 e^-2, w_2 = e^-1 * 1.5, o_2 = (w_1 + 3 w_2) / (w_1 + w_2).
    """
    q = np.array([0.0, -1.0]).reshape(1, 1, 2, 1)
    k = np.array([-2.0, 0.5]).reshape(1, 1, 2, 1)
    v = np.array([1.0, 3.0]).reshape(1, 1, 2, 1)
    w1 = math.exp(-1.0) * math.exp(-2.0)
    w2 = math.exp(-1.0) * 1.5
    expect = (w1 * 1.0 + w2 * 3.0) / (w1 + w2)
    out, _, z = oracle.linattn_recurrent(q, k, v, eps=0.0)
    _close(out[0, 0, 1, 0], expect, 1e-14, "phi negative branch")
    _close(z[0, 0, 0], math.exp(-2.0) + 1.5, 1e-14, "phi of keys summed in z")
    _close(oracle.linattn_parallel(q, k, v, eps=0.0)[0, 0, 1, 0], expect, 1e-14,
           "phi negative branch (parallel)")


# ---------------------------------------------------------------- P-2
def pin_assoc_memory():
    """Outer-product memory example: reads (1,2), (4,0), (3.8,6.2); S=[[1,5],[4,4]].

    "Linear attention", worked example "Three pairs in a two-dimensional
    memory".  Retention with gamma = 1 and q_t = k_t writes k_t v_t^T and
    reads S_t^T k_t, which is that example token by token.
    """
    g = _golden("assoc_memory_example.json")
    kk = np.array(g["k"], float)
    vv = np.array(g["v"], float)
    q = kk[None, None]
    out, S = oracle.retention_recurrent(q, kk[None, None], vv[None, None], [1.0])
    _close(out[0, 0, 0], g["read_k1_after_two"], 1e-15, "read k1")
    _close(out[0, 0, 1], g["read_k2_after_two"], 1e-15, "read k2")
    _close(out[0, 0, 2], g["read_k3_after_three"], 1e-14, "read k3")
    _close(S[0, 0], g["S_after_three"], 1e-15, "S after three writes")
    _, S2 = oracle.retention_recurrent(q[:, :, :2], kk[None, None, :2], vv[None, None, :2],
                                       [1.0])
    _close(S2[0, 0], g["S_after_two"], 1e-15, "S after two writes")
    # decode step from S_2 writing pair 3 and reading with k_1 -> (1, 5)
    o, S3 = oracle.decode_steps(kk[0].reshape(1, 1, 2), kk[2].reshape(1, 1, 2),
                                vv[2].reshape(1, 1, 2), [1.0], S2, nsteps=1)
    _close(o[0, 0], g["read_k1_after_three"], 1e-15, "decode read k1 after three")
    _close(S3[0, 0], g["S_after_three"], 1e-15, "decode S after three")


# ---------------------------------------------------------------- P-3
def _const_rows(T, dk, dv, seed):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal(dk)
    b = rng.standard_normal(dk)
    vv = rng.standard_normal(dv)
    q = np.broadcast_to(c, (1, 1, T, dk)).copy()
    k = np.broadcast_to(b, (1, 1, T, dk)).copy()
    v = np.broadcast_to(vv, (1, 1, T, dv)).copy()
    return q, k, v, c, b, vv


def pin_constant_rows_closed_form():
    """Constant q_t = c, k_t = b, v_t = u give geometric sums in closed form.

    o_t = (c.b) u (1 - g^(t+1)) / (1 - g),  S_T = b u^T (1 - g^T) / (1 - g);
    g = 1: o_t = (t + 1)(c.b) u.  This is the scalar-times-identity setting of
    "Linear Attention, RWKV, and RetNet", section 5 (the SSD duality check),
    summed in closed form; it fixes the decay carried across chunk edges.
    """
    T, dk, dv = 70, 5, 3
    for gam in (0.9, 0.5, 1.0):
        q, k, v, c, b, u = _const_rows(T, dk, dv, seed=7)
        t = np.arange(T)
        if gam == 1.0:
            geo = (t + 1).astype(float)
            geoT = float(T)
        else:
            geo = (1.0 - gam ** (t + 1)) / (1.0 - gam)
            geoT = (1.0 - gam ** T) / (1.0 - gam)
        o_exp = (c @ b) * geo[:, None] * u[None, :]
        S_exp = np.outer(b, u) * geoT
        out, S = oracle.retention_recurrent(q, k, v, [gam])
        _close(out[0, 0], o_exp, 1e-12, f"closed form o (recurrent, g={gam})")
        _close(S[0, 0], S_exp, 1e-12, f"closed form S_T (recurrent, g={gam})")
        _close(oracle.retention_parallel(q, k, v, [gam])[0, 0], o_exp, 1e-12,
               f"closed form o (parallel, g={gam})")
        for C in (1, 3, 16, 64, T):
            oc, Sc = oracle.retention_chunkwise(q, k, v, [gam], C)
            _close(oc[0, 0], o_exp, 1e-12, f"closed form o (chunk {C}, g={gam})")
            _close(Sc[0, 0], S_exp, 1e-12, f"closed form S_T (chunk {C}, g={gam})")
        rows = [(0, 0, tt) for tt in (0, 1, 31, 63, 64, T - 1)]
        _close(oracle.retention_rows(q, k, v, [gam], rows),
               o_exp[[r[2] for r in rows]], 1e-12, f"closed form rows (g={gam})")


def pin_decode_closed_form():
    """n decode steps with the same token: S_n = g^n S_0 + (1-g^n)/(1-g) k v^T."""
    rng = np.random.default_rng(3)
    N, H, dk, dv = 2, 3, 4, 6
    q = rng.standard_normal((N, H, dk))
    k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.1
    gam = np.array([0.9, 0.99, 1.0])
    for n in (1, 2, 17):
        o, S = oracle.decode_steps(q, k, v, gam, S0, nsteps=n)
        geo = np.where(gam == 1.0, float(n), (1.0 - gam ** n) / np.where(gam == 1.0, 1.0, 1.0 - gam))
        S_exp = (gam ** n)[None, :, None, None] * S0 + \
            geo[None, :, None, None] * np.einsum("nhi,nhj->nhij", k, v)
        _close(S, S_exp, 1e-12, f"decode state after {n} steps")
        o_exp = np.einsum("nhi,nhij->nhj", q, S_exp)
        _close(o, o_exp, 1e-12, f"decode read-out after {n} steps")


# ---------------------------------------------------------------- P-4 / P-5
def pin_gamma_one_is_masked_linear_attention():
    """gamma = 1 retention equals ((Q K^T) (.) L) V with L the causal ones mask.

    "Efficient and Sparse Transformers", section 6, "Linear Attention as a
    Special Case"; "Linear attention", theorem "Recurrent and parallel forms
    agree" without the normaliser.  Expected value: numpy matmul + tril.
    """
    rng = np.random.default_rng(11)
    B, H, T, dk, dv = 2, 2, 37, 5, 7
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    expect = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    out, _ = oracle.retention_recurrent(q, k, v, [1.0, 1.0])
    _close(out, expect, 1e-12, "gamma=1 recurrent vs masked QK^T V")
    _close(oracle.retention_parallel(q, k, v, [1.0, 1.0]), expect, 1e-12,
           "gamma=1 parallel vs masked QK^T V")
    oc, _ = oracle.retention_chunkwise(q, k, v, [1.0, 1.0], 8)
    _close(oc, expect, 1e-12, "gamma=1 chunkwise vs masked QK^T V")


def pin_noncausal_associativity():
    """gamma = 1: final state = K^T V and Q (K^T V) = (Q K^T) V.

    "Linear attention", section "Moving the parentheses": the summary
    K^T V is the sum of outer products over the tokens, and regrouping the
    product does not change it.
    """
    rng = np.random.default_rng(12)
    B, H, T, dk, dv = 1, 3, 50, 6, 4
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    _, S = oracle.retention_recurrent(q, k, v, [1.0] * H)
    KtV = np.swapaxes(k, -1, -2) @ v
    _close(S, KtV, 1e-12, "final state = K^T V")
    _close(q @ S, (q @ np.swapaxes(k, -1, -2)) @ v, 1e-12, "Q(K^T V) = (QK^T)V")
    _, Sc = oracle.retention_chunkwise(q, k, v, [1.0] * H, 16)
    _close(Sc, KtV, 1e-12, "chunkwise final state = K^T V")


def pin_decay_matrix_parallel_numpy():
    """Parallel form against numpy with an explicit D (non-negative powers only).

    "RetNet", single-head definition O = (QK^T (.) D) V with D_nm = g^(n-m),
    n >= m.  numpy builds D with tril and powers of (n - m) >= 0.
    """
    rng = np.random.default_rng(13)
    B, H, T, dk, dv = 1, 2, 29, 4, 6
    gam = np.array([0.8, 0.95])
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    n = np.arange(T)
    diff = n[:, None] - n[None, :]
    expect = np.empty((B, H, T, dv))
    for h in range(H):
        D = np.where(diff >= 0, gam[h] ** np.maximum(diff, 0), 0.0)
        expect[:, h] = ((q[:, h] @ np.swapaxes(k[:, h], -1, -2)) * D) @ v[:, h]
    out, _ = oracle.retention_recurrent(q, k, v, gam)
    _close(out, expect, 1e-12, "recurrent vs numpy D")
    _close(oracle.retention_parallel(q, k, v, gam), expect, 1e-12, "parallel vs numpy D")


# ---------------------------------------------------------------- P-6 / P-7
def pin_recurrent_equals_parallel():
    """Recurrent = parallel on random inputs with d_k != d_v, several heads.

    "Linear attention", theorem "Recurrent and parallel forms agree", and its
    pitfall list ("test with unequal sizes"); "Linear Attention, RWKV, and
    RetNet", section 5.
    """
    rng = np.random.default_rng(14)
    B, H, T, dk, dv = 2, 3, 45, 3, 5
    gam = np.array([0.7, 0.97, 1.0])
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    out, _ = oracle.retention_recurrent(q, k, v, gam)
    _close(out, oracle.retention_parallel(q, k, v, gam), 1e-12, "retention rec vs par")
    rows = [(b, h, t) for b in range(B) for h in range(H) for t in (0, 1, 22, T - 1)]
    _close(oracle.retention_rows(q, k, v, gam, rows),
           np.stack([out[b, h, t] for b, h, t in rows]), 1e-12, "retention rows")
    lo, _, _ = oracle.linattn_recurrent(q, k, v)
    _close(lo, oracle.linattn_parallel(q, k, v), 1e-12, "linattn rec vs par")
    _close(oracle.linattn_rows(q, k, v, rows), np.stack([lo[b, h, t] for b, h, t in rows]),
           1e-12, "linattn rows")


def pin_chunk_invariance():
    """Chunk size does not change the result: C in {1, 3, 64, T} and ragged T.

    "Efficient and Sparse Transformers", section 6, "Chunkwise form": small
    chunks approach the recurrent form, large chunks the parallel form.
    """
    rng = np.random.default_rng(15)
    B, H, T, dk, dv = 1, 2, 77, 4, 3
    gam = np.array([0.85, 0.999])
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    ref, Sref = oracle.retention_recurrent(q, k, v, gam)
    for C in (1, 3, 16, 64, T, T + 5):
        oc, Sc = oracle.retention_chunkwise(q, k, v, gam, C)
        _close(oc, ref, 1e-12, f"chunk {C} outputs")
        _close(Sc, Sref, 1e-12, f"chunk {C} final state")


# ---------------------------------------------------------------- P-8 / P-9
def pin_single_key_and_constant_values():
    """One token: retention o_1 = (q_1.k_1) v_1; linear attention o_1 = v_1.

    Constant values give constant normalised outputs.  "Linear attention",
    hand example step 1 ("as it must be with a single key") and the pitfall
    list (constant values must give constant outputs).
    """
    rng = np.random.default_rng(16)
    dk, dv = 6, 4
    q, k, v = _rand(rng, (1, 1, 1, dk)), _rand(rng, (1, 1, 1, dk)), _rand(rng, (1, 1, 1, dv))
    out, S = oracle.retention_recurrent(q, k, v, [0.9])
    _close(out[0, 0, 0], (q[0, 0, 0] @ k[0, 0, 0]) * v[0, 0, 0], 1e-14, "single key")
    _close(S[0, 0], np.outer(k[0, 0, 0], v[0, 0, 0]), 1e-14, "single key state")
    lo, _, _ = oracle.linattn_recurrent(q, k, v, eps=0.0)
    _close(lo[0, 0, 0], v[0, 0, 0], 1e-14, "single key normalised")
    T = 40
    q, k = _rand(rng, (1, 1, T, dk)), _rand(rng, (1, 1, T, dk))
    u = rng.standard_normal(dv)
    vc = np.broadcast_to(u, (1, 1, T, dv)).copy()
    lo, _, _ = oracle.linattn_recurrent(q, k, vc, eps=0.0)
    _close(lo[0, 0], np.broadcast_to(u, (T, dv)), 1e-13, "constant values")


def pin_prefill_decode_handoff():
    """fwd(T) final state + n decode steps = the last n rows of fwd(T + n).

    "Linear attention", section "Decoding, training, and what each costs"
    (prefill then decode); "RetNet", "Chunked Recurrent Representation".
    """
    rng = np.random.default_rng(17)
    B, H, T, n, dk, dv = 2, 2, 30, 5, 4, 3
    gam = np.array([0.9, 0.995])
    q, k, v = (_rand(rng, (B, H, T + n, dk)), _rand(rng, (B, H, T + n, dk)),
               _rand(rng, (B, H, T + n, dv)))
    full, Sfull = oracle.retention_recurrent(q, k, v, gam)
    _, S = oracle.retention_chunkwise(q[:, :, :T], k[:, :, :T], v[:, :, :T], gam, 8)
    for s in range(n):
        o, S = oracle.decode_steps(q[:, :, T + s], k[:, :, T + s], v[:, :, T + s], gam, S)
        _close(o, full[:, :, T + s], 1e-12, f"decode step {s}")
    _close(S, Sfull, 1e-12, "state after handoff")
    # fwd from an initial state = the tail of the full run
    tail, Stail = oracle.retention_recurrent(q[:, :, T:], k[:, :, T:], v[:, :, T:], gam,
                                             init_state=oracle.retention_recurrent(
                                                 q[:, :, :T], k[:, :, :T], v[:, :, :T],
                                                 gam)[1])
    _close(tail, full[:, :, T:], 1e-12, "fwd from initial state")
    _close(Stail, Sfull, 1e-12, "final state from initial state")


# ---------------------------------------------------------------- NEXT-1: initial state, phi decode
def pin_linattn_decode_hand_example():
    """The three-token elu+1 example, one decode step per token.

    "Linear attention", the decode-step exercise: from S = 0, z = 0 each step
    adds phi(k) v^T and phi(k), then reads o = S^T phi(q) / (z^T phi(q) + eps).
    Stepping the printed tokens must reproduce the printed S_t, z_t and o_t
    (eps = 0), and with eps = 1 the printed numerators over (denominator + 1).
    The wrapper must leave its input arrays unchanged.
    """
    g = _golden("linattn_hand_example.json")
    q = np.array(g["q"], float)
    k = np.array(g["k"], float)
    v = np.array(g["v"], float)
    num = np.array(g["numerator"], float)
    den = np.array(g["denominator"], float)
    for eps in (0.0, 1.0):
        S = np.zeros((1, 1, 2, 2))
        z = np.zeros((1, 1, 2))
        for t in range(3):
            o, S, z = oracle.linattn_decode_steps(q[t][None, None], k[t][None, None],
                                                  v[t][None, None], S, z, eps=eps)
            _close(S[0, 0], g["S"][t], 1e-15, f"decode S_{t + 1}")
            _close(z[0, 0], g["z"][t], 1e-15, f"decode z_{t + 1}")
            expect = g["o"][t] if eps == 0.0 else num[t] / (den[t] + 1.0)
            _close(o[0, 0], expect, 1e-15, f"decode o_{t + 1} (eps={eps})")
    # the wrapper copies: the caller's arrays keep their values
    S0 = np.ones((1, 1, 2, 2))
    z0 = np.ones((1, 1, 2))
    oracle.linattn_decode_steps(q[0][None, None], k[0][None, None], v[0][None, None], S0, z0)
    assert np.all(S0 == 1.0) and np.all(z0 == 1.0), "decode modified its inputs"


def pin_linattn_decode_repeated_token():
    """n steps with the same token: S_n = S_0 + n phi(k) v^T, z_n = z_0 + n phi(k).

    The read-out after n steps is then S_n^T phi(q) / (z_n^T phi(q) + eps).
    With q = k = 0 every feature is phi(0) = 1 (hand example: phi(0) = 1), so
    the closed form needs no feature map: z_n = z_0 + n, o = (1^T S_n) /
    (1^T z_n + eps).
    """
    rng = np.random.default_rng(5)
    N, H, dk, dv = 2, 3, 4, 5
    v = rng.standard_normal((N, H, dv))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.3
    z0 = rng.uniform(0.5, 2.0, (N, H, dk))
    zero = np.zeros((N, H, dk))
    for n in (1, 3, 40):
        o, S, z = oracle.linattn_decode_steps(zero, zero, v, S0, z0, eps=1e-3, nsteps=n)
        S_exp = S0 + n * v[:, :, None, :]
        z_exp = z0 + n
        _close(S, S_exp, 1e-13, f"phi decode state after {n} steps")
        _close(z, z_exp, 1e-13, f"phi decode normaliser after {n} steps")
        o_exp = S_exp.sum(axis=2) / (z_exp.sum(axis=2) + 1e-3)[..., None]
        _close(o, o_exp, 1e-13, f"phi decode read-out after {n} steps")


def pin_linattn_prefill_decode_handoff():
    """Linear attention from an initial (S, z) = the tail of one longer run.

    fwd(T) then n decode steps reproduces the last n rows of fwd(T + n);
    fwd of the tail from fwd(T)'s (S, z) reproduces the same rows and the same
    final pair.  On the hand example, token 1 as prefill and tokens 2, 3 from
    its (S_1, z_1) give the printed o_2, o_3 ("Linear attention", hand example
    and the decode-step exercise).
    """
    rng = np.random.default_rng(18)
    B, H, T, n, dk, dv = 2, 2, 25, 4, 5, 3
    q, k, v = (_rand(rng, (B, H, T + n, dk)), _rand(rng, (B, H, T + n, dk)),
               _rand(rng, (B, H, T + n, dv)))
    full, Sf, zf = oracle.linattn_recurrent(q, k, v)
    _, S, z = oracle.linattn_recurrent(q[:, :, :T], k[:, :, :T], v[:, :, :T])
    tail, St, zt = oracle.linattn_recurrent(q[:, :, T:], k[:, :, T:], v[:, :, T:],
                                            init_S=S, init_z=z)
    _close(tail, full[:, :, T:], 1e-12, "linattn fwd from initial (S, z)")
    _close(St, Sf, 1e-12, "linattn final S from initial state")
    _close(zt, zf, 1e-12, "linattn final z from initial state")
    for s in range(n):
        o, S, z = oracle.linattn_decode_steps(q[:, :, T + s], k[:, :, T + s], v[:, :, T + s], S, z)
        _close(o, full[:, :, T + s], 1e-12, f"linattn decode step {s}")
    _close(S, Sf, 1e-12, "linattn S after handoff")
    _close(z, zf, 1e-12, "linattn z after handoff")
    g = _golden("linattn_hand_example.json")
    hq = np.array(g["q"], float)[None, None]
    hk = np.array(g["k"], float)[None, None]
    hv = np.array(g["v"], float)[None, None]
    S1 = np.array(g["S"][0], float)[None, None]
    z1 = np.array(g["z"][0], float)[None, None]
    o23, S3, z3 = oracle.linattn_recurrent(hq[:, :, 1:], hk[:, :, 1:], hv[:, :, 1:], eps=0.0,
                                           init_S=S1, init_z=z1)
    _close(o23[0, 0], g["o"][1:], 1e-15, "hand example o_2, o_3 from (S_1, z_1)")
    _close(S3[0, 0], g["S"][2], 1e-15, "hand example S_3 from (S_1, z_1)")
    _close(z3[0, 0], g["z"][2], 1e-15, "hand example z_3 from (S_1, z_1)")


def pin_retention_initial_state_decays():
    """With zero keys only the initial state speaks: o_t = g^(t+1) q_t S_0.

    The recurrence S_t = g S_(t-1) + k_t v_t^T ("RetNet", "Recurrent
    Representation") with k = 0 leaves S_t = g^(t+1) S_0 after token t
    (0-based), so the read-out is the initial state decayed t + 1 times and
    the final state is g^T S_0.
    """
    rng = np.random.default_rng(19)
    B, H, T, dk, dv = 1, 3, 70, 4, 6
    gam = np.array([0.5, 0.93, 1.0])
    q = _rand(rng, (B, H, T, dk))
    k = np.zeros((B, H, T, dk))
    v = _rand(rng, (B, H, T, dv))
    S0 = _rand(rng, (B, H, dk, dv))
    out, fs = oracle.retention_recurrent(q, k, v, gam, init_state=S0)
    for h in range(H):
        pw = gam[h] ** np.arange(1, T + 1)
        _close(out[0, h], pw[:, None] * (q[0, h] @ S0[0, h]), 1e-13, f"init-state read-out h={h}")
        _close(fs[0, h], gam[h] ** T * S0[0, h], 1e-13, f"init-state final h={h}")


# ---------------------------------------------------------------- NEXT-2: gradients
def _loss(q, k, v, gam, do):
    out, _ = oracle.retention_recurrent(q, k, v, gam)
    return float(np.sum(out * do))


def pin_bwd_finite_differences():
    """The oracle's gradients against central differences of the forward.

    L = sum(out * dout) with out from the recurrent forward (pinned above);
    each entry of q, k, v is moved by +-h and the difference quotient must
    match dL/dx within the O(h^2) truncation error (the loss is quadratic in
    each input, so the central difference is exact up to rounding).
    """
    rng = np.random.default_rng(20)
    B, H, T, dk, dv = 1, 2, 7, 3, 4
    gam = np.array([0.8, 0.97])
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    do = _rand(rng, (B, H, T, dv))
    dq, dk_, dv_ = oracle.retention_bwd(q, k, v, gam, do)
    h = 1e-4
    for name, x, grad in (("q", q, dq), ("k", k, dk_), ("v", v, dv_)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], gam, do)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], gam, do)
            num[idx] = (lp - lm) / (2 * h)
        _close(grad, num, 1e-8, f"d{name} vs central differences")


def pin_bwd_parallel_closed_form():
    """Gradients of the parallel form O = (Q K^T (.) D) V, written with numpy:
    dQ = ((dO V^T) (.) D) K,  dK = ((dO V^T) (.) D)^T Q,  dV = ((Q K^T) (.) D)^T dO,
    with D built from non-negative powers only ("RetNet", single-head
    definition), on d_k != d_v and a ragged length."""
    rng = np.random.default_rng(21)
    B, H, T, dk, dv = 2, 2, 41, 5, 3
    gam = np.array([0.9, 1.0])
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    do = _rand(rng, (B, H, T, dv))
    dq, dk_, dv_ = oracle.retention_bwd(q, k, v, gam, do)
    n = np.arange(T)
    for h in range(H):
        e = n[:, None] - n[None, :]
        D = np.where(e >= 0, gam[h] ** np.maximum(e, 0), 0.0)
        for b in range(B):
            Q, K, V, dO = q[b, h], k[b, h], v[b, h], do[b, h]
            dP = (dO @ V.T) * D
            _close(dq[b, h], dP @ K, 1e-11, f"dQ closed form b={b} h={h}")
            _close(dk_[b, h], dP.T @ Q, 1e-11, f"dK closed form b={b} h={h}")
            _close(dv_[b, h], ((Q @ K.T) * D).T @ dO, 1e-11, f"dV closed form b={b} h={h}")


def pin_bwd_as_forwards():
    """The gradients are retention forwards of permuted inputs: dq is the
    causal forward of (dout, v, k); dk and dv are causal forwards of (v, dout,
    q) and (k, q, dout) run on the time-reversed sequence."""
    rng = np.random.default_rng(22)
    B, H, T, dk, dv = 1, 3, 33, 4, 6
    gam = np.array([0.7, 0.95, 1.0])
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    do = _rand(rng, (B, H, T, dv))
    dq, dk_, dv_ = oracle.retention_bwd(q, k, v, gam, do)
    f = lambda x: x[:, :, ::-1].copy()
    _close(dq, oracle.retention_recurrent(do, v, k, gam)[0], 1e-12, "dq as a forward")
    _close(dk_, f(oracle.retention_recurrent(f(v), f(do), f(q), gam)[0]), 1e-12, "dk as a reversed forward")
    _close(dv_, f(oracle.retention_recurrent(f(k), f(q), f(do), gam)[0]), 1e-12, "dv as a reversed forward")


# ---------------------------------------------------------------- NEXT-4: output normalisation
def _parallel_floor(q, k, v, gam):
    """numpy: (Q K^T (.) D) V divided by the row sums of Q K^T (.) D, floored at 1 in size."""
    B, H, T = q.shape[:3]
    out = np.zeros(q.shape[:3] + (v.shape[3],))
    n = np.arange(T)
    e = n[:, None] - n[None, :]
    for h in range(H):
        D = np.where(e >= 0, gam[h] ** np.maximum(e, 0), 0.0)
        for b in range(B):
            A = (q[b, h] @ k[b, h].T) * D
            r = A.sum(axis=1)
            out[b, h] = (A @ v[b, h]) / np.maximum(np.abs(r), 1.0)[:, None]
    return out


def pin_rowsum_floor_parallel():
    """The floored read-out equals the parallel form divided by its own score
    row sums (floor 1): the normaliser recurrence n_t = gamma n_{t-1} + k_t
    ("Linear attention", box "An LSTM whose cell is linear attention", with
    f = gamma, i = 1) must give exactly those row sums, sign included."""
    rng = np.random.default_rng(23)
    B, H, T, dk, dv = 2, 3, 45, 5, 4
    gam = np.array([0.6, 0.95, 1.0])
    q, k, v = 2.0 * _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    _close(oracle.retention_normalized(q, k, v, gam), _parallel_floor(q, k, v, gam), 1e-12, "row-sum floor")


def pin_rowsum_floor_inactive_for_small_scores():
    """Scores whose row sums stay below 1 in size leave the output unchanged."""
    rng = np.random.default_rng(24)
    q, k, v = 1e-3 * _rand(rng, (1, 2, 30, 4)), _rand(rng, (1, 2, 30, 4)), _rand(rng, (1, 2, 30, 3))
    gam = np.array([0.9, 0.5])
    _close(oracle.retention_normalized(q, k, v, gam), oracle.retention_recurrent(q, k, v, gam)[0], 1e-15,
           "floor inactive")


def pin_rowsum_floor_scale_invariance():
    """Once every row sum is at least 1 in size, scaling q leaves the output unchanged."""
    rng = np.random.default_rng(25)
    q, k, v = _rand(rng, (1, 2, 25, 4)), _rand(rng, (1, 2, 25, 4)), _rand(rng, (1, 2, 25, 3))
    gam = np.array([0.8, 1.0])
    big = oracle.retention_normalized(1e4 * q, k, v, gam)
    bigger = oracle.retention_normalized(3e4 * q, k, v, gam)
    _close(big, bigger, 1e-10, "scale invariance")


def pin_groupnorm_rows():
    """GroupNorm of the floored output: with eps = 0 every row has mean 0 and
    mean square 1, and it is the textbook standardisation of the floored rows."""
    rng = np.random.default_rng(26)
    q, k, v = _rand(rng, (2, 2, 20, 6)), _rand(rng, (2, 2, 20, 6)), _rand(rng, (2, 2, 20, 8))
    gam = np.array([0.9, 0.99])
    g0 = oracle.retention_normalized(q, k, v, gam, group=True, eps=0.0)
    _close(g0.mean(axis=-1), np.zeros(g0.shape[:3]), 1e-12, "row means")
    _close((g0 ** 2).mean(axis=-1), np.ones(g0.shape[:3]), 1e-11, "row mean squares")
    f = _parallel_floor(q, k, v, gam)
    eps = 1e-3
    mu = f.mean(axis=-1, keepdims=True)
    var = ((f - mu) ** 2).mean(axis=-1, keepdims=True)
    _close(oracle.retention_normalized(q, k, v, gam, group=True, eps=eps), (f - mu) / np.sqrt(var + eps), 1e-12,
           "GroupNorm standardisation")


# ---------------------------------------------------------------- NEXT-3: GLA gate
def pin_gla_special_cases():
    """A constant gate gamma is RetNet and a gate of 1 is plain linear
    attention ("Efficient and Sparse Transformers", section "Gated Linear
    Attention": G_t = gamma 1 and G_t = 1)."""
    rng = np.random.default_rng(27)
    B, H, T, dk, dv = 2, 3, 37, 5, 4
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    gam = np.array([0.9, 0.5, 1.0])
    lg = np.broadcast_to(np.log(gam)[None, :, None, None], (B, H, T, dk)).copy()
    o, S = oracle.gla_recurrent(q, k, v, lg)
    ro, rS = oracle.retention_recurrent(q, k, v, gam)
    _close(o, ro, 1e-12, "GLA constant gate = retention")
    _close(S, rS, 1e-12, "GLA constant gate state")
    o1, _ = oracle.gla_recurrent(q, k, v, np.zeros((B, H, T, dk)))
    n = np.arange(T)
    L = (n[:, None] >= n[None, :]).astype(float)
    for b in range(B):
        for h in range(H):
            _close(o1[b, h], ((q[b, h] @ k[b, h].T) * L) @ v[b, h], 1e-11, "GLA unit gate = masked linear attention")


def pin_gla_parallel_form():
    """Brute force with per-channel cumulative log-gates:
    o_i = sum_{j<=i} sum_c q_i[c] k_j[c] exp(sum_{s=j+1..i} lg_s[c]) v_j, on
    random gates (d_k != d_v, ragged length)."""
    rng = np.random.default_rng(28)
    B, H, T, dk, dv = 1, 2, 29, 6, 3
    q, k, v = _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dk)), _rand(rng, (B, H, T, dv))
    lg = -rng.uniform(0.0, 1.5, (B, H, T, dk))
    o, S = oracle.gla_recurrent(q, k, v, lg)
    for h in range(H):
        cum = np.cumsum(lg[0, h], axis=0)  # cum[i] = sum_{s<=i}
        exp_ = np.zeros((T, T, dk))
        for i in range(T):
            for j in range(i + 1):
                exp_[i, j] = np.exp(cum[i] - cum[j])
        A = np.einsum("ic,jc,ijc->ij", q[0, h], k[0, h], exp_)
        _close(o[0, h], A @ v[0, h], 1e-11, f"GLA parallel form h={h}")
        Sref = np.einsum("jc,jv,jc->cv", k[0, h], v[0, h], np.exp(cum[-1][None, :] - cum))
        _close(S[0, h], Sref, 1e-11, f"GLA final state h={h}")


def pin_gla_channel_reset():
    """A gate of 0 (a very negative log-gate) on every channel at token r
    erases the past: the outputs from r on equal a run that starts at r."""
    rng = np.random.default_rng(29)
    T, r = 30, 11
    q, k, v = _rand(rng, (1, 1, T, 4)), _rand(rng, (1, 1, T, 4)), _rand(rng, (1, 1, T, 5))
    lg = -rng.uniform(0.0, 0.5, (1, 1, T, 4))
    lg[0, 0, r] = -800.0
    o, _ = oracle.gla_recurrent(q, k, v, lg)
    o2, _ = oracle.gla_recurrent(q[:, :, r:], k[:, :, r:], v[:, :, r:], lg[:, :, r:])
    _close(o[:, :, r:], o2, 1e-12, "GLA reset")


# ---------------------------------------------------------------- P-10
def pin_metric_calculator():
    """The pages' analytic counts.

    "Linear attention": T = 65,536, d = 128 gives about 2.2e12 FLOPs for the
    left order and 4.3e9 for the right, 512 times fewer; the crossover is
    T* = d (strictly cheaper from d + 1); a 128 x 128 state plus normaliser is
    16,512 numbers; storing every state at T = 8192, d = 128 in fp32 is
    512 MiB; 32 heads of 128^2 fp32 state is 2 MiB, equal in numbers to an
    8-KV-head GQA cache of width 128 at 256 tokens.
    """
    left = metrics.attention_flops(65536, 128, 128, "left")
    right = metrics.attention_flops(65536, 128, 128, "right")
    assert round(left / 1e12, 1) == 2.2, left
    assert round(right / 1e9, 1) == 4.3, right
    assert left // right == 512 and left % right == 0
    assert metrics.crossover_T(128, 128) == 129
    assert metrics.crossover_T(32, 32) == 33
    d_phi, d_v = 64, 256  # T* = 2 d_phi d_v / (d_phi + d_v) = 102.4
    assert metrics.crossover_T(d_phi, d_v) == 103
    assert metrics.decode_state_numbers(128, 128) == 16512
    assert metrics.decode_flops_per_head(128, 128) == 4 * 128 * 128
    assert metrics.stored_states_bytes(8192, 128, 128) == 512 * 2 ** 20
    st = metrics.layer_state_bytes(32, 128, 128)
    assert st == 2 * 2 ** 20
    assert metrics.kv_cache_tokens_equal(32 * 128 * 128, 8, 128) == 256
    # chunkwise work: 2C(dk+dv) + 4 dk dv per head-token
    assert metrics.chunkwise_flops_per_head_token(128, 128, 128) == 131072
    assert metrics.fwd_flops(1, 32, 65536, 128, 128, 128) == 274877906944


ALL_PINS = [
    pin_hand_example_elu1,
    pin_eps_placement,
    pin_phi_negative_branch,
    pin_assoc_memory,
    pin_constant_rows_closed_form,
    pin_decode_closed_form,
    pin_gamma_one_is_masked_linear_attention,
    pin_noncausal_associativity,
    pin_decay_matrix_parallel_numpy,
    pin_recurrent_equals_parallel,
    pin_chunk_invariance,
    pin_single_key_and_constant_values,
    pin_prefill_decode_handoff,
    pin_linattn_decode_hand_example,
    pin_linattn_decode_repeated_token,
    pin_linattn_prefill_decode_handoff,
    pin_retention_initial_state_decays,
    pin_bwd_finite_differences,
    pin_bwd_parallel_closed_form,
    pin_bwd_as_forwards,
    pin_rowsum_floor_parallel,
    pin_rowsum_floor_inactive_for_small_scores,
    pin_rowsum_floor_scale_invariance,
    pin_groupnorm_rows,
    pin_gla_special_cases,
    pin_gla_parallel_form,
    pin_gla_channel_reset,
    pin_metric_calculator,
]

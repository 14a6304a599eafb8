"""Work and traffic accounting for the benchmark (host arithmetic only).

Counting convention: a product of an (m x k) and a (k x n) matrix costs 2mkn
FLOPs ("Linear attention", zerotofrontier section 21.2, section "Moving the
parentheses").  Elementwise decay and normaliser terms are lower order and,
as on that page, left out of the count.
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "f32": 157.3, "f64": 78.6}


# ---- the pages' analytic counts ("Linear attention", box "Associativity turns
# ---- quadratic cost into linear cost"; section "Decoding, training, and what
# ---- each costs"; example "When the state becomes smaller than the cache")

def attention_flops(T: int, d_phi: int, d_v: int, order: str) -> int:
    """FLOPs of the two products of non-causal linear attention."""
    if order == "left":      # (phi(Q) phi(K)^T) V
        return 2 * T * T * d_phi + 2 * T * T * d_v
    if order == "right":     # phi(Q) (phi(K)^T V)
        return 2 * T * d_phi * d_v + 2 * T * d_phi * d_v
    raise ValueError(order)


def crossover_T(d_phi: int, d_v: int) -> int:
    """Smallest positive T at which the right order is strictly cheaper."""
    T = 1
    while attention_flops(T, d_phi, d_v, "right") >= attention_flops(T, d_phi, d_v, "left"):
        T += 1
    return T


def decode_state_numbers(d_phi: int, d_v: int) -> int:
    """Numbers held by one head's decode state S (d_phi x d_v) and z (d_phi)."""
    return d_phi * d_v + d_phi


def decode_flops_per_head(d_phi: int, d_v: int) -> int:
    """About 4 d_phi d_v FLOPs per head per generated token (update + read)."""
    return 4 * d_phi * d_v


def stored_states_bytes(T: int, d_phi: int, d_v: int, bytes_per: int = 4) -> int:
    """Memory of keeping every intermediate state S_t of one head."""
    return T * d_phi * d_v * bytes_per


def layer_state_bytes(heads: int, d_k: int, d_v: int, bytes_per: int = 4) -> int:
    return heads * d_k * d_v * bytes_per


def kv_cache_tokens_equal(state_numbers: int, n_kv: int, d_k: int) -> int:
    """Tokens at which a GQA cache holds as many numbers as the state."""
    return state_numbers // (2 * n_kv * d_k)


# ---- chunkwise forward work (mode table of the same page: chunkwise work is
# ---- O(T T_c (d_phi + d_v) + T d_phi d_v))

def chunkwise_flops_per_head_token(chunk: int, dk: int, dv: int, causal: bool = False) -> int:
    """Dense: 2C(dk+dv) + 4 dk dv.  Causal minimum: (C+1)(dk+dv) + 4 dk dv.

    Terms: Q K^T and P V inside the chunk (C keys per query), Q S and the
    K^T V state update across chunks (dk x dv per token each).
    """
    if causal:
        return (chunk + 1) * (dk + dv) + 4 * dk * dv
    return 2 * chunk * (dk + dv) + 4 * dk * dv


def fwd_flops(B, H, T, dk, dv, chunk, causal=False) -> int:
    return B * H * T * chunkwise_flops_per_head_token(chunk, dk, dv, causal)


def fwd_bytes(B, H, T, dk, dv, elem_bytes: int, final_state: bool) -> int:
    """Read q, k, v once, write out once (+ the fp32 final state)."""
    b = B * H * T * (2 * dk + dv) * elem_bytes + B * H * T * dv * elem_bytes
    if final_state:
        b += B * H * dk * dv * 4
    return b


def decode_bytes(N, H, dk, dv, elem_bytes: int) -> int:
    """fp32 state read + written once, q, k, v read, out written."""
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * elem_bytes + dv * elem_bytes)


def bwd_bytes(B, H, T, dk, dv, elem_bytes: int) -> int:
    """q, k, v and dout read once, dq, dk and dv written once."""
    return B * H * T * (3 * dk + 2 * dv + dk + dv) * elem_bytes


def linattn_decode_bytes(N, H, dk, dv, elem_bytes: int) -> int:
    """The retention decode bytes plus the fp32 normaliser z read and written."""
    return decode_bytes(N, H, dk, dv, elem_bytes) + N * H * 2 * dk * 4


def decode_flops(N, H, dk, dv) -> int:
    return N * H * decode_flops_per_head(dk, dv)

"""Non-finite inputs (needs a gfx950 GPU): a NaN or Inf in one head's keys,
values or queries must not crash a kernel or leak into other heads.

The operator is a sum over earlier tokens, so a non-finite k_s or v_s makes
every later output of its head non-finite, and the head's final state too.
Masked products inside a chunk are multiplied by zero rather than skipped, so
the outputs of earlier tokens of the same chunk may turn non-finite as well;
everything before that chunk, and every other head, must equal the clean run
bit for bit.  A non-finite query only touches its own row.
"""
import numpy as np
import pytest
import torch

import retention_chunkwise_amd as rc
from retention_chunkwise_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(dtype, T, seed=90):
    w = wl.WORKLOADS["ret_fwd_mh_f32"].with_(B=2, H=3, T=T, dk=64, dv=64, dtype=dtype, chunk=64)
    return wl.make_inputs(w, seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("which,bad", [("k", float("nan")), ("v", float("inf")), ("k", float("-inf"))])
@pytest.mark.parametrize("G", [None, 3])
def test_nonfinite_key_or_value_stays_in_its_head(dtype, which, bad, G, plan):
    plan(segments=G)
    inp = _inputs(dtype, 700)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    clean_o, clean_s = rc.retention_fwd(q, k, v, inp["gamma"], chunk=64)
    t_bad = 300  # chunk 4 of 64-token chunks
    x = (k if which == "k" else v).clone()
    x[1, 2, t_bad, 5] = bad
    args = (q, x, v) if which == "k" else (q, k, x)
    print(f"[nonfinite] {dtype} {which}={bad} at (1, 2, {t_bad}) G={G}", flush=True)
    o, s = rc.retention_fwd(*args, inp["gamma"], chunk=64)
    torch.cuda.synchronize()
    o, s, clean_o, clean_s = (t.float().cpu() for t in (o, s, clean_o, clean_s))
    c0 = (t_bad // 64) * 64
    other = torch.ones(2, 3, dtype=torch.bool)
    other[1, 2] = False
    assert torch.equal(o[other], clean_o[other]) and torch.equal(s[other], clean_s[other]), "leaked into other heads"
    assert torch.equal(o[1, 2, :c0], clean_o[1, 2, :c0]), "earlier chunks changed"
    assert not torch.isfinite(o[1, 2, t_bad:]).all(dim=-1).any(), "a later row of the head stayed finite"
    assert not torch.isfinite(s[1, 2]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_query_touches_only_its_row(dtype):
    inp = _inputs(dtype, 400)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    clean_o, clean_s = rc.retention_fwd(q, k, v, inp["gamma"], chunk=64)
    qb = q.clone()
    qb[0, 1, 77, 3] = float("nan")
    o, s = rc.retention_fwd(qb, k, v, inp["gamma"], chunk=64)
    torch.cuda.synchronize()
    o, clean_o = o.float().cpu(), clean_o.float().cpu()
    assert not torch.isfinite(o[0, 1, 77]).any()
    keep = torch.ones(o.shape[:3], dtype=torch.bool)
    keep[0, 1, 77] = False
    assert torch.equal(o[keep], clean_o[keep]) and torch.equal(s.cpu(), clean_s.cpu())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_decode_and_linear_attention(dtype):
    tdt = wl.torch_dtype(dtype)
    g = torch.Generator().manual_seed(91)
    N, H, d = 4, 2, 64
    q, k, v = (torch.randn((N, H, d), generator=g).to(tdt).cuda() for _ in range(3))
    state = torch.randn((N, H, d, d), generator=g).cuda()
    k[2, 1, 0] = float("inf")
    ref_state = state.clone()
    out = rc.retention_decode_step(q, k, v, [0.9, 0.8], state)
    clean = rc.retention_decode_step(q, torch.where(torch.isinf(k), torch.zeros_like(k), k), v, [0.9, 0.8],
                                     ref_state)
    torch.cuda.synchronize()
    bad = torch.zeros(N, H, dtype=torch.bool)
    bad[2, 1] = True
    assert torch.equal(out[~bad].cpu(), clean[~bad].cpu()) and not torch.isfinite(out[2, 1].float()).all()
    assert torch.equal(state[~bad].cpu(), ref_state[~bad].cpu())
    # linear attention: a NaN value poisons its head from that token on
    w = wl.WORKLOADS["linattn_elu1_bf16"].with_(B=1, H=2, T=500, dtype=dtype)
    li = wl.make_inputs(w, 92)
    lq, lk, lv = (li[n].cuda() for n in ("q", "k", "v"))
    clean_o = rc.linear_attn_fwd(lq, lk, lv)
    lv2 = lv.clone()
    lv2[0, 0, 260, 1] = float("nan")
    o = rc.linear_attn_fwd(lq, lk, lv2)
    torch.cuda.synchronize()
    assert torch.equal(o[0, 1].cpu(), clean_o[0, 1].cpu()) and torch.equal(o[0, 0, :256].cpu(), clean_o[0, 0, :256].cpu())
    assert not torch.isfinite(o[0, 0, 260:].float()).all(dim=-1).any()

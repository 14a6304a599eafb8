"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (CPU only: no call here reaches the device)."""
import ctypes
import os
import re

import pytest

import retention_chunkwise_amd as rc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")


def _lib():
    if not os.path.exists(rc.library_path()):
        pytest.skip("libretention.so not built (run __graft_entry__.build())")
    return rc.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for n in ("retention_fwd", "retention_decode_step", "linear_attn_fwd",
              "retention_last_error", "retention_abi_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), f"libretention.so does not export {name}"


def test_debug_build_exports_the_same_abi():
    """The LDS hazard self-check build (-DRET_DEBUG) is the same C ABI."""
    path = os.path.join(os.path.dirname(rc.library_path()), "libretention_debug.so")
    if not os.path.exists(path):
        pytest.skip("libretention_debug.so not built (run __graft_entry__.build())")
    dbg = rc.load_debug_library()
    for name in _declared_functions():
        assert hasattr(dbg, name), f"libretention_debug.so does not export {name}"
    assert dbg.retention_abi_version() == _lib().retention_abi_version()


def test_abi_version_matches_header():
    text = open(HEADER).read()
    ver = int(re.search(r"#define RET_ABI_VERSION (\d+)", text).group(1))
    assert rc.abi_version() == ver if os.path.exists(rc.library_path()) else True


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((m.group(1), int(m.group(2))) for m in
                  re.finditer(r"#define (RET_\w+) \(?(-?\d+)\)?", text))
    assert consts["RET_F32"] == rc.RET_F32 and consts["RET_BF16"] == rc.RET_BF16
    assert consts["RET_PHI_ELU1"] == rc.RET_PHI_ELU1
    for code, name in rc.ERRORS.items():
        assert consts[name] == code


# ---------------------------------------------------------------- validation
FAKE = 0x10000  # a 16-byte aligned address; never dereferenced: validation fails first


def _gam(vals):
    return (ctypes.c_float * len(vals))(*vals)


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, gamma=_gam([0.9, 0.9]), chunk=64, out=FAKE * 4,
             fs=None, B=1, H=2, T=16, dk=64, dv=64, dtype=rc.RET_F32, ws=None, nws=0)
    a.update(kw)
    return lib.retention_fwd(a["q"], a["k"], a["v"], a["gamma"], a["chunk"], a["out"], a["fs"],
                             a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["ws"], a["nws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(gamma=None), -1),
    (dict(dtype=7), -3),
    (dict(chunk=96), -4),
    (dict(chunk=0), -4),
    (dict(dk=96), -2),
    (dict(dv=32), -2),
    (dict(H=0), -2),
    (dict(B=-1), -2),
    (dict(T=-5), -2),
    (dict(gamma=_gam([0.9, 1.5])), -5),
    (dict(gamma=_gam([0.0, 0.5])), -5),
    (dict(gamma=_gam([float("nan"), 0.5])), -5),
    (dict(q=FAKE + 4), -7),
    (dict(out=FAKE), -8),           # out aliases q
    (dict(fs=FAKE * 4 + 64), -8),   # final_state overlaps out
])
def test_retention_fwd_rejects(kw, code):
    lib = _lib()
    assert _fwd(lib, **kw) == code
    assert rc.last_error() != ""


def test_retention_fwd_too_many_heads():
    lib = _lib()
    H = rc.MAX_HEADS + 1
    assert _fwd(lib, H=H, gamma=_gam([0.9] * H)) == -2


def test_empty_batch_is_accepted_without_device():
    lib = _lib()
    assert _fwd(lib, B=0, q=None, k=None, v=None, out=None) == 0
    assert rc.last_error() == ""


def _dec(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, gamma=_gam([0.9]), state=FAKE * 4, out=FAKE * 64,
             N=2, H=1, dk=64, dv=64, dtype=rc.RET_BF16)
    a.update(kw)
    return lib.retention_decode_step(a["q"], a["k"], a["v"], a["gamma"], a["state"], a["out"],
                                     a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), -1),
    (dict(dtype=3), -3),
    (dict(dk=100), -2),
    (dict(gamma=_gam([-0.1])), -5),
    (dict(state=FAKE * 4 + 8), -7),
    (dict(out=FAKE * 4 + 16), -8),   # out inside state
    (dict(state=FAKE * 3), -8),      # state aliases v
])
def test_decode_rejects(kw, code):
    lib = _lib()
    assert _dec(lib, **kw) == code


def _lin(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, phi=rc.RET_PHI_ELU1, out=FAKE * 4, B=1, H=1, T=8,
             dk=64, dv=64, dtype=rc.RET_BF16, eps=1e-6, ws=None, nws=0)
    a.update(kw)
    return lib.linear_attn_fwd(a["q"], a["k"], a["v"], a["phi"], a["out"], a["B"], a["H"], a["T"],
                               a["dk"], a["dv"], a["dtype"], a["eps"], a["ws"], a["nws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(phi=0), -6),
    (dict(phi=2), -6),
    (dict(v=None), -1),
    (dict(eps=-1.0), -2),
    (dict(eps=float("inf")), -2),
    (dict(dv=48), -2),
    (dict(out=FAKE * 2), -8),
])
def test_linattn_rejects(kw, code):
    lib = _lib()
    assert _lin(lib, **kw) == code


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    if not os.path.exists(rc.library_path()):
        pytest.skip("libretention.so not built")
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        rc.retention_fwd(q, q, q, [0.9])


# ---------------------------------------------------------------- workspace
def test_workspace_sizes():
    lib = _lib()
    # fp32 walks segments too: (G - 1) states per (b, h), no pieces
    n32 = lib.retention_fwd_workspace_bytes(1, 2, 4096, 64, 64, 64, rc.RET_F32)
    assert n32 > 0 and n32 % (64 * 64 * 4 * 2) == 0
    # one chunk: one segment, no workspace
    assert lib.retention_fwd_workspace_bytes(1, 2, 100, 128, 128, 128, rc.RET_BF16) == 0
    # long bf16 sequences are split: (G - 1) * pieces fp32 states per (b, h)
    n = lib.retention_fwd_workspace_bytes(1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    assert n > 0 and n % (128 * 128 * 4 * 32) == 0
    m = lib.linear_attn_workspace_bytes(8, 16, 8192, 64, 64, rc.RET_BF16)
    assert m > 0 and m % ((64 * 64 + 64) * 4 * 128) == 0
    # invalid arguments report 0 (the call itself reports the error)
    assert lib.retention_fwd_workspace_bytes(1, 2, 4096, 96, 64, 64, rc.RET_BF16) == 0


def test_workspace_is_required_and_checked():
    lib = _lib()
    kw = dict(dtype=rc.RET_BF16, T=65536, dk=128, dv=128, chunk=128, gamma=_gam([0.9, 0.9]),
              q=FAKE, k=FAKE * 1024, v=FAKE * 2048, out=FAKE * 4096)
    need = lib.retention_fwd_workspace_bytes(1, 2, 65536, 128, 128, 128, rc.RET_BF16)
    assert need > 0
    assert _fwd(lib, **kw) == -9                                   # none given
    assert _fwd(lib, ws=FAKE * 8192, nws=need - 16, **kw) == -9    # too small
    assert _fwd(lib, ws=FAKE * 8192 + 8, nws=need, **kw) == -7     # misaligned
    assert _fwd(lib, ws=FAKE * 1024, nws=need, **kw) == -8         # overlaps k
    lneed = lib.linear_attn_workspace_bytes(1, 1, 65536, 64, 64, rc.RET_BF16)
    assert lneed > 0
    assert _lin(lib, T=65536, q=FAKE, k=FAKE * 1024, v=FAKE * 2048, out=FAKE * 4096) == -9


# ---------------------------------------------------------------- initial state, phi decode
def _fwd_s(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, gamma=_gam([0.9, 0.9]), chunk=64, init=FAKE * 5,
             out=FAKE * 4, fs=FAKE * 6, B=1, H=2, T=16, dk=64, dv=64, dtype=rc.RET_F32, ws=None, nws=0)
    a.update(kw)
    return lib.retention_fwd_from_state(a["q"], a["k"], a["v"], a["gamma"], a["chunk"], a["init"], a["out"],
                                        a["fs"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["ws"],
                                        a["nws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(init=FAKE * 5 + 8), -7),       # misaligned initial state
    (dict(init=FAKE * 6), -8),           # initial state is the final state buffer
    (dict(init=FAKE * 4), -8),           # initial state overlaps out
    (dict(dk=96), -2),
    (dict(gamma=_gam([0.9, 1.5])), -5),
])
def test_retention_fwd_from_state_rejects(kw, code):
    lib = _lib()
    assert _fwd_s(lib, **kw) == code
    assert "retention_fwd_from_state" in lib.retention_last_error().decode()


def test_retention_fwd_from_state_accepts_shared_input_and_empty_batch():
    lib = _lib()
    # an initial state may alias an input (read only); B = 0 enqueues nothing
    assert _fwd_s(lib, B=0, init=FAKE) == 0


def _lin_s(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, phi=rc.RET_PHI_ELU1, iS=FAKE * 5, iz=FAKE * 7, out=FAKE * 4,
             fS=FAKE * 6, fz=FAKE * 8, B=1, H=1, T=8, dk=64, dv=64, dtype=rc.RET_F32, eps=1e-6, ws=None, nws=0)
    a.update(kw)
    return lib.linear_attn_fwd_from_state(a["q"], a["k"], a["v"], a["phi"], a["iS"], a["iz"], a["out"], a["fS"],
                                          a["fz"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["eps"],
                                          a["ws"], a["nws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(iz=FAKE * 7 + 4), -7),
    (dict(fz=FAKE * 6), -8),            # final z inside final S
    (dict(fS=FAKE * 5), -8),            # final S is the initial S
    (dict(fz=FAKE * 7), -8),            # final z is the initial z
    (dict(phi=3), -6),
    (dict(eps=-1.0), -2),
])
def test_linattn_fwd_from_state_rejects(kw, code):
    lib = _lib()
    assert _lin_s(lib, **kw) == code
    assert "linear_attn_fwd_from_state" in lib.retention_last_error().decode()


def _ldec(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, phi=rc.RET_PHI_ELU1, S=FAKE * 4, z=FAKE * 5, out=FAKE * 6,
             N=2, H=3, dk=64, dv=64, dtype=rc.RET_BF16, eps=1e-6)
    a.update(kw)
    return lib.linear_attn_decode_step(a["q"], a["k"], a["v"], a["phi"], a["S"], a["z"], a["out"], a["N"],
                                       a["H"], a["dk"], a["dv"], a["dtype"], a["eps"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(z=None), -1),
    (dict(S=None), -1),
    (dict(z=FAKE * 5 + 4), -7),
    (dict(z=FAKE * 4), -8),             # z inside S
    (dict(out=FAKE * 5), -8),           # out overlaps z
    (dict(S=FAKE), -8),                 # S overlaps q
    (dict(phi=0), -6),
    (dict(dk=32), -2),
    (dict(dtype=7), -3),
    (dict(eps=float("inf")), -2),
])
def test_linattn_decode_rejects(kw, code):
    lib = _lib()
    assert _ldec(lib, **kw) == code
    assert "linear_attn_decode_step" in lib.retention_last_error().decode()


def test_linattn_decode_empty_is_accepted():
    lib = _lib()
    assert _ldec(lib, N=0) == 0


# ---------------------------------------------------------------- backward
def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, gamma=_gam([0.9, 0.9]), chunk=64, do=FAKE * 4, dq=FAKE * 5,
             dk=FAKE * 6, dv=FAKE * 7, B=1, H=2, T=16, d_k=64, d_v=64, dtype=rc.RET_F32, ws=None, nws=0)
    a.update(kw)
    return lib.retention_bwd(a["q"], a["k"], a["v"], a["gamma"], a["chunk"], a["do"], a["dq"], a["dk"], a["dv"],
                             a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["dtype"], a["ws"], a["nws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), -1),
    (dict(dv=None), -1),
    (dict(gamma=None), -1),
    (dict(dtype=5), -3),
    (dict(chunk=32), -4),
    (dict(gamma=_gam([0.9, 0.0])), -5),
    (dict(d_v=96), -2),
    (dict(dq=FAKE * 5 + 4), -7),
    (dict(dq=FAKE), -8),                 # dq is q
    (dict(dv=FAKE * 4), -8),             # dv overlaps dout
    (dict(dk=FAKE * 5), -8),             # dk is dq
    (dict(T=65536, dtype=rc.RET_BF16, d_k=128, d_v=128, chunk=128, q=FAKE, k=FAKE * 1024, v=FAKE * 2048,
          do=FAKE * 3072, dq=FAKE * 4096, dk=FAKE * 5120, dv=FAKE * 6144), -9),   # no workspace
])
def test_retention_bwd_rejects(kw, code):
    lib = _lib()
    assert _bwd(lib, **kw) == code
    assert "retention_bwd" in lib.retention_last_error().decode()


def test_retention_bwd_workspace_and_empty_batch():
    lib = _lib()
    n = lib.retention_bwd_workspace_bytes(1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    assert n > 0 and n == lib.retention_fwd_workspace_bytes(1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    # dq walks with widths (dv, dk), dv with (dk, dv): the larger plan sets the size
    n2 = lib.retention_bwd_workspace_bytes(1, 4, 4096, 64, 128, 64, rc.RET_F32)
    assert n2 >= lib.retention_fwd_workspace_bytes(1, 4, 4096, 64, 128, 64, rc.RET_F32)
    assert _bwd(lib, B=0) == 0


# ---------------------------------------------------------------- normalised forward
def _nrm(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, gamma=_gam([0.9, 0.9]), chunk=64, norm=rc.RET_NORM_GROUP, eps=1e-5,
             out=FAKE * 4, B=1, H=2, T=16, dk=64, dv=64, dtype=rc.RET_BF16, ws=None, nws=0)
    a.update(kw)
    return lib.retention_fwd_normalized(a["q"], a["k"], a["v"], a["gamma"], a["chunk"], a["norm"], a["eps"],
                                        a["out"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["dtype"], a["ws"],
                                        a["nws"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(norm=0), -2),
    (dict(norm=3), -2),
    (dict(eps=-1.0), -2),
    (dict(eps=0.0), -2),  # GroupNorm of a constant row needs eps > 0
    (dict(chunk=96), -4),
    (dict(gamma=_gam([0.9, 2.0])), -5),
    (dict(out=FAKE * 2), -8),
    (dict(v=FAKE * 3 + 2), -7),
    (dict(T=65536, dk=128, dv=128, q=FAKE, k=FAKE * 1024, v=FAKE * 2048, out=FAKE * 4096), -9),
])
def test_retention_fwd_normalized_rejects(kw, code):
    lib = _lib()
    assert _nrm(lib, **kw) == code
    assert "retention_fwd_normalized" in lib.retention_last_error().decode()


def test_retention_fwd_normalized_rowsum_takes_eps_zero():
    lib = _lib()
    # eps only enters GroupNorm; the floor alone accepts 0 (validation passes, then B = 0 is a no-op)
    assert _nrm(lib, norm=rc.RET_NORM_ROWSUM, eps=0.0, B=0) == 0
    assert _nrm(lib, norm=rc.RET_NORM_GROUP, eps=0.0, B=0) == -2


def test_retention_fwd_normalized_workspace():
    lib = _lib()
    n = lib.retention_fwd_normalized_workspace_bytes(1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    assert n > 0 and n % ((128 * 128 + 128) * 4) == 0
    # fp32: the value-slice walk's segment states, with a normaliser slot each
    n32 = lib.retention_fwd_normalized_workspace_bytes(4, 8, 2048, 64, 64, 64, rc.RET_F32)
    assert n32 > 0 and n32 % ((64 * 64 + 64) * 4 * 32) == 0
    assert lib.retention_fwd_normalized_workspace_bytes(1, 32, 4096, 64, 64, 64, 7) == 0
    assert _nrm(lib, B=0) == 0
    # the floor alone has no whole-row requirement
    assert _nrm(lib, B=0, dtype=rc.RET_F32, dk=128, dv=128, norm=rc.RET_NORM_ROWSUM) == 0


# ---------------------------------------------------------------- gated linear attention
def _gla(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, lg=FAKE * 4, out=FAKE * 5, fs=None, B=1, H=2, T=16, dk=64, dv=64,
             dtype=rc.RET_F32)
    a.update(kw)
    return lib.gla_fwd(a["q"], a["k"], a["v"], a["lg"], a["out"], a["fs"], a["B"], a["H"], a["T"], a["dk"],
                       a["dv"], a["dtype"], a.get("ws"), a.get("nws", 0), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(lg=None), -1),
    (dict(dk=32), -2),
    (dict(lg=FAKE * 4 + 4), -7),
    (dict(out=FAKE * 4), -8),            # out is the gate tensor
    (dict(fs=FAKE * 5), -8),             # final state overlaps out
])
def test_gla_rejects(kw, code):
    lib = _lib()
    assert _gla(lib, **kw) == code
    assert "gla_fwd" in lib.retention_last_error().decode()


def test_gla_empty_batch():
    assert _gla(_lib(), B=0) == 0
    assert _gla(_lib(), B=0, dtype=rc.RET_BF16) == 0


def test_gla_bf16_gates_stay_fp32():
    """bf16 q, k, v and out, fp32 log-gates: an output that starts where a
    bf16-sized gate tensor would end still overlaps the fp32 gates."""
    lib = _lib()
    nq16 = 2 * 16 * 64 * 2  # bytes of a [1, 2, 16, 64] bf16 tensor; the fp32 gates take twice that
    assert _gla(lib, dtype=rc.RET_BF16, lg=FAKE * 4, out=FAKE * 4 + nq16) == -8
    assert "log_gate" in lib.retention_last_error().decode()


def test_gla_workspace():
    lib = _lib()
    n = lib.gla_fwd_workspace_bytes(4, 8, 2048, 64, 64, rc.RET_F32)
    assert n > 0 and n % ((64 * 64 + 64) * 4 * 32) == 0
    assert lib.gla_fwd_workspace_bytes(4, 8, 2048, 64, 64, rc.RET_BF16) == n  # fp32 states either way
    big = 1 << 28  # 256 MiB apart: no overlap between the fake tensors
    assert _gla(lib, B=4, H=8, T=2048, q=big, k=2 * big, v=3 * big, lg=4 * big, out=5 * big) == -9


# ------------------------------------------------- retention_bwd_from_fwd validation
M64 = 0x4000000  # 64 MiB: buffers this far apart do not overlap at the sizes below


def _bwd_ff(lib, **kw):
    a = dict(q=M64, k=2 * M64, v=3 * M64, gamma=_gam([0.9, 0.9]), chunk=128, do=4 * M64, fws=None, nfws=0,
             dq=5 * M64, dk=6 * M64, dv=7 * M64, B=1, H=2, T=65536, d_k=128, d_v=128, dtype=rc.RET_BF16,
             ws=8 * M64, nws=0)
    a.update(kw)
    return lib.retention_bwd_from_fwd(a["q"], a["k"], a["v"], a["gamma"], a["chunk"], a["do"], a["fws"], a["nfws"],
                                      a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["T"], a["d_k"], a["d_v"],
                                      a["dtype"], a["ws"], a["nws"], None)


def test_bwd_from_fwd_checks_the_forward_workspace():
    lib = _lib()
    need_b = lib.retention_bwd_workspace_bytes(1, 2, 65536, 128, 128, 128, rc.RET_BF16)
    need_f = lib.retention_fwd_workspace_bytes(1, 2, 65536, 128, 128, 128, rc.RET_BF16)
    assert need_b > 0 and need_f > 0 and need_b < M64 and need_f < M64
    kw = dict(nws=need_b)
    assert _bwd_ff(lib, **kw) == -9                                          # forward needed one: NULL
    assert _bwd_ff(lib, fws=9 * M64, nfws=need_f - 16, **kw) == -9           # too small
    assert _bwd_ff(lib, fws=9 * M64 + 8, nfws=need_f, **kw) == -7            # misaligned
    assert _bwd_ff(lib, fws=5 * M64, nfws=need_f, **kw) == -8                # overlaps dq
    assert _bwd_ff(lib, fws=8 * M64, nfws=need_f, **kw) == -8                # is the backward's workspace
    assert _bwd_ff(lib, fws=9 * M64, nfws=need_f, nws=need_b - 16) == -9     # the backward's own is short
    assert _bwd_ff(lib, fws=9 * M64, nfws=need_f, dq=M64, **kw) == -8        # dq overlaps q, as retention_bwd
    assert _bwd_ff(lib, B=0, fws=9 * M64, nfws=need_f, **kw) == 0            # empty batch: nothing to do


def test_very_long_fp32_segments_stay_under_2_gib():
    """The fp32 segment-state kernel uses 32-bit offsets within a segment: a
    64M-token head at d = 128 takes more segments so that each segment's K and
    V stay under 2 GiB (the plan shows in the workspace: G - 1 state slots)."""
    lib = _lib()
    T, d, chunk = 1 << 26, 128, 64
    n = lib.retention_fwd_workspace_bytes(1, 1, T, d, d, chunk, rc.RET_F32)
    slots = n // (d * d * 4)
    assert n == slots * d * d * 4 and slots >= 1
    G = slots + 1
    nch = T // chunk
    cps = -(-nch // G)
    assert -(-nch // cps) == G
    assert cps * chunk * d * 4 < 2 ** 31
    # a shorter head keeps the usual plan
    m = lib.retention_fwd_workspace_bytes(1, 1, 1 << 20, d, d, chunk, rc.RET_F32)
    assert 0 < m <= 15 * d * d * 4


# ---------------------------------------------------------------- plan override
def test_plan_override_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"#define (RET_PATH_\w+) (\d+)", text))
    assert consts == {"RET_PATH_AUTO": rc.RET_PATH["auto"], "RET_PATH_SLICE": rc.RET_PATH["slice"],
                      "RET_PATH_SEGMENT": rc.RET_PATH["segment"]}


def test_plan_override_sets_the_workspace_plan_and_is_restored():
    lib = _lib()
    args = (1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    auto = lib.retention_fwd_workspace_bytes(*args)
    slot = 128 * 128 * 4
    assert auto > 0 and auto % (32 * slot) == 0
    with rc.plan_override(segments=1):
        assert lib.retention_fwd_workspace_bytes(*args) == 0  # one segment: no partial states
    with rc.plan_override(segments=3):
        n3 = lib.retention_fwd_workspace_bytes(*args)  # (G-1) x pieces slots per (b, h)
        assert n3 > 0 and n3 % (32 * 2 * slot) == 0 and n3 != auto
    with rc.plan_override(path="slice", segments=1):
        assert lib.retention_fwd_workspace_bytes(*args) == 0
    assert lib.retention_fwd_workspace_bytes(*args) == auto  # the context manager restored the automatic plan


@pytest.mark.parametrize("kw,code", [(dict(path="diagonal"), None), (dict(segments=-1), -2),
                                     (dict(walk_nt=3), -2), (dict(lin_chunk=32), -4)])
def test_plan_override_rejects_bad_values_and_keeps_the_previous_one(kw, code):
    lib = _lib()
    args = (1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    auto = lib.retention_fwd_workspace_bytes(*args)
    rc.set_plan_override(segments=1)
    try:
        if code is None:
            with pytest.raises(ValueError):
                rc.set_plan_override(**kw)
        else:
            with pytest.raises(rc.RetentionError) as ei:
                rc.set_plan_override(**kw)
            assert ei.value.code == code
        assert lib.retention_fwd_workspace_bytes(*args) == 0  # still G = 1
    finally:
        rc.set_plan_override()
    assert lib.retention_fwd_workspace_bytes(*args) == auto


def test_plan_override_is_per_thread():
    import threading

    lib = _lib()
    args = (1, 32, 65536, 128, 128, 128, rc.RET_BF16)
    auto = lib.retention_fwd_workspace_bytes(*args)
    seen = {}

    def other():
        seen["before"] = lib.retention_fwd_workspace_bytes(*args)
        rc.set_plan_override(segments=3)
        seen["after"] = lib.retention_fwd_workspace_bytes(*args)

    with rc.plan_override(segments=1):
        t = threading.Thread(target=other)
        t.start()
        t.join()
        assert lib.retention_fwd_workspace_bytes(*args) == 0
    assert seen["before"] == auto and seen["after"] not in (0, auto)
    assert lib.retention_fwd_workspace_bytes(*args) == auto


# ---------------------------------------------------------------- allocation-free forward
def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, gamma=_gam([0.9, 0.9]), chunk=64, out=FAKE * 4, fs=FAKE * 6, B=1, H=2,
             T=16, dk=64, dv=64, dtype=rc.RET_BF16)
    a.update(kw)
    return lib.retention_fwd_noalloc(a["q"], a["k"], a["v"], a["gamma"], a["chunk"], a["out"], a["fs"], a["B"],
                                     a["H"], a["T"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -3),
    (dict(chunk=96), -4),
    (dict(gamma=_gam([0.9, 2.0])), -5),
    (dict(out=FAKE * 2), -8),
    (dict(v=FAKE * 3 + 2), -7),
    (dict(q=None), -1),
])
def test_retention_fwd_noalloc_rejects(kw, code):
    lib = _lib()
    assert _noalloc(lib, **kw) == code
    assert "retention_fwd_noalloc" in lib.retention_last_error().decode()


def test_retention_fwd_noalloc_limit_is_checked_before_any_device_call():
    """Sizes whose segment states exceed the library's 32 MiB array are
    refused on the host (this runs without a GPU); B = 0 is a no-op."""
    lib = _lib()
    text = open(HEADER).read()
    limit = int(re.search(r"#define RET_NOALLOC_MAX_WORKSPACE (\d+)", text).group(1))
    assert limit == 32 << 20
    G = 1 << 30  # 1 GiB apart: the [1, 64, 65536, 128] bf16 tensors do not overlap
    big = dict(q=G, k=2 * G, v=3 * G, out=4 * G, fs=5 * G, H=64, T=65536, dk=128, dv=128, chunk=128,
               gamma=_gam([0.9] * 64))
    with rc.plan_override(segments=16):
        assert lib.retention_fwd_workspace_bytes(1, 64, 65536, 128, 128, 128, rc.RET_BF16) > limit
        assert _noalloc(lib, **big) == -9
        assert "retention_fwd with a workspace" in lib.retention_last_error().decode()
    assert _noalloc(lib, B=0) == 0

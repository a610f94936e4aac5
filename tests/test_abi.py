"""CPU checks of the C-ABI library: it loads, exports every function that
include/treeverify.h declares, and rejects bad host-side arguments before
touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import tree_speculative_verification_attn_amd as tv_pkg

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "treeverify.h")
TV_OK, TV_EINVAL, TV_ETOOBIG, TV_EDTYPE, TV_EWORKSPACE, TV_ESCRATCH = 0, 1, 2, 3, 4, 6


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tv_pkg.lib_path):
        from tree_speculative_verification_attn_amd import build
        build.build()
    return tv_pkg.lib()


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("tree_build_mask", "tree_attn_verify", "tree_verify_greedy", "tree_verify_mss",
              "kv_commit_accepted"):
        assert n in names
    assert set(names) == set(tv_pkg.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(7):
        assert tv_pkg.tv_status_string(code) != "unknown status"
    assert tv_pkg.tv_status_string(99) == "unknown status"


def _p(v=1):
    return ctypes.c_void_p(0x1000 * v)      # never dereferenced: calls return first


def test_host_argument_checks(L):
    assert L.tree_build_mask(1, 65, _p(), _p(), _p(), _p(), _p(), None) == TV_ETOOBIG
    assert L.tree_build_mask(-1, 3, _p(), _p(), _p(), _p(), _p(), None) == TV_EINVAL
    assert L.tree_build_mask(2, 3, None, _p(), _p(), _p(), _p(), None) == TV_EINVAL
    assert L.tree_build_mask(0, 3, None, None, None, None, None, None) == TV_OK
    args = dict(B=2, N=5, H=2, D=128, scale=0.1)

    def attn(dt=1, D=128, N=5, bs=16, ws=None, ws_bytes=0, mb=4):
        return L.tree_attn_verify(dt, 2, N, 2, D, 0.1, _p(), _p(), _p(), 10, bs, _p(), mb, _p(), _p(),
                                  _p(), _p(), ws, ws_bytes, None)
    assert attn(dt=7) == TV_EDTYPE
    assert attn(D=96) == TV_EINVAL
    assert attn(bs=8) == TV_EINVAL
    assert attn(N=70) == TV_ETOOBIG
    assert attn(N=0) == TV_OK
    need = L.tree_attn_verify_workspace(1, 2, 5, 2, 128, 400)
    assert need > 0
    assert attn(mb=400, ws=None) == TV_EWORKSPACE
    assert attn(mb=400, ws=_p(), ws_bytes=need - 1) == TV_EWORKSPACE
    assert L.tree_attn_verify_workspace(1, 2, 5, 2, 128, 4) == 0     # one chunk: no workspace
    del args

    def fused(dt=1, B=2, D=128, N=5, bs=16, ws=None, ws_bytes=0, mb=4, par=True, anc=True, ch=True, st=True):
        return L.tree_mask_attn_verify(dt, B, N, 2, D, 0.1, _p(), _p(), _p(), 10, bs, _p(), mb, _p(),
                                       _p() if par else None, _p() if anc else None, _p() if ch else None,
                                       _p(), _p() if st else None, _p(), ws, ws_bytes, None)
    assert fused(dt=7) == TV_EDTYPE
    assert fused(D=96) == TV_EINVAL
    assert fused(bs=8) == TV_EINVAL
    assert fused(N=70) == TV_ETOOBIG
    assert fused(par=False) == TV_EINVAL
    assert fused(anc=False) == TV_EINVAL
    assert fused(ch=False) == TV_EINVAL
    assert fused(st=False) == TV_EINVAL
    assert fused(N=0, ch=False) == TV_EINVAL
    assert fused(B=0, par=False, ch=False) == TV_OK
    assert fused(mb=400) == TV_EWORKSPACE
    assert fused(mb=400, ws=_p(), ws_bytes=need - 1) == TV_EWORKSPACE

    wsv = L.tree_verify_workspace(2, 5, 1000)
    assert wsv > 0
    assert L.tree_verify_workspace(2, 65, 1000) == 0
    assert L.tree_verify_greedy(2, 5, 0, _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), wsv, None) == TV_EINVAL
    assert L.tree_verify_greedy(2, 5, 1000, _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), wsv - 1,
                                None) == TV_EWORKSPACE
    assert L.tree_verify_mss(2, 5, 1000, 0, _p(), _p(), _p(), _p(), _p(), _p(), 1, 0, _p(), _p(), _p(),
                             None, _p(), wsv, None) == TV_EINVAL
    assert L.tree_verify_mss(2, 5, 1 << 21, 3, _p(), _p(), _p(), _p(), _p(), _p(), 1, 0, _p(), _p(),
                             _p(), None, _p(), wsv, None) == TV_EINVAL

    def noalloc(B=2, N=5, V=1000, R=3, logits=True):
        return L.tree_verify_mss_noalloc(B, N, V, R, _p() if logits else None, _p(), _p(), _p(), _p(), _p(),
                                         1, 0, _p(), _p(), _p(), None, None)
    assert noalloc(R=0) == TV_EINVAL
    assert noalloc(V=1 << 21) == TV_EINVAL
    assert noalloc(N=65) == TV_ETOOBIG
    assert noalloc(logits=False) == TV_EINVAL
    assert noalloc(B=0) == TV_OK
    # the fixed scratch holds 1260 requests' exchange words at V = 32000, 123 at V = 2^20
    assert L.tree_verify_workspace(1260, 5, 32000) <= tv_pkg.TV_NOALLOC_SCRATCH_BYTES
    assert L.tree_verify_workspace(1261, 5, 32000) > tv_pkg.TV_NOALLOC_SCRATCH_BYTES
    assert noalloc(B=1261, V=32000) == TV_ESCRATCH
    assert L.tree_verify_workspace(123, 5, 1 << 20) <= tv_pkg.TV_NOALLOC_SCRATCH_BYTES
    assert noalloc(B=124, V=1 << 20) == TV_ESCRATCH
    assert L.kv_commit_accepted(5, 2, 5, 2, 128, _p(), _p(), 10, 16, _p(), 4, _p(), _p(), _p(), _p(),
                                None) == TV_EDTYPE
    assert L.kv_commit_accepted(1, 2, 65, 2, 128, _p(), _p(), 10, 16, _p(), 4, _p(), _p(), _p(), _p(),
                                None) == TV_ETOOBIG
    assert L.kv_commit_accepted(1, 2, 5, 2, 128, None, _p(), 10, 16, _p(), 4, _p(), _p(), _p(), _p(),
                                None) == TV_EINVAL

    def mss_commit(N=5, R=3, dt=1, H=2, D=128, bs=16, kc=True, ws_bytes=None):
        return L.tree_verify_mss_commit(2, N, 1000, R, _p(), _p(), _p(), _p(), _p(), _p(), 1, 0, _p(), _p(),
                                        _p(), None, _p(), wsv if ws_bytes is None else ws_bytes, dt, H, D,
                                        _p() if kc else None, _p(), 10, bs, _p(), 4, _p(), None)
    assert mss_commit(dt=5) == TV_EDTYPE
    assert mss_commit(N=65) == TV_ETOOBIG
    assert mss_commit(R=0) == TV_EINVAL
    assert mss_commit(D=96) == TV_EINVAL
    assert mss_commit(H=0) == TV_EINVAL
    assert mss_commit(bs=8) == TV_EINVAL
    assert mss_commit(kc=False) == TV_EINVAL
    assert mss_commit(ws_bytes=wsv - 1) == TV_EWORKSPACE

    def multi(S=3, R=2, pn=True):
        return L.tree_verify_mss_multi(2, 5, S, 1000, R, _p(), _p(), _p() if pn else None, _p(), _p(), _p(), _p(),
                                       1, 0, _p(), _p(), _p(), None, _p(), wsv, None)
    assert multi(S=65) == TV_ETOOBIG
    assert multi(S=-1) == TV_EINVAL
    assert multi(R=0) == TV_EINVAL
    assert multi(pn=False) == TV_EINVAL
    assert L.tree_verify_mss_multi(2, 5, 3, 1000, 2, _p(), _p(), _p(), _p(), _p(), _p(), _p(), 1, 0, _p(), _p(),
                                   _p(), None, _p(), wsv - 1, None) == TV_EWORKSPACE


def test_binding_names_match_exports():
    for n in tv_pkg.EXPORTS:
        assert callable(getattr(tv_pkg, n))

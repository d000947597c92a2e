"""CPU checks of the C ABI: the library loads, exports every entry point
include/fa.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

from exact_io_aware_69_amd import _lib
from tests.visitmap import expected_visits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:int|const char\*)\s+(fa_\w+)\s*\(", text, flags=re.M))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert decl == set(_lib.SIGNATURES), decl ^ set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = declared_functions() - exported
    assert not missing, missing
    lib = _lib.lib()
    for name in declared_functions():
        assert getattr(lib, name) is not None


def test_status_strings():
    for code, name in _lib.STATUS.items():
        assert _lib.fa_status_str(code).startswith(name)
    assert "unknown" in _lib.fa_status_str(12345)


def test_tile_config():
    for d in (64, 128):
        for causal in (0, 1):
            for ps in (0, 1, 2):
                st, bm, bn = _lib.fa_tile_config(ps, d, causal)
                assert st == 0 and bm > 0 and bn > 0 and bm % 32 == 0 and bn % 32 == 0
                assert 128 % bm == 0 or bm % 128 == 0
                assert 128 % bn == 0
    # the d = 128 dQ kernel streams 64-key tiles only when causal
    assert _lib.fa_tile_config(2, 128, 1)[2] == 64 and _lib.fa_tile_config(2, 128, 0)[2] == 32
    assert _lib.fa_tile_config(2, 64, 0)[2] == _lib.fa_tile_config(2, 64, 1)[2] == 64
    assert _lib.fa_tile_config(0, 96, 0)[0] == -3
    assert _lib.fa_tile_config(7, 64, 0)[0] == -2


def test_workspace_size_is_linear_in_N():
    # two fp32 values (D and lse * log2 e) per row, rows padded to 128 per
    # head, plus the block-sparse schedule: three int32 per (head, 128-row
    # mask block)
    st, a = _lib.fa_bwd_workspace_size(2, 16, 8192, 64)
    sched = 16 * 3 * 64 * 4
    assert st == 0 and a >= 2 * 16 * 8192 * 8 + sched and a < 2 * 16 * 8192 * 8 + sched + 768
    assert _lib.fa_bwd_workspace_size(1, 1, 1, 64)[1] >= 128 * 8 + 3 * 4
    st, b = _lib.fa_bwd_workspace_size(2, 16, 16384, 64)
    assert b == 2 * a
    assert _lib.fa_bwd_workspace_size(0, 1, 1, 64)[0] == -2
    assert _lib.fa_bwd_workspace_size(1, 1, 1, 80)[0] == -3


def fwd_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, causal=0, scale=0.125, stream=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -2), (dict(H=-1), -2), (dict(N=0), -2), (dict(N=1 << 25), -2),
    (dict(d=96), -3), (dict(d=0), -3),
    (dict(scale=0.0), -4), (dict(scale=-1.0), -4), (dict(scale=math.nan), -4), (dict(scale=math.inf), -4),
    (dict(q=FAKE + 2), -8), (dict(o=FAKE + 8), -8),
])
def test_forward_argument_errors(kw, code):
    a = fwd_args(**kw)
    assert _lib.fa_fwd(**a) == code
    assert _lib.fa_fwd_blocksparse(**{**a, "block_mask": FAKE}) == code


def test_blocksparse_requires_mask():
    assert _lib.fa_fwd_blocksparse(**fwd_args(), block_mask=None) == -6


def bwd_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2, N=100, d=128,
             causal=1, scale=0.09, workspace=FAKE, workspace_bytes=1 << 20, stream=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), -1), (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1), (dict(lse=None), -1),
    (dict(N=0), -2), (dict(d=32), -3), (dict(scale=0.0), -4),
    (dict(workspace=None), -5), (dict(workspace_bytes=100), -5), (dict(workspace_bytes=2 * 100 * 4 - 1), -5),
    (dict(dk=FAKE + 4), -8), (dict(workspace=FAKE + 4), -8),
])
def test_backward_argument_errors(kw, code):
    a = bwd_args(**kw)
    assert _lib.fa_bwd(**a) == code
    a2 = dict(a)
    ws, wb, st = a2.pop("workspace"), a2.pop("workspace_bytes"), a2.pop("stream")
    assert _lib.fa_bwd_blocksparse(**a2, block_mask=FAKE, workspace=ws, workspace_bytes=wb, stream=st) == code


def test_backward_blocksparse_requires_mask():
    a = bwd_args()
    ws, wb, st = a.pop("workspace"), a.pop("workspace_bytes"), a.pop("stream")
    assert _lib.fa_bwd_blocksparse(**a, block_mask=None, workspace=ws, workspace_bytes=wb, stream=st) == -6


def test_debug_entry_points_require_maps():
    a = fwd_args()
    assert _lib.fa_fwd_debug_visits(**a, block_mask=None, visited=None) == -1
    b = bwd_args()
    ws, wb, st = b.pop("workspace"), b.pop("workspace_bytes"), b.pop("stream")
    assert _lib.fa_bwd_debug_visits(**b, block_mask=None, workspace=ws, workspace_bytes=wb, visited_kv=None,
                                    visited_q=FAKE, stream=st) == -1


# ---------------------------------------------------------------- expected visit maps (host logic)

def test_expected_visits_dense_and_causal_counts():
    # dense: every tile pair; causal with equal square tiles: lower triangle incl. diagonal
    v = expected_visits(512, 128, 128, False)
    assert v.sum() == 16
    v = expected_visits(512, 128, 128, True)
    assert v.sum() == 4 * 5 // 2
    # causal, bm=128, bn=64: query tile i sees key tiles 0..2i+1
    v = expected_visits(512, 128, 64, True)[0]
    for i in range(4):
        assert list(np.nonzero(v[i])[0]) == list(range(2 * i + 2))
    # ragged tail: N=130 -> 2 query tiles; the last one holds queries 128,129
    v = expected_visits(130, 128, 64, True)[0]
    assert v.shape == (2, 3) and v[1].tolist() == [1, 1, 1] and v[0].tolist() == [1, 1, 0]


def test_expected_visits_blocksparse():
    mask = np.array([[[1, 0, 1], [0, 1, 0], [1, 1, 1]]], dtype=np.uint8)
    v = expected_visits(300, 128, 64, False, mask)[0]
    assert v.shape == (3, 5)
    assert v[0].tolist() == [1, 1, 0, 0, 1]
    assert v[1].tolist() == [0, 0, 1, 1, 0]
    assert v[2].tolist() == [1, 1, 1, 1, 1]
    v = expected_visits(300, 128, 64, True, mask)[0]
    assert v[0].tolist() == [1, 1, 0, 0, 0]  # block (0,2) kept but entirely above the diagonal
    # key-major map for the dK/dV kernel: [key tile][query tile]
    vk = expected_visits(300, 64, 128, False, mask, key_major=True)[0]
    assert vk.shape == (3, 5) and vk[0].tolist() == [1, 1, 0, 0, 1]


def test_fwd_tiles_rejects_unsupported_configs_before_launch():
    for bm, bn in [(64, 64), (256, 32), (128, 256), (512, 64), (0, 0)]:
        assert _lib.fa_fwd_tiles(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 0, 0.125, None, bm, bn, None) == -2


def test_std_fwd_argument_errors():
    st, need = _lib.fa_std_workspace_size(1, 2, 256, 64)
    assert st == 0 and need >= 2 * 256 * 256 * 6
    assert _lib.fa_std_workspace_size(1, 1, 16385, 64)[0] == -2          # N above the baseline's limit
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, N=256, d=64, causal=0, scale=0.125,
                block_mask=None, workspace=FAKE, workspace_bytes=need, stream=None)
    assert _lib.fa_std_fwd(**{**args, "workspace_bytes": need - 1}) == -5
    assert _lib.fa_std_fwd(**{**args, "workspace": None}) == -5
    assert _lib.fa_std_fwd(**{**args, "q": None}) == -1
    assert _lib.fa_std_fwd(**{**args, "d": 96}) == -3
    assert _lib.fa_std_fwd(**{**args, "N": 16385}) == -2
    assert _lib.fa_std_fwd(**{**args, "o": FAKE + 2}) == -8


def test_fa1_fwd_argument_errors():
    st, need = _lib.fa_fa1_workspace_size(2, 3, 300, 128)
    # fp32 output rows plus 4 per-wave (max, sum) pairs per row, linear in N
    assert st == 0 and need >= 2 * 3 * 300 * (128 + 8) * 4 and need < 2 * 3 * 300 * (128 + 8) * 4 + 768
    assert _lib.fa_fa1_workspace_size(1, 1, 0, 64)[0] == -2
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, H=3, N=300, d=128, causal=1, scale=0.125,
                seq_groups=1, workspace=FAKE, workspace_bytes=need, stream=None)
    assert _lib.fa_fwd_fa1(**{**args, "seq_groups": 0}) == -2
    assert _lib.fa_fwd_fa1(**{**args, "workspace_bytes": need - 1}) == -5
    assert _lib.fa_fwd_fa1(**{**args, "workspace": None}) == -5
    assert _lib.fa_fwd_fa1(**{**args, "lse": None}) == -1
    assert _lib.fa_fwd_fa1(**{**args, "d": 80}) == -3
    assert _lib.fa_fwd_fa1(**{**args, "scale": 0.0}) == -4
    assert _lib.fa_fwd_fa1(**{**args, "workspace": FAKE + 4}) == -8


def test_dropout_argument_errors():
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, N=64, d=64, causal=0, scale=0.125,
                block_mask=None, dropout_p=0.1, seed=1, offset=0, stream=None)
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        assert _lib.fa_fwd_dropout(**{**args, "dropout_p": bad}) == -9
    assert _lib.fa_fwd_dropout(**{**args, "q": None}) == -1
    assert _lib.fa_fwd_dropout(**{**args, "d": 96}) == -3
    st, need = _lib.fa_bwd_workspace_size(1, 2, 64, 64)
    bargs = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=2, N=64, d=64,
                 causal=1, scale=0.125, block_mask=None, dropout_p=0.1, seed=1, offset=0, workspace=FAKE,
                 workspace_bytes=need, stream=None)
    assert _lib.fa_bwd_dropout(**{**bargs, "dropout_p": 1.0}) == -9
    assert _lib.fa_bwd_dropout(**{**bargs, "workspace_bytes": need - 1}) == -5
    assert _lib.fa_dropout_keep(1, 1, 8, 0.5, 1, 0, None, None) == -1
    assert _lib.fa_dropout_keep(1, 1, 0, 0.5, 1, 0, FAKE, None) == -2
    assert _lib.fa_dropout_keep(1, 1, 8, -1.0, 1, 0, FAKE, None) == -9
    assert "dropout" in _lib.fa_status_str(-9)


def test_build_id_matches_sources():
    from exact_io_aware_69_amd import _srcid
    assert _lib.fa_build_id() == _srcid.source_id()


def test_stale_library_is_refused(monkeypatch):
    from exact_io_aware_69_amd import _srcid
    monkeypatch.setattr(_srcid, "source_id", lambda: "0000000000000000")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.StaleLibraryError):
        _lib.lib()


def test_every_declaration_cites_a_passage_or_says_none():
    """Each entry point's comment block names the page passage that defines
    its operation, or states that no passage defines it."""
    text = open(HEADER).read()
    cites = ("FlashAttention-2 review", "Stanford FlashAttention summary", "PagedAttention",
             "no passage", "callers that cannot allocate")
    for name in declared_functions():
        pos = re.search(r"^\s*(?:int|const char\*)\s+" + name + r"\s*\(", text, flags=re.M).start()
        block = text[text.rfind("/*", 0, pos):text.rfind("*/", 0, pos) + 2]
        flat = " ".join(w for w in block.split() if w != "*")
        assert any(c in flat for c in cites), (name, flat[:200])


def test_noalloc_rejects_before_any_hip_call():
    """fa_bwd_noalloc checks its arguments and the scratch limit (16 MiB of
    workspace) before touching the GPU, so these run without one."""
    f = _lib.fa_bwd_noalloc
    ptrs = [FAKE] * 6 + [FAKE] * 3
    # 2 heads x 4M rows need far more than 16 MiB of workspace
    assert f(*ptrs, 2, 1, 1 << 22, 64, 0, 0.125, None, None) == -5
    st, need = _lib.fa_bwd_workspace_size(32, 16, 2048, 128)
    assert st == 0 and need <= 16 << 20
    st, need = _lib.fa_bwd_workspace_size(64, 64, 2048, 128)
    assert st == 0 and need > 16 << 20
    assert f(*ptrs, 64, 64, 2048, 128, 0, 0.125, None, None) == -5
    assert f(None, *ptrs[1:], 1, 1, 64, 64, 0, 0.125, None, None) == -1
    assert f(*ptrs, 1, 1, 64, 96, 0, 0.125, None, None) == -3
    assert f(*ptrs, 1, 1, 64, 64, 0, -1.0, None, None) == -4
    assert f(FAKE + 8, *ptrs[1:], 1, 1, 64, 64, 0, 0.125, None, None) == -8


def test_atomic_probe_rejects_bad_arguments():
    f = _lib.fa_atomic_add_probe
    assert f(None, 8192, 1, 1, None) == -1
    assert f(FAKE + 4, 8192, 1, 1, None) == -8
    assert f(FAKE, 8191, 1, 1, None) == -2
    assert f(FAKE, 8192, 0, 1, None) == -2
    assert f(FAKE, 8192, 1, 0, None) == -2

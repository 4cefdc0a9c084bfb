"""Host-side checks of the C ABI (no GPU): the library loads, exports every symbol the
header declares, and rejects bad arguments before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

import tensor_transformer_block_domino_amd as D
from tensor_transformer_block_domino_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "domino.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from tensor_transformer_block_domino_amd import build

        build.build()
    return D.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_calls():
    fns = header_functions()
    for name in ("shard_reduce", "domino_block_fwd", "domino_block_bwd", "domino_attn_block_fwd"):
        assert name in fns
    assert sorted(L.EXPORTED) == fns


def test_library_exports_every_header_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], stdout=subprocess.PIPE, text=True, check=True)
    syms = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
    for name in header_functions():
        assert name in syms, name
        assert hasattr(lib, name)


def test_struct_layouts_match_header():
    # int64 ×4 + int32 ×6 and int64 ×5 + float + int32 ×4 (padded to 8).
    assert ctypes.sizeof(L.MlpDesc) == 56
    assert ctypes.sizeof(L.AttnDesc) == 64
    assert L.AttnDesc.scale.offset == 40


def test_status_strings(lib):
    for code, name in L.STATUS_NAMES.items():
        assert D.domino_status_string(code) == name


def mlp_desc(**kw):
    base = dict(batch=2, seq=8, hidden=64, ffn_shard=32, act=0, dtype=1, row_chunks=1, col_chunks=1,
                n_partials=1, no_join=0)
    base.update(kw)
    return L.MlpDesc(**base)


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=3, row_chunks=2), L.STATUS_NAMES[2]),
    (dict(row_chunks=0), L.STATUS_NAMES[2]),
    (dict(hidden=68), L.STATUS_NAMES[3]),
    (dict(hidden=64, col_chunks=16), L.STATUS_NAMES[3]),
    (dict(ffn_shard=20), L.STATUS_NAMES[3]),
    (dict(n_partials=0), L.STATUS_NAMES[1]),
    (dict(n_partials=17), L.STATUS_NAMES[1]),
    (dict(act=7), L.STATUS_NAMES[1]),
    (dict(dtype=9), L.STATUS_NAMES[1]),
    (dict(batch=-1), L.STATUS_NAMES[2]),
])
def test_block_fwd_rejects_bad_desc(lib, kw, status):
    with pytest.raises(D.DominoError) as ei:
        D.domino_block_fwd(mlp_desc(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert str(ei.value).startswith(status)


def test_block_fwd_rejects_null_and_misaligned(lib):
    with pytest.raises(D.DominoError, match="INVALID_ARG: X is NULL"):
        D.domino_block_fwd(mlp_desc(), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    with pytest.raises(D.DominoError, match="ALIGN: A_s"):
        D.domino_block_fwd(mlp_desc(), FAKE, FAKE + 2, FAKE, FAKE, FAKE, FAKE, None, None)
    with pytest.raises(D.DominoError, match="peer_Y"):
        D.domino_block_fwd(mlp_desc(n_partials=3), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    with pytest.raises(D.DominoError, match=r"peer_Y\[1\] is NULL"):
        D.domino_block_fwd(mlp_desc(n_partials=3), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, [FAKE, None], FAKE)


def test_empty_inputs_are_noops(lib):
    # Zero tokens or zero hidden: nothing to do, nothing enqueued, no pointers needed.
    D.domino_block_fwd(mlp_desc(batch=0), None, None, None, None, None, None, None, None)
    D.domino_block_fwd(mlp_desc(hidden=0), None, None, None, None, None, None, None, None)
    D.domino_block_bwd(mlp_desc(hidden=0), None, None, None, None, None, None, None, None, None, None, None, None)
    D.shard_reduce(FAKE, 8, [FAKE], 8, 0, 8, 1)
    D.shard_reduce(FAKE, 8, [FAKE], 8, 5, 0, 1)


def test_block_bwd_rejects(lib):
    with pytest.raises(D.DominoError, match="dY is NULL"):
        D.domino_block_bwd(mlp_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, FAKE)
    with pytest.raises(D.DominoError, match="dA_s"):
        D.domino_block_bwd(mlp_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE)
    with pytest.raises(D.DominoError, match="workspace"):
        D.domino_block_bwd(mlp_desc(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 0,
                           FAKE + 4, 64)


def test_shard_reduce_rejects(lib):
    with pytest.raises(D.DominoError, match="ALIGN"):
        D.shard_reduce(FAKE, 8, [FAKE], 8, 4, 12, 1)          # cols not a multiple of 8 (bf16)
    with pytest.raises(D.DominoError, match="SHAPE"):
        D.shard_reduce(FAKE, 8, [FAKE], 8, 4, 16, 1)          # ld < cols
    with pytest.raises(D.DominoError, match="INVALID_ARG"):
        D.shard_reduce(FAKE, 8, [FAKE] * 17, 8, 4, 8, 1)      # too many partials
    with pytest.raises(D.DominoError, match="different leading"):
        D.shard_reduce(FAKE, 16, [FAKE], 8, 4, 8, 1)          # aliased with different ld
    with pytest.raises(D.DominoError, match="partials\\[1\\] is NULL"):
        D.shard_reduce(FAKE, 8, [FAKE, None], 8, 4, 8, 1)
    with pytest.raises(D.DominoError, match="bad dtype"):
        D.shard_reduce(FAKE, 8, [FAKE], 8, 4, 8, 5)


def test_attn_rejects(lib):
    def ad(**kw):
        base = dict(batch=2, seq=16, hidden=64, heads=2, head_dim=128, scale=0.0, dtype=1, row_chunks=1,
                    n_partials=1, no_join=0)
        base.update(kw)
        return L.AttnDesc(**base)

    for kw, pat in [(dict(head_dim=64), "UNSUPPORTED"), (dict(dtype=0), "UNSUPPORTED"), (dict(batch=3, row_chunks=2),
                    "SHAPE"), (dict(scale=-1.0), "INVALID_ARG"), (dict(hidden=60), "ALIGN")]:
        with pytest.raises(D.DominoError, match=pat):
            D.domino_attn_block_fwd(ad(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)


def test_every_timing_kind_is_readable(lib):
    D.domino_timing_enable(False)
    for kind in D.KERNEL_KINDS:
        assert D.domino_timing_read(kind) == (0, 0.0)
    assert max(D.KERNEL_KINDS.values()) == len(D.KERNEL_KINDS) - 1


def test_timing_read_rejects_bad_kind(lib):
    with pytest.raises(D.DominoError):
        D.domino_timing_read(99)
    D.domino_timing_enable(False)
    assert D.domino_timing_read("reduce") == (0, 0.0)
    assert D.domino_timing_kernel("reduce") == ""
    with pytest.raises(D.DominoError):
        D.domino_timing_kernel(-1)


def test_workspace_size_is_zero_for_fp32_and_sized_for_bf16(lib):
    assert D.domino_block_bwd_workspace_size(mlp_desc(dtype=0)) == 0
    big = mlp_desc(batch=4, seq=2048, hidden=2560, ffn_shard=1280)
    n = D.domino_block_bwd_workspace_size(big)
    assert n % 4 == 0 and n >= 0


def group_desc(**kw):
    base = dict(rows=4, hidden=64, eps=1e-5, p_drop=0.1)
    base.update(kw)
    return L.GroupDesc(**base)


def test_group_desc_layout():
    assert ctypes.sizeof(L.GroupDesc) == 24 and L.GroupDesc.p_drop.offset == 20


@pytest.mark.parametrize("kw,msg", [
    (dict(hidden=60), "ALIGN: hidden must be a multiple of 8"),
    (dict(hidden=8200), "UNSUPPORTED: hidden above 8192"),
    (dict(p_drop=1.0), "INVALID_ARG: p_drop"),
    (dict(p_drop=-0.1), "INVALID_ARG: p_drop"),
    (dict(eps=0.0), "INVALID_ARG: eps"),
    (dict(rows=-1), "SHAPE"),
])
def test_group_rejects_bad_desc(lib, kw, msg):
    with pytest.raises(D.DominoError, match=msg):
        D.domino_resid_ln_fwd(group_desc(**kw), FAKE, FAKE, None, None, FAKE, None, None, None, None, None)


def test_group_rejects_bad_pointers(lib):
    with pytest.raises(D.DominoError, match="INVALID_ARG: resid is NULL"):
        D.domino_resid_ln_fwd(group_desc(), None, FAKE, None, None, FAKE, None, None, None, None, None)
    with pytest.raises(D.DominoError, match="INVALID_ARG: ln_out is NULL"):
        D.domino_resid_ln_fwd(group_desc(), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, FAKE, FAKE)
    with pytest.raises(D.DominoError, match="ALIGN: keep"):
        D.domino_resid_ln_fwd(group_desc(), FAKE, FAKE, None, FAKE + 2, FAKE, None, None, None, None, None)
    with pytest.raises(D.DominoError, match="d_gamma/d_beta need d_ln"):
        D.domino_resid_ln_bwd(group_desc(), None, FAKE, None, None, None, None, None, FAKE, None, FAKE, None, None,
                              0, FAKE, 1 << 20)
    with pytest.raises(D.DominoError, match="workspace smaller"):
        D.domino_resid_ln_bwd(group_desc(), None, FAKE, None, None, None, None, None, FAKE, None, None, None, None,
                              0, FAKE, 4)
    ws = D.domino_resid_ln_bwd_workspace_size(group_desc(rows=4096, hidden=4096))
    assert ws == 3 * 512 * 4096 * 4

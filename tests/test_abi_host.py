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


def test_library_exports_no_undeclared_c_function():
    """Every unmangled function the library defines is one the header declares (internal
    helpers stay in C++ linkage)."""
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], stdout=subprocess.PIPE, text=True, check=True)
    c_funcs = {parts[-1] for parts in (line.split() for line in out.stdout.splitlines())
               if len(parts) == 3 and parts[1] == "T" and not parts[2].startswith("_")}
    assert c_funcs <= set(header_functions()), sorted(c_funcs - set(header_functions()))


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
    (dict(batch=65, row_chunks=65), L.STATUS_NAMES[4]),                    # 65 chunks: above the 64 the scheduler holds
    (dict(batch=16, row_chunks=16, hidden=640, col_chunks=5), L.STATUS_NAMES[4]),
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


# Sizes just past the kernels' 32-bit index arithmetic (operand byte offsets of 256-row
# tiles, the reduction's uint32 grid stride) are rejected before anything is enqueued; the
# largest accepted sizes pass validation (the calls then fail only on the NULL pointer
# planted to stop them before any launch).
@pytest.mark.parametrize("kw,ok", [
    (dict(hidden=1 << 22, ffn_shard=8, batch=1, seq=8), True),
    (dict(hidden=(1 << 22) + 8, ffn_shard=8, batch=1, seq=8), False),
    (dict(hidden=64, ffn_shard=1 << 22, act=0, batch=1, seq=8), True),
    (dict(hidden=64, ffn_shard=1 << 21, act=1, batch=1, seq=8), True),
    (dict(hidden=64, ffn_shard=(1 << 21) + 8, act=1, batch=1, seq=8), False),
    (dict(hidden=8192, ffn_shard=8, batch=1, seq=(1 << 22) - 2048), True),  # T·h/8 = 2^32 − 2^21
    (dict(hidden=8192, ffn_shard=8, batch=1, seq=1 << 22), False),          # T·h/8 = 2^32
])
def test_block_size_limits(lib, kw, ok):
    if ok:
        with pytest.raises(D.DominoError, match="X is NULL"):
            D.domino_block_fwd(mlp_desc(**kw), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    else:
        with pytest.raises(D.DominoError, match="UNSUPPORTED"):
            D.domino_block_fwd(mlp_desc(**kw), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)


def test_shard_reduce_size_limit(lib):
    limit = (1 << 32) - (1 << 21)       # 16-byte groups the reduction's uint32 stride can walk
    with pytest.raises(D.DominoError, match="partials\\[0\\] is NULL"):   # at the limit: accepted
        D.shard_reduce(FAKE, 8, [None], 8, limit, 8, 1)
    with pytest.raises(D.DominoError, match="region too large"):
        D.shard_reduce(FAKE, 8, [None], 8, limit + 1, 8, 1)
    with pytest.raises(D.DominoError, match="region too large"):
        D.shard_reduce(FAKE, 16, [None], 16, limit // 2 + 1, 16, 1)
    with pytest.raises(D.DominoError, match="region too large"):     # fp32: 4 elements per group
        D.shard_reduce(FAKE, 8, [None], 8, limit // 2 + 1, 8, 0)


def test_attn_size_limits(lib):
    def ad(**kw):
        base = dict(batch=1, seq=16, hidden=64, heads=2, head_dim=128, scale=0.0, dtype=1, row_chunks=1,
                    n_partials=1, no_join=0)
        base.update(kw)
        return L.AttnDesc(**base)

    with pytest.raises(D.DominoError, match="X is NULL"):
        D.domino_attn_block_fwd(ad(heads=(1 << 22) // 384), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    with pytest.raises(D.DominoError, match="UNSUPPORTED"):
        D.domino_attn_block_fwd(ad(heads=(1 << 22) // 384 + 1), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    with pytest.raises(D.DominoError, match="UNSUPPORTED"):
        D.domino_attn_block_fwd(ad(hidden=(1 << 22) + 8), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)


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


def layer_desc(**kw):
    base = dict(batch=2, seq=64, hidden=256, heads=2, head_dim=128, ffn_shard=128, act=0, eps=1e-5, p_drop=0.1,
                scale=0.0, row_chunks=2, n_partials=1, layers=1, reserved=0)
    base.update(kw)
    return L.LayerDesc(**base)


def layer_ptrs(layers=1, n_partials=1, **over):
    """Every field of the per-layer parameter, activation and gradient structs set to a valid
    (never dereferenced) address; `over` replaces fields as "params.name" / "acts.name" /
    "grads.name" = value for layer 0, or "L<l>.<struct>.name" for layer l."""
    peers = [FAKE] * (n_partials - 1)
    out = []
    for l in range(layers):
        p = {n: FAKE for n, _ in L.LayerParams._fields_}
        a = {n: FAKE for n, _ in L.LayerActs._fields_}
        g = {n: FAKE for n, _ in L.LayerGrads._fields_}
        for s in (a, g):
            for n, t in L.LayerActs._fields_ + L.LayerGrads._fields_:
                if n in s and t is not L._VP:
                    s[n] = list(peers)
        out.append({"params": p, "acts": a, "grads": g})
    for key, v in over.items():
        parts = key.split(".")
        l = int(parts[0][1:]) if parts[0].startswith("L") else 0
        struct, name = parts[-2], parts[-1]
        out[l][struct][name] = v
    return ([o["params"] for o in out], [o["acts"] for o in out], [o["grads"] for o in out])


def test_layer_desc_layout():
    assert ctypes.sizeof(L.LayerDesc) == 80 and L.LayerDesc.reserved.offset == 76
    assert ctypes.sizeof(L.LayerParams) == 14 * 8 and ctypes.sizeof(L.LayerActs) == 19 * 8
    assert ctypes.sizeof(L.LayerGrads) == 25 * 8


@pytest.mark.parametrize("kw,msg", [
    (dict(head_dim=64), "UNSUPPORTED: head_dim must be 128"),
    (dict(batch=3), "SHAPE: batch % row_chunks"),
    (dict(row_chunks=0), "SHAPE: bad row_chunks"),
    (dict(n_partials=0), "INVALID_ARG: bad n_partials"),
    (dict(n_partials=17), "INVALID_ARG: bad n_partials"),
    (dict(layers=0), "INVALID_ARG: layers must be >= 1"),
    (dict(hidden=260), "ALIGN: hidden and ffn_shard"),
    (dict(ffn_shard=100), "ALIGN: hidden and ffn_shard"),
    (dict(hidden=8200), "UNSUPPORTED: hidden above 8192"),
    (dict(act=7), "INVALID_ARG: bad act"),
    (dict(p_drop=1.0), "INVALID_ARG: p_drop"),
    (dict(eps=0.0), "INVALID_ARG: eps"),
    (dict(reserved=1), "INVALID_ARG: reserved must be 0"),
    (dict(seq=-1), "SHAPE: negative size"),
    (dict(heads=0), "UNSUPPORTED: a layer needs heads > 0"),
    (dict(ffn_shard=0), "UNSUPPORTED: a layer needs heads > 0"),
])
def test_stack_rejects_bad_desc(lib, kw, msg):
    prm, act, grd = layer_ptrs()
    with pytest.raises(D.DominoError, match=msg):
        D.domino_stack_fwd(layer_desc(**kw), FAKE, prm, act, FAKE)
    with pytest.raises(D.DominoError, match=msg):
        D.domino_stack_bwd(layer_desc(**kw), FAKE, prm, act, grd, FAKE, FAKE, 0, FAKE, 1 << 40)
    if not msg.startswith("UNSUPPORTED: a layer"):
        assert D.domino_stack_bwd_workspace_size(layer_desc(**kw)) == 0


@pytest.mark.parametrize("over,msg", [
    ({"params.A_qkv_s": None}, "INVALID_ARG: layer 0: A_qkv_s is NULL"),
    ({"params.B_s": FAKE + 2}, "ALIGN: layer 0: B_s is not 16-byte aligned"),
    ({"params.ln1_beta": FAKE + 8}, "ALIGN: layer 0: ln1_beta"),
    ({"params.keep_attn": FAKE + 2}, "ALIGN: keep is not 4-byte aligned"),
    ({"acts.ln2": None}, "INVALID_ARG: layer 0: ln2 is NULL"),
    ({"acts.y_mlp": None}, "INVALID_ARG: layer 0: y_mlp is NULL"),
    ({"L1.acts.x_in": None}, "INVALID_ARG: layer 1: x_in is NULL"),
    ({"L1.params.A_s": None}, "INVALID_ARG: layer 1: A_s is NULL"),
    ({"acts.peer_y_attn": [FAKE, None]}, r"INVALID_ARG: layer 0: peer_y_attn\[1\] is NULL"),
    ({"L1.acts.peer_y_mlp": [FAKE + 4, FAKE]}, r"ALIGN: layer 1: peer_y_mlp\[0\]"),
])
def test_stack_fwd_rejects_bad_pointers(lib, over, msg):
    prm, act, _ = layer_ptrs(layers=2, n_partials=3, **over)
    with pytest.raises(D.DominoError, match=msg):
        D.domino_stack_fwd(layer_desc(layers=2, n_partials=3), FAKE, prm, act, FAKE)


def test_stack_fwd_rejects_missing_input_and_output(lib):
    prm, act, _ = layer_ptrs()
    with pytest.raises(D.DominoError, match="INVALID_ARG: X is NULL"):
        D.domino_stack_fwd(layer_desc(), None, prm, act, FAKE)
    with pytest.raises(D.DominoError, match="INVALID_ARG: out is NULL"):
        D.domino_stack_fwd(layer_desc(), FAKE, prm, act, None)
    with pytest.raises(D.DominoError, match="ALIGN: workspace"):
        D.domino_stack_fwd(layer_desc(), FAKE, prm, act, FAKE, FAKE + 4, 1 << 20)
    # Zero tokens: nothing to do and no pointer is read.
    D.domino_stack_fwd(layer_desc(batch=0), None, [{}], [{}], None)


@pytest.mark.parametrize("over,msg", [
    ({"grads.dA_s": None}, "INVALID_ARG: layer 0: dA_s is NULL"),
    ({"grads.d_b_o": FAKE + 2}, "ALIGN: layer 0: d_b_o"),
    ({"acts.lse": None}, "INVALID_ARG: layer 0: lse is NULL"),
    ({"L1.grads.d_x_in": None}, "INVALID_ARG: layer 1: d_x_in is NULL"),
    ({"grads.peer_dx_attn": [None, FAKE]}, r"INVALID_ARG: layer 0: peer_dx_attn\[0\] is NULL"),
    ({"L1.grads.peer_dx_mlp": [FAKE, FAKE + 2]}, r"ALIGN: layer 1: peer_dx_mlp\[1\]"),
])
def test_stack_bwd_rejects_bad_pointers(lib, over, msg):
    d = layer_desc(layers=2, n_partials=3)
    prm, act, grd = layer_ptrs(layers=2, n_partials=3, **over)
    with pytest.raises(D.DominoError, match=msg):
        D.domino_stack_bwd(d, FAKE, prm, act, grd, FAKE, FAKE, 0, FAKE, 1 << 40)


def test_stack_bwd_workspace_checks(lib):
    d = layer_desc(layers=2, n_partials=3)
    prm, act, grd = layer_ptrs(layers=2, n_partials=3)
    ws = D.domino_stack_bwd_workspace_size(d)
    assert ws > 0 and ws % 16 == 0
    with pytest.raises(D.DominoError, match="workspace smaller than domino_stack_bwd_workspace_size"):
        D.domino_stack_bwd(d, FAKE, prm, act, grd, FAKE, FAKE, 0, FAKE, ws - 16)
    with pytest.raises(D.DominoError, match="workspace smaller"):
        D.domino_stack_bwd(d, FAKE, prm, act, grd, FAKE, FAKE, 0, None, ws)
    with pytest.raises(D.DominoError, match="ALIGN: workspace"):
        D.domino_stack_bwd(d, FAKE, prm, act, grd, FAKE, FAKE, 0, FAKE + 8, ws)
    with pytest.raises(D.DominoError, match="INVALID_ARG: dX is NULL"):
        D.domino_stack_bwd(d, FAKE, prm, act, grd, FAKE, None, 0, FAKE, ws)


def test_attn_bwd_rejects(lib):
    def ad(**kw):
        base = dict(batch=2, seq=16, hidden=64, heads=2, head_dim=128, scale=0.0, dtype=1, row_chunks=1,
                    n_partials=1, no_join=0)
        base.update(kw)
        return L.AttnDesc(**base)

    args = [FAKE] * 10 + [None] + [FAKE] * 3  # X .. dX_own, peer_dX, dX, dA_qkv_s, dB_o_s

    def call(desc, *, ws=FAKE, ws_bytes=1 << 30, **over):
        a = list(args)
        names = ["X", "A_qkv_s", "B_o_s", "QKV", "O", "lse", "dY", "dO", "dQKV", "dX_own", "peer_dX", "dX",
                 "dA_qkv_s", "dB_o_s"]
        d_b = over.pop("d_b_qkv_s", None)
        for k, v in over.items():
            a[names.index(k)] = v
        D.domino_attn_block_bwd(desc, *a, accumulate=0, workspace=ws, workspace_bytes=ws_bytes, d_b_qkv_s=d_b)

    for kw, pat in [(dict(head_dim=64), "UNSUPPORTED"), (dict(dtype=0), "UNSUPPORTED"),
                    (dict(batch=3, row_chunks=2), "SHAPE"), (dict(hidden=60), "ALIGN")]:
        with pytest.raises(D.DominoError, match=pat):
            call(ad(**kw))
    with pytest.raises(D.DominoError, match="INVALID_ARG: lse is NULL"):
        call(ad(), lse=None)
    with pytest.raises(D.DominoError, match="ALIGN: dO"):
        call(ad(), dO=FAKE + 2)
    with pytest.raises(D.DominoError, match=r"INVALID_ARG: peer_dX\[1\] is NULL"):
        call(ad(n_partials=3), peer_dX=[FAKE, None])
    with pytest.raises(D.DominoError, match="ALIGN: d_b_qkv_s"):
        call(ad(), d_b_qkv_s=FAKE + 4)
    ws = D.domino_attn_block_bwd_workspace_size(ad())
    assert ws > 0
    with pytest.raises(D.DominoError, match="workspace smaller than domino_attn_block_bwd_workspace_size"):
        call(ad(), ws_bytes=ws - 4)
    with pytest.raises(D.DominoError, match="ALIGN: workspace"):
        call(ad(), ws=FAKE + 4, ws_bytes=ws)

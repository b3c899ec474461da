"""The C ABI without a GPU: the library loads, exports every entry point that
include/tpshard.h declares, computes the host-only shard arithmetic, and
rejects invalid arguments before any launch (null pointers never reach a
kernel on these paths)."""
import ctypes
import os
import re

import pytest

import oracle as O
import tensor_sharded_matmul_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

pytestmark = pytest.mark.skipif(not os.path.exists(T.lib_path()),
                                reason="libtpshard.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = T.load()
    names = _declared()
    assert {"tp_col_linear", "tp_row_linear_partial", "tp_mlp_shard_fwd", "tp_mlp_shard_bwd",
            "tp_qkv_regroup", "tp_shard_shape"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version():
    assert T.tp_version() >= 1


def _mask(spec, axes):
    return [sum(1 << axes.index(a) for a in dims) for dims in spec]


def test_shard_shape_quiz_matches_oracle_and_page():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "shard_quiz.json")))
    axes = [a for a, _ in g["mesh"]]
    sizes = [s for _, s in g["mesh"]]
    got = T.tp_shard_shape(g["shape"], g["elem_bytes"], sizes, _mask(g["spec"], axes))
    assert list(got[0]) == g["local_shape"]
    assert got[1] == g["local_bytes"] and got[2] == g["total_bytes"]
    want = O.shard_shape(g["shape"], g["elem_bytes"], dict(g["mesh"]),
                         [tuple(s) for s in g["spec"]])
    assert got == want
    with pytest.raises(ValueError, match="two dims"):
        T.tp_shard_shape(g["shape"], 1, sizes, _mask(g["illegal_same_axis_spec"], axes))


@pytest.mark.parametrize("shape,spec", [((8, 6), [("X",), ("Y",)]), ((8, 6), [("Y", "X"), ()]),
                                        ((16, 4, 2), [(), ("X",), ("Y",)]), ((4,), [()]),
                                        ((6, 6), [("X",), ()])])
def test_shard_shape_agrees_with_oracle(shape, spec):
    mesh = {"X": 4, "Y": 2}
    axes = list(mesh)
    try:
        want = O.shard_shape(shape, 2, mesh, spec)
    except O.ShardError:
        with pytest.raises(ValueError):
            T.tp_shard_shape(shape, 2, list(mesh.values()), _mask(spec, axes))
        return
    assert T.tp_shard_shape(shape, 2, list(mesh.values()), _mask(spec, axes)) == want


def _raw(name):
    return getattr(T.load(), name)


NULL = ctypes.c_void_p(0)


def test_regroup_divisibility_errors_before_launch():
    f = _raw("tp_qkv_regroup")
    assert f(NULL, NULL, 8192, 64, 8, 128, 7, 0, NULL) == 2          # NOT_DIVISIBLE
    assert "must be a multiple of tensor_model_parallel_size" in T.tp_last_error()
    assert f(NULL, NULL, 8192, 48, 8, 128, 12, 0, NULL) == 2         # n_kv < t, n_kv does not divide t
    assert "replicate KV heads" in T.tp_last_error()
    assert f(NULL, NULL, 8192, 64, 8, 128, 16, 0, NULL) == 1         # replicated KV heads: valid, NULL W_qkv
    assert f(NULL, NULL, 8192, 64, 8, 128, 8, 8, NULL) == 1          # rank out of range
    assert f(NULL, NULL, 8192, 64, 8, 12, 8, 0, NULL) == 1           # d_h % 8
    assert f(NULL, NULL, 8192, 64, 8, 128, 8, 0, NULL) == 1          # NULL pointers
    assert "NULL" in T.tp_last_error()
    assert f(NULL, NULL, 0, 64, 8, 128, 8, 0, NULL) == 0             # h = 0: nothing to do


def test_kv_grad_accumulate_validates_before_launch():
    f = _raw("tp_kv_grad_accumulate")
    assert f(NULL, NULL, 8192, 64, 8, 128, 8, NULL) == 1             # t <= n_kv: no replicas
    assert "replicated only" in T.tp_last_error()
    assert f(NULL, NULL, 8192, 48, 8, 128, 12, NULL) == 2            # 8 does not divide 12
    assert f(NULL, NULL, 8192, 64, 8, 126, 16, NULL) == 1            # d_h % 4
    assert f(NULL, NULL, 8192, 64, 8, 128, 16, NULL) == 1            # NULL pointers
    assert f(NULL, NULL, 0, 64, 8, 128, 16, NULL) == 0               # h = 0: nothing to do


def test_vocab_calls_validate_before_launch():
    fwd = _raw("tp_vocab_embed_fwd")
    assert fwd(NULL, NULL, 0, 16, 1000, 8192, NULL, 0, NULL) == 1           # NULL ids
    assert fwd(NULL, NULL, 0, 16, 1000, 100, NULL, 0, NULL) == 3            # h % 64
    bwd = _raw("tp_vocab_embed_bwd")
    odd = ctypes.c_void_p(0x1010)
    assert bwd(odd, NULL, 0, 16, 1000, 32768, NULL, NULL, 0, NULL) == 3     # h above the register tile
    ce = _raw("tp_vocab_ce_fwd")
    assert ce(NULL, NULL, NULL, 0, 16, 8192, 16128, NULL, NULL, NULL, NULL, 0, NULL) == 1   # NULL targets
    assert ce(NULL, NULL, odd, -1, 16, 8192, 16128, NULL, NULL, NULL, NULL, 0, NULL) == 1   # vocab_start < 0
    comb = _raw("tp_vocab_ce_combine")
    assert comb(NULL, NULL, NULL, 0, 16, NULL, NULL, NULL, NULL) == 1               # t = 0
    ch = _raw("tp_row_linear_partial_chunked")
    assert ch(NULL, NULL, NULL, 16, 1024, 8192, 0, 0, NULL, NULL, 0, NULL) == 1     # nchunks = 0
    cb = _raw("tp_col_linear_bwd_chunked")
    assert cb(NULL, NULL, NULL, NULL, NULL, 16, 1024, 8192, 0, 65, NULL, NULL, 0, NULL) == 1  # nchunks = 65
    p = ctypes.c_void_p(0x10000)
    assert cb(p, p, p, NULL, p, 16, 1024, 8192, 0, 2, NULL, NULL, 0, NULL) == 1      # NULL dX_part
    assert "dX_part" in T.tp_last_error()
    assert cb(NULL, p, p, p, p, 16, 1024, 8192, 0, 2, NULL, NULL, 0, NULL) == 1      # dW without X


def test_regroup_width_matches_oracle():
    for n_h, n_kv, d_h, t in [(64, 8, 128, 8), (64, 8, 128, 16), (32, 8, 128, 32), (64, 8, 128, 4)]:
        assert T.regroup_width(n_h, n_kv, d_h, t) == len(O.qkv_regroup_index(n_h, n_kv, d_h, t, 0))


def test_gemm_entry_points_validate_before_launch():
    col = _raw("tp_col_linear")
    assert col(NULL, NULL, NULL, 16, 8192, 1280, 0, NULL, NULL, 0, NULL) == 1          # NULL X
    assert col(NULL, NULL, NULL, 16, 100, 1280, 0, NULL, NULL, 0, NULL) == 3           # k % 64
    assert col(NULL, NULL, NULL, 16, (1 << 20) + 64, 1280, 0, NULL, NULL, 0, NULL) == 3  # k above 2^20
    assert "too large" in T.tp_last_error()
    assert col(NULL, NULL, NULL, (1 << 30) + 1, 8192, 1280, 0, NULL, NULL, 0, NULL) == 3  # N above 2^30
    assert col(NULL, NULL, NULL, -1, 8192, 1280, 0, NULL, NULL, 0, NULL) == 1          # N < 0
    assert col(NULL, NULL, NULL, 16, 8192, 1280, 7, NULL, NULL, 0, NULL) == 1          # act
    odd = ctypes.c_void_p(0x1008)
    assert col(odd, odd, odd, 16, 8192, 1280, 0, NULL, NULL, 0, NULL) == 1             # misaligned
    assert "aligned" in T.tp_last_error()
    row = _raw("tp_row_linear_partial")
    assert row(NULL, NULL, NULL, 16, 1024, 8192, 0, NULL, 0, NULL) == 1
    fwd = _raw("tp_mlp_shard_fwd")
    assert fwd(NULL, NULL, NULL, 16, 8192, 3584, 0, NULL, NULL, NULL, 0, NULL, 0, NULL) == 1   # act NONE
    bwd = _raw("tp_mlp_shard_bwd")
    assert bwd(NULL, NULL, NULL, NULL, NULL, NULL, 16, 8192, 3584, 2, NULL, NULL, NULL, NULL, 0,
               NULL, 0, NULL) == 1
    assert T.tp_last_error() != ""


# Every call that may need scratch memory, with sizes that need some at the
# Llama-3-70B t = 8 shapes (decode-sized token counts; the narrow attention
# shards; the cross-entropy records; the embedding bookkeeping) and the arguments
# of its workspace query.
WS_CASES = {
    "tp_col_linear": (16, 8192, 1280, 0),
    "tp_row_linear_partial": (16, 8192, 8192),
    "tp_row_linear_partial_chunked": (48, 8192, 8192, 3),
    "tp_col_linear_bwd_chunked": (4096, 8192, 7168, 8),   # dX of the MLP shard in 512-row chunks
    "tp_mlp_shard_fwd": (16, 8192, 3584, 2),
    "tp_row_linear_bwd": (4096, 512, 8192),      # W_O of Llama-3-70B at t = 16
    "tp_vocab_ce_fwd": (4096, 8192, 16128),
    "tp_vocab_embed_bwd": (4096, 16128, 8192),
}


@pytest.mark.parametrize("entry", sorted(WS_CASES))
def test_workspace_queries(entry):
    n = T.workspace_size(entry, *WS_CASES[entry])
    assert n > 0 and n % 16 == 0
    # invalid sizes fail in the query as in the call (a width that is not a
    # multiple of 64)
    args = list(WS_CASES[entry])
    args[2 if entry == "tp_vocab_embed_bwd" else 1] = 100
    bad = tuple(args)
    with pytest.raises((ValueError, NotImplementedError)):
        T.workspace_size(entry, *bad)
    # NULL output pointer
    assert getattr(T.load(), entry + "_workspace_size")(*WS_CASES[entry], None) == 1


def test_workspace_query_values():
    # the split-K decode product: ksplit partials of [N, n] f32; the
    # cross-entropy records: one per 64 vocab columns per token (256 x 256
    # ping-pong tiles), or one per 112 when the weight's window needs 64-bit
    # offsets (256 x 224 tiles), 12 bytes each; the embedding bookkeeping: a
    # count, a flag per table row and a list of at most min(N, v_loc) rows
    n = T.workspace_size("tp_col_linear", 16, 8192, 1280, 0)
    assert n % (16 * 1280 * 4) == 0 and 2 <= n // (16 * 1280 * 4) <= 64
    # decode plans (256 CUs): 32-column slabs when no K split is needed (at
    # most 48 k-blocks of 32 rows per workgroup at 16 tokens, 32 at 32), else
    # 64-column slabs (24 blocks at 16 or 32 tokens). The QKV product at 16
    # tokens: 20 slabs in 12 K splits (240 workgroups); W_O: 256 slabs, no
    # split; the 32-row QKV product over K = 2048: 20 slabs x 8 splits
    assert n == 12 * 16 * 1280 * 4
    assert T.workspace_size("tp_row_linear_partial", 16, 1024, 8192) == 0
    assert T.workspace_size("tp_row_linear_partial", 32, 1024, 8192) == 0
    assert T.workspace_size("tp_col_linear", 16, 256, 4096, 2) == 0   # SwiGLU, 8192 weight columns: no split
    assert T.workspace_size("tp_col_linear", 32, 2048, 1280, 0) == 8 * 32 * 1280 * 4
    assert T.workspace_size("tp_col_linear", 32, 8192, 1280, 0) > 0
    assert T.workspace_size("tp_vocab_ce_fwd", 4096, 8192, 16128) == 4096 * 4 * (16128 // 256) * 12
    # (8192 + 512) * 131072 * 2 >= 2^31: a 131072-wide vocabulary shard
    assert T.workspace_size("tp_vocab_ce_fwd", 64, 8192, 131072) == 64 * 2 * -(-131072 // 224) * 12
    assert T.workspace_size("tp_vocab_ce_fwd", 64, 8192, 123200) == 64 * 4 * -(-123200 // 256) * 12
    r16 = lambda b: (b + 15) // 16 * 16  # noqa: E731
    assert T.workspace_size("tp_vocab_embed_bwd", 4096, 16128, 8192) == r16((1 + 16128 + 4096) * 4)
    assert T.workspace_size("tp_vocab_embed_bwd", 100000, 16128, 8192) == r16((1 + 2 * 16128) * 4)
    # a weight gradient on TN mid tiles (2112 x 1984 over 3000 tokens: 136
    # tiles of 128 x 256, 72 of 256 x 256) is not split, and dZ of the same
    # call contracts over K = 1984 < 2048 without a split: no workspace
    assert T.workspace_size("tp_row_linear_bwd", 3000, 2112, 1984) == 0
    # dO of the attention shard at 4096 tokens splits (64 large tiles)
    assert T.workspace_size("tp_row_linear_bwd", 4096, 1024, 8192) > 0
    # the GEMM2 shard in 4 and 8 token-row chunks (1024 and 512 rows): NN mid
    # tiles of 128 x 256 and 128 x 128 fill the 256 CUs, no split; 16 chunks
    # (256 rows) fill neither and split
    assert T.workspace_size("tp_row_linear_partial", 1024, 3584, 8192) == 0
    assert T.workspace_size("tp_row_linear_partial", 512, 3584, 8192) == 0
    assert T.workspace_size("tp_row_linear_partial", 256, 3584, 8192) > 0
    # dX of the MLP shard (dH [4096, 7168] W_gate|up^T) in row chunks: 2
    # chunks of 2048 rows fill the CUs with 256 x 256 tiles, 4 chunks (1024
    # rows) with NT mid tiles of 128 x 256, no split; 8 chunks (512 rows)
    # split, needing what one 512-row product needs (dW over 4096 tokens
    # needs none)
    for nc in (2, 4):
        assert T.workspace_size("tp_col_linear_bwd_chunked", 4096, 8192, 7168, nc) == 0
    n8 = T.workspace_size("tp_col_linear_bwd_chunked", 4096, 8192, 7168, 8)
    assert n8 == T.workspace_size("tp_col_linear_bwd", 512, 8192, 7168) > 0
    # the QKV forward keeps its split (160 mid tiles would leave 96 CUs idle)
    assert T.workspace_size("tp_col_linear", 4096, 8192, 1280, 0) == 3 * 4096 * 1280 * 4
    # products with enough output tiles need none
    assert T.workspace_size("tp_mlp_shard_fwd", 4096, 8192, 3584, 2) == 0
    assert T.workspace_size("tp_mlp_shard_bwd", 4096, 8192, 3584, 2) == 0
    assert T.workspace_size("tp_row_linear_partial", 0, 1024, 8192) == 0


def test_too_small_workspace_is_rejected_before_launch():
    # fake (never dereferenced) aligned device pointers: the call must stop at
    # the workspace check, before anything is enqueued
    p = ctypes.c_void_p(0x10000)
    need = T.workspace_size("tp_col_linear", 16, 8192, 1280, 0)
    col = _raw("tp_col_linear")
    assert col(p, p, p, 16, 8192, 1280, 0, NULL, p, need - 16, NULL) == 1
    assert f"needs {need} bytes" in T.tp_last_error()
    assert col(p, p, p, 16, 8192, 1280, 0, NULL, NULL, need, NULL) == 1      # NULL workspace
    assert "NULL" in T.tp_last_error()
    assert col(p, p, p, 16, 8192, 1280, 0, NULL, ctypes.c_void_p(0x10008), need, NULL) == 1
    assert "aligned" in T.tp_last_error()
    emb = _raw("tp_vocab_embed_bwd")
    need_e = T.workspace_size("tp_vocab_embed_bwd", 4096, 16128, 8192)
    assert emb(p, p, 0, 4096, 16128, 8192, p, p, need_e - 1, NULL) == 1


def test_noalloc_entry_point_validates_before_launch():
    f = _raw("tp_col_linear_noalloc")
    p = ctypes.c_void_p(0x10000)
    assert f(NULL, NULL, NULL, 16, 8192, 1280, 0, NULL, NULL) == 1          # NULL X
    assert f(p, p, p, 16, 100, 1280, 0, NULL, NULL) == 3                    # k % 64
    # the QKV product at 4096 tokens splits into more than the 16 MiB scratch
    assert T.workspace_size("tp_col_linear", 4096, 8192, 1280, 0) > 16 << 20
    assert f(p, p, p, 4096, 8192, 1280, 0, NULL, NULL) == 3
    assert "scratch" in T.tp_last_error()

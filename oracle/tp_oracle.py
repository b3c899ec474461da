"""fp64 definitions of the tensor-parallel shard computations (test infrastructure).

Notation follows [TPSP] "预备：记号": N = b*s tokens, h hidden size, F MLP width,
t TP degree, f = F/t the per-shard MLP width, n_h / n_kv query / KV heads,
d_h head width. A linear layer is Y = X W with X[N,k], W[k,n], row-major.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

__all__ = [
    "matmul_loops", "col_linear", "row_linear_partial", "gelu", "gelu_grad",
    "sigmoid", "silu", "silu_grad", "swiglu", "col_linear_act", "mlp_shard_fwd",
    "mlp_shard_bwd", "mlp_shard_bwd_saved", "mlp_shard_fwd_rows", "mlp_shard_bwd_rows",
    "mlp_shard_bwd_cols", "col_linear_bwd", "row_linear_bwd",
    "qkv_regroup_index", "qkv_regroup", "naive_split_index", "shard_shape",
    "kv_heads_of_rank", "kv_replica_ranks", "kv_grad_accumulate", "kv_replica_grad_sum",
    "vocab_ce_local", "vocab_ce_loss", "vocab_ce_bwd", "vocab_embed_fwd", "vocab_embed_bwd",
    "ShardError", "llama_layer_params", "llama_model_params",
    "llama_shard_weight_shapes", "gemm_flops", "mlp_shard_flops",
    "check_heads_divisible", "rel_err",
]


# ---------------------------------------------------------------------------
# The two block-matmul identities ([TPSP] "矩阵乘法的两种切法"; [REVISIT]
# "Tensor Parallel", Column-wise / Row-wise TP)
# ---------------------------------------------------------------------------

def matmul_loops(A, B):
    """Brute-force C[i][j] = sum_k A[i][k] B[k][j] with Python loops (tiny inputs only)."""
    A = [[float(v) for v in row] for row in np.asarray(A)]
    B = [[float(v) for v in row] for row in np.asarray(B)]
    n, k = len(A), len(A[0]) if A else 0
    m = len(B[0]) if B else 0
    C = [[0.0] * m for _ in range(n)]
    for i in range(n):
        for j in range(m):
            s = 0.0
            for p in range(k):
                s += A[i][p] * B[p][j]
            C[i][j] = s
    return np.array(C, dtype=np.float64).reshape(n, m)


def col_linear(X, W_i):
    """Column-parallel linear: Y_i = X W_i, the rank's n/t output columns.

    [TPSP] "矩阵乘法的两种切法": W split by columns, each rank holds the full X
    and W_i[k, n/t]; its output is the column block Y_i[N, n/t]; no exchange.
    """
    return np.asarray(X, np.float64) @ np.asarray(W_i, np.float64)


def row_linear_partial(X_i, W_i):
    """Row-parallel linear: P_i = X_i W_i, a full-shape [N, n] partial sum {U}.

    [TPSP] "矩阵乘法的两种切法": W split by rows into [k/t, n] blocks and X by
    its last dim into [N, k/t]; each rank's X_i W_i is only a partial sum; the
    true Y is the sum over ranks (the g exchange, not part of one shard).
    """
    return np.asarray(X_i, np.float64) @ np.asarray(W_i, np.float64)


# ---------------------------------------------------------------------------
# Elementwise non-linearities ([TPSP] "MLP：先列后行，只通信一次")
# ---------------------------------------------------------------------------

def gelu(x):
    """Exact GeLU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).

    The pages name GeLU without a formula; the erf form (not the tanh
    approximation) is the reading taken.
    """
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    """d/dx GeLU(x) = Phi(x) + x phi(x), phi the standard normal density."""
    x = np.asarray(x, np.float64)
    cdf = 0.5 * (1.0 + erf(x / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return cdf + x * pdf


def sigmoid(x):
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(x):
    """SiLU(x) = x * sigmoid(x)."""
    x = np.asarray(x, np.float64)
    return x * sigmoid(x)


def silu_grad(x):
    """d/dx SiLU(x) = s + x s (1 - s), s = sigmoid(x)."""
    x = np.asarray(x, np.float64)
    s = sigmoid(x)
    return s + x * s * (1.0 - s)


def swiglu(G, U):
    """SwiGLU gate: SiLU(G) * U, elementwise ([TPSP] MLP section, SwiGLU form)."""
    return silu(G) * np.asarray(U, np.float64)


def col_linear_act(X, W, act):
    """Column-parallel linear with its local elementwise activation.

    act="none":   Z = X W                       (H = Z)
    act="gelu":   H = X A_i,  Z = GeLU(H)
    act="swiglu": W = [W_gate,i | W_up,i] with the *same* F-index segment in
                  both halves ([TPSP] MLP section: gate and up split by columns
                  over the same segment, concatenated as one [h, 2F/t] matrix);
                  H = X W = [G | U], Z = SiLU(G) * U.
    Returns (Z, H), H the pre-activation kept for the backward.
    """
    H = col_linear(X, W)
    if act == "none":
        return H, H
    if act == "gelu":
        return gelu(H), H
    if act == "swiglu":
        f = H.shape[1] // 2
        return swiglu(H[:, :f], H[:, f:]), H
    raise ValueError(f"unknown activation {act!r}")


def mlp_shard_fwd(X, W_in, W_out, act):
    """One rank's MLP share: Z_i = act(X W_in,i), P_i = Z_i W_out,i  ({U}).

    [TPSP] "MLP：先列后行，只通信一次": first matrix column-split, elementwise
    activation local, second matrix row-split; the rank's product is a partial
    sum whose all-reduce (g) completes Y. Returns (Z, H, P).
    """
    Z, H = col_linear_act(X, W_in, act)
    P = row_linear_partial(Z, W_out)
    return Z, H, P


# ---------------------------------------------------------------------------
# Backward ([TPSP] "矩阵乘法的两种切法", backward paragraph; [REVISIT] gradients)
# ---------------------------------------------------------------------------

def col_linear_bwd(X, W_i, dY_i):
    """Column-parallel backward: dX partial = dY_i W_i^T ({U}), dW_i = X^T dY_i (local)."""
    X = np.asarray(X, np.float64)
    W_i = np.asarray(W_i, np.float64)
    dY_i = np.asarray(dY_i, np.float64)
    return dY_i @ W_i.T, X.T @ dY_i


def row_linear_bwd(X_i, W_i, dY):
    """Row-parallel backward: dX_i = dY W_i^T and dW_i = X_i^T dY, both local."""
    X_i = np.asarray(X_i, np.float64)
    W_i = np.asarray(W_i, np.float64)
    dY = np.asarray(dY, np.float64)
    return dY @ W_i.T, X_i.T @ dY


def _act_bwd(H, dZ, act):
    """Pre-activation gradient dH from dZ by the chain rule on the activation."""
    if act == "none":
        return dZ
    if act == "gelu":
        return dZ * gelu_grad(H)
    if act == "swiglu":
        f = H.shape[1] // 2
        G, U = H[:, :f], H[:, f:]
        dG = dZ * U * silu_grad(G)
        dU = dZ * silu(G)
        return np.concatenate([dG, dU], axis=1)
    raise ValueError(act)


def mlp_shard_bwd_saved(X, W_in, W_out, H, Z, dY, act):
    """Backward of one rank's MLP share from the forward's saved tensors.

    H = X W_in (the pre-activation) and Z = act(H) are the ones the forward
    keeps ([TPSP] "显存账": gate, up and the activation output are stored for
    the backward). Row-parallel backward of the second matrix (local):
    dZ = dY W_out^T, dW_out = Z^T dY; activation backward to dH;
    column-parallel backward of the first matrix: dX partial = dH W_in^T
    ({U}, completed by f's all-reduce), dW_in = X^T dH (local).
    Returns dict(dZ, dH, dX_part, dW_in, dW_out).
    """
    dZ, dW_out = row_linear_bwd(Z, W_out, dY)
    dH = _act_bwd(np.asarray(H, np.float64), dZ, act)
    dX_part, dW_in = col_linear_bwd(X, W_in, dH)
    return {"dZ": dZ, "dH": dH, "dX_part": dX_part, "dW_in": dW_in, "dW_out": dW_out}


def mlp_shard_bwd(X, W_in, W_out, dY, act):
    """Backward of one rank's MLP share, from the upstream gradient dY[N,h]:
    the forward tensors computed here in fp64 from X and the weights, then
    mlp_shard_bwd_saved. Returns dict(dZ, dH, dX_part, dW_in, dW_out, Z, H)."""
    Z, H = col_linear_act(X, W_in, act)
    g = mlp_shard_bwd_saved(X, W_in, W_out, H, Z, dY, act)
    g["Z"], g["H"] = Z, H
    return g


def mlp_shard_fwd_rows(X, W_in, W_out, act, rows):
    """Forward outputs Z, H, P restricted to token rows (each row depends only on its X row)."""
    return mlp_shard_fwd(np.asarray(X)[rows], W_in, W_out, act)


def mlp_shard_bwd_rows(X, W_in, W_out, dY, act, rows):
    """dH and dX_part restricted to token rows (row-local quantities)."""
    X = np.asarray(X)[rows]
    dY = np.asarray(dY)[rows]
    Z, H, _ = mlp_shard_fwd(X, W_in, W_out, act)
    dZ = np.asarray(dY, np.float64) @ np.asarray(W_out, np.float64).T
    dH = _act_bwd(H, dZ, act)
    return {"dH": dH, "dX_part": dH @ np.asarray(W_in, np.float64).T}


def mlp_shard_bwd_cols(X, W_in, W_out, dY, act, cols):
    """Weight gradients restricted to MLP-width columns ``cols`` (indices into [0, f)).

    dW_in[:, c] = X^T dH[:, c] for the c's of ``cols`` (and, for SwiGLU, the
    matching up columns f + c); dW_out[c, :] = Z[:, c]^T dY. Each needs the
    forward and dZ only at those columns. Returns dict(dW_in_cols, dW_out_rows)
    where dW_in_cols has the columns ``cols`` (SwiGLU: ``cols`` then ``f+cols``).
    """
    X = np.asarray(X, np.float64)
    W_in = np.asarray(W_in, np.float64)
    W_out = np.asarray(W_out, np.float64)
    dY = np.asarray(dY, np.float64)
    cols = np.asarray(cols)
    if act == "swiglu":
        f = W_in.shape[1] // 2
        sel = np.concatenate([cols, f + cols])
    else:
        sel = cols
    Z, H = col_linear_act(X, W_in[:, sel], act)
    dZ = dY @ W_out[cols].T
    dH = _act_bwd(H, dZ, act)
    return {"dW_in_cols": X.T @ dH, "dW_out_rows": Z.T @ dY}


# ---------------------------------------------------------------------------
# Head-aligned fused-QKV shard ([TPSP] "注意力：按头切，以及 GQA 的约束",
# fused-QKV layout item; "GQA：KV 头比 query 头少")
# ---------------------------------------------------------------------------

def check_heads_divisible(n_h, n_kv, t):
    """Head-count rules ([TPSP] "注意力：按头切，以及 GQA 的约束" and "GQA：KV 头比
    query 头少"; [REVISIT] Megatron's ValueError): heads are the unit of the
    split, so t <= n_h and t | n_h. With t <= n_kv each rank takes n_kv / t
    whole KV heads (t | n_kv); with n_kv < t every KV head is replicated on
    t / n_kv ranks, which needs n_kv | t."""
    if t <= 0:
        raise ValueError("TP degree must be positive")
    if n_h % t != 0:
        raise ValueError(f"num_attention_heads ({n_h}) must be a multiple of "
                         f"tensor_model_parallel_size ({t}).")
    if t <= n_kv and n_kv % t != 0:
        raise ValueError(f"num_kv_heads ({n_kv}) must be a multiple of "
                         f"tensor_model_parallel_size ({t}).")
    if t > n_kv and t % n_kv != 0:
        raise ValueError(f"tensor_model_parallel_size ({t}) must be a multiple of "
                         f"num_kv_heads ({n_kv}) to replicate KV heads.")


def kv_heads_of_rank(n_kv, t, rank):
    """KV heads held by ``rank``: [r n_kv/t, (r+1) n_kv/t) when t <= n_kv;
    with n_kv < t the single head r // (t / n_kv), which the rank's query heads
    [r n_h/t, (r+1) n_h/t) all use (contiguous grouping: query head j uses KV
    head j // (n_h / n_kv))."""
    if t <= n_kv:
        return list(range(rank * (n_kv // t), (rank + 1) * (n_kv // t)))
    return [rank // (t // n_kv)]


def qkv_regroup_index(n_h, n_kv, d_h, t, rank):
    """Source columns of rank ``rank``'s slice of the fused QKV weight.

    Source layout [h, (n_h + 2 n_kv) d_h] = [Q heads 0..n_h-1 | K heads
    0..n_kv-1 | V heads 0..n_kv-1], each head's d_h columns contiguous. The
    rank's slice holds, in order, its own query heads, its own K heads and its
    own V heads ([TPSP] "几个实现细节", fused-QKV layout): query heads
    [r n_h/t, (r+1) n_h/t) and the KV heads of kv_heads_of_rank, so each query
    group sits with the KV head it shares. With n_kv < t the KV head is a
    replica, present on t / n_kv ranks ([TPSP] "GQA：KV 头比 query 头少").
    """
    check_heads_divisible(n_h, n_kv, t)
    if not 0 <= rank < t:
        raise ValueError(f"rank {rank} out of range for TP degree {t}")
    qh = n_h // t
    kv = kv_heads_of_rank(n_kv, t, rank)
    idx = []
    for head in range(rank * qh, (rank + 1) * qh):            # own Q heads
        idx.extend(range(head * d_h, (head + 1) * d_h))
    k_base = n_h * d_h
    for head in kv:                                           # own K heads
        idx.extend(range(k_base + head * d_h, k_base + (head + 1) * d_h))
    v_base = (n_h + n_kv) * d_h
    for head in kv:                                           # own V heads
        idx.extend(range(v_base + head * d_h, v_base + (head + 1) * d_h))
    return np.array(idx, dtype=np.int64)


def qkv_regroup(W_qkv, n_h, n_kv, d_h, t, rank):
    """W_r = W_qkv[:, qkv_regroup_index(...)] (exact copy of bf16 bit patterns)."""
    return np.ascontiguousarray(np.asarray(W_qkv)[:, qkv_regroup_index(n_h, n_kv, d_h, t, rank)])


def kv_replica_ranks(n_kv, t, head):
    """Ranks holding a replica of KV head ``head`` when n_kv < t."""
    r = t // n_kv
    return list(range(head * r, (head + 1) * r))


def kv_grad_accumulate(dst, src, n_h, n_kv, d_h, t):
    """One step of the replica-gradient sum ([TPSP] "GQA：KV 头比 query 头少": the
    replicas' K/V weight gradients are different partial sums). ``dst`` and
    ``src`` are two replica ranks' weight-gradient shards [h, (n_h/t + 2) d_h]
    laid out like their W_r; returns dst with its K|V columns (the last 2 d_h)
    plus src's. The Q columns belong to each rank alone and are kept."""
    check_heads_divisible(n_h, n_kv, t)
    if not n_kv < t:
        raise ValueError("KV heads are replicated only when n_kv < t")
    out = np.array(dst, dtype=np.float64, copy=True)
    q = (n_h // t) * d_h
    out[:, q:] += np.asarray(src, dtype=np.float64)[:, q:]
    return out


def kv_replica_grad_sum(dWs, n_h, n_kv, d_h, t):
    """The synchronised K|V gradient of every KV head: for head g, the sum in
    rank order of the K|V columns of the weight-gradient shards of the ranks
    in kv_replica_ranks(g). ``dWs``: the t shards. Returns {g: [h, 2 d_h]}."""
    q = (n_h // t) * d_h
    out = {}
    for g in range(n_kv):
        acc = None
        for r in kv_replica_ranks(n_kv, t, g):
            part = np.asarray(dWs[r], dtype=np.float64)[:, q:]
            acc = part.copy() if acc is None else acc + part
        out[g] = acc
    return out


def naive_split_index(n_h, n_kv, d_h, t, rank):
    """The wrong equal column split of the fused QKV weight (for negative tests)."""
    width = (n_h + 2 * n_kv) * d_h
    w = width // t
    return np.arange(rank * w, (rank + 1) * w, dtype=np.int64)


# ---------------------------------------------------------------------------
# Vocab-parallel LM head with cross-entropy ([TPSP] "词表并行：embedding 与交叉熵",
# "LM head 与交叉熵"): W_out [h, V] split by columns (vocab), rank i holding
# vocab ids [i V/t, (i+1) V/t); the logits z^(i) = X W_i are never gathered.
# ---------------------------------------------------------------------------

def vocab_ce_local(X, W_i, targets, vocab_start):
    """Rank i's local part of the fused cross-entropy: its logits z = X W_i
    [N, V/t]; per token the local maximum m_i, the local sum
    s_i = sum_v exp(z_v - m_i) over its vocab range, and the target logit z_y
    when the target id falls in [vocab_start, vocab_start + V/t) (0 otherwise:
    the target lands on exactly one rank)."""
    z = np.asarray(X, np.float64) @ np.asarray(W_i, np.float64)
    y = np.asarray(targets, np.int64) - vocab_start
    m = z.max(axis=1)
    s = np.exp(z - m[:, None]).sum(axis=1)
    inside = (y >= 0) & (y < z.shape[1])
    zy = np.where(inside, z[np.arange(z.shape[0]), np.clip(y, 0, z.shape[1] - 1)], 0.0)
    return m, s, zy


def vocab_ce_loss(X, W_shards, targets):
    """The page's four steps over t vocab shards, each over the shard's own
    logits: (1) the global max m of the local maxima (All-Reduce MAX);
    (2) S = sum over shards of sum_v exp(z_v - m) (All-Reduce SUM); (3) z_y
    from the one shard that holds the target (All-Reduce SUM);
    (4) loss = log S + m - z_y. Returns (loss, m, S) per token."""
    X = np.asarray(X, np.float64)
    zs = [X @ np.asarray(W, np.float64) for W in W_shards]
    m = np.max([z.max(axis=1) for z in zs], axis=0)                       # step 1
    S = np.sum([np.exp(z - m[:, None]).sum(axis=1) for z in zs], axis=0)  # step 2
    y = np.asarray(targets, np.int64)
    zy = np.zeros(X.shape[0])
    start = 0
    for z in zs:                                                          # step 3
        local = y - start
        inside = (local >= 0) & (local < z.shape[1])
        zy += np.where(inside, z[np.arange(z.shape[0]), np.clip(local, 0, z.shape[1] - 1)], 0.0)
        start += z.shape[1]
    return np.log(S) + m - zy, m, S                                       # step 4


def vocab_ce_bwd(X, W_i, targets, vocab_start, m, S, dloss):
    """Rank i's backward, local given the global m and S: dl/dz_v =
    softmax(z)_v - 1[v = y] on its vocab range, scaled by the upstream dloss
    per token; then the column-parallel backward dX_part = dZ W_i^T ({U}),
    dW_i = X^T dZ. Returns (dZ, dX_part, dW_i)."""
    X = np.asarray(X, np.float64)
    W_i = np.asarray(W_i, np.float64)
    z = X @ W_i
    p = np.exp(z - np.asarray(m, np.float64)[:, None]) / np.asarray(S, np.float64)[:, None]
    y = np.asarray(targets, np.int64) - vocab_start
    rows = np.nonzero((y >= 0) & (y < z.shape[1]))[0]
    p[rows, y[rows]] -= 1.0
    dZ = p * np.asarray(dloss, np.float64)[:, None]
    return dZ, dZ @ W_i.T, X.T @ dZ


def vocab_embed_fwd(ids, E_i, vocab_start):
    """Rank i's masked lookup ([TPSP] "输入 embedding"): the rank holds rows
    [vocab_start, vocab_start + V/t) of the table; a token whose id is in that
    range gets its row, any other token a zero row. Summing the ranks' outputs
    (the g All-Reduce) gives the full lookup. Exact copy of the bit patterns
    (uint16 bf16 rows in, uint16 out)."""
    E_i = np.asarray(E_i)
    ids = np.asarray(ids, np.int64) - vocab_start
    out = np.zeros((len(ids), E_i.shape[1]), dtype=E_i.dtype)
    inside = (ids >= 0) & (ids < E_i.shape[0])
    out[inside] = E_i[ids[inside]]
    return out


def vocab_embed_bwd(ids, dY, vocab_start, v_loc):
    """Gradient of rank i's table rows: dE_i[v] = sum of dY[n] over the tokens
    n whose id is vocab_start + v (rows no token uses are zero)."""
    dY = np.asarray(dY, np.float64)
    ids = np.asarray(ids, np.int64) - vocab_start
    dE = np.zeros((v_loc, dY.shape[1]))
    for n, v in enumerate(ids):
        if 0 <= v < v_loc:
            dE[v] += dY[n]
    return dE


# ---------------------------------------------------------------------------
# Shard arithmetic ([SB6] §6.1 notation and Pop Quiz)
# ---------------------------------------------------------------------------

class ShardError(ValueError):
    pass


def shard_shape(shape, elem_bytes, mesh, spec):
    """Local shape and bytes of A[...] sharded over a device mesh.

    ``mesh``: ordered mapping axis name -> size. ``spec``: per tensor dim, a
    tuple of mesh axis names the dim is split over (empty = not split). A dim
    split over several axes is divided by the product of their sizes; an axis
    that appears twice (in one dim or across dims) is illegal; axes the spec
    does not use replicate the shard. Returns (local_shape, local_bytes,
    total_bytes) with total_bytes = local_bytes * number of devices.
    """
    if len(spec) != len(shape):
        raise ShardError("spec must name the axes of every dim")
    used = []
    local = []
    for dim, axes in zip(shape, spec):
        div = 1
        for a in axes:
            if a not in mesh:
                raise ShardError(f"unknown mesh axis {a!r}")
            if a in used:
                raise ShardError(f"mesh axis {a!r} used twice")
            used.append(a)
            div *= int(mesh[a])
        if dim % div != 0:
            raise ShardError(f"dim {dim} not divisible by {div}")
        local.append(dim // div)
    local_bytes = int(np.prod(local, dtype=np.int64)) * elem_bytes if local else elem_bytes
    devices = int(np.prod([int(v) for v in mesh.values()], dtype=np.int64)) if mesh else 1
    return tuple(local), local_bytes, local_bytes * devices


# ---------------------------------------------------------------------------
# Llama-3 parameter and FLOP accounting ([TPSP] GQA section: per-card weight
# shapes; "精确的通信量": FLOPs)
# ---------------------------------------------------------------------------

def llama_shard_weight_shapes(h, n_h, n_kv, d_h, F, t):
    """Per-card weight shapes of one Llama layer at TP degree t (column splits
    on heads / F, row splits for W_O and W_down)."""
    return {
        "W_Q": (h, n_h * d_h // t),
        "W_K": (h, n_kv * d_h // t),
        "W_V": (h, n_kv * d_h // t),
        "W_O": (n_h * d_h // t, h),
        "W_gate": (h, F // t),
        "W_up": (h, F // t),
        "W_down": (F // t, h),
    }


def llama_layer_params(h, n_h, n_kv, d_h, F, t=1):
    """Matrix parameters of one layer on one card (RMSNorm weights excluded)."""
    return sum(a * b for a, b in llama_shard_weight_shapes(h, n_h, n_kv, d_h, F, t).values())


def llama_model_params(h, n_h, n_kv, d_h, F, L, V, tied=False):
    """Whole-model parameters: L layers, 2h norm weights per layer, final norm,
    input embedding [V,h] and (untied) LM head [h,V]."""
    per_layer = llama_layer_params(h, n_h, n_kv, d_h, F) + 2 * h
    emb = V * h * (1 if tied else 2)
    return L * per_layer + h + emb


def gemm_flops(M, N, K):
    """Multiply-add count of an [M,K] x [K,N] product, 2 M N K."""
    return 2 * M * N * K


def mlp_shard_flops(N, h, f, act, backward=False):
    """GEMM FLOPs of one MLP shard (elementwise work not counted)."""
    n_w = 2 * f if act == "swiglu" else f
    fwd = gemm_flops(N, n_w, h) + gemm_flops(N, h, f)
    if not backward:
        return fwd
    # dZ = dY W_out^T, dW_out = Z^T dY, dX = dH W_in^T, dW_in = X^T dH
    return (gemm_flops(N, f, h) + gemm_flops(f, h, N)
            + gemm_flops(N, h, n_w) + gemm_flops(h, n_w, N))


def rel_err(got, want):
    """max|got - want| / max|want| (the parity metric)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if want.size == 0:
        return 0.0
    den = np.max(np.abs(want))
    num = np.max(np.abs(got - want))
    return float(num / den) if den > 0 else float(num)

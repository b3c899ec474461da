/*
 * tpshard.h — C ABI of libtpshard.so: one GPU's share of a Megatron-style
 * tensor-parallel (TP) layer on AMD Instinct MI355X (gfx950).
 *
 * Sources (pages, by title and section):
 *   [TPSP]    hs-black, "张量并行与序列并行" (scaling-tensor-parallel):
 *             "矩阵乘法的两种切法" (column- and row-parallel linear and their
 *             backward), "MLP：先列后行，只通信一次" (GeLU / SwiGLU MLP shard),
 *             "注意力：按头切，以及 GQA 的约束" (head-aligned split, fused-QKV
 *             layout, bias rule), "GQA：KV 头比 query 头少".
 *   [REVISIT] pufanyi, "ml-revisit-infra", "Tensor Parallel" (identities,
 *             gradients, the head-count ValueError).
 *   [SB6]     r00kie-liu, "Scaling Book 入门第 6 章：分片矩阵乘法", §6.1
 *             (sharding notation, Pop Quiz).
 *
 * Conventions for every call below.
 *   Layout:    all matrices are dense, row-major, contiguous (leading
 *              dimension = number of columns). A linear layer is Y = X W with
 *              X[N,k], W[k,n] ([TPSP] notation; N = b*s tokens).
 *   Types:     "bf16" = bfloat16 bit patterns (2 bytes); "f32" = IEEE float.
 *              Products accumulate in f32 on the MFMA units; bf16 outputs are
 *              rounded to nearest even.
 *   Pointers:  device pointers (hipMalloc'd or torch CUDA tensors), 16-byte
 *              aligned. The caller owns every buffer; the library keeps no
 *              pointer to them after the call returns.
 *   Workspace: a product with too few output tiles for the CUs (N <= 64
 *              tokens, or a narrow shard such as the attention projections')
 *              splits K over workgroups and sums their f32 partials in a
 *              second kernel; tp_vocab_ce_fwd keeps per-tile records and
 *              tp_vocab_embed_bwd per-row flags. That scratch is device
 *              memory the caller provides: every call that may need it takes
 *              (void* workspace, size_t workspace_bytes), and the host-only
 *              query of the same name plus "_workspace_size", given the same
 *              sizes, returns how many bytes the call needs on the current
 *              device (0: none, workspace may then be NULL). A call whose
 *              workspace is NULL or smaller than that returns
 *              TP_ERR_INVALID_ARG before enqueuing anything. The workspace
 *              must be 16-byte aligned; its contents on entry do not matter
 *              and are undefined afterwards. It is in use until the call's
 *              work on `stream` has finished, so calls that may run at the
 *              same time (on different streams) need different workspaces.
 *              The library allocates no memory, keeps no pointer and never
 *              synchronises: every call can be captured into a HIP graph.
 *   Sizes:     N (tokens) is any value from 0 to 2^30 (N = 0 is a no-op).
 *              Model widths (k, n, h, f, k_loc; the LM head's v_loc) must be positive
 *              multiples of 64 and at most 2^20 (larger: UNSUPPORTED). No
 *              limit on a buffer's size: operands and outputs above 4 GiB
 *              are addressed like small ones.
 *   Streams:   `stream` is a hipStream_t (NULL = the legacy default stream).
 *              Work is enqueued asynchronously; no host synchronisation.
 *              Faults in kernels surface at the caller's next synchronisation.
 *   Errors:    arguments are validated before any launch; on failure nothing
 *              is enqueued, a status != TP_OK is returned and a message is
 *              kept in thread-local storage (tp_last_error). Calls are
 *              re-entrant across threads (the library holds no state besides
 *              each thread's last error message, each device's CU count and
 *              the address of each device's array of tp_col_linear_noalloc).
 *   {U}:       an f32 output marked {U} is a partial sum ("unreduced" in
 *              [TPSP]/[SB6] notation): the full result is the sum of the t
 *              ranks' outputs. The exchange that sums them (an all-reduce) is
 *              not part of one GPU's share; `accumulate = 1` adds into the
 *              output instead of overwriting it, so t shards computed one
 *              after another on one device sum in rank order.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, bad size or enum   */
    TP_ERR_NOT_DIVISIBLE = 2, /* a divisibility rule of the sharding is broken */
    TP_ERR_UNSUPPORTED = 3,   /* valid request outside what is implemented     */
    TP_ERR_HIP = 4            /* the HIP runtime reported an error at launch   */
} tp_status;

typedef enum {
    TP_ACT_NONE = 0,
    TP_ACT_GELU = 1,   /* exact GeLU, x * Phi(x)                              */
    TP_ACT_SWIGLU = 2  /* SiLU(gate) * up over [gate | up] weight halves      */
} tp_act;

/* Library version, (major << 16) | minor (0.2: caller-owned workspaces). */
int tp_version(void);

/* Message of the last failed call on this thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
const char* tp_last_error(void);

/*
 * Column-parallel linear with its local activation ([TPSP] "矩阵乘法的两种切法",
 * first identity; "MLP：先列后行" for the activation; [REVISIT] Column-wise TP).
 * The rank holds the full X and the column block W_i; its output columns need
 * no exchange.
 *   X      bf16 [N, k]          input (replicated on every rank)
 *   W      bf16 [k, n_w]        act NONE / GELU: n_w = n_out.
 *                               act SWIGLU: n_w = 2*n_out, W = [W_gate | W_up],
 *                               gate column j and up column j cover the same
 *                               F index (same F segment on this rank).
 *   Y      bf16 [N, n_out]      NONE: X W;  GELU: GeLU(X W);
 *                               SWIGLU: SiLU(X W_gate) * (X W_up).
 *   H_save bf16 [N, n_w] or NULL  receives the pre-activation X W (needed by
 *                               the backward). Must be NULL for act NONE.
 * Errors: INVALID_ARG (pointers, sizes, act), UNSUPPORTED (width not a
 * multiple of 64), HIP.
 */
tp_status tp_col_linear_workspace_size(int64_t N, int64_t k, int64_t n_out,
                                       int act, size_t* bytes);
tp_status tp_col_linear(const void* X, const void* W, void* Y,
                        int64_t N, int64_t k, int64_t n_out, int act,
                        void* H_save, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * tp_col_linear for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments except the workspace, the same kernels and results. A split
 * product's partials go to a device array inside the library (16 MiB, one
 * per device, held until the process ends) instead of a workspace; a call
 * whose split needs more (tp_col_linear_workspace_size > 16 MiB, e.g. wide
 * products at more than 64 tokens) returns TP_ERR_UNSUPPORTED before any
 * launch. Nothing is allocated. Every call on one device shares that array:
 * calls that may overlap on a device (different streams, or graphs replayed
 * concurrently) race on it and must be serialised by the caller.
 */
tp_status tp_col_linear_noalloc(const void* X, const void* W, void* Y,
                                int64_t N, int64_t k, int64_t n_out, int act,
                                void* H_save, void* stream);

/*
 * Row-parallel linear, partial sum ([TPSP] "矩阵乘法的两种切法", second
 * identity; [REVISIT] Row-wise TP). The rank holds the input slice
 * Z_i[N, k_loc] and the weight row block W_i[k_loc, n]; Z_i W_i is a
 * full-shape partial sum. No bias is ever added here: a row-parallel bias
 * belongs after the exchange ([TPSP] attention section, bias item).
 *   Z  bf16 [N, k_loc]   W  bf16 [k_loc, n]
 *   P  f32  [N, n] {U}   P = Z W, or P += Z W when accumulate != 0.
 */
tp_status tp_row_linear_partial_workspace_size(int64_t N, int64_t k_loc,
                                               int64_t n, size_t* bytes);
tp_status tp_row_linear_partial(const void* Z, const void* W, float* P,
                                int64_t N, int64_t k_loc, int64_t n,
                                int accumulate, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * The row-parallel partial computed in row chunks, for overlapping its
 * exchange with the product ([SB6] §6.6 / [TPSP] "把通信藏到计算后面": the
 * reduction of chunk c can run while chunk c + 1 is computed). The result is
 * that of tp_row_linear_partial. Token rows are cut into nchunks chunks of
 * ceil(N / nchunks) rows rounded up to 16 (the last may be shorter or
 * empty); after chunk c is enqueued, events[c] (a caller-created hipEvent_t)
 * is recorded on `stream`, so another stream can wait for exactly that
 * chunk. events may be NULL (no events). 1 <= nchunks <= 64.
 */
tp_status tp_row_linear_partial_chunked_workspace_size(int64_t N, int64_t k_loc,
                                                       int64_t n, int32_t nchunks,
                                                       size_t* bytes);
tp_status tp_row_linear_partial_chunked(const void* Z, const void* W, float* P,
                                        int64_t N, int64_t k_loc, int64_t n,
                                        int accumulate, int32_t nchunks,
                                        void* const* events, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * One rank's MLP share, forward ([TPSP] "MLP：先列后行，只通信一次"): first
 * matrix column-split with the activation applied locally, second matrix
 * row-split, giving the partial sum of the layer output.
 *   X      bf16 [N, h]
 *   W_in   bf16 [h, n_w]     GELU: n_w = f (A_i);  SWIGLU: n_w = 2f, [gate|up]
 *   W_out  bf16 [f, h]       (B_i / W_down,i)
 *   Z      bf16 [N, f]       activation output (input of the row-parallel GEMM,
 *                            kept for the backward's dW_out)
 *   H_save bf16 [N, n_w] or NULL   pre-activation (needed by the backward)
 *   P      f32  [N, h] {U}   Z W_out (accumulate != 0: added into P)
 * act must be GELU or SWIGLU. f = F/t is the per-rank MLP width.
 */
tp_status tp_mlp_shard_fwd_workspace_size(int64_t N, int64_t h, int64_t f,
                                          int act, size_t* bytes);
tp_status tp_mlp_shard_fwd(const void* X, const void* W_in, const void* W_out,
                           int64_t N, int64_t h, int64_t f, int act,
                           void* Z, void* H_save, float* P, int accumulate,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * One rank's MLP share, backward ([TPSP] "矩阵乘法的两种切法", backward
 * paragraph, applied to the MLP; [REVISIT] gradients):
 *   dZ     = dY W_out^T                          (row-parallel, local)
 *   dH     = dZ through the activation:
 *            GELU:   dA = dZ * GeLU'(A)
 *            SWIGLU: dG = dZ * U * SiLU'(G),  dU = dZ * SiLU(G),  dH = [dG|dU]
 *   dX_part = dH W_in^T         {U}              (column-parallel, partial)
 *   dW_in   = X^T dH                              (local)
 *   dW_out  = Z^T dY                              (local)
 * Inputs: X bf16 [N,h], W_in bf16 [h,n_w], W_out bf16 [f,h], H_save bf16
 * [N,n_w] (the forward's pre-activation, required), Z bf16 [N,f] (the forward's
 * activation output, required), dY bf16 [N,h].
 * Outputs: dH bf16 [N,n_w] (always written; the operand of the two
 * products that follow), dX_part f32 [N,h] {U} (accumulate != 0 adds into
 * it), dW_in f32 [h,n_w], dW_out f32 [f,h]. dZ itself is never stored.
 * dX_part, dW_in and dW_out may each be NULL: that product is skipped (with
 * all three NULL the call runs only dZ and the activation backward). X is
 * read only for dW_in, W_in only for dX_part, Z only for dW_out.
 * The workspace query counts all three products.
 */
tp_status tp_mlp_shard_bwd_workspace_size(int64_t N, int64_t h, int64_t f,
                                          int act, size_t* bytes);
tp_status tp_mlp_shard_bwd(const void* X, const void* W_in, const void* W_out,
                           const void* H_save, const void* Z, const void* dY,
                           int64_t N, int64_t h, int64_t f, int act,
                           void* dH, float* dX_part, float* dW_in, float* dW_out,
                           int accumulate, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Column-parallel linear, backward ([TPSP] "矩阵乘法的两种切法": dX is a partial
 * sum over ranks, dW_i is local). Used for the fused-QKV projection.
 *   X bf16 [N,k], W bf16 [k,n], dY bf16 [N,n]
 *   dX_part f32 [N,k] {U} = dY W^T (NULL: skipped; accumulate != 0 adds)
 *   dW      f32 [k,n]     = X^T dY (NULL: skipped)
 */
tp_status tp_col_linear_bwd_workspace_size(int64_t N, int64_t k, int64_t n,
                                           size_t* bytes);
tp_status tp_col_linear_bwd(const void* X, const void* W, const void* dY,
                            float* dX_part, float* dW,
                            int64_t N, int64_t k, int64_t n, int accumulate,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The column-parallel backward with dX_part computed in row chunks, for
 * hiding its exchange ([TPSP] "把通信藏到计算后面": a column-parallel layer's
 * dX exchange can run while dW = X^T dY, which does not need it, is computed;
 * an output cut into chunks can be sent a chunk at a time). The results are
 * those of tp_col_linear_bwd. dX_part comes first, in nchunks chunks of
 * token rows (ceil(N / nchunks) rows rounded up to 16; the last may be
 * shorter or empty); after chunk c is enqueued, events[c] (a caller-created
 * hipEvent_t) is recorded on `stream`, so another stream can wait for
 * exactly that chunk. Then dW, over all N tokens, when dW is not NULL.
 * events may be NULL (no events). dX_part must not be NULL; accumulate != 0
 * adds into dX_part only. 1 <= nchunks <= 64. The chunks and dW use the
 * workspace one after another; the query counts dW.
 */
tp_status tp_col_linear_bwd_chunked_workspace_size(int64_t N, int64_t k, int64_t n,
                                                   int32_t nchunks, size_t* bytes);
tp_status tp_col_linear_bwd_chunked(const void* X, const void* W, const void* dY,
                                    float* dX_part, float* dW,
                                    int64_t N, int64_t k, int64_t n, int accumulate,
                                    int32_t nchunks, void* const* events,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Row-parallel linear, backward ([TPSP] "矩阵乘法的两种切法": both gradients are
 * local). Used for the attention output projection W_O.
 *   Z bf16 [N,k_loc], W bf16 [k_loc,n], dY bf16 [N,n]
 *   dZ bf16 [N,k_loc] = dY W^T (NULL: skipped)
 *   dW f32  [k_loc,n] = Z^T dY (NULL: skipped)
 */
tp_status tp_row_linear_bwd_workspace_size(int64_t N, int64_t k_loc, int64_t n,
                                           size_t* bytes);
tp_status tp_row_linear_bwd(const void* Z, const void* W, const void* dY,
                            void* dZ, float* dW,
                            int64_t N, int64_t k_loc, int64_t n,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-rank regroup of the fused QKV weight ([TPSP] attention section, fused
 * QKV item: an equal column split is wrong; each rank's slice must hold its
 * own Q heads, then its own K heads, then its own V heads; "GQA：KV 头比 query
 * 头少": a query group stays with the KV head it shares).
 *   W_qkv bf16 [h, (n_h + 2 n_kv) d_h] = [Q heads 0..n_h-1 | K heads 0..n_kv-1
 *         | V heads 0..n_kv-1], each head's d_h columns contiguous.
 *   W_r   bf16 [h, (n_h/t + 2 c) d_h] = [Q heads r n_h/t .. (r+1) n_h/t - 1
 *         | c K heads | the same c V heads], where
 *         t <= n_kv: c = n_kv/t, KV heads r n_kv/t .. (r+1) n_kv/t - 1;
 *         n_kv < t:  c = 1, KV head r / (t/n_kv), replicated on the t/n_kv
 *                    ranks whose query heads use it.
 * A bit-exact copy. Errors: NOT_DIVISIBLE when t does not divide n_h
 * (message in Megatron's wording, [REVISIT]), when t <= n_kv and t does not
 * divide n_kv, or when n_kv < t and n_kv does not divide t; INVALID_ARG for
 * rank outside [0, t), d_h not a multiple of 8, bad pointers.
 */
tp_status tp_qkv_regroup(const void* W_qkv, void* W_r, int64_t h,
                         int32_t n_h, int32_t n_kv, int32_t d_h,
                         int32_t t, int32_t rank, void* stream);

/*
 * Replicated KV heads, backward ([TPSP] "GQA：KV 头比 query 头少": with n_kv < t
 * each KV head sits on t/n_kv ranks, and their K/V weight gradients are
 * different partial sums that an extra exchange must sum). The single-device
 * stand-in for that exchange: called once per further replica, in rank
 * order, it adds the K|V columns of one replica rank's weight-gradient shard
 * into another's.
 *   dW_dst, dW_src f32 [h, (n_h/t + 2) d_h], laid out like the ranks' W_r
 *   (tp_col_linear_bwd's dW of the QKV projection);
 *   dW_dst[:, (n_h/t) d_h :] += dW_src[:, (n_h/t) d_h :]; the Q columns of
 *   dW_dst are left as they are.
 * Errors: INVALID_ARG unless n_kv < t (no replicas otherwise), for d_h not a
 * multiple of 4 or bad pointers; NOT_DIVISIBLE as for tp_qkv_regroup.
 */
tp_status tp_kv_grad_accumulate(float* dW_dst, const float* dW_src, int64_t h,
                                int32_t n_h, int32_t n_kv, int32_t d_h,
                                int32_t t, void* stream);

/*
 * Vocab-parallel LM head with fused cross-entropy, one rank's share
 * ([TPSP] "词表并行：embedding 与交叉熵", "LM head 与交叉熵"): W_out [h, V] is
 * split by columns; rank i holds vocab ids [vocab_start, vocab_start + v_loc)
 * (v_loc = V/t, the vocabulary padded so that it divides into multiples of
 * 64). Its logits z = X W_i [N, v_loc] are never written to memory.
 *   X bf16 [N,h], W_i bf16 [h,v_loc], targets int32 [N] (vocab ids over the
 *   whole vocabulary; 4-byte aligned).
 *   m_i, s_i, zy_i f32 [N]: per token the local max of z, sum of
 *   exp(z - m_i) over the rank's range, and z of the target when the target
 *   is in the range (0 otherwise).
 * Its workspace holds per-tile records, 12 bytes per token and 64-column
 * block: N * 4 * ceil(v_loc / 256) * 12 bytes; when (h + 512) * v_loc * 2
 * reaches 2^31 (a weight window past 32-bit offsets), one per 112-column
 * block: N * 2 * ceil(v_loc / 224) * 12 bytes.
 */
tp_status tp_vocab_ce_fwd_workspace_size(int64_t N, int64_t h, int64_t v_loc,
                                         size_t* bytes);
tp_status tp_vocab_ce_fwd(const void* X, const void* W_i, const int32_t* targets,
                          int64_t vocab_start, int64_t N, int64_t h, int64_t v_loc,
                          float* m_i, float* s_i, float* zy_i, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The exchange of the fused cross-entropy, on one device (the page's three
 * All-Reduces of [N]-sized statistics: MAX of the local maxima, SUM of the
 * exponential sums, SUM of the target logits): the t ranks' statistics,
 * stacked f32 [t][N] in rank order, give per token m = max_i m_i,
 * S = sum_i s_i exp(m_i - m) (each rank's sum rescaled to the global max),
 * z_y = sum_i zy_i, and loss = log S + m - z_y.
 *   loss f32 [N]; m, S f32 [N] (either may be NULL) for the backward.
 */
tp_status tp_vocab_ce_combine(const float* m_parts, const float* s_parts,
                              const float* zy_parts, int32_t t, int64_t N,
                              float* loss, float* m, float* S, void* stream);

/*
 * Backward of one rank's share, local given the global m and S ([TPSP] "LM
 * head 与交叉熵": dl/dz_v = softmax(z)_v - 1[v = y]):
 *   dZ bf16 [N,v_loc] = (exp(z - m) / S - one-hot(target)) * dloss, with z
 *   recomputed as X W_i (dZ is caller-owned scratch, like dH);
 *   dX_part f32 [N,h] = dZ W_i^T ({U}; accumulate = 1 adds into it);
 *   dW_i f32 [h,v_loc] = X^T dZ.
 *   m, S, dloss f32 [N] (dloss: the upstream gradient of each token's loss).
 */
tp_status tp_vocab_ce_bwd_workspace_size(int64_t N, int64_t h, int64_t v_loc,
                                         size_t* bytes);
tp_status tp_vocab_ce_bwd(const void* X, const void* W_i, const int32_t* targets,
                          int64_t vocab_start, const float* m, const float* S,
                          const float* dloss, int64_t N, int64_t h, int64_t v_loc,
                          void* dZ, float* dX_part, float* dW_i, int accumulate,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Vocab-parallel input embedding, one rank's share ([TPSP] "输入 embedding"):
 * the rank holds table rows [vocab_start, vocab_start + v_loc). A token whose
 * id is in that range gets its row, any other token a zero row; the sum of
 * the ranks' outputs (the exchange after this row-parallel layer) is the
 * full lookup.
 *   ids int32 [N] (4-byte aligned), E_i bf16 [v_loc, h], out bf16 [N, h].
 *   accumulate = 0: out is overwritten (zero rows included, a bit-exact
 *   copy); accumulate = 1: the rank's rows are added into out (in f32,
 *   rounded once to bf16: exact over ranks that partition the vocabulary)
 *   and the other rows are left as they are, so calling the t ranks in turn
 *   on one buffer sums their outputs.
 */
tp_status tp_vocab_embed_fwd(const int32_t* ids, const void* E_i, int64_t vocab_start,
                             int64_t N, int64_t v_loc, int64_t h, void* out,
                             int accumulate, void* stream);

/*
 * Its backward: dE_i f32 [v_loc, h], row v = the sum of dY[n] over the tokens
 * n whose id is vocab_start + v, added in token order (deterministic); rows
 * no token uses are zero. dY f32 [N, h]. h <= 16384 (else UNSUPPORTED).
 * Its workspace holds a row count, a flag per table row and a list of the
 * rows the tokens use: 4 * (1 + v_loc + min(N, v_loc)) bytes rounded up to
 * 16, cleared by the call itself (any earlier contents are fine).
 */
tp_status tp_vocab_embed_bwd_workspace_size(int64_t N, int64_t v_loc, int64_t h,
                                            size_t* bytes);
tp_status tp_vocab_embed_bwd(const int32_t* ids, const float* dY, int64_t vocab_start,
                             int64_t N, int64_t v_loc, int64_t h, float* dE_i,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shard arithmetic of a tensor over a device mesh ([SB6] §6.1): host only,
 * no device work. A[I_{XY}, J] splits dim I over mesh axes X and Y (divided
 * by their product); axes no dim uses replicate the shard.
 *   shape[ndim], elem_bytes > 0, axis_sizes[n_axes] (n_axes <= 32),
 *   dim_axis_mask[ndim]: bit a set = dim is split over mesh axis a.
 * Outputs: local_shape_out[ndim], *local_bytes_out, *total_bytes_out
 * (= local bytes times the number of devices, the product of axis sizes).
 * Errors: INVALID_ARG when one mesh axis splits two dims (A[I_X, J_X] is
 * illegal) or for bad arguments; NOT_DIVISIBLE when a dim does not divide.
 */
tp_status tp_shard_shape(int32_t ndim, const int64_t* shape, int32_t elem_bytes,
                         int32_t n_axes, const int64_t* axis_sizes,
                         const uint32_t* dim_axis_mask,
                         int64_t* local_shape_out, int64_t* local_bytes_out,
                         int64_t* total_bytes_out);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */

/*
 * libcce: Cut Cross-Entropy for AMD MI355X (gfx950), C ABI.
 *
 * What is computed (Cut Cross-Entropy abstract, taxoreview.com page dblp:393/3562, sentences
 * 3-6 and 9): token embeddings E [N,D], classifier rows C [V,D] and targets t [N] give
 *
 *     z[n,v]  = E[n,:] . C[v,:]                         (logits: kept on chip, never stored)
 *     lse[n]  = log sum_v exp(z[n,v])                    (log-sum-exp over the vocabulary)
 *     loss[n] = lse[n] - z[n, t[n]]     (0 when t[n] == ignore_index)
 *
 * and the gradients of sum_n dloss[n] loss[n]: dE = G C and dC = G^T E, where
 * G[n,v] = dloss[n] (softmax[n,v] - [v == t[n]]).  The backward skips the 64 x 64 blocks of G
 * whose softmax entries all lie below filter_eps and that hold no target (sentence 9's
 * gradient filtering); an optional entry floor drops single entries inside the kept blocks.
 *
 * Conventions shared by every call:
 *   - E and C are row-major and contiguous, of the same dtype (cce_dtype); D is the row length.
 *   - targets is int64 [N]; a row whose target equals ignore_index is "ignored": its loss is 0,
 *     its gradient rows are 0, and it never makes a filter block significant.
 *   - All array arguments are device pointers into memory the caller owns (hipMalloc or a
 *     framework allocator).  E, C, dE, dC and the workspace must be 16-byte aligned (the
 *     kernels move them in 16-byte vectors); a misaligned one is rejected with
 *     CCE_ERR_INVALID_ARGUMENT.  The library never allocates or frees device memory and the
 *     calls of this header keep no state between calls; scratch memory is the caller's
 *     workspace (query its size first).  Two exceptions: cce_forward_no_workspace keeps its
 *     scratch in a static device array (below), and the benchmark timing hook of
 *     cce_timing.h is process-wide state, off unless started.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work on
 *     that stream and returns; no host synchronisation happens inside.  Calls that share a
 *     workspace must not run concurrently on different streams.
 *   - Argument errors are detected on the host before anything is enqueued, and reported as
 *     CCE_ERR_INVALID_ARGUMENT / CCE_ERR_UNSUPPORTED / CCE_ERR_WORKSPACE_TOO_SMALL; launch
 *     failures as CCE_ERR_HIP.  N == 0 is a valid no-op.
 *   - Validity: N >= 0, V >= 1, D >= 1, D % 8 == 0 for bf16 and D % 4 == 0 for fp32,
 *     N, V, D < 2^31, non-null pointers when N > 0, filter_eps and entry_floor finite and >= 0.
 *   - Limits of the gfx950 kernels (CCE_ERR_UNSUPPORTED beyond them): N <= 2^24, V <= 2^24,
 *     D <= 65536.
 *   - Two environment variables tune the backward's plan (for measurements; unset, the plan
 *     below applies).  Each is read once per process, when a backward is first planned, and
 *     the workspace queries follow the same plan:
 *       CCE_VC  vocabulary chunk rows (rounded down to a multiple of 256, at most 8192): only
 *               narrows the chunks;
 *       CCE_NC  token block size (rounded down to a multiple of 256, 256 .. 65536): replaces
 *               the default 16384 (bf16) / 8192 (fp32), so the G store of the backward grows
 *               to 2 * Nc * Vc * sizeof(dtype) bytes (up to 2 GiB for bf16) when it widens them.
 */
#ifndef LIBCCE_CCE_H
#define LIBCCE_CCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two enums are int-sized, and their range sentinels make every int value a valid object
 * of the type, so a caller's out-of-range value (which the calls reject) is never undefined in
 * the library's C++. */
typedef enum {
  CCE_OK = 0,
  CCE_ERR_INVALID_ARGUMENT = 1,
  CCE_ERR_UNSUPPORTED = 2,
  CCE_ERR_WORKSPACE_TOO_SMALL = 3,
  CCE_ERR_HIP = 4,
  CCE_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  CCE_STATUS_RANGE_MAX_ = 0x7fffffff
} cce_status;

typedef enum {
  CCE_F32 = 0,
  CCE_BF16 = 1,
  CCE_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  CCE_DTYPE_RANGE_MAX_ = 0x7fffffff
} cce_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* cce_status_string(cce_status s);

/* Device workspace bytes needed by cce_forward / cce_backward / cce_loss_mean for a problem
 * (pure host functions; 0 for invalid sizes).  grad_dtype is the dtype the gradients are
 * requested in (the backward needs fp32 accumulators only for bf16 gradients).
 *   forward : splits * N * 8 bytes, splits <= 256 vocabulary ranges (an LSE partial per token
 *             and range), rounded to 256 bytes: O(N).
 *   backward: the softmax-gradient store of two (token block, vocabulary chunk) pairs in
 *             flight, 2 * Nc * Vc * sizeof(dtype) bytes with Nc <= 16384 tokens (8192 for
 *             fp32 inputs) and Vc <= 8192 columns, and their 64 x 64 block flags: bounded by a
 *             constant (at most 512 MiB unless CCE_NC widens the token blocks), however large
 *             N and V are;
 *             + 4 * ceil(N/256) bytes (each token tile's smallest LSE);
 *             + with bf16 gradients, N * D * 4 bytes for the fp32 dE accumulator and, when N
 *               exceeds one token block, Vc * D * 4 bytes for one chunk's fp32 dC accumulator.
 *             No N * V term.
 *   mean    : forward + backward + 8 * roundup(N,64) + 256. */
size_t cce_forward_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dtype);
size_t cce_backward_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dtype,
                                    cce_dtype grad_dtype);
size_t cce_loss_mean_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dtype,
                                     cce_dtype grad_dtype);

/* Forward (abstract sentences 4-6): per-token loss and log-sum-exp.
 *   E [N,D], C [V,D]     dtype `dtype`, device, read only.
 *   targets [N]          int64, device.  Values outside [0,V) other than ignore_index are
 *                        errors found on the device: that row's loss is NaN and *err_flag is
 *                        set to 1 (if err_flag is non-NULL); read it after synchronising.
 *   loss [N], lse [N]    fp32, device, written.  lse is the natural-log LSE; it is written
 *                        for ignored rows too.
 *   tile_max             fp32, device, NULL or cce_tile_max_count() floats (4-byte aligned),
 *                        written: for every 256-token x 256-row tile of the logits (token tile
 *                        i, vocabulary tile j) and each of its eight 128-row x 64-token parts
 *                        w, the largest logit times log2(e), at [(i * ceil(V/256) + j) * 8 +
 *                        w] (-inf where a part holds no row < V or no token < N).  Passed on
 *                        to cce_backward, it lets the backward skip negligible tiles.  It is
 *                        N * V / 2048 bytes (1 MB at N = 8192, V = 256000): an optional output
 *                        with an N * V term, outside the O(N) workspace.
 *   ws, ws_bytes         device workspace of at least cce_forward_workspace_bytes().
 *   err_flag             device int32 or NULL; only ever set to 1, never cleared. */
cce_status cce_forward(const void* E, const void* C, const int64_t* targets,
                       int64_t N, int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                       float* loss, float* lse, float* tile_max, void* ws, size_t ws_bytes,
                       int32_t* err_flag, void* stream);

/* cce_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments, results and errors
 * as cce_forward without the workspace: the forward's scratch (the per-token LSE partials,
 * cce_forward_workspace_bytes() of it) lives in a static device array of
 * cce_forward_no_workspace_max_bytes() = 16 MiB that each GPU holds for the life of the
 * process.  Problems needing more (N * splits * 8 bytes > 16 MiB, e.g. N > 2^21 with one
 * vocabulary range) are refused on the host with CCE_ERR_WORKSPACE_TOO_SMALL.  The array's
 * device address is looked up once per device, on the first call with that device current.
 * Every call on one GPU shares the array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller.  Nothing in it needs clearing; each
 * call overwrites what it reads. */
cce_status cce_forward_no_workspace(const void* E, const void* C, const int64_t* targets,
                                    int64_t N, int64_t V, int64_t D, cce_dtype dtype,
                                    int64_t ignore_index, float* loss, float* lse,
                                    float* tile_max, int32_t* err_flag, void* stream);
size_t cce_forward_no_workspace_max_bytes(void);

/* Floats of cce_forward's tile_max for a problem: ceil(N/256) * ceil(V/256) * 8 (pure host;
 * 0 for invalid sizes). */
int64_t cce_tile_max_count(int64_t N, int64_t V, int64_t D, cce_dtype dtype);

/* Backward (abstract sentences 4 and 9): dE and dC of sum_n dloss[n] * loss[n].
 *   dloss                fp32, device: [N] when dloss_stride == 1, one scalar when 0.
 *   E, C, targets        as in cce_forward.  Invalid targets do not fault; their rows get no
 *                        one-hot term (the forward reports them).
 *   lse [N]              fp32, device: the lse written by cce_forward for the same E, C.
 *   tile_max             NULL, or the tile_max written by cce_forward for the same E, C and
 *                        targets: with filter_eps > 0, a 256 x 256 tile whose largest logit
 *                        minus the smallest LSE of its non-ignored tokens lies below
 *                        ln(filter_eps) (by a margin of 2^-10 in log2 units) and that holds no
 *                        token's target is not recomputed: every block of it is negligible, and
 *                        it is flagged and counted as such.  The results are the same as
 *                        without tile_max.
 *   filter_eps           gradient filtering threshold on softmax values (not scaled by dloss);
 *                        0 disables it.  A 64-token x 64-vocabulary block of G is skipped (taken
 *                        as 0) when all of its softmax entries are < filter_eps and it holds no
 *                        target of a non-ignored row.  2^-12 is the benchmarks' threshold.
 *   entry_floor          0 (off, the default reading) or a softmax threshold: inside the blocks
 *                        that are kept, an entry other than the row's target whose softmax
 *                        value is < entry_floor is dropped too.  An approximation on top of the
 *                        block filter, for callers that accept it: it moves row n of dE by at
 *                        most dloss[n] * entry_floor * sum_v |C[v]| and row v of dC by at most
 *                        entry_floor * sum_n dloss[n] |E[n]| (Euclidean norms).
 *   dE [N,D], dC [V,D]   device, overwritten (no need to clear them first), in grad_dtype:
 *                        CCE_F32, or CCE_BF16 (accumulated in fp32, rounded to nearest even
 *                        once at the end; 16-byte aligned like every array argument).
 *   ws, ws_bytes         device workspace of at least cce_backward_workspace_bytes(..., grad_dtype).
 *   skip_stats           device int64[2] or NULL: [0] = skipped 64x64 blocks,
 *                        [1] = all blocks, ceil(N/64) * ceil(V/64). */
cce_status cce_backward(const float* dloss, int64_t dloss_stride, const void* E, const void* C,
                        const int64_t* targets, const float* lse, const float* tile_max,
                        int64_t N, int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                        float filter_eps, float entry_floor, void* dE, void* dC,
                        cce_dtype grad_dtype, void* ws, size_t ws_bytes, int64_t* skip_stats,
                        void* stream);

/* Mean-reduced convenience call: loss_mean = sum over non-ignored rows of loss / N_valid and
 * the gradients of that mean (dloss = 1 / N_valid for every row).  With N_valid == 0 the mean
 * and both gradients are 0.  loss_mean and n_valid (NULL allowed) are device scalars.
 *   filter_eps, entry_floor, dE, dC, grad_dtype as in cce_backward.
 *   ws: at least cce_loss_mean_workspace_bytes(..., grad_dtype); err_flag, skip_stats as
 *   above. */
cce_status cce_loss_mean(const void* E, const void* C, const int64_t* targets, int64_t N,
                         int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                         float filter_eps, float entry_floor, float* loss_mean, int64_t* n_valid,
                         void* dE, void* dC, cce_dtype grad_dtype, void* ws, size_t ws_bytes,
                         int32_t* err_flag, int64_t* skip_stats, void* stream);

/* Vocabulary-sharded form of the same computation (the tensor-parallel classifier head: each
 * device holds rows [vocab_offset, vocab_offset + V) of the full classifier, V_total rows in
 * all).  The log-sum-exp over the full vocabulary is the log-sum-exp of the shards' LSEs
 * (sentence 5's log-sum-exp, split over devices), so a forward is one cce_forward_shard per
 * shard, an exchange of 2 floats per token and shard, and one cce_merge_shards; the backward is
 * one cce_backward_shard per shard with the merged LSE, each giving its shard's rows of dC and
 * a partial dE that the shards sum.
 *
 * cce_forward_shard: E [N,D], C [V,D] = this shard's rows, targets [N] in the full vocabulary.
 *   lse_shard [N]     fp32, device, written: log sum over this shard's rows of exp(E C^T).
 *   target_logit [N]  fp32, device, written: E[n] . C[t[n] - vocab_offset] when the target is
 *                     one of this shard's rows (and not ignore_index), else 0.
 *   tile_max          NULL or cce_tile_max_count(N, V, D, dtype) floats: as in cce_forward,
 *                     over this shard's rows.
 *   ws, ws_bytes      at least cce_forward_workspace_bytes(N, V, D, dtype).
 *   Targets outside the shard are not errors here; cce_merge_shards checks them. */
cce_status cce_forward_shard(const void* E, const void* C, const int64_t* targets, int64_t N,
                             int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                             int64_t vocab_offset, float* lse_shard, float* target_logit,
                             float* tile_max, void* ws, size_t ws_bytes, void* stream);

/* cce_merge_shards: lse_shards [n_shards][N] and target_logits [n_shards][N] (fp32, device,
 * shard-major), as written by cce_forward_shard for shards that together cover [0, V_total)
 * once.  Writes lse [N] and loss [N] exactly as cce_forward does (loss 0 for ignored rows; a
 * target outside [0, V_total) gives NaN and sets *err_flag to 1 when err_flag is non-NULL).
 * No workspace. */
cce_status cce_merge_shards(const float* lse_shards, const float* target_logits,
                            int64_t n_shards, int64_t N, const int64_t* targets,
                            int64_t ignore_index, int64_t V_total, float* loss, float* lse,
                            int32_t* err_flag, void* stream);

/* cce_backward_shard: cce_backward for one shard.  lse [N] is the merged (full-vocabulary) LSE;
 * tile_max is NULL or this shard's tile_max from cce_forward_shard; dC [V,D] receives this
 * shard's rows of dC; dE [N,D] receives this shard's term of dE (the shards' dE sum to the full
 * dE).  Filter blocks are aligned to the shard's rows (64-row blocks from vocab_offset).
 * Workspace: cce_backward_workspace_bytes(N, V, D, dtype, grad_dtype). */
cce_status cce_backward_shard(const float* dloss, int64_t dloss_stride, const void* E,
                              const void* C, const int64_t* targets, const float* lse,
                              const float* tile_max, int64_t N, int64_t V, int64_t D,
                              cce_dtype dtype, int64_t ignore_index, int64_t vocab_offset,
                              float filter_eps, float entry_floor, void* dE, void* dC,
                              cce_dtype grad_dtype, void* ws, size_t ws_bytes,
                              int64_t* skip_stats, void* stream);

/* Launch-shape introspection for reports (pure host): the vocabulary split count of the
 * forward, the widest vocabulary chunk Vc of the backward (chunks are balanced: ceil(V / 8192)
 * chunks of whole 256-row tiles), and the token block Nc of the backward (balanced blocks of
 * whole 256-token tiles, at most 16384 tokens for bf16 inputs and 8192 for fp32). */
int64_t cce_forward_splits(int64_t N, int64_t V, int64_t D, cce_dtype dtype);
int64_t cce_backward_chunk(int64_t N, int64_t V, int64_t D, cce_dtype dtype);
int64_t cce_backward_token_block(int64_t N, int64_t V, int64_t D, cce_dtype dtype);

#ifdef __cplusplus
}
#endif

#endif /* LIBCCE_CCE_H */

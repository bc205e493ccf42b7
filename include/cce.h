/*
 * libcce: Cut Cross-Entropy for AMD MI355X (gfx950), C ABI.
 *
 * The operation (the Cut Cross-Entropy abstract on taxoreview.com, page dblp:393/3562,
 * sentences 3-6): for token embeddings E [N,D] and classifier rows C [V,D],
 *
 *     z[n,v]  = E[n,:] . C[v,:]                         (logits, never written to memory)
 *     lse[n]  = log sum_v exp(z[n,v])                    (log-sum-exp over the vocabulary)
 *     loss[n] = lse[n] - z[n, t[n]]     (0 when t[n] == ignore_index)
 *
 * and its gradients dE = G C, dC = G^T E with G[n,v] = dloss[n] (softmax[n,v] - [v == t[n]]),
 * where the backward skips gradient blocks whose softmax entries are all below filter_eps and
 * drops single entries below filter_eps * 2^-8 (same abstract, sentence 9).  The N x V logit
 * matrix is never materialised in device memory.
 *
 * Conventions shared by every call:
 *   - E and C are row-major and contiguous, of the same dtype (cce_dtype); D is the row length.
 *   - targets is int64 [N]; a row whose target equals ignore_index is "ignored": its loss is 0,
 *     its gradient rows are 0, and it never makes a filter block significant.
 *   - All array arguments are device pointers into memory the caller owns (hipMalloc or a
 *     framework allocator).  E, C, dE, dC and the workspace must be 16-byte aligned (the
 *     kernels move them in 16-byte vectors); a misaligned one is rejected with
 *     CCE_ERR_INVALID_ARGUMENT.  The library never allocates or frees device memory and keeps
 *     no per-call state; scratch memory is the caller's workspace (query its size first).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work on
 *     that stream and returns; no host synchronisation happens inside.  Calls that share a
 *     workspace must not run concurrently on different streams.
 *   - Argument errors are detected on the host before anything is enqueued, and reported as
 *     CCE_ERR_INVALID_ARGUMENT / CCE_ERR_UNSUPPORTED / CCE_ERR_WORKSPACE_TOO_SMALL; launch
 *     failures as CCE_ERR_HIP.  N == 0 is a valid no-op.
 *   - Validity: N >= 0, V >= 1, D >= 1, D % 8 == 0 for bf16 and D % 4 == 0 for fp32,
 *     N, V, D < 2^31, non-null pointers when N > 0, filter_eps finite and >= 0.
 *   - Limits of the gfx950 kernels (CCE_ERR_UNSUPPORTED beyond them): N <= 2^24, V <= 2^24,
 *     D <= 65536.
 */
#ifndef LIBCCE_CCE_H
#define LIBCCE_CCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCE_OK = 0,
  CCE_ERR_INVALID_ARGUMENT = 1,
  CCE_ERR_UNSUPPORTED = 2,
  CCE_ERR_WORKSPACE_TOO_SMALL = 3,
  CCE_ERR_HIP = 4
} cce_status;

typedef enum { CCE_F32 = 0, CCE_BF16 = 1 } cce_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* cce_status_string(cce_status s);

/* Device workspace bytes needed by cce_forward / cce_backward / cce_loss_mean for a problem.
 * Pure host functions.  Each formula is linear in N for fixed V and D (no N*V term):
 *   forward : splits * N * 8 bytes, splits <= 256 vocabulary ranges (an on-chip LSE partial
 *             per token and range), rounded to 256 bytes;
 *   backward: 2 * roundup(N,256) * Vc * sizeof(dtype): the softmax-gradient tile store of two
 *             vocabulary chunks in flight (Vc <= 8192 columns), plus their 64x64 block flags,
 *             plus N * D * 4 bytes for the fp32 dE accumulator used when the gradients are
 *             requested in bf16, plus 4 * ceil(N/256) bytes (each token tile's smallest LSE);
 *   mean    : forward + backward + 8 * roundup(N,64) + 256.
 * Returns 0 for invalid sizes. */
size_t cce_forward_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dtype);
size_t cce_backward_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dtype);
size_t cce_loss_mean_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dtype);

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
 *                        to cce_backward, it lets the backward skip negligible tiles.
 *   ws, ws_bytes         device workspace of at least cce_forward_workspace_bytes().
 *   err_flag             device int32 or NULL; only ever set to 1, never cleared. */
cce_status cce_forward(const void* E, const void* C, const int64_t* targets,
                       int64_t N, int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                       float* loss, float* lse, float* tile_max, void* ws, size_t ws_bytes,
                       int32_t* err_flag, void* stream);

/* Floats of cce_forward's tile_max for a problem: ceil(N/256) * ceil(V/256) * 8 (pure host;
 * 0 for invalid sizes).  Optional output, so not part of the O(N) workspace. */
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
 *                        0 disables it.  A 64-token x 64-vocabulary block of G is skipped when
 *                        all of its softmax entries are < filter_eps and it holds no target of
 *                        a non-ignored row; in the blocks that are kept, an entry other than
 *                        the row's target is dropped (taken as 0) when its softmax value is
 *                        < filter_eps * 2^-8.  2^-12 is the threshold used by the benchmarks.
 *   dE [N,D], dC [V,D]   device, overwritten (no need to clear them first), in grad_dtype:
 *                        CCE_F32, or CCE_BF16 (accumulated in fp32, rounded to nearest even
 *                        once at the end; 16-byte aligned like every array argument).
 *   ws, ws_bytes         device workspace of at least cce_backward_workspace_bytes().
 *   skip_stats           device int64[2] or NULL: [0] = skipped 64x64 blocks,
 *                        [1] = all blocks, ceil(N/64) * ceil(V/64). */
cce_status cce_backward(const float* dloss, int64_t dloss_stride, const void* E, const void* C,
                        const int64_t* targets, const float* lse, const float* tile_max,
                        int64_t N, int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                        float filter_eps, void* dE, void* dC, cce_dtype grad_dtype, void* ws,
                        size_t ws_bytes, int64_t* skip_stats, void* stream);

/* Mean-reduced convenience call: loss_mean = sum over non-ignored rows of loss / N_valid and
 * the gradients of that mean (dloss = 1 / N_valid for every row).  With N_valid == 0 the mean
 * and both gradients are 0.  loss_mean and n_valid (NULL allowed) are device scalars.
 *   dE, dC, grad_dtype as in cce_backward.
 *   ws: at least cce_loss_mean_workspace_bytes(); err_flag, skip_stats as above. */
cce_status cce_loss_mean(const void* E, const void* C, const int64_t* targets, int64_t N,
                         int64_t V, int64_t D, cce_dtype dtype, int64_t ignore_index,
                         float filter_eps, float* loss_mean, int64_t* n_valid, void* dE,
                         void* dC, cce_dtype grad_dtype, void* ws, size_t ws_bytes,
                         int32_t* err_flag, int64_t* skip_stats, void* stream);

/* Vocabulary-sharded form of the same computation (the tensor-parallel classifier head: each
 * device holds rows [vocab_offset, vocab_offset + V) of the full classifier, V_total rows in
 * all).  The log-sum-exp over the full vocabulary is the log-sum-exp of the shards' LSEs (the
 * abstract's on-the-fly log-sum-exp, sentence 5, split over devices), so a forward is one
 * cce_forward_shard per shard, an exchange of 2 floats per token and shard, and one
 * cce_merge_shards; the backward is one cce_backward_shard per shard with the merged LSE, each
 * giving its shard's rows of dC and a partial dE that the shards sum.
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
 * Workspace: cce_backward_workspace_bytes(N, V, D, dtype). */
cce_status cce_backward_shard(const float* dloss, int64_t dloss_stride, const void* E,
                              const void* C, const int64_t* targets, const float* lse,
                              const float* tile_max, int64_t N, int64_t V, int64_t D,
                              cce_dtype dtype, int64_t ignore_index, int64_t vocab_offset,
                              float filter_eps, void* dE, void* dC, cce_dtype grad_dtype,
                              void* ws, size_t ws_bytes, int64_t* skip_stats, void* stream);

/* Launch-shape introspection for reports (pure host): the vocabulary split count of the
 * forward and the vocabulary chunk width Vc of the backward for a problem. */
int64_t cce_forward_splits(int64_t N, int64_t V, int64_t D, cce_dtype dtype);
int64_t cce_backward_chunk(int64_t N, int64_t V, int64_t D, cce_dtype dtype);

/* Kernel kinds, for per-kernel timing. */
typedef enum {
  CCE_KERNEL_FWD_LSE = 0,     /* logit tiles + online log-sum-exp partials     (2 N V D flops)   */
  CCE_KERNEL_FWD_FINISH = 1,  /* partial merge, target gather-dot, loss                          */
  CCE_KERNEL_BWD_G = 2,       /* logit recompute, softmax - onehot, filter of the first chunk    */
  CCE_KERNEL_BWD_FUSED = 3,   /* per chunk c: dE += G C and dC = G^T E of chunk c (4 N Vc D)
                                 with the recompute of chunk c + 1                (2 N Vc' D)  */
  CCE_KERNEL_AUX = 4,         /* small helpers (statistics init, mean, zero fill)                */
  CCE_KERNEL_KINDS = 5
} cce_kernel_kind;

/* Benchmark timing hook (host only, not thread safe, process-wide).  cce_timing_begin starts
 * recording a HIP event pair around each of the next launches (at most max_launches) of every
 * kernel kind whose bit is set in kind_mask, on the stream the kernel is launched on.
 * cce_timing_end waits for the recorded events, writes the summed durations in milliseconds
 * and the launch counts per kind into ms[CCE_KERNEL_KINDS] and launches[CCE_KERNEL_KINDS]
 * (host arrays), releases the events and stops recording.  Returns CCE_ERR_HIP if an event
 * call fails, CCE_ERR_INVALID_ARGUMENT for max_launches < 1 or NULL outputs. */
cce_status cce_timing_begin(uint32_t kind_mask, int32_t max_launches);
cce_status cce_timing_end(float* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LIBCCE_CCE_H */

// Cut Cross-Entropy kernels for gfx950.
//
// Method: the Cut Cross-Entropy abstract (taxoreview.com page dblp:393/3562, sentences 4-6
// and 9).  Per token the loss is its LSE over the vocabulary less its target's logit, so the
// forward keeps each logit tile in registers, folds it into a running (max, sum) and gathers
// the one target logit separately; no N x V array is ever written.  The backward recomputes
// the logit tiles and leaves out the blocks of the softmax gradient that the filter proves
// negligible.
//
//   k_fwd_lse     S = C_tile E_tile^T on MFMA, online (max, sum exp) per token over the
//                 workgroup's vocabulary range, one partial per (range, token).
//   k_fwd_finish  merge of the partials (no atomics), target logit by gather-dot, loss; in
//                 shard mode the LSE over a shard of the vocabulary and the target logit.
//   k_merge_shards  merge of per-shard LSEs and target logits into loss and LSE.
//   k_bwd_g       recomputes S for a vocabulary chunk (tile_bwd_g), forms
//                 G = dloss (softmax - onehot) in registers, flags negligible 64 x 64 blocks,
//                 drops entries below the optional entry floor, stores the rest of G.
//   k_bwd_fused   per (vocabulary chunk, token block) pair: dE (+)= G C_chunk (tile_bwd_de)
//                 and dC_chunk (+)= G^T E_block (tile_bwd_dc), skipping flagged K stages,
//                 together with tile_bwd_g of the next pair.
//   k_f32_to_bf16, k_zero_f32, k_mean, k_skip_init  small helpers (bf16 gradient output,
//                 empty batches, the mean-reduced call, the skip statistics).
#pragma once

#include "tile_engine.hpp"

namespace cce {

// NST double-operand stage buffers as distinct LDS objects (unused ones shrink to 16 bytes).
#define CCE_STAGE_BUFFERS(KB, NST, B)                                                          \
  __shared__ __attribute__((aligned(1024))) char sA0_[Geo<KB>::kOpBytes];                     \
  __shared__ __attribute__((aligned(1024))) char sB0_[Geo<KB>::kOpBytes];                     \
  __shared__ __attribute__((aligned(1024))) char sA1_[Geo<KB>::kOpBytes];                     \
  __shared__ __attribute__((aligned(1024))) char sB1_[Geo<KB>::kOpBytes];                     \
  __shared__ __attribute__((aligned(1024))) char sA2_[(NST) > 2 ? Geo<KB>::kOpBytes : 16];    \
  __shared__ __attribute__((aligned(1024))) char sB2_[(NST) > 2 ? Geo<KB>::kOpBytes : 16];    \
  __shared__ __attribute__((aligned(1024))) char sA3_[(NST) > 3 ? Geo<KB>::kOpBytes : 16];    \
  __shared__ __attribute__((aligned(1024))) char sB3_[(NST) > 3 ? Geo<KB>::kOpBytes : 16];    \
  Bufs<NST> B;                                                                                  \
  {                                                                                             \
    char* const pa_[4] = {sA0_, sA1_, sA2_, sA3_};                                              \
    char* const pb_[4] = {sB0_, sB1_, sB2_, sB3_};                                              \
    _Pragma("unroll") for (int i_ = 0; i_ < (NST); ++i_) {                                      \
      B.a[i_] = pa_[i_];                                                                        \
      B.b[i_] = pb_[i_];                                                                        \
    }                                                                                           \
  }

// Stages of K for a contraction of length K, padded to a multiple of NST (padding stages
// load zeros).
template <typename T, int KB, int NST>
__host__ __device__ constexpr int padded_stages(int K) {
  constexpr int KS = KB / (int)sizeof(T);
  const int n = (K + KS - 1) / KS;
  return (n + NST - 1) / NST * NST;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

// ------------------------------------------------------------------------------------------
// Forward: per (token tile, vocabulary range) partial log-sum-exp in base 2.
//   part[split * N + n] = (m, s): m = max_v z*log2(e) over the range, s = sum 2^(z*log2(e) - m)
// Optionally (tile_max != nullptr) the largest z*log2(e) of each wave's 128 x 64 part of every
// 256 x 256 tile, tile_max[((token tile) * n_vt + vocabulary tile) * 8 + wave], for the backward
// to prove whole tiles negligible without recomputing them (tokens at or past N excluded).
// ------------------------------------------------------------------------------------------
// KT: D is not a multiple of NST stages of K, so the stages at the end of a row need the
// per-lane K mask (the common shapes compile without it).
template <typename T, int KB, int NST, bool KT>
__global__ __launch_bounds__(kThreads, 1) void k_fwd_lse(const T* __restrict__ E,
                                                         const T* __restrict__ C, int N, int V,
                                                         int D, int n_split, int n_vt,
                                                         int n_items, float2* __restrict__ part,
                                                         float* __restrict__ tile_max) {
  CCE_STAGE_BUFFERS(KB, NST, B)
  __shared__ float2 sRed[4][kWaveN];
  constexpr int KS = KB / (int)sizeof(T);
  constexpr int I = Geo<KB>::kIssue;

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= n_items) return;
  const int tb = item / n_split, sp = item % n_split;
  const int vt0 = (int)((int64_t)sp * n_vt / n_split);
  const int vt1 = (int)((int64_t)(sp + 1) * n_vt / n_split);
  const int n_k = padded_stages<T, KB, NST>(D);
  const int iters = (vt1 - vt0) * n_k;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave_m(wave), wn = wave_n(wave);
  const int tok0 = tb * kTile;

  float m_run[kNB], s_run[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }
  Acc acc;   // defined by the first stage of each vocabulary tile

  const int ldb = D * (int)sizeof(T);
  uint32_t off[I];  // C and E tiles share the row length, hence the offsets
  kmajor_offsets<KB>(off, ldb, wave, lane);
  // Classifier tile of the stages being issued: the current vocabulary tile (stages
  // [t_first, t_first + n_k) of the stream) or, for the look-ahead, the next one.
  int t_first = 0, v_cur = vt0 * kTile;
  const T* c_cur = C + (int64_t)v_cur * D;
  auto issue = [&](int it) {
    const bool live = it < iters;   // past the end of the stream: zeros
    const bool nx = it >= t_first + n_k;
    const int k0 = (it - t_first - (nx ? n_k : 0)) * KS;
    // valid K chunks from k0 (<= 0 on padding stages: all zeros)
    const int kc = KT ? (D - k0) / Traits<T>::kEpc : Geo<KB>::kChunks;
    const uint32_t soff = (uint32_t)k0 * sizeof(T);
    const Rsrc rsC = kmajor_rsrc(c_cur + (nx ? (int64_t)kTile * D : 0),
                                                   live ? V - v_cur - (nx ? kTile : 0) : 0, ldb);
    const Rsrc rsE =
        kmajor_rsrc(E + (int64_t)tok0 * D, live ? N - tok0 : 0, ldb);
    return stage_issue<KB>(
        [=, &off](char* l, int q0, int q1) { kmajor_issue<KB>(rsC, off, soff, kc, l, wave, lane, q0, q1); },
        [=, &off](char* l, int q0, int q1) { kmajor_issue<KB>(rsE, off, soff, kc, l, wave, lane, q0, q1); });
  };
  // Online log-sum-exp update for the finished tile, one token column group (ni) at a time.
  // Single pass against the running maximum m: t = z log2(e) - m, s += sum 2^t, with eight
  // independent partial sums and maxima so the VALU work pipelines; afterwards the pair is
  // rebased to the new maximum.  If some value exceeds the running maximum by more than 2^64
  // (always on the first tile, where m = -inf), the wave recomputes the group exactly.
  auto epilogue = [&](int vt) {
    if (vt * kTile + kTile > V) {
      // last vocabulary tile: rows at or past V take no part (-inf)
      const int lim = V - vt * kTile - kWaveM * wm - acc_row_l(lane);
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
        for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (acc_row_c(mi, r) >= lim) acc[mi][ni][r] = -INFINITY;
    }
    float zmax = -INFINITY;   // largest z log2(e) of the wave's valid token columns
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) {
      const float m = m_run[ni];
      const bool col_ok = tok0 + kWaveN * wn + 32 * ni + (lane & 31) < N;
      float ps[8], pm[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) { ps[k] = 0.f; pm[k] = -INFINITY; }
#pragma unroll
      for (int i = 0; i < 16 * kMB; ++i) {
        const float t = __builtin_fmaf(acc[i >> 4][ni][i & 15], kLog2e, -m);
        ps[i & 7] += exp2_fast(t);
        pm[i & 7] = fmaxf(pm[i & 7], t);
      }
      const float tmax = fmaxf(fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3])),
                               fmaxf(fmaxf(pm[4], pm[5]), fmaxf(pm[6], pm[7])));
      // exact path also while m = -inf (nothing seen yet: t would be -inf + inf for masked rows)
      if (__ballot(!(tmax <= 64.f) || m == -INFINITY) != 0ull) {
        // exact update (rare): new maximum first, then the sum against it
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16 * kMB; ++i) mx = fmaxf(mx, acc[i >> 4][ni][i & 15]);
        const float m_new = fmaxf(m, mx * kLog2e);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        if (col_ok) zmax = fmaxf(zmax, mx * kLog2e);
#pragma unroll
        for (int k = 0; k < 8; ++k) ps[k] = 0.f;
#pragma unroll
        for (int i = 0; i < 16 * kMB; ++i)
          ps[i & 7] += exp2_fast(__builtin_fmaf(acc[i >> 4][ni][i & 15], kLog2e, -m_use));
        const float tile = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
        s_run[ni] = s_run[ni] * exp2_fast(m - m_use) + tile;
        m_run[ni] = m_new;
      } else {
        const float tile = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
        const float up = fmaxf(tmax, 0.f);       // rebase so that s stays O(number of terms)
        s_run[ni] = (s_run[ni] + tile) * exp2_fast(-up);
        m_run[ni] = m + up;
        if (col_ok) zmax = fmaxf(zmax, tmax + m);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tile_max) {
      zmax = wave_max(zmax);
      if (lane == 0) tile_max[((int64_t)tb * n_vt + vt) * kWaves + wave] = zmax;
    }
  };

  const int n_tiles = vt1 - vt0;
  run_prologue<KB, NST>(iters, issue, B);
  for (int t = 0; t < n_tiles; ++t) {
    t_first = t * n_k;
    v_cur = (vt0 + t) * kTile;
    c_cur = C + (int64_t)v_cur * D;
    run_stream<T, KB, NST, true, true, true>(t * n_k, n_k, iters, issue, B, acc, wm, wn, lane);
    epilogue(vt0 + t);
  }

  // merge the two row halves of each column (lanes l and l ^ 32), then the two waves that
  // share columns (wm = 0, 1) through LDS
#pragma unroll
  for (int ni = 0; ni < kNB; ++ni) {
    const float mo = __shfl_xor(m_run[ni], 32);
    const float so = __shfl_xor(s_run[ni], 32);
    const float mn = fmaxf(m_run[ni], mo);
    const float mu = mn == -INFINITY ? 0.f : mn;
    s_run[ni] = s_run[ni] * exp2_fast(m_run[ni] - mu) + so * exp2_fast(mo - mu);
    m_run[ni] = mn;
  }
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) sRed[wn][32 * ni + lane] = make_float2(m_run[ni], s_run[ni]);
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) {
      const float2 o = sRed[wn][32 * ni + lane];
      const float mn = fmaxf(m_run[ni], o.x);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float s = s_run[ni] * exp2_fast(m_run[ni] - mu) + o.y * exp2_fast(o.x - mu);
      const int n = tok0 + kWaveN * wn + 32 * ni + lane;
      if (n < N) part[(int64_t)sp * N + n] = make_float2(mn, s);
    }
  }
}


// ------------------------------------------------------------------------------------------
// Forward finish: one wave per token.  LSE = ln2 * (M + log2 sum_i s_i 2^(m_i - M)); the
// target logit is a gather-dot of E[n] with C[t[n]] in fp32; loss = LSE - z_t.
// ------------------------------------------------------------------------------------------
constexpr int kFinishThreads = 256;   // 4 tokens per workgroup, one wave each

// Shard mode (zt != nullptr): C holds rows [voff, voff + V) of a larger vocabulary; the kernel
// writes the LSE over those rows and zt[n] = the target logit when the target falls in them
// (else 0), and no loss: the shards' results are merged by k_merge_shards.
template <typename T>
__global__ __launch_bounds__(kFinishThreads) void k_fwd_finish(
    const T* __restrict__ E, const T* __restrict__ C, const int64_t* __restrict__ tgt, int N,
    int V, int D, int n_split, const float2* __restrict__ part, int64_t ignore_index,
    float* __restrict__ loss, float* __restrict__ lse, int32_t* __restrict__ err, int64_t voff,
    float* __restrict__ zt) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  float m = -INFINITY;
  for (int s = lane; s < n_split; s += 64) m = fmaxf(m, part[(int64_t)s * N + n].x);
  m = wave_max(m);
  const float mu = m == -INFINITY ? 0.f : m;
  float sum = 0.f;
  for (int s = lane; s < n_split; s += 64) {
    const float2 p = part[(int64_t)s * N + n];
    sum += p.y * exp2_fast(p.x - mu);
  }
  sum = wave_sum(sum);
  const float l = (mu + log2f(sum)) * kLn2;
  const int64_t t = tgt[n];
  const bool ignored = t == ignore_index;
  const int64_t tl = t - voff;                     // row of the target within C
  const bool here = !ignored && tl >= 0 && tl < V;
  const bool bad = !ignored && !here && !zt;       // outside [0, V) is an error when unsharded
  float z = 0.f;
  if (here) {
    const T* e = E + (int64_t)n * D;
    const T* c = C + tl * (int64_t)D;
    for (int d = lane * 4; d < D; d += 256) {
#pragma unroll
      for (int i = 0; i < 4; ++i) z += (float)e[d + i] * (float)c[d + i];
    }
    z = wave_sum(z);
  }
  if (lane == 0) {
    lse[n] = l;
    if (zt) {
      zt[n] = here ? z : 0.f;
    } else {
      loss[n] = ignored ? 0.f : (bad ? __builtin_nanf("") : l - z);
      if (bad && err) *err = 1;
    }
  }
}

// Merge of S vocabulary shards (k_fwd_finish in shard mode): lse = log sum_s exp lse_s, the
// target logit is the one shard's contribution (the others wrote 0), loss = lse - z_t (0 for
// ignored rows; NaN and *err = 1 for a target outside [0, V_total)).  One thread per token.
__global__ void k_merge_shards(const float* __restrict__ lse_s, const float* __restrict__ zt_s,
                               int S, int N, const int64_t* __restrict__ tgt,
                               int64_t ignore_index, int64_t v_total, float* __restrict__ loss,
                               float* __restrict__ lse, int32_t* __restrict__ err) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, lse_s[(int64_t)s * N + n]);
  const float mu = m == -INFINITY ? 0.f : m;
  float sum = 0.f, z = 0.f;
  for (int s = 0; s < S; ++s) {
    sum += exp2_fast((lse_s[(int64_t)s * N + n] - mu) * kLog2e);
    z += zt_s[(int64_t)s * N + n];
  }
  const float l = mu + log2f(sum) * kLn2;
  const int64_t t = tgt[n];
  const bool ignored = t == ignore_index;
  const bool bad = !ignored && (t < 0 || t >= v_total);
  lse[n] = l;
  loss[n] = ignored ? 0.f : (bad ? __builtin_nanf("") : l - z);
  if (bad && err) *err = 1;
}

// ------------------------------------------------------------------------------------------
// Backward, step 1 for one vocabulary chunk [v0, v0 + vc): recompute the logit tile, form
// G = dloss (p - onehot) with p = 2^(z log2 e - lse log2 e), decide the 64 x 64 filter blocks
// and store G (chunk-local columns, row stride ldg) for the blocks that are kept.
//   flags[(n / 64) * fstride + v_local / 64] = 1 if the block is skipped (G not stored).
// ------------------------------------------------------------------------------------------
// Arguments of the backward steps for one pair of a token block and a vocabulary chunk
// [v0, v0 + vc).  The token-indexed pointers (E, tgt, lse, dloss, dE, tile_max, tile_lse_min)
// start at the block's first token, so N and n_pad are the block's token counts.
template <typename T>
struct BwdArgs {
  const T* E;                 // [N, D]
  const T* C;                 // [V, D]
  const int64_t* tgt;         // [N]
  const float* lse;           // [N]
  const float* dloss;         // [N] or scalar (dstride 0)
  int64_t dstride;
  int N, V, D, n_pad;         // n_pad: N rounded up to the tile
  int v0, vc;                 // chunk origin and width
  int n_tb, n_vtc, n_dt;      // token tiles, chunk vocabulary tiles, hidden-dimension tiles
  T* G;                       // [n_pad, ldg] softmax-gradient store of the chunk
  int64_t ldg;
  uint8_t* flags;             // [n_pad / 64, fstride] skipped 64 x 64 blocks of the chunk
  int fstride;
  float eps;
  float p_floor;              // entry floor: non-target p below it are dropped (0: off)
  int64_t ignore_index;
  int64_t voff;               // vocabulary index of C's row 0 (a shard of a larger vocabulary)
  unsigned long long* skip_count;
  float* dE;                  // [N, D] fp32 running sum of dE over the chunks
  int accumulate;             // dE += (later chunks) instead of dE = (first chunk)
  const float* dc_in;         // [vc, D] fp32 running sum of the chunk's dC over the token
                              // blocks so far, or nullptr (first block: start from 0)
  void* dc_out;               // [vc, D] where the chunk's dC (so far) goes
  int dc_bf16;                // dc_out is bf16 (the last block of bf16 gradients), else fp32
  const float* tile_max;      // the forward's tile maxima (k_fwd_lse); readable when unused
  const float* tile_lse_min;  // [n_tb] smallest lse log2(e) of each token tile (k_tile_lse_min)
  int tile_skip;              // 1: skip tiles that tile_max proves negligible
  int n_vt_all;               // vocabulary tiles of C (index of tile_max)
  float skip_bound;           // log2(eps) less a margin: tiles below it are not recomputed
};

template <typename T, int KB, int NST, bool KT>
__device__ __forceinline__ void tile_bwd_g(const BwdArgs<T>& A, int lin, const Bufs<NST>& B) {
  const T* __restrict__ E = A.E;
  const T* __restrict__ C = A.C;
  const int64_t* __restrict__ tgt = A.tgt;
  const float* __restrict__ lse = A.lse;
  const float* __restrict__ dloss = A.dloss;
  const int64_t dstride = A.dstride;
  const int N = A.N, D = A.D, v0 = A.v0, vc = A.vc, n_tb = A.n_tb, n_vtc = A.n_vtc;
  T* __restrict__ G = A.G;
  const int64_t ldg = A.ldg;
  uint8_t* __restrict__ flags = A.flags;
  const int fstride = A.fstride;
  const float eps = A.eps;
  const int64_t ignore_index = A.ignore_index;
  unsigned long long* __restrict__ skip_count = A.skip_count;
  constexpr int KS = KB / (int)sizeof(T);
  constexpr int I = Geo<KB>::kIssue;

  int tb, vt;
  grouped_tile(lin, n_tb, n_vtc, tb, vt);
  if (tb >= n_tb || vt >= n_vtc) return;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave_m(wave), wn = wave_n(wave);
  const int tok0 = tb * kTile, vl0 = vt * kTile;  // vl0: chunk-local first vocab row
  const int n_k = padded_stages<T, KB, NST>(D);
  const T* Cc = C + (int64_t)v0 * D;

  Acc acc;
  zero_acc(acc);
  const int ldb = D * (int)sizeof(T);
  uint32_t off[I];
  kmajor_offsets<KB>(off, ldb, wave, lane);
  auto issue = [&](int it) {
    const bool live = it < n_k;   // past the end of the stream: zeros
    const Rsrc rsC = kmajor_rsrc(Cc + (int64_t)vl0 * D, live ? vc - vl0 : 0, ldb);
    const Rsrc rsE = kmajor_rsrc(E + (int64_t)tok0 * D, live ? N - tok0 : 0, ldb);
    const int k0 = it * KS;
    const int kc = KT ? (D - k0) / Traits<T>::kEpc : Geo<KB>::kChunks;
    const uint32_t soff = (uint32_t)k0 * sizeof(T);
    return stage_issue<KB>(
        [=, &off](char* l, int q0, int q1) { kmajor_issue<KB>(rsC, off, soff, kc, l, wave, lane, q0, q1); },
        [=, &off](char* l, int q0, int q1) { kmajor_issue<KB>(rsE, off, soff, kc, l, wave, lane, q0, q1); });
  };
  // per column (token) constants, loaded before the main loop so their latency is hidden
  float coef[kNB], lse2[kNB];
  int trow[kNB];
  bool valid[kNB];
#pragma unroll
  for (int ni = 0; ni < kNB; ++ni) {
    const int n = tok0 + kWaveN * wn + 32 * ni + (lane & 31);
    bool ok = false;
    float w = 0.f, l2 = 0.f;
    int tr = -1;
    if (n < N) {
      const int64_t t = tgt[n];
      ok = t != ignore_index;
      w = dloss[(int64_t)n * dstride];
      l2 = lse[n] * kLog2e;
      // target row within the wave's rows
      const int64_t tl = t - A.voff - (int64_t)v0 - vl0 - kWaveM * wm;
      tr = (ok && tl >= 0 && tl < 128) ? (int)tl : -1;
    }
    valid[ni] = ok;
    coef[ni] = ok ? w : 0.f;
    lse2[ni] = l2;
    trow[ni] = tr;
  }

  // With the forward's tile maxima: if max z log2(e) over the tile, less the smallest
  // lse log2(e) of its non-ignored tokens, is below log2(eps) (by a margin that covers the
  // rounding of both sides), every p of the tile is below eps, and if no token of the tile has
  // its target among the tile's rows, every block of it is negligible.  The recompute is then
  // skipped and the blocks are flagged as the epilogue would flag them.  The two bounds are
  // read through the constant address space (scalar loads, counted apart from the stage
  // loads), so their latency overlaps the first stage's.
  // The loads are unconditional (without maxima both pointers lead to 256 readable bytes and
  // the offsets are 0), so no branch makes the compiler wait for them before the stage loads.
  typedef const __attribute__((address_space(4))) float* cfloat_p;
  const int on = A.tile_skip;
  const cfloat_p tm =
      (cfloat_p)A.tile_max + ((int64_t)tb * A.n_vt_all + ((v0 + vl0) >> 8)) * kWaves * on;
  float tmv[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tmv[w] = tm[w];
  const float lmin = ((cfloat_p)A.tile_lse_min)[tb * on];
  run_prologue<KB, NST>(n_k, issue, B);
  float zt = -INFINITY;   // taken after the stage loads are issued, so they wait for nothing
#pragma unroll
  for (int w = 0; w < kWaves; ++w) zt = fmaxf(zt, tmv[w]);
  if (on && zt - lmin < A.skip_bound) {
    // every p of the tile is below eps; skip it unless a token's target lies in its rows
    __shared__ int sHasTarget[kWaves];
    bool here = false;
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) here |= trow[ni] >= 0;
    const bool any_t = __ballot(here) != 0ull;
    if (lane == 0) sHasTarget[wave] = any_t ? 1 : 0;
    __syncthreads();
    int has_t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) has_t |= sHasTarget[w];
    if (!has_t) {
      wait_vmcnt<0>();   // the first stage's loads land before the workgroup ends
      const int nblk = tok0 + kWaveN * wn;
      int n_skipped = 0;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int vblk = vl0 + kWaveM * wm + 64 * a;
        if (vblk < vc && nblk < N) ++n_skipped;
        if (lane == 0) flags[(int64_t)(nblk >> 6) * fstride + (vblk >> 6)] = 1;
      }
      if (skip_count && lane == 0 && n_skipped)
        atomicAdd(skip_count, (unsigned long long)n_skipped);
      return;
    }
  }
  run_stream<T, KB, NST, true, true>(0, n_k, n_k, issue, B, acc, wm, wn, lane);

  // epilogue: p = 2^(z log2 e - lse log2 e); G = coef (p - [row == target]); per lane and
  // 64 x 64 block the largest p (independent maxima, no serial chains).  With the optional
  // entry floor (the caller's p_floor > 0), non-target entries with p < p_floor are dropped
  // from G; the target entry never is.  p_floor = 0 drops nothing (p < 0 never holds).
  const bool filter = eps > 0.f;
  const float p_floor = A.p_floor;
  const bool full = vl0 + kTile <= vc;
  if (!full) {
    // last tile of the chunk: rows at or past vc get p = 0
    const int lim = vc - vl0 - kWaveM * wm - acc_row_l(lane);
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
      for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row_c(mi, r) >= lim) acc[mi][ni][r] = -INFINITY;
  }
  // rows (within the wave's 128) are acc_row_c(mi, r) + acc_row_l(lane): compare the constant
  // part with a per-lane value
  int tcmp[kNB];
#pragma unroll
  for (int ni = 0; ni < kNB; ++ni) tcmp[ni] = trow[ni] - acc_row_l(lane);

  // The wave's 64 token columns are one filter block wide and its 128 vocabulary rows two
  // blocks (a = 0, 1: register blocks mi = 2a, 2a + 1).  Each block is finished in turn --
  // G, the wave-wide keep decision, its flag -- then its values go out.
  //
  // bf16 G goes out through LDS: a lane's registers hold 4 consecutive vocabulary entries of
  // one token (8 bytes), and the 64 lanes of a store would touch 64 token rows of G.  Each wave
  // instead writes its 128 x 64 block, token-major, into its own 16 KB of the (now idle) stage
  // buffers, then stores 16 bytes per lane, 256 contiguous bytes per token.  The 16-byte chunk c
  // of token row n sits at chunk c ^ (n % 16), which keeps both LDS passes free of bank
  // conflicts.
  constexpr bool kStaged = sizeof(T) == 2 && 2 * NST * Geo<KB>::kOpBytes >= kWaves * 16384;
  int n_skipped = 0;
  const int nblk = tok0 + kWaveN * wn;          // token start of the wave's block
  bool kept[2] = {false, false};
  lds_char_t* stg = nullptr;                    // this wave's 16 KB of LDS
  if constexpr (kStaged) {
    constexpr int kPer = Geo<KB>::kOpBytes / 16384;   // waves per operand buffer
    const int buf = wave / kPer;
    // LDS addresses of the operand buffers, chosen as integers (a choice between the generic
    // pointers would hide from the compiler that the pipeline's reads are LDS reads)
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const uint32_t la = (uint32_t)(uintptr_t)(lds_char_t*)B.a[i];
      const uint32_t lb = (uint32_t)(uintptr_t)(lds_char_t*)B.b[i];
      base = buf == 2 * i ? la : buf == 2 * i + 1 ? lb : base;
    }
    stg = (lds_char_t*)(uintptr_t)(base + (wave % kPer) * 16384);
    stage_barrier();   // every wave has read its last stage (each waited for its own loads)
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float pmax[kNB];
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) pmax[ni] = 0.f;
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) {
      // the one-hot term only where some column of the wave has its target in this block
      // (a uniform branch; fma with a zero addend rounds like the general form)
      const bool any_t = __ballot(trow[ni] >= 64 * a && trow[ni] < 64 * a + 64) != 0ull;
      if (any_t) {
#pragma unroll
        for (int mi = 2 * a; mi < 2 * a + 2; ++mi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(__builtin_fmaf(acc[mi][ni][r], kLog2e, -lse2[ni]));
            pmax[ni] = fmaxf(pmax[ni], p);
            const bool is_t = acc_row_c(mi, r) == tcmp[ni];
            acc[mi][ni][r] =
                __builtin_fmaf(coef[ni], p < p_floor && !is_t ? 0.f : p, is_t ? -coef[ni] : 0.f);
          }
      } else {
#pragma unroll
        for (int mi = 2 * a; mi < 2 * a + 2; ++mi)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(__builtin_fmaf(acc[mi][ni][r], kLog2e, -lse2[ni]));
            pmax[ni] = fmaxf(pmax[ni], p);
            acc[mi][ni][r] = __builtin_fmaf(coef[ni], p < p_floor ? 0.f : p, 0.f);
          }
      }
    }
    bool sig = false;
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) {
      const bool has_t = trow[ni] >= 64 * a && trow[ni] < 64 * a + 64;
      sig |= valid[ni] && (pmax[ni] >= eps || has_t);
    }
    // block decision (wave-wide), flag, statistics
    const int vblk = vl0 + kWaveM * wm + 64 * a;  // chunk-local vocab start of the block
    const bool in_range = vblk < vc && nblk < N;
    const bool keep = in_range && (!filter || __ballot(sig) != 0ull);
    if (in_range && !keep) ++n_skipped;
    if (lane == 0) flags[(int64_t)(nblk >> 6) * fstride + (vblk >> 6)] = keep ? 0 : 1;
    kept[a] = keep;
    if (!keep) continue;
    if constexpr (kStaged) {
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
#pragma unroll
      for (int mi = 2 * a; mi < 2 * a + 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNB; ++ni) {
          const int nl = 32 * ni + (lane & 31);
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int c = 4 * mi + rq;   // vocabulary entries 8c .. 8c + 7 of the wave's rows
            bf16x4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (__bf16)acc[mi][ni][4 * rq + i];
            *(__attribute__((address_space(3))) bf16x4_t*)(stg + nl * 256 + ((c ^ (nl & 15)) << 4) +
                                                           8 * (lane >> 5)) = v;
          }
        }
      continue;
    }
    // store: 4 consecutive vocab rows of one token per lane and register group
#pragma unroll
    for (int mi = 2 * a; mi < 2 * a + 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni) {
        const int n = tok0 + kWaveN * wn + 32 * ni + (lane & 31);
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int vloc = vl0 + kWaveM * wm + 32 * mi + 8 * rq + 4 * (lane >> 5);
          T* dst = G + (int64_t)n * ldg + vloc;
          if constexpr (sizeof(T) == 2) {
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
            bf16x4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (__bf16)acc[mi][ni][4 * rq + i];
            *(bf16x4_t*)dst = v;
          } else {
            f32x4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[mi][ni][4 * rq + i];
            *(f32x4_t*)dst = v;
          }
        }
      }
  }
  if constexpr (kStaged) {
    // 4 tokens per store, 16 lanes per token row (256 bytes); chunks 0..7 belong to block 0
    const int c = lane & 15;
    const bool mine = c < 8 ? kept[0] : kept[1];
    if (kept[0] || kept[1]) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int nl = 4 * i + (lane >> 4);
        const bf16x8_t v =
            *(const __attribute__((address_space(3))) bf16x8_t*)(stg + nl * 256 + ((c ^ (nl & 15)) << 4));
        if (mine)   // streamed out: the next launch reads it, this one never does
          __builtin_nontemporal_store(
              v, (bf16x8_t*)(G + (int64_t)(nblk + nl) * ldg + vl0 + kWaveM * wm + 8 * c));
      }
    }
  }
  if (skip_count && lane == 0 && n_skipped) atomicAdd(skip_count, (unsigned long long)n_skipped);
}

// Writes this wave's 128 x 64 accumulators to a row-major bf16 matrix out[rows][ld] at
// (row0, col0), rounding to nearest even; rows >= row_lim and columns >= col_lim are dropped.
__device__ __forceinline__ void store_tile_bf16(__bf16* __restrict__ out, int64_t ld, int row0,
                                                int row_lim, int col0, int col_lim, Acc& acc,
                                                int lane) {
  const bool full = row0 + kWaveM <= row_lim && col0 + kWaveN <= col_lim;
#pragma unroll
  for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + 32 * mi + acc_row(r, lane), col = col0 + 32 * ni + (lane & 31);
        if (full || (row < row_lim && col < col_lim))
          out[(int64_t)row * ld + col] = (__bf16)acc[mi][ni][r];
      }
}

// acc = in[rows, cols] of the wave's 128 x 64 part of a row-major fp32 matrix (zero outside the
// limits): the running sum of a tile that this workgroup alone updates in the launch.
__device__ __forceinline__ void load_tile(const float* __restrict__ in, int64_t ld, int row0,
                                          int row_lim, int col0, int col_lim, Acc& acc,
                                          int lane) {
  if (row0 + kWaveM <= row_lim && col0 + kWaveN <= col_lim) {
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[mi][ni][r] =
              in[(int64_t)(row0 + 32 * mi + acc_row(r, lane)) * ld + col0 + 32 * ni + (lane & 31)];
  } else {
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * mi + acc_row(r, lane), col = col0 + 32 * ni + (lane & 31);
          acc[mi][ni][r] =
              (row < row_lim && col < col_lim) ? in[(int64_t)row * ld + col] : 0.f;
        }
  }
}

// Writes this wave's 128 x 64 accumulators to a row-major fp32 matrix out[rows][ld] at
// (row0, col0); rows >= row_lim and columns >= col_lim are dropped.  For each register a
// half-wave writes 32 consecutive columns (128 bytes).  The stores are non-temporal: a tile's
// result is read again by a later launch at the earliest, so it should not displace the
// operand lines the running tiles share in the L2.
__device__ __forceinline__ void store_tile(float* __restrict__ out, int64_t ld, int row0,
                                           int row_lim, int col0, int col_lim, const Acc& acc,
                                           int lane) {
  if (row0 + kWaveM <= row_lim && col0 + kWaveN <= col_lim) {
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_nontemporal_store(
              acc[mi][ni][r],
              &out[(int64_t)(row0 + 32 * mi + acc_row(r, lane)) * ld + col0 + 32 * ni + (lane & 31)]);
  } else {
#pragma unroll
    for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNB; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * mi + acc_row(r, lane), col = col0 + 32 * ni + (lane & 31);
          if (row < row_lim && col < col_lim)
            __builtin_nontemporal_store(acc[mi][ni][r], &out[(int64_t)row * ld + col]);
        }
  }
}

// Builds the list of K stages of a backward product that are not entirely skipped.  Entry =
// (stage << 4) | mask, mask bit b set = the b-th 64-wide block of the tile's rows/columns is
// skipped within the stage (its operand chunk is loaded as zeros).
//   rowwise: flags of stage s are flags[(fr0 + b) * fstride + s * KS / 64]   (dE: K = vocab)
//   else   : flags of stage s are flags[(s * KS / 64) * fstride + fc0 + b]   (dC: K = tokens)
// The list comes in three segments, each in stage order and padded to a multiple of NST with
// all-zero stages (mask 15): stages whose live blocks are all in rows 0..127 (blocks 0, 1),
// then stages with live blocks in both 128-row halves of the tile, then stages whose live
// blocks are all in rows 128..255.  seg[k] = padded length of segment k.  wave_cnt: 6 x kWaves
// ints of LDS.
template <int KS, int NST>
__device__ __forceinline__ void build_stage_list(const uint8_t* __restrict__ flags, int fstride,
                                                 int n_stages, bool rowwise, int fixed0,
                                                 int* list, int* wave_cnt, int (&seg)[3]) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  // segment of stage s: 0 only rows 0..127 live, 1 both halves, 2 only rows 128..255, -1 none
  auto classify = [&](int s, uint32_t& mask) -> int {
    mask = 15u;
    if (s >= n_stages) return -1;
    const int fk = (s * KS) >> 6;
    mask = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint8_t f = rowwise ? flags[(int64_t)(fixed0 + b) * fstride + fk]
                                : flags[(int64_t)fk * fstride + fixed0 + b];
      mask |= (f ? 1u : 0u) << b;
    }
    const bool lo = (mask & 3u) != 3u, hi = (mask >> 2) != 3u;
    return lo && hi ? 1 : lo ? 0 : hi ? 2 : -1;
  };
  const unsigned long long below = (1ull << lane) - 1ull;
  // stages [0, kThreads): one per thread, classified once; later stages only counted here
  uint32_t mask0;
  const int k0 = classify(threadIdx.x, mask0);
  int rest[3] = {0, 0, 0};
  for (int base = kThreads; base < n_stages; base += kThreads) {
    uint32_t mask;
    const int k = classify(base + threadIdx.x, mask);
#pragma unroll
    for (int j = 0; j < 3; ++j) rest[j] += __popcll(__ballot(k == j));
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int c = __popcll(__ballot(k0 == j));
    if (lane == 0) {
      wave_cnt[j * kWaves + wave] = c;
      wave_cnt[(3 + j) * kWaves + wave] = rest[j];
    }
  }
  __syncthreads();
  // segment j starts at `start`; its first-step entries go first, in wave order, then its later
  // entries from pos[j]; pads fill its end
  int pos[3], start = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    int n0 = 0, nb = 0, nr = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = wave_cnt[j * kWaves + w];
      n0 += c;
      nb += w < wave ? c : 0;
      nr += wave_cnt[(3 + j) * kWaves + w];
    }
    const unsigned long long bal = __ballot(k0 == j);
    if (k0 == j) list[start + nb + __popcll(bal & below)] = ((int)threadIdx.x << 4) | (int)mask0;
    seg[j] = (n0 + nr + NST - 1) / NST * NST;
    // pads: all-zero stages (every block masked), so the pipeline runs whole rounds
    if (threadIdx.x == 0)
      for (int i = start + n0 + nr; i < start + seg[j]; ++i) list[i] = 15;
    pos[j] = start + n0;
    start += seg[j];
  }
  // later stages: each after the earlier ones of its segment
  for (int base = kThreads; base < n_stages; base += kThreads) {
    uint32_t mask;
    const int k = classify(base + threadIdx.x, mask);
    __syncthreads();   // the counts of the previous step have been read
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int c = __popcll(__ballot(k == j));
      if (lane == 0) wave_cnt[j * kWaves + wave] = c;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      int off = pos[j], sum = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int c = wave_cnt[j * kWaves + w];
        off += w < wave ? c : 0;
        sum += c;
      }
      const unsigned long long bal = __ballot(k == j);
      if (k == j) list[off + __popcll(bal & below)] = ((base + (int)threadIdx.x) << 4) | (int)mask;
      pos[j] += sum;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------
// Backward, step 2: dE[tok tile, d tile] (+)= sum over the chunk's vocabulary of
// G[tok, v] C[v0 + v, d].  A = G (K-major, K = vocab), B = C chunk (MN-major).
// ------------------------------------------------------------------------------------------
template <typename T, int KB, int NST>
__device__ __forceinline__ void tile_bwd_de(const BwdArgs<T>& A, int lin, const Bufs<NST>& B,
                                            int* sList, int* sCnt) {
  constexpr int KS = KB / (int)sizeof(T);
  constexpr int I = Geo<KB>::kIssue;
  const T* __restrict__ G = A.G;
  const int64_t ldg = A.ldg;
  const T* __restrict__ Cc = A.C + (int64_t)A.v0 * A.D;
  const int D = A.D, N = A.N, vc = A.vc, n_tb = A.n_tb, n_dt = A.n_dt;
  const int kv = (vc + KS - 1) / KS * KS;
  const uint8_t* __restrict__ flags = A.flags;
  const int fstride = A.fstride;
  float* __restrict__ dE = A.dE;
  const int accumulate = A.accumulate;
  int tb, dt;
  grouped_tile(lin, n_tb, n_dt, tb, dt);
  if (tb >= n_tb || dt >= n_dt) return;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave_m(wave), wn = wave_n(wave);
  const int tok0 = tb * kTile, d0 = dt * kTile;
  const int n_stages = kv / KS;
  int seg[3];
  build_stage_list<KS, NST>(flags, fstride, n_stages, true, tb * 4, sList, sCnt, seg);
  const int n_act = seg[0] + seg[1] + seg[2];

  // dE of this tile accumulates over the chunks: the running sum is read into the
  // accumulators up front (its latency overlaps the pipeline's first loads) and written back
  // with plain stores; one workgroup per tile and launch, launches in stream order
  if (n_act == 0 && accumulate) return;
  Acc acc;
  if (accumulate)
    load_tile(dE, D, tok0 + kWaveM * wm, N, d0 + kWaveN * wn, D, acc, lane);
  else
    zero_acc(acc);
  const int ldb = D * (int)sizeof(T);
  uint32_t offA[I], offB[I];
  kmajor_offsets<KB>(offA, (int)ldg * (int)sizeof(T), wave, lane);
  mn_offsets<T, KB>(offB, ldb, d0, D, wave, lane);
  const T* gt = G + (int64_t)tok0 * ldg;
  const int g_rec = kTile * (int)ldg * (int)sizeof(T);
  // issue(i) is called once per i, in order: each call reads the list entry of the next one,
  // so no call waits for an LDS read (the empty asm keeps the compiler from working on the
  // next entry as soon as it arrives, which would wait for the LDS reads issued since)
  int next_e = sList[0];
  auto issue = [&](int i) {
    const bool live = i < n_act;   // past the end of the list: zeros
    asm volatile("" : "+v"(next_e));
    const int e = __builtin_amdgcn_readfirstlane(next_e);
    next_e = sList[i + 1 < n_act ? i + 1 : 0];
    const int k0 = (e >> 4) * KS;
    const bool zero = (e >> (wave >> 1)) & 1;  // wave w loads token rows 32 w .. 32 w + 31
    const Rsrc ra = make_rsrc(gt, (zero || !live) ? 0 : g_rec);
    const Rsrc rb = mn_rsrc<T, KB>(Cc + (int64_t)k0 * D + d0,
                                                     live ? vc - k0 : 0, ldb, d0 * (int)sizeof(T));
    const uint32_t soff = (uint32_t)k0 * sizeof(T);
    return stage_issue<KB>(
        [=, &offA](char* l, int q0, int q1) {
          kmajor_issue<KB>(ra, offA, soff, Geo<KB>::kChunks, l, wave, lane, q0, q1);
        },
        [=, &offB](char* l, int q0, int q1) { mn_issue<T, KB>(rb, offB, 0u, l, wave, lane, q0, q1); });
  };
  run_segments<T, KB, NST, true, false>(seg, issue, B, acc, wm, wn, lane);
  store_tile(dE, D, tok0 + kWaveM * wm, N, d0 + kWaveN * wn, D, acc, lane);
}

// ------------------------------------------------------------------------------------------
// Backward, step 3: dC[v0 + v, d] = sum over tokens of G[tok, v] E[tok, d] for the chunk.
// A = G (MN-major, K = tokens), B = E (MN-major).
// ------------------------------------------------------------------------------------------
constexpr int kDcPiece = 1024;   // token stages handled per stage list of the dC product

template <typename T, int KB, int NST>
__device__ __forceinline__ void tile_bwd_dc(const BwdArgs<T>& A, int lin, const Bufs<NST>& B,
                                            int* sList, int* sCnt) {
  constexpr int KS = KB / (int)sizeof(T);
  constexpr int I = Geo<KB>::kIssue;
  constexpr int kPiece = kDcPiece;
  const T* __restrict__ G = A.G;
  const int64_t ldg = A.ldg;
  const T* __restrict__ E = A.E;
  const int D = A.D, N = A.N, n_pad = A.n_pad, vc = A.vc, n_vtc = A.n_vtc, n_dt = A.n_dt;
  const uint8_t* __restrict__ flags = A.flags;
  const int fstride = A.fstride;
  int vt, dt;
  grouped_tile(lin, n_vtc, n_dt, vt, dt);
  if (vt >= n_vtc || dt >= n_dt) return;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave_m(wave), wn = wave_n(wave);
  const int vl0 = vt * kTile, d0 = dt * kTile;
  const int n_stages = n_pad / KS;
  const int ldb = D * (int)sizeof(T);
  const int ldgb = (int)ldg * (int)sizeof(T);
  uint32_t offA[I], offB[I];
  mn_offsets<T, KB>(offA, ldgb, vl0, (int)ldg, wave, lane);
  mn_offsets<T, KB>(offB, ldb, d0, D, wave, lane);
  // dC of the chunk accumulates over the token blocks: the running sum (dc_in, fp32) is read
  // into the accumulators up front, like dE's; the first block starts from zero
  Acc acc;
  if (A.dc_in)
    load_tile(A.dc_in, D, vl0 + kWaveM * wm, vc, d0 + kWaveN * wn, D, acc, lane);
  else
    zero_acc(acc);
  bool live_any = false;
  for (int sbase = 0; sbase < n_stages; sbase += kPiece) {
    const int cnt = min(kPiece, n_stages - sbase);
    int seg[3];
    build_stage_list<KS, NST>(flags + (int64_t)((sbase * KS) >> 6) * fstride, fstride, cnt,
                              false, vt * 4, sList, sCnt, seg);
    const int n_act = seg[0] + seg[1] + seg[2];
    live_any |= n_act > 0;
    int next_e = sList[0];   // list entry of the next issue() call (calls come in order)
    auto issue = [&](int i) {
      const bool live = i < n_act;   // past the end of the list: zeros
      asm volatile("" : "+v"(next_e));
      const int e = __builtin_amdgcn_readfirstlane(next_e);
      next_e = sList[i + 1 < n_act ? i + 1 : 0];
      const int k0 = (sbase + (e >> 4)) * KS;
      const uint32_t zc = (uint32_t)(e & 15);
      const Rsrc ra = mn_rsrc<T, KB>(
          G + (int64_t)k0 * ldg + vl0, live ? n_pad - k0 : 0, ldgb, vl0 * (int)sizeof(T));
      const Rsrc rb = mn_rsrc<T, KB>(E + (int64_t)k0 * D + d0,
                                                       live ? N - k0 : 0, ldb, d0 * (int)sizeof(T));
      return stage_issue<KB>(
          [=, &offA](char* l, int q0, int q1) { mn_issue<T, KB>(ra, offA, zc, l, wave, lane, q0, q1); },
          [=, &offB](char* l, int q0, int q1) { mn_issue<T, KB>(rb, offB, 0u, l, wave, lane, q0, q1); });
    };
    run_segments<T, KB, NST, false, false>(seg, issue, B, acc, wm, wn, lane);
    __syncthreads();
  }
  // nothing added and the running sum stays where it is: no store needed
  if (!live_any && (const void*)A.dc_in == A.dc_out) return;
  if (A.dc_bf16)
    store_tile_bf16((__bf16*)A.dc_out, D, vl0 + kWaveM * wm, vc, d0 + kWaveN * wn, D, acc, lane);
  else
    store_tile((float*)A.dc_out, D, vl0 + kWaveM * wm, vc, d0 + kWaveN * wn, D, acc, lane);
}

// Work items of the backward launches: one per tile (grouped_tile).
__host__ __device__ inline int bwd_items(int rows, int cols) { return rows * cols; }

// Backward step 1 alone (the first chunk): one G tile per workgroup.
template <typename T, int KB, int NST, bool KT>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_g(BwdArgs<T> A) {
  CCE_STAGE_BUFFERS(KB, NST, B)
  tile_bwd_g<T, KB, NST, KT>(A, xcd_remap(blockIdx.x, gridDim.x), B);
}

// Backward steps 2 and 3 of chunk c (dE and dC tiles, the long ones) fused with step 1 of
// chunk c + 1 (G tiles of the next chunk into the other G buffer, the short ones), so the
// short tiles fill the CUs that the 2 x (N/256) x (D/256) long tiles leave idle.  Workgroups
// [0, r_de) compute dE tiles, [r_de, r_de + r_dc) dC tiles, the rest G tiles of `next`
// (none when n_next_items == 0).  Each range is a multiple of 8 and renumbered per XCD.
template <typename T, int KB, int NST, bool KT>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_fused(BwdArgs<T> A, BwdArgs<T> next,
                                                           int r_de, int r_dc) {
  CCE_STAGE_BUFFERS(KB, NST, B)
  __shared__ int sList[kDcPiece + 3 * NST];
  __shared__ int sCnt[6 * kWaves];
  const int b = blockIdx.x;
  if (b < r_de) {
    tile_bwd_de<T, KB, NST>(A, xcd_remap(b, r_de), B, sList, sCnt);
  } else if (b < r_de + r_dc) {
    tile_bwd_dc<T, KB, NST>(A, xcd_remap(b - r_de, r_dc), B, sList, sCnt);
  } else {
    const int n = (int)gridDim.x - r_de - r_dc;
    tile_bwd_g<T, KB, NST, KT>(next, xcd_remap(b - r_de - r_dc, n), B);
  }
}

// Smallest lse log2(e) over the non-ignored tokens of each 256-token tile (+inf if none): the
// token side of the backward's bound for skipping tiles.  One workgroup per token tile.
__global__ __launch_bounds__(256) void k_tile_lse_min(const float* __restrict__ lse,
                                                      const int64_t* __restrict__ tgt, int N,
                                                      int64_t ignore_index,
                                                      float* __restrict__ out) {
  __shared__ float s[4];
  const int n = blockIdx.x * 256 + threadIdx.x;
  float v = INFINITY;
  if (n < N && tgt[n] != ignore_index) v = lse[n] * kLog2e;
  v = wave_min(v);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = fminf(fminf(s[0], s[1]), fminf(s[2], s[3]));
}

// p[0..n) = 0 (a kernel rather than a memset, so the call stays safe under graph capture)
__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// out[i] = bf16(in[i]) (round to nearest even), 4 elements per thread and step (n % 4 == 0).
__global__ void k_f32_to_bf16(const float* __restrict__ in, __bf16* __restrict__ out, int64_t n) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n;
       i += (int64_t)gridDim.x * blockDim.x * 4) {
    const f32x4_t v = *(const f32x4_t*)(in + i);
    bf16x4_t o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (__bf16)v[k];
    *(bf16x4_t*)(out + i) = o;
  }
}

// skip_stats = {0, total}
__global__ void k_skip_init(int64_t* __restrict__ stats, int64_t total) {
  if (threadIdx.x == 0) {
    stats[0] = 0;
    stats[1] = total;
  }
}

// Mean over non-ignored rows; writes loss_mean, the per-row upstream gradient 1 / N_valid
// (0 when N_valid == 0) and N_valid.  One workgroup, fixed reduction order.
__global__ __launch_bounds__(1024) void k_mean(const float* __restrict__ loss,
                                               const int64_t* __restrict__ tgt, int N,
                                               int64_t ignore_index, float* __restrict__ mean,
                                               float* __restrict__ dloss_out,
                                               int64_t* __restrict__ n_valid_out) {
  __shared__ double sSum[1024];
  __shared__ long long sCnt[1024];
  double s = 0.0;
  long long c = 0;
  for (int n = threadIdx.x; n < N; n += 1024) {
    if (tgt[n] != ignore_index) {
      s += (double)loss[n];
      ++c;
    }
  }
  sSum[threadIdx.x] = s;
  sCnt[threadIdx.x] = c;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      sSum[threadIdx.x] += sSum[threadIdx.x + o];
      sCnt[threadIdx.x] += sCnt[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long cnt = sCnt[0];
    *mean = cnt ? (float)(sSum[0] / (double)cnt) : 0.f;
    *dloss_out = cnt ? (float)(1.0 / (double)cnt) : 0.f;
    if (n_valid_out) *n_valid_out = cnt;
  }
}

}  // namespace cce

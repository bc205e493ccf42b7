// Cut Cross-Entropy kernels for gfx950.
//
// Method: the Cut Cross-Entropy abstract (taxoreview.com page dblp:393/3562).  The loss needs
// only the correct token's logit plus the log-sum-exp over all logits, computed on the fly
// (sentences 4-5); matrix products and the log-sum-exp reduction run in on-chip memory so the
// N x V logits never reach global memory (sentence 6); the backward skips gradient work whose
// softmax contribution is negligible (sentence 9).
//
//   k_fwd_lse     S = C_tile E_tile^T on MFMA, online (max, sum exp) per token over the
//                 workgroup's vocabulary range, one partial per (range, token).
//   k_fwd_finish  merge of the partials (no atomics), target logit by gather-dot, loss.
//   k_bwd_g       recomputes S for a vocabulary chunk, forms G = dloss (softmax - onehot) in
//                 registers, flags negligible 64 x 64 blocks, stores the rest of G (bf16).
//   k_bwd_de      dE (+)= G C over the chunk, skipping flagged K stages.
//   k_bwd_dc      dC_chunk = G^T E, skipping flagged K stages.
//   k_mean, k_skip_init  small helpers for the mean-reduced call and the skip statistics.
#pragma once

#include "tile_engine.hpp"

namespace cce {

// ------------------------------------------------------------------------------------------
// Forward: per (token tile, vocabulary range) partial log-sum-exp in base 2.
//   part[split * N + n] = (m, s): m = max_v z*log2(e) over the range, s = sum 2^(z*log2(e) - m)
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void k_fwd_lse(const T* __restrict__ E,
                                                         const T* __restrict__ C, int N, int V,
                                                         int D, int n_split, int n_vt,
                                                         int n_items, float2* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) char sA0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kOpBytes];
  __shared__ float2 sRed[4][128];
  constexpr int KS = Traits<T>::kKs;

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= n_items) return;
  const int tb = item / n_split, sp = item % n_split;
  const int vt0 = (int)((int64_t)sp * n_vt / n_split);
  const int vt1 = (int)((int64_t)(sp + 1) * n_vt / n_split);
  const int n_k = ((D + 2 * KS - 1) / (2 * KS)) * 2;  // stages per tile, padded to even
  const int iters = (vt1 - vt0) * n_k;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int tok0 = tb * kTile;

  float m_run[4], s_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }
  f32x16_t acc[4][4];
  zero_acc(acc);

  const int64_t ldb = (int64_t)D * sizeof(T);
  uint32_t off[8];  // C and E tiles share the row length, hence the offsets
  kmajor_offsets(off, ldb, wave, lane);
  auto issue = [&](int it, char* a, char* b) {
    const int vt = vt0 + it / n_k, k0 = (it % n_k) * KS;
    const int kc = (D - k0) / Traits<T>::kEpc;  // <= 0 on the padding stage: all zeros
    const int64_t kb = (int64_t)k0 * sizeof(T);
    kmajor_issue(C + (int64_t)vt * kTile * D + k0, off, tile_records(V, (int64_t)vt * kTile, ldb, kb),
                 kc, a, wave, lane);
    kmajor_issue(E + (int64_t)tok0 * D + k0, off, tile_records(N, tok0, ldb, kb), kc, b, wave,
                 lane);
  };
  // Online log-sum-exp update for the finished tile, one token column group (ni) at a time so
  // that only 64 accumulators are in flight; each group is cleared for the next tile.
  auto epilogue = [&](int vt) {
    const int vbase = vt * kTile + 128 * wm;
    const bool full = vt * kTile + kTile <= V;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      float mx = -INFINITY;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = full || vbase + 32 * mi + acc_row(r, lane) < V;
          mx = fmaxf(mx, ok ? acc[mi][ni][r] : -INFINITY);
        }
      const float m_new = fmaxf(m_run[ni], mx * kLog2e);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float s = s_run[ni] * exp2_fast(m_run[ni] - m_use);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = full || vbase + 32 * mi + acc_row(r, lane) < V;
          const float e = exp2_fast(__builtin_fmaf(acc[mi][ni][r], kLog2e, -m_use));
          s += ok ? e : 0.f;
          acc[mi][ni][r] = 0.f;
        }
      s_run[ni] = s;
      m_run[ni] = m_new;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_tiles = vt1 - vt0;
  if (iters > 0) issue(0, sA0, sB0);
  for (int t = 0; t < n_tiles; ++t) {
    run_stream<T, true, true>(t * n_k, n_k, iters, issue, sA0, sB0, sA1, sB1, acc, wm, wn, lane);
    epilogue(vt0 + t);
  }

  // merge the two row halves of each column (lanes l and l ^ 32), then the two waves that
  // share columns (wm = 0, 1) through LDS
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const float mo = __shfl_xor(m_run[ni], 32);
    const float so = __shfl_xor(s_run[ni], 32);
    const float mn = fmaxf(m_run[ni], mo);
    const float mu = mn == -INFINITY ? 0.f : mn;
    s_run[ni] = s_run[ni] * exp2_fast(m_run[ni] - mu) + so * exp2_fast(mo - mu);
    m_run[ni] = mn;
  }
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) sRed[wn][32 * ni + lane] = make_float2(m_run[ni], s_run[ni]);
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const float2 o = sRed[wn][32 * ni + lane];
      const float mn = fmaxf(m_run[ni], o.x);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float s = s_run[ni] * exp2_fast(m_run[ni] - mu) + o.y * exp2_fast(o.x - mu);
      const int n = tok0 + 128 * wn + 32 * ni + lane;
      if (n < N) part[(int64_t)sp * N + n] = make_float2(mn, s);
    }
  }
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

// ------------------------------------------------------------------------------------------
// Forward finish: one wave per token.  LSE = ln2 * (M + log2 sum_i s_i 2^(m_i - M)); the
// target logit is a gather-dot of E[n] with C[t[n]] in fp32; loss = LSE - z_t.
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_fwd_finish(
    const T* __restrict__ E, const T* __restrict__ C, const int64_t* __restrict__ tgt, int N,
    int V, int D, int n_split, const float2* __restrict__ part, int64_t ignore_index,
    float* __restrict__ loss, float* __restrict__ lse, int32_t* __restrict__ err) {
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
  const bool bad = !ignored && (t < 0 || t >= V);
  float z = 0.f;
  if (!ignored && !bad) {
    const T* e = E + (int64_t)n * D;
    const T* c = C + t * (int64_t)D;
    for (int d = lane * 4; d < D; d += 256) {
#pragma unroll
      for (int i = 0; i < 4; ++i) z += (float)e[d + i] * (float)c[d + i];
    }
    z = wave_sum(z);
  }
  if (lane == 0) {
    lse[n] = l;
    loss[n] = ignored ? 0.f : (bad ? __builtin_nanf("") : l - z);
    if (bad && err) *err = 1;
  }
}

// ------------------------------------------------------------------------------------------
// Backward, step 1 for one vocabulary chunk [v0, v0 + vc): recompute the logit tile, form
// G = dloss (p - onehot) with p = 2^(z log2 e - lse log2 e), decide the 64 x 64 filter blocks
// and store G (chunk-local columns, row stride ldg) for the blocks that are kept.
//   flags[(n / 64) * fstride + v_local / 64] = 1 if the block is skipped (G not stored).
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_g(
    const T* __restrict__ E, const T* __restrict__ C, const int64_t* __restrict__ tgt,
    const float* __restrict__ lse, const float* __restrict__ dloss, int64_t dstride, int N,
    int V, int D, int v0, int vc, int n_tb, int n_vtc, T* __restrict__ G, int64_t ldg,
    uint8_t* __restrict__ flags, int fstride, float eps, int64_t ignore_index,
    unsigned long long* __restrict__ skip_count) {
  __shared__ __attribute__((aligned(1024))) char sA0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kOpBytes];
  constexpr int KS = Traits<T>::kKs;

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  int tb, vt;
  grouped_tile(lin, n_vtc, tb, vt);
  if (tb >= n_tb || vt >= n_vtc) return;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int tok0 = tb * kTile, vl0 = vt * kTile;  // vl0: chunk-local first vocab row
  const int n_k = ((D + 2 * KS - 1) / (2 * KS)) * 2;  // padded to even: last stage may be zeros
  const T* Cc = C + (int64_t)v0 * D;

  f32x16_t acc[4][4];
  zero_acc(acc);
  const int64_t ldb = (int64_t)D * sizeof(T);
  uint32_t off[8];
  kmajor_offsets(off, ldb, wave, lane);
  auto issue = [&](int it, char* a, char* b) {
    const int k0 = it * KS;
    const int kc = (D - k0) / Traits<T>::kEpc;
    const int64_t kb = (int64_t)k0 * sizeof(T);
    kmajor_issue(Cc + (int64_t)vl0 * D + k0, off, tile_records(vc, vl0, ldb, kb), kc, a, wave,
                 lane);
    kmajor_issue(E + (int64_t)tok0 * D + k0, off, tile_records(N, tok0, ldb, kb), kc, b, wave,
                 lane);
  };
  issue(0, sA0, sB0);
  run_stream<T, true, true>(0, n_k, n_k, issue, sA0, sB0, sA1, sB1, acc, wm, wn, lane);

  // epilogue: per column (token) constants
  const bool filter = eps > 0.f;
  bool sig[2][2] = {{false, false}, {false, false}};
  float coef[4], lse2[4];
  int trow[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int n = tok0 + 128 * wn + 32 * ni + (lane & 31);
    bool valid = false;
    float w = 0.f, l2 = 0.f;
    int tr = -1;
    if (n < N) {
      const int64_t t = tgt[n];
      valid = t != ignore_index;
      w = dloss[(int64_t)n * dstride];
      l2 = lse[n] * kLog2e;
      const int64_t tl = t - (int64_t)v0 - vl0 - 128 * wm;  // target row within this wave's rows
      tr = (valid && tl >= 0 && tl < 128) ? (int)tl : -1;
    }
    coef[ni] = valid ? w : 0.f;
    lse2[ni] = l2;
    trow[ni] = valid ? tr : -2;  // -2 marks an ignored or padded column
  }
  const bool full = vl0 + kTile <= vc;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * mi + acc_row(r, lane);  // row within this wave's 128 rows
        float p = exp2_fast(acc[mi][ni][r] * kLog2e - lse2[ni]);
        if (!full && vl0 + 128 * wm + row >= vc) p = 0.f;
        const bool is_t = row == trow[ni];
        sig[mi >> 1][ni >> 1] |= (trow[ni] != -2) && (p >= eps || is_t);
        acc[mi][ni][r] = coef[ni] * (is_t ? p - 1.f : p);
      }

  // block decisions (wave-wide), flags, statistics
  int n_skipped = 0;
  bool keep[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int vblk = vl0 + 128 * wm + 64 * a;   // chunk-local vocab start of the block
      const int nblk = tok0 + 128 * wn + 64 * b;  // token start of the block
      const bool in_range = vblk < vc && nblk < N;
      const bool any = __ballot(sig[a][b]) != 0ull;
      const bool k = in_range && (!filter || any);
      keep[a][b] = k;
      if (in_range && !k) ++n_skipped;
      if (lane == 0) flags[(int64_t)(nblk >> 6) * fstride + (vblk >> 6)] = k ? 0 : 1;
    }
  if (skip_count && lane == 0 && n_skipped) atomicAdd(skip_count, (unsigned long long)n_skipped);

  // store the kept blocks: 4 consecutive vocab rows of one token per lane and register group
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if (!keep[mi >> 1][ni >> 1]) continue;
      const int n = tok0 + 128 * wn + 32 * ni + (lane & 31);
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int vloc = vl0 + 128 * wm + 32 * mi + 8 * rq + 4 * (lane >> 5);
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

// Writes (or adds) this wave's 128 x 128 accumulators to a row-major fp32 matrix out[rows][ld]
// at (row0, col0); rows >= row_lim and columns >= col_lim are dropped.  For each register a
// half-wave writes 32 consecutive columns (128 bytes).
__device__ __forceinline__ void store_tile(float* __restrict__ out, int64_t ld, int row0,
                                           int row_lim, int col0, int col_lim,
                                           f32x16_t (&acc)[4][4], int lane, bool add) {
  const bool full = row0 + 128 <= row_lim && col0 + 128 <= col_lim;
  if (full && !add) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          out[(int64_t)(row0 + 32 * mi + acc_row(r, lane)) * ld + col0 + 32 * ni + (lane & 31)] =
              acc[mi][ni][r];
  } else if (full) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* p =
              out + (int64_t)(row0 + 32 * mi + acc_row(r, lane)) * ld + col0 + 32 * ni + (lane & 31);
          *p += acc[mi][ni][r];
        }
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * mi + acc_row(r, lane), col = col0 + 32 * ni + (lane & 31);
          if (row < row_lim && col < col_lim) {
            float* p = out + (int64_t)row * ld + col;
            *p = add ? *p + acc[mi][ni][r] : acc[mi][ni][r];
          }
        }
  }
}

// Builds the list of K stages of a backward product that are not entirely skipped.  Entry =
// (stage << 4) | mask, mask bit b set = the b-th 64-wide block of the tile's rows/columns is
// skipped within the stage (its operand chunk is loaded as zeros).
//   rowwise: flags of stage s are flags[(fr0 + b) * fstride + s * KS / 64]   (dE: K = vocab)
//   else   : flags of stage s are flags[(s * KS / 64) * fstride + fc0 + b]   (dC: K = tokens)
template <int KS>
__device__ __forceinline__ int build_stage_list(const uint8_t* __restrict__ flags, int fstride,
                                                int n_stages, bool rowwise, int fixed0,
                                                int* list, int* wave_cnt) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  int total = 0;
  for (int base = 0; base < n_stages; base += kThreads) {
    const int s = base + threadIdx.x;
    uint32_t mask = 15u;
    if (s < n_stages) {
      const int fk = (s * KS) >> 6;
      mask = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint8_t f = rowwise ? flags[(int64_t)(fixed0 + b) * fstride + fk]
                                  : flags[(int64_t)fk * fstride + fixed0 + b];
        mask |= (f ? 1u : 0u) << b;
      }
    }
    const bool active = s < n_stages && mask != 15u;
    const unsigned long long bal = __ballot(active);
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (active) list[off + before] = (s << 4) | (int)mask;
    total += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
  }
  // pad to an even count with an all-zero stage (every block masked), so the main loop runs
  // whole pairs of stages
  if (total & 1) {
    if (threadIdx.x == 0) list[total] = 15;
    __syncthreads();
    ++total;
  }
  return total;
}

// ------------------------------------------------------------------------------------------
// Backward, step 2: dE[tok tile, d tile] (+)= sum over the chunk's vocabulary of
// G[tok, v] C[v0 + v, d].  A = G (K-major, K = vocab), B = C chunk (MN-major).
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_de(
    const T* __restrict__ G, int64_t ldg, const T* __restrict__ Cc, int D, int N, int kv,
    int vc, const uint8_t* __restrict__ flags, int fstride, int n_tb, int n_dt,
    float* __restrict__ dE, int accumulate) {
  __shared__ __attribute__((aligned(1024))) char sA0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kOpBytes];
  __shared__ int sList[8192 / 32 + 8];  // stages of one chunk (+1 padding)
  __shared__ int sCnt[4];
  constexpr int KS = Traits<T>::kKs;

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  int tb, dt;
  grouped_tile(lin, n_dt, tb, dt);
  if (tb >= n_tb || dt >= n_dt) return;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int tok0 = tb * kTile, d0 = dt * kTile;
  const int n_stages = kv / KS;
  const int n_act = build_stage_list<KS>(flags, fstride, n_stages, true, tb * 4, sList, sCnt);

  f32x16_t acc[4][4];
  zero_acc(acc);
  if (n_act == 0 && accumulate) return;
  const int64_t ldb = (int64_t)D * sizeof(T);
  uint32_t offA[8], offB[8];
  kmajor_offsets(offA, ldg * (int64_t)sizeof(T), wave, lane);
  mn_offsets<T>(offB, ldb, d0, D, wave, lane);
  auto issue = [&](int i, char* a, char* b) {
    const int e = __builtin_amdgcn_readfirstlane(sList[i]);
    const int k0 = (e >> 4) * KS;
    const bool zero = (e >> wave) & 1;  // wave w loads the tile's token rows 64 w .. 64 w + 63
    kmajor_issue(G + (int64_t)tok0 * ldg + k0, offA, zero ? 0 : kRecords, 8, a, wave, lane);
    mn_issue<T>(Cc + (int64_t)k0 * D + d0, offB, tile_records(vc, k0, ldb, (int64_t)d0 * sizeof(T)),
                0u, b, wave, lane);
  };
  if (n_act > 0) {
    issue(0, sA0, sB0);
    run_stream<T, true, false>(0, n_act, n_act, issue, sA0, sB0, sA1, sB1, acc, wm, wn, lane);
  }
  store_tile(dE, D, tok0 + 128 * wm, N, d0 + 128 * wn, D, acc, lane, accumulate != 0);
}

// ------------------------------------------------------------------------------------------
// Backward, step 3: dC[v0 + v, d] = sum over tokens of G[tok, v] E[tok, d] for the chunk.
// A = G (MN-major, K = tokens), B = E (MN-major).
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_dc(
    const T* __restrict__ G, int64_t ldg, const T* __restrict__ E, int D, int N, int n_pad,
    int vc, const uint8_t* __restrict__ flags, int fstride, int n_vtc, int n_dt,
    float* __restrict__ dCc) {
  __shared__ __attribute__((aligned(1024))) char sA0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sA1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[kOpBytes];
  __shared__ int sList[4096 + 8];
  __shared__ int sCnt[4];
  constexpr int KS = Traits<T>::kKs;

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  int vt, dt;
  grouped_tile(lin, n_dt, vt, dt);
  if (vt >= n_vtc || dt >= n_dt) return;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int vl0 = vt * kTile, d0 = dt * kTile;
  const int n_stages = n_pad / KS;

  const int64_t ldb = (int64_t)D * sizeof(T);
  uint32_t offA[8], offB[8];
  mn_offsets<T>(offA, ldg * (int64_t)sizeof(T), vl0, (int)ldg, wave, lane);
  mn_offsets<T>(offB, ldb, d0, D, wave, lane);
  f32x16_t acc[4][4];
  zero_acc(acc);
  // token stages are processed in pieces of at most 4096 list entries
  for (int sbase = 0; sbase < n_stages; sbase += 4096) {
    const int cnt = min(4096, n_stages - sbase);
    const int n_act = build_stage_list<KS>(flags + (int64_t)((sbase * KS) >> 6) * fstride,
                                           fstride, cnt, false, vt * 4, sList, sCnt);
    auto issue = [&](int i, char* a, char* b) {
      const int e = __builtin_amdgcn_readfirstlane(sList[i]);
      const int k0 = (sbase + (e >> 4)) * KS;
      mn_issue<T>(G + (int64_t)k0 * ldg + vl0, offA, kRecords, (uint32_t)(e & 15), a, wave, lane);
      mn_issue<T>(E + (int64_t)k0 * D + d0, offB, tile_records(N, k0, ldb, (int64_t)d0 * sizeof(T)),
                  0u, b, wave, lane);
    };
    if (n_act > 0) {
      issue(0, sA0, sB0);
      run_stream<T, false, false>(0, n_act, n_act, issue, sA0, sB0, sA1, sB1, acc, wm, wn, lane);
    }
    __syncthreads();
  }
  store_tile(dCc, D, vl0 + 128 * wm, vc, d0 + 128 * wn, D, acc, lane, false);
}

// p[0..n) = 0 (a kernel rather than a memset, so the call stays safe under graph capture)
__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
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

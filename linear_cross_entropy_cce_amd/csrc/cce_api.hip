// libcce C ABI: argument validation, launch planning and kernel launches (include/cce.h,
// include/cce_timing.h).
//
// Host-side plan for the Cut Cross-Entropy abstract's method (taxoreview.com page
// dblp:393/3562, sentences 4-6 and 9):
//   forward : k_fwd_lse over (token tile x vocabulary range), then k_fwd_finish;
//   backward: the (token, vocabulary) plane is cut into pairs of a token block (<= Nc tokens)
//             and a vocabulary chunk (<= Vc rows), taken chunk by chunk and, within a chunk,
//             block by block.  k_bwd_g recomputes the first pair's G, then one k_bwd_fused per
//             pair p computes dE and dC of p and the G of p + 1, all on the caller's stream;
//             only the G of two pairs (Nc x Vc each) ever lives in the workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "cce.h"
#include "cce_timing.h"

#ifndef CCE_KB
#define CCE_KB 128
#endif
#ifndef CCE_NST
#define CCE_NST 2
#endif
#include "cce_kernels.hpp"

namespace {

using namespace cce;

constexpr int64_t kMaxRows = int64_t(1) << 24;
constexpr int64_t kMaxD = 65536;
constexpr int kAssumedCUs = 256;  // MI355X; only shapes the launch plan, never correctness

// Pipeline shape of every MFMA kernel: KB bytes of K per operand row and stage, NST stages in
// flight (LDS: NST x 2 x 256 x KB bytes).
constexpr int kKB = CCE_KB;
constexpr int kNST = CCE_NST;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t dtype_size(cce_dtype dt) { return dt == CCE_BF16 ? 2 : 4; }

bool sizes_ok(int64_t N, int64_t V, int64_t D, cce_dtype dt) {
  if (dt != CCE_F32 && dt != CCE_BF16) return false;
  if (N < 0 || V < 1 || D < 1) return false;
  if (D % (dt == CCE_BF16 ? 8 : 4) != 0) return false;
  return true;
}
// The kernels move E, C, the gradients and the workspace in 16-byte vectors.
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }
bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return false;
  return true;
}

bool sizes_supported(int64_t N, int64_t V, int64_t D) {
  return N <= kMaxRows && V <= kMaxRows && D <= kMaxD;
}

// Number of vocabulary ranges of the forward.  Cost model: waves of workgroups times tiles per
// workgroup; among plans within 3% of the best, prefer 8 ranges, which with 4 token tiles
// fills one XCD's 32 CUs with 4 + 8 distinct operand tiles.
int64_t plan_splits(int64_t N, int64_t V) {
  const int64_t n_tb = ceil_div(std::max<int64_t>(N, 1), kTile), n_vt = ceil_div(V, kTile);
  const int64_t smax = std::min<int64_t>(n_vt, 256);
  double best = 1e300;
  std::vector<double> cost(smax + 1, 0.0);
  for (int64_t s = 1; s <= smax; ++s) {
    cost[s] = (double)ceil_div(n_tb * s, kAssumedCUs) * (double)ceil_div(n_vt, s);
    best = std::min(best, cost[s]);
  }
  int64_t pick = 1;
  double pick_dist = 1e300;
  for (int64_t s = 1; s <= smax; ++s) {
    if (cost[s] > best * 1.03) continue;
    const double dist = std::fabs(std::log2((double)s) - 3.0);
    if (dist < pick_dist) { pick_dist = dist; pick = s; }
  }
  return pick;
}

int64_t env_int(const char* name, int64_t dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  const long long x = std::strtoll(v, &end, 10);
  return (end && *end == 0 && x > 0) ? (int64_t)x : dflt;
}

// Balanced split of `tiles` 256-wide tiles into the fewest parts of at most `max_tiles` each:
// part i covers tiles [i * tiles / parts, (i + 1) * tiles / parts), so parts differ by at most
// one tile and none is a short tail.
struct Split {
  int64_t parts, tiles;
  int64_t begin(int64_t i) const { return i * tiles / parts; }
  int64_t widest() const { return ceil_div(tiles, parts); }
};
Split balanced(int64_t tiles, int64_t max_tiles) {
  Split s;
  s.tiles = tiles;
  s.parts = ceil_div(tiles, std::max<int64_t>(max_tiles, 1));
  return s;
}

// Vocabulary chunks of the backward: at most 8192 rows (32 tiles) each; CCE_VC (a multiple of
// 256, at most 8192) narrows them.
Split plan_chunks(int64_t V) {
  static const int64_t vc_env = env_int("CCE_VC", 8192);
  const int64_t vc = std::max<int64_t>(kTile, std::min<int64_t>(vc_env, 8192) / kTile * kTile);
  return balanced(ceil_div(V, kTile), vc / kTile);
}
// Token blocks of the backward: at most 16384 tokens for bf16 inputs and 8192 for fp32 (so the
// G store of two pairs stays within 512 MiB); CCE_NC (a multiple of 256) overrides it.
Split plan_blocks(int64_t N, cce_dtype dt) {
  static const int64_t nc_env = env_int("CCE_NC", 0);
  const int64_t dflt = dt == CCE_BF16 ? 16384 : 8192;
  const int64_t nc =
      nc_env > 0 ? std::max<int64_t>(kTile, std::min<int64_t>(nc_env, 65536)) / kTile * kTile
                 : dflt;
  return balanced(ceil_div(std::max<int64_t>(N, 1), kTile), nc / kTile);
}
int64_t plan_chunk(int64_t V) { return plan_chunks(V).widest() * kTile; }

// Backward workspace: G and flags of two pairs in flight (p and p + 1, Nc x Vc each), the
// smallest lse log2(e) of each token tile (for skipping tiles with the forward's tile maxima),
// and, for bf16 gradients only, the fp32 running sums: dE [N, D] over the chunks and one
// chunk's dC [Vc, D] over the token blocks (when there is more than one block).
struct BwdLayout {
  Split blocks, chunks;
  int64_t nc, vc, fstride, n_pad;
  size_t g_bytes, flag_bytes, tmin_offset, de_offset, de_bytes, dc_offset, dc_bytes, total;
};
BwdLayout bwd_layout(int64_t N, int64_t V, int64_t D, cce_dtype dt, cce_dtype gdt) {
  BwdLayout L;
  L.blocks = plan_blocks(N, dt);
  L.chunks = plan_chunks(V);
  L.nc = L.blocks.widest() * kTile;
  L.vc = L.chunks.widest() * kTile;
  L.n_pad = ceil_div(std::max<int64_t>(N, 1), kTile) * kTile;
  L.fstride = L.vc / 64;
  L.g_bytes = align_up((size_t)L.nc * (size_t)L.vc * dtype_size(dt));
  L.flag_bytes = align_up((size_t)(L.nc / 64) * (size_t)L.fstride);
  L.tmin_offset = 2 * (L.g_bytes + L.flag_bytes);
  L.de_offset = L.tmin_offset + align_up((size_t)(L.n_pad / kTile) * 4);
  const bool bf = gdt == CCE_BF16;
  L.de_bytes = bf ? align_up((size_t)std::max<int64_t>(N, 1) * (size_t)D * 4) : 0;
  L.dc_offset = L.de_offset + L.de_bytes;
  L.dc_bytes = bf && L.blocks.parts > 1 ? align_up((size_t)L.vc * (size_t)D * 4) : 0;
  L.total = L.dc_offset + L.dc_bytes;
  return L;
}
size_t fwd_bytes(int64_t N, int64_t V) {
  return align_up((size_t)plan_splits(N, V) * (size_t)std::max<int64_t>(N, 1) * 8);
}
size_t mean_extra_bytes(int64_t N) {
  return align_up((size_t)ceil_div(std::max<int64_t>(N, 1), 64) * 64 * 8) + kAlign;
}

cce_status launch_status() {
  return hipGetLastError() == hipSuccess ? CCE_OK : CCE_ERR_HIP;
}

// Benchmark timing hook (cce_timing.h): event pairs around launches of the selected kernel
// kinds.  Process-wide and off unless a benchmark starts it.
struct Timing {
  bool on = false;
  uint32_t mask = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;   // 2 per launch slot
  std::vector<int> kind;
};
Timing g_timing;

struct TimedLaunch {
  bool rec = false;
  hipStream_t st;
  TimedLaunch(int kind, hipStream_t s) : st(s) {
    Timing& T = g_timing;
    if (T.on && ((T.mask >> kind) & 1u) && T.used < (int)T.kind.size()) {
      rec = hipEventRecord(T.ev[2 * T.used], st) == hipSuccess;
      if (rec) T.kind[T.used] = kind;
    }
  }
  ~TimedLaunch() {
    if (rec) {
      Timing& T = g_timing;
      if (hipEventRecord(T.ev[2 * T.used + 1], st) == hipSuccess) ++T.used;
    }
  }
};

int grid_for(int64_t items) { return (int)(ceil_div(items, 8) * 8); }

// Whether D leaves a partial group of NST stages of K (then the kernels mask K per lane).
template <typename T>
bool k_tail(int64_t D) {
  return D % ((int64_t)kNST * kKB / (int64_t)sizeof(T)) != 0;
}

// Floats of the forward's tile maxima: one per wave of every 256 x 256 (token, vocabulary) tile.
int64_t tile_max_count(int64_t N, int64_t V) {
  return ceil_div(std::max<int64_t>(N, 1), kTile) * ceil_div(V, kTile) * kWaves;
}

template <typename T>
cce_status forward_impl(const T* E, const T* C, const int64_t* tgt, int64_t N, int64_t V,
                        int64_t D, int64_t ii, float* loss, float* lse, float* tile_max,
                        void* ws, int32_t* err, hipStream_t st, int64_t voff = 0,
                        float* zt = nullptr) {
  const int64_t n_split = plan_splits(N, V);
  const int64_t n_tb = ceil_div(N, kTile), n_vt = ceil_div(V, kTile);
  const int64_t items = n_tb * n_split;
  float2* part = (float2*)ws;
  {
    TimedLaunch tl(CCE_KERNEL_FWD_LSE, st);
    if (k_tail<T>(D))
      hipLaunchKernelGGL((k_fwd_lse<T, kKB, kNST, true>), dim3(grid_for(items)), dim3(kThreads), 0,
                         st, E, C, (int)N, (int)V, (int)D, (int)n_split, (int)n_vt, (int)items, part,
                         tile_max);
    else
      hipLaunchKernelGGL((k_fwd_lse<T, kKB, kNST, false>), dim3(grid_for(items)), dim3(kThreads), 0,
                         st, E, C, (int)N, (int)V, (int)D, (int)n_split, (int)n_vt, (int)items, part,
                         tile_max);
  }
  if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  TimedLaunch tl(CCE_KERNEL_FWD_FINISH, st);
  hipLaunchKernelGGL(k_fwd_finish<T>, dim3((unsigned)ceil_div(N, 4)), dim3(kFinishThreads), 0, st, E,
                     C, tgt, (int)N, (int)V, (int)D, (int)n_split, part, ii, loss, lse, err, voff,
                     zt);
  return launch_status();
}

template <typename T>
cce_status backward_impl(const float* dloss, int64_t dstride, const T* E, const T* C,
                         const int64_t* tgt, const float* lse, const float* tile_max, int64_t N,
                         int64_t V, int64_t D, int64_t ii, int64_t voff, float eps,
                         float p_floor, void* dE, void* dC, cce_dtype gdt, void* ws,
                         int64_t* skip_stats, hipStream_t st, cce_dtype dt) {
  const BwdLayout L = bwd_layout(N, V, D, dt, gdt);
  const bool bf = gdt == CCE_BF16;
  // dE accumulates over the chunks in fp32: in place, or in the workspace for bf16 output
  float* dE_acc = bf ? (float*)((char*)ws + L.de_offset) : (float*)dE;
  float* dC_acc = (float*)((char*)ws + L.dc_offset);   // bf16 gradients, several blocks
  const int64_t n_dt = ceil_div(D, kTile);
  const int64_t n_blk = L.blocks.parts, n_pairs = L.chunks.parts * n_blk;
  const int64_t n_vt_all = ceil_div(V, kTile);
  if (skip_stats) {
    TimedLaunch tl(CCE_KERNEL_AUX, st);
    hipLaunchKernelGGL(k_skip_init, dim3(1), dim3(64), 0, st, skip_stats,
                       ceil_div(N, 64) * ceil_div(V, 64));
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  }
  float* tile_lse_min = (float*)((char*)ws + L.tmin_offset);
  const bool tile_skip = tile_max != nullptr && eps > 0.f;
  if (tile_skip) {
    TimedLaunch tl(CCE_KERNEL_AUX, st);
    hipLaunchKernelGGL(k_tile_lse_min, dim3((unsigned)(L.n_pad / kTile)), dim3(256), 0, st, lse,
                       tgt, (int)N, ii, tile_lse_min);
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  }
  // pair p = (chunk c, token block b), p = c * n_blk + b; its G and flags use buffer p % 2
  auto args = [&](int64_t p) {
    const int64_t c = p / n_blk, b = p % n_blk;
    const int64_t n0 = L.blocks.begin(b) * kTile;
    const int64_t n1 = std::min<int64_t>(N, L.blocks.begin(b + 1) * kTile);
    const int64_t v0 = L.chunks.begin(c) * kTile;
    const int64_t v1 = std::min<int64_t>(V, L.chunks.begin(c + 1) * kTile);
    const int buf = (int)(p & 1);
    BwdArgs<T> A;
    A.E = E + n0 * D; A.C = C; A.tgt = tgt + n0; A.lse = lse + n0;
    A.dloss = dloss + n0 * dstride; A.dstride = dstride;
    A.N = (int)(n1 - n0); A.V = (int)V; A.D = (int)D;
    A.n_pad = (int)(ceil_div(n1 - n0, kTile) * kTile);
    A.v0 = (int)v0;
    A.vc = (int)(v1 - v0);
    A.n_tb = A.n_pad / kTile; A.n_vtc = (int)ceil_div(A.vc, kTile); A.n_dt = (int)n_dt;
    A.G = (T*)((char*)ws + buf * L.g_bytes);
    A.ldg = L.vc;
    A.flags = (uint8_t*)ws + 2 * L.g_bytes + buf * L.flag_bytes;
    A.fstride = (int)L.fstride;
    A.eps = eps; A.p_floor = p_floor; A.ignore_index = ii; A.voff = voff;
    A.skip_count = (unsigned long long*)skip_stats;
    A.dE = dE_acc + n0 * D;
    A.accumulate = c > 0 ? 1 : 0;
    // dC of the chunk: fp32 gradients add up in dC itself; bf16 gradients of several blocks
    // in the chunk accumulator, the last block rounding the sum into dC
    const bool last_blk = b == n_blk - 1;
    if (!bf) {
      A.dc_in = b > 0 ? (const float*)dC + v0 * D : nullptr;
      A.dc_out = (float*)dC + v0 * D;
      A.dc_bf16 = 0;
    } else {
      A.dc_in = b > 0 ? dC_acc : nullptr;
      A.dc_out = last_blk ? (void*)((__bf16*)dC + v0 * D) : (void*)dC_acc;
      A.dc_bf16 = last_blk ? 1 : 0;
    }
    // without maxima, both pointers lead to the token-tile minima (at least 256 bytes) and the
    // kernel reads their first floats only
    const int64_t tb0 = n0 / kTile;
    A.tile_max = tile_skip ? tile_max + tb0 * n_vt_all * kWaves : tile_lse_min;
    A.tile_lse_min = tile_skip ? tile_lse_min + tb0 : tile_lse_min;
    A.tile_skip = tile_skip ? 1 : 0;
    A.n_vt_all = (int)n_vt_all;
    A.skip_bound = eps > 0.f ? std::log2(eps) - 1.f / 1024.f : -INFINITY;
    return A;
  };
  {
    const BwdArgs<T> A0 = args(0);
    TimedLaunch tl(CCE_KERNEL_BWD_G, st);
    const dim3 grid(grid_for(bwd_items(A0.n_tb, A0.n_vtc)));
    if (k_tail<T>(D))
      hipLaunchKernelGGL((k_bwd_g<T, kKB, kNST, true>), grid, dim3(kThreads), 0, st, A0);
    else
      hipLaunchKernelGGL((k_bwd_g<T, kKB, kNST, false>), grid, dim3(kThreads), 0, st, A0);
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  }
  for (int64_t p = 0; p < n_pairs; ++p) {
    const BwdArgs<T> A = args(p);
    const bool more = p + 1 < n_pairs;
    const BwdArgs<T> Nx = more ? args(p + 1) : A;
    const int r_de = grid_for(bwd_items(A.n_tb, A.n_dt));
    const int r_dc = grid_for(bwd_items(A.n_vtc, A.n_dt));
    const int r_g = more ? grid_for(bwd_items(Nx.n_tb, Nx.n_vtc)) : 0;
    TimedLaunch tl(CCE_KERNEL_BWD_FUSED, st);
    const dim3 grid(r_de + r_dc + r_g);
    if (k_tail<T>(D))
      hipLaunchKernelGGL((k_bwd_fused<T, kKB, kNST, true>), grid, dim3(kThreads), 0, st, A, Nx,
                         r_de, r_dc);
    else
      hipLaunchKernelGGL((k_bwd_fused<T, kKB, kNST, false>), grid, dim3(kThreads), 0, st, A, Nx,
                         r_de, r_dc);
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  }
  if (bf) {
    TimedLaunch tl(CCE_KERNEL_AUX, st);
    const int64_t n = N * D;
    hipLaunchKernelGGL(k_f32_to_bf16, dim3((unsigned)std::min<int64_t>(ceil_div(n, 1024), 4096)),
                       dim3(256), 0, st, (const float*)dE_acc, (__bf16*)dE, n);
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  }
  return CCE_OK;
}

}  // namespace

extern "C" {

const char* cce_status_string(cce_status s) {
  switch (s) {
    case CCE_OK: return "CCE_OK";
    case CCE_ERR_INVALID_ARGUMENT: return "CCE_ERR_INVALID_ARGUMENT";
    case CCE_ERR_UNSUPPORTED: return "CCE_ERR_UNSUPPORTED";
    case CCE_ERR_WORKSPACE_TOO_SMALL: return "CCE_ERR_WORKSPACE_TOO_SMALL";
    case CCE_ERR_HIP: return "CCE_ERR_HIP";
    default: break;
  }
  return "CCE_ERR_UNKNOWN";
}

size_t cce_forward_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D)) return 0;
  return fwd_bytes(N, V);
}

bool grad_dtype_ok(cce_dtype g) { return g == CCE_F32 || g == CCE_BF16; }

size_t cce_backward_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dt,
                                    cce_dtype gdt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D) || !grad_dtype_ok(gdt)) return 0;
  return bwd_layout(N, V, D, dt, gdt).total;
}

int64_t cce_tile_max_count(int64_t N, int64_t V, int64_t D, cce_dtype dt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D)) return 0;
  return tile_max_count(N, V);
}

size_t cce_loss_mean_workspace_bytes(int64_t N, int64_t V, int64_t D, cce_dtype dt,
                                     cce_dtype gdt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D) || !grad_dtype_ok(gdt)) return 0;
  return fwd_bytes(N, V) + bwd_layout(N, V, D, dt, gdt).total + mean_extra_bytes(N);
}

int64_t cce_forward_splits(int64_t N, int64_t V, int64_t D, cce_dtype dt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D)) return 0;
  return plan_splits(N, V);
}

int64_t cce_backward_chunk(int64_t N, int64_t V, int64_t D, cce_dtype dt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D)) return 0;
  return plan_chunk(V);
}

int64_t cce_backward_token_block(int64_t N, int64_t V, int64_t D, cce_dtype dt) {
  if (!sizes_ok(N, V, D, dt) || !sizes_supported(N, V, D)) return 0;
  return plan_blocks(N, dt).widest() * kTile;
}

cce_status cce_forward(const void* E, const void* C, const int64_t* targets, int64_t N,
                       int64_t V, int64_t D, cce_dtype dt, int64_t ignore_index, float* loss,
                       float* lse, float* tile_max, void* ws, size_t ws_bytes, int32_t* err_flag,
                       void* stream) {
  if (!sizes_ok(N, V, D, dt)) return CCE_ERR_INVALID_ARGUMENT;
  if (!sizes_supported(N, V, D)) return CCE_ERR_UNSUPPORTED;
  if (N == 0) return CCE_OK;
  if (!E || !C || !targets || !loss || !lse || !ws) return CCE_ERR_INVALID_ARGUMENT;
  if (!all_aligned16({E, C, ws}) || !aligned4(tile_max)) return CCE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < fwd_bytes(N, V)) return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  if (dt == CCE_BF16)
    return forward_impl<__bf16>((const __bf16*)E, (const __bf16*)C, targets, N, V, D,
                                ignore_index, loss, lse, tile_max, ws, err_flag, st);
  return forward_impl<float>((const float*)E, (const float*)C, targets, N, V, D, ignore_index,
                             loss, lse, tile_max, ws, err_flag, st);
}

}  // extern "C"

namespace {

// cce_backward and cce_backward_shard: vocabulary rows [voff, voff + V) in C.
cce_status backward_entry(const float* dloss, int64_t dloss_stride, const void* E,
                          const void* C, const int64_t* targets, const float* lse,
                          const float* tile_max, int64_t N, int64_t V, int64_t D, cce_dtype dt,
                          int64_t ignore_index,
                          int64_t voff, float filter_eps, float entry_floor, void* dE, void* dC,
                          cce_dtype grad_dtype, void* ws, size_t ws_bytes, int64_t* skip_stats,
                          void* stream) {
  if (!sizes_ok(N, V, D, dt)) return CCE_ERR_INVALID_ARGUMENT;
  if (!sizes_supported(N, V, D)) return CCE_ERR_UNSUPPORTED;
  if (!std::isfinite(filter_eps) || filter_eps < 0.f) return CCE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(entry_floor) || entry_floor < 0.f) return CCE_ERR_INVALID_ARGUMENT;
  if (dloss_stride != 0 && dloss_stride != 1) return CCE_ERR_INVALID_ARGUMENT;
  if (!grad_dtype_ok(grad_dtype)) return CCE_ERR_INVALID_ARGUMENT;
  if (voff < 0) return CCE_ERR_INVALID_ARGUMENT;
  if (N == 0) {
    // nothing to reduce: dC is still defined (all zero) and so are the statistics
    if (!dC || !aligned16(dC)) return CCE_ERR_INVALID_ARGUMENT;
    hipStream_t st = (hipStream_t)stream;
    const int64_t n = V * D * (int64_t)dtype_size(grad_dtype) / 4;   // 4-byte words
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)std::min<int64_t>(ceil_div(n, 1024), 4096)),
                       dim3(256), 0, st, (float*)dC, n);
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
    if (skip_stats) {
      hipLaunchKernelGGL(k_skip_init, dim3(1), dim3(64), 0, st, skip_stats, (int64_t)0);
      if (launch_status() != CCE_OK) return CCE_ERR_HIP;
    }
    return CCE_OK;
  }
  if (!dloss || !E || !C || !targets || !lse || !dE || !dC || !ws)
    return CCE_ERR_INVALID_ARGUMENT;
  if (!all_aligned16({E, C, dE, dC, ws}) || !aligned4(tile_max)) return CCE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < bwd_layout(N, V, D, dt, grad_dtype).total) return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  if (dt == CCE_BF16)
    return backward_impl<__bf16>(dloss, dloss_stride, (const __bf16*)E, (const __bf16*)C,
                                 targets, lse, tile_max, N, V, D, ignore_index, voff,
                                 filter_eps, entry_floor, dE, dC, grad_dtype, ws, skip_stats, st,
                                 dt);
  return backward_impl<float>(dloss, dloss_stride, (const float*)E, (const float*)C, targets,
                              lse, tile_max, N, V, D, ignore_index, voff, filter_eps,
                              entry_floor, dE, dC, grad_dtype, ws, skip_stats, st, dt);
}

}  // namespace

extern "C" {

cce_status cce_backward(const float* dloss, int64_t dloss_stride, const void* E, const void* C,
                        const int64_t* targets, const float* lse, const float* tile_max,
                        int64_t N, int64_t V, int64_t D, cce_dtype dt, int64_t ignore_index,
                        float filter_eps, float entry_floor, void* dE, void* dC,
                        cce_dtype grad_dtype, void* ws, size_t ws_bytes, int64_t* skip_stats,
                        void* stream) {
  return backward_entry(dloss, dloss_stride, E, C, targets, lse, tile_max, N, V, D, dt,
                        ignore_index, 0, filter_eps, entry_floor, dE, dC, grad_dtype, ws,
                        ws_bytes, skip_stats, stream);
}

cce_status cce_backward_shard(const float* dloss, int64_t dloss_stride, const void* E,
                              const void* C, const int64_t* targets, const float* lse,
                              const float* tile_max, int64_t N, int64_t V, int64_t D,
                              cce_dtype dt, int64_t ignore_index, int64_t vocab_offset,
                              float filter_eps, float entry_floor, void* dE, void* dC,
                              cce_dtype grad_dtype, void* ws, size_t ws_bytes,
                              int64_t* skip_stats, void* stream) {
  return backward_entry(dloss, dloss_stride, E, C, targets, lse, tile_max, N, V, D, dt,
                        ignore_index, vocab_offset, filter_eps, entry_floor, dE, dC, grad_dtype,
                        ws, ws_bytes, skip_stats, stream);
}

cce_status cce_forward_shard(const void* E, const void* C, const int64_t* targets, int64_t N,
                             int64_t V, int64_t D, cce_dtype dt, int64_t ignore_index,
                             int64_t vocab_offset, float* lse_shard, float* target_logit,
                             float* tile_max, void* ws, size_t ws_bytes, void* stream) {
  if (!sizes_ok(N, V, D, dt)) return CCE_ERR_INVALID_ARGUMENT;
  if (!sizes_supported(N, V, D)) return CCE_ERR_UNSUPPORTED;
  if (vocab_offset < 0) return CCE_ERR_INVALID_ARGUMENT;
  if (N == 0) return CCE_OK;
  if (!E || !C || !targets || !lse_shard || !target_logit || !ws)
    return CCE_ERR_INVALID_ARGUMENT;
  if (!all_aligned16({E, C, ws}) || !aligned4(tile_max)) return CCE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < fwd_bytes(N, V)) return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  if (dt == CCE_BF16)
    return forward_impl<__bf16>((const __bf16*)E, (const __bf16*)C, targets, N, V, D,
                                ignore_index, nullptr, lse_shard, tile_max, ws, nullptr, st,
                                vocab_offset, target_logit);
  return forward_impl<float>((const float*)E, (const float*)C, targets, N, V, D, ignore_index,
                             nullptr, lse_shard, tile_max, ws, nullptr, st, vocab_offset,
                             target_logit);
}

cce_status cce_merge_shards(const float* lse_shards, const float* target_logits,
                            int64_t n_shards, int64_t N, const int64_t* targets,
                            int64_t ignore_index, int64_t V_total, float* loss, float* lse,
                            int32_t* err_flag, void* stream) {
  if (N < 0 || n_shards < 1 || n_shards > 65536 || V_total < 1 || N > kMaxRows)
    return CCE_ERR_INVALID_ARGUMENT;
  if (N == 0) return CCE_OK;
  if (!lse_shards || !target_logits || !targets || !loss || !lse) return CCE_ERR_INVALID_ARGUMENT;
  hipStream_t st = (hipStream_t)stream;
  TimedLaunch tl(CCE_KERNEL_FWD_FINISH, st);
  hipLaunchKernelGGL(k_merge_shards, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, st,
                     lse_shards, target_logits, (int)n_shards, (int)N, targets, ignore_index,
                     V_total, loss, lse, err_flag);
  return launch_status();
}

cce_status cce_loss_mean(const void* E, const void* C, const int64_t* targets, int64_t N,
                         int64_t V, int64_t D, cce_dtype dt, int64_t ignore_index,
                         float filter_eps, float entry_floor, float* loss_mean,
                         int64_t* n_valid, void* dE, void* dC, cce_dtype grad_dtype, void* ws,
                         size_t ws_bytes, int32_t* err_flag, int64_t* skip_stats, void* stream) {
  if (!sizes_ok(N, V, D, dt)) return CCE_ERR_INVALID_ARGUMENT;
  if (!sizes_supported(N, V, D)) return CCE_ERR_UNSUPPORTED;
  if (!std::isfinite(filter_eps) || filter_eps < 0.f) return CCE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(entry_floor) || entry_floor < 0.f) return CCE_ERR_INVALID_ARGUMENT;
  if (!grad_dtype_ok(grad_dtype)) return CCE_ERR_INVALID_ARGUMENT;
  if (!loss_mean || !dC || !ws) return CCE_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!E || !C || !targets || !dE)) return CCE_ERR_INVALID_ARGUMENT;
  if (!all_aligned16({dC, ws}) || (N > 0 && !all_aligned16({E, C, dE})))
    return CCE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < cce_loss_mean_workspace_bytes(N, V, D, dt, grad_dtype))
    return CCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = (hipStream_t)stream;
  const size_t fb = fwd_bytes(N, V), bb = bwd_layout(N, V, D, dt, grad_dtype).total;
  char* base = (char*)ws;
  char* extra = base + fb + bb;
  const size_t rows = (size_t)ceil_div(std::max<int64_t>(N, 1), 64) * 64;
  float* loss = (float*)extra;
  float* lse = loss + rows;
  float* dloss = (float*)(extra + align_up(rows * 8));
  if (N == 0) {
    hipLaunchKernelGGL(k_mean, dim3(1), dim3(1024), 0, st, (const float*)nullptr,
                       (const int64_t*)nullptr, 0, ignore_index, loss_mean, dloss, n_valid);
    if (launch_status() != CCE_OK) return CCE_ERR_HIP;
    return cce_backward(dloss, 0, E, C, targets, lse, nullptr, 0, V, D, dt, ignore_index,
                        filter_eps, entry_floor, dE, dC, grad_dtype, base + fb, bb, skip_stats,
                        stream);
  }
  cce_status s = cce_forward(E, C, targets, N, V, D, dt, ignore_index, loss, lse, nullptr, base,
                             fb, err_flag, stream);
  if (s != CCE_OK) return s;
  {
    TimedLaunch tl(CCE_KERNEL_AUX, st);
    hipLaunchKernelGGL(k_mean, dim3(1), dim3(1024), 0, st, loss, targets, (int)N, ignore_index,
                       loss_mean, dloss, n_valid);
  }
  if (launch_status() != CCE_OK) return CCE_ERR_HIP;
  return cce_backward(dloss, 0, E, C, targets, lse, nullptr, N, V, D, dt, ignore_index,
                      filter_eps, entry_floor, dE, dC, grad_dtype, base + fb, bb, skip_stats,
                      stream);
}

cce_status cce_timing_begin(uint32_t kind_mask, int32_t max_launches) {
  if (max_launches < 1) return CCE_ERR_INVALID_ARGUMENT;
  Timing& T = g_timing;
  for (hipEvent_t e : T.ev) (void)hipEventDestroy(e);
  T = Timing();
  T.ev.resize(2 * (size_t)max_launches);
  for (auto& e : T.ev)
    if (hipEventCreate(&e) != hipSuccess) return CCE_ERR_HIP;
  T.kind.assign((size_t)max_launches, 0);
  T.mask = kind_mask;
  T.on = true;
  return CCE_OK;
}

cce_status cce_timing_end(float* ms, int64_t* launches) {
  if (!ms || !launches) return CCE_ERR_INVALID_ARGUMENT;
  Timing& T = g_timing;
  for (int k = 0; k < CCE_KERNEL_KINDS; ++k) { ms[k] = 0.f; launches[k] = 0; }
  cce_status st = CCE_OK;
  for (int i = 0; i < T.used; ++i) {
    float t = 0.f;
    if (hipEventSynchronize(T.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, T.ev[2 * i], T.ev[2 * i + 1]) != hipSuccess) {
      st = CCE_ERR_HIP;
      continue;
    }
    ms[T.kind[i]] += t;
    launches[T.kind[i]] += 1;
  }
  for (hipEvent_t e : T.ev) (void)hipEventDestroy(e);
  T = Timing();
  return st;
}

}  // extern "C"

// Tile engine for the Cut Cross-Entropy kernels on gfx950 (MI355X, CDNA4).
//
// Every hot kernel of the library is a 256 x 256 output tile of a matrix product
// acc[m][n] = sum_k A[m][k] B[n][k] computed by one workgroup of 256 threads (4 waves of 64):
//   * each wave owns a 128 x 128 quarter as 4 x 4 blocks of 32 x 32 fp32 accumulators
//     (v_mfma_f32_32x32x16_bf16 for bf16 operands, v_mfma_f32_32x32x2f32 for fp32);
//   * operands stream HBM -> LDS with direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds),
//     one stage of 128 bytes of K per operand row, double buffered in two separate LDS
//     objects so the loads of stage s+1 overlap the MFMAs of stage s;
//   * an operand is either K-major (row = m or n, K contiguous, e.g. E[N,D] and C[V,D] when
//     contracting over D) or MN-major (row = k, m/n contiguous, e.g. C when contracting over
//     the vocabulary).  K-major fragments are read with ds_read_b128, MN-major bf16 fragments
//     with the gfx950 transposing LDS read ds_read_b64_tr_b16, so no operand is ever
//     transposed in HBM.
//
// Accumulator layout (32 x 32 block, lane l, register r, verified on MI355X):
//   column = l % 32, row = 8 * (r / 4) + 4 * (l / 32) + r % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kThreads = 256;
constexpr int kTile = 256;           // tile rows (M) and columns (N)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
  static constexpr int kEpc = 8;     // elements per 16-byte chunk
  static constexpr int kKs = 64;     // K per stage (128 bytes per K-major row)
  typedef bf16x8_t frag_t;
};
template <> struct Traits<float> {
  static constexpr int kEpc = 4;
  static constexpr int kKs = 32;
  typedef f32x4_t frag_t;
};

__device__ __forceinline__ void wait_vmcnt0() {
  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Wave index as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------------------------------
// HBM -> LDS stage loads with buffer_load ... lds.  Each wave issues 8 instructions per
// operand; one instruction moves 64 lanes x 16 bytes into 1 KB of consecutive LDS.  Every
// lane keeps a fixed byte offset per instruction relative to the stage's tile origin (a
// uniform pointer turned into a buffer descriptor); masked lanes use an offset past the
// descriptor's range, which the hardware answers with zeros.  The XOR swizzles make the
// fragment reads below free of bank conflicts: a lane picks which global chunk lands in its
// fixed LDS slot.
// ---------------------------------------------------------------------------------------
constexpr uint32_t kOob = 0x80000000u;         // offset answered with zeros
constexpr int kRecords = 0x7FFFFFF0;           // descriptor range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, records, 0x00020000);
}

__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

// Stage geometry.  KB = bytes of K per K-major operand row per stage (128 or 64), so one
// operand's share of a stage is 256 x KB bytes, and each wave issues KB / 16 direct-to-LDS
// instructions per operand and stage.
template <int KB>
struct Geo {
  static_assert(KB == 128 || KB == 64, "stage K bytes");
  static constexpr int kChunks = KB / 16;         // 16-byte chunks per K-major row
  static constexpr int kIssue = KB / 16;          // instructions per wave per operand
  static constexpr int kRowsPerWin = 256 / KB;    // K-major rows per 256-byte bank window
  static constexpr int kOpBytes = 256 * KB;       // one operand's share of one stage
  static constexpr int kGroups = KB / 32;         // MFMA k-groups per stage
};

// K-major operand: 256 rows x KB bytes per stage.  LDS slot (row r, chunk pc) holds logical K
// chunk pc ^ f(r), f(r) = (r / rows-per-window) mod chunks, which spreads the 16 rows read by
// one quarter-wave over distinct banks.  Instruction q of wave w fills 1 KB of consecutive
// LDS, i.e. rows (w * I + q) * (1024 / KB) onwards (I = instructions per wave), so wave w
// covers rows 64 w .. 64 w + 63.
template <int KB>
__device__ __forceinline__ int kmajor_row(int wave, int q, int lane) {
  return (wave * Geo<KB>::kIssue + q) * (1024 / KB) + lane / Geo<KB>::kChunks;
}
template <int KB>
__device__ __forceinline__ int kmajor_chunk(int r, int lane) {
  return (lane % Geo<KB>::kChunks) ^ ((r / Geo<KB>::kRowsPerWin) % Geo<KB>::kChunks);
}

// Offsets of this lane's chunks relative to the tile origin (row0, k0).  Rows past the
// operand's end are cut off by the descriptor range (tile_records), not here.
template <int KB>
__device__ __forceinline__ void kmajor_offsets(uint32_t (&off)[Geo<KB>::kIssue], int64_t ld_bytes,
                                               int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    const int r = kmajor_row<KB>(wave, q, lane);
    off[q] = (uint32_t)(r * ld_bytes) + 16u * kmajor_chunk<KB>(r, lane);
  }
}

// Valid bytes from a tile origin at (row0, k0) of a row-major operand with row_lim rows:
// every chunk of a row < row_lim lies below it and every chunk of a later row above it.
__device__ __forceinline__ int tile_records(int64_t row_lim, int64_t row0, int64_t ld_bytes,
                                            int64_t k0_bytes) {
  const int64_t b = (row_lim - row0) * ld_bytes - k0_bytes;
  return b <= 0 ? 0 : (b > kRecords ? kRecords : (int)b);
}

// One slice of a stage: instructions [Q0, Q1) of this wave.  k_chunks = valid 16-byte K
// chunks left from k0 (>= chunks per row: full stage).
template <int KB>
__device__ __forceinline__ void kmajor_issue(const void* origin,
                                             const uint32_t (&off)[Geo<KB>::kIssue], int records,
                                             int k_chunks, char* lds, int wave, int lane,
                                             int q0 = 0, int q1 = Geo<KB>::kIssue) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(origin, records);
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    if (q < q0 || q >= q1) continue;
    uint32_t o = off[q];
    if (k_chunks < Geo<KB>::kChunks)
      o = kmajor_chunk<KB>(kmajor_row<KB>(wave, q, lane), lane) < k_chunks ? o : kOob;
    lds_load16(rs, lds + (wave * Geo<KB>::kIssue + q) * 1024, o);
  }
}

// MN-major operand: KB / sizeof(T) rows of k, each RB = 256 * sizeof(T) bytes of columns.
// LDS slot (row k, chunk pc) holds logical column chunk pc ^ (4 * (k & 3)).
template <typename T, int KB>
__device__ __forceinline__ int mn_row(int wave, int q, int lane) {
  constexpr int RB = 256 * (int)sizeof(T);
  return ((wave * Geo<KB>::kIssue + q) * 1024 + lane * 16) / RB;
}
template <typename T, int KB>
__device__ __forceinline__ int mn_col(int wave, int q, int lane) {  // first column of the chunk
  constexpr int RB = 256 * (int)sizeof(T);
  const int r = mn_row<T, KB>(wave, q, lane);
  const int pc = (((wave * Geo<KB>::kIssue + q) * 1024 + lane * 16) % RB) >> 4;
  return (pc ^ (4 * (r & 3))) * Traits<T>::kEpc;
}

// Offsets for a tile whose first column is col0 (columns >= col_lim masked here; rows past
// the end are cut off by the descriptor range).
template <typename T, int KB>
__device__ __forceinline__ void mn_offsets(uint32_t (&off)[Geo<KB>::kIssue], int64_t ld_bytes,
                                           int col0, int col_lim, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    const int r = mn_row<T, KB>(wave, q, lane), c = mn_col<T, KB>(wave, q, lane);
    off[q] = (col0 + c < col_lim) ? (uint32_t)(r * ld_bytes) + (uint32_t)(c * sizeof(T)) : kOob;
  }
}

// One slice of a stage: instructions [Q0, Q1).  zero_cols bit b = load zeros for columns
// 64 b .. 64 b + 63 of the tile.
template <typename T, int KB>
__device__ __forceinline__ void mn_issue(const void* origin, const uint32_t (&off)[Geo<KB>::kIssue],
                                         int records, uint32_t zero_cols, char* lds, int wave,
                                         int lane, int q0 = 0, int q1 = Geo<KB>::kIssue) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(origin, records);
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    if (q < q0 || q >= q1) continue;
    uint32_t o = off[q];
    if (zero_cols) o = ((zero_cols >> (mn_col<T, KB>(wave, q, lane) >> 6)) & 1u) ? kOob : o;
    lds_load16(rs, lds + (wave * Geo<KB>::kIssue + q) * 1024, o);
  }
}

// ---------------------------------------------------------------------------------------
// LDS -> register fragments for one k-group (16 bf16 or 8 fp32 values of K).  A lane
// provides row/column (lane % 32) and half (lane / 32) of the K group.
// ---------------------------------------------------------------------------------------

// K-major: row is the tile row of this lane.
template <typename T, int KB>
__device__ __forceinline__ typename Traits<T>::frag_t frag_k(const char* tile, int row, int g,
                                                             int lane) {
  const int lc = 2 * g + (lane >> 5);
  const int pc = lc ^ ((row / Geo<KB>::kRowsPerWin) % Geo<KB>::kChunks);
  return *(const typename Traits<T>::frag_t*)(tile + row * KB + pc * 16);
}

// MN-major bf16: two transposing reads of 4 x 16 bits.  Within each 16-lane group the
// hardware hands lane j element i of the 4 values addressed by lane 4 * i + j / 4, so lane s
// of a group addresses k row (base + s / 4) at columns 4 * (s % 4) .. + 3 of its 16 columns.
__device__ __forceinline__ bf16x8_t frag_mn_bf16(const char* tile, int col0, int g, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int col = col0 + 16 * (q & 1) + 4 * (j & 3);
  const int pc = (col >> 3) ^ (4 * (j >> 2));
  const int r0 = 16 * g + 8 * (q >> 1) + (j >> 2);
  const char* p0 = tile + r0 * 512 + pc * 16 + (col & 7) * 2;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + 4 * 512));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// MN-major fp32: element i of the fragment is k = 8 g + 4 (lane / 32) + i, column lane % 32.
__device__ __forceinline__ f32x4_t frag_mn_f32(const char* tile, int col0, int g, int lane) {
  const int col = col0 + (lane & 31);
  f32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * g + 4 * (lane >> 5) + i;
    const int pc = (col >> 2) ^ (4 * (r & 3));
    v[i] = *(const float*)(tile + r * 1024 + pc * 16 + (col & 3) * 4);
  }
  return v;
}

template <typename T, int KB, bool KMAJOR>
__device__ __forceinline__ typename Traits<T>::frag_t frag(const char* tile, int blk0, int g,
                                                           int lane) {
  if constexpr (KMAJOR) {
    return frag_k<T, KB>(tile, blk0 + (lane & 31), g, lane);
  } else if constexpr (sizeof(T) == 2) {
    return frag_mn_bf16(tile, blk0, g, lane);
  } else {
    return frag_mn_f32(tile, blk0, g, lane);
  }
}

__device__ __forceinline__ void mma(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16_t& acc, const f32x4_t& a, const f32x4_t& b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
}

// One stage of MFMAs for this wave: KB / 32 k-groups x 4 x 4 blocks.  Before the MFMAs of
// k-group g it reads the fragments of group g + 1 from LDS and calls part(g), which issues
// slice g of a later stage's direct-to-LDS loads; spreading the loads over the stage keeps
// the address units from stalling the MFMA issue.  The scheduling barriers keep the compiler
// from regrouping the reads, loads and MFMAs.
struct NoIssue {
  __device__ __forceinline__ void operator()(int) const {}
};

template <typename T, int KB, bool AK, bool BK, typename Part = NoIssue>
__device__ __forceinline__ void compute_stage(const char* As, const char* Bs,
                                              f32x16_t (&acc)[4][4], int wm, int wn, int lane,
                                              Part&& part = Part()) {
  typedef typename Traits<T>::frag_t F;
  F a[2][4], b[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[0][i] = frag<T, KB, AK>(As, 128 * wm + 32 * i, 0, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[0][i] = frag<T, KB, BK>(Bs, 128 * wn + 32 * i, 0, lane);
#pragma unroll
  for (int g = 0; g < Geo<KB>::kGroups; ++g) {
    const int c = g & 1, n = c ^ 1;
    if (g + 1 < Geo<KB>::kGroups) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[n][i] = frag<T, KB, AK>(As, 128 * wm + 32 * i, g + 1, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) b[n][i] = frag<T, KB, BK>(Bs, 128 * wn + 32 * i, g + 1, lane);
    }
    part(g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) mma(acc[mi][ni], a[c][mi], b[c][ni]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// s_waitcnt vmcnt(n) for a compile-time n (expcnt, lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS buffers of a pipeline of NST stages: NST distinct objects per operand, so the compiler
// can tell that the direct-to-LDS loads of one stage never touch the buffers being read.
template <int NST>
struct Bufs {
  char* a[NST];
  char* b[NST];
};

// Waits until at most `keep` stages of loads (of this wave) are still in flight.
template <int KB, int NST>
__device__ __forceinline__ void wait_stages(int keep) {
  constexpr int I = 2 * Geo<KB>::kIssue;   // instructions per stage (both operands)
  if (NST >= 4 && keep >= 2) {
    wait_vmcnt<(NST >= 4 ? 2 : 0) * I>();
  } else if (NST >= 3 && keep >= 1) {
    wait_vmcnt<(NST >= 3 ? 1 : 0) * I>();
  } else {
    wait_vmcnt<0>();
  }
}

// Workgroup barrier between pipeline stages.  Each wave has already waited (vmcnt) for its
// own direct-to-LDS loads of the stage about to be read, and every LDS read of the buffer about
// to be refilled has been consumed by an MFMA, so no memory fence is needed: __syncthreads()
// would add one that waits for ALL outstanding loads, including the prefetched stages.  The
// empty asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Software pipeline over stages [base, base + n) of a stream of `total` stages; base and n
// are multiples of NST, so stage g lives in buffer g % NST.  Stages base .. base + NST - 2
// must already be issued (run_prologue); while stage g is computed, the loads of stages
// g + 1 .. g + NST - 1 are in flight.  Issuing continues into the next tile of the stream.
// issue(g) prepares stage g and returns st with st(a, b, p) starting slice p of its loads
// into LDS buffers (a, b); the slices p = 0 .. KB / 32 - 1 together cover both operands.
template <typename T, int KB, int NST, bool AK, bool BK, typename Issue>
__device__ __forceinline__ void run_stream(int base, int n, int total, Issue&& issue,
                                           const Bufs<NST>& B, f32x16_t (&acc)[4][4], int wm,
                                           int wn, int lane) {
  constexpr int P = NST - 1;   // prefetch distance
  for (int j = 0; j < n; j += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int g = base + j + u;
      // stages issued after g: g + 1 .. min(g + P - 1, total - 1)
      const int ahead = min(P - 1, total - 1 - g);
      wait_stages<KB, NST>(ahead);
      stage_barrier();
      const bool more = g + P < total;
      char* const na = B.a[(u + P) % NST];
      char* const nb = B.b[(u + P) % NST];
      const auto st = issue(more ? g + P : g);   // per-stage address setup, once
      compute_stage<T, KB, AK, BK>(B.a[u], B.b[u], acc, wm, wn, lane, [&](int p) {
        if (more) st(na, nb, p);
      });
    }
  }
}

// Issues the first NST - 1 stages of a stream (fewer if the stream is shorter).
template <int KB, int NST, typename Issue>
__device__ __forceinline__ void run_prologue(int total, Issue&& issue, const Bufs<NST>& B) {
#pragma unroll
  for (int u = 0; u < NST - 1; ++u)
    if (u < total) {
      const auto st = issue(u);
#pragma unroll
      for (int p = 0; p < Geo<KB>::kGroups; ++p) st(B.a[u], B.b[u], p);
    }
}

// Slice p of a stage covers instructions [p * kPer, (p + 1) * kPer) of each operand.
template <int KB>
struct Slices {
  static constexpr int kPer = Geo<KB>::kIssue / Geo<KB>::kGroups;   // = 2
};

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Row of accumulator register r (0..15) of a 32 x 32 block for this lane.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8).
// Renumber so that each XCD receives a contiguous range of logical work items, which then
// share operand tiles through that XCD's L2.  nblocks must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

// Logical item -> (row tile, column tile) in super-blocks of 4 x 8 tiles, so the 32
// workgroups an XCD runs at once read 4 + 8 distinct operand tiles.
__device__ __forceinline__ void grouped_tile(int lin, int cols, int& r, int& c) {
  const int sb_cols = (cols + 7) >> 3;
  const int sb = lin >> 5, w = lin & 31;
  r = (sb / sb_cols) * 4 + (w >> 3);
  c = (sb % sb_cols) * 8 + (w & 7);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace cce

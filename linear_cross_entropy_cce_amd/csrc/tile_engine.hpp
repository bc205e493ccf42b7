// Tile engine for the Cut Cross-Entropy kernels on gfx950 (MI355X, CDNA4).
//
// Every hot kernel of the library is a 256 x 256 output tile of a matrix product
// acc[m][n] = sum_k A[m][k] B[n][k] computed by one workgroup of 512 threads (8 waves of 64,
// two per SIMD, so one wave's MFMAs cover the other's LDS, barrier and load waits):
//   * wave w owns rows 128 (w / 4) .. + 127 and columns 64 (w % 4) .. + 63 as 4 x 2 blocks of
//     32 x 32 fp32 accumulators (v_mfma_f32_32x32x16_bf16 for bf16 operands,
//     v_mfma_f32_32x32x2f32 for fp32);
//   * operands stream HBM -> LDS with direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds),
//     one stage of KB bytes of K per operand row, NST stages in NST separate LDS objects so the
//     loads of later stages overlap the MFMAs of the current one;
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
typedef __attribute__((address_space(3))) char lds_char_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 256;           // tile rows (M) and columns (N)
constexpr int kWaveM = 128;          // rows of a wave's accumulator tile
constexpr int kWaveN = 64;           // columns of a wave's accumulator tile
constexpr int kMB = kWaveM / 32;     // 32 x 32 blocks per wave along M
constexpr int kNB = kWaveN / 32;     // ... along N
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef f32x16_t Acc[kMB][kNB];

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
  static constexpr int kEpc = 8;     // elements per 16-byte chunk
  typedef bf16x8_t frag_t;
};
template <> struct Traits<float> {
  static constexpr int kEpc = 4;
  typedef f32x4_t frag_t;
};

// Wave index as a scalar (uniform) value, and the wave's place in the tile.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
__device__ __forceinline__ int wave_m(int wave) { return wave >> 2; }
__device__ __forceinline__ int wave_n(int wave) { return wave & 3; }

// s_waitcnt vmcnt(n) for a compile-time n (expcnt, lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ---------------------------------------------------------------------------------------
// HBM -> LDS stage loads with buffer_load ... lds.  One instruction moves 64 lanes x 16 bytes
// into 1 KB of consecutive LDS.  Every lane keeps a fixed byte offset per instruction relative
// to a tile origin (a uniform pointer turned into a buffer descriptor); masked lanes use an
// offset past the descriptor's range, which the hardware answers with zeros.  The XOR
// swizzles make the fragment reads below free of bank conflicts: a lane picks which global
// chunk lands in its fixed LDS slot.
// ---------------------------------------------------------------------------------------
constexpr uint32_t kOob = 0x80000000u;         // offset answered with zeros

// Buffer descriptor (V#) of a raw buffer: base address (48 bits, stride 0), byte range, and the
// same format word as the compiler's buffer-resource builtin.  Base and range are
// workgroup-uniform; readfirstlane states it, so the descriptor always lives in scalar
// registers.
typedef i32x4_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* p, int records) {
  const uint64_t a = (uint64_t)p;
  Rsrc w;
  w.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  w.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  w.z = __builtin_amdgcn_readfirstlane(records);
  w.w = 0x00020000;
  return w;
}

// One direct-to-LDS load: 64 lanes x 16 bytes from rsrc at voff + soff into LDS at lds (+ 16
// bytes per lane).  Written as inline asm: the compiler then does not know that the
// instruction writes LDS, so it adds no wait for it before later LDS reads of other buffers
// (it cannot tell the transposing reads apart from the buffer being filled).  The pipeline
// waits for these loads itself (wait_stages before the barrier of the stage that reads them).
// No register receives data, so no register can be reused while the load is in flight.
// The LDS destination goes in through M0, named as an input operand ("{m0}"): the compiler
// writes M0 itself before the statement and knows that the statement leaves it unchanged, so
// M0 is never clobbered behind its back.  The s_nop is the wait state the hardware needs
// between a write of M0 and an LDS-DMA load that reads it.
__device__ __forceinline__ void lds_load16(Rsrc rs, char* lds, uint32_t voff, uint32_t soff) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_char_t*)lds;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane((int)la))
               : "memory");
}

// Stage geometry.  KB = bytes of K per K-major operand row per stage (128 or 64): one
// operand's share of a stage is 256 x KB bytes = KB / 4 instructions of 1 KB, KB / 32 per wave.
template <int KB>
struct Geo {
  static_assert(KB == 128 || KB == 64, "stage K bytes");
  static constexpr int kChunks = KB / 16;                 // 16-byte chunks per K-major row
  static constexpr int kIssue = 256 * KB / 1024 / kWaves; // instructions per wave per operand
  static constexpr int kRowsPerWin = 256 / KB;            // K-major rows per 256-byte window
  static constexpr int kOpBytes = 256 * KB;               // one operand's share of one stage
  static constexpr int kGroups = KB / 32;                 // MFMA k-groups per stage
};

// K-major operand: 256 rows x KB bytes per stage.  LDS slot (row r, chunk pc) holds logical K
// chunk pc ^ f(r), f(r) = (r / rows-per-window) mod chunks, which spreads the 16 rows read by
// one quarter-wave over distinct banks.  Instruction q of wave w fills rows
// (w * I + q) * (1024 / KB) onwards (I instructions per wave), so wave w covers the 32 rows
// 32 w .. 32 w + 31.
template <int KB>
__device__ __forceinline__ int kmajor_row(int wave, int q, int lane) {
  return (wave * Geo<KB>::kIssue + q) * (1024 / KB) + lane / Geo<KB>::kChunks;
}
template <int KB>
__device__ __forceinline__ int kmajor_chunk(int r, int lane) {
  return (lane % Geo<KB>::kChunks) ^ ((r / Geo<KB>::kRowsPerWin) % Geo<KB>::kChunks);
}

// Offsets of this lane's chunks relative to the tile origin (row0, k0).  Rows past the
// operand's end are cut off by the descriptor range (kmajor_rsrc), not here.
template <int KB>
__device__ __forceinline__ void kmajor_offsets(uint32_t (&off)[Geo<KB>::kIssue], int64_t ld_bytes,
                                               int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    const int r = kmajor_row<KB>(wave, q, lane);
    off[q] = (uint32_t)(r * ld_bytes) + 16u * kmajor_chunk<KB>(r, lane);
  }
}

// Descriptor of a K-major operand tile whose first row (at K = 0) is `origin`, with rows_left
// rows of the operand from there: its range ends with the tile's last valid row, so later
// rows load as zeros.  Stages step through K with the scalar offset of the loads, which
// leaves the row test unchanged (a chunk never reaches past its own row).
__device__ __forceinline__ Rsrc kmajor_rsrc(const void* origin, int rows_left,
                                                              int ld_bytes) {
  const int rows = rows_left < kTile ? rows_left : kTile;   // min, multiply, max (no med3)
  const int rec = rows * ld_bytes;
  return make_rsrc(origin, rec > 0 ? rec : 0);
}

// Instructions [q0, q1) of this wave's share of a stage at byte offset soff along K.
// k_chunks = valid 16-byte K chunks left from the stage's K origin (>= chunks per row: full).
template <int KB>
__device__ __forceinline__ void kmajor_issue(Rsrc rs,
                                             const uint32_t (&off)[Geo<KB>::kIssue],
                                             uint32_t soff, int k_chunks, char* lds, int wave,
                                             int lane, int q0 = 0, int q1 = Geo<KB>::kIssue) {
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    if (q < q0 || q >= q1) continue;
    uint32_t o = off[q];
    if (k_chunks < Geo<KB>::kChunks)
      o = kmajor_chunk<KB>(kmajor_row<KB>(wave, q, lane), lane) < k_chunks ? o : kOob;
    lds_load16(rs, lds + (wave * Geo<KB>::kIssue + q) * 1024, o, soff);
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

// Descriptor of one MN-major stage whose origin (row k0, column col0) is `origin`, with
// rows_left rows of the operand from k0 and col0 at byte col0_bytes of its row: the range ends
// with the stage's last valid row.
template <typename T, int KB>
__device__ __forceinline__ Rsrc mn_rsrc(const void* origin, int rows_left,
                                                          int ld_bytes, int col0_bytes) {
  constexpr int R = KB / (int)sizeof(T);
  // min, multiply, then max (a clamp of the row count would become a vector med3 and pull the
  // rest of the arithmetic onto the VALU); a negative row count gives a negative, then empty,
  // range
  const int rows = rows_left < R ? rows_left : R;
  const int rec = rows * ld_bytes - col0_bytes;
  return make_rsrc(origin, rec > 0 ? rec : 0);
}

// Instructions [q0, q1).  zero_cols bit b = load zeros for columns 64 b .. 64 b + 63.
template <typename T, int KB>
__device__ __forceinline__ void mn_issue(Rsrc rs,
                                         const uint32_t (&off)[Geo<KB>::kIssue],
                                         uint32_t zero_cols, char* lds, int wave, int lane,
                                         int q0 = 0, int q1 = Geo<KB>::kIssue) {
#pragma unroll
  for (int q = 0; q < Geo<KB>::kIssue; ++q) {
    if (q < q0 || q >= q1) continue;
    uint32_t o = off[q];
    if (zero_cols) o = ((zero_cols >> (mn_col<T, KB>(wave, q, lane) >> 6)) & 1u) ? kOob : o;
    lds_load16(rs, lds + (wave * Geo<KB>::kIssue + q) * 1024, o, 0u);
  }
}

// The loads of one stage: fa(lds, q0, q1) / fb(lds, q0, q1) issue instructions [q0, q1) of
// operand A / B into the given LDS buffer.
template <int KB, typename FA, typename FB>
struct StageIssue {
  FA fa;
  FB fb;
  __device__ __forceinline__ void operator()(char* a, char* b, int q0, int q1) const {
    fa(a, q0, q1);
    fb(b, q0, q1);
  }
  // instruction j of the stage's 2 x I: those of operand A first
  __device__ __forceinline__ void one(char* a, char* b, int j) const {
    constexpr int I = Geo<KB>::kIssue;
    if (j < I)
      fa(a, j, j + 1);
    else
      fb(b, j - I, j - I + 1);
  }
};
template <int KB, typename FA, typename FB>
__device__ __forceinline__ StageIssue<KB, FA, FB> stage_issue(FA fa, FB fb) {
  return StageIssue<KB, FA, FB>{fa, fb};
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
// The same products into a fresh accumulator: the MFMA's C operand is the constant 0, so the
// accumulator needs no clearing before its first k-group.
__device__ __forceinline__ void mma_fresh(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, f32x16_t{}, 0, 0, 0);
}
__device__ __forceinline__ void mma_fresh(f32x16_t& acc, const f32x4_t& a, const f32x4_t& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], f32x16_t{}, 0, 0, 0);
#pragma unroll
  for (int i = 1; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
}

// Pins an accumulator in the instruction order.  MFMA builtins have no side effects, so the
// code generator may move them across loads and barriers; an (empty) volatile asm statement
// that reads and writes the accumulator cannot move relative to other side effects, and the
// MFMAs that produce or consume the accumulator stay on their side of it.
__device__ __forceinline__ void pin(f32x16_t& acc) { asm volatile("" : "+v"(acc)); }

// Fragments of two k-groups (slots 0 and 1: group g of a stage lives in slot g % 2).
template <typename T>
struct Frags {
  typename Traits<T>::frag_t a[2][kMB], b[2][kNB];
};

// The MFMAs of one k-group held in slot `slot`.
template <typename T>
__device__ __forceinline__ void mma_group(Acc& acc, const Frags<T>& f, int slot) {
#pragma unroll
  for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) mma(acc[mi][ni], f.a[slot][mi], f.b[slot][ni]);
}

// One stage of MFMAs for this wave: KB / 32 k-groups x 4 x 2 blocks, with the last k-group
// carried into the next stage.  Right after the stage's barrier nothing in LDS has been read
// yet, so the wave starts with the previous stage's last k-group, whose fragments are already
// in registers (slot 1), while the first fragments of this stage arrive.  Those 8 MFMAs also
// carry the loads of a later stage, one after each, so the address units never stall the MFMA
// issue and the loads get the rest of the stage to land; the later stage's addresses
// (part.make(): descriptors, list lookups) are worked out after the first of them has issued.
// Then groups 0 .. G - 2 of this stage run, each while the next group's fragments are read;
// the last group's fragments are read during group G - 2 and waited for before the stage ends,
// so every read of this stage's LDS buffers is complete at the next barrier (other waves then
// refill them).  Scheduling barriers and the accumulator pins keep this order.  A stream starts
// with zero fragments in slot 1 and ends with flush_carried().
//
// first (uniform; set only for the stage that opens a FRESH stream): there is no carried
// k-group; its MFMA slots multiply zero fragments into C = 0, which defines the accumulators,
// so nothing has to clear them (or the carried fragments) beforehand.  The two variants of the
// carried slots sit behind one uniform branch per stage.
template <typename T, int KB, bool AK, bool BK, typename Part>
__device__ __forceinline__ void compute_stage(const char* As, const char* Bs, Acc& acc,
                                              Frags<T>& f, int wm, int wn, int lane,
                                              const Part& part, bool first = false) {
  constexpr int G = Geo<KB>::kGroups;
  static_assert(G % 2 == 0, "the last k-group of a stage lives in slot 1");
  auto read = [&](int slot, int g) {
#pragma unroll
    for (int i = 0; i < kMB; ++i)
      f.a[slot][i] = frag<T, KB, AK>(As, kWaveM * wm + 32 * i, g, lane);
#pragma unroll
    for (int i = 0; i < kNB; ++i)
      f.b[slot][i] = frag<T, KB, BK>(Bs, kWaveN * wn + 32 * i, g, lane);
  };
  read(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  // the carried k-group: MFMA j, then load j; the pins keep MFMA j after load j - 1 and before
  // load j.  In the first stage of a fresh stream the same slots hold 0 x 0 + 0 products,
  // which define the accumulators.
  auto carried = [&](const bool fresh) {
    typename Traits<T>::frag_t z{};
    auto one = [&](int mi, int ni) {
      if (fresh) {
        asm volatile("" : "+v"(z));   // eight distinct products: no common subexpression
        mma_fresh(acc[mi][ni], z, z);
      } else {
        pin(acc[mi][ni]);
        mma(acc[mi][ni], f.a[1][mi], f.b[1][ni]);
      }
      pin(acc[mi][ni]);
    };
    one(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    const auto st = part.make();
#pragma unroll
    for (int j = 0; j < kMB * kNB; ++j) {
      if (j > 0) one(j / kNB, j % kNB);
      part.one(st, j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (first)
    carried(true);
  else
    carried(false);
#pragma unroll
  for (int g = 0; g + 1 < G; ++g) {
    read((g + 1) & 1, g + 1);
    mma_group(acc, f, g & 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the last group's fragments are in registers before the stage ends
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  // every MFMA issued so far before whatever follows (the next stage's wait and barrier)
#pragma unroll
  for (int mi = 0; mi < kMB; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNB; ++ni) pin(acc[mi][ni]);
}

// Start and end of a stream of compute stages: no carried k-group yet (zero fragments add
// nothing), and the last stage's carried k-group.
template <typename T>
__device__ __forceinline__ void clear_carried(Frags<T>& f) {
#pragma unroll
  for (int i = 0; i < kMB; ++i) f.a[1][i] = typename Traits<T>::frag_t{};
#pragma unroll
  for (int i = 0; i < kNB; ++i) f.b[1][i] = typename Traits<T>::frag_t{};
}
template <typename T>
__device__ __forceinline__ void flush_carried(Acc& acc, const Frags<T>& f) {
  mma_group(acc, f, 1);
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

// LDS buffers of a pipeline of NST stages: NST distinct objects per operand, so the compiler
// can tell that the direct-to-LDS loads of one stage never touch the buffers being read.
template <int NST>
struct Bufs {
  char* a[NST];
  char* b[NST];
};

// Waits until at most `keep` stages of this wave's loads are still in flight.
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

// Loads of one later stage, spread over the MFMAs of the current one (compute_stage):
// make() prepares the stage (issue(i)), one(st, j) issues its j-th load.
template <int KB, typename Issue>
struct StagePart {
  Issue& issue;
  int i;
  char* na;
  char* nb;
  __device__ __forceinline__ auto make() const { return issue(i); }
  template <typename St>
  __device__ __forceinline__ void one(const St& st, int j) const {
    if (j < 2 * Geo<KB>::kIssue) st.one(na, nb, j);
  }
};

// One round of NST stages g0 .. g0 + NST - 1 (stage g0 + u in buffer u).  Every stage issues
// the loads of stage g + P (P = NST - 1) into the buffer freed by stage g - 1; past the end of
// the stream issue() hands out empty descriptors, so those loads only fill zeros.  (A branch
// around them would split the MFMA sequence, and a separate copy of the last round costs
// the register allocator a second live copy of the accumulators.)
template <typename T, int KB, int NST, bool AK, bool BK, typename Issue>
__device__ __forceinline__ void run_round(int g0, Issue& issue, const Bufs<NST>& B, Acc& acc,
                                          Frags<T>& f, int wm, int wn, int lane,
                                          bool first = false) {
  constexpr int P = NST - 1;   // prefetch distance
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    // stage g0 + u has landed once at most P - 1 later stages are still in flight
    wait_stages<KB, NST>(P - 1);
    stage_barrier();
    const StagePart<KB, Issue> part{issue, g0 + u + P, B.a[(u + P) % NST], B.b[(u + P) % NST]};
    compute_stage<T, KB, AK, BK>(B.a[u], B.b[u], acc, f, wm, wn, lane, part, first && u == 0);
  }
}

// Software pipeline over stages [base, base + n) of a stream of `total` stages; base and n
// are multiples of NST, so stage g lives in buffer g % NST.  Stages base .. base + NST - 2
// must already be issued (run_prologue); while stage g is computed, the loads of stages
// g + 1 .. g + NST - 1 are in flight.  Issuing continues into the next tile of the stream.
// issue(g) prepares stage g (for g >= total: loads of zeros) and returns a StageIssue for it.
// At the end of the stream the zero loads are waited for, so no load into LDS is left in
// flight.
// FRESH: the stream defines the accumulators (their previous contents are ignored); it then
// needs n >= NST.  Otherwise it adds to them.
template <typename T, int KB, int NST, bool AK, bool BK, bool FRESH = false, typename Issue>
__device__ __forceinline__ void run_stream(int base, int n, int total, Issue&& issue,
                                           const Bufs<NST>& B, Acc& acc, int wm, int wn,
                                           int lane) {
  Frags<T> f;
  if constexpr (!FRESH) clear_carried(f);
  for (int g0 = base; g0 < base + n; g0 += NST)
    run_round<T, KB, NST, AK, BK>(g0, issue, B, acc, f, wm, wn, lane, FRESH && g0 == base);
  flush_carried(acc, f);
  if (base + n >= total) wait_vmcnt<0>();
}

// The same pipeline for a wave that has no MFMAs in stages [base, base + n): it issues its share
// of the loads and keeps the waits and barriers of the waves that compute.
template <int KB, int NST, typename Issue>
__device__ __forceinline__ void run_stream_idle(int base, int n, int total, Issue&& issue,
                                                const Bufs<NST>& B) {
  constexpr int P = NST - 1;
  for (int g0 = base; g0 < base + n; g0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      wait_stages<KB, NST>(P - 1);
      stage_barrier();
      const auto st = issue(g0 + u + P);
      st(B.a[(u + P) % NST], B.b[(u + P) % NST], 0, Geo<KB>::kIssue);
    }
  }
  if (base + n >= total) wait_vmcnt<0>();
}

// Issues the first NST - 1 stages of a stream (fewer if the stream is shorter).
template <int KB, int NST, typename Issue>
__device__ __forceinline__ void run_prologue(int total, Issue&& issue, const Bufs<NST>& B) {
#pragma unroll
  for (int u = 0; u < NST - 1; ++u)
    if (u < total) {
      const auto st = issue(u);
      st(B.a[u], B.b[u], 0, Geo<KB>::kIssue);
    }
}

// A stage list in three segments (lengths seg[0..2], multiples of NST): stages where only rows
// 0..127 of the tile's A operand are live, stages where both halves are, stages where only
// rows 128..255 are.  The waves of rows 0..127 (wm = 0) compute the first two segments, those
// of rows 128..255 the last two: their rows of A are all zero in the other segment.  A wave
// outside its range issues its loads and keeps the barriers, so its SIMD partner of the other
// half runs alone.  Each wave runs one compute loop over one contiguous range.
template <typename T, int KB, int NST, bool AK, bool BK, typename Issue>
__device__ __forceinline__ void run_segments(const int (&seg)[3], Issue&& issue,
                                             const Bufs<NST>& B, Acc& acc, int wm, int wn,
                                             int lane) {
  const int total = seg[0] + seg[1] + seg[2];
  if (total == 0) return;
  const int c0 = wm == 0 ? 0 : seg[0];
  const int c1 = wm == 0 ? seg[0] + seg[1] : total;
  run_prologue<KB, NST>(total, issue, B);
  run_stream_idle<KB, NST>(0, c0, total, issue, B);
  run_stream<T, KB, NST, AK, BK>(c0, c1 - c0, total, issue, B, acc, wm, wn, lane);
  run_stream_idle<KB, NST>(c1, total - c1, total, issue, B);
}

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < kMB; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Row of accumulator register r (0..15) of a 32 x 32 block for this lane.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
// The same split into a compile-time part (block mi of the wave's rows, register r) and a
// per-lane part: row within the wave's 128 rows = acc_row_c(mi, r) + acc_row_l(lane).  Tests
// against a row bound then compare a constant with one per-lane value, instead of keeping
// 64 row indices per lane alive.
__host__ __device__ constexpr int acc_row_c(int mi, int r) {
  return 32 * mi + 8 * (r >> 2) + (r & 3);
}
__device__ __forceinline__ int acc_row_l(int lane) { return 4 * (lane >> 5); }

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8).
// Renumber so that each XCD receives a contiguous range of logical work items, which then
// share operand tiles through that XCD's L2.  nblocks must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

// Logical item -> (row tile, column tile) of a rows x cols tile grid, in super-blocks of up to
// 4 x 8 tiles (narrower or shorter at the right and bottom edges), so the 32 workgroups an XCD
// runs at once read about 4 + 8 distinct operand tiles.  Items are numbered row group by row
// group and, within one, column group by column group; exactly rows x cols items are valid
// (lin >= rows x cols gives r >= rows).
__device__ __forceinline__ void grouped_tile(int lin, int rows, int cols, int& r, int& c) {
  const int rg = lin / (4 * cols);
  const int hr = min(4, rows - 4 * rg);
  if (hr <= 0) { r = rows; c = 0; return; }
  int w = lin - rg * 4 * cols;
  const int cg = w / (hr * 8);
  const int wc = min(8, cols - 8 * cg);
  w -= cg * hr * 8;
  r = 4 * rg + w / wc;
  c = 8 * cg + w % wc;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace cce

// Device-side building blocks shared by the forward, backward and decode
// kernels: fragment types, the MFMA wrappers for gfx950 (32x32 products, and
// 16x16x32 ones for row sums), operand loads, the LDS key permutation and
// transpose reads, buffer-to-LDS copies, barriers, output staging through LDS
// and the workgroup -> (head, tile) mapping.
//
// MFMA conventions (v_mfma_f32_32x32x16_{bf16,f16}, v_mfma_f32_32x32x2_f32),
// wave64, lane l, g = l / 32:
//   A operand (32 rows x 16 k): lane l holds row l % 32 and 8 k values of group g;
//   B operand (16 k x 32 cols): lane l holds col l % 32 and 8 k values of group g;
//   C/D (32 x 32 fp32, 16 regs): reg r of lane l is row 8*(r/4) + 4*g + (r%4),
//                                col l % 32.
// Which physical k a (group, slot) pair stands for is irrelevant as long as A
// and B agree, so every kernel picks the k order that lets a C tile be fed back
// as a B operand without moving data between lanes: slot s of group g of a
// 16-wide k step is k = 8*(s/4) + 4*g + (s%4)  (the C row order above).  Tiles
// stored transposed in LDS (contraction index along the row) place that k order
// contiguously per lane, see perm16().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct FragOf;
template <> struct FragOf<bf16_t> { using type = bf16x8; };
template <> struct FragOf<f16_t> { using type = f16x8; };
template <> struct FragOf<float> { using type = f32x8; };
// 8 consecutive k values of one lane: one MFMA operand (two 16-byte halves for fp32).
template <typename T> using frag_t = typename FragOf<T>::type;

// Elements per 16-byte chunk.
template <typename T> constexpr int kEPC = 16 / (int)sizeof(T);

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// fp32: eight k=2 MFMAs, slot s of both groups per instruction.
__device__ __forceinline__ f32x16 mma(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

// Round 8 fp32 values to the operand type (round-to-nearest-even).
template <typename T> __device__ __forceinline__ frag_t<T> to_frag(f32x8 x);
template <> __device__ __forceinline__ bf16x8 to_frag<bf16_t>(f32x8 x) {
  return __builtin_convertvector(x, bf16x8);
}
template <> __device__ __forceinline__ f16x8 to_frag<f16_t>(f32x8 x) {
  return __builtin_convertvector(x, f16x8);
}
template <> __device__ __forceinline__ f32x8 to_frag<float>(f32x8 x) { return x; }

// acc + the sum of the 8 values of an fp32 operand fragment (the 16-bit
// kernels form their sums on the matrix pipe, see rowsum_sel_frag).
__device__ __forceinline__ float frag_sum(f32x8 f, float acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += f[i];
  return acc;
}

// Registers 8h..8h+7 of a 32x32 accumulator.
template <int H> __device__ __forceinline__ f32x8 half8(const f32x16& c) {
  if constexpr (H == 0) return __builtin_shufflevector(c, c, 0, 1, 2, 3, 4, 5, 6, 7);
  else return __builtin_shufflevector(c, c, 8, 9, 10, 11, 12, 13, 14, 15);
}

// Operand load of 8 consecutive elements (16-byte aligned address).
template <typename T> __device__ __forceinline__ frag_t<T> ld_frag(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(frag_t<T>, *reinterpret_cast<const u32x4*>(p));
  } else {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    u32x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag_t<T>, ab);
  }
}

template <typename T> __device__ __forceinline__ frag_t<T> zero_frag() {
  if constexpr (sizeof(T) == 2) return __builtin_bit_cast(frag_t<T>, (u32x4)(0u));
  else return __builtin_bit_cast(frag_t<T>, (u32x8)(0u));
}

// All-ones MFMA operand (16-bit types): ones^T P sums the columns of P.
template <typename T> __device__ __forceinline__ frag_t<T> one_frag() {
  static_assert(sizeof(T) == 2, "16-bit operands only");
  constexpr unsigned one2 = __is_same(T, bf16_t) ? 0x3F803F80u : 0x3C003C00u;
  return __builtin_bit_cast(frag_t<T>, (u32x4)(one2));
}

// Row sums of a P^T fragment (the B operand of the 32x32x16 products: lane l
// holds query l % 32 and 8 keys of group l / 32) on v_mfma_f32_16x16x32, half
// the cycles of an all-ones 32x32x16 product and a 4-register result.  In the
// 16x16x32 layout lane l supplies row l % 16 of A, column l % 16 of B and
// k-segment l / 16 (8 k values) of both; the result's element r of lane l is
// row 4 (l / 16) + r, column l % 16.  Read as a 32-row B operand, column n of
// the fragment holds query n's keys in segments 0 and 2 and query n + 16's in
// segments 1 and 3, so an A with row 0 all ones over segments 0, 2 and row 4
// over segments 1, 3 (zeros elsewhere) leaves query q's sum in element 0 of
// lane q for q < 32, and zeros in lanes 32-63.
template <typename T> __device__ __forceinline__ frag_t<T> rowsum_sel_frag(int lane) {
  return (lane & 15) == 4 * ((lane >> 4) & 1) ? one_frag<T>() : zero_frag<T>();
}
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() { return (f32x16)(0.0f); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maxima of fp32 values as single instructions.  The compiler's fmaxf first
// quiets signalling NaNs (an extra max per input that is not known to be
// canonical, e.g. every MFMA result); scores are never NaN for finite inputs,
// and -inf from masking orders correctly, so the plain instructions suffice.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Max over lanes l and l ^ 32 (the two halves of the wave) with one lane-swap
// instruction instead of an LDS permute: after the swap one copy holds the
// lower half in both halves and the other the upper half.
__device__ __forceinline__ float vmax_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// An empty volatile asm statement: placed first in a rarely taken branch (the
// causal/tail mask), it keeps the compiler from if-converting the branch into
// unconditional selects that every tile would then execute.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }

// Race-check builds (FA_DEBUG_SYNC, a separate library): at every workgroup
// barrier each wave first drains all of its outstanding memory operations —
// buffer-to-LDS copies, loads, LDS accesses — so every copy lands in the phase
// that issues it instead of one or more phases later, and no LDS access is in
// flight across a barrier.  The schedule changes, the arithmetic does not:
// outputs must be bitwise equal to the production build's.
#ifdef FA_DEBUG_SYNC
constexpr bool kDebugSync = true;
#else
constexpr bool kDebugSync = false;
#endif

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses,
// not for its global loads, so register-staged prefetches stay in flight
// across it.  The scheduling fences keep arithmetic on its side of the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kDebugSync) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// Position, inside a transposed LDS row, of contraction index k (k % 4 == 0):
// within each group of 16, the 4-wide chunks 1 and 2 swap places, so that the
// 8 k values slot s = 0..7 of lane group g (k = 8*(s/4) + 4*g + s%4) sit at
// positions 8*g .. 8*g+7 and one 16-byte read fetches them.
__device__ __forceinline__ int perm16(int k) {
  const int c = (k >> 2) & 3;
  const int cs = ((c & 1) << 1) | (c >> 1);
  return (k & ~15) | (cs << 2);
}

// Byte-addressed LDS pointers.  Kernels cast their __shared__ buffer once to
// this address space, so every later access is a plain ds_read/ds_write with
// immediate offsets and no generic-pointer checks.
typedef __attribute__((address_space(3))) char lds_t;

template <typename V> __device__ __forceinline__ V lds_ld(const lds_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) V*>(p);
}
template <typename V> __device__ __forceinline__ void lds_st(lds_t* p, V v) {
  *reinterpret_cast<__attribute__((address_space(3))) V*>(p) = v;
}

// 32 rows of 16-bit outputs held one row per lane, as an MFMA C tile holds
// them (lane l: row l % 32, element 4 rg + e of accumulator db at column
// 32 db + 8 rg + 4 (l / 32) + e), scaled by sc (per lane, i.e. per row) and
// written to rows[0 .. nvalid) (row stride D) through this wave's LDS staging
// rows: each lane writes its row into the staging tile (rows padded by 16 B
// against bank conflicts), then reads back 16 contiguous bytes, so every store
// instruction writes whole rows (D / 8 lanes per row) instead of 8 bytes of
// each of 32 rows.  kStageBytes of LDS per wave, which the caller must not
// be using in any other wave.
template <int D> constexpr int kStageRow = D * 2 + 16;
template <int D> constexpr int kStageBytes = 32 * kStageRow<D>;
template <typename T, int D>
__device__ __forceinline__ void store_rows_lds(lds_t* stg, const f32x16 (&acc)[D / 32], float sc,
                                               T* rows, int nvalid, int lane) {
  static_assert(sizeof(T) == 2, "16-bit outputs");
  constexpr int SROW = kStageRow<D>, LPR = D / 8, RPI = 64 / LPR;
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      T v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (T)(acc[db][4 * rg + e] * sc);
      lds_st<u32x2>(stg + l32 * SROW + (db * 32 + 8 * rg + 4 * g) * 2, __builtin_bit_cast(u32x2, v4));
    }
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / LPR, cc = lane % LPR;
    const u32x4 v = lds_ld<u32x4>(stg + r * SROW + cc * 16);
    if (r < nvalid) *reinterpret_cast<u32x4*>(rows + (size_t)r * D + cc * 8) = v;
  }
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each 16-lane group the
// instruction returns to lane i, as element e, element i % 4 of the 4-element
// vector addressed by lane 4*e + i/4 of the group.  So if lane j of the group
// points at row (k0 + j/4), columns n0 + 4*(j%4) .. +3 of a row-major 16-bit
// matrix X, lane i receives X[k0 + e][n0 + i] for e = 0..3: four consecutive
// rows of one column, i.e. a column fragment of the transposed matrix.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Row-major tile of 16-bit elements in LDS, D per row and no padding, with
// the 16-byte chunks of row r XOR-permuted by swz(r).  The permutation makes
// both access patterns the kernels use conflict-free on a 64-bank LDS:
//  - 16-byte operand reads: 16 consecutive rows at one logical chunk land
//    in 16 distinct chunk slots;
//  - transpose reads: 8 consecutive rows (8-aligned) x 64 bytes spread evenly,
//    two rows per slot (the minimum for 512 bytes).
template <int D> struct SwzTile {
  static_assert(D == 64 || D == 128, "head dimension");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // Byte offset of 16-byte chunk `ch` of row `r`.
  __device__ static __forceinline__ int off(int r, int ch) {
    return r * kRowBytes + ((ch ^ swz(r)) << 4);
  }
  // Per-lane byte offset for the A-operand read of rows R0 + lane%32 (R0 a
  // multiple of 16), k step t (elements 16t + 8g .. +7).
  __device__ static __forceinline__ int a_off(int lane, int t) {
    const int r = lane & 31, g = lane >> 5;
    return off(r, 2 * t + g);
  }
  // Per-lane byte offset for the transpose read that yields, for lane l, the
  // 4 elements X[16u + 8h + 4g + e][32db + l%32], e = 0..3, of a tile X whose
  // rows are the contraction index (g = l/32).  Add 16u * kRowBytes for u.
  __device__ static __forceinline__ int tr_off(int lane, int h, int db) {
    const int j = lane & 15, nh = (lane >> 4) & 1, g = lane >> 5;
    const int r = 8 * h + 4 * g + (j >> 2);
    const int ch = 4 * db + 2 * nh + ((j >> 1) & 1);
    return off(r, ch) + (j & 1) * 8;
  }
};

// One MFMA operand from two LDS transpose reads (rows 16u..16u+7 and
// 16u+8..16u+15 of a tile whose rows are the contraction index).
template <typename T>
__device__ __forceinline__ frag_t<T> tr_frag(const lds_t* p0, const lds_t* p1) {
  const u32x2 lo = lds_read_tr16(p0);
  const u32x2 hi = lds_read_tr16(p1);
  return __builtin_bit_cast(frag_t<T>, (u32x4){lo[0], lo[1], hi[0], hi[1]});
}

// Extract 16-bit element i (0..7) of a 16-byte chunk.
__device__ __forceinline__ unsigned elem16(const u32x4& c, int i) {
  const unsigned w = c[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// Store 4-row x 16-byte block `blk` (rows r..r+3 of a row-major tile, one chunk
// each) transposed: element e of every chunk goes to LDS row (col0 + e) at
// positions perm16(r)..+3 of the contraction index.
template <typename T>
__device__ __forceinline__ void store_transposed_4rows(T* base, int row_stride, int col0, int r,
                                                      const u32x4 (&blk)[4]) {
  const int pos = perm16(r);  // r is a multiple of 4
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 w;
      w[0] = elem16(blk[0], e) | (elem16(blk[1], e) << 16);
      w[1] = elem16(blk[2], e) | (elem16(blk[3], e) << 16);
      *reinterpret_cast<u32x2*>(base + (size_t)(col0 + e) * row_stride + pos) = w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 w = {blk[0][e], blk[1][e], blk[2][e], blk[3][e]};
      *reinterpret_cast<u32x4*>(base + (size_t)(col0 + e) * row_stride + pos) = w;
    }
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer descriptor over `bytes` bytes from `base` (raw, unswizzled; word 3 =
// 32-bit data format, the gfx9 setting for plain loads).  Loads whose offset
// falls past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// The same descriptor as four dwords (for inline assembly).
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  u32x4 r;
  r[0] = (unsigned)b;
  r[1] = (unsigned)(b >> 32) & 0xffffu;
  r[2] = bytes;
  r[3] = 0x00020000u;
  return r;
}

// Copy of 64 lanes x 16 bytes from a buffer straight into LDS: lane i's chunk
// (byte offset voff in the descriptor's range, zeros past its end) lands at
// LDS byte address m0 + 16 i.  Issued from inline assembly, so the compiler
// neither knows of it nor fences LDS reads behind it: the caller waits for it
// (s_waitcnt vmcnt) before the barrier that publishes the data, and before the
// workgroup ends.
__device__ __forceinline__ void dma16(u32x4 rsrc, unsigned m0, int voff) {
  unsigned m0_out;   // M0 as an output operand: the compiler knows it changes
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds"
               : "={m0}"(m0_out) : "s"(m0), "v"(voff), "s"(rsrc) : "memory");
}
// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDebugSync ? 0 : N) : "memory");
}

// The same with 4 bytes per lane (lane i's dword lands at m0 + 4 i).
__device__ __forceinline__ void dma4(u32x4 rsrc, unsigned m0, int voff) {
  unsigned m0_out;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds"
               : "={m0}"(m0_out) : "s"(m0), "v"(voff), "s"(rsrc) : "memory");
}

// Element e of a 16-byte chunk of T, widened to fp32.
template <typename T> __device__ __forceinline__ float chunk_elem(const u32x4& c, int e) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(float, c[e]);
  } else if constexpr (__is_same(T, bf16_t)) {
    return __builtin_bit_cast(float, elem16(c, e) << 16);
  } else {
    return (float)__builtin_bit_cast(f16_t, (unsigned short)elem16(c, e));
  }
}

// Workgroup index -> (batch*head, tile index).  Workgroups are handed to the 8
// XCDs round-robin by index; when B*H is a multiple of 8 every XCD gets a
// contiguous range of heads (so K/V of a head stay in one XCD's L2), and inside
// it tiles are ordered heavy-first when `reverse` (causal: the last query tiles
// see the most keys).
__device__ __forceinline__ void map_block(int w, int ntiles, int BH, bool reverse, int& bh,
                                          int& tile) {
  if ((BH & 7) == 0) {
    const int x = w & 7, s = w >> 3, hpx = BH >> 3;
    bh = x * hpx + s % hpx;
    tile = s / hpx;
  } else {
    bh = w % BH;
    tile = w / BH;
  }
  if (reverse) tile = ntiles - 1 - tile;
}

// Closed-form class of tile (i, j) with Br x Bc tiles: 0 no visible element,
// 1 all visible, 2 partial (| 4 when the tile reaches past n).
__device__ __forceinline__ int tile_code(int i, int j, int br, int bc, int n, bool causal) {
  const int last_row = min((i + 1) * br, n) - 1;
  const int c0 = j * bc;
  if (causal && c0 > last_row) return 0;
  const bool inside = (i + 1) * br <= n && (j + 1) * bc <= n;
  const bool full = inside && (!causal || (j + 1) * bc - 1 <= i * br);
  return full ? 1 : (2 | (inside ? 0 : 4));
}

}  // namespace fa

// Split-K decode: attention of a short block of queries (e.g. one new token)
// against a long key/value cache of Nk keys, with the query heads that share a
// key/value head (grouped-query attention) packed into one block of at most 32
// query rows.
//
// Method: Lecture 9 notes (cs2680.com), section 9.8 — decode attention reads
// the whole cache once for very little arithmetic (about one FLOP per byte in
// 16-bit types), so it is bound by memory bandwidth, and at small batch one
// workgroup per head leaves most of the chip idle; splitting the cache along
// the sequence lets many compute units each reduce over a slice, and a combine
// step merges the slices' partial softmax statistics with the same running-max
// rescaling as section 9.4.  CMU 11-868 FlashAttention notes (quidproquo.cc),
// slide pages 57-60: Flash-Decoding splits along the key/value length so the
// GPU has enough work; the merge is the rescaling identity of slide page 12.
//
// Two kernels:
//   dec_split_kernel   one workgroup per (key/value head, slice); each of its
//                      four waves takes every fourth 32-key tile of the slice
//                      and keeps its own running max m, denominators l (fp32
//                      probabilities) and lq (probabilities as rounded for the
//                      P V product) and unnormalised output; the workgroup
//                      merges the four in LDS and writes one partial per slice
//                      (with a single slice in a whole call: O and LSE, and
//                      the combine is not launched);
//   dec_combine_kernel one workgroup per (key/value head, query row), four
//                      thread groups over the slices' partials: brings every
//                      partial to the common max, adds, divides once.
//
// gfx950 mapping of the split kernel.  The cache is read exactly once, so the
// kernel is a stream: every wave owns a private ring of LDS stages (32 KB per
// wave: two stages of a K and a V tile at d = 128, four at d = 64) filled by
// buffer-to-LDS copies (1 KB per wave instruction, no staging registers), and
// keeps two tiles in flight while it computes; the LDS the rings occupy (128
// KB) bounds the bytes a CU can have in flight.  The loop needs no workgroup
// barrier: a wave only reads what its own copies wrote, after waiting for
// them (the two barriers after the loop serve the merge).  The arithmetic
// reuses the forward's MFMA layout: S^T (32 keys x 32 queries) = K Q^T with
// Q^T held in registers, O^T += V^T P^T with V^T from LDS transpose reads of
// the swizzled row-major V tile; query rows past the block are zero rows
// whose results are never stored.  The g query heads of a key/value group
// fill the 32 query columns of the MFMA tile together (the GQA packing of the
// CMU notes' decoding slides), so each head's cache is read once for all of
// them.  Scores are scaled by c = scale*log2(e) inside the FMA that feeds
// exp2, and the running max only moves when a tile exceeds it by more than 2^8
// (exact: all three accumulators carry the same factor).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {
constexpr float kDecLazyRescale = 8.0f;   // log2 of the largest unnormalised probability
constexpr int kDecWaveLds = 32 * 1024;    // LDS bytes per wave
}  // namespace

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kDecWaves) void dec_split_kernel(DecArgs<T> a) {
  using Tile = SwzTile<D>;
  constexpr int BC = kDecBC;
  constexpr int RB = Tile::kRowBytes;
  constexpr int TB = BC * RB;                 // bytes of one K or V tile
  constexpr int STAGE = 2 * TB;               // K tile, then V tile
  constexpr int NS = kDecWaveLds / STAGE;     // ring depth
  constexpr int SEG = TB / 1024;              // 1 KB copies per tile and tensor
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static_assert(BC == 32 && NS >= 2 && SEG * 1024 == TB, "tile shape");

  __shared__ __attribute__((aligned(16))) char smem[kDecWaves * kDecWaveLds];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  lds_t* const L = (lds_t*)smem + wave * kDecWaveLds;
  const unsigned lds_base = (unsigned)(size_t)L;

  const int split = blockIdx.x % a.splits;
  const int bh = blockIdx.x / a.splits;
  const int Nq = a.Nq, Nk = a.Nk;
  const T* __restrict__ Kh = a.K + (size_t)bh * Nk * D;
  const T* __restrict__ Vh = a.V + (size_t)bh * Nk * D;

  // Tiles of this wave: t_begin + wave + kDecWaves * i, i < nmine.
  const int nT = (Nk + BC - 1) / BC;
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(nT, t_begin + a.tiles_per_split);
  const int first = t_begin + wave;
  const int nmine = first < t_end ? (t_end - first + kDecWaves - 1) / kDecWaves : 0;

  // Q^T operand: lane holds query l32 (zero rows past Nq), d = 16t + 8g .. +7.
  frag_t<T> qf[D / 16];
  {
    const T* qrow = a.Q + ((size_t)bh * Nq + min(l32, Nq - 1)) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = ld_frag(qrow + 16 * t + 8 * g);
      if (l32 >= Nq) qf[t] = zero_frag<T>();
    }
  }
  // Row l32 is query l32 % qlen of its query head, at sequence position
  // Nk - qlen + l32 % qlen (bottom-right alignment).
  const int qlen = a.qlen;
  const int qpos = Nk - qlen + l32 % qlen;

  // Copy of one tile: segment k (1 KB) of it is filled by lane i with physical
  // chunk 64k + i, i.e. row r = (64k + i) / CPR, physical chunk pc, which holds
  // logical chunk pc ^ swz(r) of that row.  The descriptor ends at the tile's
  // last row inside the cache, so rows past Nk arrive as zeros.
  int dma_off[SEG];
#pragma unroll
  for (int k = 0; k < SEG; ++k) {
    const int ci = 64 * k + lane;
    const int r = ci / CPR, pc = ci % CPR;
    dma_off[k] = r * RB + ((pc ^ Tile::swz(r)) << 4);
  }
  auto copy_tile = [&](int i) {
    const int kv0 = (first + kDecWaves * i) * BC;
    const unsigned bytes = (unsigned)(min(Nk - kv0, BC) * RB);
    const unsigned st = lds_base + (unsigned)((i % NS) * STAGE);
    const u32x4 rk = raw_rsrc(Kh + (size_t)kv0 * D, bytes);
    const u32x4 rv = raw_rsrc(Vh + (size_t)kv0 * D, bytes);
#pragma unroll
    for (int k = 0; k < SEG; ++k) dma16(rk, st + k * 1024, dma_off[k]);
#pragma unroll
    for (int k = 0; k < SEG; ++k) dma16(rv, st + TB + k * 1024, dma_off[k]);
  };

  int a_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a_off[t] = Tile::a_off(lane, t);
  int tr_off[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) tr_off[h][db] = Tile::tr_off(lane, h, db);

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = zero16();
  // The rounded-P denominator on 16x16x32 products (rowsum_sel_frag): element 0
  // of lane q < 32 holds query q's sum, lanes 32-63 hold zeros.
  f32x4 osum = {0.f, 0.f, 0.f, 0.f};
  float m = -1e30f;           // running max (log2 units of scaled scores), possibly stale
  float lsum = 0.f;           // this lane's half of the fp32 denominator
  const frag_t<T> rsel = rowsum_sel_frag<T>(lane);
  const float c = a.scale_log2;

#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nmine) copy_tile(i);

  for (int i = 0; i < nmine; ++i) {
    // Refill the stage read in iteration i - 1 (its reads finished there).
    if (i + NS - 1 < nmine) {
      copy_tile(i + NS - 1);
      wait_vmcnt<2 * SEG * (NS - 1)>();   // tile i's copies have landed
    } else {
      wait_vmcnt<0>();
    }
    const lds_t* kb = L + (i % NS) * STAGE;
    const lds_t* vb = kb + TB;
    const int kv0 = (first + kDecWaves * i) * BC;

    frag_t<T> kf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) kf[t] = lds_ld<frag_t<T>>(kb + a_off[t]);
    f32x16 s = zero16();
#pragma unroll
    for (int t = 0; t < D / 16; ++t) s = mma(kf[t], qf[t], s);

    // Keys past the cache, and (causal) keys after the query's position.
    if (kv0 + BC > Nk || (CAUSAL && kv0 + BC - 1 > Nk - qlen)) {
      keep_branch();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= Nk || (CAUSAL && key > qpos)) s[r] = -INFINITY;
      }
    }
    float mx4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mx4[q] = vmax(vmax3(s[q], s[q + 4], s[q + 8]), s[q + 12]);
    const float mc = vmax_halves(vmax(vmax3(mx4[0], mx4[1], mx4[2]), mx4[3])) * c;
    if (__ballot(mc > m + kDecLazyRescale)) {
      const float m_new = fmaxf(m, mc);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
      osum[0] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], c, -m);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r]);
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) rs4[r & 3] += s[r];
    lsum += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);

    // O^T += V^T P^T over the two 16-key steps of the tile.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const frag_t<T> pf = to_frag<T>(u ? half8<1>(s) : half8<0>(s));
      frag_t<T> vf[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        vf[db] = tr_frag<T>(vb + 16 * u * RB + tr_off[0][db], vb + 16 * u * RB + tr_off[1][db]);
      osum = mma16(rsel, pf, osum);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = mma(vf[db], pf, o[db]);
    }
    // Every read of this stage has returned before a later copy refills it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  wait_vmcnt<0>();   // no copy may land after the wave ends

  // Merge the four waves' partials of this slice in LDS (the rings are free
  // once every wave has drained its copies and passed the barrier), then write
  // one partial per slice: with M the largest of the waves' maxima, o, l and lq
  // are the sums of the waves' values times 2^(m_w - M).
  const float ltot = lsum + __shfl_xor(lsum, 32);
  constexpr int OROW = D + 4;                      // padded row of floats
  float* const mo = reinterpret_cast<float*>(smem);            // [waves][32][OROW]
  float* const ms = mo + kDecWaves * 32 * OROW;                // [waves][32][4]
  __syncthreads();
  {
    float* mw = mo + (wave * 32 + l32) * OROW;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<f32x4*>(mw + 32 * db + 8 * rg + 4 * g) =
            (f32x4){o[db][4 * rg], o[db][4 * rg + 1], o[db][4 * rg + 2], o[db][4 * rg + 3]};
    // Queries q and q + 16 share a column of the row-sum products, whose zero
    // selector entries still multiply the other query's probabilities: a NaN
    // there (a NaN input in that row) makes this sum NaN as well.  The query's
    // own fp32 sum is then finite and stands in for it (the two differ only by
    // the rounding of P); a NaN of the query's own leaves both NaN.
    const float lq = __builtin_isnan(osum[0]) && !__builtin_isnan(ltot) ? ltot : osum[0];
    if (g == 0)
      *reinterpret_cast<f32x4*>(ms + (wave * 32 + l32) * 4) = (f32x4){m, ltot, lq, 0.f};
  }
  __syncthreads();
  const size_t prow0 = ((size_t)bh * a.splits + split) * Nq;   // this slice's partial rows
  for (int idx = threadIdx.x; idx < Nq * D; idx += 64 * kDecWaves) {
    const int r = idx / D, col = idx - r * D;
    f32x4 st[kDecWaves];
    float M = -1e30f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      st[w] = *reinterpret_cast<const f32x4*>(ms + (w * 32 + r) * 4);
      M = fmaxf(M, st[w][0]);
    }
    float acc = 0.f, l = 0.f, lq = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float wt = fast_exp2(st[w][0] - M);
      acc += wt * mo[(w * 32 + r) * OROW + col];
      l += wt * st[w][1];
      lq += wt * st[w][2];
    }
    if (a.direct) {
      // The only slice: finish here (what the combine does with one partial,
      // whose weight is exactly 1).
      a.O[(prow0 + r) * D + col] = (T)(acc / lq);
      if (col == 0) a.LSE[prow0 + r] = (M + __builtin_log2f(l)) * kLn2;
    } else {
      a.part_o[(prow0 + r) * D + col] = acc;
      if (col == 0) *reinterpret_cast<f32x4*>(a.part_s + (prow0 + r) * 4) = (f32x4){M, l, lq, 0.f};
    }
  }
}

// Merge of the partials of one (key/value head, query row).  With M the largest
// partial max: O = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) lq_p,
// LSE = ln 2 * (M + log2 sum_p 2^(m_p - M) l_p).  A partial that saw no
// visible key has m_p = -1e30 and weight exactly zero.  The block is kDecCombineGroups
// groups of D threads; thread x of group j owns column x of the partials
// p = j, j + groups, ...  The statistics are first loaded by all threads into LDS
// (one round of loads, not a chain), the partial outputs eight at a time per
// thread so their loads overlap; the groups' sums are added through LDS.
template <typename T, int D>
__global__ __launch_bounds__(D * kDecCombineGroups) void dec_combine_kernel(DecArgs<T> a) {
  constexpr int NG = kDecCombineGroups, NT = D * NG;
  __shared__ f32x4 st_s[kDecMaxPartials];
  __shared__ float red[NT / 64];
  __shared__ float part[3][NG][D];
  const int t = threadIdx.x, col = t % D, grp = t / D;
  const int row = blockIdx.x;               // bh * Nq + query row
  const int bh = row / a.Nq, q = row - bh * a.Nq;
  const int P = a.splits;
  const size_t base = (size_t)bh * P * a.Nq + q;   // partial p's row: base + p * Nq
  const f32x4* ps = reinterpret_cast<const f32x4*>(a.part_s);
  float mloc = -1e30f;
  for (int p = t; p < P; p += NT) {
    const f32x4 v = ps[base + (size_t)p * a.Nq];
    st_s[p] = v;
    mloc = fmaxf(mloc, v[0]);
  }
  // Block-wide max: within each wave, then across the waves through LDS.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if ((t & 63) == 0) red[t >> 6] = mloc;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) M = fmaxf(M, red[w]);

  float acc = 0.f, den = 0.f, lsum = 0.f;
  const float* po = a.part_o + base * D + col;
  const size_t pstride = (size_t)a.Nq * D;
  int p = grp;
  for (; p + 7 * NG < P; p += 8 * NG) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = po[(size_t)(p + u * NG) * pstride];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const f32x4 sv = st_s[p + u * NG];
      const float w = fast_exp2(sv[0] - M);
      acc += w * x[u];
      lsum += w * sv[1];
      den += w * sv[2];
    }
  }
  for (; p < P; p += NG) {
    const f32x4 sv = st_s[p];
    const float w = fast_exp2(sv[0] - M);
    acc += w * po[(size_t)p * pstride];
    lsum += w * sv[1];
    den += w * sv[2];
  }
  part[0][grp][col] = acc;
  part[1][grp][col] = den;
  part[2][grp][col] = lsum;
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int j = 1; j < NG; ++j) {
      acc += part[0][j][col];
      den += part[1][j][col];
      lsum += part[2][j][col];
    }
    a.O[(size_t)row * D + col] = (T)(acc / den);
    if (col == 0) a.LSE[row] = (M + __builtin_log2f(lsum)) * kLn2;
  }
}

template <typename T, int D>
static hipError_t launch_dec_d(const DecArgs<T>& a, bool causal, int stage, hipStream_t st) {
  DecArgs<T> args = a;
  void* kargs[] = {&args};
  hipError_t e = hipSuccess;
  if (stage != 1) {
    const void* fn = causal ? reinterpret_cast<const void*>(&dec_split_kernel<T, D, true>)
                            : reinterpret_cast<const void*>(&dec_split_kernel<T, D, false>);
    e = hipLaunchKernel(fn, dim3((unsigned)(a.BH * a.splits)), dim3(64 * kDecWaves), kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  if (stage != 0 && !a.direct) {
    e = hipLaunchKernel(reinterpret_cast<const void*>(&dec_combine_kernel<T, D>),
                        dim3((unsigned)(a.BH * a.Nq)), dim3(D * kDecCombineGroups), kargs, 0, st);
  }
  return e;
}

template <typename T>
hipError_t launch_decode(const DecArgs<T>& a, int d, bool causal, int stage, hipStream_t st) {
  return d == 64 ? launch_dec_d<T, 64>(a, causal, stage, st)
                 : launch_dec_d<T, 128>(a, causal, stage, st);
}

template hipError_t launch_decode<bf16_t>(const DecArgs<bf16_t>&, int, bool, int, hipStream_t);
template hipError_t launch_decode<f16_t>(const DecArgs<f16_t>&, int, bool, int, hipStream_t);

}  // namespace fa

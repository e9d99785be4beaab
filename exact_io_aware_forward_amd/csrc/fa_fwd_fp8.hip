// FP8 forward: exact attention over E4M3 codes of Q J and K J (J the random
// orthogonal Hadamard rotation of fa_fp8_quantize_rows) with one fp32 scale per
// row, V and the probabilities in 16 bits.
//
// Method: CMU 11-868 FlashAttention notes (quidproquo.cc), "FlashAttention-3:
// asynchrony and FP8 on Hopper", slide page 24 — Q K^T in FP8, with Q and K
// multiplied by one Hadamard matrix first, which leaves the product unchanged
// and spreads outliers; pages 47-49 report the FP8 forward.  Only the scores go
// through FP8: S = scale * (sq_i Qc_i) . (sk_j Kc_j) with sq, sk the row scales,
// and the softmax and P V are those of the 16-bit forward (fa_fwd.hip): online
// softmax with a running max and denominator (Lecture 9 notes, cs2680.com,
// section 9.4), lazy rescaling, the rounded-P denominator for O, one LSE per row.
//
// gfx950 mapping: the 16-bit ping-pong forward (two wave groups of 4, 256 query
// rows per workgroup, 64-key tiles through a four-deep LDS ring filled by
// buffer-to-LDS copies), with S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4
// (E4M3 operands, unit block scales).  Its operands: lane l holds row l % 32
// of A (a key) and column l % 32 of B (a query), 32 bytes each, byte i of a
// lane in wave half h paired with byte i of the other operand's lane in the
// same half; the accumulator layout is that of the 16-bit 32x32 MFMA.  So a
// lane in half h takes bytes 32h .. 32h + 31 of each 64-byte slice of d from
// its key's row (two 16-byte LDS reads) and from its query's row (registers),
// with no transpose.  The query's scale folds into the lane's exp2 factor (a
// lane owns one query); the key scales, 16 per lane and 32-key block, multiply
// the scores before the row max.  d = 128 takes two MFMAs per 32-key block
// where the 16-bit path takes eight.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// log2 of the largest unnormalised probability the lazy rescale lets through;
// P is rounded to T for the P V product, so 2^tau must be finite in T (bf16
// has fp32's exponent range, fp16 stops at 65504).
template <typename T> constexpr float kLazyRescaleF8 = __is_same(T, bf16_t) ? 24.0f : 8.0f;

__device__ __forceinline__ f32x16 mma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  // Format 0 (OCP E4M3) for both operands; block scale exponents 127: x 1.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// A tile of E4M3 codes in LDS: 64 rows of D bytes, 16-byte chunk ch of row r
// at physical chunk ch ^ swz(r).  The operand reads (16 lanes: 16 consecutive
// rows at one logical chunk) then cover the 16 distinct 16-byte bank groups.
template <int D> struct CodeTile {
  static_assert(D == 64 || D == 128, "head dimension");
  static constexpr int kChunks = D / 16;
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (D == 128) return (r >> 1) & 7;
    else return (r >> 2) & 3;
  }
  __device__ static __forceinline__ int off(int r, int ch) { return r * D + ((ch ^ swz(r)) << 4); }
};

}  // namespace

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_kernel(Fp8FwdArgs<T> a) {
  using VTile = SwzTile<D>;
  using KTile = CodeTile<D>;
  constexpr int BR = kFwdBR, BC = kFwdBC, NT = 512;
  static_assert(BR == 256 && BC == 64, "8 waves x 32 rows, two 32-key blocks per tile");
  constexpr int RB = VTile::kRowBytes;     // V row bytes (16-bit)
  constexpr int TB = BC * RB;              // bytes of one V tile
  constexpr int KTB = BC * D;              // bytes of one K code tile
  constexpr int NB = 4;                    // ring depth
  constexpr int SPW = TB / 1024 / 8;       // 1 KB V copy segments per wave per tile
  constexpr int KSEG = KTB / 1024;         // 1 KB K copy segments per tile (8 or 4)
  constexpr int NSL = D / 64;              // 64-byte slices of d (fp8 MFMAs per 32-key block)
  static_assert(SPW * 8 * 1024 == TB && KSEG * 1024 == KTB, "tiles split into 1 KB segments");
  // Copies per wave and slot pair: its V segments, one K segment (waves past
  // KSEG repeat one, same bytes to the same place), the tile's 64 key scales
  // (every wave, same bytes to the same place) — equal counts for every wave.
  constexpr int NCOPY = SPW + 1 + 1;

  // LDS: V ring, K code ring, key-scale ring (read with K, in the matrix slots
  // of the tile; twice as deep as the others, its stage set at run time).
  constexpr int NSB = 2 * NB;
  __shared__ __attribute__((aligned(16))) char smem[NB * TB + NB * KTB + NSB * 256];
  lds_t* const L = (lds_t*)smem;
  const unsigned lds_base = (unsigned)(size_t)L;
  auto Vbuf = [&](int j) -> int { return (j & (NB - 1)) * TB; };
  auto Kbuf = [&](int j) -> int { return NB * TB + (j & (NB - 1)) * KTB; };
  auto Sbuf = [&](int j) -> int { return NB * TB + NB * KTB + (j & (NSB - 1)) * 256; };

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;
  const int rblk = 2 * (wave & 3) + grp;   // the two waves of a SIMD hold adjacent row blocks

  int bh, qi;
  map_block(blockIdx.x, a.nQ, a.BH, CAUSAL, bh, qi);
  const size_t hrow = (size_t)bh * N;   // first row of the head in [B*H*N]
  const unsigned char* __restrict__ Kch = a.Kc + hrow * D;
  const float* __restrict__ Ksh = a.Ks + hrow;
  const T* __restrict__ Vh = a.V + hrow * D;
  const int nK = a.nK;

  const int q0 = qi * BR;
  const int qw0 = q0 + 32 * rblk;
  const int qrow = qw0 + l32;
  int jend = nK;
  if (CAUSAL) jend = min(nK, (min(q0 + BR, N) - 1) / BC + 1);
  int wend = qw0 < N ? jend : 0;
  if (CAUSAL && qw0 < N) wend = min(jend, (qw0 + 31) / BC + 1);

  // Q codes as B operands: lane holds query qrow, bytes 64 sl + 32 g .. +31.
  i32x8 qf[NSL];
  float cq;   // this lane's exp2 factor: scale * log2(e) * (its query's row scale)
  {
    const int qc = min(qrow, N - 1);
    const unsigned char* qp = a.Qc + (hrow + qc) * D + 32 * g;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const u32x4 lo = ld16(qp + 64 * sl);
      const u32x4 hi = ld16(qp + 64 * sl + 16);
      qf[sl] = __builtin_bit_cast(i32x8, (u32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      if (qrow >= N) qf[sl] = (i32x8)(0);
    }
    cq = a.scale_log2 * a.Qs[hrow + qc];
  }

  // Copy offsets.  V: segment sg (1 KB) of a tile by wave sg / SPW, lane i
  // filling physical chunk i of it (row r = (64 sg + i) / CPR, physical chunk
  // pc, logical chunk pc ^ swz(r)).  K: segment wave % KSEG, the same way.
  constexpr int CPR = D / 8;   // 16-byte chunks per V row
  int vdma[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int ci = (wave * SPW + k) * 64 + lane;
    const int r = ci / CPR, pc = ci % CPR;
    vdma[k] = r * RB + ((pc ^ VTile::swz(r)) << 4);
  }
  const int kseg = wave % KSEG;
  int kdma;
  {
    const int ci = kseg * 64 + lane;
    const int r = ci / KTile::kChunks, pc = ci % KTile::kChunks;
    kdma = r * D + ((pc ^ KTile::swz(r)) << 4);
  }
  auto copy_v = [&](int j, int buf_off) {
    const int kv0 = j * BC;
    const u32x4 rsrc = raw_rsrc(Vh + (size_t)kv0 * D, (unsigned)((N - kv0) * RB));
#pragma unroll
    for (int k = 0; k < SPW; ++k)
      dma16(rsrc, lds_base + buf_off + (wave * SPW + k) * 1024, vdma[k]);
  };
  auto copy_k = [&](int j, int kbuf_off, int sbuf_off) {
    const int kv0 = j * BC;
    const u32x4 rk = raw_rsrc(Kch + (size_t)kv0 * D, (unsigned)((N - kv0) * D));
    dma16(rk, lds_base + kbuf_off + kseg * 1024, kdma);
    const u32x4 rs = raw_rsrc(Ksh + kv0, (unsigned)((N - kv0) * 4));
    dma4(rs, lds_base + sbuf_off, lane * 4);
  };

  // Per-lane operand offsets.  K: row l % 32 (+ 32 per block), chunks
  // 4 sl + 2 g and + 1.  V^T fragments by transpose reads (16-bit path).
  int k_off[NSL][2];
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
    for (int h = 0; h < 2; ++h) k_off[sl][h] = KTile::off(l32, 4 * sl + 2 * g + h);
  int tr_off[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      tr_off[h][db] = VTile::tr_off(lane, h, db);
      asm volatile("" : "+v"(tr_off[h][db]));
    }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = zero16();
  f32x16 s[2];
  s[0] = zero16();
  s[1] = zero16();
  frag_t<T> pf[BC / 16];
#pragma unroll
  for (int u = 0; u < BC / 16; ++u) pf[u] = zero_frag<T>();
  float m = -1e30f;   // running max of the scaled (log2-domain) scores, possibly stale
  float lsum = 0.f;   // this lane's part of the denominator (fp32 probabilities)
  // The rounded-P denominator on 16x16x32 products (rowsum_sel_frag): element 0
  // of lane q < 32 holds query q's sum, lanes 32-63 hold zeros.
  f32x4 osum = {0.f, 0.f, 0.f, 0.f};
  const frag_t<T> rsel = rowsum_sel_frag<T>(lane);
  frag_t<T> vpre[2][D / 32];

  // Prologue: K(0..2) with their scales and V(0..1) in the rings; the first
  // matrix slot multiplies the zero P by V buffer 3, which is zeroed.
  copy_k(0, Kbuf(0), Sbuf(0));
  copy_k(min(1, jend - 1), Kbuf(1), Sbuf(1));
  copy_k(min(2, jend - 1), Kbuf(2), Sbuf(2));   // (scale buffers 0..2 of the deeper ring)
  copy_v(0, Vbuf(0));
  copy_v(min(1, jend - 1), Vbuf(1));
#pragma unroll
  for (int c2 = 0; c2 < TB / 16 / NT; ++c2)
    lds_st<u32x4>(L + Vbuf(3) + (tid + c2 * NT) * 16, (u32x4)(0u));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  auto read_vpre = [&](int j) {
    const lds_t* vb = L + Vbuf(j);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        vpre[u][db] = tr_frag<T>(vb + 16 * u * RB + tr_off[0][db], vb + 16 * u * RB + tr_off[1][db]);
  };
  read_vpre(-1);

  // Matrix slot of tile t: P(t-1) V(t-1) (16-bit, V^T by transpose reads),
  // then S(t) = K(t) Q^T on the fp8 MFMA, its K operand reads issued during
  // the last P V steps, times the key scales (this wave's vector ALU is free
  // between its MFMAs; the other wave's softmax is the busy one).
  auto matrix_slot = [&](int t, int st) {
    __builtin_amdgcn_s_setprio(2);
    constexpr int NV = D / 32, NU = BC / 16;
    const lds_t* vb = L + Vbuf(st + NB - 1);
    const lds_t* kb = L + Kbuf(st);
    auto rd_v = [&](int u, int db) {
      return tr_frag<T>(vb + 16 * u * RB + tr_off[0][db], vb + 16 * u * RB + tr_off[1][db]);
    };
    frag_t<T> vf[3][NV];
    u32x4 kr[2][NSL][2];
    f32x4 ks[2][4];   // scales of this lane's keys: block kb, rows 8 j + 4 g .. + 3
    const lds_t* sb = L + Sbuf(t);
#pragma unroll
    for (int db = 0; db < NV; ++db) {
      vf[0][db] = vpre[0][db];
      vf[1][db] = vpre[1][db];
    }
    __builtin_amdgcn_sched_barrier(0);
    float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int r = 0; r < 8; ++r) rs4[r & 3] += s[u >> 1][8 * (u & 1) + r];
      osum = mma16(rsel, pf[u], osum);
#pragma unroll
      for (int db = 0; db < NV; ++db) {
        o[db] = mma(vf[u % 3][db], pf[u], o[db]);
        if (u + 2 < NU) vf[(u + 2) % 3][db] = rd_v(u + 2, db);
      }
      if (u >= 2) {   // K code reads and key scales of block u - 2
        const int kb2 = u - 2;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
          for (int h = 0; h < 2; ++h) kr[kb2][sl][h] = lds_ld<u32x4>(kb + kb2 * 32 * D + k_off[sl][h]);
#pragma unroll
        for (int j = 0; j < 4; ++j) ks[kb2][j] = lds_ld<f32x4>(sb + 4 * (32 * kb2 + 8 * j + 4 * g));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);
    // The key scales multiply each block's scores as soon as its products are
    // in: block 0's alongside block 1's MFMAs, block 1's at the end.
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      s[kb2] = zero16();
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) {
        const u32x4 lo = kr[kb2][sl][0], hi = kr[kb2][sl][1];
        const i32x8 kf = __builtin_bit_cast(
            i32x8, (u32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        s[kb2] = mma_e4m3(kf, qf[sl], s[kb2]);
      }
      if (kb2 == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[0][4 * j + e] *= ks[0][j][e];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s[1][4 * j + e] *= ks[1][j][e];
    __builtin_amdgcn_s_setprio(0);
  };

  // Softmax of tile t (its scores already carry the key scales): as the
  // 16-bit forward (mask, lazy rescale, exp2 with this lane's factor).
  auto softmax = [&](int t, int st) {
    if (t < 0 || t >= wend) {
#pragma unroll
      for (int u = 0; u < BC / 16; ++u) pf[u] = zero_frag<T>();
      s[0] = zero16();
      s[1] = zero16();
      return;
    }
    const int kv0 = t * BC;
    if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0)) {
      keep_branch();
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb2 * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= N || (CAUSAL && key > qrow)) s[kb2][r] = -INFINITY;
        }
    }
    float mx4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float x = vmax3(s[0][q], s[0][q + 4], s[0][q + 8]);
      x = vmax3(x, s[0][q + 12], s[1][q]);
      x = vmax3(x, s[1][q + 4], s[1][q + 8]);
      mx4[q] = vmax(x, s[1][q + 12]);
    }
    const float mx = vmax_halves(vmax(vmax3(mx4[0], mx4[1], mx4[2]), mx4[3]));
    const float mc = mx * cq;
    if (__ballot(mc > m + kLazyRescaleF8<T>)) {
      const float m_new = fmaxf(m, mc);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
      osum[0] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = __builtin_fmaf(s[kb2][r], cq, -m);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = fast_exp2(s[kb2][r]);
#pragma unroll
    for (int u = 0; u < BC / 16; ++u)
      pf[u] = to_frag<T>((u & 1) ? half8<1>(s[u >> 1]) : half8<0>(s[u >> 1]));
  };

  // Softmax slot of tile t in slot pair p: this wave's copies of the pair
  // (K(p+3) into the buffer of K(p-1) and its scales into that of K(p-5),
  // both last read in slot 2p-1 or before; V(p+2) into that of V(p-2), last
  // read in slot 2p-1), the read-ahead of V(t), the softmax, and a wait for
  // its copies of pair p-1.
  auto softmax_slot = [&](int t, int p, int st) {
    copy_k(min(p + 3, jend - 1), Kbuf(p + 3), Sbuf(p + 3));   // p: runtime, the scale stage too
    copy_v(min(p + 2, jend - 1), Vbuf(p + 2));
    read_vpre(st);
    __builtin_amdgcn_sched_barrier(0);
    softmax(t, st);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<NCOPY>();
  };

  if (grp == 1) {
    softmax_slot(-1, 0, NB - 1);
    lds_barrier();
  }
  for (int u0 = 0;; u0 += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (u0 + k > jend) break;
      matrix_slot(u0 + k, k);
      lds_barrier();
      softmax_slot(u0 + k, u0 + k + grp, k);
      lds_barrier();
    }
    if (u0 + NB > jend) break;
  }
  if (grp == 0) lds_barrier();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
  lds_barrier();   // every wave's copies have landed and its reads returned: LDS is free for O
  static_assert(8 * kStageBytes<D> <= sizeof(smem), "O staging fits the ring");

  if (qw0 < N) {
    const float ltot = lsum + __shfl_xor(lsum, 32);
    float lqtot = osum[0] + __shfl_xor(osum[0], 32);
    // Queries q and q + 16 share a column of the row-sum products, whose zero
    // selector entries still multiply the other query's probabilities: a NaN
    // there (a NaN input in that row) makes this sum NaN as well.  The query's
    // own fp32 sum is then finite and stands in for it (the two differ only by
    // the rounding of P); a NaN of the query's own leaves both NaN.
    if (__builtin_isnan(lqtot) && !__builtin_isnan(ltot)) lqtot = ltot;
    store_rows_lds<T, D>(L + wave * kStageBytes<D>, o, 1.0f / lqtot, a.O + (hrow + qw0) * D, N - qw0, lane);
    if (g == 0 && qrow < N) a.LSE[hrow + qrow] = (m + __builtin_log2f(ltot)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_fwd_fp8_inst(const Fp8FwdArgs<T>& a, hipStream_t st) {
  Fp8FwdArgs<T> args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_fp8_kernel<T, D, CAUSAL>),
                         dim3((unsigned)(a.nQ * a.BH)), dim3(512), kargs, 0, st);
}

template <typename T>
hipError_t launch_fwd_fp8(const Fp8FwdArgs<T>& a, int d, bool causal, hipStream_t st) {
  if (d == 64)
    return causal ? launch_fwd_fp8_inst<T, 64, true>(a, st) : launch_fwd_fp8_inst<T, 64, false>(a, st);
  return causal ? launch_fwd_fp8_inst<T, 128, true>(a, st) : launch_fwd_fp8_inst<T, 128, false>(a, st);
}

template hipError_t launch_fwd_fp8<bf16_t>(const Fp8FwdArgs<bf16_t>&, int, bool, hipStream_t);
template hipError_t launch_fwd_fp8<f16_t>(const Fp8FwdArgs<f16_t>&, int, bool, hipStream_t);

}  // namespace fa

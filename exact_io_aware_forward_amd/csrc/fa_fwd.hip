// Forward kernels: exact attention with online softmax, one workgroup per
// (batch*head, query tile of kFwdRows rows: 256, or 512 for 16-bit inputs at
// d = 64 without the causal mask).  fwd_pp_kernel serves bf16/fp16 inputs,
// fwd_kernel fp32 inputs.
//
// Method: Lecture 9 notes (cs2680.com), section 9.4 — walk the key/value tiles,
// keep per query row a running max m and a running denominator l relative to
// m, rescale the unnormalised output by exp(m_old - m_new) when the max moves,
// divide by l once after the last tile; CMU 11-868 FlashAttention notes
// (quidproquo.cc), "Tiling: fix the wrong denominator afterward", slide page
// 12 — the rescaling makes each tile's update exact.  The only statistic saved
// is the row log-sum-exp (slide page 14, Lecture 9 section 9.6).
//
// Rescaling is lazy: m only moves when a tile's row max exceeds it by more
// than tau (in exp2 units: 24 for bf16, 8 for fp16 and fp32), otherwise the
// tile's probabilities are formed against the stale m and may reach 2^tau.
// The result is unchanged — O and l carry the same factor, and
// LSE = m + log l for whatever m was used — and the O rescale (D/2 multiplies
// per lane) drops out of almost every tile.  This is
// the conditional-rescaling idea of the FlashAttention-4 slides (CMU notes,
// "FlashAttention-4: asymmetric scaling on Blackwell", slides 51-52).
// Two denominators are kept: l from the fp32 probabilities (for LSE) and lq
// from the probabilities as rounded for the PV product (for O), so O's weights
// sum to one exactly whatever the rounding of the largest probability.
//
// gfx950 mapping (both kernels).  8 waves x 32 query rows (one workgroup of 256
// rows per CU, two waves per SIMD), so each K/V byte brought on chip serves 256
// queries (fwd_pp_kernel at d = 64 without the causal mask: 8 waves x 2 x 32
// rows, 512 queries); K/V tiles of 64 keys.  Per wave, 32-row block and tile:
//   S^T (keys x queries) = K Q^T   — A = K rows from LDS, B = Q^T held in
//                                    registers for the whole kernel;
//   online softmax on S^T: lane l owns query l % 32, so the row statistics live
//   in one lane pair (l, l ^ 32) and need a single cross-half exchange;
//   O^T (d x queries) += V^T P^T   — A = V^T read with the LDS transpose read
//                                    from the row-major V tile (fp32: from a
//                                    transposed LDS copy), B = P^T straight from
//                                    the S^T accumulator.
// Scores are scaled by c = scale*log2(e) inside one FMA feeding exp2.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

// log2 of the largest unnormalised probability the lazy rescale lets through.
// P is rounded to T for the P V product, so 2^tau must be finite in T: bf16 has
// the exponent range of fp32, fp16 stops at 65504.  A larger tau means fewer
// rescales: with keys whose scores spread over tens of exp2 units (outlier
// rows), the running max keeps growing and tau = 8 rescales two tiles in five.
template <typename T> constexpr float kLazyRescale = __is_same(T, bf16_t) ? 24.0f : 8.0f;

// LDS layout of the fp32 kernel (fwd_kernel).
template <typename T, int D> struct FwdLayout {
  static constexpr int BR = kFwdBR, BC = kFwdBC, NT = 64 * kFwdWaves;
  static constexpr int ES = sizeof(T);
  // K rows padded by 16 B: 8 consecutive rows of one 16-byte column hit distinct banks.
  static constexpr int KROW = D * ES + 16;
  // V: a transposed copy [d][key] with the key order of perm16().
  static constexpr int VROW = (BC + 8) * ES;
  static constexpr int KBYTES = BC * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BYTES = 2 * (KBYTES + VBYTES);
  static constexpr int CPR = D * ES / 16;         // 16-byte chunks per row
  static constexpr int KCH = BC * CPR / NT;       // chunks per thread per tile
  static constexpr int VBLK = (BC / 4) * CPR;     // V copied in 4-row blocks
  static constexpr int VPT = (VBLK + NT - 1) / NT;
  static_assert(KCH * NT == BC * CPR, "tile must split evenly over the workgroup");
};

}  // namespace

template <typename T, int D, bool CAUSAL, bool MAP>
__global__ __launch_bounds__(64 * kFwdWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs<T> a) {
  static_assert(sizeof(T) == 4, "fp32 inputs only; 16-bit inputs run fwd_pp_kernel");
  using Lay = FwdLayout<T, D>;
  constexpr int BR = Lay::BR, BC = Lay::BC, NT = Lay::NT, ES = Lay::ES;
  constexpr int EPC = kEPC<T>;
  constexpr int KROW = Lay::KROW, VROW = Lay::VROW, CPR = Lay::CPR;
  constexpr int KCH = Lay::KCH;

  __shared__ __attribute__((aligned(16))) char smem[Lay::BYTES];
  lds_t* const Kbuf0 = (lds_t*)smem;
  lds_t* const Vbuf0 = Kbuf0 + 2 * Lay::KBYTES;

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  int bh, qi;
  map_block(blockIdx.x, a.nQ, a.BH, CAUSAL, bh, qi);
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / a.group) * N * D;   // the query head's key/value head
  const T* __restrict__ Qh = a.Q + hoff;
  const T* __restrict__ Kh = a.K + kvoff;
  const T* __restrict__ Vh = a.V + kvoff;

  const int q0 = qi * BR;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool wave_rows = qw0 < N;

  // Q^T operand: lane holds query qrow, d = 16t + 8g .. +7.
  frag_t<T> qf[D / 16];
  {
    const int qc = min(qrow, N - 1);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = ld_frag(Qh + (size_t)qc * D + 16 * t + 8 * g);
      if (qrow >= N) qf[t] = zero_frag<T>();
    }
  }

  const int nK = a.nK;
  int jend = nK;
  if (CAUSAL) jend = min(nK, (min(q0 + BR, N) - 1) / BC + 1);

  // Register staging of one K/V tile: chunk c of this thread is row
  // (tid + c*NT) / CPR, 16-byte column (tid + c*NT) % CPR.
  u32x4 kst[KCH];
  u32x4 vst[Lay::VPT * 4];

  // Rows past N are loaded from row N-1 (always valid) and replaced by zeros
  // only when the tile is written to LDS, so no wait on a load sits next to
  // its issue: the loads of tile j+1 stay in flight while tile j is computed.
  // The prefetch of tile j is issued in four parts spread over the compute
  // phases (scheduling fences keep them there): all waves issuing a whole tile
  // at once after the barrier queue behind each other in the vector-memory
  // path.  Parts 0, 1: K chunks; part 2: all of V (4-row blocks for the
  // transposed copy); part 3 issues nothing.
  auto load_part = [&](int j, int part) {
    const int kv0 = j * BC;
    const int last = N - 1 - kv0;
    const T* kt = Kh + (size_t)kv0 * D;
    const T* vt = Vh + (size_t)kv0 * D;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      if (part != (c * 2) / KCH) continue;
      const int idx = tid + c * NT;
      kst[c] = ld16(kt + (unsigned)(min(idx / CPR, last) * D + (idx % CPR) * EPC));
    }
    if (part != 2) return;
#pragma unroll
    for (int b = 0; b < Lay::VPT; ++b) {
      const int blk = tid + b * NT;
      if (Lay::VBLK % NT == 0 || blk < Lay::VBLK) {
        const int kc = blk % (BC / 4), dc = blk / (BC / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vst[4 * b + e] = ld16(vt + (unsigned)(min(4 * kc + e, last) * D + dc * EPC));
      }
    }
  };
  auto load_tile = [&](int j) {
#pragma unroll
    for (int part = 0; part < 4; ++part) load_part(j, part);
  };
  auto store_tile = [&](int buf, int j) {
    lds_t* kb = Kbuf0 + buf * Lay::KBYTES;
    lds_t* vb = Vbuf0 + buf * Lay::VBYTES;
    const int valid = N - j * BC;  // rows [0, valid) of the tile are real
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / CPR, ch = idx % CPR;
      const bool ok = row < valid;
      lds_st<u32x4>(kb + row * KROW + ch * 16, ok ? kst[c] : (u32x4)(0u));
    }
#pragma unroll
    for (int b = 0; b < Lay::VPT; ++b) {
      const int blk = tid + b * NT;
      if (Lay::VBLK % NT == 0 || blk < Lay::VBLK) {
        const int kc = blk % (BC / 4), dc = blk / (BC / 4);
        u32x4 blk4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) blk4[e] = 4 * kc + e < valid ? vst[4 * b + e] : (u32x4)(0u);
        store_transposed_4rows<T>(reinterpret_cast<T*>(smem) +
                                      (2 * Lay::KBYTES + buf * Lay::VBYTES) / ES,
                                  VROW / ES, dc * EPC, 4 * kc, blk4);
      }
    }
  };

  // Per-lane LDS byte offsets of the operand reads (tile-invariant).
  const int k_lane = l32 * KROW + 8 * g * ES;                  // + kb*32*KROW + 16t*ES
  const int v_lane = l32 * VROW + 8 * g * ES;                  // + u, db immediates

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = zero16();
  float m = -1e30f;   // running max of the scaled (log2-domain) scores, possibly stale
  float lsum = 0.f;   // this lane's part of the running denominator (fp32 probabilities)
  float lq = 0.f;     // the same over the probabilities as rounded for PV
  const float c = a.scale_log2;

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  for (int j = 0; j < jend; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < jend;
    if (more) load_part(j + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int kv0 = j * BC;
    const int code = tile_code(qi, j, BR, BC, N, CAUSAL);
    if (MAP && tid == 0) a.map[((size_t)bh * a.nQ + qi) * nK + j] = (unsigned char)code;

    const bool active = wave_rows && (!CAUSAL || kv0 <= qw0 + 31);
    if (active) {
      const lds_t* kb_ = Kbuf0 + buf * Lay::KBYTES + k_lane;
      const lds_t* vb_ = Vbuf0 + buf * Lay::VBYTES + v_lane;
      const bool need_mask = code != 1 && ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0));
      f32x16 s[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        frag_t<T> kf[D / 16];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) kf[t] = lds_ld<frag_t<T>>(kb_ + kb * 32 * KROW + 16 * t * ES);
        __builtin_amdgcn_sched_barrier(0);
        s[kb] = zero16();
#pragma unroll
        for (int t = 0; t < D / 16; ++t) s[kb] = mma(kf[t], qf[t], s[kb]);
      }
      if (need_mask) {
        keep_branch();
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
          }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) load_part(j + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mc = mx * c;
      if (__ballot(mc > m + kLazyRescale<T>)) {
        const float m_new = fmaxf(m, mc);
        const float alpha = fast_exp2(m - m_new);
        m = m_new;
        lsum *= alpha;
        lq *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) load_part(j + 1, 2);
      __builtin_amdgcn_sched_barrier(0);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -m));
          s[kb][r] = p;
          rs += p;
        }
      lsum += rs;
#pragma unroll
      for (int u = 0; u < BC / 16; ++u) {
        const frag_t<T> pf = to_frag<T>((u & 1) ? half8<1>(s[u >> 1]) : half8<0>(s[u >> 1]));
        lq = frag_sum(pf, lq);
        frag_t<T> vfs[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) vfs[db] = lds_ld<frag_t<T>>(vb_ + db * 32 * VROW + 16 * u * ES);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = mma(vfs[db], pf, o[db]);
        if (u == 1) {
          __builtin_amdgcn_sched_barrier(0);
          if (more) load_part(j + 1, 3);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (more) {
#pragma unroll
      for (int part = 1; part < 4; ++part) load_part(j + 1, part);
    }
    if (more) store_tile(buf ^ 1, j + 1);
    __syncthreads();
  }

  if (MAP && tid == 0)
    for (int j = jend; j < nK; ++j) a.map[((size_t)bh * a.nQ + qi) * nK + j] = 0;

  if (wave_rows) {
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float lqtot = lq + __shfl_xor(lq, 32);
    if (qrow < N) {
      const float inv = 1.0f / lqtot;
      T* orow = a.O + hoff + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          T v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (T)(o[db][4 * rg + e] * inv);
          *reinterpret_cast<u32x4*>(orow + db * 32 + 8 * rg + 4 * g) = __builtin_bit_cast(u32x4, v4);
        }
      if (g == 0) a.LSE[(size_t)bh * N + qrow] = (m + __builtin_log2f(ltot)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// 16-bit forward: two wave groups in ping-pong.
//
// The same online-softmax recurrence as fwd_kernel, arranged for the CU's
// pipes: waves w and w + 4 of a workgroup run on the same SIMD, so waves 0-3
// (group 0) and 4-7 (group 1) are offset by half a key tile.  The loop runs
// in slots separated by workgroup barriers; in every slot one wave of each
// SIMD issues matrix work — the P V^T product of the previous tile and the
// K Q^T product of the next — while the other computes the softmax of its
// current tile on the vector ALU, so the matrix cores are not left idle while
// exponentials are computed.  For a wave of group grp, slot s is phase
// p = s - grp: even p = 2t runs S(t) = K(t) Q^T and O += V(t-1)^T P(t-1), odd
// p = 2t + 1 turns S(t) into P(t) (lazy rescale, exp2).
//
// K and V tiles (64 keys) live in a ring of four swizzled row-major LDS
// buffers each, filled by buffer-to-LDS copies that bypass registers: in slot
// pair u (slots 2u, 2u+1) every wave, in its softmax slot, issues its share of
// K(u+3) and V(u+2) and, at the end of the slot, waits for its copies of pair
// u-1; the copies of pair u are first read in slot 2u+5 (the read-ahead of
// V(u+2) by group 0), after the barriers that follow every wave's wait.  Rows past N come in as zeros
// (the descriptor ends at row N); they meet only masked scores (probability
// exactly 0).
template <typename T, int D, bool CAUSAL, bool MAP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(FwdArgs<T> a) {
  using Tile = SwzTile<D>;
  constexpr int BR = kFwdRows(D, CAUSAL, true), BC = kFwdBC, NT = 512;
  constexpr int RBW = BR / kFwdBR;         // 32-row blocks per wave (one or two)
  static_assert(kFwdBR == 256 && BC == 64, "8 waves x 32 rows, two 32-key blocks per tile");
  constexpr int RB = Tile::kRowBytes;
  constexpr int TB = BC * RB;              // bytes of one K or V tile
  constexpr int NB = 4;                    // ring depth
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int SPW = TB / 1024 / 8;       // 1 KB copy segments per wave per tile
  static_assert(SPW * 8 * 1024 == TB, "tile must split into 1 KB segments over 8 waves");

  __shared__ __attribute__((aligned(16))) char smem[2 * NB * TB];
  lds_t* const L = (lds_t*)smem;
  const unsigned lds_base = (unsigned)(size_t)L;

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int g = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;
  const int rblk = 2 * (wave & 3) + grp;   // the two waves of a SIMD hold adjacent row blocks

  // Each wave holds RBW blocks of 32 query rows (two for 16-bit, d = 64, no
  // causal mask; see kFwdRows): every K and V fragment read from LDS then
  // feeds RBW products, and each key tile carries RBW times the rows.
  int bh, qi;
  map_block(blockIdx.x, a.nQ, a.BH, CAUSAL, bh, qi);
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / a.group) * N * D;   // the query head's key/value head
  const T* __restrict__ Qh = a.Q + hoff;
  const T* __restrict__ Kh = a.K + kvoff;
  const T* __restrict__ Vh = a.V + kvoff;
  const int nK = a.nK;
  if (MAP)
    for (int j = tid; j < nK; j += NT)
      a.map[((size_t)bh * a.nQ + qi) * nK + j] = (unsigned char)tile_code(qi, j, BR, BC, N, CAUSAL);

  const int q0 = qi * BR;
  const int qw0 = q0 + 32 * RBW * rblk;   // block b of this wave: rows qw0 + 32 b ..
  int jend = nK;
  if (CAUSAL) jend = min(nK, (min(q0 + BR, N) - 1) / BC + 1);
  // Key tiles this wave computes: [0, wend).  Causal: tiles past the wave's
  // last row see only masked scores and are skipped.
  int wend = qw0 < N ? jend : 0;
  if (CAUSAL && qw0 < N) wend = min(jend, (qw0 + 32 * RBW - 1) / BC + 1);

  // Q^T operands: in block b, lane holds query qw0 + 32 b + l32, d = 16t + 8g .. +7.
  frag_t<T> qf[RBW][D / 16];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int qrow = qw0 + 32 * b + l32;
    const int qc = min(qrow, N - 1);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[b][t] = ld_frag(Qh + (size_t)qc * D + 16 * t + 8 * g);
      if (qrow >= N) qf[b][t] = zero_frag<T>();
    }
  }

  // Tile copies.  Segment sg (1 KB, 4 rows at d = 128) of a tile is copied by
  // wave sg / SPW; lane i of it fills physical chunk i of the segment, i.e.
  // row r = (64 sg + i) / CPR, physical chunk pc = (64 sg + i) % CPR, which
  // holds logical chunk pc ^ swz(r) of that row.
  int dma_off[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int ci = (wave * SPW + k) * 64 + lane;
    const int r = ci / CPR, pc = ci % CPR;
    dma_off[k] = r * RB + ((pc ^ Tile::swz(r)) << 4);
  }
  auto Kbuf = [&](int j) -> int { return (j & (NB - 1)) * TB; };          // byte offsets in smem
  auto Vbuf = [&](int j) -> int { return (NB + (j & (NB - 1))) * TB; };
  auto copy_tile = [&](const T* base, int j, int buf_off) {
    const int kv0 = j * BC;
    u32x4 rsrc = raw_rsrc(base + (size_t)kv0 * D, (unsigned)((N - kv0) * RB));
    // The descriptor is uniform.  In the instrumented instances, whose map
    // writes raise the scalar-register pressure, readfirstlane makes that
    // explicit so that it stays in scalar registers (the copy takes it there);
    // elsewhere it would only add vector instructions.
    if constexpr (MAP)
      rsrc = (u32x4){(unsigned)__builtin_amdgcn_readfirstlane(rsrc[0]), (unsigned)__builtin_amdgcn_readfirstlane(rsrc[1]),
                     (unsigned)__builtin_amdgcn_readfirstlane(rsrc[2]), (unsigned)__builtin_amdgcn_readfirstlane(rsrc[3])};
#pragma unroll
    for (int k = 0; k < SPW; ++k)
      dma16(rsrc, lds_base + buf_off + (wave * SPW + k) * 1024, dma_off[k]);
  };

  // Per-lane operand offsets into a swizzled tile: K rows l%32 (A operand of
  // S^T, elements 16t + 8g .. +7), V^T fragments by transpose reads.
  int a_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a_off[t] = Tile::a_off(lane, t);
  int tr_off[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      // Transpose reads are of V only: the offset includes the V ring's base
      // (64 KB, past the 16-bit immediate range of LDS reads), so the stage
      // and row offsets left to add fit the immediate.  Opaque to the
      // compiler, so that base + offset stays an addition it can fold.
      tr_off[h][db] = Tile::tr_off(lane, h, db) + NB * TB;
      asm volatile("" : "+v"(tr_off[h][db]));
    }

  // Per block: O accumulators, S (then P in fp32), P as MFMA operands, the
  // running max of the scaled (log2-domain) scores (possibly stale), this
  // lane's part of the fp32 denominator, and the denominator over the
  // probabilities as rounded for P V, formed by the matrix pipe (16x16x32
  // products with a selector A, see rowsum_sel_frag: element 0 of lane q < 32
  // holds query q's sum, lanes 32-63 hold zeros).
  f32x16 o[RBW][D / 32];
  f32x16 s[RBW][2];
  frag_t<T> pf[RBW][BC / 16];
  float m[RBW], lsum[RBW];
  f32x4 osum[RBW];
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[b][db] = zero16();
    s[b][0] = zero16();
    s[b][1] = zero16();
#pragma unroll
    for (int u = 0; u < BC / 16; ++u) pf[b][u] = zero_frag<T>();
    m[b] = -1e30f;
    lsum[b] = 0.f;
    osum[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const frag_t<T> rsel = rowsum_sel_frag<T>(lane);
  const float c = a.scale_log2;
  frag_t<T> vpre[2][D / 32];   // V fragments u = 0, 1 of the next matrix slot, read ahead

  // Prologue: K(0..2) and V(0..1) in the ring; the first matrix slot
  // multiplies the zero P by V buffer 3, which is zeroed.
  copy_tile(Kh, 0, Kbuf(0));
  copy_tile(Kh, min(1, jend - 1), Kbuf(1));
  copy_tile(Kh, min(2, jend - 1), Kbuf(2));
  copy_tile(Vh, 0, Vbuf(0));
  copy_tile(Vh, min(1, jend - 1), Vbuf(1));
#pragma unroll
  for (int c2 = 0; c2 < TB / 16 / NT; ++c2)
    lds_st<u32x4>(L + Vbuf(3) + (tid + c2 * NT) * 16, (u32x4)(0u));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  auto read_vpre = [&](int j) {
    const lds_t* vb = L + Vbuf(j) - NB * TB;   // tr_off holds the V ring base
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        vpre[u][db] = tr_frag<T>(vb + 16 * u * RB + tr_off[0][db], vb + 16 * u * RB + tr_off[1][db]);
  };
  read_vpre(-1);

  // Matrix slot of tile t: P(t-1) V(t-1), then S(t) = K(t) Q^T, as one
  // software-pipelined stream: the operand reads of each step are issued one
  // step ahead, between the MFMAs of the step before (the V reads of u = 0, 1
  // before the conversion of P; the first K reads during the last P V steps),
  // so the matrix pipe does not wait on LDS latency at the phase boundary.
  // Both products run in every matrix slot, so the accumulators never pass
  // through a branch (which costs register copies): P is zero for t = 0 and
  // past the wave's last tile (V is then zeros or real rows, never garbage),
  // and S past the last tile is computed from stale K and never used.
  auto matrix_slot = [&](int t, int st) {   // st = t % NB, a constant
    // Raised issue priority: when both waves of a SIMD have an instruction
    // ready, the MFMA of this wave goes first, so the vector work of the other
    // wave fills the gaps instead of delaying the matrix pipe.
    __builtin_amdgcn_s_setprio(2);
    constexpr int NV = D / 32, NU = BC / 16, NF = D / 16;
    const lds_t* vb = L + Vbuf(st + NB - 1) - NB * TB;   // tr_off holds the V ring base
    const lds_t* kb = L + Kbuf(st);
    auto rd_v = [&](int u, int db) {
      return tr_frag<T>(vb + 16 * u * RB + tr_off[0][db], vb + 16 * u * RB + tr_off[1][db]);
    };
    frag_t<T> vf[3][NV];
    frag_t<T> kf[2][NF];
#pragma unroll
    for (int db = 0; db < NV; ++db) {
      vf[0][db] = vpre[0][db];
      vf[1][db] = vpre[1][db];
    }
    __builtin_amdgcn_sched_barrier(0);
    // P V: step u reads ahead V(u+2) (u < 2) or the K fragments of block 0.
    // The fp32 row sums of P(t-1) (still in s) are formed alongside, vector
    // work that fits between the MFMAs of this slot.
    float rs4[RBW][4];
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) rs4[b][q] = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int b = 0; b < RBW; ++b) {
#pragma unroll
        for (int r = 0; r < 8; ++r) rs4[b][r & 3] += s[b][u >> 1][8 * (u & 1) + r];
        osum[b] = mma16(rsel, pf[b][u], osum[b]);
      }
#pragma unroll
      for (int db = 0; db < NV; ++db) {
#pragma unroll
        for (int b = 0; b < RBW; ++b) o[b][db] = mma(vf[u % 3][db], pf[b][u], o[b][db]);
        if (u + 2 < NU) {
          vf[(u + 2) % 3][db] = rd_v(u + 2, db);
        } else {
          const int i = (u - 2) * NV + db;   // K block 0, NF / (2 NV) reads per MFMA
#pragma unroll
          for (int h = 0; h < NF / (2 * NV); ++h) {
            const int tt = i * (NF / (2 * NV)) + h;
            kf[0][tt] = lds_ld<frag_t<T>>(kb + a_off[tt]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < RBW; ++b) lsum[b] += (rs4[b][0] + rs4[b][1]) + (rs4[b][2] + rs4[b][3]);
    // S = K Q^T: block 0 reads ahead block 1.
#pragma unroll
    for (int b = 0; b < RBW; ++b) {
      s[b][0] = zero16();
      s[b][1] = zero16();
    }
#pragma unroll
    for (int i = 0; i < NF; ++i) {
#pragma unroll
      for (int b = 0; b < RBW; ++b) s[b][0] = mma(kf[0][i], qf[b][i], s[b][0]);
      kf[1][i] = lds_ld<frag_t<T>>(kb + 32 * RB + a_off[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
      for (int b = 0; b < RBW; ++b) s[b][1] = mma(kf[1][i], qf[b][i], s[b][1]);
    __builtin_amdgcn_s_setprio(0);
  };
  auto softmax = [&](int t) {
    if (t < 0 || t >= wend) {   // P = 0: the next matrix slot adds nothing
#pragma unroll
      for (int b = 0; b < RBW; ++b) {
#pragma unroll
        for (int u = 0; u < BC / 16; ++u) pf[b][u] = zero_frag<T>();
        s[b][0] = zero16();
        s[b][1] = zero16();
      }
      return;
    }
    const int kv0 = t * BC;
    if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0)) {
      keep_branch();
#pragma unroll
      for (int b = 0; b < RBW; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (CAUSAL && key > qw0 + 32 * b + l32)) s[b][kb][r] = -INFINITY;
          }
    }
    // Reductions run as four independent chains of three-input maxima: one
    // wave alone issues this vector work, so dependent-instruction latency
    // would show.  Chain q takes the elements r % 4 == q of both key blocks.
    // One rescale branch serves all row blocks (a block whose max has not
    // moved past the threshold rescales exactly, by alpha <= 1).
    float mc[RBW];
    bool up = false;
#pragma unroll
    for (int b = 0; b < RBW; ++b) {
      float mx4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x = vmax3(s[b][0][q], s[b][0][q + 4], s[b][0][q + 8]);
        x = vmax3(x, s[b][0][q + 12], s[b][1][q]);
        x = vmax3(x, s[b][1][q + 4], s[b][1][q + 8]);
        mx4[q] = vmax(x, s[b][1][q + 12]);
      }
      mc[b] = vmax_halves(vmax(vmax3(mx4[0], mx4[1], mx4[2]), mx4[3])) * c;
      up = up || (mc[b] > m[b] + kLazyRescale<T>);
    }
    if (__ballot(up)) {
#pragma unroll
      for (int b = 0; b < RBW; ++b) {
        const float m_new = fmaxf(m[b], mc[b]);
        const float alpha = fast_exp2(m[b] - m_new);
        m[b] = m_new;
        lsum[b] *= alpha;
        osum[b][0] *= alpha;   // the only element read (zero in lanes 32-63)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[b][db] *= alpha;
      }
    }
    // Scale and shift every score first, then exponentiate: no exp2 waits on
    // the instruction just before it.
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][kb][r] = __builtin_fmaf(s[b][kb][r], c, -m[b]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][kb][r] = fast_exp2(s[b][kb][r]);
#pragma unroll
    for (int b = 0; b < RBW; ++b)
#pragma unroll
      for (int u = 0; u < BC / 16; ++u)
        pf[b][u] = to_frag<T>((u & 1) ? half8<1>(s[b][u >> 1]) : half8<0>(s[b][u >> 1]));
  };

  // Softmax slot of tile t in slot pair p: this wave's copies of the pair
  // (K(p+3) into the buffer of K(p-1), last read in slot 2p-1; V(p+2) into
  // that of V(p-2), last read in slot 2p-1), the read-ahead of the first V
  // fragments of its next matrix slot (tile t+1, so V(t)), the softmax, and
  // at the end a wait for its copies of pair p-1 (all but this slot's).  Past
  // the last tile the copies repeat tile jend-1 into buffers no later slot
  // reads, so every slot runs the same instructions.
  auto softmax_slot = [&](int t, int p, int st) {   // st = t % NB, a constant
    copy_tile(Kh, min(p + 3, jend - 1), Kbuf(p + 3));
    copy_tile(Vh, min(p + 2, jend - 1), Vbuf(p + 2));
    read_vpre(st);
    __builtin_amdgcn_sched_barrier(0);
    softmax(t);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * SPW>();   // this wave's copies of pair p-1 have landed
  };

  // Slot pair u: slot 2u (group 0: matrix slot of tile u; group 1: softmax
  // slot of tile u-1), slot 2u+1 (group 0: softmax of tile u; group 1: matrix
  // slot of tile u); both softmax slots of pair u carry the copies of pair u.
  // Both groups run one straight-line loop body, so the accumulators stay in
  // place; group 1 enters one slot late, and an extra barrier for group 0 at
  // the end keeps the barrier counts equal.  The loop is unrolled by the ring
  // depth, so the ring stage of every LDS read is a constant: each address is
  // a per-lane offset plus an immediate, with no address arithmetic per tile.
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

  // One 32-row block at a time through this wave's staging rows.
#pragma unroll
  for (int b = 0; b < RBW; ++b) {
    const int r0 = qw0 + 32 * b;
    if (r0 < N) {
      const float ltot = lsum[b] + __shfl_xor(lsum[b], 32);
      float lqtot = osum[b][0] + __shfl_xor(osum[b][0], 32);
      // Queries q and q + 16 share a column of the row-sum products, whose zero
      // selector entries still multiply the other query's probabilities: a NaN
      // there (a NaN input in that row) makes this sum NaN as well.  The query's
      // own fp32 sum is then finite and stands in for it (the two differ only by
      // the rounding of P); a NaN of the query's own leaves both NaN.
      if (__builtin_isnan(lqtot) && !__builtin_isnan(ltot)) lqtot = ltot;
      store_rows_lds<T, D>(L + wave * kStageBytes<D>, o[b], 1.0f / lqtot, a.O + hoff + (size_t)r0 * D, N - r0, lane);
      if (g == 0 && r0 + l32 < N) a.LSE[(size_t)bh * N + r0 + l32] = (m[b] + __builtin_log2f(ltot)) * kLn2;
    }
  }
}

template <typename T, int D, bool CAUSAL, bool MAP>
hipError_t launch_fwd_inst(const FwdArgs<T>& a, hipStream_t st) {
  FwdArgs<T> args = a;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)(a.nQ * a.BH)), block(64 * kFwdWaves);
  if constexpr (sizeof(T) == 2)
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_pp_kernel<T, D, CAUSAL, MAP>), grid,
                           dim3(512), kargs, 0, st);
  else
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_kernel<T, D, CAUSAL, MAP>), grid,
                           block, kargs, 0, st);
}

template <typename T>
hipError_t launch_fwd(const FwdArgs<T>& a, int d, bool causal, bool map, hipStream_t st) {
  if (d == 64) {
    if (causal) return map ? launch_fwd_inst<T, 64, true, true>(a, st) : launch_fwd_inst<T, 64, true, false>(a, st);
    return map ? launch_fwd_inst<T, 64, false, true>(a, st) : launch_fwd_inst<T, 64, false, false>(a, st);
  }
  if (causal) return map ? launch_fwd_inst<T, 128, true, true>(a, st) : launch_fwd_inst<T, 128, true, false>(a, st);
  return map ? launch_fwd_inst<T, 128, false, true>(a, st) : launch_fwd_inst<T, 128, false, false>(a, st);
}

template hipError_t launch_fwd<bf16_t>(const FwdArgs<bf16_t>&, int, bool, bool, hipStream_t);
template hipError_t launch_fwd<f16_t>(const FwdArgs<f16_t>&, int, bool, bool, hipStream_t);
template hipError_t launch_fwd<float>(const FwdArgs<float>&, int, bool, bool, hipStream_t);

}  // namespace fa

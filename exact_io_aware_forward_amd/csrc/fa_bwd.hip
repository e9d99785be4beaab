// Backward kernels: D = rowsum(dO * O), then dK/dV and dQ by recomputing the
// probabilities from Q, K and the saved log-sum-exp instead of storing them
// (Lecture 9 notes, cs2680.com, section 9.6; CMU 11-868 FlashAttention notes,
// quidproquo.cc, "Recomputation: compute a little more, move a lot less",
// slide page 14).  The gradient formulas are the chain rule through the row
// softmax: P = exp(scale*S - LSE), dV = P^T dO, dP = dO V^T,
// dS = P * (dP - D), dK = scale * dS^T Q, dQ = scale * dS K.
//
// Two accumulation kernels and no atomics: the dK/dV kernel owns a key tile
// and walks query tiles; the dQ kernel owns a query tile and walks key tiles.
// Every product is laid out so the recomputed tile is consumed as an MFMA B
// operand straight from its accumulator registers (see fa_device.h).  Operands
// whose contraction index is the row index in memory (dO and Q for dV/dK, K
// for dQ) are read from the same row-major LDS tile with the LDS transpose
// read, so each streamed tile is stored once; tiles read both ways use the
// XOR-swizzled layout of SwzTile.  Streamed tiles reach LDS by buffer-to-LDS
// copies into a four-stage ring, issued two (dQ) or three (dK/dV) tiles ahead; rows past N come
// in as zeros.  In both accumulation kernels the vector work of one tile
// overlaps matrix work: dK/dV (one wave per SIMD) is software-pipelined within
// the wave, dQ runs two wave groups in ping-pong.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ------------------------------------------------------------------ preprocess
// D[row] = sum_c dO[row, c] * O[row, c] in fp32; one group of D/EPC lanes per row.
// Also L2[row] = LSE[row] * log2(e), the form the dK/dV kernel streams.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                     const T* __restrict__ dO,
                                                     const float* __restrict__ LSE,
                                                     float* __restrict__ Dvec,
                                                     float* __restrict__ L2, long rows) {
  constexpr int EPC = kEPC<T>;
  constexpr int LPR = D / EPC;
  constexpr int RPB = 256 / LPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ld16(O + row * D + sub * EPC);
    const u32x4 b = ld16(dO + row * D + sub * EPC);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc = __builtin_fmaf(chunk_elem<T>(a, e), chunk_elem<T>(b, e), acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && sub == 0) {
    Dvec[row] = acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ------------------------------------------------------------------ dK / dV
// One workgroup per 128-key tile (4 waves x 32 keys), walking query tiles of
// BQ = kDkvBQ(D) rows from the causal diagonal.  At d = 128 a wave needs more
// than 256 registers (dK and dV accumulators, K and V fragments, S and dP), so
// one wave runs per SIMD; at d = 64 with 32-query tiles it fits in 256 and two
// workgroups share a compute unit.  Per query tile i and wave:
//   A(i): S = Q K^T and dP = dO V^T (Q and dO rows from LDS, K and V of the
//         wave's keys held in registers as B operands);
//   B(i): P = exp2(S c - LSE log2e), dS = P (dP - D) on the vector ALU;
//   C(i): dV^T += dO^T P and dK^T += Q^T dS (the transposed operands by the
//         LDS transpose read).
// With one wave per SIMD the matrix and vector work have to overlap within the
// wave (at d = 64 the second wave helps): the loop is software-pipelined so that B(i) and A(i+1), which are
// independent once B has read S(i) and dP(i), form one instruction stream for
// the scheduler to interleave, followed by C(i).  Query tiles (Q, dO, LSE*log2e, D) stream through a ring
// of four LDS stages filled by buffer-to-LDS copies: in iteration i each wave
// issues its share of tile i+3 and, before the barrier that ends the
// iteration, waits for its copies of tile i+2 (read from iteration i+1 on).
// Rows past N come in as zeros: with Q = dO = 0 and D = 0 such a row adds
// nothing to dV, dK or dS whatever its P.
template <typename T, int D, bool CAUSAL, bool MAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void bwd_dkdv_kernel(BwdArgs<T> a) {
  using Tile = SwzTile<D>;
  constexpr int BKV = kDkvBKV;  // keys per workgroup (4 waves x 32)
  constexpr int BQ = kDkvBQ(D);  // queries per streamed tile
  constexpr int RB = Tile::kRowBytes;
  constexpr int CPR = Tile::kChunks;
  constexpr int TB = BQ * RB;                // one Q or dO tile
  constexpr int SB = 2 * TB + 2 * 256;      // stage: Q, dO, LSE*log2e, D (256 B each, BQ used)
  constexpr int NS = 4;                      // ring depth
  constexpr int SPW = TB / 1024 / 4;         // 1 KB copy segments per wave per Q or dO tile
  static_assert((BQ == 32 || BQ == 64) && SPW * 4 * 1024 == TB,
                "tile must split into 1 KB segments over 4 waves");
  constexpr int NF = D / 16, NV = D / 32, NU = BQ / 16, QB = BQ / 32;
  constexpr int NDMA = 2 * SPW + 1;          // copies per wave per tile

  __shared__ __attribute__((aligned(16))) char smem[NS * SB];
  lds_t* const L = (lds_t*)smem;
  const unsigned lds_base = (unsigned)(size_t)L;
  auto stage = [&](int i) { return (i & (NS - 1)) * SB; };   // byte offset of tile i's stage

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int nKV = (N + BKV - 1) / BKV;

  // One workgroup per (key/value head, part of its group, key tile).  The G
  // query heads sharing the key/value head are adjacent; the GS parts take
  // GW = G / GS of them each (bq0 .. bq0 + GW - 1) and walk them one after the
  // other, so dK and dV accumulate their sum in registers (no atomics).  With
  // GS > 1 each part stores its fp32 sums and a reduction kernel adds the
  // parts in a fixed order.
  const int G = a.group, GS = a.gsplit, GW = G / GS;
  const int BHkv = a.BH / G;
  int bhv, kj;
  map_block(blockIdx.x, nKV, BHkv * GS, false, bhv, kj);
  const int bh = bhv / GS, sp = bhv - bh * GS;   // key/value head, part of its group
  const size_t hoff = (size_t)bh * N * D;
  const size_t bq0 = (size_t)bh * G + (size_t)sp * GW;
  const T* __restrict__ Qh = a.Q + bq0 * N * D;
  const T* __restrict__ dOh = a.dO + bq0 * N * D;
  const float* __restrict__ L2h = a.L2 + bq0 * N;
  const float* __restrict__ Dh = a.Dvec + bq0 * N;

  const int k0 = kj * BKV;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;

  // K and V of this lane's key as B operands (col = key, d = 16t + 8g ..).
  frag_t<T> kf[NF], vf[NF];
  {
    const int kc = min(key, N - 1);
#pragma unroll
    for (int t = 0; t < NF; ++t) {
      kf[t] = ld_frag(a.K + hoff + (size_t)kc * D + 16 * t + 8 * g);
      vf[t] = ld_frag(a.V + hoff + (size_t)kc * D + 16 * t + 8 * g);
    }
  }

  const int nQb = (N + BQ - 1) / BQ;
  const int i0 = CAUSAL ? k0 / BQ : 0;
  // Stream position u (0 .. nU - 1) is query tile i0 + u % n1 of query head
  // u / n1 of the group; the ring stage follows u.  Positions are visited in
  // order, so the copy front and the current tile are kept as (row of the
  // head's first row, first query row of the tile) and advanced by additions.
  const int n1 = nQb - i0;
  const int nU = GW * n1;
  const int qa_first = i0 * BQ, qa_end = nQb * BQ;
  int cp_pos = 0, cp_qa = qa_first;   // next position to copy
  const T* cp_q = Qh;                 // its head's Q, dO, LSE*log2e and D
  const T* cp_do = dOh;
  const float* cp_l2 = L2h;
  const float* cp_d = Dh;
  int cur_qa = qa_first;              // first query row of the tile being computed
  // Instrumented instance: the class of every (key tile, query tile) pair, by
  // the same closed-form rule that sets i0 (query tiles before i0 are code 0).
  if (MAP)
    for (int i = tid; i < nQb; i += 256)
      a.map_dkdv[((size_t)bh * nKV + kj) * nQb + i] = (unsigned char)tile_code(i, kj, BQ, BKV, N, CAUSAL);

  // Copies of query tile i: segment sg (1 KB) of the Q and dO tiles by wave
  // sg / SPW, lane l filling physical chunk l of the segment (row r, logical
  // chunk pc ^ swz(r)); one float per lane of LSE*log2e (waves 0, 2) or D
  // (waves 1, 3), the pairs writing the same values.
  int dma_off[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int ci = (wave * SPW + k) * 64 + lane;
    const int r = ci / CPR, pc = ci % CPR;
    dma_off[k] = r * RB + ((pc ^ Tile::swz(r)) << 4);
  }
  // Copy of the tile at the copy front into the stage of position u (u is the
  // front, or past the end: then the last tile is copied again, into its own
  // stage, with the same data); the front advances while it is before the end.
  auto copy_tile = [&](int u) {
    const int qa = cp_qa;
    const unsigned rows_bytes = (unsigned)((N - qa) * RB);
    const u32x4 rq = raw_rsrc(cp_q + (size_t)qa * D, rows_bytes);
    const u32x4 rd = raw_rsrc(cp_do + (size_t)qa * D, rows_bytes);
    const u32x4 rv = raw_rsrc(((wave & 1) ? cp_d : cp_l2) + qa, (unsigned)((N - qa) * 4));
    // Advance without branches (selects only), so the loop body stays one
    // basic block for the scheduler's interleave of B1(i) with A(i+1).
    const int adv = cp_pos < nU - 1 ? 1 : 0;
    cp_pos += adv;
    const int nqa = cp_qa + adv * BQ;
    const bool wrap = nqa >= qa_end;            // only after an advance
    cp_qa = wrap ? qa_first : nqa;
    const int hrows = wrap ? N : 0;
    cp_q += (size_t)hrows * D;
    cp_do += (size_t)hrows * D;
    cp_l2 += hrows;
    cp_d += hrows;
    const unsigned st = lds_base + stage(u);
#pragma unroll
    for (int k = 0; k < SPW; ++k) dma16(rq, st + (wave * SPW + k) * 1024, dma_off[k]);
#pragma unroll
    for (int k = 0; k < SPW; ++k) dma16(rd, st + TB + (wave * SPW + k) * 1024, dma_off[k]);
    // 64 floats from row qa (past row BQ they belong to the next tile and are
    // not read).
    dma4(rv, st + 2 * TB + (wave & 1) * 256, lane * 4);
  };

  // Tile-invariant per-lane LDS offsets.
  int a_off[NF];
#pragma unroll
  for (int t = 0; t < NF; ++t) a_off[t] = Tile::a_off(lane, t);
  int tr_off[2][NV];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < NV; ++db) tr_off[h][db] = Tile::tr_off(lane, h, db);

  f32x16 dv[NV], dk[NV];
#pragma unroll
  for (int db = 0; db < NV; ++db) {
    dv[db] = zero16();
    dk[db] = zero16();
  }
  const float c = a.scale_log2;

  // A(i): S and dP of tile i into (s, dp).  Step k (query block k / NF,
  // d step k % NF) reads its Q and dO fragments AH steps ahead, so only a
  // short window of operand registers is live.
  auto tile_a = [&](int i, f32x16(&s)[QB], f32x16(&dp)[QB]) {
    constexpr int AH = 4, NK = QB * NF;
    const lds_t* qs = L + stage(i);
    const lds_t* ds = qs + TB;
    frag_t<T> af[AH + 1], bf[AH + 1];
    auto rd = [&](int k) {
      const int off = (k / NF) * 32 * RB + a_off[k % NF];
      af[k % (AH + 1)] = lds_ld<frag_t<T>>(qs + off);
      bf[k % (AH + 1)] = lds_ld<frag_t<T>>(ds + off);
    };
#pragma unroll
    for (int k = 0; k < AH; ++k) rd(k);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (k + AH < NK) rd(k + AH);
      const int qb = k / NF, t = k % NF;
      if (t == 0) {
        s[qb] = zero16();
        dp[qb] = zero16();
      }
      s[qb] = mma(af[k % (AH + 1)], kf[t], s[qb]);
      dp[qb] = mma(bf[k % (AH + 1)], vf[t], dp[qb]);
    }
  };
  // B(i), in two parts.  B1 reads S(i) and dP(i) into fresh registers and
  // forms P and dP - D; it shares a basic block with A(i+1), so the scheduler
  // can interleave the two.  B2 masks the diagonal (a branch, taken on
  // diagonal tiles only), forms dS and the operand fragments.
  frag_t<T> pf[NU], sf[NU];
  f32x16 pv[QB], sv[QB];
  auto tile_b1 = [&](int i, const f32x16(&s)[QB], const f32x16(&dp)[QB]) {
    const lds_t* lb = L + stage(i) + 2 * TB;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ql = qb * 32 + 8 * rg + 4 * g;
        const f32x4 l4 = lds_ld<f32x4>(lb + 4 * ql);
        const f32x4 d4 = lds_ld<f32x4>(lb + 256 + 4 * ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          pv[qb][r] = fast_exp2(__builtin_fmaf(s[qb][r], c, -l4[e]));
          sv[qb][r] = dp[qb][r] - d4[e];
        }
      }
  };
  auto tile_b2 = [&](int u) {
    const int qa = cur_qa;
    if (CAUSAL && qa < kw0 + 31) {   // diagonal tiles: masked scores -> P = 0
      keep_branch();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key > qa + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3)) pv[qb][r] = 0.f;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[qb][r] *= pv[qb][r];
      pf[2 * qb] = to_frag<T>(half8<0>(pv[qb]));
      pf[2 * qb + 1] = to_frag<T>(half8<1>(pv[qb]));
      sf[2 * qb] = to_frag<T>(half8<0>(sv[qb]));
      sf[2 * qb + 1] = to_frag<T>(half8<1>(sv[qb]));
    }
  };
  // C(i): dV^T += dO^T P, dK^T += Q^T dS.  Step k (u = k / NV, db = k % NV)
  // reads its two transposed fragments CH steps ahead.
  auto tile_c = [&](int i) {
    constexpr int CH = 2, NK = NU * NV;
    const lds_t* qs = L + stage(i);
    const lds_t* ds = qs + TB;
    frag_t<T> tq[CH + 1], td[CH + 1];
    auto rd = [&](int k) {
      const int u = k / NV, db = k % NV;
      td[k % (CH + 1)] = tr_frag<T>(ds + 16 * u * RB + tr_off[0][db], ds + 16 * u * RB + tr_off[1][db]);
      tq[k % (CH + 1)] = tr_frag<T>(qs + 16 * u * RB + tr_off[0][db], qs + 16 * u * RB + tr_off[1][db]);
    };
#pragma unroll
    for (int k = 0; k < CH; ++k) rd(k);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (k + CH < NK) rd(k + CH);
      const int u = k / NV, db = k % NV;
      dv[db] = mma(td[k % (CH + 1)], pf[u], dv[db]);
      dk[db] = mma(tq[k % (CH + 1)], sf[u], dk[db]);
    }
  };
  // One iteration: copies of tile i+3, B1(i) with A(i+1), B2(i), C(i), wait
  // for this wave's copies of tile i+2, barrier.  B1(i) reads S(i) and dP(i)
  // into fresh registers at its start, after which A(i+1) may overwrite them:
  // one set of accumulators serves both tiles.
  f32x16 s[QB], dp[QB];
  auto iteration = [&](int u) {
    copy_tile(min(u + 3, nU - 1));
    tile_b1(u, s, dp);
    tile_a(u + 1, s, dp);
    __builtin_amdgcn_sched_barrier(0);
    tile_b2(u);
    tile_c(u);
    cur_qa = cur_qa + BQ >= qa_end ? qa_first : cur_qa + BQ;
    wait_vmcnt<NDMA>();
    lds_barrier();
  };

  if (nU > 0) {
    copy_tile(0);
    copy_tile(min(1, nU - 1));
    copy_tile(min(2, nU - 1));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    tile_a(0, s, dp);
    for (int u = 0; u < nU; ++u) iteration(u);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
  }
  lds_barrier();   // every wave's copies have landed and its reads returned: LDS is free

  static_assert(4 * kStageBytes<D> <= NS * SB, "output staging fits the ring");
  if (GS == 1) {
    // dK and dV through this wave's LDS staging rows, one after the other.
    lds_t* const stg = L + wave * kStageBytes<D>;
    store_rows_lds<T, D>(stg, dk, a.scale, a.dK + hoff + (size_t)kw0 * D, N - kw0, lane);
    store_rows_lds<T, D>(stg, dv, 1.0f, a.dV + hoff + (size_t)kw0 * D, N - kw0, lane);
  } else if (key < N) {
    const size_t tensor = (size_t)GS * BHkv * N * D;   // floats per partial tensor
    float* pk = a.dkv_part + (((size_t)sp * BHkv + bh) * N + key) * D;
    float* pv = pk + tensor;
#pragma unroll
    for (int db = 0; db < NV; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int col = db * 32 + 8 * rg + 4 * g;
        const f32x4 k4 = {dk[db][4 * rg] * a.scale, dk[db][4 * rg + 1] * a.scale,
                          dk[db][4 * rg + 2] * a.scale, dk[db][4 * rg + 3] * a.scale};
        const f32x4 v4 = {dv[db][4 * rg], dv[db][4 * rg + 1], dv[db][4 * rg + 2], dv[db][4 * rg + 3]};
        *reinterpret_cast<f32x4*>(pk + col) = k4;
        *reinterpret_cast<f32x4*>(pv + col) = v4;
      }
  }
}

// Sum of the GS parts' fp32 dK and dV, in part order (deterministic), rounded
// once to the output type.  Thread i handles four consecutive elements.
template <typename T>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ part,
                                                            T* __restrict__ dK, T* __restrict__ dV,
                                                            long n4, int GS) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* pk = reinterpret_cast<const f32x4*>(part);
  const f32x4* pv = pk + (size_t)GS * n4;
  f32x4 sk = pk[i], sv = pv[i];
  for (int s = 1; s < GS; ++s) {
    sk += pk[(size_t)s * n4 + i];
    sv += pv[(size_t)s * n4 + i];
  }
  T k4[4], v4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k4[e] = (T)sk[e];
    v4[e] = (T)sv[e];
  }
  *reinterpret_cast<u32x2*>(dK + 4 * i) = __builtin_bit_cast(u32x2, k4);
  *reinterpret_cast<u32x2*>(dV + 4 * i) = __builtin_bit_cast(u32x2, v4);
}

// ------------------------------------------------------------------ dQ
// One workgroup of 8 waves per 256-query tile (32 queries per wave), walking
// key tiles of BKV = kDqBKV(D) rows up to the causal diagonal.  Per key tile j
// and wave:
//   A(j): S^T = K Q^T and dP^T = V dO^T - D (K and V rows from LDS; Q^T and
//         dO^T of the wave's queries held in registers as B operands);
//   B(j): P = exp2(S c - LSE log2e), dS = P (dP - D) on the vector ALU, in
//         place, and dS^T as B operands;
//   C(j): dQ^T += K^T dS^T (K^T by the LDS transpose read).
// The waves run in ping-pong like the 16-bit forward: waves w and w + 4 share
// a SIMD and form two groups offset by one slot; slots are separated by
// workgroup barriers, and a wave alternates a matrix slot M(j) = C(j-1), A(j)
// (raised issue priority, LDS reads four product steps ahead, each step
// fenced) with a vector slot V(j) = B(j), so in every slot one wave of each
// SIMD issues MFMAs while the other does its vector work (measured at N = 4096,
// d = 128: 6 % faster than two independent 4-wave workgroups per CU, the same
// registers per wave).  Key tiles (K and V) stream through a ring of four LDS
// stages shared by the 8 waves: in slot pair p every wave copies its eighth
// of tile p + 2 in its vector slot, into the stage of tile p - 2 (last read in
// slot 2p - 1), and waits for its copies of pair p - 1 at the end of that
// slot; tile p + 1 is first read in slot 2p + 2.  Keys past N come in as
// zeros and are masked (P = 0).
template <typename T, int D, bool CAUSAL, bool MAP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs<T> a) {
  using Tile = SwzTile<D>;
  constexpr int BQ = kDqBQ;        // queries per workgroup (8 waves x 32)
  static_assert(BQ == 256, "8 waves x 32 queries");
  constexpr int BKV = kDqBKV(D);   // keys per streamed tile
  constexpr int RB = Tile::kRowBytes;
  constexpr int CPR = Tile::kChunks;
  constexpr int TB = BKV * RB;               // one K or V tile
  constexpr int SB = 2 * TB;                 // stage: K, V
  constexpr int NS = 4;                      // ring depth
  constexpr int SPW = TB / 1024 / 8;         // 1 KB copy segments per wave per K or V tile
  static_assert(SPW >= 1 && SPW * 8 * 1024 == TB, "tile must split into 1 KB segments over 8 waves");
  constexpr int NF = D / 16, NV = D / 32, NU = BKV / 16, KB = BKV / 32;
  constexpr int NC = NU * NV, NA = KB * NF;  // product steps of C and of A
  constexpr int NDMA = 2 * SPW;              // copies per wave per slot pair
  constexpr int CH = 3, LA = 4;              // C fragments read in the vector slot; read-ahead
  static_assert(CH <= NC && CH <= LA, "read-ahead covers the prefetched fragments");
  constexpr int RING = NS * SB, STG = 8 * kStageBytes<D>;

  __shared__ __attribute__((aligned(16))) char smem[RING > STG ? RING : STG];
  lds_t* const L = (lds_t*)smem;
  const unsigned lds_base = (unsigned)(size_t)L;

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;
  const int rblk = 2 * (wave & 3) + grp;   // the two waves of a SIMD hold adjacent row blocks
  const int nQb = (N + BQ - 1) / BQ;

  int bh, qi;
  map_block(blockIdx.x, nQb, a.BH, CAUSAL, bh, qi);
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / a.group) * N * D;   // the query head's key/value head
  const T* __restrict__ Kh = a.K + kvoff;
  const T* __restrict__ Vh = a.V + kvoff;

  const int q0 = qi * BQ;
  const int qw0 = q0 + 32 * rblk;
  const int qrow = qw0 + l32;

  // Q and dO of this wave's rows as B operands, and for the fused preprocess
  // the same fragments of O and the row's LSE, all requested before the first
  // key tiles' copies.
  frag_t<T> qf[NF], dof[NF];
  u32x4 ofr[NF];
  float lse_row;
  {
    const int qc = min(qrow, N - 1);
#pragma unroll
    for (int t = 0; t < NF; ++t) {
      qf[t] = ld_frag(a.Q + hoff + (size_t)qc * D + 16 * t + 8 * g);
      dof[t] = ld_frag(a.dO + hoff + (size_t)qc * D + 16 * t + 8 * g);
      ofr[t] = __builtin_bit_cast(u32x4, ld_frag(a.O + hoff + (size_t)qc * D + 16 * t + 8 * g));
    }
    lse_row = a.LSE[(size_t)bh * N + qc];
  }
  float dq_d = 0.f, lse2 = 0.f;

  const int nKb = (N + BKV - 1) / BKV;
  int jend = nKb;
  if (CAUSAL) jend = min(nKb, (min(q0 + BQ, N) - 1) / BKV + 1);
  // Key tiles this wave has work in: [0, wend).
  int wend = qw0 < N ? jend : 0;
  if (CAUSAL && qw0 < N) wend = min(jend, min(qw0 + 31, N - 1) / BKV + 1);
  if (MAP)
    for (int j = tid; j < nKb; j += 512)
      a.map_dq[((size_t)bh * nQb + qi) * nKb + j] = (unsigned char)tile_code(qi, j, BQ, BKV, N, CAUSAL);

  int dma_off[SPW];
#pragma unroll
  for (int k = 0; k < SPW; ++k) {
    const int ci = (wave * SPW + k) * 64 + lane;
    const int r = ci / CPR, pc = ci % CPR;
    dma_off[k] = r * RB + ((pc ^ Tile::swz(r)) << 4);
  }
  auto copy_tile = [&](int j, int sg) {   // this wave's share of tile j into ring stage sg
    const int kv0 = j * BKV;
    const unsigned rows_bytes = (unsigned)((N - kv0) * RB);
    const u32x4 rk = raw_rsrc(Kh + (size_t)kv0 * D, rows_bytes);
    const u32x4 rv = raw_rsrc(Vh + (size_t)kv0 * D, rows_bytes);
    const unsigned st = lds_base + sg * SB;
#pragma unroll
    for (int k = 0; k < SPW; ++k) dma16(rk, st + (wave * SPW + k) * 1024, dma_off[k]);
#pragma unroll
    for (int k = 0; k < SPW; ++k) dma16(rv, st + TB + (wave * SPW + k) * 1024, dma_off[k]);
  };

  int a_off[NF];
#pragma unroll
  for (int t = 0; t < NF; ++t) {
    a_off[t] = Tile::a_off(lane, t);
    asm volatile("" : "+v"(a_off[t]));
  }
  int tr_off[2][NV];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < NV; ++db) {
      tr_off[h][db] = Tile::tr_off(lane, h, db);
      asm volatile("" : "+v"(tr_off[h][db]));
    }

  f32x16 dq[NV];
#pragma unroll
  for (int db = 0; db < NV; ++db) dq[db] = zero16();
  const float c = a.scale_log2;
  f32x16 s[KB], dp[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    s[kb] = zero16();
    dp[kb] = zero16();
  }
  frag_t<T> sf[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) sf[u] = zero_frag<T>();
  frag_t<T> cpre[CH];   // the first C fragments of the next matrix slot

  auto rd_c = [&](int sg, int k) {   // K^T fragment of C step k from stage sg
    const lds_t* ks = L + sg * SB;
    const int u = k / NV, db = k % NV;
    return tr_frag<T>(ks + 16 * u * RB + tr_off[0][db], ks + 16 * u * RB + tr_off[1][db]);
  };

  // Matrix slot of tile j (stage sg = j % NS): C(j-1) from the previous stage
  // (dS of tile j-1, zero before the first tile), then A(j), as one stream
  // whose LDS reads run LA steps ahead; each step is fenced.
  auto matrix_slot = [&](int sg) {
    __builtin_amdgcn_s_setprio(2);
    const int sp = (sg + NS - 1) & (NS - 1);
    const lds_t* ks = L + sg * SB;
    const lds_t* vs = ks + TB;
    frag_t<T> tk[NC], af[NA], bf[NA];
#pragma unroll
    for (int k = 0; k < CH; ++k) tk[k] = cpre[k];
    auto rd = [&](int i) {
      if (i < NC) {
        tk[i] = rd_c(sp, i);
      } else {
        const int k = i - NC;
        const int off = (k / NF) * 32 * RB + a_off[k % NF];
        af[k] = lds_ld<frag_t<T>>(ks + off);
        bf[k] = lds_ld<frag_t<T>>(vs + off);
      }
    };
#pragma unroll
    for (int i = CH; i < LA; ++i) rd(i);
#pragma unroll
    for (int i = 0; i < NC + NA; ++i) {
      if (i + LA < NC + NA) rd(i + LA);
      if (i < NC) {
        dq[i % NV] = mma(tk[i], sf[i / NV], dq[i % NV]);
      } else {
        const int k = i - NC, kb = k / NF, t = k % NF;
        if (t == 0) {
          s[kb] = zero16();
          dp[kb] = (f32x16)(-dq_d);
        }
        s[kb] = mma(af[k], qf[t], s[kb]);
        dp[kb] = mma(bf[k], dof[t], dp[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Vector slot of tile j (stage sg = j % NS) in slot pair p: this wave's
  // copies of tile p + 2, B(j) in place (P, then dS = P (dP - D) and its
  // operand fragments; zero where the wave has no work), the first C
  // fragments of the next matrix slot, and a wait for the copies of pair p-1.
  auto vector_slot = [&](int j, int p, int sg) {
    copy_tile(min(p + 2, jend - 1), (p + 2) & (NS - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (j < 0 || j >= wend) {
#pragma unroll
      for (int u = 0; u < NU; ++u) sf[u] = zero_frag<T>();
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -lse2));
      const int kv0 = j * BKV;
      if ((kv0 + BKV > N) || (CAUSAL && kv0 + BKV - 1 > qw0)) {
        keep_branch();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (kk >= N || (CAUSAL && kk > qrow)) s[kb][r] = 0.f;
          }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[kb][r] *= s[kb][r];
        sf[2 * kb] = to_frag<T>(half8<0>(dp[kb]));
        sf[2 * kb + 1] = to_frag<T>(half8<1>(dp[kb]));
      }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) cpre[k] = rd_c(sg, k);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<NDMA>();
  };

  // Prologue: tiles 0 and 1 in stages 0 and 1; stage 3's K tile, read by the
  // first matrix slot's C step (with dS = 0), zeroed.
  copy_tile(0, 0);
  copy_tile(min(1, jend - 1), 1);
#pragma unroll
  for (int c2 = 0; c2 < TB / 16 / 512; ++c2)
    lds_st<u32x4>(L + 3 * SB + (tid + c2 * 512) * 16, (u32x4)(0u));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // The preprocess for this workgroup's rows, fused: D = rowsum(dO * O) from
  // the dO and O fragments (the two lane halves hold the two halves of a row),
  // and LSE * log2(e).  Both are stored for the dK/dV kernel, which runs after
  // this one.  The fragments pass through an empty asm after the wait, so the
  // arithmetic is not hoisted above the copies (which would then wait for the
  // loads before they are issued).
  {
#pragma unroll
    for (int t = 0; t < NF; ++t) asm volatile("" : "+v"(dof[t]), "+v"(ofr[t]));
    asm volatile("" : "+v"(lse_row));
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < NF; ++t) {
      const u32x4 dc = __builtin_bit_cast(u32x4, dof[t]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(chunk_elem<T>(dc, e), chunk_elem<T>(ofr[t], e), acc);
    }
    dq_d = acc + __shfl_xor(acc, 32);
    lse2 = lse_row * kLog2e;
    if (qrow < N && g == 0) {
      a.Dvec[(size_t)bh * N + qrow] = dq_d;
      a.L2[(size_t)bh * N + qrow] = lse2;
    }
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < CH; ++k) cpre[k] = rd_c(3, k);   // stage 3's zeros, published by the barrier

  // Slot pair u: group 0 runs M(u) then V(u); group 1, one slot later, V(u-1)
  // then M(u).  Both run one straight-line body (unrolled by the ring depth,
  // so every LDS read has a constant stage); group 1 enters with V(-1) and
  // group 0 leaves with one extra barrier, so the barrier counts match.
  if (grp == 1) {
    vector_slot(-1, 0, NS - 1);
    lds_barrier();
  }
  for (int u0 = 0;; u0 += NS) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (u0 + k > jend) break;
      matrix_slot(k);
      lds_barrier();
      vector_slot(u0 + k, u0 + k + grp, k);
      lds_barrier();
    }
    if (u0 + NS > jend) break;
  }
  if (grp == 0) lds_barrier();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may land after the workgroup ends
  lds_barrier();   // every wave's copies have landed and its reads returned: LDS is free

  static_assert(8 * kStageBytes<D> <= sizeof(smem), "output staging fits");
  store_rows_lds<T, D>(L + wave * kStageBytes<D>, dq, a.scale, a.dQ + hoff + (size_t)qw0 * D, N - qw0, lane);
}

// ------------------------------------------------------------------ launch
template <typename T, int D, bool CAUSAL>
hipError_t launch_stage_inst(const BwdArgs<T>& a, BwdStage stage, hipStream_t st) {
  BwdArgs<T> args = a;
  void* kargs[] = {&args};
  const dim3 block(256);
  switch (stage) {
    case BwdStage::kPreprocess: {
      constexpr int RPB = 256 / (D / kEPC<T>);
      long rows = (long)a.BH * a.N;
      const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
      const T* O = a.O;
      const T* dO = a.dO;
      const float* LSE = a.LSE;
      float* Dv = a.Dvec;
      float* L2 = a.L2;
      void* pargs[] = {&O, &dO, &LSE, &Dv, &L2, &rows};
      return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_pre_kernel<T, D>), grid, block,
                             pargs, 0, st);
    }
    case BwdStage::kDkDv: {
      const int nKV = (a.N + kDkvBKV - 1) / kDkvBKV;
      const void* k = a.map_dkdv ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<T, D, CAUSAL, true>)
                                 : reinterpret_cast<const void*>(&bwd_dkdv_kernel<T, D, CAUSAL, false>);
      const hipError_t e =
          hipLaunchKernel(k, dim3((unsigned)(nKV * (a.BH / a.group) * a.gsplit)), block, kargs, 0, st);
      if (e != hipSuccess || a.gsplit == 1) return e;
      const long n4 = (long)(a.BH / a.group) * a.N * D / 4;
      const float* part = a.dkv_part;
      T* dK = a.dK;
      T* dV = a.dV;
      int gs = a.gsplit;
      long n4v = n4;
      void* rargs[] = {&part, &dK, &dV, &n4v, &gs};
      return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_reduce_kernel<T>),
                             dim3((unsigned)((n4 + 255) / 256)), block, rargs, 0, st);
    }
    default: {
      const int nQb = (a.N + kDqBQ - 1) / kDqBQ;
      const void* k = a.map_dq ? reinterpret_cast<const void*>(&bwd_dq_kernel<T, D, CAUSAL, true>)
                               : reinterpret_cast<const void*>(&bwd_dq_kernel<T, D, CAUSAL, false>);
      return hipLaunchKernel(k, dim3((unsigned)(nQb * a.BH)), dim3(512), kargs, 0, st);
    }
  }
}

template <typename T>
hipError_t launch_bwd_stage(const BwdArgs<T>& a, int d, bool causal, BwdStage stage,
                            hipStream_t st) {
  if (d == 64)
    return causal ? launch_stage_inst<T, 64, true>(a, stage, st)
                  : launch_stage_inst<T, 64, false>(a, stage, st);
  return causal ? launch_stage_inst<T, 128, true>(a, stage, st)
                : launch_stage_inst<T, 128, false>(a, stage, st);
}

template <typename T>
hipError_t launch_bwd(const BwdArgs<T>& a, int d, bool causal, hipStream_t st) {
  // dQ first: it forms D and LSE * log2(e) of its rows, which dK/dV reads.
  for (BwdStage s : {BwdStage::kDq, BwdStage::kDkDv}) {
    const hipError_t e = launch_bwd_stage<T>(a, d, causal, s, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template hipError_t launch_bwd_stage<bf16_t>(const BwdArgs<bf16_t>&, int, bool, BwdStage,
                                             hipStream_t);
template hipError_t launch_bwd_stage<f16_t>(const BwdArgs<f16_t>&, int, bool, BwdStage,
                                            hipStream_t);
template hipError_t launch_bwd<bf16_t>(const BwdArgs<bf16_t>&, int, bool, hipStream_t);
template hipError_t launch_bwd<f16_t>(const BwdArgs<f16_t>&, int, bool, hipStream_t);

}  // namespace fa

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
// XOR-swizzled layout of SwzTile.  Prefetch loads of the next tile read a
// clamped (always valid) row and are zeroed only when written to LDS, so they
// stay in flight during the current tile's compute; they are issued in parts
// spread over the compute phases (scheduling fences keep them there), because
// all waves issuing a whole tile at once after the barrier queue behind each
// other in the vector-memory path.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ------------------------------------------------------------------ preprocess
// D[row] = sum_c dO[row, c] * O[row, c] in fp32; one group of D/EPC lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                     const T* __restrict__ dO,
                                                     float* __restrict__ Dvec, long rows) {
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
  if (row < rows && sub == 0) Dvec[row] = acc;
}

namespace {

// Store 4 fp32 values of an accumulator row group, scaled, as T (4 consecutive columns).
template <typename T>
__device__ __forceinline__ void store4(T* dst, const f32x16& acc, int rg, float sc) {
  T v4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v4[e] = (T)(acc[4 * rg + e] * sc);
  *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, v4);
}

}  // namespace

// ------------------------------------------------------------------ dK / dV
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs<T> a) {
  using Tile = SwzTile<D>;
  constexpr int BKV = kDkvBKV;  // keys per workgroup (4 waves x 32)
  constexpr int BQ = kDkvBQ;    // queries per streamed tile
  constexpr int EPC = kEPC<T>;
  constexpr int NT = 256;
  constexpr int CPR = Tile::kChunks;
  constexpr int CPT = BQ * CPR / NT;            // 16-byte chunks per thread per tile
  constexpr int TBYTES = BQ * Tile::kRowBytes;  // one Q or dO tile
  constexpr int SBYTES = 2 * TBYTES + 2 * BQ * 4;
  static_assert(CPT * NT == BQ * CPR, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) char smem[2 * SBYTES];
  // stage b: Q tile, dO tile, LSE*log2e [BQ], D [BQ]
  auto Qb = [&](int b) { return (lds_t*)smem + b * SBYTES; };
  auto dOb = [&](int b) { return (lds_t*)smem + b * SBYTES + TBYTES; };
  auto Lb = [&](int b) { return (lds_t*)smem + b * SBYTES + 2 * TBYTES; };
  auto Db = [&](int b) { return (lds_t*)smem + b * SBYTES + 2 * TBYTES + BQ * 4; };

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int nKV = (N + BKV - 1) / BKV;

  int bh, kj;
  map_block(blockIdx.x, nKV, a.BH, false, bh, kj);
  const size_t hoff = (size_t)bh * N * D;
  const T* __restrict__ Qh = a.Q + hoff;
  const T* __restrict__ dOh = a.dO + hoff;
  const float* __restrict__ LSEh = a.LSE + (size_t)bh * N;
  const float* __restrict__ Dh = a.Dvec + (size_t)bh * N;

  const int k0 = kj * BKV;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;

  // K and V of this lane's key as B operands (col = key, d = 16t + 8g ..).
  frag_t<T> kf[D / 16], vf[D / 16];
  {
    const int kc = min(key, N - 1);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      kf[t] = ld_frag(a.K + hoff + (size_t)kc * D + 16 * t + 8 * g);
      vf[t] = ld_frag(a.V + hoff + (size_t)kc * D + 16 * t + 8 * g);
    }
  }

  const int nQb = (N + BQ - 1) / BQ;
  const int i0 = CAUSAL ? k0 / BQ : 0;

  u32x4 qst[CPT], dost[CPT];
  float lse_st = 0.f, d_st = 0.f;
  // Part c (0..3) of the prefetch of query tile i: chunk c of Q and dO (parts
  // beyond CPT are empty), part 0 also the LSE and D rows.
  auto load_part = [&](int i, int c) {
    const int qa = i * BQ;
    if (c < CPT) {
      const int idx = tid + c * NT;
      const unsigned off = (unsigned)(min(idx / CPR, N - 1 - qa) * D + (idx % CPR) * EPC);
      qst[c] = ld16(Qh + (size_t)qa * D + off);
      dost[c] = ld16(dOh + (size_t)qa * D + off);
    }
    if (c == 0) {
      if (tid < BQ) lse_st = LSEh[min(qa + tid, N - 1)];
      else if (tid < 2 * BQ) d_st = Dh[min(qa + tid - BQ, N - 1)];
    }
  };
  auto load_tile = [&](int i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) load_part(i, c);
  };
  auto store_tile = [&](int b, int i) {
    const int valid = N - i * BQ;  // rows [0, valid) are real queries
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / CPR, ch = idx % CPR;
      const bool ok = row < valid;
      lds_st<u32x4>(Qb(b) + Tile::off(row, ch), ok ? qst[c] : (u32x4)(0u));
      lds_st<u32x4>(dOb(b) + Tile::off(row, ch), ok ? dost[c] : (u32x4)(0u));
    }
    // Padding rows: LSE = +inf makes P = 0; D = 0.
    if (tid < BQ) lds_st<float>(Lb(b) + 4 * tid, tid < valid ? lse_st * kLog2e : INFINITY);
    else if (tid < 2 * BQ) lds_st<float>(Db(b) + 4 * (tid - BQ), tid - BQ < valid ? d_st : 0.f);
  };

  // Tile-invariant per-lane LDS offsets.
  int a_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a_off[t] = Tile::a_off(lane, t);
  int tr_off[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) tr_off[h][db] = Tile::tr_off(lane, h, db);

  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dv[db] = zero16();
    dk[db] = zero16();
  }
  const float c = a.scale_log2;

  if (i0 < nQb) {
    load_tile(i0);
    store_tile(0, i0);
  }
  __syncthreads();

  static_assert(CPT <= 4, "prefetch is issued in at most four parts");
  for (int i = i0; i < nQb; ++i) {
    const int buf = (i - i0) & 1;
    const bool more = i + 1 < nQb;
    if (more) load_part(i + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int qa = i * BQ;
    const bool active = kw0 < N && (!CAUSAL || kw0 <= qa + BQ - 1);
    if (active) {
      const bool need_mask = CAUSAL && qa < kw0 + 31;
      const lds_t* qs = Qb(buf);
      const lds_t* ds = dOb(buf);
      // S = Q K^T and dP = dO V^T (rows of the C tiles are queries, cols keys).
      f32x16 s[BQ / 32], dp[BQ / 32];
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        frag_t<T> af[D / 16], bf[D / 16];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          af[t] = lds_ld<frag_t<T>>(qs + qb * 32 * Tile::kRowBytes + a_off[t]);
          bf[t] = lds_ld<frag_t<T>>(ds + qb * 32 * Tile::kRowBytes + a_off[t]);
        }
        s[qb] = zero16();
        dp[qb] = zero16();
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          s[qb] = mma(af[t], kf[t], s[qb]);
          dp[qb] = mma(bf[t], vf[t], dp[qb]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (more) load_part(i + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      // Causal diagonal tiles only: masked scores -> -inf, so P = 0 below.
      if (need_mask) {
        keep_branch();
#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key > qa + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3)) s[qb][r] = -INFINITY;
      }
      // P = exp2(S*c - LSE*log2e), dS = P * (dP - D).
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int ql = qb * 32 + 8 * rg + 4 * g;
          const f32x4 l4 = lds_ld<f32x4>(Lb(buf) + 4 * ql);
          const f32x4 d4 = lds_ld<f32x4>(Db(buf) + 4 * ql);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            const float p = fast_exp2(__builtin_fmaf(s[qb][r], c, -l4[e]));
            s[qb][r] = p;
            dp[qb][r] = p * (dp[qb][r] - d4[e]);
          }
        }
      __builtin_amdgcn_sched_barrier(0);
      if (more) load_part(i + 1, 2);
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS, the transposed operands read with the
      // LDS transpose read from the row-major tiles.
#pragma unroll
      for (int u = 0; u < BQ / 16; ++u) {
        const frag_t<T> pf = to_frag<T>((u & 1) ? half8<1>(s[u >> 1]) : half8<0>(s[u >> 1]));
        const frag_t<T> sf = to_frag<T>((u & 1) ? half8<1>(dp[u >> 1]) : half8<0>(dp[u >> 1]));
        const int ub = 16 * u * Tile::kRowBytes;
        frag_t<T> tq[D / 32], td[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          td[db] = tr_frag<T>(ds + ub + tr_off[0][db], ds + ub + tr_off[1][db]);
          tq[db] = tr_frag<T>(qs + ub + tr_off[0][db], qs + ub + tr_off[1][db]);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = mma(td[db], pf, dv[db]);
          dk[db] = mma(tq[db], sf, dk[db]);
        }
        if (u == 1) {
          __builtin_amdgcn_sched_barrier(0);
          if (more) load_part(i + 1, 3);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (more) {
#pragma unroll
      for (int c = 1; c < 4; ++c) load_part(i + 1, c);
    }
    if (more) store_tile(buf ^ 1, i + 1);
    __syncthreads();
  }

  if (key < N) {
    T* dkrow = a.dK + hoff + (size_t)key * D;
    T* dvrow = a.dV + hoff + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int col = db * 32 + 8 * rg + 4 * g;
        store4<T>(dkrow + col, dk[db], rg, a.scale);
        store4<T>(dvrow + col, dv[db], rg, 1.0f);
      }
  }
}

// ------------------------------------------------------------------ dQ
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BwdArgs<T> a) {
  using Tile = SwzTile<D>;
  constexpr int BQ = kDqBQ;    // queries per workgroup (4 waves x 32)
  constexpr int BKV = kDqBKV;  // keys per streamed tile
  constexpr int EPC = kEPC<T>;
  constexpr int NT = 256;
  constexpr int CPR = Tile::kChunks;
  constexpr int CPT = BKV * CPR / NT;
  constexpr int VROW = D * 2 + 16;               // V: padded rows (row reads only)
  constexpr int KBYTES = BKV * Tile::kRowBytes;  // K: swizzled (row and transpose reads)
  constexpr int SBYTES = KBYTES + BKV * VROW;
  static_assert(CPT * NT == BKV * CPR, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) char smem[2 * SBYTES];
  auto Kb = [&](int b) { return (lds_t*)smem + b * SBYTES; };
  auto Vb = [&](int b) { return (lds_t*)smem + b * SBYTES + KBYTES; };

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int nQb = (N + BQ - 1) / BQ;

  int bh, qi;
  map_block(blockIdx.x, nQb, a.BH, CAUSAL, bh, qi);
  const size_t hoff = (size_t)bh * N * D;
  const T* __restrict__ Kh = a.K + hoff;
  const T* __restrict__ Vh = a.V + hoff;

  const int q0 = qi * BQ;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool wave_rows = qw0 < N;

  frag_t<T> qf[D / 16], dof[D / 16];
  {
    const int qc = min(qrow, N - 1);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = ld_frag(a.Q + hoff + (size_t)qc * D + 16 * t + 8 * g);
      dof[t] = ld_frag(a.dO + hoff + (size_t)qc * D + 16 * t + 8 * g);
    }
  }
  const float lse2 = a.LSE[(size_t)bh * N + min(qrow, N - 1)] * kLog2e;
  const float dq_d = a.Dvec[(size_t)bh * N + min(qrow, N - 1)];

  const int nKb = (N + BKV - 1) / BKV;
  int jend = nKb;
  if (CAUSAL) jend = min(nKb, (min(q0 + BQ, N) - 1) / BKV + 1);

  u32x4 kst[CPT], vst[CPT];
  // Part c (0..3) of the prefetch of key tile j: chunk c of K and V.
  auto load_part = [&](int j, int c) {
    if (c < CPT) {
      const int kv0 = j * BKV;
      const int idx = tid + c * NT;
      const unsigned off = (unsigned)(min(idx / CPR, N - 1 - kv0) * D + (idx % CPR) * EPC);
      kst[c] = ld16(Kh + (size_t)kv0 * D + off);
      vst[c] = ld16(Vh + (size_t)kv0 * D + off);
    }
  };
  auto load_tile = [&](int j) {
#pragma unroll
    for (int c = 0; c < 4; ++c) load_part(j, c);
  };
  auto store_tile = [&](int b, int j) {
    const int valid = N - j * BKV;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / CPR, ch = idx % CPR;
      const bool ok = row < valid;
      lds_st<u32x4>(Kb(b) + Tile::off(row, ch), ok ? kst[c] : (u32x4)(0u));
      lds_st<u32x4>(Vb(b) + row * VROW + ch * 16, ok ? vst[c] : (u32x4)(0u));
    }
  };

  int a_off[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a_off[t] = Tile::a_off(lane, t);
  int tr_off[2][D / 32];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) tr_off[h][db] = Tile::tr_off(lane, h, db);
  const int v_off = l32 * VROW + 16 * g;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = zero16();
  const float c = a.scale_log2;

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  static_assert(CPT <= 4, "prefetch is issued in at most four parts");
  for (int j = 0; j < jend; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < jend;
    if (more) load_part(j + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int kv0 = j * BKV;
    const bool active = wave_rows && (!CAUSAL || kv0 <= qw0 + 31);
    if (active) {
      const bool need_mask = (kv0 + BKV > N) || (CAUSAL && kv0 + BKV - 1 > qw0);
      const lds_t* ks = Kb(buf);
      const lds_t* vs = Vb(buf);
      // S^T = K Q^T and dP^T = V dO^T (cols of the C tiles are this lane's query).
      // The operand reads of key block 1 are issued between the MFMAs of block
      // 0; the K^T fragments of the dQ product are read before the element-wise
      // step so that their latency hides behind it.
      static_assert(BKV == 64, "two key blocks of 32 per tile");
      f32x16 st[2], dpt[2];
      frag_t<T> af[2][D / 16], bf[2][D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        af[0][t] = lds_ld<frag_t<T>>(ks + a_off[t]);
        bf[0][t] = lds_ld<frag_t<T>>(vs + v_off + 32 * t);
      }
      __builtin_amdgcn_sched_barrier(0);
      st[0] = zero16();
      dpt[0] = zero16();
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        st[0] = mma(af[0][t], qf[t], st[0]);
        dpt[0] = mma(bf[0][t], dof[t], dpt[0]);
        af[1][t] = lds_ld<frag_t<T>>(ks + 32 * Tile::kRowBytes + a_off[t]);
        bf[1][t] = lds_ld<frag_t<T>>(vs + 32 * VROW + v_off + 32 * t);
      }
      if (more) load_part(j + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      st[1] = zero16();
      dpt[1] = zero16();
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        st[1] = mma(af[1][t], qf[t], st[1]);
        dpt[1] = mma(bf[1][t], dof[t], dpt[1]);
      }
      frag_t<T> tk[BKV / 16][D / 32];
#pragma unroll
      for (int u = 0; u < BKV / 16; ++u)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int ub = 16 * u * Tile::kRowBytes;
          tk[u][db] = tr_frag<T>(ks + ub + tr_off[0][db], ks + ub + tr_off[1][db]);
        }
      if (more) load_part(j + 1, 2);
      __builtin_amdgcn_sched_barrier(0);
      // Diagonal or ragged tiles only: masked scores -> -inf, so P = 0 below.
      if (need_mask) {
        keep_branch();
#pragma unroll
        for (int kb = 0; kb < BKV / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (kk >= N || (CAUSAL && kk > qrow)) st[kb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < BKV / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[kb][r], c, -lse2));
          dpt[kb][r] = p * (dpt[kb][r] - dq_d);
        }
      if (more) load_part(j + 1, 3);
      __builtin_amdgcn_sched_barrier(0);
      // dQ^T += K^T dS^T.  All dS fragments are formed first, in registers of
      // their own: rewriting one operand register between MFMAs that read it
      // would make each conversion wait for the previous MFMAs' operand reads.
      frag_t<T> sf[BKV / 16];
#pragma unroll
      for (int u = 0; u < BKV / 16; ++u)
        sf[u] = to_frag<T>((u & 1) ? half8<1>(dpt[u >> 1]) : half8<0>(dpt[u >> 1]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < BKV / 16; ++u)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mma(tk[u][db], sf[u], dq[db]);
    } else if (more) {
#pragma unroll
      for (int c = 1; c < 4; ++c) load_part(j + 1, c);
    }
    if (more) store_tile(buf ^ 1, j + 1);
    __syncthreads();
  }

  if (qrow < N) {
    T* dqrow = a.dQ + hoff + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) store4<T>(dqrow + db * 32 + 8 * rg + 4 * g, dq[db], rg, a.scale);
  }
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
      float* Dv = a.Dvec;
      void* pargs[] = {&O, &dO, &Dv, &rows};
      return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_pre_kernel<T, D>), grid, block,
                             pargs, 0, st);
    }
    case BwdStage::kDkDv: {
      const int nKV = (a.N + kDkvBKV - 1) / kDkvBKV;
      return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<T, D, CAUSAL>),
                             dim3((unsigned)(nKV * a.BH)), block, kargs, 0, st);
    }
    default: {
      const int nQb = (a.N + kDqBQ - 1) / kDqBQ;
      return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<T, D, CAUSAL>),
                             dim3((unsigned)(nQb * a.BH)), block, kargs, 0, st);
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
  for (BwdStage s : {BwdStage::kPreprocess, BwdStage::kDkDv, BwdStage::kDq}) {
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

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
// operand straight from its accumulator registers (see fa_device.h), and every
// operand whose contraction index is a row index in memory (dO and Q for
// dV/dK, K for dQ) gets an extra transposed copy in LDS.
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

// ------------------------------------------------------------------ dK / dV
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs<T> a) {
  constexpr int BKV = kDkvBKV;  // keys per workgroup (4 waves x 32)
  constexpr int BQ = kDkvBQ;    // queries per streamed tile
  constexpr int EPC = kEPC<T>;
  constexpr int RS = D + 8;                // row-major Q / dO stride
  constexpr int TS = BQ + 8;               // transposed Q^T / dO^T stride
  constexpr int NT = 256;
  constexpr int NBLK = (BQ / 4) * (D / EPC);  // 4-row x 16-byte blocks per tile
  constexpr int BPT = (NBLK + NT - 1) / NT;

  __shared__ __attribute__((aligned(32))) T Qs[2][BQ * RS];
  __shared__ __attribute__((aligned(32))) T dOs[2][BQ * RS];
  __shared__ __attribute__((aligned(32))) T Qts[2][D * TS];
  __shared__ __attribute__((aligned(32))) T dOts[2][D * TS];
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];

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
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    kf[t] = key < N ? ld_frag(a.K + hoff + (size_t)key * D + 16 * t + 8 * g) : zero_frag<T>();
    vf[t] = key < N ? ld_frag(a.V + hoff + (size_t)key * D + 16 * t + 8 * g) : zero_frag<T>();
  }

  const int nQb = (N + BQ - 1) / BQ;
  const int i0 = CAUSAL ? k0 / BQ : 0;

  u32x4 qst[BPT][4], dost[BPT][4];
  float lse_st = 0.f, d_st = 0.f;

  auto load_tile = [&](int i) {
    const int qa = i * BQ;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = tid + b * NT;
      if (NBLK % NT == 0 || blk < NBLK) {
        const int rc = blk % (BQ / 4), dc = blk / (BQ / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = qa + 4 * rc + e;
          qst[b][e] = q < N ? ld16(Qh + (size_t)q * D + dc * EPC) : (u32x4)(0u);
          dost[b][e] = q < N ? ld16(dOh + (size_t)q * D + dc * EPC) : (u32x4)(0u);
        }
      }
    }
    if (tid < BQ) {
      const int q = qa + tid;
      lse_st = q < N ? LSEh[q] * kLog2e : INFINITY;  // padding rows get P = 0
    } else if (tid < 2 * BQ) {
      const int q = qa + tid - BQ;
      d_st = q < N ? Dh[q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = tid + b * NT;
      if (NBLK % NT == 0 || blk < NBLK) {
        const int rc = blk % (BQ / 4), dc = blk / (BQ / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<u32x4*>(&Qs[buf][(4 * rc + e) * RS + dc * EPC]) = qst[b][e];
          *reinterpret_cast<u32x4*>(&dOs[buf][(4 * rc + e) * RS + dc * EPC]) = dost[b][e];
        }
        store_transposed_4rows<T>(Qts[buf], TS, dc * EPC, 4 * rc, qst[b]);
        store_transposed_4rows<T>(dOts[buf], TS, dc * EPC, 4 * rc, dost[b]);
      }
    }
    if (tid < BQ) lse2s[buf][tid] = lse_st;
    else if (tid < 2 * BQ) Ds[buf][tid - BQ] = d_st;
  };

  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dv[db] = zero16();
    dk[db] = zero16();
  }
  const float c = a.scale_log2;

  if (i0 < nQb) {
    load_tile(i0);
    store_tile(0);
  }
  __syncthreads();

  for (int i = i0; i < nQb; ++i) {
    const int buf = (i - i0) & 1;
    if (i + 1 < nQb) load_tile(i + 1);
    const int qa = i * BQ;
    const bool active = kw0 < N && (!CAUSAL || kw0 <= qa + BQ - 1);
    if (active) {
      const bool need_mask = CAUSAL && qa < kw0 + 31;
      f32x16 s[BQ / 32], dp[BQ / 32];
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        s[qb] = zero16();
        dp[qb] = zero16();
        const T* qp = &Qs[buf][(qb * 32 + l32) * RS + 8 * g];
        const T* dop = &dOs[buf][(qb * 32 + l32) * RS + 8 * g];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) s[qb] = mma(ld_frag(qp + 16 * t), kf[t], s[qb]);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) dp[qb] = mma(ld_frag(dop + 16 * t), vf[t], dp[qb]);
      }
      // P = exp2(S*c - LSE*log2e), dS = P * (dP - D); rows of the C tiles are queries.
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int ql = qb * 32 + 8 * rg + 4 * g;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[buf][ql]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][ql]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            float p = fast_exp2(__builtin_fmaf(s[qb][r], c, -l4[e]));
            if (need_mask && key > qa + ql + e) p = 0.f;
            s[qb][r] = p;
            dp[qb][r] = p * (dp[qb][r] - d4[e]);
          }
        }
#pragma unroll
      for (int u = 0; u < BQ / 16; ++u) {
        const frag_t<T> pf = to_frag<T>((u & 1) ? half8<1>(s[u >> 1]) : half8<0>(s[u >> 1]));
        const frag_t<T> sf = to_frag<T>((u & 1) ? half8<1>(dp[u >> 1]) : half8<0>(dp[u >> 1]));
        const T* dotp = &dOts[buf][l32 * TS + 16 * u + 8 * g];
        const T* qtp = &Qts[buf][l32 * TS + 16 * u + 8 * g];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = mma(ld_frag(dotp + db * 32 * TS), pf, dv[db]);
          dk[db] = mma(ld_frag(qtp + db * 32 * TS), sf, dk[db]);
        }
      }
    }
    if (i + 1 < nQb) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (key < N) {
    T* dkrow = a.dK + hoff + (size_t)key * D;
    T* dvrow = a.dV + hoff + (size_t)key * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        T k4[4], v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (T)(dk[db][4 * rg + e] * sc);
          v4[e] = (T)(dv[db][4 * rg + e]);
        }
        const int col = db * 32 + 8 * rg + 4 * g;
        *reinterpret_cast<u32x2*>(dkrow + col) = __builtin_bit_cast(u32x2, k4);
        *reinterpret_cast<u32x2*>(dvrow + col) = __builtin_bit_cast(u32x2, v4);
      }
  }
}

// ------------------------------------------------------------------ dQ
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BwdArgs<T> a) {
  constexpr int BQ = kDqBQ;    // queries per workgroup (4 waves x 32)
  constexpr int BKV = kDqBKV;  // keys per streamed tile
  constexpr int EPC = kEPC<T>;
  constexpr int RS = D + 8;
  constexpr int TS = BKV + 8;
  constexpr int NT = 256;
  constexpr int NBLK = (BKV / 4) * (D / EPC);
  constexpr int BPT = (NBLK + NT - 1) / NT;

  __shared__ __attribute__((aligned(32))) T Ks[2][BKV * RS];
  __shared__ __attribute__((aligned(32))) T Vs[2][BKV * RS];
  __shared__ __attribute__((aligned(32))) T Kts[2][D * TS];

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
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    qf[t] = qrow < N ? ld_frag(a.Q + hoff + (size_t)qrow * D + 16 * t + 8 * g) : zero_frag<T>();
    dof[t] = qrow < N ? ld_frag(a.dO + hoff + (size_t)qrow * D + 16 * t + 8 * g) : zero_frag<T>();
  }
  const float lse2 = qrow < N ? a.LSE[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dq_d = qrow < N ? a.Dvec[(size_t)bh * N + qrow] : 0.f;

  const int nKb = (N + BKV - 1) / BKV;
  int jend = nKb;
  if (CAUSAL) jend = min(nKb, (min(q0 + BQ, N) - 1) / BKV + 1);

  u32x4 kst[BPT][4], vst[BPT][4];
  auto load_tile = [&](int j) {
    const int kv0 = j * BKV;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = tid + b * NT;
      if (NBLK % NT == 0 || blk < NBLK) {
        const int rc = blk % (BKV / 4), dc = blk / (BKV / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = kv0 + 4 * rc + e;
          kst[b][e] = kk < N ? ld16(Kh + (size_t)kk * D + dc * EPC) : (u32x4)(0u);
          vst[b][e] = kk < N ? ld16(Vh + (size_t)kk * D + dc * EPC) : (u32x4)(0u);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = tid + b * NT;
      if (NBLK % NT == 0 || blk < NBLK) {
        const int rc = blk % (BKV / 4), dc = blk / (BKV / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *reinterpret_cast<u32x4*>(&Ks[buf][(4 * rc + e) * RS + dc * EPC]) = kst[b][e];
          *reinterpret_cast<u32x4*>(&Vs[buf][(4 * rc + e) * RS + dc * EPC]) = vst[b][e];
        }
        store_transposed_4rows<T>(Kts[buf], TS, dc * EPC, 4 * rc, kst[b]);
      }
    }
  };

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = zero16();
  const float c = a.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < jend; ++j) {
    const int buf = j & 1;
    if (j + 1 < jend) load_tile(j + 1);
    const int kv0 = j * BKV;
    const bool active = wave_rows && (!CAUSAL || kv0 <= qw0 + 31);
    if (active) {
      const bool need_mask = (kv0 + BKV > N) || (CAUSAL && kv0 + BKV - 1 > qw0);
      f32x16 st[BKV / 32], dpt[BKV / 32];
#pragma unroll
      for (int kb = 0; kb < BKV / 32; ++kb) {
        st[kb] = zero16();
        dpt[kb] = zero16();
        const T* kp = &Ks[buf][(kb * 32 + l32) * RS + 8 * g];
        const T* vp = &Vs[buf][(kb * 32 + l32) * RS + 8 * g];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) st[kb] = mma(ld_frag(kp + 16 * t), qf[t], st[kb]);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) dpt[kb] = mma(ld_frag(vp + 16 * t), dof[t], dpt[kb]);
      }
      // Columns of the C tiles are this lane's query; rows are keys.
#pragma unroll
      for (int kb = 0; kb < BKV / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(st[kb][r], c, -lse2));
          if (need_mask) {
            const int kk = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (kk >= N || (CAUSAL && kk > qrow)) p = 0.f;
          }
          dpt[kb][r] = p * (dpt[kb][r] - dq_d);
        }
#pragma unroll
      for (int u = 0; u < BKV / 16; ++u) {
        const frag_t<T> sf = to_frag<T>((u & 1) ? half8<1>(dpt[u >> 1]) : half8<0>(dpt[u >> 1]));
        const T* ktp = &Kts[buf][l32 * TS + 16 * u + 8 * g];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mma(ld_frag(ktp + db * 32 * TS), sf, dq[db]);
      }
    }
    if (j + 1 < jend) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qrow < N) {
    T* dqrow = a.dQ + hoff + (size_t)qrow * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        T q4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q4[e] = (T)(dq[db][4 * rg + e] * sc);
        *reinterpret_cast<u32x2*>(dqrow + db * 32 + 8 * rg + 4 * g) = __builtin_bit_cast(u32x2, q4);
      }
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

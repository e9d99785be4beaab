// Forward kernel: exact attention with online softmax, one workgroup per
// (batch*head, 128-row query tile).
//
// Method: Lecture 9 notes (cs2680.com), section 9.4 — walk the key/value tiles,
// keep per query row a running max m and a running denominator l relative to
// m, rescale the unnormalised output by exp(m_old - m_new) whenever the max
// grows, divide by l once after the last tile; CMU 11-868 FlashAttention notes
// (quidproquo.cc), "Tiling: fix the wrong denominator afterward", slide page
// 12 — the rescaling makes each tile's update exact.  The only statistic saved
// is the row log-sum-exp (slide page 14, Lecture 9 section 9.6).
//
// gfx950 mapping.  4 waves x 32 query rows; K/V tiles of 64 keys double-buffered
// in LDS through registers (the global loads of tile j+1 are in flight while
// tile j is computed).  Per wave and tile:
//   S^T (keys x queries) = K Q^T   — A = K rows from LDS, B = Q^T held in
//                                    registers for the whole kernel;
//   online softmax on S^T: lane l owns query l % 32, so the row statistics live
//   in one lane pair (l, l ^ 32) and need a single cross-half exchange;
//   O^T (d x queries) += V^T P^T   — A = V^T from an LDS copy stored transposed,
//                                    B = P^T straight from the S^T accumulator.
// Scores are scaled by c = scale*log2(e) inside one FMA feeding exp2.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename T, int D, bool CAUSAL, bool MAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdArgs<T> a) {
  constexpr int BR = kFwdBR;
  constexpr int BC = kFwdBC;
  constexpr int EPC = kEPC<T>;
  constexpr int KS = D + 8;   // K row stride in LDS (elements)
  constexpr int VS = BC + 8;  // V^T row stride in LDS (elements)
  constexpr int NT = 256;
  constexpr int KCH = BC * D / EPC / NT;        // K 16-byte chunks per thread
  constexpr int VBLK = (BC / 4) * (D / EPC);    // 4-key x 16-byte blocks of V
  constexpr int VPT = (VBLK + NT - 1) / NT;
  static_assert(KCH * NT * EPC == BC * D, "K tile must split evenly");

  __shared__ __attribute__((aligned(32))) T Ks[2][BC * KS];
  __shared__ __attribute__((aligned(32))) T Vts[2][D * VS];

  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  int bh, qi;
  map_block(blockIdx.x, a.nQ, a.BH, CAUSAL, bh, qi);
  const size_t hoff = (size_t)bh * N * D;
  const T* __restrict__ Qh = a.Q + hoff;
  const T* __restrict__ Kh = a.K + hoff;
  const T* __restrict__ Vh = a.V + hoff;

  const int q0 = qi * BR;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool wave_rows = qw0 < N;

  // Q^T operand: lane holds query qrow, d = 16t + 8g .. +7.
  frag_t<T> qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    qf[t] = qrow < N ? ld_frag(Qh + (size_t)qrow * D + 16 * t + 8 * g) : zero_frag<T>();

  const int nK = a.nK;
  int jend = nK;
  if (CAUSAL) jend = min(nK, (min(q0 + BR, N) - 1) / BC + 1);

  u32x4 kst[KCH];
  u32x4 vst[VPT][4];

  auto load_tile = [&](int j) {
    const int kv0 = j * BC;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / (D / EPC), col = (idx % (D / EPC)) * EPC;
      const int key = kv0 + row;
      kst[c] = key < N ? ld16(Kh + (size_t)key * D + col) : (u32x4)(0u);
    }
#pragma unroll
    for (int b = 0; b < VPT; ++b) {
      const int blk = tid + b * NT;
      if (VBLK % NT == 0 || blk < VBLK) {
        const int kc = blk % (BC / 4), dc = blk / (BC / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kv0 + 4 * kc + e;
          vst[b][e] = key < N ? ld16(Vh + (size_t)key * D + dc * EPC) : (u32x4)(0u);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT;
      const int row = idx / (D / EPC), col = (idx % (D / EPC)) * EPC;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KS + col]) = kst[c];
    }
#pragma unroll
    for (int b = 0; b < VPT; ++b) {
      const int blk = tid + b * NT;
      if (VBLK % NT == 0 || blk < VBLK) {
        const int kc = blk % (BC / 4), dc = blk / (BC / 4);
        store_transposed_4rows<T>(Vts[buf], VS, dc * EPC, 4 * kc, vst[b]);
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = zero16();
  float m = -1e30f;   // running max of the scaled (log2-domain) scores
  float lsum = 0.f;   // this lane's part of the running denominator
  const float c = a.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < jend; ++j) {
    const int buf = j & 1;
    if (j + 1 < jend) load_tile(j + 1);
    const int kv0 = j * BC;
    const int code = tile_code(qi, j, BR, BC, N, CAUSAL);
    if (MAP && tid == 0) a.map[((size_t)bh * a.nQ + qi) * nK + j] = (unsigned char)code;

    const bool active = wave_rows && (!CAUSAL || kv0 <= qw0 + 31);
    if (active) {
      const bool need_mask = code != 1 && ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0));
      f32x16 s[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        s[kb] = zero16();
        const T* kp = &Ks[buf][(kb * 32 + l32) * KS + 8 * g];
#pragma unroll
        for (int t = 0; t < D / 16; ++t) s[kb] = mma(ld_frag(kp + 16 * t), qf[t], s[kb]);
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx * c);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -m));
          s[kb][r] = p;
          rs += p;
        }
      lsum = lsum * alpha + rs;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      }
#pragma unroll
      for (int u = 0; u < BC / 16; ++u) {
        const f32x8 p8 = (u & 1) ? half8<1>(s[u >> 1]) : half8<0>(s[u >> 1]);
        const frag_t<T> pf = to_frag<T>(p8);
        const T* vp = &Vts[buf][l32 * VS + 16 * u + 8 * g];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = mma(ld_frag(vp + db * 32 * VS), pf, o[db]);
      }
    }
    if (j + 1 < jend) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (MAP && tid == 0)
    for (int j = jend; j < nK; ++j) a.map[((size_t)bh * a.nQ + qi) * nK + j] = 0;

  if (wave_rows) {
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (qrow < N) {
      const float inv = 1.0f / ltot;
      T* orow = a.O + hoff + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          T v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (T)(o[db][4 * rg + e] * inv);
          T* dst = orow + db * 32 + 8 * rg + 4 * g;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, v4);
          } else {
            *reinterpret_cast<u32x4*>(dst) = __builtin_bit_cast(u32x4, v4);
          }
        }
      if (g == 0) a.LSE[(size_t)bh * N + qrow] = (m + __builtin_log2f(ltot)) * kLn2;
    }
  }
}

template <typename T, int D, bool CAUSAL, bool MAP>
hipError_t launch_fwd_inst(const FwdArgs<T>& a, hipStream_t st) {
  FwdArgs<T> args = a;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)(a.nQ * a.BH)), block(256);
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

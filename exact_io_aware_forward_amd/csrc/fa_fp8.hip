// FP8 input stage of incoherent processing: every row x of Q or K (d = 64 or
// 128 values) becomes x J, J = diag(s) H / sqrt(d) with H the Sylvester Hadamard
// matrix and s a vector of random signs, then E4M3 codes with one fp32 scale
// per row (the row's largest magnitude maps to 448).
//
// Method: CMU 11-868 FlashAttention notes (quidproquo.cc), "FlashAttention-3:
// asynchrony and FP8 on Hopper", slide page 24 — outliers inflate FP8
// quantisation error; multiplying Q and K by the same random orthogonal
// Hadamard matrix leaves QK^T unchanged and spreads each outlier over all
// coordinates.
//
// gfx950 mapping.  The pass reads each 16-bit row once and writes one byte per
// value: it is bound by HBM bandwidth, so it is written as a coalesced stream,
// not as a matrix product.  A row is held by d/8 consecutive lanes, eight
// values per lane (one 16-byte load); row groups walk the rows with a grid
// stride and load the next row before transforming the current one.  H
// factors over the bits of the coordinate index: for bit b, the pair of
// indices that differ only in b becomes (sum, difference), the lower index
// taking the sum.  The three low
// bits are in-register butterflies; the higher bits pair lanes, exchanged with
// xor shuffles inside the row's lane group.  The row maximum is a shuffle
// reduction over the same group; codes are formed two at a time by the
// hardware's round-to-nearest-even E4M3 conversion and stored as 8 bytes per
// lane.
#include <algorithm>

#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kQuantThreads = 256;
// Resident workgroups of the grid-stride loop: 16 per CU (at most 32 waves of
// 36 registers fit), measured 4-6 % faster than one workgroup per 16 rows.
constexpr long long kQuantMaxWorkgroups = 4096;

// One row held by the L = D/8 lanes of a row group: x J (when rotating), the
// row's scale, and the eight E4M3 codes of this lane packed in two words.
template <typename T, int D>
__device__ __forceinline__ void rotate_quantize_row(uint4 raw, const float* sg, bool rotate,
                                                    float norm, int lane_in_row, float& scale,
                                                    int& w0, int& w1) {
  constexpr int L = D / 8;
  float x[8];
  const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
  if (rotate) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= sg[e];
    // In-register butterflies over index bits 0, 1, 2.
#pragma unroll
    for (int bit = 1; bit < 8; bit <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e & bit) continue;
        const float lo = x[e], hi = x[e | bit];
        x[e] = lo + hi;
        x[e | bit] = lo - hi;
      }
    }
    // Butterflies over the lane bits: the lane whose bit is clear keeps the sum
    // (other + x), the other lane the difference (other - x), one fma each.
#pragma unroll
    for (int m = 1; m < L; m <<= 1) {
      const float sgn = (lane_in_row & m) ? -1.f : 1.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = fmaf(sgn, x[e], __shfl_xor(x[e], m));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= norm;
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int m = 1; m < L; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  scale = amax > 0.f ? amax / 448.f : 1.f;
  // 448 / amax overflows for amax below 448 / FLT_MAX (about 2^-119): a row
  // whose largest magnitude is below 2^-100 is first multiplied by 2^100,
  // which is exact and leaves every ratio y_j / amax, hence every code, as it
  // was.  The scale stays amax / 448 (an fp32 subnormal for such rows).
  float amax_u = amax;
  if (amax > 0.f && amax < 0x1p-100f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= 0x1p100f;
    amax_u = amax * 0x1p100f;
  }
  // Values are brought to code units by one multiplication with 448 / amax
  // (not a division per value); the two differ by at most one rounding.
  const float inv = amax > 0.f ? 448.f / amax_u : 1.f;
  w0 = 0;
  w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * inv, x[5] * inv, w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * inv, x[7] * inv, w1, true);
}

template <typename T, int D>
__global__ __launch_bounds__(kQuantThreads) void fp8_rotate_quantize_kernel(Fp8QuantArgs<T> a) {
  constexpr int L = D / 8;                     // lanes per row
  constexpr int kRowsPerPass = kQuantThreads / L;
  const int lane_in_row = threadIdx.x % L;
  const long long stride = (long long)gridDim.x * kRowsPerPass;
  long long row = (long long)blockIdx.x * kRowsPerPass + threadIdx.x / L;
  float sg[8];
  const bool rotate = a.signs != nullptr;
  if (rotate) {
    const float4 s0 = *reinterpret_cast<const float4*>(a.signs + lane_in_row * 8);
    const float4 s1 = *reinterpret_cast<const float4*>(a.signs + lane_in_row * 8 + 4);
    sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
    sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
  }
  // Grid-stride over rows; the next row's load is issued before the current
  // row is transformed.  All lanes of a row group share the row, so the xor
  // shuffles only ever pair lanes that are active together.
  uint4 cur = row < a.rows ? *reinterpret_cast<const uint4*>(a.X + row * D + lane_in_row * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
  while (row < a.rows) {
    const long long next = row + stride;
    const uint4 nxt = next < a.rows
                          ? *reinterpret_cast<const uint4*>(a.X + next * D + lane_in_row * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
    float scale;
    int w0, w1;
    rotate_quantize_row<T, D>(cur, sg, rotate, a.inv_sqrt_d, lane_in_row, scale, w0, w1);
    *reinterpret_cast<uint2*>(a.codes + row * D + lane_in_row * 8) =
        make_uint2((unsigned)w0, (unsigned)w1);
    if (lane_in_row == 0) a.scales[row] = scale;
    row = next;
    cur = nxt;
  }
}

}  // namespace

template <typename T>
hipError_t launch_fp8_quantize(const Fp8QuantArgs<T>& a, int d, hipStream_t st) {
  const int rows_per_block = kQuantThreads / (d / 8);
  const long long blocks =
      std::min((a.rows + rows_per_block - 1) / rows_per_block, kQuantMaxWorkgroups);
  const dim3 grid((unsigned)blocks), block(kQuantThreads);
  if (d == 128)
    hipLaunchKernelGGL((fp8_rotate_quantize_kernel<T, 128>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((fp8_rotate_quantize_kernel<T, 64>), grid, block, 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_fp8_quantize<bf16_t>(const Fp8QuantArgs<bf16_t>&, int, hipStream_t);
template hipError_t launch_fp8_quantize<f16_t>(const Fp8QuantArgs<f16_t>&, int, hipStream_t);

}  // namespace fa

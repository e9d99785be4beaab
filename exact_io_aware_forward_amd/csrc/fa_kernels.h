// Internal interface between the C ABI (fa_api.cpp) and the kernel files:
// argument blocks, tile shapes and launchers.  Not installed; the public
// interface is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

// Tile shapes (compile-time; where one depends on the head dimension, the dtype
// or the causal mask, the function that gives it says how).
// Forward: 8 waves x 32 query rows per workgroup (kFwdRows below for the 512-row
// case), 64-key tiles streamed.
constexpr int kFwdWaves = 8;
constexpr int kFwdBR = 32 * kFwdWaves, kFwdBC = 64;
// Query rows per forward workgroup: kFwdBR, except with 16-bit inputs, d = 64
// and no causal mask, where each wave holds two 32-row blocks (512 rows) so
// that every K and V fragment it reads from LDS feeds two products.
constexpr int kFwdRows(int d, bool causal, bool sixteen_bit) {
  return sixteen_bit && d == 64 && !causal ? 2 * kFwdBR : kFwdBR;
}
// dK/dV: 4 waves x 32 keys per workgroup; query tiles of kDkvBQ(d) rows
// streamed.  At d = 64 the smaller tile lets two workgroups share a compute
// unit (two waves per SIMD, each hiding the other's LDS and matrix latency).
constexpr int kDkvBKV = 128;
constexpr int kDkvBQ(int d) { return d == 64 ? 32 : 64; }
// dQ: 8 waves x 32 query rows per workgroup (two groups in ping-pong); key
// tiles of kDqBKV(d) rows streamed, sized so that a wave stays within 256
// registers (two waves per SIMD) at both head dimensions.
constexpr int kDqBQ = 256;
constexpr int kDqBKV(int d) { return d == 128 ? 32 : 64; }
// dK/dV workgroups the group split aims for (grouped key/value heads): two per
// CU of an MI355X, enough for the causal tiles' unequal work to balance
// (measured: grouped backward then within 1 % of multi-head).
constexpr int kDkvTargetWorkgroups = 512;

template <typename T> struct FwdArgs {
  const T* Q;
  const T* K;
  const T* V;
  T* O;
  float* LSE;
  unsigned char* map;  // tile codes, only written by the instrumented instance
  int N, BH, nQ, nK;   // BH = B * H query heads
  int group;           // query heads per key/value head (1: multi-head attention)
  float scale_log2;    // scale * log2(e)
};

template <typename T> struct BwdArgs {
  const T* Q;
  const T* K;
  const T* V;
  const T* O;
  const T* dO;
  const float* LSE;
  float* Dvec;         // workspace: rowsum(dO * O), float32 [B*H*N]
  float* L2;           // workspace: LSE * log2(e), float32 [B*H*N]
  unsigned char* map_dkdv;  // tile codes of the dK/dV kernel [BH][key tiles][query tiles], or null
  unsigned char* map_dq;    // tile codes of the dQ kernel [BH][query tiles][key tiles], or null
  T* dQ;
  T* dK;
  T* dV;
  int N, BH;           // BH = B * H query heads; K, V, dK, dV have BH / group heads
  int group;           // query heads per key/value head (1: multi-head attention)
  int gsplit;          // dK/dV workgroups per (key/value head, key tile), dividing group
  float* dkv_part;     // workspace (gsplit > 1): fp32 partial dK then dV, [gsplit][BH/group][N][d]
  float scale;
  float scale_log2;
};

// Split-K decode: 4 waves per workgroup, 32-key tiles, at most 32 query rows
// per key/value head.
constexpr int kDecWaves = 4, kDecBC = 32, kDecMaxQ = 32;
// Workgroups the default split count aims for: one per compute unit of an
// MI355X (each split workgroup holds 128 KB of LDS, so one runs per CU).
constexpr int kDecTargetWorkgroups = 256;
// Fewest 32-key tiles per slice the default split count allows (four per wave).
constexpr int kDecMinTilesPerSplit = 4 * kDecWaves;
// Most partials (slices) per head the combine kernel merges; the slice count is
// clamped to kDecMaxPartials / kDecWaves = 512, well inside it.
constexpr int kDecMaxPartials = 2048;
// Thread groups per combine workgroup (each walks every kDecCombineGroups-th partial).
constexpr int kDecCombineGroups = 4;

// Rows: the g = H / Hkv query heads sharing a key/value head are adjacent, so
// their g * qlen query rows are one contiguous block of Q and O per key/value
// head; they are processed together against that head's cache.
template <typename T> struct DecArgs {
  const T* Q;          // [BH, Nq, d] (= [B, H, qlen, d])
  const T* K;          // [BH, Nk, d]
  const T* V;
  T* O;                // [BH, Nq, d]
  float* LSE;          // [BH, Nq]
  float* part_o;       // workspace: unnormalised partial outputs, float32 [BH][splits][Nq][d]
  float* part_s;       // workspace: (m, l, lq, 0) per partial row, float32 [BH][splits][Nq][4]
  int Nq;              // query rows per key/value head: g * qlen
  int qlen;            // queries per query head (row r is query r % qlen of its head)
  int Nk;
  int BH;              // B * Hkv
  int splits;          // slices of the cache per head, one partial each
  int tiles_per_split; // 32-key tiles per slice (the last slice may hold fewer)
  int direct;          // one slice, whole call: the split kernel writes O and LSE itself
  float scale_log2;    // scale * log2(e)
};

template <typename T>
hipError_t launch_fwd(const FwdArgs<T>& a, int d, bool causal, bool map, hipStream_t st);

// The backward stages.  The preprocess forms D = rowsum(dO * O) and
// LSE * log2(e) per query row; the dQ kernel forms the same two for its own
// rows and stores them too, so launch_bwd runs dQ and then dK/dV on one stream
// (the separate preprocess serves callers that run dK/dV first).
enum class BwdStage { kPreprocess, kDkDv, kDq };

template <typename T>
hipError_t launch_bwd_stage(const BwdArgs<T>& a, int d, bool causal, BwdStage stage,
                            hipStream_t st);

template <typename T>
hipError_t launch_bwd(const BwdArgs<T>& a, int d, bool causal, hipStream_t st);

// stage -1: split kernel then combine kernel; 0: split kernel only; 1: combine only.
template <typename T>
hipError_t launch_decode(const DecArgs<T>& a, int d, bool causal, int stage, hipStream_t st);

// FP8 input stage: rows of X rotated by diag(signs) H / sqrt(d) (no rotation when
// signs is null), then E4M3 codes with one fp32 scale per row.
template <typename T> struct Fp8QuantArgs {
  const T* X;              // [rows][d]
  const float* signs;      // [d], +-1, or null
  unsigned char* codes;    // [rows][d] E4M3 bytes
  float* scales;           // [rows]
  long long rows;
  float inv_sqrt_d;
};

template <typename T>
hipError_t launch_fp8_quantize(const Fp8QuantArgs<T>& a, int d, hipStream_t st);

// FP8 forward: scores from E4M3 codes of Q J and K J with one fp32 scale per
// row; V, O in T.  All [B*H][N][d] (codes bytes), scales and LSE [B*H][N].
template <typename T> struct Fp8FwdArgs {
  const unsigned char* Qc;
  const float* Qs;
  const unsigned char* Kc;
  const float* Ks;
  const T* V;
  T* O;
  float* LSE;
  int N, BH, nQ, nK;
  float scale_log2;    // scale * log2(e)
};

template <typename T>
hipError_t launch_fwd_fp8(const Fp8FwdArgs<T>& a, int d, bool causal, hipStream_t st);

// Static scratch of the allocation-free backward (fa_scratch.hip): 8 MiB, the
// preprocess's two float32 per query row for up to 2^20 rows (B * H * N).
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;
// Device address of the scratch array on the device `stream` belongs to (the
// current device for the null stream), looked up once per device.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

}  // namespace fa

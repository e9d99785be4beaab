// C ABI of libfa.so (declared in include/fa.h): argument validation, kernel
// instance selection and launch on the caller's stream.  Validation runs before
// anything is launched; nothing here allocates, frees or synchronises.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_kernels.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* msg, const char* detail = nullptr) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s%s%s", msg, detail ? ": " : "",
                detail ? detail : "");
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// LSE is read and written one float per lane: 4-byte alignment is enough.
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape and scalar checks shared by every entry point.
int check_common(int B, int H, int N, int d, float scale, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0) return fail(FA_ERR_INVALID_ARG, "B, H and N must be positive");
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_INVALID_ARG, "unknown dtype");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  if (!(scale > 0.f)) return fail(FA_ERR_UNSUPPORTED, "scale must be > 0");
  // Element count of one tensor and workgroup counts must stay in range.
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  const unsigned long long elems = bh * (unsigned long long)N * (unsigned long long)d;
  if (bh >= (1ull << 31) || elems > (1ull << 56))
    return fail(FA_ERR_INVALID_ARG, "tensor too large");
  // The kernels address one head's rows through buffer descriptors with 32-bit
  // byte ranges: a head must stay below 2 GB in 16-bit elements.
  if ((unsigned long long)N * (unsigned long long)d >= (1ull << 30))
    return fail(FA_ERR_UNSUPPORTED, "N * d must be below 2^30 (one head below 2 GB)");
  const unsigned long long tiles = bh * (((unsigned long long)N + 31) / 32);
  if (tiles >= (1ull << 31)) return fail(FA_ERR_INVALID_ARG, "too many tiles for one launch");
  return FA_OK;
}

template <typename T>
int run_forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                int Hkv, int N, int d, int causal, float scale, unsigned char* map,
                hipStream_t st) {
  fa::FwdArgs<T> a;
  a.Q = static_cast<const T*>(Q);
  a.K = static_cast<const T*>(K);
  a.V = static_cast<const T*>(V);
  a.O = static_cast<T*>(O);
  a.LSE = LSE;
  a.map = map;
  a.N = N;
  a.BH = B * H;
  const int rows = fa::kFwdRows(d, causal != 0, sizeof(T) == 2);   // query rows per workgroup
  a.nQ = (N + rows - 1) / rows;
  a.nK = (N + fa::kFwdBC - 1) / fa::kFwdBC;
  a.group = H / Hkv;
  a.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e = fa::launch_fwd<T>(a, d, causal != 0, map != nullptr, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed", hipGetErrorString(e));
  return FA_OK;
}

int forward_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                 int Hkv, int N, int d, int causal, float scale, int dtype, unsigned char* map,
                 void* stream) {
  g_last_error[0] = '\0';
  if (!Q || !K || !V || !O || !LSE) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
  const int s = check_common(B, H, N, d, scale, dtype);
  if (s != FA_OK) return s;
  if (Hkv <= 0 || H % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hkv must be positive and divide H");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
    return fail(FA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!aligned4(LSE)) return fail(FA_ERR_INVALID_ARG, "LSE must be 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case FA_BF16:
      return run_forward<fa::bf16_t>(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, scale, map, st);
    case FA_F16:
      return run_forward<fa::f16_t>(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, scale, map, st);
    default:
      return run_forward<float>(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, scale, map, st);
  }
}

// dK/dV workgroups per (key/value head, key tile) for grouped heads: the
// smallest divisor of the group size G that gives the target workgroup count
// (else G itself); 1 for multi-head attention.
int dkdv_gsplit(int B, int Hkv, int G, int N) {
  const long long base = (long long)B * Hkv * ((N + fa::kDkvBKV - 1) / fa::kDkvBKV);
  int best = 1;
  for (int s = 1; s <= G; ++s) {
    if (G % s) continue;
    best = s;
    if (base * s >= fa::kDkvTargetWorkgroups) break;
  }
  return best;
}

// Floats of the backward workspace: D and LSE*log2(e) per query row, then, when
// the group is split, fp32 partial dK and dV from a 16-byte aligned offset.
size_t bwd_part_offset(int B, int H, int N) {
  return ((size_t)2 * B * H * N + 3) & ~(size_t)3;
}
size_t bwd_ws_floats(int B, int H, int Hkv, int N, int d) {
  const size_t rows = (size_t)B * H * N;
  const int gs = dkdv_gsplit(B, Hkv, H / Hkv, N);
  if (gs == 1) return 2 * rows;
  return bwd_part_offset(B, H, N) + 2 * (size_t)gs * B * Hkv * N * d;
}

template <typename T>
int run_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                 int causal, int d, float scale, float* Dvec, float* L2, int stage,
                 unsigned char* map_dkdv, unsigned char* map_dq, hipStream_t st) {
  fa::BwdArgs<T> a;
  a.Q = static_cast<const T*>(Q);
  a.K = static_cast<const T*>(K);
  a.V = static_cast<const T*>(V);
  a.O = static_cast<const T*>(O);
  a.dO = static_cast<const T*>(dO);
  a.LSE = LSE;
  a.Dvec = Dvec;
  a.L2 = L2;
  a.map_dkdv = map_dkdv;
  a.map_dq = map_dq;
  a.dQ = static_cast<T*>(dQ);
  a.dK = static_cast<T*>(dK);
  a.dV = static_cast<T*>(dV);
  a.N = N;
  a.BH = B * H;
  a.group = H / Hkv;
  a.gsplit = dkdv_gsplit(B, Hkv, H / Hkv, N);
  a.dkv_part = Dvec + bwd_part_offset(B, H, N);
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e;
  if (stage < 0) {
    e = fa::launch_bwd<T>(a, d, causal != 0, st);
  } else {
    const fa::BwdStage s = stage == 0 ? fa::BwdStage::kPreprocess
                           : stage == 1 ? fa::BwdStage::kDkDv : fa::BwdStage::kDq;
    e = fa::launch_bwd_stage<T>(a, d, causal != 0, s, st);
  }
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed", hipGetErrorString(e));
  return FA_OK;
}

// stage -1 = the whole backward (dQ, which also forms D and LSE*log2(e), then
// dK/dV); 0 = preprocess; 1 = dK/dV; 2 = dQ.  Each stage needs only the
// pointers it touches.
// With use_scratch, workspace and workspace_bytes are ignored and the library's
// static scratch array serves as the workspace (fa_backward_noalloc).
int backward_impl(int stage, const void* Q, const void* K, const void* V, const void* O,
                  const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B, int H,
                  int Hkv, int N, int d, int causal, float scale, int dtype, void* workspace,
                  size_t workspace_bytes, unsigned char* map_dkdv, unsigned char* map_dq,
                  void* hip_stream, bool use_scratch = false) {
  g_last_error[0] = '\0';
  if (stage < -1 || stage > 2) return fail(FA_ERR_INVALID_ARG, "unknown backward stage");
  const bool all = stage < 0, pre = all || stage == 0, dkdv = all || stage == 1,
             dq = all || stage == 2;
  const bool uses_qkv = dkdv || dq;
  const struct { const void* p; bool used; bool lse; } ptrs[] = {
      {O, pre || dq, false}, {dO, true, false}, {Q, uses_qkv, false}, {K, uses_qkv, false},
      {V, uses_qkv, false}, {LSE, true, true}, {dK, dkdv, false}, {dV, dkdv, false},
      {dQ, dq, false}};
  for (const auto& t : ptrs) {
    if (!t.used) continue;
    if (!t.p) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
    if (t.lse ? !aligned4(t.p) : !aligned16(t.p))
      return fail(FA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned, LSE 4-byte");
  }
  const int s = check_common(B, H, N, d, scale, dtype);
  if (s != FA_OK) return s;
  if (Hkv <= 0 || H % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hkv must be positive and divide H");
  if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "the backward pass supports fp16 and bf16");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (use_scratch) {
    const size_t need = bwd_ws_floats(B, H, Hkv, N, d) * sizeof(float);
    if (need > fa::kNoallocScratchBytes) {
      char msg[160];
      std::snprintf(msg, sizeof(msg), "%zu bytes of scratch needed, the static array holds %zu "
                    "(B * H * N at most %zu)", need, fa::kNoallocScratchBytes,
                    fa::kNoallocScratchBytes / (2 * sizeof(float)));
      return fail(FA_ERR_WORKSPACE, "input too large for the allocation-free backward", msg);
    }
    const hipError_t e = fa::noalloc_scratch(st, &workspace);
    if (e != hipSuccess)
      return fail(FA_ERR_HIP, "scratch address lookup failed", hipGetErrorString(e));
    workspace_bytes = fa::kNoallocScratchBytes;
  }
  if (!workspace || workspace_bytes < bwd_ws_floats(B, H, Hkv, N, d) * sizeof(float) ||
      !aligned16(workspace))
    return fail(FA_ERR_WORKSPACE, "workspace missing, misaligned or too small");
  float* Dvec = static_cast<float*>(workspace);
  float* L2 = Dvec + (size_t)B * H * N;
  if (dtype == FA_BF16)
    return run_backward<fa::bf16_t>(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Hkv, N, causal, d,
                                    scale, Dvec, L2, stage, map_dkdv, map_dq, st);
  return run_backward<fa::f16_t>(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Hkv, N, causal, d, scale,
                                 Dvec, L2, stage, map_dkdv, map_dq, st);
}

// Slice count and tiles per slice of a decode call; num_splits 0 = the default
// (enough workgroups for every compute unit, at least four tiles per wave).
// Never more slices than tiles or than the combine kernel merges (512).
// Returns the effective slice count (no empty slice).
int decode_splits(int B, int H, int Nk, int num_splits, int* tiles_per_split) {
  const long long nT = ((long long)Nk + fa::kDecBC - 1) / fa::kDecBC;
  const long long bh = (long long)B * H;
  long long s = num_splits;
  if (s <= 0) {
    s = (fa::kDecTargetWorkgroups + bh - 1) / bh;
    s = std::min(s, nT / fa::kDecMinTilesPerSplit);
    s = std::max(s, 1ll);
  }
  s = std::min(s, nT);
  s = std::min(s, (long long)(fa::kDecMaxPartials / fa::kDecWaves));
  const long long tps = (nT + s - 1) / s;
  *tiles_per_split = (int)tps;
  return (int)((nT + tps - 1) / tps);
}

// Shape checks of the decode entry points (before any pointer is looked at).
int check_decode_shape(int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int dtype,
                       int num_splits) {
  const int s = check_common(B, H, Nk, d, scale, dtype);
  if (s != FA_OK) return s;
  if (Hkv <= 0 || H % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hkv must be positive and divide H");
  if (Nq <= 0) return fail(FA_ERR_INVALID_ARG, "Nq must be positive");
  if (Nq > Nk) return fail(FA_ERR_INVALID_ARG, "decode needs Nq <= Nk");
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0");
  if ((long long)(H / Hkv) * Nq > fa::kDecMaxQ)
    return fail(FA_ERR_UNSUPPORTED, "decode supports at most 32 query rows per key/value head");
  if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "decode supports fp16 and bf16");
  int tps = 0;
  const int splits = decode_splits(B, Hkv, Nk, num_splits, &tps);
  if ((long long)B * Hkv * splits >= (1ll << 31) || (long long)B * H * Nq >= (1ll << 31))
    return fail(FA_ERR_INVALID_ARG, "too many workgroups for one launch");
  return FA_OK;
}

size_t decode_ws_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int num_splits) {
  int tps = 0;
  const int splits = decode_splits(B, Hkv, Nk, num_splits, &tps);
  const size_t rows = (size_t)B * H * splits * Nq;   // = B*Hkv heads x g*Nq rows per slice
  return rows * ((size_t)d + 4) * sizeof(float);
}

template <typename T>
int run_decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
               int Hkv, int Nq, int Nk, int d, int causal, float scale, int num_splits,
               void* workspace, int stage, hipStream_t st) {
  fa::DecArgs<T> a;
  a.Q = static_cast<const T*>(Q);
  a.K = static_cast<const T*>(K);
  a.V = static_cast<const T*>(V);
  a.O = static_cast<T*>(O);
  a.LSE = LSE;
  a.Nq = (H / Hkv) * Nq;
  a.qlen = Nq;
  a.Nk = Nk;
  a.BH = B * Hkv;
  a.splits = decode_splits(B, Hkv, Nk, num_splits, &a.tiles_per_split);
  a.direct = (a.splits == 1 && stage < 0) ? 1 : 0;
  a.part_o = static_cast<float*>(workspace);
  a.part_s = a.part_o + (size_t)a.BH * a.splits * a.Nq * d;
  a.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e = fa::launch_decode<T>(a, d, causal != 0, stage, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed", hipGetErrorString(e));
  return FA_OK;
}

// stage -1 = split kernel and combine; 0 = split kernel; 1 = combine.
int decode_impl(int stage, const void* Q, const void* K, const void* V, void* O, float* LSE,
                int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale, int dtype,
                int num_splits, void* workspace, size_t workspace_bytes, void* hip_stream) {
  g_last_error[0] = '\0';
  if (stage < -1 || stage > 1) return fail(FA_ERR_INVALID_ARG, "unknown decode stage");
  const bool split = stage != 1, combine = stage != 0;
  const struct { const void* p; bool used; bool lse; } ptrs[] = {
      {Q, split, false}, {K, split, false}, {V, split, false}, {O, combine, false},
      {LSE, combine, true}};
  for (const auto& t : ptrs) {
    if (!t.used) continue;
    if (!t.p) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
    if (t.lse ? !aligned4(t.p) : !aligned16(t.p))
      return fail(FA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned, LSE 4-byte");
  }
  const int s = check_decode_shape(B, H, Hkv, Nq, Nk, d, scale, dtype, num_splits);
  if (s != FA_OK) return s;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < decode_ws_bytes(B, H, Hkv, Nq, Nk, d, num_splits))
    return fail(FA_ERR_WORKSPACE, "workspace missing, misaligned or too small");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (dtype == FA_BF16)
    return run_decode<fa::bf16_t>(Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, causal, scale,
                                  num_splits, workspace, stage, st);
  return run_decode<fa::f16_t>(Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, causal, scale, num_splits,
                               workspace, stage, st);
}

}  // namespace

extern "C" {

int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
               int N, int d, int causal, float scale, int dtype, void* hip_stream) {
  return forward_impl(Q, K, V, O, LSE, B, H, H, N, d, causal, scale, dtype, nullptr, hip_stream);
}

int fa_forward_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                   int H, int Hkv, int N, int d, int causal, float scale, int dtype,
                   void* hip_stream) {
  return forward_impl(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, scale, dtype, nullptr,
                      hip_stream);
}

int fa_forward_blockmap(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                        int H, int N, int d, int causal, float scale, int dtype,
                        unsigned char* tile_codes, void* hip_stream) {
  if (!tile_codes) return fail(FA_ERR_INVALID_ARG, "null tile_codes pointer");
  return forward_impl(Q, K, V, O, LSE, B, H, H, N, d, causal, scale, dtype, tile_codes,
                      hip_stream);
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

size_t fa_backward_gqa_workspace_size(int B, int H, int Hkv, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || Hkv <= 0 || H % Hkv != 0) return 0;
  if (d != 64 && d != 128) return 0;
  return bwd_ws_floats(B, H, Hkv, N, d) * sizeof(float);
}

int fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N, int d,
                int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                void* hip_stream) {
  return backward_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, causal, scale, dtype,
                       workspace, workspace_bytes, nullptr, nullptr, hip_stream);
}

int fa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                        int H, int N, int d, int causal, float scale, int dtype,
                        void* hip_stream) {
  return backward_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, causal, scale, dtype,
                       nullptr, 0, nullptr, nullptr, hip_stream, true);
}

int fa_backward_gqa(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                    int d, int causal, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* hip_stream) {
  return backward_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Hkv, N, d, causal, scale,
                       dtype, workspace, workspace_bytes, nullptr, nullptr, hip_stream);
}

int fa_backward_blockmap(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                         int H, int N, int d, int causal, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, unsigned char* dkdv_codes,
                         unsigned char* dq_codes, void* hip_stream) {
  if (!dkdv_codes || !dq_codes) {
    g_last_error[0] = '\0';
    return fail(FA_ERR_INVALID_ARG, "null tile code pointer");
  }
  return backward_impl(-1, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, causal, scale, dtype,
                       workspace, workspace_bytes, dkdv_codes, dq_codes, hip_stream);
}

int fa_backward_stage(int stage, const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                      int H, int N, int d, int causal, float scale, int dtype, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  if (stage < 0 || stage > 2) {
    g_last_error[0] = '\0';
    return fail(FA_ERR_INVALID_ARG, "unknown backward stage");
  }
  return backward_impl(stage, Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, H, N, d, causal, scale,
                       dtype, workspace, workspace_bytes, nullptr, nullptr, hip_stream);
}

int fa_decode_num_splits(int B, int H, int Hkv, int Nq, int Nk, int d) {
  g_last_error[0] = '\0';
  const int s = check_decode_shape(B, H, Hkv, Nq, Nk, d, 1.0f, FA_BF16, 0);
  if (s != FA_OK) return s;
  int tps = 0;
  return decode_splits(B, Hkv, Nk, 0, &tps);
}

size_t fa_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, int num_splits) {
  if (check_decode_shape(B, H, Hkv, Nq, Nk, d, 1.0f, FA_BF16, num_splits) != FA_OK) return 0;
  return decode_ws_bytes(B, H, Hkv, Nq, Nk, d, num_splits);
}

int fa_decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
              int Hkv, int Nq, int Nk, int d, int causal, float scale, int dtype, int num_splits,
              void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_impl(-1, Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits,
                     workspace, workspace_bytes, hip_stream);
}

int fa_decode_stage(int stage, const void* Q, const void* K, const void* V, void* O, float* LSE,
                    int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                    void* hip_stream) {
  if (stage < 0 || stage > 1) {
    g_last_error[0] = '\0';
    return fail(FA_ERR_INVALID_ARG, "unknown decode stage");
  }
  return decode_impl(stage, Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, causal, scale, dtype,
                     num_splits, workspace, workspace_bytes, hip_stream);
}

int fa_tile_config(int kernel_id, int d, int dtype, int* Br, int* Bc) {
  if (!Br || !Bc) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  switch (kernel_id) {
    case 0: *Br = fa::kFwdRows(d, true, dtype != FA_F32); *Bc = fa::kFwdBC; return FA_OK;
    case 3: *Br = fa::kFwdRows(d, false, dtype != FA_F32); *Bc = fa::kFwdBC; return FA_OK;
    case 1:
      if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
      *Br = fa::kDkvBQ(d); *Bc = fa::kDkvBKV; return FA_OK;
    case 2:
      if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
      *Br = fa::kDqBQ; *Bc = fa::kDqBKV(d); return FA_OK;
    default: return FA_ERR_INVALID_ARG;
  }
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_last_error; }

int fa_fp8_quantize_rows(const void* X, long long rows, int d, int dtype, const float* signs,
                         unsigned char* codes, float* scales, void* hip_stream) {
  g_last_error[0] = '\0';
  if (rows < 0) return fail(FA_ERR_INVALID_ARG, "rows must not be negative");
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_INVALID_ARG, "unknown dtype");
  if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "FP8 quantisation takes fp16 or bf16 rows");
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "row length must be 64 or 128");
  if (rows == 0) return FA_OK;  // nothing to read or write; pointers may be null
  if (!X || !codes || !scales) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
  if (rows >= (1ll << 31)) return fail(FA_ERR_INVALID_ARG, "too many rows for one launch");
  if (!aligned16(X) || (signs && !aligned16(signs)) ||
      (reinterpret_cast<uintptr_t>(codes) & 7u) || (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(FA_ERR_INVALID_ARG,
                "X and signs must be 16-byte, codes 8-byte and scales 4-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (dtype == FA_BF16) {
    fa::Fp8QuantArgs<fa::bf16_t> a{static_cast<const fa::bf16_t*>(X), signs, codes, scales, rows,
                                   1.0f / std::sqrt((float)d)};
    e = fa::launch_fp8_quantize(a, d, st);
  } else {
    fa::Fp8QuantArgs<fa::f16_t> a{static_cast<const fa::f16_t*>(X), signs, codes, scales, rows,
                                  1.0f / std::sqrt((float)d)};
    e = fa::launch_fp8_quantize(a, d, st);
  }
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed", hipGetErrorString(e));
  return FA_OK;
}

int fa_forward_fp8(const void* Qc, const float* Qs, const void* Kc, const float* Ks,
                   const void* V, void* O, float* LSE, int B, int H, int N, int d, int causal,
                   float scale, int dtype, void* hip_stream) {
  g_last_error[0] = '\0';
  if (!Qc || !Qs || !Kc || !Ks || !V || !O || !LSE)
    return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
  const int s = check_common(B, H, N, d, scale, dtype);
  if (s != FA_OK) return s;
  if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "the FP8 forward takes fp16 or bf16 V");
  if (!aligned16(Qc) || !aligned16(Kc) || !aligned16(V) || !aligned16(O) ||
      !aligned4(Qs) || !aligned4(Ks) || !aligned4(LSE))
    return fail(FA_ERR_INVALID_ARG, "codes, V and O must be 16-byte, scales and LSE 4-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  auto fill = [&](auto& a) {
    a.Qc = static_cast<const unsigned char*>(Qc);
    a.Qs = Qs;
    a.Kc = static_cast<const unsigned char*>(Kc);
    a.Ks = Ks;
    a.LSE = LSE;
    a.N = N;
    a.BH = B * H;
    a.nQ = (N + fa::kFwdBR - 1) / fa::kFwdBR;
    a.nK = (N + fa::kFwdBC - 1) / fa::kFwdBC;
    a.scale_log2 = scale * 1.4426950408889634f;
  };
  if (dtype == FA_BF16) {
    fa::Fp8FwdArgs<fa::bf16_t> a;
    fill(a);
    a.V = static_cast<const fa::bf16_t*>(V);
    a.O = static_cast<fa::bf16_t*>(O);
    e = fa::launch_fwd_fp8(a, d, causal != 0, st);
  } else {
    fa::Fp8FwdArgs<fa::f16_t> a;
    fill(a);
    a.V = static_cast<const fa::f16_t*>(V);
    a.O = static_cast<fa::f16_t*>(O);
    e = fa::launch_fwd_fp8(a, d, causal != 0, st);
  }
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed", hipGetErrorString(e));
  return FA_OK;
}

}  // extern "C"

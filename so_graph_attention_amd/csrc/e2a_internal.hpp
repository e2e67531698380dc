// Internal helpers shared by the libe2a translation units: status handling,
// the per-thread error message, HIP error checks and bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/e2a.h"

namespace e2a {

// Records a formatted message for e2a_last_error_message() and returns s.
e2a_status fail(e2a_status s, const char* fmt, ...);
void clear_error();

#define E2A_HIP_CHECK(expr)                                                               \
  do {                                                                                    \
    hipError_t e2a_err_ = (expr);                                                         \
    if (e2a_err_ != hipSuccess)                                                           \
      return ::e2a::fail(E2A_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e2a_err_)); \
  } while (0)

#define E2A_LAUNCH_CHECK()                                                                 \
  do {                                                                                     \
    hipError_t e2a_err_ = hipGetLastError();                                               \
    if (e2a_err_ != hipSuccess)                                                            \
      return ::e2a::fail(E2A_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e2a_err_)); \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bf16 <-> fp32 (storage conversion only).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, size_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// Neighbour build (neighbors.hip).
e2a_status build_neighbors_impl(const float* pos, int64_t n, const int32_t* batch, const float* box,
                                float cutoff, int64_t* row_ptr, int32_t* col, int64_t cap,
                                int64_t* n_edges, void* ws, size_t ws_bytes, hipStream_t stream);
size_t neighbors_workspace_bytes(int64_t n);
// Exclusive scan of n int32 values into out[0..n] (total at out[n]); bsum needs
// scan_bsum_count(n) int64 entries of scratch.
e2a_status exclusive_scan_i32(const int32_t* in, int64_t n, int32_t* out, int64_t* bsum, hipStream_t s);
int64_t scan_bsum_count(int64_t n);
// Bounding box of n positions into out[0..6] (min xyz, max xyz, 1 if any
// coordinate is not finite); partial needs kBboxPartialFloats floats.
constexpr int kBboxPartialFloats = 8 * 256;
e2a_status launch_bbox(const float* pos, int64_t n, float* partial, float* out, hipStream_t s);
// The first stage alone (partial boxes of up to 256 blocks, 8 floats each:
// min, max, non-finite flag); returns the number of partials.
int launch_bbox_partial(const float* pos, int64_t n, float* partial, hipStream_t s);

// Attention (attention_*.hip).
struct AttnPlan {
  const e2a_attn_args* a;
  float* q;           // workspace f32 [N, C]
  float* k;           // workspace f32 [N, C]
  uint16_t* wqk_t;    // workspace bf16 [2][C][C]: W_q^T, W_k^T for the matrix-core q/k (bf16 storage)
  void* mfma_ws;      // workspace of the MFMA path (packed weights, atom order)
  float box[3];
  int periodic;
  bool conv;          // sum of the messages (no attention weights, no log-normaliser)
};
e2a_status launch_qk(const AttnPlan& p, hipStream_t s);
e2a_status launch_attention_reference(const AttnPlan& p, hipStream_t s);
bool mfma_supported(int L, int C, int H, int dtype);
size_t mfma_workspace_bytes(int64_t n, int L, int C, bool backward);
e2a_status launch_attention_mfma(const AttnPlan& p, hipStream_t s);
// The MFMA build's packed SO(2) image (bytes, and the packing), and the
// spatial destination order it uses unless the caller gives one.
size_t mfma_packed_bytes(int L);
e2a_status pack_so2_mfma(const void* w_so2, void* out, int L, hipStream_t s);
size_t order_workspace_bytes(int64_t n);
// The bf16 copy of the cotangent the matrix-core feature gradient leaves in
// its workspace (mfma_ws of a BwdPlan).
const uint16_t* mfma_grad_bf16(const void* mfma_ws, int64_t n, int L);
// ... and where it keeps delta = sum G o per atom and head [N, H].
const float* mfma_delta(const void* mfma_ws, int64_t n, int L);
e2a_status destination_order(const float* pos, int64_t n, int32_t* order, void* ws, hipStream_t s);
// Feature gradient (attention_backward.hip).
struct BwdPlan {
  const e2a_attn_args* a;
  const float* grad_out;   // dL/do [N, K, C]
  float* grad_feat;        // dL/dh [N, K, C]
  float* q;                // workspace f32 [N, C]
  float* k;                // workspace f32 [N, C]
  float* dq;               // workspace f32 [N, C]
  float* dk;               // workspace f32 [N, C] (matrix-core path: dk when wdk is not set)
  float* ds;               // workspace f32 [E, H]
  float* wqkt;             // workspace f32 [2][C][C]: W_q^T, W_k^T
  void* mfma_ws;           // workspace of the matrix-core path
  float* wdq;              // if set: dq_j = sum_j' ds_jj' k_j' / sqrt(C/H), f32 [N, C]
  float* wdk;              // if set: dk_j = sum_i ds_ij q_i / sqrt(C/H), f32 [N, C]
  float* w_rad;            // if set (matrix-core path): dW_rad from the query pass itself, f32 [8, L+1, C]
  bool ds_later;           // matrix-core path: no query pass and no l = 0 terms (ds is formed later,
                           // and launch_bwd_qk is called after it)
  float box[3];
  int periodic;
};
// Scalar passes (any shape), and the matrix-core passes with their helpers.
// grad_feat may be null: then only ds (and wdq, wdk if set) are formed.
e2a_status launch_attention_backward(const BwdPlan& p, hipStream_t s);
e2a_status launch_backward_mfma(const BwdPlan& p, hipStream_t s);
e2a_status launch_bwd_delta(const BwdPlan& p, float* delta, hipStream_t s);
e2a_status launch_bwd_qk(const BwdPlan& p, hipStream_t s);
// dW_rad by the matrix-core radial pass (the MFMA build's shapes), into w_rad.
e2a_status launch_radial_mfma(const BwdPlan& p, float* w_rad, hipStream_t s);

// One block around the layer (block.hip).
struct BlockWs {
  size_t n1, attn, h1, n2, z, inv2, wf;   // Norm1, layer output / FFN hidden, h1, Norm2 / gated act, gate logits,
                                         // Norm2's inverse RMS per atom and degree, node-wise weights
  size_t attn_ws, attn_ws_bytes;    // the layer's own workspace
  size_t total;
};
BlockWs block_ws_layout(int64_t n, int L, int C, int H, int dtype);
bool block_uses_mfma(int C, int dtype);
struct BlockPlan {
  const e2a_block_args* b;
  BlockWs ws;
  e2a_status (*attention)(const e2a_attn_args* a, hipStream_t s);   // the checked forward
};
e2a_status launch_block(const BlockPlan& p, hipStream_t s);
// q = h0 W_q, k = h0 W_k on the matrix cores (bf16 storage, C a multiple of 32):
// bf16 products are exact, sums fp32.
e2a_status launch_qk_mfma(const uint16_t* feat, const uint16_t* wq, const uint16_t* wk, uint16_t* wqk_t, int64_t n,
                          int K, int C, float* q, float* k, hipStream_t s);

// Weight gradients (attention_wgrad.hip), after ds and dq, dk are formed.
struct WgradPlan {
  const e2a_attn_args* a;
  const float* grad_out;   // G [N, K, C]
  const float* q;          // f32 [N, C]
  const float* k;          // f32 [N, C]
  const float* dq;         // f32 [N, C] (needed for w_q)
  const float* dk;         // f32 [N, C] (needed for w_k)
  float* w_q;              // outputs, each optional
  float* w_k;
  float* w_rad;
  float* w_so2;
  float* pos;              // dL/dx [N, 3] (optional)
  const uint16_t* grad_bf; // G in bf16 (round to nearest even) if the call already made it, else null
  float* ds;               // if set (with pos; bf16, C = 128, H = 8): the softmax gradient [E, H] of every
                           // edge, formed from the batches' y and dy instead of a query pass
  const float* delta;      // with ds: delta = sum G o per atom and head [N, H]
  void* ws;                // wgrad_workspace_bytes(...)
  float box[3];
  int periodic;
};
size_t wgrad_workspace_bytes(int64_t n, int64_t e, int L, int C, int H, int dtype);
e2a_status launch_weight_grads(const WgradPlan& p, hipStream_t s);

}  // namespace e2a

// C ABI of libe2a: argument checks (host only, before any launch), workspace
// carving and dispatch.  See include/e2a.h for the contract of each call.
#include <cmath>
#include <cstring>
#include <mutex>

#include "e2a_internal.hpp"

namespace e2a {

namespace {
thread_local char g_msg[512] = "";
}

e2a_status fail(e2a_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_msg[0] = '\0'; }

namespace {

struct AttnWs {
  size_t q, k, wqk_t, w, total;
};

AttnWs attn_ws_layout(int64_t n, int L, int C, int H, int dtype) {
  AttnWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.q = take(sizeof(float) * (size_t)n * C);
  w.k = take(sizeof(float) * (size_t)n * C);
  w.wqk_t = take(block_uses_mfma(C, dtype) ? sizeof(uint16_t) * 2 * (size_t)C * C : 0);
  w.w = take(mfma_supported(L, C, H, dtype) ? mfma_workspace_bytes(n, L, C, false) : 0);
  w.total = off;
  return w;
}

struct BwdWs {
  size_t q, k, dq, dk, ds, wqkt, wqk_bf, mfma, total;
};

// The matrix-core region is sized whenever (L, C, H) has a bf16 build, so
// that the size does not depend on the storage type.
BwdWs bwd_ws_layout(int64_t n, int64_t e, int L, int C, int H) {
  BwdWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.q = take(sizeof(float) * (size_t)n * C);
  w.k = take(sizeof(float) * (size_t)n * C);
  w.dq = take(sizeof(float) * (size_t)n * C);
  w.dk = take(sizeof(float) * (size_t)n * C);
  w.ds = take(sizeof(float) * (size_t)e * H);
  w.wqkt = take(sizeof(float) * 2 * (size_t)C * C);
  w.wqk_bf = take(sizeof(uint16_t) * 2 * (size_t)C * C);
  w.mfma = take(mfma_supported(L, C, H, E2A_DTYPE_BF16) ? mfma_workspace_bytes(n, L, C, true) : 0);
  w.total = off;
  return w;
}

bool finite_positive(float x) { return std::isfinite(x) && x > 0.0f; }

// The weight-gradient call: the feature-gradient workspace, dq and dk, and
// the batches of the weight GEMMs.
struct WBwdWs {
  BwdWs b;
  size_t dq, dk, wg, total;
};

WBwdWs wbwd_ws_layout(int64_t n, int64_t e, int L, int C, int H) {
  WBwdWs w{};
  w.b = bwd_ws_layout(n, e, L, C, H);
  size_t off = w.b.total;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.dq = take(sizeof(float) * (size_t)n * C);
  w.dk = take(sizeof(float) * (size_t)n * C);
  w.wg = take(wgrad_workspace_bytes(n, e, L, C, H, E2A_DTYPE_F32));
  w.total = off;
  return w;
}

// Checks shared by the backward calls (all inputs; the outputs are checked
// by each call).
// Device arrays are read in 16-byte vectors: every array argument must start
// on a 16-byte boundary (hipMalloc and PyTorch's allocator give 256).
bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

e2a_status check_alignment(const e2a_attn_args* a, const void* grad_out) {
  const void* ptrs[] = {a->pos,     a->row_ptr, a->col, a->feat,         a->w_q,    a->w_k,
                        a->w_rad,   a->w_so2,   a->out, a->out_lse,      a->workspace,
                        a->w_so2_packed, a->order, grad_out};
  const char* names[] = {"pos",   "row_ptr", "col", "feat",         "w_q",   "w_k",      "w_rad",
                         "w_so2", "out",     "out_lse", "workspace", "w_so2_packed", "order", "grad_out"};
  for (size_t t = 0; t < sizeof(ptrs) / sizeof(ptrs[0]); ++t)
    if (misaligned(ptrs[t])) return fail(E2A_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[t]);
  return E2A_OK;
}

// The matrix-core build covers the call (the feature gradient then runs the
// fused kernel's passes).
bool rad_mfma_path(const e2a_attn_args* a) {
  const bool mfma_ok = mfma_supported(a->L, a->C, a->H, a->dtype);
  return a->variant == E2A_VARIANT_MFMA || (a->variant == E2A_VARIANT_AUTO && mfma_ok);
}

e2a_status check_bwd_args(const e2a_attn_args* a, const float* grad_out) {
  if (!a) return fail(E2A_ERR_INVALID_ARG, "args is NULL");
  if (a->n_atoms < 0 || a->n_atoms > INT32_MAX) return fail(E2A_ERR_INVALID_ARG, "n_atoms out of range");
  if (a->n_edges < 0) return fail(E2A_ERR_INVALID_ARG, "n_edges < 0");
  if (a->L < 0 || a->L > 4) return fail(E2A_ERR_INVALID_ARG, "L=%d outside 0..4", a->L);
  if (a->C <= 0 || a->H <= 0) return fail(E2A_ERR_INVALID_ARG, "C and H must be positive");
  if (a->C % a->H != 0) return fail(E2A_ERR_INVALID_ARG, "C=%d is not a multiple of H=%d", a->C, a->H);
  if (a->H > 192) return fail(E2A_ERR_UNSUPPORTED, "H=%d; the backward kernels take at most 192 heads", a->H);
  if (a->n_rbf != 8) return fail(E2A_ERR_INVALID_ARG, "n_rbf=%d; only 8 is supported", a->n_rbf);
  if (a->dtype != E2A_DTYPE_F32 && a->dtype != E2A_DTYPE_BF16) return fail(E2A_ERR_INVALID_ARG, "dtype=%d", a->dtype);
  if (a->variant < E2A_VARIANT_AUTO || a->variant > E2A_VARIANT_MFMA)
    return fail(E2A_ERR_INVALID_ARG, "variant=%d", a->variant);
  if (a->variant == E2A_VARIANT_MFMA && !mfma_supported(a->L, a->C, a->H, a->dtype))
    return fail(E2A_ERR_UNSUPPORTED, "MFMA kernel not built for L=%d C=%d H=%d dtype=%d", a->L, a->C, a->H, a->dtype);
  if (!finite_positive(a->cutoff)) return fail(E2A_ERR_INVALID_ARG, "cutoff must be finite and > 0");
  if (a->n_atoms > 0) {
    const void* ptrs[] = {a->pos, a->row_ptr, a->feat, a->w_q, a->w_k, a->w_rad, a->w_so2, a->out, a->out_lse,
                          grad_out};
    const char* names[] = {"pos", "row_ptr", "feat", "w_q", "w_k", "w_rad", "w_so2", "out", "out_lse",
                           "grad_out"};
    for (int t = 0; t < 10; ++t)
      if (!ptrs[t]) return fail(E2A_ERR_INVALID_ARG, "%s is NULL", names[t]);
    if (a->n_edges > 0 && !a->col) return fail(E2A_ERR_INVALID_ARG, "col is NULL");
    const e2a_status al = check_alignment(a, grad_out);
    if (al != E2A_OK) return al;
  }
  if (a->box)
    for (int d = 0; d < 3; ++d)
      if (!finite_positive(a->box[d])) return fail(E2A_ERR_INVALID_ARG, "box[%d] must be finite and > 0", d);
  return E2A_OK;
}

// The feature gradient's plan over the workspace layout ws.
BwdPlan bwd_plan(const e2a_attn_args* a, const float* grad_out, float* grad_feat, float* wdq, float* wdk, char* base,
                 const BwdWs& ws) {
  BwdPlan pl{};
  pl.a = a;
  pl.grad_out = grad_out;
  pl.grad_feat = grad_feat;
  pl.q = reinterpret_cast<float*>(base + ws.q);
  pl.k = reinterpret_cast<float*>(base + ws.k);
  pl.dq = reinterpret_cast<float*>(base + ws.dq);
  pl.dk = reinterpret_cast<float*>(base + ws.dk);
  pl.ds = reinterpret_cast<float*>(base + ws.ds);
  pl.wqkt = reinterpret_cast<float*>(base + ws.wqkt);
  pl.mfma_ws = base + ws.mfma;
  pl.wdq = wdq;
  pl.wdk = wdk;
  pl.periodic = a->box != nullptr;
  for (int d = 0; d < 3; ++d) pl.box[d] = a->box ? a->box[d] : 0.0f;
  return pl;
}

// q, k, then the query pass (ds) and, with grad_feat, the value pass and the
// l = 0 terms; dq and dk to wdq, wdk when those are set; dW_rad from the
// query pass into w_rad when that is set (matrix-core path only).  With
// ds_later (matrix-core path) the query pass and the l = 0 terms are left
// out: the caller forms ds itself and then calls launch_bwd_qk.
e2a_status run_backward(const e2a_attn_args* a, const float* grad_out, float* grad_feat, float* wdq, float* wdk,
                        char* base, const BwdWs& ws, hipStream_t s, float* w_rad = nullptr, bool ds_later = false) {
  AttnPlan qk{};
  qk.a = a;
  qk.q = reinterpret_cast<float*>(base + ws.q);
  qk.k = reinterpret_cast<float*>(base + ws.k);
  qk.wqk_t = reinterpret_cast<uint16_t*>(base + ws.wqk_bf);
  BwdPlan pl = bwd_plan(a, grad_out, grad_feat, wdq, wdk, base, ws);
  e2a_status st = launch_qk(qk, s);
  if (st != E2A_OK) return st;
  const bool mfma_ok = mfma_supported(a->L, a->C, a->H, a->dtype);
  const bool use_mfma = a->variant == E2A_VARIANT_MFMA || (a->variant == E2A_VARIANT_AUTO && mfma_ok);
  pl.w_rad = use_mfma ? w_rad : nullptr;
  pl.ds_later = use_mfma && ds_later;
  return use_mfma ? launch_backward_mfma(pl, s) : launch_attention_backward(pl, s);
}

}  // namespace
}  // namespace e2a

using namespace e2a;

extern "C" {

int e2a_version(void) { return E2A_ABI_VERSION; }

const char* e2a_status_string(e2a_status s) {
  switch (s) {
    case E2A_OK: return "E2A_OK";
    case E2A_ERR_INVALID_ARG: return "E2A_ERR_INVALID_ARG";
    case E2A_ERR_CAPACITY: return "E2A_ERR_CAPACITY";
    case E2A_ERR_BOX_TOO_SMALL: return "E2A_ERR_BOX_TOO_SMALL";
    case E2A_ERR_UNSUPPORTED: return "E2A_ERR_UNSUPPORTED";
    case E2A_ERR_HIP: return "E2A_ERR_HIP";
    default: return "E2A_ERR_UNKNOWN";
  }
}

const char* e2a_last_error_message(void) { return g_msg; }

size_t e2a_neighbors_workspace_bytes(int64_t n_atoms) {
  return n_atoms < 0 ? 0 : neighbors_workspace_bytes(n_atoms);
}

e2a_status e2a_build_neighbors(const float* pos, int64_t n_atoms, const int32_t* batch, const float* box,
                               float cutoff, int64_t* row_ptr, int32_t* col, int64_t col_capacity,
                               int64_t* n_edges, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (n_atoms < 0 || n_atoms > INT32_MAX) return fail(E2A_ERR_INVALID_ARG, "n_atoms=%lld out of range", (long long)n_atoms);
  if (!n_edges) return fail(E2A_ERR_INVALID_ARG, "n_edges is NULL");
  if (!row_ptr) return fail(E2A_ERR_INVALID_ARG, "row_ptr is NULL");
  if (n_atoms > 0 && !pos) return fail(E2A_ERR_INVALID_ARG, "pos is NULL");
  if (col_capacity < 0) return fail(E2A_ERR_INVALID_ARG, "col_capacity < 0");
  if (col_capacity > 0 && !col) return fail(E2A_ERR_INVALID_ARG, "col is NULL");
  if (!finite_positive(cutoff)) return fail(E2A_ERR_INVALID_ARG, "cutoff must be finite and > 0");
  if (box) {
    for (int d = 0; d < 3; ++d) {
      if (!finite_positive(box[d])) return fail(E2A_ERR_INVALID_ARG, "box[%d] must be finite and > 0", d);
      if (box[d] < 2.0f * cutoff)
        return fail(E2A_ERR_BOX_TOO_SMALL, "box[%d]=%g < 2*cutoff=%g", d, (double)box[d], 2.0 * cutoff);
    }
  }
  const size_t need = neighbors_workspace_bytes(n_atoms);
  if (n_atoms > 0 && (!workspace || workspace_bytes < need))
    return fail(E2A_ERR_INVALID_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  return build_neighbors_impl(pos, n_atoms, batch, box, cutoff, row_ptr, col, col_capacity, n_edges, workspace,
                              workspace_bytes, static_cast<hipStream_t>(stream));
}

int64_t e2a_so2_param_count(int L, int C) {
  if (L < 0 || C <= 0) return 0;
  int64_t n = 0;
  for (int m = 0; m <= L; ++m) {
    const int64_t k = (int64_t)(L + 1 - m) * C;
    n += (m == 0 ? 1 : 2) * k * k;
  }
  return n;
}

size_t e2a_so2_packed_bytes(int L, int C, int dtype) {
  if (L < 1 || L > 4 || !mfma_supported(L, C, 8, dtype)) return 0;
  return mfma_packed_bytes(L);
}

e2a_status e2a_pack_so2_weights(const void* w_so2, void* w_packed, int L, int C, int dtype, void* stream) {
  clear_error();
  if (L < 0 || L > 4) return fail(E2A_ERR_INVALID_ARG, "L=%d outside 0..4", L);
  if (e2a_so2_packed_bytes(L, C, dtype) == 0)
    return fail(E2A_ERR_UNSUPPORTED, "no matrix-core build (packed image) for L=%d C=%d dtype=%d", L, C, dtype);
  if (!w_so2 || !w_packed) return fail(E2A_ERR_INVALID_ARG, "w_so2 and w_packed must be set");
  return pack_so2_mfma(w_so2, w_packed, L, static_cast<hipStream_t>(stream));
}

size_t e2a_destination_order_workspace_bytes(int64_t n_atoms) {
  return n_atoms < 0 ? 0 : order_workspace_bytes(n_atoms);
}

e2a_status e2a_destination_order(const float* pos, int64_t n_atoms, int32_t* order, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  clear_error();
  if (n_atoms < 0 || n_atoms > INT32_MAX) return fail(E2A_ERR_INVALID_ARG, "n_atoms out of range");
  if (n_atoms == 0) return E2A_OK;
  if (!pos || !order) return fail(E2A_ERR_INVALID_ARG, "pos and order must be set");
  const size_t need = order_workspace_bytes(n_atoms);
  if (!workspace || workspace_bytes < need)
    return fail(E2A_ERR_INVALID_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  return destination_order(pos, n_atoms, order, workspace, static_cast<hipStream_t>(stream));
}

size_t e2a_attention_workspace_bytes(int64_t n_atoms, int L, int C, int H, int dtype) {
  if (n_atoms < 0 || L < 0 || L > 4 || C <= 0 || H <= 0) return 0;
  return attn_ws_layout(n_atoms, L, C, H, dtype).total;
}

}  // extern "C"

namespace {

// Shared body of the attention and convolution entry points: host-side
// argument checks, then the launches.  The convolution needs no W_q / W_k and
// writes no log-normaliser.
e2a_status check_layer_args(const e2a_attn_args* a, bool conv) {
  if (!a) return fail(E2A_ERR_INVALID_ARG, "args is NULL");
  if (a->n_atoms < 0 || a->n_atoms > INT32_MAX) return fail(E2A_ERR_INVALID_ARG, "n_atoms out of range");
  if (a->n_edges < 0) return fail(E2A_ERR_INVALID_ARG, "n_edges < 0");
  if (a->L < 0 || a->L > 4) return fail(E2A_ERR_INVALID_ARG, "L=%d outside 0..4", a->L);
  if (a->C <= 0 || a->H <= 0) return fail(E2A_ERR_INVALID_ARG, "C and H must be positive");
  if (a->C % a->H != 0) return fail(E2A_ERR_INVALID_ARG, "C=%d is not a multiple of H=%d", a->C, a->H);
  if (a->n_rbf != 8) return fail(E2A_ERR_INVALID_ARG, "n_rbf=%d; only 8 is supported", a->n_rbf);
  if (a->dtype != E2A_DTYPE_F32 && a->dtype != E2A_DTYPE_BF16) return fail(E2A_ERR_INVALID_ARG, "dtype=%d", a->dtype);
  if (a->variant < E2A_VARIANT_AUTO || a->variant > E2A_VARIANT_MFMA)
    return fail(E2A_ERR_INVALID_ARG, "variant=%d", a->variant);
  if (!finite_positive(a->cutoff)) return fail(E2A_ERR_INVALID_ARG, "cutoff must be finite and > 0");
  if (a->n_atoms > 0) {
    const void* ptrs[] = {a->pos, a->row_ptr, a->feat, a->w_rad, a->w_so2, a->out, a->w_q, a->w_k};
    const char* names[] = {"pos", "row_ptr", "feat", "w_rad", "w_so2", "out", "w_q", "w_k"};
    const int need = conv ? 6 : 8;
    for (int t = 0; t < need; ++t)
      if (!ptrs[t]) return fail(E2A_ERR_INVALID_ARG, "%s is NULL", names[t]);
    if (a->n_edges > 0 && !a->col) return fail(E2A_ERR_INVALID_ARG, "col is NULL");
    const e2a_status al = check_alignment(a, nullptr);
    if (al != E2A_OK) return al;
  }
  if (a->box)
    for (int d = 0; d < 3; ++d)
      if (!finite_positive(a->box[d])) return fail(E2A_ERR_INVALID_ARG, "box[%d] must be finite and > 0", d);
  const bool mfma_ok = mfma_supported(a->L, a->C, a->H, a->dtype);
  if (a->variant == E2A_VARIANT_MFMA && !mfma_ok)
    return fail(E2A_ERR_UNSUPPORTED, "MFMA kernel not built for L=%d C=%d H=%d dtype=%d", a->L, a->C, a->H, a->dtype);
  const AttnWs ws = attn_ws_layout(a->n_atoms, a->L, a->C, a->H, a->dtype);
  if (a->n_atoms > 0 && (!a->workspace || a->workspace_bytes < ws.total))
    return fail(E2A_ERR_INVALID_ARG, "workspace too small: %zu < %zu", a->workspace_bytes, ws.total);
  return E2A_OK;
}

e2a_status run_layer(const e2a_attn_args* a, void* stream, bool conv) {
  e2a_status chk = check_layer_args(a, conv);
  if (chk != E2A_OK) return chk;
  if (a->n_atoms == 0) return E2A_OK;
  const bool mfma_ok = mfma_supported(a->L, a->C, a->H, a->dtype);
  const AttnWs ws = attn_ws_layout(a->n_atoms, a->L, a->C, a->H, a->dtype);

  AttnPlan pl{};
  pl.a = a;
  char* base = static_cast<char*>(a->workspace);
  pl.q = reinterpret_cast<float*>(base + ws.q);
  pl.k = reinterpret_cast<float*>(base + ws.k);
  pl.wqk_t = reinterpret_cast<uint16_t*>(base + ws.wqk_t);
  pl.mfma_ws = base + ws.w;
  pl.periodic = a->box != nullptr;
  pl.conv = conv;
  for (int d = 0; d < 3; ++d) pl.box[d] = a->box ? a->box[d] : 0.0f;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (!conv) {
    e2a_status st = launch_qk(pl, s);
    if (st != E2A_OK) return st;
  }
  const bool use_mfma = a->variant == E2A_VARIANT_MFMA || (a->variant == E2A_VARIANT_AUTO && mfma_ok);
  return use_mfma ? launch_attention_mfma(pl, s) : launch_attention_reference(pl, s);
}

}  // namespace

extern "C" {

e2a_status e2a_attention_fwd(const e2a_attn_args* a, void* stream) {
  clear_error();
  return run_layer(a, stream, false);
}

}  // extern "C"

namespace {

// Scratch of e2a_attention_fwd_noalloc: one array per GPU, loaded with the
// library's code object and held until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = E2A_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array (looked up on the first
// call on that device, with the device current).
e2a_status scratch_of_current_device(void** out) {
  int dev = 0;
  E2A_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(E2A_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    E2A_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(E2A_ERR_HIP, "hipGetSymbolAddress returned a null scratch address on device %d", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return E2A_OK;
}

}  // namespace

extern "C" {

e2a_status e2a_attention_fwd_noalloc(const e2a_attn_args* a, void* stream) {
  clear_error();
  if (!a) return fail(E2A_ERR_INVALID_ARG, "args is NULL");
  // 0 for shapes no entry point takes: run_layer then names the bad argument
  const size_t need = e2a_attention_workspace_bytes(a->n_atoms, a->L, a->C, a->H, a->dtype);
  if (need > kNoAllocScratchBytes)
    return fail(E2A_ERR_INVALID_ARG,
                "n_atoms=%lld, L=%d, C=%d needs %zu bytes of scratch; e2a_attention_fwd_noalloc holds %zu "
                "(use e2a_attention_fwd with a workspace)",
                (long long)a->n_atoms, a->L, a->C, need, kNoAllocScratchBytes);
  e2a_attn_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (need > 0 && a->n_atoms > 0) {
    e2a_status st = scratch_of_current_device(&b.workspace);
    if (st != E2A_OK) return st;
    b.workspace_bytes = kNoAllocScratchBytes;
  }
  return run_layer(&b, stream, false);
}

e2a_status e2a_conv_fwd(const e2a_attn_args* a, void* stream) {
  clear_error();
  return run_layer(a, stream, true);
}

}  // extern "C"

namespace {

e2a_status block_attention(const e2a_attn_args* a, hipStream_t s) { return run_layer(a, s, false); }

BlockWs block_layout_full(int64_t n, int L, int C, int H, int dtype) {
  BlockWs w = block_ws_layout(n, L, C, H, dtype);
  w.attn_ws_bytes = attn_ws_layout(n, L, C, H, dtype).total;
  w.total = align_up(w.attn_ws + w.attn_ws_bytes, 256);
  return w;
}

}  // namespace

extern "C" {

size_t e2a_block_workspace_bytes(int64_t n_atoms, int L, int C, int H, int dtype) {
  if (n_atoms < 0 || L < 0 || L > 4 || C <= 0 || H <= 0 || (dtype != E2A_DTYPE_F32 && dtype != E2A_DTYPE_BF16))
    return 0;
  return block_layout_full(n_atoms, L, C, H, dtype).total;
}

e2a_status e2a_block_fwd(const e2a_block_args* b, void* stream) {
  clear_error();
  if (!b) return fail(E2A_ERR_INVALID_ARG, "args is NULL");
  if (b->n_atoms < 0 || b->n_atoms > INT32_MAX) return fail(E2A_ERR_INVALID_ARG, "n_atoms out of range");
  if (b->L < 0 || b->L > 4) return fail(E2A_ERR_INVALID_ARG, "L=%d outside 0..4", b->L);
  if (b->C <= 0 || b->H <= 0) return fail(E2A_ERR_INVALID_ARG, "C and H must be positive");
  if (b->dtype != E2A_DTYPE_F32 && b->dtype != E2A_DTYPE_BF16) return fail(E2A_ERR_INVALID_ARG, "dtype=%d", b->dtype);
  if (b->C % 4 != 0) return fail(E2A_ERR_UNSUPPORTED, "block: C=%d is not a multiple of 4", b->C);
  if (b->n_atoms * (2 * b->L + 1) >= (int64_t)INT32_MAX)
    return fail(E2A_ERR_UNSUPPORTED, "block: n_atoms * (2L+1) must stay below 2^31");
  if (b->n_atoms > 0) {
    const void* ptrs[] = {b->h_in, b->h_out, b->norm1, b->w_o, b->norm2, b->w_1, b->w_2};
    const char* names[] = {"h_in", "h_out", "norm1", "w_o", "norm2", "w_1", "w_2"};
    for (int t = 0; t < 7; ++t)
      if (!ptrs[t]) return fail(E2A_ERR_INVALID_ARG, "%s is NULL", names[t]);
    if (b->L > 0 && !b->w_gate) return fail(E2A_ERR_INVALID_ARG, "w_gate is NULL");
    // the norms read h_in and the last GEMM writes h_out 16 bytes a lane
    if (misaligned(b->h_in)) return fail(E2A_ERR_INVALID_ARG, "h_in is not 16-byte aligned");
    if (misaligned(b->h_out)) return fail(E2A_ERR_INVALID_ARG, "h_out is not 16-byte aligned");
  }
  const BlockWs ws = block_layout_full(b->n_atoms, b->L, b->C, b->H, b->dtype);
  if (b->n_atoms > 0 && (!b->workspace || b->workspace_bytes < ws.total))
    return fail(E2A_ERR_INVALID_ARG, "workspace too small: %zu < %zu", b->workspace_bytes, ws.total);
  // the layer's own argument checks (pointers, shapes, variant) on a dry
  // copy of its arguments, before anything is launched
  e2a_attn_args a{};
  a.pos = b->pos;
  a.box = b->box;
  a.n_atoms = b->n_atoms;
  a.row_ptr = b->row_ptr;
  a.col = b->col;
  a.n_edges = b->n_edges;
  a.cutoff = b->cutoff;
  a.L = b->L;
  a.C = b->C;
  a.H = b->H;
  a.n_rbf = b->n_rbf;
  a.dtype = b->dtype;
  a.variant = b->variant;
  a.w_q = b->w_q;
  a.w_k = b->w_k;
  a.w_rad = b->w_rad;
  a.w_so2 = b->w_so2;
  a.feat = b->workspace;
  a.out = reinterpret_cast<float*>(b->workspace);
  a.workspace = b->workspace;
  a.workspace_bytes = ws.attn_ws_bytes;
  e2a_status st = check_layer_args(&a, false);
  if (st != E2A_OK) return st;
  if (b->n_atoms == 0) return E2A_OK;
  BlockPlan p{};
  p.b = b;
  p.ws = ws;
  p.attention = block_attention;
  return launch_block(p, static_cast<hipStream_t>(stream));
}

size_t e2a_attention_bwd_workspace_bytes(int64_t n_atoms, int64_t n_edges, int L, int C, int H) {
  if (n_atoms < 0 || n_edges < 0 || L < 0 || L > 4 || C <= 0 || H <= 0) return 0;
  return bwd_ws_layout(n_atoms, n_edges, L, C, H).total;
}

e2a_status e2a_attention_bwd(const e2a_attn_args* a, const float* grad_out, float* grad_feat, void* stream) {
  clear_error();
  e2a_status st = check_bwd_args(a, grad_out);
  if (st != E2A_OK) return st;
  if (a->n_atoms > 0 && !grad_feat) return fail(E2A_ERR_INVALID_ARG, "grad_feat is NULL");
  const BwdWs ws = bwd_ws_layout(a->n_atoms, a->n_edges, a->L, a->C, a->H);
  if (a->n_atoms > 0 && (!a->workspace || a->workspace_bytes < ws.total))
    return fail(E2A_ERR_INVALID_ARG, "workspace too small: %zu < %zu", a->workspace_bytes, ws.total);
  if (a->n_atoms == 0) return E2A_OK;
  return run_backward(a, grad_out, grad_feat, nullptr, nullptr, static_cast<char*>(a->workspace), ws,
                      static_cast<hipStream_t>(stream));
}

size_t e2a_attention_bwd_weights_workspace_bytes(int64_t n_atoms, int64_t n_edges, int L, int C, int H) {
  if (n_atoms < 0 || n_edges < 0 || L < 0 || L > 4 || C <= 0 || H <= 0) return 0;
  return wbwd_ws_layout(n_atoms, n_edges, L, C, H).total;
}

e2a_status e2a_attention_bwd_weights(const e2a_attn_args* a, const float* grad_out, float* grad_feat,
                                     float* grad_w_q, float* grad_w_k, float* grad_w_rad, float* grad_w_so2,
                                     float* grad_pos, void* stream) {
  clear_error();
  e2a_status st = check_bwd_args(a, grad_out);
  if (st != E2A_OK) return st;
  if (!grad_feat && !grad_w_q && !grad_w_k && !grad_w_rad && !grad_w_so2 && !grad_pos)
    return fail(E2A_ERR_INVALID_ARG, "no output requested");
  const WBwdWs ws = wbwd_ws_layout(a->n_atoms, a->n_edges, a->L, a->C, a->H);
  if (a->n_atoms > 0 && (!a->workspace || a->workspace_bytes < ws.total))
    return fail(E2A_ERR_INVALID_ARG, "workspace too small: %zu < %zu", a->workspace_bytes, ws.total);
  if (a->n_atoms == 0) return E2A_OK;
  char* base = static_cast<char*>(a->workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* dq = reinterpret_cast<float*>(base + ws.dq);
  float* dk = reinterpret_cast<float*>(base + ws.dk);
  const bool want_qk = grad_w_q || grad_w_k;
  // dW_rad by the fused kernel's radial accumulation where the MFMA build
  // covers the shape, so that the batches need neither SO2(x) for it
  // (without the positions) nor dyhat beside dy (with them); when the query
  // pass runs anyway it accumulates dW_rad itself
  const bool mfma_ok = mfma_supported(a->L, a->C, a->H, a->dtype);
  const bool rad_mfma = grad_w_rad &&
                        (a->variant == E2A_VARIANT_MFMA || (a->variant == E2A_VARIANT_AUTO && mfma_ok));
  const bool rad_in_query = rad_mfma && (grad_feat || want_qk);
  // dL/dh with the positions and no weight but W_so2 (the forces): the edge
  // batches hold y and dy, from which ds follows without a query pass (one
  // read of the two against one more pass of the fused kernel)
  const bool ds_batches = grad_pos && grad_feat && !want_qk && !grad_w_rad && rad_mfma_path(a) &&
                          a->dtype == E2A_DTYPE_BF16 && a->C == 128 && a->H == 8 && a->L >= 1;
  if (grad_feat || want_qk) {
    // the softmax gradient ds (and dL/dh when asked for); dq, dk from it
    st = run_backward(a, grad_out, grad_feat, want_qk ? dq : nullptr, want_qk ? dk : nullptr, base, ws.b, s,
                      rad_in_query ? grad_w_rad : nullptr, ds_batches);
  } else {
    // dW_rad, dW_so2 and the positions need only q and k (for the
    // attention weights)
    AttnPlan qk{};
    qk.a = a;
    qk.q = reinterpret_cast<float*>(base + ws.b.q);
    qk.k = reinterpret_cast<float*>(base + ws.b.k);
    qk.wqk_t = reinterpret_cast<uint16_t*>(base + ws.b.wqk_bf);
    st = launch_qk(qk, s);
  }
  if (st != E2A_OK) return st;
  if (rad_mfma && !rad_in_query) {
    BwdPlan rp{};
    rp.a = a;
    rp.grad_out = grad_out;
    rp.q = reinterpret_cast<float*>(base + ws.b.q);
    rp.k = reinterpret_cast<float*>(base + ws.b.k);
    rp.mfma_ws = base + ws.b.mfma;
    rp.periodic = a->box != nullptr;
    for (int d = 0; d < 3; ++d) rp.box[d] = a->box ? a->box[d] : 0.0f;
    st = launch_radial_mfma(rp, grad_w_rad, s);
    if (st != E2A_OK) return st;
  }
  WgradPlan wp{};
  wp.a = a;
  wp.grad_out = grad_out;
  wp.q = reinterpret_cast<const float*>(base + ws.b.q);
  wp.k = reinterpret_cast<const float*>(base + ws.b.k);
  wp.dq = dq;
  wp.dk = dk;
  wp.w_q = grad_w_q;
  wp.w_k = grad_w_k;
  wp.w_rad = rad_mfma ? nullptr : grad_w_rad;
  wp.w_so2 = grad_w_so2;
  wp.pos = grad_pos;
  // the matrix-core feature gradient left the cotangent in bf16 (k_prep_grad)
  if ((grad_feat || want_qk) && rad_mfma_path(a)) wp.grad_bf = mfma_grad_bf16(base + ws.b.mfma, a->n_atoms, a->L);
  if (ds_batches) {
    wp.ds = reinterpret_cast<float*>(base + ws.b.ds);
    wp.delta = mfma_delta(base + ws.b.mfma, a->n_atoms, a->L);
  }
  wp.ws = base + ws.wg;
  wp.periodic = a->box != nullptr;
  for (int d = 0; d < 3; ++d) wp.box[d] = a->box ? a->box[d] : 0.0f;
  st = launch_weight_grads(wp, s);
  if (st != E2A_OK || !ds_batches) return st;
  // the l = 0 terms of dL/dh from the batches' ds
  return launch_bwd_qk(bwd_plan(a, grad_out, grad_feat, nullptr, nullptr, base, ws.b), s);
}

}  // extern "C"

// Weight and position gradients of the fused layer: dL/dW_q, dL/dW_k,
// dL/dW_rad, the per-m SO(2) blocks dL/dW_so2 and dL/dx, for a cotangent
// G = dL/do (the position gradient's own steps are described with its
// kernels below).
//
// arXiv 2601.16622, technical summary section 2.1 (the EAAS message: rotate
// in, per-m SO(2) mix, radial scale, rotate out) and section 2.2 (attention
// weights from invariant logits; the backward recomputes per-edge quantities
// from the per-destination softmax statistics).  With the edge cotangent
// alpha_ij G_i of the message v_ij = D^T (rho * SO2(D h_j)):
//   dyhat = D (alpha G_i)                          edge-frame cotangent of rho * y
//   drho[l][c] = sum_m y[l,m][c] dyhat[l,m][c]     y = SO2(x), x = D h_j
//   dW_rad[k][l][c] = sum over edges of e_k(r) drho[l][c]
//   dy = rho * dyhat
//   dW0 = X0^T dY0,  dW1 = Xp^T dYp + Xm^T dYm,  dW2 = Xp^T dYm - Xm^T dYp
//   dW_q = sum_i h_{i,0}^T dq_i,  dW_k = sum_j h_{j,0}^T dk_j.
// Each of these is a sum over all edges (or atoms) into a matrix far larger
// than a workgroup can hold, so unlike the forward this path keeps per-edge
// tensors: for a batch of edges it writes x and dyhat in the row layout of
// the per-m GEMMs (block 0: one row per edge, [B][(L+1)C]; block m > 0: the
// +m rows [B][(L+1-m)C], then the -m rows), forms Y = SO2(X) and the weight
// gradients as GEMMs, and moves on to the next batch.  The GEMMs sum in a
// fixed order (split-K partials reduced in order), so results are
// bit-reproducible.
#include <type_traits>

#include "e2a_geometry.hpp"
#include "e2a_internal.hpp"

namespace e2a {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int64_t kWgBatch = 262144;  // edges per batch (14 GB of batch tensors at L = 4, C = 128)
constexpr int kEB = 32;               // edges per gather workgroup (16: 0.5-0.7 ms more per training call, 8: 7 ms)
constexpr int64_t kRhoPer = 8;        // edges per k_wg_rho range

template <typename T>
__device__ __forceinline__ void store_as(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_as<float>(float* p, int64_t i, float v) {
  p[i] = v;
}
template <>
__device__ __forceinline__ void store_as<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16_rne(v);
}

// Element offsets of the per-m matrices in one batch tensor.
struct BatchLayout {
  int64_t B;         // rows per matrix (edges per batch)
  int64_t moff[5];   // block m: m = 0 one [B][K_0]; m > 0 [B][K_m] (+m rows) then [B][K_m] (-m rows)
  int64_t total;
};

BatchLayout batch_layout(int64_t B, int L, int C) {
  BatchLayout b{};
  b.B = B;
  int64_t o = 0;
  for (int m = 0; m <= L; ++m) {
    b.moff[m] = o;
    o += (m == 0 ? 1 : 2) * B * (int64_t)(L + 1 - m) * C;
  }
  b.total = o;
  return b;
}

// Place of row (l, m) channel c of batch edge b in a batch tensor.
__device__ __forceinline__ int64_t batch_index(const BatchLayout& bl, int L, int C, int64_t b, int l, int m, int c) {
  const int am = m < 0 ? -m : m;
  const int64_t km = (int64_t)(L + 1 - am) * C;
  return bl.moff[am] + (m < 0 ? bl.B * km : 0) + b * km + (int64_t)(l - am) * C + c;
}

__global__ void k_edge_rows(const int64_t* __restrict__ row_ptr, int64_t n, int32_t* __restrict__ src) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) src[e] = static_cast<int32_t>(i);
}

// Wt[n][k] = W[k][n] for one km x km block (the Y products read both
// operands along k).
template <typename T>
__global__ void k_transpose_block(const T* __restrict__ w, int64_t km, T* __restrict__ wt) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= km * km) return;
  const int64_t k = t / km, n = t - k * km;
  wt[n * km + k] = w[t];
}

// G in bf16, round to nearest even (the force kernel's operand, when the
// call has no copy from its feature gradient).
__global__ void k_to_bf16(const float* __restrict__ g, uint16_t* __restrict__ out, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) out[i] = f32_to_bf16_rne(g[i]);
}

__global__ void k_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

struct GatherParams {
  const float* pos;
  const int32_t* col;
  const int32_t* src;
  const float* q;
  const float* k;
  const float* lse;
  const float* grad;
  float box[3];
  int periodic;
  float cutoff;
  int C, H;
  int64_t e0, nb;   // the batch: edges e0 .. e0 + nb - 1 of the neighbour list
  BatchLayout bl;
  float* rbf;       // [B][8]
  float* rbfd;      // if set: d e_k / d r, [B][8]
  float* alpha;     // if set: the edges' attention weights, [B][H]
  const void* w_rad;   // the cotangent rows are written as dy = rho dyhat
  float* dyhat;        // if set: dyhat itself too, fp32, in the batch layout
};

// Degree l of the gather: one (edge, channel) per work item reads the
// degree's 2l + 1 feature and cotangent entries once and writes all 2l + 1
// rows of x and dy = rho dyhat (and of dyhat when asked for).
template <int L, int l, typename T>
__device__ __forceinline__ void gather_degree(const GatherParams& p, const T* __restrict__ feat, T* __restrict__ X,
                                              T* __restrict__ GT, const float* D, const float* al, const float* rb,
                                              const int* ii, const int* jj, int64_t b0, int tid) {
  constexpr int K = (L + 1) * (L + 1);
  constexpr int WS = wig_size(L);
  constexpr int w = 2 * l + 1;
  const int C = p.C, H = p.H, dh = C / H;
  const T* wr = static_cast<const T*>(p.w_rad);
  // one (edge, channel) of the degree; wrc holds the channel's radial weights
  auto item = [&](int s, int c, const float (&wrc)[8]) {
    if (ii[s] < 0) return;
    const T* hj = feat + ((int64_t)jj[s] * K + l * l) * C + c;
    const float* gi = p.grad + ((int64_t)ii[s] * K + l * l) * C + c;
    float hv[w], gv[w];
#pragma unroll
    for (int n = 0; n < w; ++n) {
      hv[n] = load_as_f32(hj, (size_t)n * C);
      gv[n] = gi[(int64_t)n * C];
    }
    const float a0 = al[s * H + c / dh];
    float rho = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) rho += rb[s * 8 + kk] * wrc[kk];
    const float a = a0 * rho;
    const float* Dl = D + s * WS + wig_off(l);
#pragma unroll
    for (int mi = 0; mi < w; ++mi) {
      float x = 0.0f, g = 0.0f;
#pragma unroll
      for (int n = 0; n < w; ++n) {
        x += Dl[mi * w + n] * hv[n];
        g += Dl[mi * w + n] * gv[n];
      }
      const int64_t idx = batch_index(p.bl, L, C, b0 + s, l, mi - l, c);
      store_as(X, idx, x);
      store_as(GT, idx, g * a);
      if (p.dyhat) p.dyhat[idx] = g * a0;
    }
  };
  auto load_wr = [&](int c, float (&wrc)[8]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) wrc[kk] = load_as_f32(wr, (size_t)(kk * (L + 1) + l) * C + c);
  };
  if (blockDim.x % C == 0) {
    // the thread keeps one channel for all its edges (C = 128: two edges a
    // pass), so its radial weights are loaded once per degree
    const int c = tid % C, step = blockDim.x / C;
    float wrc[8];
    load_wr(c, wrc);
    for (int s = tid / C; s < kEB; s += step) item(s, c, wrc);
  } else {
    for (int t = tid; t < kEB * C; t += blockDim.x) {
      const int s = t / C, c = t - s * C;
      float wrc[8];
      load_wr(c, wrc);
      item(s, c, wrc);
    }
  }
  if constexpr (l < L) gather_degree<L, l + 1, T>(p, feat, X, GT, D, al, rb, ii, jj, b0, tid);
}

// The same for bf16 storage with 16-byte accesses: one (edge, 8 channels)
// per work item, so that feature rows are read, and x and dy rows written,
// 16 bytes a lane, and every D entry read from LDS serves 8 channels.  Each
// channel's sums run in the order of gather_degree, so the results are the
// same bit for bit.  Needs C / 8 to divide the workgroup and a head to span
// a multiple of 8 channels.
template <int L, int l>
__device__ __forceinline__ void gather_degree_vec(const GatherParams& p, const uint16_t* __restrict__ feat,
                                                  uint16_t* __restrict__ X, uint16_t* __restrict__ GT,
                                                  const float* D, const float* al, const float* rb, const int* ii,
                                                  const int* jj, int64_t b0, int tid) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int K = (L + 1) * (L + 1);
  constexpr int WS = wig_size(L);
  constexpr int w = 2 * l + 1;
  const int C = p.C, H = p.H, dh = C / H;
  const int per = C / 8;                       // work items per edge
  const int o = tid % per, c0 = 8 * o;
  const uint16_t* wr = static_cast<const uint16_t*>(p.w_rad);
  auto lo16 = [](uint32_t u) { return __uint_as_float(u << 16); };
  auto hi16 = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
  for (int s = tid / per; s < kEB; s += blockDim.x / per) {
    if (ii[s] < 0) continue;
    const float* Dl = D + s * WS + wig_off(l);
    // x = D h_j, the feature rows kept packed
    {
      const uint16_t* hj = feat + ((int64_t)jj[s] * K + l * l) * C + c0;
      u32x4 hw[w];
#pragma unroll
      for (int n = 0; n < w; ++n) hw[n] = *reinterpret_cast<const u32x4*>(hj + (size_t)n * C);
#pragma unroll 1
      for (int mi = 0; mi < w; ++mi) {
        float x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = 0.0f;
#pragma unroll
        for (int n = 0; n < w; ++n) {
          const float d = Dl[mi * w + n];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            x[2 * q] += d * lo16(hw[n][q]);
            x[2 * q + 1] += d * hi16(hw[n][q]);
          }
        }
        u32x4 xo;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xo[q] = static_cast<uint32_t>(f32_to_bf16_rne(x[2 * q])) |
                  (static_cast<uint32_t>(f32_to_bf16_rne(x[2 * q + 1])) << 16);
        *reinterpret_cast<u32x4*>(X + batch_index(p.bl, L, C, b0 + s, l, mi - l, c0)) = xo;
      }
    }
    // dy = rho D (alpha G_i)
    const float a0 = al[s * H + c0 / dh];
    float a[8];
    {
      // the 8 channels' radial weights (L1-resident across the edges)
      float rho[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) rho[q] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(wr + (size_t)(kk * (L + 1) + l) * C + c0);
        const float r = rb[s * 8 + kk];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rho[2 * q] += r * lo16(u[q]);
          rho[2 * q + 1] += r * hi16(u[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) a[q] = a0 * rho[q];
    }
    const float* gi = p.grad + ((int64_t)ii[s] * K + l * l) * C + c0;
    f32x4 gw[w][2];
#pragma unroll
    for (int n = 0; n < w; ++n) {
      gw[n][0] = *reinterpret_cast<const f32x4*>(gi + (size_t)n * C);
      gw[n][1] = *reinterpret_cast<const f32x4*>(gi + (size_t)n * C + 4);
    }
#pragma unroll 1
    for (int mi = 0; mi < w; ++mi) {
      float g[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) g[q] = 0.0f;
#pragma unroll
      for (int n = 0; n < w; ++n) {
        const float d = Dl[mi * w + n];
#pragma unroll
        for (int q = 0; q < 8; ++q) g[q] += d * gw[n][q >> 2][q & 3];
      }
      const int64_t idx = batch_index(p.bl, L, C, b0 + s, l, mi - l, c0);
      u32x4 go;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        go[q] = static_cast<uint32_t>(f32_to_bf16_rne(g[2 * q] * a[2 * q])) |
                (static_cast<uint32_t>(f32_to_bf16_rne(g[2 * q + 1] * a[2 * q + 1])) << 16);
      *reinterpret_cast<u32x4*>(GT + idx) = go;
      if (p.dyhat) {
        *reinterpret_cast<f32x4*>(p.dyhat + idx) = f32x4{g[0] * a0, g[1] * a0, g[2] * a0, g[3] * a0};
        *reinterpret_cast<f32x4*>(p.dyhat + idx + 4) = f32x4{g[4] * a0, g[5] * a0, g[6] * a0, g[7] * a0};
      }
    }
  }
  if constexpr (l < L) gather_degree_vec<L, l + 1>(p, feat, X, GT, D, al, rb, ii, jj, b0, tid);
}

// D^l (l = 2..L) of the workgroup's edges from D^1 and D^{l-1}, one (edge,
// row) per thread and level (the row recursion of the fused kernel).
template <int L, int l>
__device__ __forceinline__ void gather_wigner(float* D, const int* ii, int tid) {
  if constexpr (l <= L) {
    constexpr int WS = wig_size(L), w = 2 * l + 1, wp = 2 * l - 1;
    for (int t = tid; t < kEB * w; t += blockDim.x) {
      const int s = t / w, mi = t - s * w;
      if (ii[s] < 0) continue;
      float* De = D + s * WS;
      float r1[3][3];
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) r1[a][b] = De[wig_off(1) + a * 3 + b];
      const float* Dp = De + wig_off(l - 1);
      auto rp = [&](int a) { return Dp + (a + l - 1) * wp; };
      float out[w];
      ir_row<l>(mi - l, r1, rp, out);
#pragma unroll
      for (int n = 0; n < w; ++n) De[wig_off(l) + mi * w + n] = out[n];
    }
    __syncthreads();
    gather_wigner<L, l + 1>(D, ii, tid);
  }
}

// The 16-byte gather applies: C / 8 items per edge dividing the workgroup,
// heads of a multiple of 8 channels.
__host__ __device__ inline bool gather_vec_ok(int C, int H, int threads) {
  return C % 8 == 0 && threads % (C / 8) == 0 && (C / H) % 8 == 0;
}

// x = D h_j and dyhat = D (alpha G_i) (or rho dyhat) for kEB edges of the
// batch: the edges' frames, D^0, D^1 and radial bases (one lane of the first
// wave per edge) while the other waves compute the attention weights (one
// (edge, head) per thread), then D^2 .. D^L row by row, then the degrees one
// after another.
template <int L, typename T>
__global__ void __launch_bounds__(256) k_wg_gather(GatherParams p, const T* __restrict__ feat, T* __restrict__ X,
                                                   T* __restrict__ GT) {
  constexpr int WS = wig_size(L);
  extern __shared__ float sm[];
  float* D = sm;                       // [kEB][WS]
  float* al = D + kEB * WS;            // [kEB][H]
  __shared__ float rb[kEB * 8];
  __shared__ int ii[kEB], jj[kEB];
  const int C = p.C, H = p.H, dh = C / H;
  const int64_t b0 = (int64_t)blockIdx.x * kEB;
  const int tid = threadIdx.x;
  static_assert(kEB <= 64, "one lane of the first wave per edge");
  if (tid < kEB) {
    const int64_t b = b0 + tid;
    ii[tid] = -1;
    if (b < p.nb) {
      const int64_t e = p.e0 + b;
      const int i = p.src[e], j = p.col[e];
      ii[tid] = i;
      jj[tid] = j;
      float r3[3];
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        float dx = p.pos[3 * (int64_t)j + d] - p.pos[3 * (int64_t)i + d];
        if (p.periodic) {
          if (dx > 0.5f * p.box[d]) dx -= p.box[d];
          else if (dx < -0.5f * p.box[d]) dx += p.box[d];
        }
        r3[d] = dx;
      }
      float u[3];
      const float r = edge_unit(r3, u);
      float R[3][3];
      edge_rotation(u, R);
      float* De = D + tid * WS;
      De[0] = 1.0f;
      if constexpr (L >= 1) wigner_l1(R, De + wig_off(1), 3);
      float e8[8];
      radial_basis8(r, p.cutoff, e8);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        p.rbf[b * 8 + kk] = e8[kk];
        rb[tid * 8 + kk] = e8[kk];
      }
      if (p.rbfd) {
        radial_basis8_deriv(r, p.cutoff, e8);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) p.rbfd[b * 8 + kk] = e8[kk];
      }
    }
  } else if (tid >= 64) {
    const float inv = 1.0f / sqrtf(static_cast<float>(dh));
    for (int t = tid - 64; t < kEB * H; t += blockDim.x - 64) {
      const int s = t / H, h = t - s * H;
      const int64_t b = b0 + s;
      if (b >= p.nb) continue;
      const int64_t e = p.e0 + b;
      const int64_t i = p.src[e], j = p.col[e];
      const float* qi = p.q + i * C + h * dh;
      const float* kj = p.k + j * C + h * dh;
      float sv = 0.0f;
      for (int d = 0; d < dh; ++d) sv += qi[d] * kj[d];
      const float a = expf(sv * inv - p.lse[i * H + h]);
      al[s * H + h] = a;
      if (p.alpha) p.alpha[b * H + h] = a;
    }
  }
  __syncthreads();
  gather_wigner<L, 2>(D, ii, tid);
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (gather_vec_ok(C, H, blockDim.x)) {
      gather_degree_vec<L, 0>(p, feat, X, GT, D, al, rb, ii, jj, b0, tid);
      return;
    }
  }
  gather_degree<L, 0, T>(p, feat, X, GT, D, al, rb, ii, jj, b0, tid);
}

// dW_rad partials from the edge batches: drho[b][l][c] = sum_m y[l,m][c]
// dyhat[l,m][c], summed into this range's part of dW_rad, part[z][k][(l, c)]
// (+)= sum over the range's edges b of rbf[b][k] drho[b][l][c] (added to
// what the slot holds from earlier batches when acc_parts is set).  One
// thread per (degree, channel) and range of edges (consecutive threads take
// consecutive channels, so the row reads coalesce); each edge's 2l + 1 rows
// are loaded together.
template <int L, int l, typename YT>
__device__ __forceinline__ void rho_degree(const BatchLayout& bl, int64_t nb, int C, int64_t per, int z, int c,
                                           const float* __restrict__ rbf, const YT* __restrict__ Y,
                                           const float* __restrict__ dyhat, float* __restrict__ part,
                                           bool acc_parts) {
  constexpr int w = 2 * l + 1;
  const int lc = l * C + c;
  float acc[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) acc[kk] = 0.0f;
  const int64_t b1 = (z + 1) * per < nb ? (z + 1) * per : nb;
  for (int64_t b = z * per; b < b1; ++b) {
    float g[w], y[w];
#pragma unroll
    for (int q = 0; q < w; ++q) {
      const int64_t idx = batch_index(bl, L, C, b, l, q - l, c);
      g[q] = dyhat[idx];
      y[q] = load_as_f32(Y, (size_t)idx);
    }
    float dr = 0.0f;
#pragma unroll
    for (int q = 0; q < w; ++q) dr += y[q] * g[q];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) acc[kk] += rbf[b * 8 + kk] * dr;
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    float* pp = part + ((int64_t)z * 8 + kk) * (L + 1) * C + lc;
    *pp = acc_parts ? *pp + acc[kk] : acc[kk];
  }
}

// The thread's degree ld as a compile-time constant (uniform over a wave when
// C is a multiple of 64).
template <int L, int l, typename YT>
__device__ __forceinline__ void rho_dispatch(int ld, const BatchLayout& bl, int64_t nb, int C, int64_t per, int z,
                                             int c, const float* __restrict__ rbf, const YT* __restrict__ Y,
                                             const float* __restrict__ dyhat, float* __restrict__ part,
                                             bool acc_parts) {
  if (ld == l) {
    rho_degree<L, l, YT>(bl, nb, C, per, z, c, rbf, Y, dyhat, part, acc_parts);
    return;
  }
  if constexpr (l < L) rho_dispatch<L, l + 1, YT>(ld, bl, nb, C, per, z, c, rbf, Y, dyhat, part, acc_parts);
}

template <int L, typename YT>
__global__ void k_wg_rho(BatchLayout bl, int64_t nb, int C, int64_t per, const float* __restrict__ rbf,
                         const YT* __restrict__ Y, const float* __restrict__ dyhat, float* __restrict__ part,
                         bool acc_parts) {
  const int lc = blockIdx.x * blockDim.x + threadIdx.x;
  const int z = blockIdx.y;
  if (lc >= (L + 1) * C) return;
  const int l = lc / C, c = lc - l * C;
  rho_dispatch<L, 0, YT>(l, bl, nb, C, per, z, c, rbf, Y, dyhat, part, acc_parts);
}

// ------------------------------------------------------------ positions ----
// The layer depends on an edge vector r = x_j - x_i through its length (the
// radial basis) and its direction (the Wigner blocks of the frame R).  The
// frame is any rotation taking r_hat to z (the SO(2) mix commutes with
// rotations about z), so turning r_hat by a small rotation w, r_hat ->
// r_hat + w x r_hat, may be followed by R -> R (1 - [w]x), D^l -> D^l(R) +
// dD^l with dR = -R [w]x: smooth everywhere, unlike the angles of R.  Then
//   dL/dw_a = sum_l <dL/dD^l, dD^l/dw_a>,
//   dL/dD^l[m][n] = sum_c dx[l,m][c] h_j[l,n][c] + yhat[l,m][c] alpha G_i[l,n][c]
// (x = D h_j enters the mix, v = D^T yhat leaves it, yhat = rho y, dx =
// SO2^T(rho dyhat)), and dL/dr = s r_hat + (T x r_hat) / |r| with
// T_a = dL/dw_a and s = sum_{l,c} drho[l][c] d rho[l][c] / d r.
struct ForceParams {
  const float* pos;
  const int32_t* col;
  const int32_t* src;
  const float* grad;    // G [N, K, C]
  const float* alpha;   // [B][H]
  const float* rbf;     // [B][8]
  const void* Y;        // batch tensor: y = SO2(x) (fp32, or bf16 for the matrix-core kernel)
  const void* dX;       // batch tensor: dx = SO2^T(dy) (the same type)
  const float* rbfd;    // [B][8]: d e_k / d r
  const uint16_t* gbf;  // G in bf16 [N, K, C] (the matrix-core kernel)
  float* gedge;         // [E][3]: dL/dr of every edge
  float box[3];
  int periodic;
  int C, H;
  int64_t e0;
  BatchLayout bl;
};

// Degree l's share of T_a = <dL/dD, dD/dw_a> for the wave's edge, where
// dL/dD^l[m][n] = sum_c dx[m][c] h_j[n][c] + yhat[m][c] (alpha G_i)[n][c]: per
// channel (every 64th for the lane) the tangent blocks are applied to h_j and
// alpha G_i first, T_a += sum_m dx[m] (D_a h)[m] + yhat[m] (D_a alpha G)[m], so
// that no (2l + 1)^2 partial of dL/dD is held per lane; the wave sums the
// three numbers at the end.  The lane also sums its channels' share of the
// edge length's term, drho[l][c] d rho[l][c] / d r with drho = sum_m y[m]
// dyhat[m] and dyhat = D^l (alpha G_i), into svl.
template <int L, int l, typename T>
__device__ __forceinline__ void force_degree(const ForceParams& p, const T* __restrict__ feat,
                                             const T* __restrict__ w_rad, int64_t b, int i, int j,
                                             const float (*D)[wig_size(L)], float (&T3)[3], float& svl,
                                             int lane) {
  constexpr int K = (L + 1) * (L + 1);
  constexpr int w = 2 * l + 1;
  const int C = p.C, H = p.H, dh = C / H;
  for (int c = lane; c < C; c += 64) {
    float rho = 0.0f, dro = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const float wr = load_as_f32(w_rad, (size_t)(kk * (L + 1) + l) * C + c);
      rho += p.rbf[b * 8 + kk] * wr;
      dro += p.rbfd[b * 8 + kk] * wr;
    }
    const float a = p.alpha[b * H + c / dh];
    float dx[w], yv[w], hv[w], ag[w];
#pragma unroll
    for (int q = 0; q < w; ++q) {
      const int64_t idx = batch_index(p.bl, L, C, b, l, q - l, c);
      dx[q] = static_cast<const float*>(p.dX)[idx];
      yv[q] = static_cast<const float*>(p.Y)[idx];
      hv[q] = load_as_f32(feat, (size_t)(((int64_t)j * K + l * l + q) * C + c));
      ag[q] = a * p.grad[((int64_t)i * K + l * l + q) * C + c];
    }
    // an offset the compiler cannot see through: the tangent entries do not
    // depend on the channel, and hoisted out of this loop all 3 (2l + 1)^2 of
    // them would be held in registers
    int z = 0;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const float* Dt = D[1 + t] + wig_off(l) + z;
      // yhat = rho y: rho applied once to the second sum
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int m = 0; m < w; ++m) {
        float u = 0.0f, v = 0.0f;
#pragma unroll
        for (int n = 0; n < w; ++n) {
          u += Dt[m * w + n] * hv[n];
          v += Dt[m * w + n] * ag[n];
        }
        s1 += dx[m] * u;
        s2 += yv[m] * v;
      }
      T3[t] += s1 + rho * s2;
    }
    {
      const float* D0 = D[0] + wig_off(l) + z;
      float dr = 0.0f;
#pragma unroll
      for (int m = 0; m < w; ++m) {
        float g = 0.0f;
#pragma unroll
        for (int n = 0; n < w; ++n) g += D0[m * w + n] * ag[n];
        dr += yv[m] * g;
      }
      svl += dr * dro;
    }
  }
  if constexpr (l < L) force_degree<L, l + 1, T>(p, feat, w_rad, b, i, j, D, T3, svl, lane);
}

// Block l >= 2 of D (component 0) and of its three tangents dD/dw_a
// (components 1 .. 3), one row per lane (4 (2l + 1) <= 36 lanes), every wave
// of the workgroup reaching the barrier.  Component 0 takes the tangent rule
// with D in place of dD, which gives twice the row of D^l (halved exactly),
// so that the lanes of a wave run one path.
template <int L, int l>
__device__ __forceinline__ void force_wigner(float (*D)[wig_size(L)], bool live, int lane) {
  constexpr int w = 2 * l + 1;
  if (live && lane < 4 * w) {
    const int comp = lane / w, m = lane - comp * w - l;
    float o[w];
    wigner_tangent_row<l>(m, D[0], D[comp], o);
    const float h = comp == 0 ? 0.5f : 1.0f;
#pragma unroll
    for (int n = 0; n < w; ++n) D[comp][wig_off(l) + (m + l) * w + n] = o[n] * h;
  }
  __syncthreads();
  if constexpr (l < L) force_wigner<L, l + 1>(D, live, lane);
}

// Edge e's ends (i, j), its direction and length (fr = r_hat, |r|), and
// D^0, D^1 with the three tangents dD^1/dw_a (components 1 .. 3 of D).
template <int L>
__device__ __forceinline__ void force_edge_setup(const ForceParams& p, int64_t e, float (*D)[wig_size(L)], float* fr,
                                                 int* ij) {
  const int i = p.src[e], j = p.col[e];
  ij[0] = i;
  ij[1] = j;
  float r3[3];
  for (int d = 0; d < 3; ++d) {
    float dx = p.pos[3 * (int64_t)j + d] - p.pos[3 * (int64_t)i + d];
    if (p.periodic) {
      if (dx > 0.5f * p.box[d]) dx -= p.box[d];
      else if (dx < -0.5f * p.box[d]) dx += p.box[d];
    }
    r3[d] = dx;
  }
  float u[3];
  const float r = edge_unit(r3, u);
  fr[0] = u[0];
  fr[1] = u[1];
  fr[2] = u[2];
  fr[3] = r;
  float R[3][3];
  edge_rotation(u, R);
  D[0][0] = 1.0f;
  D[1][0] = D[2][0] = D[3][0] = 0.0f;
  if constexpr (L >= 1) {
    wigner_l1(R, &D[0][wig_off(1)], 3);
    for (int a = 0; a < 3; ++a) {
      float dR[3][3];
      frame_tangent(R, a, dR);
      wigner_l1(dR, &D[1 + a][wig_off(1)], 3);
    }
  }
}

// dL/dr of the edge from T_a and s (lane 0): (T x u) / |r| + s u; an edge
// of zero length has no direction to move along and contributes nothing.
__device__ __forceinline__ void force_write(const ForceParams& p, int64_t e, const float* u, const float (&T3)[3],
                                            float sv) {
  const bool has_len = u[3] > 0.0f;
  const float ir = has_len ? 1.0f / u[3] : 0.0f;
  const float s = has_len ? sv : 0.0f;
  p.gedge[e * 3 + 0] = (T3[1] * u[2] - T3[2] * u[1]) * ir + s * u[0];
  p.gedge[e * 3 + 1] = (T3[2] * u[0] - T3[0] * u[2]) * ir + s * u[1];
  p.gedge[e * 3 + 2] = (T3[0] * u[1] - T3[1] * u[0]) * ir + s * u[2];
}

// LDS written by some lanes of a wave and then read by others: the wave's
// LDS operations complete in order, so only the compiler has to be kept from
// moving them across this point.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// force_wigner for one wave's own edge, without workgroup barriers.
template <int L, int l>
__device__ __forceinline__ void force_wigner_wave(float (*D)[wig_size(L)], int lane) {
  constexpr int w = 2 * l + 1;
  if (lane < 4 * w) {
    const int comp = lane / w, m = lane - comp * w - l;
    float o[w];
    wigner_tangent_row<l>(m, D[0], D[comp], o);
    const float h = comp == 0 ? 0.5f : 1.0f;
#pragma unroll
    for (int n = 0; n < w; ++n) D[comp][wig_off(l) + (m + l) * w + n] = o[n] * h;
  }
  wave_sync();
  if constexpr (l < L) force_wigner_wave<L, l + 1>(D, lane);
}

// One edge per wave, four per workgroup.  Lane 0 sets up the frame, D^1 and
// its tangents; the degrees 2 .. L follow one row per lane; then the
// products, summed over the channels within the wave.
constexpr int kForceEdges = 4;
template <int L, typename T>
__global__ void __launch_bounds__(64 * kForceEdges) k_wg_force(ForceParams p, int64_t nb, const T* __restrict__ feat,
                                                               const T* __restrict__ w_rad) {
  constexpr int WS = wig_size(L);
  __shared__ float Ds[kForceEdges][4][WS];   // D and its three tangents dD/dw_a
  __shared__ float fr[kForceEdges][4];       // r_hat, |r|
  __shared__ int ijs[kForceEdges][2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t b = (int64_t)blockIdx.x * kForceEdges + wv;
  const bool live = b < nb;                  // every wave still takes part in the barriers
  const int64_t e = p.e0 + b;
  float (*D)[WS] = Ds[wv];
  if (lane == 0 && live) force_edge_setup<L>(p, e, D, fr[wv], ijs[wv]);
  __syncthreads();
  if constexpr (L >= 2) force_wigner<L, 2>(D, live, lane);
  if (!live) return;
  // T_a = <dL/dD, dD/dw_a>: each lane's share, then the wave's sum
  float T3[3] = {0.0f, 0.0f, 0.0f};
  float sv = 0.0f;   // the edge length's share
  force_degree<L, 0, T>(p, feat, w_rad, b, ijs[wv][0], ijs[wv][1], D, T3, sv, lane);
  for (int o = 32; o > 0; o >>= 1) sv += __shfl_xor(sv, o);
  for (int a = 0; a < 3; ++a)
    for (int o = 32; o > 0; o >>= 1) T3[a] += __shfl_xor(T3[a], o);
  if (lane == 0) force_write(p, e, fr[wv], T3, sv);
}

// The same T_a and s on the matrix cores (bf16 storage, C a multiple of 32),
// with the sums over channels taken first:
//   P^l[m][n] = sum_c dx[l,m][c] h_j[l,n][c] + rho[l][c] alpha[c] y[l,m][c] G_i[l,n][c],
//   M^l[m][n] = sum_c (d rho / d r)[l][c] alpha[c] y[l,m][c] G_i[l,n][c],
//   T_a = sum_l <P^l, dD^l/dw_a>,   s = sum_l <M^l, D^l>.
// All K x K row pairs of an edge form one product: rows (l, m) -> l^2 + l + m
// on both sides, v_mfma_f32_32x32x16_bf16 over 16 channels a step, each lane
// reading its own fragment (row lane % 32, channels 16 t + 8 (lane / 32) ..
// + 7) from global memory; only pairs within one degree are used.  The
// factors rho alpha and (d rho / d r) alpha of every (l, c) are formed per
// edge in LDS from the radial weights, which the workgroup stages once for
// its 32 edges.  y and dx arrive in bf16, and G_i as the bf16 copy (round
// to nearest even) the call's feature gradient made or run_wgrad makes;
// rho alpha y is rounded to bf16 for the products, whose sums are fp32.  Each wave works through its
// own edges with no workgroup barrier after the staging, so that the waves'
// latency-bound set-up and their loads overlap.
constexpr int kFmWaves = 4, kFmIters = 8;   // 32 edges per workgroup, one per wave at a time
constexpr int kFmBatch = 2;                 // channel steps whose loads are issued together
template <int L, int CT>
__global__ void __launch_bounds__(64 * kFmWaves, 2) k_wg_force_mfma(ForceParams p, int64_t nb,
                                                                 const uint16_t* __restrict__ feat,
                                                                 const uint16_t* __restrict__ w_rad) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  typedef float f32x8v __attribute__((ext_vector_type(8)));
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  constexpr int K = (L + 1) * (L + 1);
  constexpr int WS = wig_size(L);
  static_assert(K <= 32, "the rows (l, m) of an edge fit one 32-row tile");
  extern __shared__ __attribute__((aligned(16))) float fsm[];
  __shared__ float Ds[kFmWaves][4][WS];   // D and its three tangents, per wave
  __shared__ float frs[kFmWaves][4];
  __shared__ int ijs[kFmWaves][2];
  const int C = CT > 0 ? CT : p.C, H = p.H, dh = C / H;
  const int LC = (L + 1) * C;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float* wr = fsm;                         // [8][L + 1][C] radial weights
  float* tab = fsm + 8 * LC + wv * 2 * LC; // [2][L + 1][C]: rho alpha, (d rho / d r) alpha
  for (int t = tid; t < 8 * LC; t += blockDim.x) wr[t] = bf16_to_f32(w_rad[t]);
  __syncthreads();
  float (*D)[WS] = Ds[wv];
  // The lane's operand row (l, m) and its degree.  Rows K .. 31 of A and
  // columns K .. 31 of B only reach output rows and columns that are never
  // read, so their lanes load row K - 1 instead (valid memory, and no branch
  // around the loads).
  const int row = lane & 31, hk = lane >> 5;
  const int rowc = row < K ? row : K - 1;
  int lr = 0;
  while ((lr + 1) * (lr + 1) <= rowc) ++lr;
  const int mr = rowc - lr * lr - lr;
  const uint16_t* dXb = static_cast<const uint16_t*>(p.dX);
  const uint16_t* Yb = static_cast<const uint16_t*>(p.Y);
  for (int it = 0; it < kFmIters; ++it) {
    const int64_t b = ((int64_t)blockIdx.x * kFmIters + it) * kFmWaves + wv;
    if (b >= nb) break;
    const int64_t e = p.e0 + b;
    wave_sync();   // the previous edge's reads of D and the tables are done
    if (lane == 0) force_edge_setup<L>(p, e, D, frs[wv], ijs[wv]);
    wave_sync();
    if constexpr (L >= 2) force_wigner_wave<L, 2>(D, lane);
    {
      float rb[8], rd[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        rb[k] = p.rbf[b * 8 + k];
        rd[k] = p.rbfd[b * 8 + k];
      }
      for (int t = lane; t < LC; t += 64) {
        float r = 0.0f, d = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          r += rb[k] * wr[k * LC + t];
          d += rd[k] * wr[k * LC + t];
        }
        const float a = p.alpha[b * H + (t % C) / dh];
        tab[t] = r * a;
        tab[LC + t] = d * a;
      }
    }
    wave_sync();
    const int i = ijs[wv][0], j = ijs[wv][1];
    const int64_t bi = batch_index(p.bl, L, C, b, lr, mr, 0);
    const uint16_t* dxr = dXb + bi;
    const uint16_t* yr = Yb + bi;
    const uint16_t* hr = feat + ((int64_t)j * K + rowc) * C;
    const uint16_t* gr = p.gbf + ((int64_t)i * K + rowc) * C;
    const float* ra = tab + lr * C;
    f32x16 accT = {}, accS = {};
    // One step: 16 channels from c0 = 16 t + 8 (lane / 32) of the loaded rows.
    auto step = [&](int c0, const bf16x8& adx, const bf16x8& bh, const u32x4v& yw, const bf16x8& bg) {
      const f32x4v r0 = *reinterpret_cast<const f32x4v*>(ra + c0);
      const f32x4v r1 = *reinterpret_cast<const f32x4v*>(ra + c0 + 4);
      const f32x4v d0 = *reinterpret_cast<const f32x4v*>(ra + LC + c0);
      const f32x4v d1 = *reinterpret_cast<const f32x4v*>(ra + LC + c0 + 4);
      f32x8v yv, rv8, dv8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yv[2 * q] = __uint_as_float(yw[q] << 16);
        yv[2 * q + 1] = __uint_as_float(yw[q] & 0xffff0000u);
        rv8[q] = r0[q];
        rv8[4 + q] = r1[q];
        dv8[q] = d0[q];
        dv8[4 + q] = d1[q];
      }
      const bf16x8 a1 = __builtin_convertvector(yv * rv8, bf16x8);
      const bf16x8 a2 = __builtin_convertvector(yv * dv8, bf16x8);
      accT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(adx, bh, accT, 0, 0, 0);
      accT = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bg, accT, 0, 0, 0);
      accS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, bg, accS, 0, 0, 0);
    };
    if constexpr (CT > 0) {
      // C known at compile time: the steps' loads are issued kFmBatch at a
      // time ahead of their products, a few round trips per edge instead of
      // one per step
      constexpr int NS = CT / 16, NB = kFmBatch < NS ? kFmBatch : NS;
      static_assert(NS % NB == 0, "whole batches of steps");
#pragma unroll
      for (int t0 = 0; t0 < NS; t0 += NB) {
        bf16x8 ldx[NB], lh[NB];
        u32x4v ly[NB];
        bf16x8 lg[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const int c0 = 16 * (t0 + t) + 8 * hk;
          ldx[t] = *reinterpret_cast<const bf16x8*>(dxr + c0);
          lh[t] = *reinterpret_cast<const bf16x8*>(hr + c0);
          ly[t] = *reinterpret_cast<const u32x4v*>(yr + c0);
          lg[t] = *reinterpret_cast<const bf16x8*>(gr + c0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NB; ++t) step(16 * (t0 + t) + 8 * hk, ldx[t], lh[t], ly[t], lg[t]);
      }
    } else {
      for (int c0 = 8 * hk; c0 < C; c0 += 16)
        step(c0, *reinterpret_cast<const bf16x8*>(dxr + c0), *reinterpret_cast<const bf16x8*>(hr + c0),
             *reinterpret_cast<const u32x4v*>(yr + c0), *reinterpret_cast<const bf16x8*>(gr + c0));
    }
    // register r holds (row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32)
    float T3[3] = {0.0f, 0.0f, 0.0f};
    float sv = 0.0f;
    if (row < K) {
      const int lc = lr, wn = 2 * lc + 1, n = row - lc * lc;   // the column's degree (column index = row)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ir = 8 * (r >> 2) + 4 * hk + (r & 3);
        if (ir >= lc * lc && ir < (lc + 1) * (lc + 1)) {
          const int off = wig_off(lc) + (ir - lc * lc) * wn + n;
          T3[0] += accT[r] * D[1][off];
          T3[1] += accT[r] * D[2][off];
          T3[2] += accT[r] * D[3][off];
          sv += accS[r] * D[0][off];
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) sv += __shfl_xor(sv, o);
    for (int a = 0; a < 3; ++a)
      for (int o = 32; o > 0; o >>= 1) T3[a] += __shfl_xor(T3[a], o);
    if (lane == 0) force_write(p, e, frs[wv], T3, sv);
  }
}

size_t force_mfma_smem(int L, int C) { return sizeof(float) * (size_t)(8 + 2 * kFmWaves) * (L + 1) * C; }
// Dynamic and static LDS within the 64 KB a launch gets without a raised limit.
bool force_mfma_fits(int L, int C) {
  return force_mfma_smem(L, C) + sizeof(float) * kFmWaves * 4 * (size_t)wig_size(L) + 256 <= 65536;
}

// dL/dx_a = sum over edges (i, a) of dL/dr minus sum over edges (a, j): the
// edges (i, a) are found in the ascending rows of a's neighbours (the graph
// is symmetric), one atom per thread, in a fixed order.
__global__ void k_pos_assemble(const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col, int64_t n,
                               const float* __restrict__ gedge, float* __restrict__ grad_pos) {
  const int64_t a = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (a >= n) return;
  float g[3] = {0.0f, 0.0f, 0.0f};
  for (int64_t e = row_ptr[a]; e < row_ptr[a + 1]; ++e) {
    const int i = col[e];
    int64_t lo = row_ptr[i], hi = row_ptr[i + 1];
    const int64_t end = hi;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (col[mid] < a) lo = mid + 1;
      else hi = mid;
    }
    for (int d = 0; d < 3; ++d) {
      g[d] -= gedge[e * 3 + d];
      if (lo < end && col[lo] == a) g[d] += gedge[lo * 3 + d];
    }
  }
  for (int d = 0; d < 3; ++d) grad_pos[a * 3 + d] = g[d];
}

// The softmax gradient of the batch's edges from the batch tensors, for a
// call that asks for dL/dh and the positions but no weights (so no query
// pass runs).  With y = SO2(x) and dy = rho D (alpha G_i) in the batch
// layout, the sum of y dy over every (l, m) and the head's channels is
// alpha_h dL/dalpha_h (the rotate-out puts D^T (rho y) where G_i meets it), so
//   ds_h = sum y dy - alpha_h delta_{i,h},
// the quantity the query pass forms from its own products (softmax backward,
// technical summary section 2.2).  C = 128, H = 8, bf16 y and dy.  One wave
// per edge: the edge's 2L + 1 rows (m = 0, then +m and -m for m = 1 .. L)
// are read as 16-byte vectors, lane l taking vectors l, l + 64, ... of their
// concatenation; every row holds a whole multiple of 16 vectors (128
// channels), so vector v carries channels of head (v mod 16) / 2 and a
// lane's head is (l mod 16) / 2 throughout.  The eight lanes of a head are
// then summed (exchanges across bits 0, 4 and 5 of the lane index).
constexpr int kDsEdges = 4;   // edges (waves) per workgroup
template <int L>
__global__ void __launch_bounds__(64 * kDsEdges) k_wg_ds(BatchLayout bl, int64_t nb, int64_t e0,
                                                         const int32_t* __restrict__ src,
                                                         const uint16_t* __restrict__ Y,
                                                         const uint16_t* __restrict__ DY,
                                                         const float* __restrict__ alpha,
                                                         const float* __restrict__ delta, float* __restrict__ ds) {
  constexpr int C = 128, H = 8;
  constexpr int NV = (L + 1) * (L + 1) * C / 8;   // vectors of one edge
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kDsEdges + (threadIdx.x >> 6);
  if (b >= nb) return;
  float acc = 0.0f;
  for (int v = lane; v < NV; v += 64) {
    // row r of the edge (r = 0: m = 0; r = 2m - 1, 2m: +m, -m) and the
    // vector's place in it
    int m = 0, neg = 0, w = v;
    while (w >= (L + 1 - m) * (C / 8)) {
      w -= (L + 1 - m) * (C / 8);
      if (m == 0 || neg) { ++m; neg = 0; }
      else neg = 1;
    }
    const int64_t km = (int64_t)(L + 1 - m) * C;
    const int64_t at = bl.moff[m] + (neg ? bl.B * km : 0) + b * km + 8 * (int64_t)w;
    const uint4 yv = *reinterpret_cast<const uint4*>(Y + at);
    const uint4 dv = *reinterpret_cast<const uint4*>(DY + at);
    const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w}, dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += __uint_as_float(yw[q] << 16) * __uint_as_float(dw[q] << 16);
      acc += __uint_as_float(yw[q] & 0xffff0000u) * __uint_as_float(dw[q] & 0xffff0000u);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16 && (lane & 1) == 0) {
    const int h = lane >> 1;
    const int64_t e = e0 + b;
    const float a = alpha[b * H + h];
    ds[e * H + h] = acc - a * delta[(int64_t)src[e] * H + h];
  }
}

// ---------------------------------------------------------------- GEMMs ----
// C[m * ldc + n] += alpha * sum_k A(m, k) B(k, n), A(m, k) = A[m sam + k sak],
// B(k, n) = B[k sbk + n sbn].  With A2 set the k range is two segments: k <
// K1 reads A and B, k >= K1 reads A2 and B2 (same strides) at k - K1, the
// second product negated when neg2 is set, so that a sum of two products
// is one launch and one write.  One workgroup per output tile and k-range;
// with several k-ranges each writes alpha times its partial tile (or adds it
// to what its slot holds, so that several products and several edge batches
// can share one set of partials) and a second kernel adds the partials in
// order.
struct Gemm {
  const void* A;
  int64_t sam, sak;
  const void* B;
  int64_t sbk, sbn;
  int64_t M, N, K;
  float alpha;
  float* C;
  int64_t ldc;
  uint16_t* Cb;    // if set: the output is written here as bf16 (C = alpha AB, C unused)
  float* part;     // [S][M][N] when S > 1
  const void* A2;  // if set: second segment (the matrix-core kernel only)
  const void* B2;
  int64_t K1;      // first segment's length, a multiple of 32
  bool neg2;
  int S;
  int64_t kper;    // k per split, a multiple of 32
  bool overwrite;  // C = alpha AB instead of C += alpha AB
  bool part_acc;   // S > 1: add alpha AB to the partials instead of storing it
  bool vec_out;    // Cb, S = 1: N and ldc multiples of 8, Cb 16-byte aligned (set by the launcher)
};

// bf16 x bf16 on the matrix cores: a 128 x 128 output tile per workgroup,
// four waves of 64 x 64 (2 x 2 tiles of v_mfma_f32_32x32x16_bf16), 32-deep k
// slices double-buffered in LDS with k contiguous (the layout the fragments
// read).  An operand whose contiguous dimension is k is copied in 16-byte
// vectors; one contiguous along m (or n) is read in 16-byte vectors along m
// and transposed on its way into LDS; anything else (or a ragged edge) goes
// element by element.
constexpr int kTM = 128, kBK = 32, kPad = 8;
struct GemmSmem {
  uint16_t a[2][kTM][kBK + kPad];
  uint16_t b[2][kTM][kBK + kPad];
};

// bf16 output tile through LDS: the accumulators (register r of tile (i, j):
// row 64 wm + 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4, column 64 wn + 32 j +
// lane % 32) go to a [128][136] bf16 tile, then 16 threads store each row's
// 256 bytes, 16 bytes a lane.  The caller has synchronised the workgroup
// after its last read of `tile`'s memory; out rows are ldc apart.
__device__ __forceinline__ void store_tile_bf16(const f32x16 (&acc)[2][2], float alpha, uint16_t* tile,
                                                uint16_t* out, int64_t ldc, int64_t m0, int64_t n0, int64_t M,
                                                int64_t N, int tid) {
  constexpr int ldo = kTM + 8;
  const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tile[(wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * ldo + wn * 64 + j * 32 + (lane & 31)] =
            f32_to_bf16_rne(alpha * acc[i][j][r]);
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kTM * kTM / 8 / 256; ++p) {
    const int idx = tid + 256 * p;
    const int rr = idx >> 4, c8 = (idx & 15) * 8;
    if (m0 + rr < M && n0 + c8 < N)
      *reinterpret_cast<uint4*>(out + (m0 + rr) * ldc + n0 + c8) = *reinterpret_cast<const uint4*>(tile + rr * ldo + c8);
  }
}

// One 128 x 32 slice of an operand X(r, k) = X[r sr + k sk] (rows r0 ..
// r0+127 of m or n, k0 .. k0+31), fetched into registers first and written
// to LDS ([r - r0][k - k0]) after the current slice's products, so that the
// global loads' latency overlaps them.  vk / vr: 16-byte vectors along k or
// along r are allowed; otherwise (and on ragged edges) element by element.
// EXACT: the caller guarantees that k ranges and the extent along the vector
// are multiples of 8, so a ragged tile edge is a whole vector past the end and
// reads as zeros, with no element-by-element path.
struct Slice {
  uint32_t v[2][4];
};

template <bool EXACT>
__device__ __forceinline__ void fetch_slice(const uint16_t* __restrict__ X, int64_t sr, int64_t sk, int64_t r0,
                                            int64_t R, int64_t k0, int64_t ke, bool vk, bool vr, int tid,
                                            Slice& f) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int idx = tid + 256 * v;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (vk || !vr) {
      // rows idx / 4, k offset 8 (idx % 4)
      const int r = idx >> 2, kq = (idx & 3) * 8;
      const int64_t m = r0 + r, k = k0 + kq;
      if (EXACT) {
        // k and ke are multiples of 8: k < ke means the whole vector is in range
        if (m < R && k < ke) w = *reinterpret_cast<const u32x4*>(X + m * sr + k);
      } else if (vk && m < R && k + 8 <= ke) {
        w = *reinterpret_cast<const u32x4*>(X + m * sr + k);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t e = (m < R && k + q < ke) ? X[m * sr + (k + q) * sk] : 0u;
          w[q >> 1] |= e << (16 * (q & 1));
        }
      }
    } else {
      // rows 8 (tid / 16) .. +7 at k = 2 (tid % 16) + v: each thread holds a
      // pair of neighbouring k for 8 rows, written to LDS as 32-bit words
      const int kq = 2 * (tid & 15) + v, rq = (tid >> 4) * 8;
      const int64_t m = r0 + rq, k = k0 + kq;
      if (EXACT) {
        // m and R are multiples of 8: m < R means rows m .. m + 7 are in range
        if (k < ke && m < R) w = *reinterpret_cast<const u32x4*>(X + m + k * sk);
      } else if (k < ke && m + 8 <= R) {
        w = *reinterpret_cast<const u32x4*>(X + m + k * sk);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t e = (k < ke && m + q < R) ? X[(m + q) + k * sk] : 0u;
          w[q >> 1] |= e << (16 * (q & 1));
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) f.v[v][q] = w[q];
  }
}

__device__ __forceinline__ void commit_slice(const Slice& f, bool vr_layout, uint16_t (*dst)[kBK + kPad], int tid) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int idx = tid + 256 * v;
    if (!vr_layout) {
      const int r = idx >> 2, kq = (idx & 3) * 8;
      *reinterpret_cast<u32x4*>(&dst[r][kq]) = u32x4{f.v[v][0], f.v[v][1], f.v[v][2], f.v[v][3]};
    } else if (v == 1) {
      // v = 0 and 1 hold k = 2 (tid % 16) and that + 1 for rows 8 (tid / 16) ..
      const int kp = tid & 15, rq = (tid >> 4) * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t lo = (f.v[0][q >> 1] >> (16 * (q & 1))) & 0xffffu;
        const uint32_t hi = (f.v[1][q >> 1] >> (16 * (q & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(&dst[rq + q][2 * kp]) = lo | (hi << 16);
      }
    }
  }
}

__host__ __device__ __forceinline__ bool aligned16(const void* p, int64_t stride) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0 && stride % 8 == 0;
}

// Operand layouts: 16-byte vectors along k, along m (or n), or element by
// element.  kAny: decided per launch from the strides and alignments.
constexpr int kVecK = 1, kVecR = 2, kElem = 0, kAny = -1;

__host__ __device__ __forceinline__ int operand_layout(const void* X, const void* X2, int64_t sr, int64_t sk) {
  if (sk == 1 && aligned16(X, sr) && (!X2 || aligned16(X2, sr))) return kVecK;
  if (sr == 1 && aligned16(X, sk) && (!X2 || aligned16(X2, sk))) return kVecR;
  return kElem;
}

template <int AV, int BV, bool EXACT>
__device__ __forceinline__ void gemm_body(const Gemm& g, GemmSmem& sm) {
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B);
  const uint16_t* A2 = static_cast<const uint16_t*>(g.A2);
  const uint16_t* B2 = static_cast<const uint16_t*>(g.B2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // Workgroups are dealt to the 8 XCDs in turn (id mod 8).  Work item w runs
  // on XCD w / (share), so that each XCD takes a contiguous run of items (n
  // tile fastest, then m tile, then k range): the tiles that read the same
  // rows of an operand run side by side under one L2.
  const uint32_t nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
  const uint32_t id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const uint32_t q = total / 8, r = total % 8, xcd = id % 8, local = id / 8;
  const uint32_t wi = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  const uint32_t bx = wi % nx, by = (wi / nx) % ny, bz = wi / (nx * ny);
  const int64_t m0 = (int64_t)by * kTM, n0 = (int64_t)bx * kTM;
  const int64_t kb = (int64_t)bz * g.kper;
  const int64_t ke = kb + g.kper < g.K ? kb + g.kper : g.K;
  const int64_t k1 = A2 ? g.K1 : g.K;   // end of the first segment
  // A(m, k) = A[m sam + k sak]; B(k, n) = B[n sbn + k sbk]
  const int av = AV == kAny ? operand_layout(A, A2, g.sam, g.sak) : AV;
  const int bv = BV == kAny ? operand_layout(B, B2, g.sbn, g.sbk) : BV;
  const bool avk = av == kVecK, avr = av == kVecR, bvk = bv == kVecK, bvr = bv == kVecR;
  // the slice at k0 (a multiple of 32 from kb, never across K1)
  auto fetch = [&](int64_t k0, Slice& fa, Slice& fb) {
    if (k0 < k1) {
      const int64_t e1 = ke < k1 ? ke : k1;
      fetch_slice<EXACT>(A, g.sam, g.sak, m0, g.M, k0, e1, avk, avr, tid, fa);
      fetch_slice<EXACT>(B, g.sbn, g.sbk, n0, g.N, k0, e1, bvk, bvr, tid, fb);
    } else {
      fetch_slice<EXACT>(A2, g.sam, g.sak, m0, g.M, k0 - k1, ke - k1, avk, avr, tid, fa);
      fetch_slice<EXACT>(B2, g.sbn, g.sbk, n0, g.N, k0 - k1, ke - k1, bvk, bvr, tid, fb);
      if (g.neg2)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) fb.v[v][q] ^= 0x80008000u;   // bf16 sign bits
    }
  };
  f32x16 acc[2][2] = {};
  Slice fa, fb;
  int buf = 0;
  if (kb < ke) {
    fetch(kb, fa, fb);
    commit_slice(fa, avr, sm.a[0], tid);
    commit_slice(fb, bvr, sm.b[0], tid);
  }
  __syncthreads();
  for (int64_t k0 = kb; k0 < ke; k0 += kBK) {
    const bool more = k0 + kBK < ke;
    if (more) fetch(k0 + kBK, fa, fb);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const bf16x8*>(&sm.a[buf][wm * 64 + t * 32 + (lane & 31)][ks + 8 * (lane >> 5)]);
        bfr[t] = *reinterpret_cast<const bf16x8*>(&sm.b[buf][wn * 64 + t * 32 + (lane & 31)][ks + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      commit_slice(fa, avr, sm.a[buf ^ 1], tid);
      commit_slice(fb, bvr, sm.b[buf ^ 1], tid);
    }
    __syncthreads();
    buf ^= 1;
  }
  if (g.vec_out) {
    // the loop ended with a barrier: the slices' LDS is free
    store_tile_bf16(acc, g.alpha, reinterpret_cast<uint16_t*>(&sm), g.Cb, g.ldc, m0, n0, g.M, g.N, tid);
    return;
  }
  // register r: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m < g.M && n < g.N) {
          const float v = acc[i][j][r];
          if (g.S > 1) {
            float* pp = g.part + ((int64_t)bz * g.M + m) * g.N + n;
            *pp = g.part_acc ? *pp + g.alpha * v : g.alpha * v;
          } else if (g.Cb) {
            g.Cb[m * g.ldc + n] = f32_to_bf16_rne(g.alpha * v);
          } else if (g.overwrite) {
            g.C[m * g.ldc + n] = g.alpha * v;
          } else {
            g.C[m * g.ldc + n] += g.alpha * v;
          }
        }
      }
}

// The weight products Xᵀ dY with both operands contiguous along m (and n):
// each 32-deep k slice is copied to LDS as it lies in memory, [k][m], every
// k row's 128 values (256 bytes) read by 16 neighbouring lanes, and the
// MFMA fragments (8 consecutive k of one row) come from gfx950's LDS
// transpose reads.  ds_read_b64_tr_b16 gives lane i of each 16-lane group,
// in slot q, element i % 4 of the 4 elements at lane 4 q + i / 4's address,
// so a lane 16 g + s of the wave (q = s / 4, p = s % 4) that points at row
// k0 + q, column c0 + 16 (g % 2) + 4 p receives T[k0 + q'][c0 + 16 (g % 2) + i]
// for q' = 0..3: four consecutive k of its own fragment row; k0 = 8 (g / 2)
// and + 4 for the second read.
constexpr int kTrPad = 16;   // row stride 144 values (288 bytes)
struct GemmSmemTr {
  uint16_t a[2][kBK][kTM + kTrPad];
  uint16_t b[2][kBK][kTM + kTrPad];
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t (*T)[kTM + kTrPad], int k0, int c0, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (sl >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (sl & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&T[row][col]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&T[row + 4][col]));
  const i16x4 v[2] = {lo, hi};
  bf16x8 r;
  __builtin_memcpy(&r, v, 16);
  return r;
}

__device__ __forceinline__ void gemm_body_tr(const Gemm& g, GemmSmemTr& sm) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B);
  const uint16_t* A2 = static_cast<const uint16_t*>(g.A2);
  const uint16_t* B2 = static_cast<const uint16_t*>(g.B2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
  const uint32_t id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const uint32_t q8 = total / 8, r8 = total % 8, xcd = id % 8, local = id / 8;
  const uint32_t wi = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + local;
  const uint32_t bx = wi % nx, by = (wi / nx) % ny, bz = wi / (nx * ny);
  const int64_t m0 = (int64_t)by * kTM, n0 = (int64_t)bx * kTM;
  const int64_t kb = (int64_t)bz * g.kper;
  const int64_t ke = kb + g.kper < g.K ? kb + g.kper : g.K;
  const int64_t k1 = A2 ? g.K1 : g.K;
  // thread t copies k rows t / 16 and t / 16 + 16 of the slice, columns
  // 8 (t % 16) .. + 7 (A(m, k) = A[m + k sak], B(k, n) = B[n + k sbk])
  const int kr = tid >> 4, cq = (tid & 15) * 8;
  auto fetch = [&](int64_t k0, u32x4 (&fa)[2], u32x4 (&fb)[2]) {
    const bool seg2 = k0 >= k1;
    const uint16_t* X = seg2 ? A2 : A;
    const uint16_t* Y = seg2 ? B2 : B;
    const int64_t kk0 = seg2 ? k0 - k1 : k0, kend = seg2 ? ke - k1 : (ke < k1 ? ke : k1);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int64_t k = kk0 + kr + 16 * v;
      const bool kin = k < kend;
      fa[v] = (kin && m0 + cq < g.M) ? *reinterpret_cast<const u32x4*>(X + m0 + cq + k * g.sak) : u32x4{0, 0, 0, 0};
      fb[v] = (kin && n0 + cq < g.N) ? *reinterpret_cast<const u32x4*>(Y + n0 + cq + k * g.sbk) : u32x4{0, 0, 0, 0};
      if (seg2 && g.neg2) fb[v] ^= 0x80008000u;   // bf16 sign bits
    }
  };
  auto commit = [&](const u32x4 (&fa)[2], const u32x4 (&fb)[2], int bsel) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      *reinterpret_cast<u32x4*>(&sm.a[bsel][kr + 16 * v][cq]) = fa[v];
      *reinterpret_cast<u32x4*>(&sm.b[bsel][kr + 16 * v][cq]) = fb[v];
    }
  };
  f32x16 acc[2][2] = {};
  u32x4 fa[2], fb[2];
  int buf = 0;
  if (kb < ke) {
    fetch(kb, fa, fb);
    commit(fa, fb, 0);
  }
  __syncthreads();
  for (int64_t k0 = kb; k0 < ke; k0 += kBK) {
    const bool more = k0 + kBK < ke;
    if (more) fetch(k0 + kBK, fa, fb);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = tr_frag(sm.a[buf], ks, wm * 64 + t * 32, lane);
        bfr[t] = tr_frag(sm.b[buf], ks, wn * 64 + t * 32, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) commit(fa, fb, buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // register r: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m < g.M && n < g.N) {
          const float v = acc[i][j][r];
          if (g.S > 1) {
            float* pp = g.part + ((int64_t)bz * g.M + m) * g.N + n;
            *pp = g.part_acc ? *pp + g.alpha * v : g.alpha * v;
          } else if (g.overwrite) {
            g.C[m * g.ldc + n] = g.alpha * v;
          } else {
            g.C[m * g.ldc + n] += g.alpha * v;
          }
        }
      }
}

__global__ void __launch_bounds__(256, 4) k_gemm_mfma_tr(Gemm g) {
  __shared__ __attribute__((aligned(16))) GemmSmemTr sm;
  gemm_body_tr(g, sm);
}

// Complex pairs of products: with operands A1, A2 and B1, B2,
//   P = aP (A1 B1 + s1 A2 B2),   Q = aQ (A1 B2 + s2 A2 B1)   (s1, s2 = +-1),
// the shape of every m > 0 block of the SO(2) mix and of its gradients
// (y+ = x+ W1 - x- W2, y- = x+ W2 + x- W1; dx+ = dy+ W1^T + dy- W2^T,
// dx- = -(dy+ W2^T - dy- W1^T); dW1 += x+^T dy+ + x-^T dy-,
// dW2 += x+^T dy- - x-^T dy+), from one read of the four operands' slices
// instead of two launches that each read all four.  KK: A(m, k) =
// A[m sa + k], B(k, n) = B[n sb + k] (the edge-row products, bf16 outputs,
// one k range); TR: A(m, k) = A[m + k sa], B(k, n) = B[n + k sb] (the weight
// products, fragments by LDS transpose reads, split-k partials).  Twice the
// accumulators of the single products: two workgroups per CU.
struct GemmCx {
  const uint16_t* A1;
  const uint16_t* A2;
  const uint16_t* B1;
  const uint16_t* B2;
  int64_t sa, sb;
  int64_t M, N, K;
  float aP, aQ;
  bool s1neg, s2neg;
  uint16_t* P_bf;      // KK outputs, row stride ldc
  uint16_t* Q_bf;
  int64_t ldc;
  float* P_part;       // TR: [S][M][N] partials of P and Q
  float* Q_part;
  bool part_acc;
  int64_t kper;
  bool vec_out;        // KK: N and ldc multiples of 8, P_bf and Q_bf 16-byte aligned (set by the launcher)
};

constexpr size_t kCxSmemKK = 4 * 2 * (size_t)kTM * (kBK + kPad) * sizeof(uint16_t);
constexpr size_t kCxSmemTR = 4 * 2 * (size_t)kBK * (kTM + kTrPad) * sizeof(uint16_t);

template <bool TR>
__device__ __forceinline__ void gemm_body_cx(const GemmCx& g, uint16_t* smem) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
  const uint32_t id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const uint32_t q8 = total / 8, r8 = total % 8, xcd = id % 8, local = id / 8;
  const uint32_t wi = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + local;
  const uint32_t bx = wi % nx, by = (wi / nx) % ny, bz = wi / (nx * ny);
  const int64_t m0 = (int64_t)by * kTM, n0 = (int64_t)bx * kTM;
  const int64_t kb = (int64_t)bz * g.kper;
  const int64_t ke = kb + g.kper < g.K ? kb + g.kper : g.K;
  // slice buffers: operand o (A1, A2, B1, B2), buffer b
  constexpr int RS = TR ? kTM + kTrPad : kBK + kPad;       // row length
  constexpr int SL = TR ? kBK * RS : kTM * RS;             // values per slice buffer
  auto slice = [&](int o, int b) { return smem + (size_t)(2 * o + b) * SL; };
  const uint16_t* ops[4] = {g.A1, g.A2, g.B1, g.B2};
  u32x4 f[4][2];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const int64_t r0 = o < 2 ? m0 : n0, R = o < 2 ? g.M : g.N, st = o < 2 ? g.sa : g.sb;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if constexpr (TR) {
          const int64_t k = k0 + (tid >> 4) + 16 * v, c = r0 + (tid & 15) * 8;
          if (k < ke && c < R) w = *reinterpret_cast<const u32x4*>(ops[o] + c + k * st);
        } else {
          const int idx = tid + 256 * v;
          const int64_t r = r0 + (idx >> 2), k = k0 + (idx & 3) * 8;
          if (r < R && k < ke) w = *reinterpret_cast<const u32x4*>(ops[o] + r * st + k);
        }
        f[o][v] = w;
      }
    }
  };
  auto commit = [&](int b) {
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      uint16_t* d = slice(o, b);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        if constexpr (TR) {
          *reinterpret_cast<u32x4*>(d + ((tid >> 4) + 16 * v) * RS + (tid & 15) * 8) = f[o][v];
        } else {
          const int idx = tid + 256 * v;
          *reinterpret_cast<u32x4*>(d + (idx >> 2) * RS + (idx & 3) * 8) = f[o][v];
        }
      }
    }
  };
  auto frag = [&](int o, int b, int ks, int c0) -> bf16x8 {
    const uint16_t* d = slice(o, b);
    if constexpr (TR) {
      return tr_frag(reinterpret_cast<const uint16_t(*)[kTM + kTrPad]>(d), ks, c0, lane);
    } else {
      return *reinterpret_cast<const bf16x8*>(d + (c0 + (lane & 31)) * RS + ks + 8 * (lane >> 5));
    }
  };
  auto neg = [](bf16x8 x) {
    u32x4 u = __builtin_bit_cast(u32x4, x);
    u ^= 0x80008000u;
    return __builtin_bit_cast(bf16x8, u);
  };
  f32x16 accP[2][2] = {}, accQ[2][2] = {};
  int buf = 0;
  if (kb < ke) {
    fetch(kb);
    commit(0);
  }
  __syncthreads();
  for (int64_t k0 = kb; k0 < ke; k0 += kBK) {
    const bool more = k0 + kBK < ke;
    if (more) fetch(k0 + kBK);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 a1[2], a2[2], b1[2], b2[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a1[t] = frag(0, buf, ks, wm * 64 + t * 32);
        a2[t] = frag(1, buf, ks, wm * 64 + t * 32);
        b1[t] = frag(2, buf, ks, wn * 64 + t * 32);
        b2[t] = frag(3, buf, ks, wn * 64 + t * 32);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 b2s = g.s1neg ? neg(b2[j]) : b2[j];
        const bf16x8 b1s = g.s2neg ? neg(b1[j]) : b1[j];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          accP[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], accP[i][j], 0, 0, 0);
          accP[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[i], b2s, accP[i][j], 0, 0, 0);
          accQ[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b2[j], accQ[i][j], 0, 0, 0);
          accQ[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2[i], b1s, accQ[i][j], 0, 0, 0);
        }
      }
    }
    if (more) commit(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  if constexpr (!TR) {
    if (g.vec_out) {
      // the loop ended with a barrier: the slices' LDS is free; P's tile,
      // then Q's in the same place
      store_tile_bf16(accP, g.aP, smem, g.P_bf, g.ldc, m0, n0, g.M, g.N, tid);
      __syncthreads();
      store_tile_bf16(accQ, g.aQ, smem, g.Q_bf, g.ldc, m0, n0, g.M, g.N, tid);
      return;
    }
  }
  // register r: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m < g.M && n < g.N) {
          const float vp = g.aP * accP[i][j][r], vq = g.aQ * accQ[i][j][r];
          if constexpr (TR) {
            float* pp = g.P_part + ((int64_t)bz * g.M + m) * g.N + n;
            float* pq = g.Q_part + ((int64_t)bz * g.M + m) * g.N + n;
            *pp = g.part_acc ? *pp + vp : vp;
            *pq = g.part_acc ? *pq + vq : vq;
          } else {
            g.P_bf[m * g.ldc + n] = f32_to_bf16_rne(vp);
            g.Q_bf[m * g.ldc + n] = f32_to_bf16_rne(vq);
          }
        }
      }
}

template <bool TR>
__global__ void __launch_bounds__(256, 2) k_gemm_cx(GemmCx g) {
  extern __shared__ __attribute__((aligned(16))) uint16_t cx_smem[];
  gemm_body_cx<TR>(g, cx_smem);
}

// One complex pair over S k ranges (TR: partials; KK: S = 1).
template <bool TR>
e2a_status launch_gemm_cx(const GemmCx& g0, int S, hipStream_t st) {
  GemmCx g = g0;
  g.vec_out = !TR && g.N % 8 == 0 && g.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(g.P_bf) & 15) == 0 &&
              (reinterpret_cast<uintptr_t>(g.Q_bf) & 15) == 0;
  const dim3 grid(static_cast<unsigned>((g.N + kTM - 1) / kTM), static_cast<unsigned>((g.M + kTM - 1) / kTM),
                  static_cast<unsigned>(S));
  const size_t smem = TR ? kCxSmemTR : kCxSmemKK;
  E2A_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_cx<TR>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem)));
  k_gemm_cx<TR><<<grid, 256, smem, st>>>(g);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

// Any layouts, three workgroups per CU (168 VGPRs).
__global__ void __launch_bounds__(256, 3) k_gemm_mfma(Gemm g) {
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  gemm_body<kAny, kAny, false>(g, sm);
}

// Fixed layout with every extent a multiple of 8: without the per-launch
// choice and the element-by-element path the kernel fits 128 VGPRs, so four
// workgroups share a CU (the LDS holds exactly four) and a third more slices
// are in flight; the loop is bound by the slices' load latency.
// Both operands contiguous along k: the products of the edges' rows with the
// SO(2) blocks (y = SO2(x), dx = SO2ᵀ(dy)).
__global__ void __launch_bounds__(256, 4) k_gemm_mfma_kk(Gemm g) {
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  gemm_body<kVecK, kVecK, true>(g, sm);
}

// Any operand types, fp32 on the vector ALUs: 64 x 64 tiles, a 4 x 4 block of
// outputs per thread, 16-deep k slices in LDS.
template <typename TA, typename TB>
__global__ void __launch_bounds__(256) k_gemm_valu(Gemm g) {
  constexpr int BK = 16;
  __shared__ float As[BK][64];
  __shared__ float Bs[BK][64];
  const TA* A = static_cast<const TA*>(g.A);
  const TB* B = static_cast<const TB*>(g.B);
  const int tid = threadIdx.x;
  const int tm = tid >> 4, tn = tid & 15;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  const int64_t kb = (int64_t)blockIdx.z * g.kper;
  const int64_t ke = kb + g.kper < g.K ? kb + g.kper : g.K;
  float acc[4][4] = {};
  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;   // 0 .. 1023 over (k, row)
      // the contiguous dimension runs across neighbouring threads
      int kk, r;
      if (g.sak == 1) { kk = idx & 15; r = idx >> 4; } else { r = idx & 63; kk = idx >> 6; }
      const int64_t m = m0 + r, k = k0 + kk;
      As[kk][r] = (m < g.M && k < ke) ? load_as_f32(A, (size_t)(m * g.sam + k * g.sak)) : 0.0f;
      int kb2, c;
      if (g.sbk == 1) { kb2 = idx & 15; c = idx >> 4; } else { c = idx & 63; kb2 = idx >> 6; }
      const int64_t n = n0 + c, k2 = k0 + kb2;
      Bs[kb2][c] = (n < g.N && k2 < ke) ? load_as_f32(B, (size_t)(k2 * g.sbk + n * g.sbn)) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[kk][tm * 4 + u];
        b[u] = Bs[kk][tn * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * b[v];
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + tm * 4 + u, n = n0 + tn * 4 + v;
      if (m < g.M && n < g.N) {
        if (g.S > 1) {
          float* pp = g.part + ((int64_t)blockIdx.z * g.M + m) * g.N + n;
          *pp = g.part_acc ? *pp + g.alpha * acc[u][v] : g.alpha * acc[u][v];
        } else if (g.overwrite) g.C[m * g.ldc + n] = g.alpha * acc[u][v];
        else g.C[m * g.ldc + n] += g.alpha * acc[u][v];
      }
    }
}

__global__ void k_gemm_reduce(Gemm g) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= g.M * g.N) return;
  float s = 0.0f;
  for (int z = 0; z < g.S; ++z) s += g.part[z * g.M * g.N + t];
  const int64_t m = t / g.N, n = t - m * g.N;
  if (g.Cb) g.Cb[m * g.ldc + n] = f32_to_bf16_rne(s);
  else if (g.overwrite) g.C[m * g.ldc + n] = s;
  else g.C[m * g.ldc + n] += s;
}

constexpr int64_t kTargetGroups = 1024;   // workgroups a GEMM launch aims for

template <typename TA, typename TB>
constexpr int64_t tile_of() {
  return std::is_same<TA, uint16_t>::value && std::is_same<TB, uint16_t>::value ? kTM : 64;
}

// Launches the product kernel for g with g.S k-ranges of g.kper (set by the caller).
template <typename TA, typename TB>
e2a_status launch_gemm(const Gemm& g0, hipStream_t st) {
  constexpr int64_t tm = tile_of<TA, TB>();
  Gemm g = g0;
  g.vec_out = tm == kTM && g.Cb && g.S == 1 && g.N % 8 == 0 && g.ldc % 8 == 0 &&
              (reinterpret_cast<uintptr_t>(g.Cb) & 15) == 0;
  const dim3 grid(static_cast<unsigned>((g.N + tm - 1) / tm), static_cast<unsigned>((g.M + tm - 1) / tm),
                  static_cast<unsigned>(g.S));
  if constexpr (tm == kTM) {
    const int av = operand_layout(g.A, g.A2, g.sam, g.sak), bv = operand_layout(g.B, g.B2, g.sbn, g.sbk);
    // the fixed-layout instances read whole vectors only: k ranges (and the
    // second segment's start) and the vector extents must be multiples of 8
    const bool k8 = g.K % 8 == 0 && g.kper % 8 == 0 && (!g.A2 || g.K1 % 8 == 0);
    if (av == kVecR && bv == kVecR && k8 && g.M % 8 == 0 && g.N % 8 == 0)
      k_gemm_mfma_tr<<<grid, 256, 0, st>>>(g);
    else if (av == kVecK && bv == kVecK && k8)
      k_gemm_mfma_kk<<<grid, 256, 0, st>>>(g);
    else
      k_gemm_mfma<<<grid, 256, 0, st>>>(g);
  } else
    k_gemm_valu<TA, TB><<<grid, 256, 0, st>>>(g);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

e2a_status reduce_parts(const Gemm& g, hipStream_t st) {
  k_gemm_reduce<<<static_cast<unsigned>((g.M * g.N + 255) / 256), 256, 0, st>>>(g);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

// k-ranges for a product with `tiles` output tiles: about kTargetGroups
// workgroups, at least 256 k per range, at most `smax`.
int64_t pick_splits(int64_t tiles, int64_t K, int64_t smax) {
  int64_t S = (kTargetGroups + tiles - 1) / tiles;
  if (S > (K + 255) / 256) S = (K + 255) / 256;
  if (S > smax) S = smax;
  return S < 1 ? 1 : S;
}

// One product into C, its partials (if any) in part.
template <typename TA, typename TB>
e2a_status gemm(Gemm g, int64_t part_floats, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return E2A_OK;
  constexpr int64_t tm = tile_of<TA, TB>();
  const int64_t tiles = ((g.M + tm - 1) / tm) * ((g.N + tm - 1) / tm);
  const int64_t S = pick_splits(tiles, g.K, part_floats / (g.M * g.N));
  g.S = static_cast<int>(S);
  g.kper = ((g.K + S - 1) / S + 31) / 32 * 32;
  g.part_acc = false;
  e2a_status e = launch_gemm<TA, TB>(g, st);
  if (e != E2A_OK || S == 1) return e;
  return reduce_parts(g, st);
}

// The SO(2) weight gradients sum over every batch: each of the 2L + 1
// matrices keeps dw_splits(m) partials for the whole call, which every batch's
// products add to, and one reduction at the end.  The m = 0 products run on
// k_gemm_mfma_tr, four workgroups per CU (122 VGPRs a lane, 36 KB of LDS
// each), 1024 on the 256 CUs, and a launch with a few workgroups more than
// that takes a second round: the split count fills the 1024 slots without
// passing them (tiles x S <= 1024).  The m > 0 pairs (bf16) run on
// k_gemm_cx<true>, two workgroups per CU: dw_splits_pair fills 512 slots.
constexpr int64_t kGemmSlots = 1024;
int64_t dw_splits(int L, int C, int m) {
  const int64_t km = (int64_t)(L + 1 - m) * C;
  const int64_t t = (km + kTM - 1) / kTM;
  const int64_t S = kGemmSlots / (t * t);
  return S < 1 ? 1 : S;
}
// The complex-pair kernel (m > 0, bf16) runs two workgroups per CU: 512
// slots, and as many k ranges as fill them (at most dw_splits, which sizes
// the partial buffers).
int64_t dw_splits_pair(int L, int C, int m) {
  const int64_t km = (int64_t)(L + 1 - m) * C;
  const int64_t t = (km + kTM - 1) / kTM;
  const int64_t S = kGemmSlots / 2 / (t * t);
  return S < 1 ? 1 : S;
}

int64_t dw_part_floats(int L, int C) {
  int64_t f = 0;
  for (int m = 0; m <= L; ++m) {
    const int64_t km = (int64_t)(L + 1 - m) * C;
    f += (m == 0 ? 1 : 2) * dw_splits(L, C, m) * km * km;
  }
  return f;
}

Gemm make_gemm(const void* A, int64_t sam, int64_t sak, const void* B, int64_t sbk, int64_t sbn, int64_t M,
               int64_t N, int64_t K, float alpha, float* C, int64_t ldc, float* part, bool overwrite = false) {
  Gemm g{};
  g.overwrite = overwrite;
  g.A = A;
  g.sam = sam;
  g.sak = sak;
  g.B = B;
  g.sbk = sbk;
  g.sbn = sbn;
  g.M = M;
  g.N = N;
  g.K = K;
  g.alpha = alpha;
  g.C = C;
  g.ldc = ldc;
  g.part = part;
  return g;
}

struct WgWs {
  size_t src, X, GT, Y, rbf, part, dwpart, rhopart, wt;
  size_t rbfd, alpha, dX, gedge;   // position gradient only (dX also holds dyhat for the dW_rad batches)
  size_t gbf;                      // the cotangent in bf16 for the matrix-core force kernel
  size_t total;
  int64_t B, part_floats;
};

WgWs wg_ws_layout(int64_t n, int64_t e, int L, int C, int H) {
  WgWs w{};
  const int64_t B = e < kWgBatch ? (e > 0 ? e : 1) : kWgBatch;
  const int64_t per = B * (int64_t)(L + 1) * (L + 1) * C;   // elements of one batch tensor
  const int64_t K0 = (int64_t)(L + 1) * C;
  int64_t pf = 16 * K0 * K0;
  if (256 * (int64_t)C * C > pf) pf = 256 * (int64_t)C * C;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.src = take(sizeof(int32_t) * (size_t)(e > 0 ? e : 1));
  w.X = take(sizeof(float) * (size_t)per);     // sized for fp32 storage
  w.GT = take(sizeof(float) * (size_t)per);
  w.Y = take(sizeof(float) * (size_t)per);
  w.rbf = take(sizeof(float) * 8 * (size_t)B);
  w.part = take(sizeof(float) * (size_t)pf);
  w.dwpart = take(sizeof(float) * (size_t)dw_part_floats(L, C));
  w.rhopart = take(sizeof(float) * (size_t)((B + kRhoPer - 1) / kRhoPer) * 8 * K0);
  int64_t so2 = 0;
  for (int m = 0; m <= L; ++m) so2 += (m == 0 ? 1 : 2) * ((int64_t)(L + 1 - m) * C) * ((int64_t)(L + 1 - m) * C);
  w.wt = take(sizeof(float) * (size_t)so2);   // sized for fp32 storage
  w.rbfd = take(sizeof(float) * 8 * (size_t)B);
  w.alpha = take(sizeof(float) * (size_t)B * H);
  w.dX = take(sizeof(float) * (size_t)per);
  w.gedge = take(sizeof(float) * 3 * (size_t)(e > 0 ? e : 1));
  w.gbf = take(sizeof(uint16_t) * (size_t)n * (L + 1) * (L + 1) * C);
  w.total = off;
  w.B = B;
  w.part_floats = pf;
  return w;
}

// Second k segment of a product (matrix-core kernel): A2, B2 at k - K1.
void pair_segments(Gemm& g, const void* A2, const void* B2, int64_t K1, bool neg2) {
  g.A2 = A2;
  g.B2 = B2;
  g.K1 = K1;
  g.neg2 = neg2;
}

template <int L, typename T>
e2a_status run_wgrad(const WgradPlan& pl, hipStream_t st) {
  // bf16 products run on the matrix-core kernel, which takes two k segments
  constexpr bool kPairs = std::is_same<T, uint16_t>::value;
  const e2a_attn_args* a = pl.a;
  constexpr int K = (L + 1) * (L + 1);
  const int C = a->C, H = a->H;
  const int64_t n = a->n_atoms, E = a->n_edges;
  const int64_t K0 = (int64_t)(L + 1) * C;
  const WgWs W = wg_ws_layout(n, E, L, C, H);
  char* wb = static_cast<char*>(pl.ws);
  float* part = reinterpret_cast<float*>(wb + W.part);
  auto zero = [&](float* p, int64_t cnt) {
    if (!p || cnt <= 0) return;
    k_zero<<<static_cast<unsigned>((cnt + 255) / 256), 256, 0, st>>>(p, cnt);
  };
  int64_t so2_count = 0;
  for (int m = 0; m <= L; ++m) so2_count += (m == 0 ? 1 : 2) * ((int64_t)(L + 1 - m) * C) * ((int64_t)(L + 1 - m) * C);
  zero(pl.w_q, (int64_t)C * C);
  zero(pl.w_k, (int64_t)C * C);
  zero(pl.w_rad, 8 * K0);
  zero(pl.w_so2, so2_count);
  zero(pl.pos, 3 * n);
  E2A_LAUNCH_CHECK();
  const T* feat = static_cast<const T*>(a->feat);
  // dW_q = sum_i h_{i,0}^T dq_i, dW_k likewise (A(m, k) = h_k[0][m])
  if (pl.w_q) {
    const e2a_status e = gemm<T, float>(make_gemm(feat, 1, (int64_t)K * C, pl.dq, C, 1, C, C, n, 1.0f, pl.w_q, C,
                                                  part), W.part_floats, st);
    if (e != E2A_OK) return e;
  }
  if (pl.w_k) {
    const e2a_status e = gemm<T, float>(make_gemm(feat, 1, (int64_t)K * C, pl.dk, C, 1, C, C, n, 1.0f, pl.w_k, C,
                                                  part), W.part_floats, st);
    if (e != E2A_OK) return e;
  }
  if ((!pl.w_rad && !pl.w_so2 && !pl.pos) || E == 0) return E2A_OK;
  const bool need_y = pl.w_rad || pl.pos;   // drho needs SO2(x)
  // where dW_rad is asked of the batches (builds without the fused radial
  // pass), the gather also keeps dyhat (in the dx buffer, free until the dx
  // products) for the drho pass; the force kernel forms its own drho
  const bool rho_pass = pl.w_rad != nullptr;

  int32_t* src = reinterpret_cast<int32_t*>(wb + W.src);
  k_edge_rows<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(a->row_ptr, n, src);
  E2A_LAUNCH_CHECK();
  T* X = reinterpret_cast<T*>(wb + W.X);
  T* GT = reinterpret_cast<T*>(wb + W.GT);
  float* Y = reinterpret_cast<float*>(wb + W.Y);
  // y = SO2(x) and dx = SO2^T(dy) are kept in bf16 where every block takes
  // the one-launch pair path (bf16 storage, C a multiple of 32) and the
  // matrix-core force kernel, which reads them as its operands, fits
  const bool yb = kPairs && C % kBK == 0 && force_mfma_fits(L, C);
  auto to_out = [&](Gemm g, size_t buf, int64_t off) {
    if (yb) {
      g.Cb = reinterpret_cast<uint16_t*>(wb + buf) + off;
      g.C = nullptr;
    } else {
      g.C = reinterpret_cast<float*>(wb + buf) + off;
    }
    return g;
  };
  if (pl.ds && !(pl.pos && pl.delta && yb && C == 128 && H == 8 && L >= 1))
    return fail(E2A_ERR_UNSUPPORTED, "ds from the edge batches needs the positions, bf16, C = 128, H = 8, L >= 1");
  if (pl.pos && yb && !pl.grad_bf) {
    // the matrix-core force kernel reads G in bf16; this call has no copy yet
    const int64_t cnt = n * K * C;
    k_to_bf16<<<static_cast<unsigned>((cnt + 255) / 256), 256, 0, st>>>(pl.grad_out,
                                                                       reinterpret_cast<uint16_t*>(wb + W.gbf), cnt);
    E2A_LAUNCH_CHECK();
  }
  float* rbf = reinterpret_cast<float*>(wb + W.rbf);
  const BatchLayout bl = batch_layout(W.B, L, C);
  const T* wso2 = static_cast<const T*>(a->w_so2);
  int64_t woff[L + 1];
  {
    int64_t o = 0;
    for (int m = 0; m <= L; ++m) {
      woff[m] = o;
      const int64_t km = (int64_t)(L + 1 - m) * C;
      o += (m == 0 ? 1 : 2) * km * km;
    }
  }
  // W^T per block, for the Y products
  T* wt = reinterpret_cast<T*>(wb + W.wt);
  if (need_y)
    for (int m = 0; m <= L; ++m) {
      const int64_t km = (int64_t)(L + 1 - m) * C;
      for (int w2 = 0; w2 < (m == 0 ? 1 : 2); ++w2) {
        k_transpose_block<T><<<static_cast<unsigned>((km * km + 255) / 256), 256, 0, st>>>(
            wso2 + woff[m] + w2 * km * km, km, wt + woff[m] + w2 * km * km);
        E2A_LAUNCH_CHECK();
      }
    }
  float* rhopart = reinterpret_cast<float*>(wb + W.rhopart);
  for (int64_t e0 = 0; e0 < E; e0 += W.B) {
    const int64_t nb = E - e0 < W.B ? E - e0 : W.B;
    GatherParams gp{};
    gp.pos = a->pos;
    gp.col = a->col;
    gp.src = src;
    gp.q = pl.q;
    gp.k = pl.k;
    gp.lse = a->out_lse;
    gp.grad = pl.grad_out;
    for (int d = 0; d < 3; ++d) gp.box[d] = pl.box[d];
    gp.periodic = pl.periodic;
    gp.cutoff = a->cutoff;
    gp.C = C;
    gp.H = H;
    gp.e0 = e0;
    gp.nb = nb;
    gp.bl = bl;
    gp.rbf = rbf;
    gp.rbfd = pl.pos ? reinterpret_cast<float*>(wb + W.rbfd) : nullptr;
    gp.alpha = pl.pos ? reinterpret_cast<float*>(wb + W.alpha) : nullptr;
    gp.w_rad = a->w_rad;
    gp.dyhat = rho_pass ? reinterpret_cast<float*>(wb + W.dX) : nullptr;
    const size_t smem = sizeof(float) * kEB * (wig_size(L) + H);
    k_wg_gather<L, T><<<static_cast<unsigned>((nb + kEB - 1) / kEB), 256, smem, st>>>(gp, feat, X, GT);
    E2A_LAUNCH_CHECK();
    // Y = SO2(X): Y0 = X0 W0; Yp = Xp W1 - Xm W2; Ym = Xp W2 + Xm W1 (for
    // drho and the rotate-out's share of the position gradient)
    for (int m = 0; need_y && m <= L; ++m) {
      const int64_t km = (int64_t)(L + 1 - m) * C;
      const T* Xp = X + bl.moff[m];
      float* Yp = Y + bl.moff[m];
      const T* W1 = wt + woff[m];   // W1^T (W0^T for m = 0), [n][k]
      e2a_status e;
      if (m == 0) {
        e = gemm<T, T>(to_out(make_gemm(Xp, km, 1, W1, 1, km, nb, km, km, 1.0f, nullptr, km, part, true), W.Y,
                              bl.moff[m]),
                       W.part_floats, st);
        if (e != E2A_OK) return e;
        continue;
      }
      const T* Xm = Xp + bl.B * km;
      float* Ym = Yp + bl.B * km;
      const T* W2 = W1 + km * km;
      if (yb) {
        // y+ = x+ W1 - x- W2 and y- = x+ W2 + x- W1 from one read of the four slices
        GemmCx g{};
        g.A1 = reinterpret_cast<const uint16_t*>(Xp);
        g.A2 = reinterpret_cast<const uint16_t*>(Xm);
        g.B1 = reinterpret_cast<const uint16_t*>(W1);
        g.B2 = reinterpret_cast<const uint16_t*>(W2);
        g.sa = g.sb = km;
        g.M = nb;
        g.N = g.K = g.kper = km;
        g.aP = g.aQ = 1.0f;
        g.s1neg = true;
        g.P_bf = reinterpret_cast<uint16_t*>(wb + W.Y) + bl.moff[m];
        g.Q_bf = g.P_bf + bl.B * km;
        g.ldc = km;
        e = launch_gemm_cx<false>(g, 1, st);
        if (e != E2A_OK) return e;
        continue;
      }
      if (kPairs && km % kBK == 0) {
        // one launch per output: Yp = [Xp | Xm] [W1; -W2], Ym = [Xp | Xm] [W2; W1]
        for (int t = 0; t < 2; ++t) {
          Gemm g = to_out(make_gemm(Xp, km, 1, t == 0 ? W1 : W2, 1, km, nb, km, 2 * km, 1.0f, nullptr, km, part,
                                    true),
                          W.Y, bl.moff[m] + (t == 0 ? 0 : bl.B * km));
          pair_segments(g, Xm, t == 0 ? W2 : W1, km, t == 0);
          e = gemm<T, T>(g, W.part_floats, st);
          if (e != E2A_OK) return e;
        }
        continue;
      }
      const struct { const T* x; const T* w; float* y; float s; bool first; } terms[4] = {
          {Xp, W1, Yp, 1.0f, true}, {Xm, W2, Yp, -1.0f, false}, {Xp, W2, Ym, 1.0f, true}, {Xm, W1, Ym, 1.0f, false}};
      for (const auto& t : terms) {
        e = gemm<T, T>(make_gemm(t.x, km, 1, t.w, 1, km, nb, km, km, t.s, t.y, km, part, t.first), W.part_floats,
                       st);
        if (e != E2A_OK) return e;
      }
    }
    // dW_rad[k][(l, c)] += sum_b rbf[b][k] drho[b][(l, c)] through per-range
    // partials added in order
    if (rho_pass) {
      const int64_t per = kRhoPer;
      const int64_t nz = (nb + per - 1) / per;
      const dim3 grid(static_cast<unsigned>((K0 + 255) / 256), static_cast<unsigned>(nz));
      const float* dyh = reinterpret_cast<const float*>(wb + W.dX);
      if (yb)
        k_wg_rho<L, uint16_t><<<grid, 256, 0, st>>>(bl, nb, C, per, rbf, reinterpret_cast<const uint16_t*>(wb + W.Y),
                                                    dyh, rhopart, e0 > 0);
      else
        k_wg_rho<L, float><<<grid, 256, 0, st>>>(bl, nb, C, per, rbf, Y, dyh, rhopart, e0 > 0);
      E2A_LAUNCH_CHECK();
    }
    if (pl.w_so2) {
      float* dwp = reinterpret_cast<float*>(wb + W.dwpart);
      for (int m = 0; m <= L; ++m) {
        const int64_t km = (int64_t)(L + 1 - m) * C;
        const int64_t S = dw_splits(L, C, m);
        const T* Xp = X + bl.moff[m];
        const T* DYp = GT + bl.moff[m];
        float* p1 = dwp;
        float* p2 = dwp + S * km * km;
        dwp += (m == 0 ? 1 : 2) * S * km * km;
        // A(m', k) = X[k][m'] (transposed rows), B(k, n) = dY[k][n]
        const T* Xm = Xp + bl.B * km;
        const T* DYm = DYp + bl.B * km;
        if (kPairs && m > 0 && km % 8 == 0) {
          // dW1 (+)= x+^T dy+ + x-^T dy-, dW2 (+)= x+^T dy- - x-^T dy+ in one launch
          // (16-byte rows: km a multiple of 8)
          GemmCx g{};
          g.A1 = reinterpret_cast<const uint16_t*>(Xp);
          g.A2 = reinterpret_cast<const uint16_t*>(Xm);
          g.B1 = reinterpret_cast<const uint16_t*>(DYp);
          g.B2 = reinterpret_cast<const uint16_t*>(DYm);
          g.sa = g.sb = km;
          g.M = g.N = km;
          g.K = nb;
          g.aP = g.aQ = 1.0f;
          g.s2neg = true;
          g.P_part = p1;
          g.Q_part = p2;
          g.part_acc = e0 > 0;
          const int64_t Sp = dw_splits_pair(L, C, m);
          g.kper = ((nb + Sp - 1) / Sp + kBK - 1) / kBK * kBK;
          const e2a_status e = launch_gemm_cx<true>(g, static_cast<int>(Sp), st);
          if (e != E2A_OK) return e;
          continue;
        }
        if (kPairs && nb % kBK == 0) {
          // one launch per matrix: p1 (+)= [Xp; Xm]^T [dYp; dYm], p2 (+)= [Xp; Xm]^T [dYm; -dYp]
          for (int t = 0; t < (m == 0 ? 1 : 2); ++t) {
            Gemm g = make_gemm(Xp, 1, km, t == 0 ? DYp : DYm, km, 1, km, km, m == 0 ? nb : 2 * nb, 1.0f, nullptr,
                               km, t == 0 ? p1 : p2);
            if (m > 0) pair_segments(g, Xm, t == 0 ? DYm : DYp, nb, t == 1);
            g.S = static_cast<int>(S);
            g.kper = ((g.K + S - 1) / S + 31) / 32 * 32;
            g.part_acc = e0 > 0;
            const e2a_status e = launch_gemm<T, T>(g, st);
            if (e != E2A_OK) return e;
          }
          continue;
        }
        const struct { const T* x; const T* dy; float* part; float s; bool first; } terms[4] = {
            {Xp, DYp, p1, 1.0f, true}, {Xm, DYm, p1, 1.0f, false}, {Xp, DYm, p2, 1.0f, true},
            {Xm, DYp, p2, -1.0f, false}};
        for (int t = 0; t < (m == 0 ? 1 : 4); ++t) {
          Gemm g = make_gemm(terms[t].x, 1, km, terms[t].dy, km, 1, km, km, nb, terms[t].s, nullptr, km,
                             terms[t].part);
          g.S = static_cast<int>(S);
          g.kper = ((nb + S - 1) / S + 31) / 32 * 32;
          g.part_acc = !(e0 == 0 && terms[t].first);
          const e2a_status e = launch_gemm<T, T>(g, st);
          if (e != E2A_OK) return e;
        }
      }
    }
    if (pl.pos) {
      // dx = SO2^T(dy): dX0 = dY0 W0^T; dXp = dYp W1^T + dYm W2^T;
      // dXm = -dYp W2^T + dYm W1^T (W read as [n][k]: contiguous along k)
      float* dX = reinterpret_cast<float*>(wb + W.dX);
      for (int m = 0; m <= L; ++m) {
        const int64_t km = (int64_t)(L + 1 - m) * C;
        const T* DYp = GT + bl.moff[m];
        const T* W1 = wso2 + woff[m];
        float* dXp = dX + bl.moff[m];
        e2a_status e;
        if (m == 0) {
          e = gemm<T, T>(to_out(make_gemm(DYp, km, 1, W1, 1, km, nb, km, km, 1.0f, nullptr, km, part, true), W.dX,
                                bl.moff[m]),
                         W.part_floats, st);
          if (e != E2A_OK) return e;
          continue;
        }
        const T* DYm = DYp + bl.B * km;
        const T* W2 = W1 + km * km;
        float* dXm = dXp + bl.B * km;
        if (yb) {
          // dx+ = dy+ W1^T + dy- W2^T and dx- = -(dy+ W2^T - dy- W1^T) in one launch
          GemmCx g{};
          g.A1 = reinterpret_cast<const uint16_t*>(DYp);
          g.A2 = reinterpret_cast<const uint16_t*>(DYm);
          g.B1 = reinterpret_cast<const uint16_t*>(W1);
          g.B2 = reinterpret_cast<const uint16_t*>(W2);
          g.sa = g.sb = km;
          g.M = nb;
          g.N = g.K = g.kper = km;
          g.aP = 1.0f;
          g.aQ = -1.0f;
          g.s2neg = true;
          g.P_bf = reinterpret_cast<uint16_t*>(wb + W.dX) + bl.moff[m];
          g.Q_bf = g.P_bf + bl.B * km;
          g.ldc = km;
          e = launch_gemm_cx<false>(g, 1, st);
          if (e != E2A_OK) return e;
          continue;
        }
        if (kPairs && km % kBK == 0) {
          // one launch per output: dXp = [dYp | dYm] [W1^T; W2^T], dXm = [dYm | dYp] [W1^T; -W2^T]
          for (int t = 0; t < 2; ++t) {
            Gemm g = to_out(make_gemm(t == 0 ? DYp : DYm, km, 1, W1, 1, km, nb, km, 2 * km, 1.0f, nullptr, km, part,
                                      true),
                            W.dX, bl.moff[m] + (t == 0 ? 0 : bl.B * km));
            pair_segments(g, t == 0 ? DYm : DYp, W2, km, t == 1);
            e = gemm<T, T>(g, W.part_floats, st);
            if (e != E2A_OK) return e;
          }
          continue;
        }
        const struct { const T* dy; const T* w; float* x; float s; bool first; } terms[4] = {
            {DYp, W1, dXp, 1.0f, true}, {DYm, W2, dXp, 1.0f, false}, {DYp, W2, dXm, -1.0f, true},
            {DYm, W1, dXm, 1.0f, false}};
        for (const auto& t : terms) {
          e = gemm<T, T>(make_gemm(t.dy, km, 1, t.w, 1, km, nb, km, km, t.s, t.x, km, part, t.first),
                         W.part_floats, st);
          if (e != E2A_OK) return e;
        }
      }
      if (pl.ds) {
        if constexpr (kPairs && L >= 1) {
          k_wg_ds<L><<<static_cast<unsigned>((nb + kDsEdges - 1) / kDsEdges), 64 * kDsEdges, 0, st>>>(
              bl, nb, e0, src, reinterpret_cast<const uint16_t*>(wb + W.Y), reinterpret_cast<const uint16_t*>(GT),
              reinterpret_cast<const float*>(wb + W.alpha), pl.delta, pl.ds);
          E2A_LAUNCH_CHECK();
        }
      }
      ForceParams fp{};
      fp.pos = a->pos;
      fp.col = a->col;
      fp.src = src;
      fp.grad = pl.grad_out;
      fp.alpha = reinterpret_cast<const float*>(wb + W.alpha);
      fp.rbf = rbf;
      fp.Y = wb + W.Y;
      fp.dX = wb + W.dX;
      fp.rbfd = reinterpret_cast<const float*>(wb + W.rbfd);
      fp.gbf = pl.grad_bf ? pl.grad_bf : reinterpret_cast<const uint16_t*>(wb + W.gbf);
      fp.gedge = reinterpret_cast<float*>(wb + W.gedge);
      for (int d = 0; d < 3; ++d) fp.box[d] = pl.box[d];
      fp.periodic = pl.periodic;
      fp.C = C;
      fp.H = H;
      fp.e0 = e0;
      fp.bl = bl;
      if constexpr (kPairs) {
        if (yb) {
          constexpr int64_t per = kFmWaves * kFmIters;
          const unsigned grid = static_cast<unsigned>((nb + per - 1) / per);
          const size_t smem = force_mfma_smem(L, C);
          if (C == 128)
            k_wg_force_mfma<L, 128><<<grid, 64 * kFmWaves, smem, st>>>(fp, nb, feat,
                                                                      static_cast<const uint16_t*>(a->w_rad));
          else
            k_wg_force_mfma<L, 0><<<grid, 64 * kFmWaves, smem, st>>>(fp, nb, feat,
                                                                    static_cast<const uint16_t*>(a->w_rad));
          E2A_LAUNCH_CHECK();
          continue;
        }
      }
      k_wg_force<L, T><<<static_cast<unsigned>((nb + kForceEdges - 1) / kForceEdges), 64 * kForceEdges, 0, st>>>(
          fp, nb, feat, static_cast<const T*>(a->w_rad));
      E2A_LAUNCH_CHECK();
    }
  }
  if (pl.pos) {
    k_pos_assemble<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(
        a->row_ptr, a->col, n, reinterpret_cast<const float*>(wb + W.gedge), pl.pos);
    E2A_LAUNCH_CHECK();
  }
  if (pl.w_rad) {
    // the edge ranges' partials of dW_rad, added in order (the first batch
    // is the largest, so it set every slot)
    Gemm r = make_gemm(nullptr, 0, 0, nullptr, 0, 0, 8, K0, 0, 1.0f, pl.w_rad, K0, rhopart);
    r.S = static_cast<int>((W.B + kRhoPer - 1) / kRhoPer);
    r.overwrite = true;
    const e2a_status e = reduce_parts(r, st);
    if (e != E2A_OK) return e;
  }
  if (pl.w_so2) {
    // the partials of every matrix, added in order into its block of dW_so2
    const float* dwp = reinterpret_cast<const float*>(wb + W.dwpart);
    for (int m = 0; m <= L; ++m) {
      const int64_t km = (int64_t)(L + 1 - m) * C;
      const int64_t S = dw_splits(L, C, m);
      for (int w = 0; w < (m == 0 ? 1 : 2); ++w) {
        Gemm r = make_gemm(nullptr, 0, 0, nullptr, 0, 0, km, km, 0, 1.0f, pl.w_so2 + woff[m] + w * km * km, km,
                           const_cast<float*>(dwp));
        // the k ranges the batches used (the buffers keep S slots per matrix)
        r.S = static_cast<int>(kPairs && m > 0 && km % 8 == 0 ? dw_splits_pair(L, C, m) : S);
        r.overwrite = true;
        const e2a_status e = reduce_parts(r, st);
        if (e != E2A_OK) return e;
        dwp += S * km * km;
      }
    }
  }
  return E2A_OK;
}

template <typename T>
e2a_status run_wgrad_dtype(const WgradPlan& pl, hipStream_t st) {
  switch (pl.a->L) {
    case 0: return run_wgrad<0, T>(pl, st);
    case 1: return run_wgrad<1, T>(pl, st);
    case 2: return run_wgrad<2, T>(pl, st);
    case 3: return run_wgrad<3, T>(pl, st);
    case 4: return run_wgrad<4, T>(pl, st);
    default: return fail(E2A_ERR_UNSUPPORTED, "L=%d", pl.a->L);
  }
}

}  // namespace

size_t wgrad_workspace_bytes(int64_t n, int64_t e, int L, int C, int H, int dtype) {
  (void)dtype;
  return wg_ws_layout(n, e, L, C, H).total;
}

e2a_status launch_weight_grads(const WgradPlan& pl, hipStream_t s) {
  if (pl.a->n_atoms == 0) return E2A_OK;
  return pl.a->dtype == E2A_DTYPE_BF16 ? run_wgrad_dtype<uint16_t>(pl, s) : run_wgrad_dtype<float>(pl, s);
}

}  // namespace e2a

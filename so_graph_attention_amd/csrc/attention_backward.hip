// Feature gradient of the fused layer, dL/dh for a cotangent G = dL/do.
//
// arXiv 2601.16622, English technical summary section 2.2 ("On-the-Fly
// Equivariant Attention"): the layer keeps only per-destination softmax
// statistics on chip and recomputes per-edge quantities instead of storing
// them, which is what makes training at linear activation memory possible.
// The backward follows the same plan: from the forward's output o and
// log-normaliser lse it recomputes each edge's weight and message.
//
//   query pass, one workgroup per destination i:
//     delta_i^h = sum_{k, c in h} G_i o_i; for each j in N(i) the message
//     v_ij, alpha_ij = exp(s_ij - lse_i), dalpha = sum_{k, c in h} G_i v_ij,
//     ds_ij = alpha_ij (dalpha - delta_i) (kept, one float per edge and
//     head), dq_i = sum_j ds_ij k_j / sqrt(C/H);
//   value pass, one workgroup per atom j, over i in N(j) (the radius graph is
//     symmetric, so these are the destinations whose lists hold j):
//     dk_j = sum_i ds_ij q_i / sqrt(C/H) and the transposed message
//     dh_j += D_ij^T SO2^T(rho_ij * D_ij (alpha_ij G_i)), where D_ij, rho_ij
//     belong to the edge from centre i to neighbour j; then the l = 0 block
//     gets dq_j W_q^T + dk_j W_k^T.
//
// Every product is fp32 on the vector ALUs, in LDS-resident per-edge tiles,
// like the scalar forward kernel.  Weight and position gradients are not
// computed.
#include "e2a_geometry.hpp"
#include "e2a_internal.hpp"

namespace e2a {
namespace {

struct BwdParams {
  const float* pos;
  const int64_t* row_ptr;
  const int32_t* col;
  const float* q;       // [N, C]
  const float* k;       // [N, C]
  const float* out;     // forward output o [N, K, C]
  const float* lse;     // forward log-normaliser [N, H]
  const float* grad;    // G = dL/do [N, K, C]
  float* ds;            // [E, H]
  float* dq;            // [N, C]
  float* grad_feat;     // [N, K, C]
  float* wdq;           // optional outputs of k_bwd_qk: dq, dk [N, C]
  float* wdk;
  float box[3];
  int periodic;
  float cutoff;
  int C, H;
};

// Frame of the edge from centre a to neighbour b (r = x_b - x_a, minimum
// image; the same fp32 operations as the forward kernels), its Wigner blocks
// and its radial basis.  One thread.
template <int L>
__device__ void edge_frame(const BwdParams& p, int64_t a, int64_t b, float* D, float* rbf) {
  float r3[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    float dx = p.pos[3 * b + d] - p.pos[3 * a + d];
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
  wigner_blocks<L>(R, D);
  radial_basis8(r, p.cutoff, rbf);
}

__device__ __forceinline__ int degree_of(int comp) {
  int l = 0;
  while ((l + 1) * (l + 1) <= comp) ++l;
  return l;
}

// dst[l, m][c] = sum_n D^l[m][n] src[l, n][c]  (src read through `ld`).
template <int L, typename LD>
__device__ void rot_apply(const float* D, const LD& ld, float* dst, int C) {
  constexpr int K = (L + 1) * (L + 1);
  for (int t = threadIdx.x; t < K * C; t += blockDim.x) {
    const int comp = t / C, c = t % C;
    const int l = degree_of(comp);
    const float* Dl = D + wig_off(l) + (comp - l * l) * (2 * l + 1);
    float v = 0.0f;
    for (int n = 0; n < 2 * l + 1; ++n) v += Dl[n] * ld((l * l + n) * C + c);
    dst[t] = v;
  }
}

// dst[l, n][c] (+)= sum_m D^l[m][n] src[l, m][c]  (D^T).
template <int L, bool ACC>
__device__ void rot_apply_t(const float* D, const float* src, float* dst, int C) {
  constexpr int K = (L + 1) * (L + 1);
  for (int t = threadIdx.x; t < K * C; t += blockDim.x) {
    const int comp = t / C, c = t % C;
    const int l = degree_of(comp);
    const int ni = comp - l * l;
    const float* Dl = D + wig_off(l);
    float v = 0.0f;
    for (int mi = 0; mi < 2 * l + 1; ++mi) v += Dl[mi * (2 * l + 1) + ni] * src[(l * l + mi) * C + c];
    dst[t] = ACC ? dst[t] + v : v;
  }
}

// rho[l][c] = sum_k e_k W_rad[k][l][c].
template <int L, typename T>
__device__ void radial(const float* rbf, const T* w_rad, float* rho, int C) {
  for (int t = threadIdx.x; t < (L + 1) * C; t += blockDim.x) {
    float v = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) v += rbf[kk] * load_as_f32(w_rad, (size_t)kk * (L + 1) * C + t);
    rho[t] = v;
  }
}

template <int L>
__device__ void block_offsets(int C, int64_t (&woff)[L + 1]) {
  int64_t o = 0;
#pragma unroll
  for (int m = 0; m <= L; ++m) {
    woff[m] = o;
    const int64_t km = (int64_t)(L + 1 - m) * C;
    o += (m == 0 ? 1 : 2) * km * km;
  }
}

// Per-m SO(2) mix (technical summary section 2.1): y = SO2(x).
template <int L, typename T>
__device__ void so2_forward(const float* x, float* y, const T* w_so2, const int64_t (&woff)[L + 1], int C) {
  constexpr int K = (L + 1) * (L + 1);
  for (int t = threadIdx.x; t < K * C; t += blockDim.x) {
    const int comp = t / C, co = t % C;
    const int lo = degree_of(comp);
    const int m = comp - lo * lo - lo;
    const int am = m < 0 ? -m : m;
    const int64_t km = (int64_t)(L + 1 - am) * C;
    float acc = 0.0f;
    if (am == 0) {
      const T* W0 = w_so2 + woff[0];
      for (int li = 0; li <= L; ++li) {
        const float* xr = x + (li * li + li) * C;
        const T* wr = W0 + (int64_t)(li * C) * km + (int64_t)lo * C + co;
        for (int ci = 0; ci < C; ++ci) acc += xr[ci] * load_as_f32(wr, (size_t)ci * km);
      }
    } else {
      const T* W1 = w_so2 + woff[am];
      const T* W2 = W1 + km * km;
      for (int li = am; li <= L; ++li) {
        const float* xp = x + (li * li + li + am) * C;
        const float* xm = x + (li * li + li - am) * C;
        const int64_t base = (int64_t)((li - am) * C) * km + (int64_t)(lo - am) * C + co;
        for (int ci = 0; ci < C; ++ci) {
          const float w1 = load_as_f32(W1, base + (size_t)ci * km);
          const float w2 = load_as_f32(W2, base + (size_t)ci * km);
          acc += m > 0 ? xp[ci] * w1 - xm[ci] * w2 : xp[ci] * w2 + xm[ci] * w1;
        }
      }
    }
    y[t] = acc;
  }
}

// Transpose of the per-m mix: dx = SO2^T(dy),
//   m = 0: dx_0 = dy_0 W0^T;  m > 0: dx_+ = dy_+ W1^T + dy_- W2^T,
//   dx_- = -dy_+ W2^T + dy_- W1^T.
template <int L, typename T>
__device__ void so2_transpose(const float* dy, float* dx, const T* w_so2, const int64_t (&woff)[L + 1], int C) {
  constexpr int K = (L + 1) * (L + 1);
  for (int t = threadIdx.x; t < K * C; t += blockDim.x) {
    const int comp = t / C, ci = t % C;
    const int li = degree_of(comp);
    const int m = comp - li * li - li;
    const int am = m < 0 ? -m : m;
    const int64_t km = (int64_t)(L + 1 - am) * C;
    float acc = 0.0f;
    if (am == 0) {
      const T* wr = w_so2 + woff[0] + (int64_t)(li * C + ci) * km;
      for (int lo = 0; lo <= L; ++lo) {
        const float* dr = dy + (lo * lo + lo) * C;
        for (int co = 0; co < C; ++co) acc += dr[co] * load_as_f32(wr, (size_t)lo * C + co);
      }
    } else {
      const T* W1 = w_so2 + woff[am] + (int64_t)((li - am) * C + ci) * km;
      const T* W2 = W1 + km * km;
      for (int lo = am; lo <= L; ++lo) {
        const float* dp = dy + (lo * lo + lo + am) * C;
        const float* dm = dy + (lo * lo + lo - am) * C;
        const size_t cb = (size_t)(lo - am) * C;
        for (int co = 0; co < C; ++co) {
          const float w1 = load_as_f32(W1, cb + co);
          const float w2 = load_as_f32(W2, cb + co);
          acc += m > 0 ? dp[co] * w1 + dm[co] * w2 : -dp[co] * w2 + dm[co] * w1;
        }
      }
    }
    dx[t] = acc;
  }
}

// Query pass: one workgroup per destination i.
template <int L, typename T>
__global__ void __launch_bounds__(256) k_bwd_query(BwdParams p, const T* __restrict__ feat,
                                                    const T* __restrict__ w_rad, const T* __restrict__ w_so2) {
  constexpr int K = (L + 1) * (L + 1);
  const int C = p.C, H = p.H, dh = C / H;
  extern __shared__ float smem[];
  float* G = smem;                  // [K][C] cotangent of o_i
  float* xt = G + K * C;            // [K][C] rotated features, then the message v_ij
  float* yt = xt + K * C;           // [K][C] SO(2)-mixed features
  float* rho = yt + K * C;          // [L+1][C]
  float* qi = rho + (L + 1) * C;    // [C]
  float* dqa = qi + C;              // [C] dq accumulator
  float* D = dqa + C;               // [wig_size(L)]
  float* delta = D + wig_size(L);   // [H]
  float* alpha = delta + H;         // [H]
  float* dsh = alpha + H;           // [H]
  __shared__ float rbf[8];
  __shared__ int jsh;
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const float inv = 1.0f / sqrtf(static_cast<float>(dh));
  int64_t woff[L + 1];
  block_offsets<L>(C, woff);

  for (int t = tid; t < K * C; t += blockDim.x) G[t] = p.grad[i * K * C + t];
  for (int t = tid; t < C; t += blockDim.x) { qi[t] = p.q[i * C + t]; dqa[t] = 0.0f; }
  __syncthreads();
  // delta_i^h = sum_{k, c in h} G_i o_i, one thread per head (fixed order)
  if (tid < H) {
    float s = 0.0f;
    for (int kk = 0; kk < K; ++kk)
      for (int c = tid * dh; c < (tid + 1) * dh; ++c) s += G[kk * C + c] * p.out[(i * K + kk) * C + c];
    delta[tid] = s;
  }
  const int64_t e0 = p.row_ptr[i], e1 = p.row_ptr[i + 1];
  for (int64_t e = e0; e < e1; ++e) {
    if (tid == 0) {
      const int j = p.col[e];
      jsh = j;
      edge_frame<L>(p, i, j, D, rbf);
    }
    __syncthreads();
    const int j = jsh;
    if (tid >= 64 && tid < 64 + H) {
      const int h = tid - 64;
      float s = 0.0f;
      for (int d = 0; d < dh; ++d) s += qi[h * dh + d] * p.k[(int64_t)j * C + h * dh + d];
      alpha[h] = expf(s * inv - p.lse[i * H + h]);
    }
    const T* hj = feat + (int64_t)j * K * C;
    rot_apply<L>(D, [&](int idx) { return load_as_f32(hj, (size_t)idx); }, xt, C);
    radial<L>(rbf, w_rad, rho, C);
    __syncthreads();
    so2_forward<L>(xt, yt, w_so2, woff, C);
    __syncthreads();
    // v = D^T (rho * y), into xt
    for (int t = tid; t < K * C; t += blockDim.x) yt[t] *= rho[degree_of(t / C) * C + t % C];
    __syncthreads();
    rot_apply_t<L, false>(D, yt, xt, C);
    __syncthreads();
    if (tid < H) {
      float da = 0.0f;
      for (int kk = 0; kk < K; ++kk)
        for (int c = tid * dh; c < (tid + 1) * dh; ++c) da += G[kk * C + c] * xt[kk * C + c];
      const float ds = alpha[tid] * (da - delta[tid]);
      p.ds[e * H + tid] = ds;
      dsh[tid] = ds;
    }
    __syncthreads();
    for (int c = tid; c < C; c += blockDim.x) dqa[c] += dsh[c / dh] * p.k[(int64_t)j * C + c] * inv;
    __syncthreads();
  }
  __syncthreads();
  for (int c = tid; c < C; c += blockDim.x) p.dq[i * C + c] = dqa[c];
}

// Value pass: one workgroup per atom j, over the destinations i whose
// neighbour lists hold j (the rows of j itself, the graph being symmetric).
template <int L, typename T>
__global__ void __launch_bounds__(256) k_bwd_value(BwdParams p, const T* __restrict__ w_q, const T* __restrict__ w_k,
                                                    const T* __restrict__ w_rad, const T* __restrict__ w_so2) {
  constexpr int K = (L + 1) * (L + 1);
  const int C = p.C, H = p.H, dh = C / H;
  extern __shared__ float smem[];
  float* acc = smem;                // [K][C] dL/dh_j from the values
  float* xt = acc + K * C;          // [K][C]
  float* yt = xt + K * C;           // [K][C]
  float* rho = yt + K * C;          // [L+1][C]
  float* qi = rho + (L + 1) * C;    // [C] q of the centre i
  float* kj = qi + C;               // [C]
  float* dka = kj + C;              // [C] dk accumulator
  float* D = dka + C;               // [wig_size(L)]
  float* alpha = D + wig_size(L);   // [H]
  float* dsv = alpha + H;           // [H]
  __shared__ float rbf[8];
  __shared__ int ish;
  __shared__ int64_t esh;
  const int64_t j = blockIdx.x;
  const int tid = threadIdx.x;
  const float inv = 1.0f / sqrtf(static_cast<float>(dh));
  int64_t woff[L + 1];
  block_offsets<L>(C, woff);

  for (int t = tid; t < K * C; t += blockDim.x) acc[t] = 0.0f;
  for (int t = tid; t < C; t += blockDim.x) { kj[t] = p.k[j * C + t]; dka[t] = 0.0f; }
  __syncthreads();
  const int64_t t0 = p.row_ptr[j], t1 = p.row_ptr[j + 1];
  for (int64_t t = t0; t < t1; ++t) {
    if (tid == 0) {
      const int i = p.col[t];
      ish = i;
      // position of j in the (ascending) row of i; -1 if the row lacks j (a
      // graph that is not symmetric: the edge then contributes nothing)
      const int64_t end = p.row_ptr[i + 1];
      int64_t lo = p.row_ptr[i], hi = end;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (p.col[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      esh = (lo < end && p.col[lo] == j) ? lo : -1;
      edge_frame<L>(p, i, j, D, rbf);
    }
    __syncthreads();
    const int i = ish;
    const int64_t eij = esh;
    for (int c = tid; c < C; c += blockDim.x) qi[c] = p.q[(int64_t)i * C + c];
    __syncthreads();
    if (tid >= 64 && tid < 64 + H) {
      const int h = tid - 64;
      float s = 0.0f;
      for (int d = 0; d < dh; ++d) s += qi[h * dh + d] * kj[h * dh + d];
      alpha[h] = eij >= 0 ? expf(s * inv - p.lse[(int64_t)i * H + h]) : 0.0f;
      dsv[h] = eij >= 0 ? p.ds[eij * H + h] : 0.0f;
    }
    const float* Gi = p.grad + (int64_t)i * K * C;
    rot_apply<L>(D, [&](int idx) { return Gi[idx]; }, xt, C);
    radial<L>(rbf, w_rad, rho, C);
    __syncthreads();
    // dy = rho * D (alpha G_i): alpha is constant over the components
    for (int e = tid; e < K * C; e += blockDim.x) {
      const int c = e % C;
      xt[e] *= rho[degree_of(e / C) * C + c] * alpha[c / dh];
    }
    __syncthreads();
    so2_transpose<L>(xt, yt, w_so2, woff, C);
    __syncthreads();
    rot_apply_t<L, true>(D, yt, acc, C);
    for (int c = tid; c < C; c += blockDim.x) dka[c] += dsv[c / dh] * qi[c] * inv;
    __syncthreads();
  }
  // dh_j = values + (l = 0) dq_j W_q^T + dk_j W_k^T
  for (int e = tid; e < K * C; e += blockDim.x) {
    float v = acc[e];
    if (e < C) {
      for (int cp = 0; cp < C; ++cp)
        v += p.dq[j * C + cp] * load_as_f32(w_q, (size_t)e * C + cp) + dka[cp] * load_as_f32(w_k, (size_t)e * C + cp);
    }
    p.grad_feat[j * K * C + e] = v;
  }
}

// delta_i^h = sum_{k, c in h} G_i o_i: one workgroup per atom, one thread
// per channel (coalesced rows), then a sum over each head's channels.
__global__ void k_bwd_delta(const float* __restrict__ grad, const float* __restrict__ out, int K, int C, int H,
                            float* __restrict__ delta) {
  extern __shared__ float sc[];
  const int64_t i = blockIdx.x;
  const int dh = C / H;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float v = 0.0f;
    for (int kk = 0; kk < K; ++kk) v += grad[(i * K + kk) * C + c] * out[(i * K + kk) * C + c];
    sc[c] = v;
  }
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float v = 0.0f;
    for (int c = h * dh; c < (h + 1) * dh; ++c) v += sc[c];
    delta[i * H + h] = v;
  }
}

// W_q^T and W_k^T in fp32, so that the l = 0 terms read them by rows.
template <typename T>
__global__ void k_wqk_transpose(const T* __restrict__ w_q, const T* __restrict__ w_k, int C, float* __restrict__ wt) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)C * C) return;
  const int64_t c = t / C, cp = t % C;
  wt[cp * C + c] = load_as_f32(w_q, t);
  wt[(int64_t)C * C + cp * C + c] = load_as_f32(w_k, t);
}

// The l = 0 terms of the gradient after the matrix-core passes, in two
// launches.  First one workgroup per atom j: dq_j = sum_{j' in N(j)} ds_jj'
// k_j' / sqrt(C/H), dk_j = sum_{i in N(j)} ds_ij q_i / sqrt(C/H) (ds_ij found
// in the ascending row of i, once per edge, in tiles of blockDim edges), into
// dqo and dko (wdq, wdk when the weight gradients want them, else scratch).
// The edges of a tile are split over G = blockDim / C thread groups (one
// channel per thread; G = 1 and several channels per thread when C exceeds
// blockDim), two edges in flight per thread, and the groups' sums meet in
// LDS.  Then, when grad_feat is set, grad_feat[j][0] += dq_j W_q^T +
// dk_j W_k^T over tiles of kQkAtoms atoms, which share each read of W_q^T
// and W_k^T (wt).
__global__ void __launch_bounds__(256) k_bwd_qk(BwdParams p, float* __restrict__ dqo, float* __restrict__ dko) {
  const int C = p.C, H = p.H, dh = C / H;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int G = C <= nthr ? nthr / C : 1;          // edge groups
  const int g = tid / C, c0 = tid - g * C;         // this thread's group and channel (G > 1)
  extern __shared__ float smem[];
  float* part = smem;                              // [2][G][C] group sums (G > 1); [2][C] sums (G = 1)
  int64_t* rev = reinterpret_cast<int64_t*>(smem + 2 * (G > 1 ? nthr : C));   // [blockDim]: j in row i, or -1
  const int64_t j = blockIdx.x;
  const float inv = 1.0f / sqrtf(static_cast<float>(dh));
  const int64_t t0 = p.row_ptr[j], t1 = p.row_ptr[j + 1];
  if (G == 1)
    for (int c = tid; c < C; c += nthr) part[c] = part[C + c] = 0.0f;
  float aq = 0.0f, ak = 0.0f;
  for (int64_t base = t0; base < t1; base += nthr) {
    const int64_t t = base + tid;
    if (t < t1) {
      const int i = p.col[t];
      const int64_t end = p.row_ptr[i + 1];
      int64_t lo = p.row_ptr[i], hi = end;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (p.col[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      rev[tid] = (lo < end && p.col[lo] == j) ? lo : -1;
    }
    __syncthreads();
    const int nt = t1 - base < (int64_t)nthr ? static_cast<int>(t1 - base) : nthr;
    if (G > 1) {
      if (g < G) {
        const int h = c0 / dh;
        int u = g;
        for (; u + G < nt; u += 2 * G) {   // two edges' loads in flight
          const int i0 = p.col[base + u], i1 = p.col[base + u + G];
          const int64_t e0 = rev[u], e1 = rev[u + G];
          const float s0 = p.ds[(base + u) * H + h], s1 = p.ds[(base + u + G) * H + h];
          const float k0 = p.k[(int64_t)i0 * C + c0], k1 = p.k[(int64_t)i1 * C + c0];
          const float r0 = e0 >= 0 ? p.ds[e0 * H + h] * p.q[(int64_t)i0 * C + c0] : 0.0f;
          const float r1 = e1 >= 0 ? p.ds[e1 * H + h] * p.q[(int64_t)i1 * C + c0] : 0.0f;
          aq += s0 * k0;
          ak += r0;
          aq += s1 * k1;
          ak += r1;
        }
        if (u < nt) {
          const int i = p.col[base + u];
          aq += p.ds[(base + u) * H + h] * p.k[(int64_t)i * C + c0];
          const int64_t e = rev[u];
          if (e >= 0) ak += p.ds[e * H + h] * p.q[(int64_t)i * C + c0];
        }
      }
    } else {
      for (int c = tid; c < C; c += nthr) {   // each thread owns its channels' sums
        const int h = c / dh;
        float sq = 0.0f, sk = 0.0f;
        for (int u = 0; u < nt; ++u) {
          const int i = p.col[base + u];
          sq += p.ds[(base + u) * H + h] * p.k[(int64_t)i * C + c];
          const int64_t e = rev[u];
          if (e >= 0) sk += p.ds[e * H + h] * p.q[(int64_t)i * C + c];
        }
        part[c] += sq;
        part[C + c] += sk;
      }
    }
    __syncthreads();
  }
  if (G > 1) {
    if (g < G) {
      part[g * C + c0] = aq;
      part[(G + g) * C + c0] = ak;
    }
    __syncthreads();
    for (int c = tid; c < C; c += nthr) {
      float sq = 0.0f, sk = 0.0f;
      for (int q = 0; q < G; ++q) {
        sq += part[q * C + c];
        sk += part[(G + q) * C + c];
      }
      dqo[j * C + c] = sq * inv;
      dko[j * C + c] = sk * inv;
    }
  } else {
    for (int c = tid; c < C; c += nthr) {
      dqo[j * C + c] = part[c] * inv;
      dko[j * C + c] = part[C + c] * inv;
    }
  }
}

// grad_feat[j][0] += dq_j W_q^T + dk_j W_k^T for kQkAtoms atoms per
// workgroup: the atoms' dq, dk rows in LDS, W_q^T and W_k^T (wt) read once
// per thread group; group g (G = blockDim / C of them, one channel per
// thread) takes atoms g, g + G, ... (at most kQkRows); with C beyond
// blockDim each thread takes channels tid, tid + blockDim, ... atom by atom.
constexpr int kQkAtoms = 32;
constexpr int kQkRows = 16;
__global__ void __launch_bounds__(256) k_bwd_qk_proj(const float* __restrict__ dqo, const float* __restrict__ dko,
                                                     const float* __restrict__ wt, int64_t n, int C, int K,
                                                     float* __restrict__ grad_feat) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int G = C <= nthr ? nthr / C : 1;
  const int g = tid / C, c0 = tid - g * C;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int64_t j0 = (int64_t)blockIdx.x * kQkAtoms;
  const int na = n - j0 < kQkAtoms ? static_cast<int>(n - j0) : kQkAtoms;
  const float* wqt = wt;
  const float* wkt = wt + (size_t)C * C;
  if (G > 1) {
    float* dq = smem;                 // [kQkAtoms][C]
    float* dk = smem + kQkAtoms * C;  // [kQkAtoms][C]
    for (int t = tid; t < na * C; t += nthr) {
      dq[t] = dqo[j0 * C + t];
      dk[t] = dko[j0 * C + t];
    }
    __syncthreads();
    if (g >= G) return;
    float acc[kQkRows];
#pragma unroll
    for (int r = 0; r < kQkRows; ++r) acc[r] = 0.0f;
    int cp = 0;
    if (C % 4 == 0)   // four k at a time: one 16-byte LDS read per row and matrix
      for (; cp < C; cp += 4) {
        float wq[4], wk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wq[u] = wqt[(size_t)(cp + u) * C + c0];
          wk[u] = wkt[(size_t)(cp + u) * C + c0];
        }
#pragma unroll
        for (int r = 0; r < kQkRows; ++r) {
          const int a = g + r * G;
          if (a < na) {
            const float4 q4 = *reinterpret_cast<const float4*>(dq + a * C + cp);
            const float4 k4 = *reinterpret_cast<const float4*>(dk + a * C + cp);
            acc[r] += q4.x * wq[0] + k4.x * wk[0];
            acc[r] += q4.y * wq[1] + k4.y * wk[1];
            acc[r] += q4.z * wq[2] + k4.z * wk[2];
            acc[r] += q4.w * wq[3] + k4.w * wk[3];
          }
        }
      }
    for (; cp < C; ++cp) {
      const float wq = wqt[(size_t)cp * C + c0], wk = wkt[(size_t)cp * C + c0];
#pragma unroll
      for (int r = 0; r < kQkRows; ++r) {
        const int a = g + r * G;
        if (a < na) acc[r] += dq[a * C + cp] * wq + dk[a * C + cp] * wk;
      }
    }
#pragma unroll
    for (int r = 0; r < kQkRows; ++r) {
      const int a = g + r * G;
      if (a < na) grad_feat[(j0 + a) * K * C + c0] += acc[r];
    }
  } else {
    for (int a = 0; a < na; ++a)
      for (int c = tid; c < C; c += nthr) {
        float v = 0.0f;
        for (int cp = 0; cp < C; ++cp)
          v += dqo[(j0 + a) * C + cp] * wqt[(size_t)cp * C + c] + dko[(j0 + a) * C + cp] * wkt[(size_t)cp * C + c];
        grad_feat[(j0 + a) * K * C + c] += v;
      }
  }
}

BwdParams bwd_params(const BwdPlan& pl) {
  const e2a_attn_args* a = pl.a;
  BwdParams p{};
  p.pos = a->pos;
  p.row_ptr = a->row_ptr;
  p.col = a->col;
  p.q = pl.q;
  p.k = pl.k;
  p.out = a->out;
  p.lse = a->out_lse;
  p.grad = pl.grad_out;
  p.ds = pl.ds;
  p.dq = pl.dq;
  p.grad_feat = pl.grad_feat;
  p.wdq = pl.wdq;
  p.wdk = pl.wdk;
  for (int d = 0; d < 3; ++d) p.box[d] = pl.box[d];
  p.periodic = pl.periodic;
  p.cutoff = a->cutoff;
  p.C = a->C;
  p.H = a->H;
  return p;
}

template <int L, typename T>
e2a_status launch_bwd_typed(const BwdPlan& pl, hipStream_t s) {
  const e2a_attn_args* a = pl.a;
  constexpr int K = (L + 1) * (L + 1);
  const BwdParams p = bwd_params(pl);
  const size_t smem = sizeof(float) * (3 * K * a->C + (L + 1) * a->C + 3 * a->C + wig_size(L) + 3 * a->H);
  if (smem > 160 * 1024) return fail(E2A_ERR_UNSUPPORTED, "backward kernels: C=%d too large for LDS", a->C);
  hipLaunchKernelGGL((k_bwd_query<L, T>), dim3(a->n_atoms), dim3(256), smem, s, p, static_cast<const T*>(a->feat),
                     static_cast<const T*>(a->w_rad), static_cast<const T*>(a->w_so2));
  E2A_LAUNCH_CHECK();
  if (pl.grad_feat) {
    hipLaunchKernelGGL((k_bwd_value<L, T>), dim3(a->n_atoms), dim3(256), smem, s, p, static_cast<const T*>(a->w_q),
                       static_cast<const T*>(a->w_k), static_cast<const T*>(a->w_rad),
                       static_cast<const T*>(a->w_so2));
    E2A_LAUNCH_CHECK();
  }
  if (pl.wdq) {
    // dq, dk for the weight gradients (the value pass adds its own l = 0 terms)
    BwdPlan qk = pl;
    qk.grad_feat = nullptr;
    return launch_bwd_qk(qk, s);
  }
  return E2A_OK;
}

template <typename T>
e2a_status launch_bwd_dtype(const BwdPlan& pl, hipStream_t s) {
  switch (pl.a->L) {
    case 0: return launch_bwd_typed<0, T>(pl, s);
    case 1: return launch_bwd_typed<1, T>(pl, s);
    case 2: return launch_bwd_typed<2, T>(pl, s);
    case 3: return launch_bwd_typed<3, T>(pl, s);
    case 4: return launch_bwd_typed<4, T>(pl, s);
    default: return fail(E2A_ERR_UNSUPPORTED, "L=%d", pl.a->L);
  }
}

}  // namespace

e2a_status launch_bwd_delta(const BwdPlan& pl, float* delta, hipStream_t s) {
  const e2a_attn_args* a = pl.a;
  const int K = (a->L + 1) * (a->L + 1);
  k_bwd_delta<<<a->n_atoms, 128, sizeof(float) * a->C, s>>>(pl.grad_out, a->out, K, a->C, a->H, delta);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

e2a_status launch_bwd_qk(const BwdPlan& pl, hipStream_t s) {
  const e2a_attn_args* a = pl.a;
  const int K = (a->L + 1) * (a->L + 1);
  const BwdParams p = bwd_params(pl);
  const int64_t cc = (int64_t)a->C * a->C;
  if (a->dtype == E2A_DTYPE_BF16)
    hipLaunchKernelGGL(k_wqk_transpose<uint16_t>, dim3((cc + 255) / 256), dim3(256), 0, s,
                       static_cast<const uint16_t*>(a->w_q), static_cast<const uint16_t*>(a->w_k), a->C, pl.wqkt);
  else
    hipLaunchKernelGGL(k_wqk_transpose<float>, dim3((cc + 255) / 256), dim3(256), 0, s,
                       static_cast<const float*>(a->w_q), static_cast<const float*>(a->w_k), a->C, pl.wqkt);
  E2A_LAUNCH_CHECK();
  // dq, dk to the weight gradients' arrays, or to scratch when only dL/dh wants them
  float* dqo = pl.wdq ? pl.wdq : pl.dq;
  float* dko = pl.wdk ? pl.wdk : pl.dk;
  const int G = a->C <= 256 ? 256 / a->C : 1;
  const size_t smem = sizeof(float) * 2 * (G > 1 ? 256 : (size_t)a->C) + sizeof(int64_t) * 256;
  if (smem > 64 * 1024) return fail(E2A_ERR_UNSUPPORTED, "l = 0 gradient terms: C=%d too large for LDS", a->C);
  hipLaunchKernelGGL(k_bwd_qk, dim3(static_cast<unsigned>(a->n_atoms)), dim3(256), smem, s, p, dqo, dko);
  E2A_LAUNCH_CHECK();
  if (pl.grad_feat) {
    const size_t psmem = G > 1 ? sizeof(float) * 2 * kQkAtoms * (size_t)a->C : 0;
    hipLaunchKernelGGL(k_bwd_qk_proj, dim3(static_cast<unsigned>((a->n_atoms + kQkAtoms - 1) / kQkAtoms)), dim3(256),
                       psmem, s, dqo, dko, pl.wqkt, a->n_atoms, a->C, K, pl.grad_feat);
  }
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

e2a_status launch_attention_backward(const BwdPlan& pl, hipStream_t s) {
  if (pl.a->n_atoms == 0) return E2A_OK;
  return pl.a->dtype == E2A_DTYPE_BF16 ? launch_bwd_dtype<uint16_t>(pl, s) : launch_bwd_dtype<float>(pl, s);
}

}  // namespace e2a

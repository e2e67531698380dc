// Scalar (VALU) kernels of the on-the-fly equivariant attention layer:
//   * the q/k prologue from the invariant l = 0 features, and
//   * a reference fused attention kernel for any L <= 4, C, H and for fp32
//     or bf16 storage.
//
// arXiv 2601.16622, English technical summary section 2.2 ("On-the-Fly
// Equivariant Attention"): one workgroup owns one destination atom and
// streams its neighbours j in N(i).  For each neighbour it builds the edge
// frame and its Wigner-D blocks on chip, rotates h_j in, applies the per-m
// SO(2) mix of section 2.1, scales by the radial weights, rotates back and
// folds the result into an online softmax.  Only the running max, the
// normaliser and the value accumulator live across neighbours, all in LDS; no
// per-edge tensor is written to device memory.  With the convolution flag
// (section 2.1: the EAAS convolution stage) every edge weight is 1 and the
// messages are simply summed.
//
// This kernel keeps every product in fp32 on the vector ALUs.  It serves the
// fp32 configurations (where bf16 matrix cores would miss a 1e-5 tolerance)
// and shapes the MFMA kernel is not built for.
#include "e2a_geometry.hpp"
#include "e2a_internal.hpp"

namespace e2a {
namespace {

// q = h0 W_q, k = h0 W_k for 16 atoms per block; thread c owns output channel c.
template <typename T>
__global__ void k_qk(const T* __restrict__ feat, const T* __restrict__ wq, const T* __restrict__ wk,
                     int64_t n, int C, int ncomp, float* __restrict__ q, float* __restrict__ k) {
  extern __shared__ __attribute__((aligned(16))) float h0[];  // [16][C]
  const int64_t i0 = blockIdx.x * 16ll;
  const int nb = (n - i0) < 16 ? static_cast<int>(n - i0) : 16;
  for (int t = threadIdx.x; t < nb * C; t += blockDim.x) {
    const int a = t / C, c = t % C;
    h0[a * C + c] = load_as_f32(feat, (size_t)(i0 + a) * ncomp * C + c);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float aq[16], ak[16];
#pragma unroll
    for (int a = 0; a < 16; ++a) { aq[a] = 0.0f; ak[a] = 0.0f; }
    // four input channels per step: one 16-byte LDS read per atom instead of
    // four (the sums still run over cp in order)
    int cp = 0;
    if (C % 4 == 0) {
#pragma unroll 2
      for (; cp < C; cp += 4) {
        float wqv[4], wkv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wqv[u] = load_as_f32(wq, (size_t)(cp + u) * C + c);
          wkv[u] = load_as_f32(wk, (size_t)(cp + u) * C + c);
        }
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const float4 hv = *reinterpret_cast<const float4*>(h0 + (a < nb ? a : 0) * C + cp);
          aq[a] += hv.x * wqv[0];
          ak[a] += hv.x * wkv[0];
          aq[a] += hv.y * wqv[1];
          ak[a] += hv.y * wkv[1];
          aq[a] += hv.z * wqv[2];
          ak[a] += hv.z * wkv[2];
          aq[a] += hv.w * wqv[3];
          ak[a] += hv.w * wkv[3];
        }
      }
    }
    for (; cp < C; ++cp) {
      const float wqv = load_as_f32(wq, (size_t)cp * C + c);
      const float wkv = load_as_f32(wk, (size_t)cp * C + c);
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float hv = h0[(a < nb ? a : 0) * C + cp];
        aq[a] += hv * wqv;
        ak[a] += hv * wkv;
      }
    }
    for (int a = 0; a < nb; ++a) {
      q[(i0 + a) * C + c] = aq[a];
      k[(i0 + a) * C + c] = ak[a];
    }
  }
}

struct RefParams {
  const float* pos;
  const int64_t* row_ptr;
  const int32_t* col;
  const float* q;
  const float* k;
  float* out;
  float* out_lse;
  float box[3];
  int periodic;
  float cutoff;
  int C, H;
  int conv;   // convolution: every edge weight 1, no normaliser
};

template <int L, typename T>
__global__ void __launch_bounds__(256) k_attention_reference(RefParams p, const T* __restrict__ feat,
                                                              const T* __restrict__ w_rad,
                                                              const T* __restrict__ w_so2) {
  constexpr int K = (L + 1) * (L + 1);
  constexpr int NW = wig_size(L);
  const int C = p.C, H = p.H, dh = C / H;
  extern __shared__ float smem[];
  float* xt = smem;              // [K][C] rotated-in features
  float* yt = xt + K * C;        // [K][C] SO(2)-mixed features
  float* acc = yt + K * C;       // [K][C] value accumulator
  float* rho = acc + K * C;      // [L+1][C]
  float* qi = rho + (L + 1) * C; // [C]
  float* D = qi + C;             // [NW]
  float* st = D + NW;            // [H] scale, [H] p, [H] m, [H] l
  float* sp = st + H;
  float* sm = sp + H;
  float* sl = sm + H;
  __shared__ float rbf[8];
  __shared__ int jsh;

  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const float inv_sqrt_dh = 1.0f / sqrtf(static_cast<float>(dh));

  for (int t = tid; t < K * C; t += blockDim.x) acc[t] = 0.0f;
  if (!p.conv)
    for (int t = tid; t < C; t += blockDim.x) qi[t] = p.q[i * C + t];
  for (int t = tid; t < H; t += blockDim.x) { sm[t] = -INFINITY; sl[t] = 0.0f; }
  const float xi[3] = {p.pos[3 * i], p.pos[3 * i + 1], p.pos[3 * i + 2]};
  __syncthreads();

  // offsets of the per-m weight blocks in the logical layout
  int64_t woff[L + 1];
  {
    int64_t o = 0;
#pragma unroll
    for (int m = 0; m <= L; ++m) {
      woff[m] = o;
      const int64_t km = (int64_t)(L + 1 - m) * C;
      o += (m == 0 ? 1 : 2) * km * km;
    }
  }

  const int64_t e0 = p.row_ptr[i], e1 = p.row_ptr[i + 1];
  for (int64_t e = e0; e < e1; ++e) {
    if (tid == 0) {
      const int j = p.col[e];
      jsh = j;
      float r3[3];
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        float dx = p.pos[3 * (int64_t)j + d] - xi[d];
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
    // threads 64.. take the heads in turn (any H), while thread 0 builds the
    // edge's geometry
    for (int h = tid - 64; tid >= 64 && h < H; h += static_cast<int>(blockDim.x) - 64) {
      if (p.conv) {
        // convolution: weight 1 for every edge, nothing to rescale
        sl[h] = 1.0f;
        sm[h] = 0.0f;
        st[h] = 1.0f;
        sp[h] = 1.0f;
        continue;
      }
      const int j = p.col[e];
      float s = 0.0f;
      for (int d = 0; d < dh; ++d) s += qi[h * dh + d] * p.k[(int64_t)j * C + h * dh + d];
      s *= inv_sqrt_dh;
      const float mo = sm[h];
      const float mn = fmaxf(mo, s);
      const float sc = expf(mo - mn);
      const float pe = expf(s - mn);
      sl[h] = sl[h] * sc + pe;
      sm[h] = mn;
      st[h] = sc;
      sp[h] = pe;
    }
    __syncthreads();
    const int j = jsh;
    const T* hj = feat + (int64_t)j * K * C;
    // rotate in: x^l = D^l h_j^l
    for (int t = tid; t < K * C; t += blockDim.x) {
      const int comp = t / C, c = t % C;
      int l = 0;
      while ((l + 1) * (l + 1) <= comp) ++l;
      const int mi = comp - l * l;  // m + l
      const float* Dl = D + wig_off(l) + mi * (2 * l + 1);
      float v = 0.0f;
      for (int n2 = 0; n2 < 2 * l + 1; ++n2) v += Dl[n2] * load_as_f32(hj, (size_t)(l * l + n2) * C + c);
      xt[t] = v;
    }
    for (int t = tid; t < (L + 1) * C; t += blockDim.x) {
      float v = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) v += rbf[kk] * load_as_f32(w_rad, (size_t)kk * (L + 1) * C + t);
      rho[t] = v;
    }
    __syncthreads();
    // per-m SO(2) mix
    for (int t = tid; t < K * C; t += blockDim.x) {
      const int comp = t / C, co = t % C;
      int lo = 0;
      while ((lo + 1) * (lo + 1) <= comp) ++lo;
      const int m = comp - lo * lo - lo;
      const int am = m < 0 ? -m : m;
      const int64_t km = (int64_t)(L + 1 - am) * C;
      float y = 0.0f;
      if (am == 0) {
        const T* W0 = w_so2 + woff[0];
        for (int li = 0; li <= L; ++li) {
          const float* xr = xt + (li * li + li) * C;
          const T* wr = W0 + (int64_t)(li * C) * km + (int64_t)lo * C + co;
          for (int ci = 0; ci < C; ++ci) y += xr[ci] * load_as_f32(wr, (size_t)ci * km);
        }
      } else {
        const T* W1 = w_so2 + woff[am];
        const T* W2 = W1 + km * km;
        for (int li = am; li <= L; ++li) {
          const float* xp = xt + (li * li + li + am) * C;
          const float* xm = xt + (li * li + li - am) * C;
          const int64_t rbase = (int64_t)((li - am) * C) * km + (int64_t)(lo - am) * C + co;
          for (int ci = 0; ci < C; ++ci) {
            const float w1 = load_as_f32(W1, rbase + (size_t)ci * km);
            const float w2 = load_as_f32(W2, rbase + (size_t)ci * km);
            y += (m > 0) ? (xp[ci] * w1 - xm[ci] * w2) : (xp[ci] * w2 + xm[ci] * w1);
          }
        }
      }
      yt[t] = y;
    }
    __syncthreads();
    // radial scale, rotate out (v^l = D^l^T yhat^l), online-softmax accumulate
    for (int t = tid; t < K * C; t += blockDim.x) {
      const int comp = t / C, c = t % C;
      int l = 0;
      while ((l + 1) * (l + 1) <= comp) ++l;
      const int ni = comp - l * l;  // m' + l
      const float* Dl = D + wig_off(l);
      float v = 0.0f;
      for (int mi = 0; mi < 2 * l + 1; ++mi) v += Dl[mi * (2 * l + 1) + ni] * yt[(l * l + mi) * C + c];
      v *= rho[l * C + c];
      const int h = c / dh;
      acc[t] = acc[t] * st[h] + sp[h] * v;
    }
    __syncthreads();
  }
  // epilogue
  for (int t = tid; t < K * C; t += blockDim.x) {
    const int h = (t % C) / dh;
    const float l = sl[h];
    p.out[i * K * C + t] = l > 0.0f ? acc[t] / l : 0.0f;
  }
  if (p.out_lse)
    for (int t = tid; t < H; t += blockDim.x) p.out_lse[i * H + t] = sl[t] > 0.0f ? sm[t] + logf(sl[t]) : -INFINITY;
}

template <int L, typename T>
e2a_status launch_ref_typed(const AttnPlan& pl, hipStream_t s) {
  const e2a_attn_args* a = pl.a;
  RefParams p{};
  p.pos = a->pos;
  p.row_ptr = a->row_ptr;
  p.col = a->col;
  p.q = pl.q;
  p.k = pl.k;
  p.out = a->out;
  p.out_lse = pl.conv ? nullptr : a->out_lse;
  p.conv = pl.conv ? 1 : 0;
  for (int d = 0; d < 3; ++d) p.box[d] = pl.box[d];
  p.periodic = pl.periodic;
  p.cutoff = a->cutoff;
  p.C = a->C;
  p.H = a->H;
  constexpr int K = (L + 1) * (L + 1);
  const size_t smem = sizeof(float) * (3 * K * a->C + (L + 1) * a->C + a->C + wig_size(L) + 4 * a->H);
  if (smem > 160 * 1024) return fail(E2A_ERR_UNSUPPORTED, "reference kernel: C=%d too large for LDS", a->C);
  if (a->n_atoms == 0) return E2A_OK;
  hipLaunchKernelGGL((k_attention_reference<L, T>), dim3(a->n_atoms), dim3(256), smem, s, p,
                     static_cast<const T*>(a->feat), static_cast<const T*>(a->w_rad),
                     static_cast<const T*>(a->w_so2));
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

template <typename T>
e2a_status launch_ref_dtype(const AttnPlan& pl, hipStream_t s) {
  switch (pl.a->L) {
    case 0: return launch_ref_typed<0, T>(pl, s);
    case 1: return launch_ref_typed<1, T>(pl, s);
    case 2: return launch_ref_typed<2, T>(pl, s);
    case 3: return launch_ref_typed<3, T>(pl, s);
    case 4: return launch_ref_typed<4, T>(pl, s);
    default: return fail(E2A_ERR_UNSUPPORTED, "L=%d", pl.a->L);
  }
}

}  // namespace

e2a_status launch_qk(const AttnPlan& pl, hipStream_t s) {
  const e2a_attn_args* a = pl.a;
  if (a->n_atoms == 0) return E2A_OK;
  const int ncomp = (a->L + 1) * (a->L + 1);
  if (block_uses_mfma(a->C, a->dtype))
    return launch_qk_mfma(static_cast<const uint16_t*>(a->feat), static_cast<const uint16_t*>(a->w_q),
                          static_cast<const uint16_t*>(a->w_k), pl.wqk_t, a->n_atoms, ncomp, a->C, pl.q, pl.k, s);
  const int threads = std::min(256, ((a->C + 63) / 64) * 64);
  const dim3 grid((a->n_atoms + 15) / 16);
  const size_t smem = sizeof(float) * 16 * a->C;
  if (a->dtype == E2A_DTYPE_BF16)
    hipLaunchKernelGGL(k_qk<uint16_t>, grid, dim3(threads), smem, s, static_cast<const uint16_t*>(a->feat),
                       static_cast<const uint16_t*>(a->w_q), static_cast<const uint16_t*>(a->w_k), a->n_atoms,
                       a->C, ncomp, pl.q, pl.k);
  else
    hipLaunchKernelGGL(k_qk<float>, grid, dim3(threads), smem, s, static_cast<const float*>(a->feat),
                       static_cast<const float*>(a->w_q), static_cast<const float*>(a->w_k), a->n_atoms, a->C,
                       ncomp, pl.q, pl.k);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

e2a_status launch_attention_reference(const AttnPlan& pl, hipStream_t s) {
  if (pl.a->dtype == E2A_DTYPE_BF16) return launch_ref_dtype<uint16_t>(pl, s);
  return launch_ref_dtype<float>(pl, s);
}

}  // namespace e2a

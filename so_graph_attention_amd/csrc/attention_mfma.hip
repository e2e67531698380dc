// Fused on-the-fly equivariant attention on the gfx950 matrix cores.
//
// arXiv 2601.16622, English technical summary section 2.2 ("On-the-Fly
// Equivariant Attention"): the layer is node-centric.  A workgroup owns one
// destination atom i and streams its neighbour list in chunks of 32 edges;
// the running max, normaliser and value accumulator of the online softmax
// stay on chip across chunks, and no per-edge tensor reaches device memory.
// Section 2.1 ("Equivariant Axis-Aligned Sparsification"): each edge's
// features are rotated into the frame where the edge is the z axis, the
// dense tensor product becomes one block GEMM per |m| (the SO(2) mix), and the
// result is rotated back.
//
// Mapping onto CDNA4 (C = 128, H = 8, bf16 storage, fp32 accumulation):
//   * per chunk, 32 lanes build the edge frames, D^1 and the radial basis;
//     all 256 threads then extend D^2..D^L level by level (one matrix entry
//     per thread per step) and compute the 32 x 8 logits;
//   * per |m| block the 256 threads rotate h_j into the aligned frame and
//     write the GEMM operand A (rows = edges, and for m > 0 the +m rows of 16
//     edges followed by their -m rows) to LDS as bf16;
//   * wave w owns output channels [32 w, 32 w + 32) of every l_out and runs
//     v_mfma_f32_32x32x16_bf16 over K = (L+1-m) C with B fragments streamed
//     from a pre-packed weight image (one 16-byte load per lane per k-step);
//   * the epilogue combines the W1/W2 products into y_{+m}, y_{-m} (both rows
//     of an edge land in the same lane), scales by alpha and by the radial
//     weights (one extra MFMA against the radial basis), and folds the partial
//     rotate-out D^T of this |m| into per-lane accumulators for all (l, m').
#include "e2a_geometry.hpp"
#include "e2a_internal.hpp"

namespace e2a {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kC = 128;      // channels
constexpr int kH = 8;        // heads
constexpr int kDH = 16;      // channels per head
constexpr int kET = 32;      // edges per chunk
constexpr int kThreads = 256;

// Wigner-D rows in LDS are padded to a multiple of 4 floats (16-byte reads).
__host__ __device__ constexpr int dpad(int l) { return ((2 * l + 1) + 3) / 4 * 4; }
__host__ __device__ constexpr int doff(int l) {
  int o = 0;
  for (int k = 0; k < l; ++k) o += (2 * k + 1) * dpad(k);
  return o;
}

template <int L>
struct Shape {
  static constexpr int K = (L + 1) * (L + 1);
  static constexpr int DSZ = doff(L + 1);                       // fp32 D floats per edge
  static constexpr int DT = wig_size(L) * kET;                  // fp16 transposed D, [entry][edge]
  static constexpr int km(int m) { return (L + 1 - m) * kC; }   // GEMM K (= N) of block m
  static constexpr int astride(int m) { return km(m) + 8; }     // bf16 per A row (padded)
  static constexpr int arows(int m) { return m == 0 ? kET : 2 * kET; }
  static constexpr int abytes(int m) { return arows(m) * astride(m) * 2; }
  static constexpr int amax() {
    int b = 0;
    for (int m = 0; m <= L; ++m) b = abytes(m) > b ? abytes(m) : b;
    return b;
  }
  static constexpr int fps(int m) { return m == 0 ? 1 : 2; }   // B fragments per k-step
  // packed weight image, in 16-byte vectors: for m, for l_out - m, for wave, for k-step, for W, lane
  static constexpr int64_t wblock(int m) { return (int64_t)(km(m) / 16) * fps(m) * 64; }
  static constexpr int64_t woff(int m) {
    int64_t o = 0;
    for (int k = 0; k < m; ++k) o += (int64_t)(L + 1 - k) * 4 * wblock(k);
    return o;
  }
  static constexpr int64_t wtotal() { return woff(L + 1); }
  // logical layout offsets (elements)
  static constexpr int64_t loff(int m) {
    int64_t o = 0;
    for (int k = 0; k < m; ++k) o += (int64_t)fps(k) * km(k) * km(k);
    return o;
  }
  // LDS layout (bytes)
  static constexpr int off_D = amax();
  static constexpr int off_DT = off_D + kET * DSZ * 4;
  static constexpr int off_rbf = off_DT + DT * 2;
  static constexpr int off_alpha = off_rbf + kET * 8 * 4;
  static constexpr int off_q = off_alpha + kET * kH * 4;
  static constexpr int off_j = off_q + kC * 4;
  static constexpr int off_stat = off_j + kET * 4;
  static constexpr int total = off_stat + 3 * kH * 4;
};

template <typename V>
__device__ __forceinline__ V to_vec8(const float* x) {
  f32x8 v;
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = x[q];
  return __builtin_convertvector(v, V);
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 raw, float* h) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    h[2 * t] = __uint_as_float(w[t] << 16);
    h[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
  }
}

// Hides a value's origin from the optimiser so that lane-dependent addresses
// are recomputed where they are used instead of being hoisted out of the edge
// loop and kept live in registers for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(const f16x8 a, const f16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of a 32x32 MFMA result held by accumulator register r of a lane in
// half h (lanes 0-31: h = 0, lanes 32-63: h = 1); the column is lane % 32.
__device__ __forceinline__ constexpr int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

struct MfmaParams {
  const float* pos;
  const int64_t* row_ptr;
  const int32_t* col;
  const float* q;
  const float* k;
  const uint16_t* feat;
  const bf16x8* wpk;
  const f16x8* radpk;
  float* out;
  float* out_lse;
  float box[3];
  int periodic;
  float cutoff;
};

struct Smem {
  uint16_t* A;
  float* D;
  _Float16* DT;
  float* rbf;
  float* alpha;
  float* q;
  int* j;
  float* m_run;
  float* l_run;
  float* scale;
};

// Rotate the chunk's neighbour features into the edge frames and write the
// GEMM operand of block M (bf16, padded rows) to LDS.
template <int L, int M>
__device__ __forceinline__ void build_a(const MfmaParams& p, const Smem& s, int tid) {
  using S = Shape<L>;
  constexpr int NL = L + 1 - M;
  constexpr int stride = S::astride(M);
  tid = opaque(tid);
#pragma unroll 1
  for (int t = tid; t < kET * NL * 16; t += kThreads) {
    const int g = t & 15;
    const int el = t >> 4;
    const int e = el / NL;
    const int l = M + el % NL;
    const uint16_t* hp = p.feat + ((int64_t)s.j[e] * S::K + l * l) * kC + 8 * g;
    const float* De = s.D + e * S::DSZ + doff(l);
    const float* Dp = De + (l + M) * dpad(l);
    const float* Dm = De + (l - M) * dpad(l);
    float xp[8], xm[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) { xp[q] = 0.0f; xm[q] = 0.0f; }
    for (int n = 0; n < 2 * l + 1; ++n) {
      float hv[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(hp + n * kC), hv);
      const float dp = Dp[n];
#pragma unroll
      for (int q = 0; q < 8; ++q) xp[q] += dp * hv[q];
      if (M > 0) {
        const float dm = Dm[n];
#pragma unroll
        for (int q = 0; q < 8; ++q) xm[q] += dm * hv[q];
      }
    }
    if (M == 0) {
      *reinterpret_cast<bf16x8*>(s.A + e * stride + l * kC + 8 * g) = to_vec8<bf16x8>(xp);
    } else {
      const int row = 32 * (e >> 4) + (e & 15);
      const int colk = (l - M) * kC + 8 * g;
      *reinterpret_cast<bf16x8*>(s.A + row * stride + colk) = to_vec8<bf16x8>(xp);
      *reinterpret_cast<bf16x8*>(s.A + (row + 16) * stride + colk) = to_vec8<bf16x8>(xm);
    }
  }
}

// A operand of the rotate-out contraction: row n of D^l rows `mrow`, for the
// 8 edges eg + crow(q, h), q = 0..7, as fp16.  Rows n >= 2l+1 are zero.
__device__ __forceinline__ f16x8 dt_frag(const _Float16* row_base, int eg, int h, bool valid) {
  f16x8 v = {};
  if (valid) {
    const f16x4 a = *reinterpret_cast<const f16x4*>(row_base + eg + 4 * h);
    const f16x4 b = *reinterpret_cast<const f16x4*>(row_base + eg + 8 + 4 * h);
    v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  return v;
}

// GEMM of block M for this wave's 32 output channels, then the epilogue:
// y_{+-m} from the W1/W2 products, u = alpha * rho * y (rho from one MFMA
// against the radial basis), and the partial rotate-out
// acc_lo[n][c] += sum_{edges, +-} D^lo[lo +- M][n] u_{+-}[c], itself an MFMA
// contraction over the chunk's edges.
template <int L, int M>
__device__ __forceinline__ void mma_block(const MfmaParams& p, const Smem& s, int lane, int wave,
                                          const f16x8 (&arbf)[3], const float (&alpha)[16],
                                          f32x16 (&nacc)[L + 1]) {
  using S = Shape<L>;
  constexpr int KS = S::km(M) / 16;
  constexpr int stride = S::astride(M);
  const f16x8 zero8 = {};
#pragma unroll
  for (int lo = M; lo <= L; ++lo) {
    lane = opaque(lane);
    const int half = lane >> 5;
    const int c_own = 32 * wave + (lane & 31);
    const int row = lane & 31;
    const int kof = 8 * half;
    const bf16x8* bp = p.wpk + S::woff(M) + (int64_t)((lo - M) * 4 + wave) * S::wblock(M) + lane;
    const f16x8 brad = half == 0 ? p.radpk[lo * kC + c_own] : zero8;
    const int n = row;
    const bool nvalid = n < 2 * lo + 1;
    const _Float16* dt_lo = s.DT + wig_off(lo) * kET;
    if (M == 0) {
      f32x16 c0 = {};
      const uint16_t* ap = s.A + row * stride + kof;
#pragma unroll 2
      for (int st = 0; st < KS; ++st) {
        const bf16x8 b = bp[st * 64];
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + st * 16);
        c0 = mfma_bf16(a, b, c0);
      }
      const f32x16 rho = mfma_f16(arbf[0], brad, f32x16{});
      float u[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) u[r] = alpha[r] * rho[r] * c0[r];
      const _Float16* drow = dt_lo + (lo * (2 * lo + 1) + n) * kET;
      nacc[lo] = mfma_f16(dt_frag(drow, 0, half, nvalid), to_vec8<f16x8>(u), nacc[lo]);
      nacc[lo] = mfma_f16(dt_frag(drow, 16, half, nvalid), to_vec8<f16x8>(u + 8), nacc[lo]);
    } else {
      f32x16 c00 = {}, c01 = {}, c10 = {}, c11 = {};
      const uint16_t* ap0 = s.A + row * stride + kof;
      const uint16_t* ap1 = ap0 + 32 * stride;
#pragma unroll 2
      for (int st = 0; st < KS; ++st) {
        const bf16x8 b1 = bp[(2 * st) * 64];
        const bf16x8 b2 = bp[(2 * st + 1) * 64];
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ap0 + st * 16);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ap1 + st * 16);
        c00 = mfma_bf16(a0, b1, c00);
        c01 = mfma_bf16(a0, b2, c01);
        c10 = mfma_bf16(a1, b1, c10);
        c11 = mfma_bf16(a1, b2, c11);
      }
      const _Float16* drow_p = dt_lo + ((lo + M) * (2 * lo + 1) + n) * kET;
      const _Float16* drow_m = dt_lo + ((lo - M) * (2 * lo + 1) + n) * kET;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x16 C1 = t == 0 ? c00 : c10;
        const f32x16 C2 = t == 0 ? c01 : c11;
        const f32x16 rho = mfma_f16(arbf[1 + t], brad, f32x16{});
        float up[8], um[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sc = alpha[r + 8 * t] * rho[r];
          up[r] = sc * (C1[r] - C2[r + 8]);
          um[r] = sc * (C2[r] + C1[r + 8]);
        }
        nacc[lo] = mfma_f16(dt_frag(drow_p, 16 * t, half, nvalid), to_vec8<f16x8>(up), nacc[lo]);
        nacc[lo] = mfma_f16(dt_frag(drow_m, 16 * t, half, nvalid), to_vec8<f16x8>(um), nacc[lo]);
      }
    }
  }
}

template <int L, int M>
__device__ __forceinline__ void do_block(const MfmaParams& p, const Smem& s, int tid, int lane, int wave,
                                         const f16x8 (&arbf)[3], const float (&alpha)[16],
                                         f32x16 (&nacc)[L + 1]) {
  build_a<L, M>(p, s, tid);
  __syncthreads();
  mma_block<L, M>(p, s, lane, wave, arbf, alpha, nacc);
  __syncthreads();
  if constexpr (M < L) do_block<L, M + 1>(p, s, tid, lane, wave, arbf, alpha, nacc);
}

template <int L>
__global__ void __launch_bounds__(kThreads, 1) k_attn_mfma(MfmaParams p) {
  using S = Shape<L>;
  constexpr int K = S::K;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Smem s;
  s.A = reinterpret_cast<uint16_t*>(smem);
  s.D = reinterpret_cast<float*>(smem + S::off_D);
  s.DT = reinterpret_cast<_Float16*>(smem + S::off_DT);
  s.rbf = reinterpret_cast<float*>(smem + S::off_rbf);
  s.alpha = reinterpret_cast<float*>(smem + S::off_alpha);
  s.q = reinterpret_cast<float*>(smem + S::off_q);
  s.j = reinterpret_cast<int*>(smem + S::off_j);
  s.m_run = reinterpret_cast<float*>(smem + S::off_stat);
  s.l_run = s.m_run + kH;
  s.scale = s.l_run + kH;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i = blockIdx.x;

  if (tid < kC) s.q[tid] = p.q[i * kC + tid];
  if (tid < kH) { s.m_run[tid] = -INFINITY; s.l_run[tid] = 0.0f; }
  f32x16 nacc[L + 1];
#pragma unroll
  for (int l = 0; l <= L; ++l) nacc[l] = f32x16{};
  const float xi[3] = {p.pos[3 * i], p.pos[3 * i + 1], p.pos[3 * i + 2]};
  const int64_t e_beg = p.row_ptr[i], e_end = p.row_ptr[i + 1];

  for (int64_t e0 = e_beg; e0 < e_end; e0 += kET) {
    const int ne = (e_end - e0) < kET ? static_cast<int>(e_end - e0) : kET;
    __syncthreads();
    // edge frames, D^0, D^1 and the radial basis: one lane per edge
    if (tid < kET) {
      float* De = s.D + tid * S::DSZ;
      float R[3][3] = {{0, 0, 0}, {0, 0, 0}, {0, 0, 0}};
      float d0 = 0.0f;
      float e8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      int j = static_cast<int>(i);
      if (tid < ne) {
        j = p.col[e0 + tid];
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
        const float r = sqrtf(r3[0] * r3[0] + r3[1] * r3[1] + r3[2] * r3[2]);
        const float u[3] = {r3[0] / r, r3[1] / r, r3[2] / r};
        edge_rotation(u, R);
        d0 = 1.0f;
        radial_basis8(r, p.cutoff, e8);
      }
      s.j[tid] = j;
      De[0] = d0;
      s.DT[tid] = static_cast<_Float16>(d0);
      float D1[9];
      wigner_l1(R, D1, 3);
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          De[doff(1) + a * dpad(1) + b] = D1[3 * a + b];
          s.DT[(wig_off(1) + 3 * a + b) * kET + tid] = static_cast<_Float16>(D1[3 * a + b]);
        }
#pragma unroll
      for (int k = 0; k < 8; ++k) s.rbf[tid * 8 + k] = e8[k];
    }
    // logits s_ij^h = <q_i^h, k_j^h> / sqrt(16): one (edge, head) per thread
    {
      const int e = tid >> 3, h = tid & 7;
      float sv = -INFINITY;
      if (e < ne) {
        const int j = p.col[e0 + e];
        const float4* kp = reinterpret_cast<const float4*>(p.k + (int64_t)j * kC + h * kDH);
        float d = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 kv = kp[t];
          const float* qv = s.q + h * kDH + 4 * t;
          d += kv.x * qv[0] + kv.y * qv[1] + kv.z * qv[2] + kv.w * qv[3];
        }
        sv = d * 0.25f;
      }
      s.alpha[e * kH + h] = sv;
    }
    __syncthreads();
    // online softmax update (one thread per head) while the others extend D
    if (tid < kH) {
      const int h = tid;
      float mx = s.m_run[h];
      for (int e = 0; e < ne; ++e) mx = fmaxf(mx, s.alpha[e * kH + h]);
      const float sc = expf(s.m_run[h] - mx);
      float sum = 0.0f;
      for (int e = 0; e < kET; ++e) {
        const float a = e < ne ? expf(s.alpha[e * kH + h] - mx) : 0.0f;
        s.alpha[e * kH + h] = a;
        sum += a;
      }
      s.l_run[h] = s.l_run[h] * sc + sum;
      s.m_run[h] = mx;
      s.scale[h] = sc;
    }
#pragma unroll
    for (int l = 2; l <= L; ++l) {
      const int w = 2 * l + 1;
#pragma unroll 1
      for (int t = opaque(tid); t < kET * w * w; t += kThreads) {
        const int e = t / (w * w), idx = t % (w * w);
        const int mi = idx / w, ni = idx % w;
        float* De = s.D + e * S::DSZ;
        const float* D1 = De + doff(1);
        const float* Dp = De + doff(l - 1);
        const int pp = dpad(l - 1);
        auto r1 = [&](int a, int b) { return D1[(a + 1) * dpad(1) + (b + 1)]; };
        auto rp = [&](int a, int b) { return Dp[(a + l - 1) * pp + (b + l - 1)]; };
        const float v = ir_entry(l, mi - l, ni - l, r1, rp);
        De[doff(l) + mi * dpad(l) + ni] = v;
        s.DT[(wig_off(l) + idx) * kET + e] = static_cast<_Float16>(v);
      }
      __syncthreads();
    }
    __syncthreads();
    // per-lane constants of this chunk: attention weights of the 16 edges
    // whose rows this lane holds, the radial-basis A operands, and the
    // rescale of the running accumulators
    float alpha[16];
    f16x8 arbf[3];
    {
      const int ln = opaque(lane);
      const int half = ln >> 5;
      const int h_own = (32 * wave + (ln & 31)) / kDH;
#pragma unroll
      for (int r = 0; r < 16; ++r) alpha[r] = s.alpha[crow(r, half) * kH + h_own];
      const float sc = s.scale[h_own];
#pragma unroll
      for (int l = 0; l <= L; ++l) nacc[l] *= sc;
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int r = ln & 31;
      arbf[0] = to_vec8<f16x8>(half == 0 ? s.rbf + r * 8 : z);
      arbf[1] = to_vec8<f16x8>(half == 0 ? s.rbf + (r & 15) * 8 : z);
      arbf[2] = to_vec8<f16x8>(half == 0 ? s.rbf + (16 + (r & 15)) * 8 : z);
    }
    do_block<L, 0>(p, s, tid, lane, wave, arbf, alpha, nacc);
  }
  __syncthreads();
  {
    const int half = lane >> 5;
    const int c_own = 32 * wave + (lane & 31);
    const float l = s.l_run[c_own / kDH];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int lo = 0; lo <= L; ++lo)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = crow(r, half);
        if (n < 2 * lo + 1) p.out[(i * K + lo * lo + n) * kC + c_own] = nacc[lo][r] * inv;
      }
  }
  if (p.out_lse && tid < kH)
    p.out_lse[i * kH + tid] = s.l_run[tid] > 0.0f ? s.m_run[tid] + logf(s.l_run[tid]) : -INFINITY;
}

// Logical SO(2) weights -> B-fragment image: vector v holds, for lane
// v % 64 of one k-step, the 8 values W[k0 .. k0+7][n] with k0 = 16 s + 8 (lane/32)
// and n = (l_out - m) C + 32 wave + lane % 32.
template <int L>
__global__ void k_pack_so2(const uint16_t* __restrict__ w, bf16x8* __restrict__ out) {
  using S = Shape<L>;
  const int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (v >= S::wtotal()) return;
  int m = 0;
  while (m < L && v >= S::woff(m + 1)) ++m;
  const int64_t rem = v - S::woff(m);
  const int64_t blk = rem / S::wblock(m);
  const int within = static_cast<int>(rem % S::wblock(m));
  const int lo_rel = static_cast<int>(blk / 4), wv = static_cast<int>(blk % 4);
  const int sf = within / 64, lane = within % 64;
  const int fps = S::fps(m);
  const int st = sf / fps, wsel = sf % fps;
  const int64_t km = S::km(m);
  const uint16_t* base = w + S::loff(m) + wsel * km * km;
  const int64_t k0 = 16 * st + 8 * (lane / 32);
  const int64_t n = (int64_t)lo_rel * kC + 32 * wv + lane % 32;
  uint16_t vals[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) vals[q] = base[(k0 + q) * km + n];
  uint4 o;
  o.x = vals[0] | (uint32_t(vals[1]) << 16);
  o.y = vals[2] | (uint32_t(vals[3]) << 16);
  o.z = vals[4] | (uint32_t(vals[5]) << 16);
  o.w = vals[6] | (uint32_t(vals[7]) << 16);
  *reinterpret_cast<uint4*>(out + v) = o;
}

// W_rad [8][L+1][C] -> [(L+1) C] vectors of 8 basis weights.
template <int L>
__global__ void k_pack_rad(const uint16_t* __restrict__ w, f16x8* __restrict__ out) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= (L + 1) * kC) return;
  float vals[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) vals[q] = __uint_as_float(uint32_t(w[q * (L + 1) * kC + v]) << 16);
  out[v] = to_vec8<f16x8>(vals);
}

template <int L>
size_t packed_bytes() {
  return align_up(Shape<L>::wtotal() * 16, 256) + align_up((L + 1) * kC * 16, 256);
}

template <int L>
e2a_status launch_typed(const AttnPlan& pl, hipStream_t st) {
  using S = Shape<L>;
  const e2a_attn_args* a = pl.a;
  bf16x8* wpk = static_cast<bf16x8*>(pl.w_packed);
  f16x8* radpk = reinterpret_cast<f16x8*>(static_cast<char*>(pl.w_packed) + align_up(S::wtotal() * 16, 256));
  {
    const int64_t nv = S::wtotal();
    k_pack_so2<L><<<(nv + 255) / 256, 256, 0, st>>>(static_cast<const uint16_t*>(a->w_so2), wpk);
    k_pack_rad<L><<<((L + 1) * kC + 255) / 256, 256, 0, st>>>(static_cast<const uint16_t*>(a->w_rad), radpk);
    E2A_LAUNCH_CHECK();
  }
  MfmaParams p{};
  p.pos = a->pos;
  p.row_ptr = a->row_ptr;
  p.col = a->col;
  p.q = pl.q;
  p.k = pl.k;
  p.feat = static_cast<const uint16_t*>(a->feat);
  p.wpk = wpk;
  p.radpk = radpk;
  p.out = a->out;
  p.out_lse = a->out_lse;
  for (int d = 0; d < 3; ++d) p.box[d] = pl.box[d];
  p.periodic = pl.periodic;
  p.cutoff = a->cutoff;
  E2A_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_mfma<L>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, S::total));
  hipLaunchKernelGGL(k_attn_mfma<L>, dim3(a->n_atoms), dim3(kThreads), S::total, st, p);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

}  // namespace

bool mfma_supported(int L, int C, int H, int dtype) {
  return L >= 1 && L <= 4 && C == kC && H == kH && dtype == E2A_DTYPE_BF16;
}

size_t mfma_packed_weight_bytes(int L, int C) {
  if (C != kC) return 0;
  switch (L) {
    case 1: return packed_bytes<1>();
    case 2: return packed_bytes<2>();
    case 3: return packed_bytes<3>();
    case 4: return packed_bytes<4>();
    default: return 0;
  }
}

e2a_status launch_attention_mfma(const AttnPlan& pl, hipStream_t s) {
  switch (pl.a->L) {
    case 1: return launch_typed<1>(pl, s);
    case 2: return launch_typed<2>(pl, s);
    case 3: return launch_typed<3>(pl, s);
    case 4: return launch_typed<4>(pl, s);
    default: return fail(E2A_ERR_UNSUPPORTED, "MFMA kernel: L=%d", pl.a->L);
  }
}

}  // namespace e2a

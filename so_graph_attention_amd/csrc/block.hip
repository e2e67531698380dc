// One block around the on-the-fly attention layer: per-degree RMS norms, the
// per-degree channel projection with its residual, and the gated
// feed-forward network with its residual.
//
// arXiv 2601.16622 (E2Former-V2) places the fused attention layer inside its
// model (abstract; English technical summary section 2, "Methodology") but
// prints none of the block around it.  The reading built here is the plainest
// equivariant pre-norm residual block:
//   h1  = h + Proj(Attn(Norm1(h))),   out = h1 + FFN(Norm2(h1)),
// where Norm scales each atom's degree-l block by the inverse RMS over its
// (m, c) entries times a gain per (l, c); Proj, W1 and W2 are one channel
// matrix per degree, the same for every m; the FFN takes SiLU of its scalars
// and gates every channel of each degree l >= 1 by the sigmoid of invariant
// scalars n0 W_gate.  All of it acts on channels or through invariants, so it
// commutes with rotations.
//
// Every step here is node-wise (no edges): a few GEMMs of N (2l+1) rows by
// C x C per degree, on the matrix cores for bf16 storage.
#include <algorithm>

#include "e2a_internal.hpp"

namespace e2a {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNormEps = 1e-6f;   // the norm's epsilon, inside the square root

template <typename T>
__device__ __forceinline__ void store_as(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void store_as<float>(float* p, size_t i, float v) {
  p[i] = v;
}
template <>
__device__ __forceinline__ void store_as<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16_rne(v);
}

__device__ __forceinline__ int degree_of(int comp) {
  int l = 0;
  while ((l + 1) * (l + 1) <= comp) ++l;
  return l;
}

// out[a][l*l + m][c] = gamma[l][c] h[a][l*l + m][c] / sqrt(mean_{m,c} h^2 + eps),
// one wave per atom, fp32 sums, 16-byte loads (C is a multiple of 4).  OutT
// is the storage of the result (bf16 for the attention layer's input, or fp32).
template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, const float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float4 v) {
  *reinterpret_cast<uint2*>(p) = uint2{f32_to_bf16_rne(v.x) | (uint32_t(f32_to_bf16_rne(v.y)) << 16),
                                       f32_to_bf16_rne(v.z) | (uint32_t(f32_to_bf16_rne(v.w)) << 16)};
}

template <typename GT, typename OutT>
__global__ void __launch_bounds__(256) k_degree_norm(const float* __restrict__ h, const GT* __restrict__ gamma,
                                                     OutT* __restrict__ out, int64_t n, int L, int C) {
  const int lane = threadIdx.x & 63;
  const int64_t a = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (a >= n) return;
  const int K = (L + 1) * (L + 1);
  const unsigned c4 = static_cast<unsigned>(C / 4);
  const float* ha = h + a * K * C;
  OutT* oa = out + a * K * C;
  for (int l = 0; l <= L; ++l) {
    const unsigned cnt4 = static_cast<unsigned>((2 * l + 1) * C / 4);
    const float4* hl = reinterpret_cast<const float4*>(ha + l * l * C);
    float ss = 0.0f;
    for (unsigned t = lane; t < cnt4; t += 64) {
      const float4 v = hl[t];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(4 * cnt4) + kNormEps);
    for (unsigned t = lane; t < cnt4; t += 64) {
      const float4 v = hl[t];
      const unsigned c = (t % c4) * 4;
      float4 o;
      o.x = v.x * inv * load_as_f32(gamma, (size_t)l * C + c);
      o.y = v.y * inv * load_as_f32(gamma, (size_t)l * C + c + 1);
      o.z = v.z * inv * load_as_f32(gamma, (size_t)l * C + c + 2);
      o.w = v.w * inv * load_as_f32(gamma, (size_t)l * C + c + 3);
      store4(oa + l * l * C + 4 * t, o);
    }
  }
}

// act[a][comp][c] = SiLU(u) for l = 0, u * sigmoid(z[a][(l-1) C + c]) for l >= 1;
// atoms in turn per workgroup, four channels per thread (the fp32 VALU path;
// the matrix-core path applies the gate in its first FFN product).
template <typename OutT>
__global__ void __launch_bounds__(256) k_gate(const float* __restrict__ u, const float* __restrict__ z,
                                              OutT* __restrict__ act, int64_t n, int L, int C) {
  const int K = (L + 1) * (L + 1);
  const unsigned kc4 = static_cast<unsigned>(K * C / 4), c4 = static_cast<unsigned>(C / 4);
  for (int64_t a = blockIdx.x; a < n; a += gridDim.x) {
    const float4* ua = reinterpret_cast<const float4*>(u + a * K * C);
    const float* za = z + a * L * C;
    for (unsigned t = threadIdx.x; t < kc4; t += blockDim.x) {
      const unsigned comp = t / c4, c = (t % c4) * 4;
      const float4 x = ua[t];
      float4 v;
      if (comp == 0) {
        v.x = x.x / (1.0f + expf(-x.x));
        v.y = x.y / (1.0f + expf(-x.y));
        v.z = x.z / (1.0f + expf(-x.z));
        v.w = x.w / (1.0f + expf(-x.w));
      } else {
        const float* g = za + (degree_of(static_cast<int>(comp)) - 1) * C + c;
        v.x = x.x / (1.0f + expf(-g[0]));
        v.y = x.y / (1.0f + expf(-g[1]));
        v.z = x.z / (1.0f + expf(-g[2]));
        v.w = x.w / (1.0f + expf(-g[3]));
      }
      store4(act + a * K * C + 4 * t, v);
    }
  }
}

// Rows of the per-degree GEMM: degree l has n (2l+1) rows; row r is atom
// r / (2l+1), component l*l + r % (2l+1).  Tiles are numbered by groups of
// `group` consecutive atoms, and within a group by degree l_lo..l_hi, in
// tiles of at most tile_rows rows.  (Measured at 100k atoms: one group of all
// atoms, i.e. degree by degree, runs faster than groups of 32 atoms, whose
// degree-0 tiles are three quarters empty.)
struct DegGemm {
  const void* x;            // [n][kx][cin], fp32 or bf16 (XT)
  const uint16_t* wb;       // bf16 weights, degree l at wb + l * w_deg_stride, [cin][cout]
  const float* wf;          // fp32 weights (VALU path), same layout
  int64_t w_deg_stride;     // elements between degrees' matrices (0: one matrix for all)
  void* y;                  // [n][ky][cout], fp32 (or bf16 with y_bf16 on the matrix-core path)
  const float* res;         // optional fp32 residual, layout of y
  int64_t n;
  int kx, ky;               // components per atom in x and y
  int y_comp0;              // y component of degree l's row m: comp(l, m) - y_comp0 (ky = 1: 0)
  int cin, cout;
  int l_lo, l_hi;           // degrees computed
  int tile_start[6];        // first tile of degree l_lo + i within a group; [l_hi - l_lo + 1] = tiles per group
  const uint16_t* wb2;      // optional second bf16 product (grid z = 1): the same x times wb2 into y2
  void* y2;
  int tile_rows;            // rows per tile (set by the launcher)
  int64_t group;            // atoms per tile group (set by the launcher)
  bool y_bf16;              // y stored as bf16 (matrix-core path only)
  bool gate;                // epilogue: SiLU on degree 0, u * sigmoid(z) on degree l >= 1
  const float* gate_z;      // gate logits z[a][(l - 1) cout + c], atom stride z_stride (NULL when L = 0)
  int64_t z_stride;
  // x rows normalised per atom and degree before the product (matrix-core
  // path, fp32 x): x[l,m,c] inv_in[a][l] gamma[l][c], gamma bf16, inv_in the
  // per-atom inverse RMS that an earlier product's stats_out wrote
  const uint16_t* norm_gamma;
  const float* inv_in;
  // the epilogue writes 1 / sqrt(mean_{m,c} y[l]^2 + eps) of every atom's
  // degree-l rows of y (the stored values, residual included) to
  // stats_out[a][l] (matrix-core path, cout <= 128); the tiles then hold
  // whole atoms
  float* stats_out;
  int stats_ld;             // entries per atom in inv_in / stats_out (L + 1)
  bool atom_tiles;          // tile rows of degree l: (tile_rows / (2l+1)) (2l+1)
};

constexpr int kRows = 64;
constexpr int kCols = 64;
// Degree, first row and end row (exclusive) of tile `tile`.
__device__ __forceinline__ void tile_degree(const DegGemm& g, int tile, int& l, int64_t& row0, int64_t& row_end) {
  const int per = g.tile_start[g.l_hi - g.l_lo + 1];
  const int64_t grp = tile / per;
  const int in = tile % per;
  int i = 0;
  while (in >= g.tile_start[i + 1]) ++i;
  l = g.l_lo + i;
  const int64_t w = 2 * l + 1;
  const int64_t g0 = grp * g.group * w;
  const int64_t tr = g.atom_tiles ? g.tile_rows / w * w : g.tile_rows;
  row0 = g0 + (int64_t)(in - g.tile_start[i]) * tr;
  int64_t e = g0 + g.group * w;
  if (e > row0 + tr) e = row0 + tr;
  if (e > g.n * w) e = g.n * w;
  row_end = e;
}

// bf16 matrix-core path, computed transposed: y^T = W^T x^T for a tile of
// 128 node rows and 128 output channels per workgroup.  The MFMA's rows are
// output channels (wave w owns 32 of them; their W^T fragments, k contiguous
// in the transposed copy wt, sit in registers for the whole tile) and its
// columns are node rows (x rounded to bf16 and staged in LDS, k contiguous;
// optionally normalised per atom first, the RMS norm folded into the
// product).  The results go through an fp32 LDS tile, 64 rows at a time, and
// 32 consecutive threads read each row back, so the residual loads and the
// stores of y cover whole rows.  Optional epilogue: the FFN's gate (SiLU on
// degree 0, sigmoid of the gate logits z on degree l >= 1).
constexpr int kMRows = 128;
constexpr int kMCols = 128;
constexpr int kMaxCin = 128;   // x staging and the weight registers cover cin <= 128

// Eight consecutive values of x as loaded (fp32 or bf16 bits).
template <typename XT>
struct XT8;
template <>
struct XT8<float> {
  float4 a, b;
};
template <>
struct XT8<uint16_t> {
  uint4 a;
};
__device__ __forceinline__ XT8<float> load8(const float* p) {
  return XT8<float>{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}
__device__ __forceinline__ XT8<uint16_t> load8(const uint16_t* p) {
  return XT8<uint16_t>{*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ void store8_bf16(const XT8<float>& x, uint16_t* dst) {
  const float v[8] = {x.a.x, x.a.y, x.a.z, x.a.w, x.b.x, x.b.y, x.b.z, x.b.w};
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = f32_to_bf16_rne(v[2 * q]) | (uint32_t(f32_to_bf16_rne(v[2 * q + 1])) << 16);
  *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ void store8_bf16(const XT8<uint16_t>& x, uint16_t* dst) {
  *reinterpret_cast<uint4*>(dst) = x.a;
}

// The matrix-core path rounds the gated activations to bf16, so the gate
// uses the hardware exp2 and reciprocal (each within a few fp32 ulps, far
// below bf16's 2^-9): sigmoid(z) = 1 / (1 + 2^(-z log2 e)); z -> -inf gives
// 1 / inf = 0, z -> +inf gives 1.
__device__ __forceinline__ float sigmoid_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
__device__ __forceinline__ float silu(float u) { return u * sigmoid_fast(u); }
__device__ __forceinline__ float gated(float u, float z) { return u * sigmoid_fast(z); }

// Norm2 of the staged x rows (fp32 values in registers, before they are
// rounded to bf16): x <- (x inv) gamma[l][c] with the atom's inverse RMS from
// inv_in, the arithmetic of the standalone norm.
__device__ __forceinline__ void scale_rows(const DegGemm& g, XT8<float> (&xv)[kMRows * (kMaxCin / 8) / 256], int l,
                                           unsigned w, unsigned row0, unsigned nrows, int tid) {
  constexpr int kSteps = kMRows * (kMaxCin / 8) / 256;
  const int cin = g.cin, kg = cin / 8;
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int t = tid + 256 * q;
    const int r = t / kg, k8 = (t % kg) * 8;
    const unsigned row = row0 + static_cast<unsigned>(r);
    if (t >= kMRows * kg || row >= nrows) continue;
    const float inv = g.inv_in[(size_t)(row / w) * g.stats_ld + l];
    // 8 gains in one 16-byte load (gamma 16-byte aligned, checked on the host)
    const uint4 gv = *reinterpret_cast<const uint4*>(g.norm_gamma + (size_t)l * cin + k8);
    auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
    auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
    XT8<float>& x = xv[q];
    x.a.x = x.a.x * inv * lo(gv.x);
    x.a.y = x.a.y * inv * hi(gv.x);
    x.a.z = x.a.z * inv * lo(gv.y);
    x.a.w = x.a.w * inv * hi(gv.y);
    x.b.x = x.b.x * inv * lo(gv.z);
    x.b.y = x.b.y * inv * hi(gv.z);
    x.b.z = x.b.z * inv * lo(gv.w);
    x.b.w = x.b.w * inv * hi(gv.w);
  }
}

// Byte offset of the epilogue's row sums (mode 2) in dynamic LDS: past both
// the x tile and the output staging tile.
__host__ __device__ constexpr size_t rowsum_offset(int cin) {
  return sizeof(uint16_t) * (size_t)kMRows * (cin + 8) > sizeof(float) * (size_t)64 * (kMCols + 4)
             ? sizeof(uint16_t) * (size_t)kMRows * (cin + 8)
             : sizeof(float) * (size_t)64 * (kMCols + 4);
}

// NM: 0 plain; 1 the x rows scaled by inv_in and the gains (Norm2 folded in);
// 2 the epilogue writes Norm2's per-atom inverse RMS of y to stats_out.
template <typename XT, typename YT, int NM>
__global__ void __launch_bounds__(256, 4) k_deg_gemm_mfma(DegGemm g) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int cin = g.cin, ldk = g.cin + 8, kg = g.cin / 8;
  uint16_t* Xs = reinterpret_cast<uint16_t*>(smem);   // [kMRows][ldk]
  int l;
  int64_t row0, row_end;
  tile_degree(g, blockIdx.x, l, row0, row_end);
  const unsigned w = 2 * l + 1;
  const unsigned nrows = static_cast<unsigned>(row_end);   // < 2^31 (checked on the host)
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, r32 = lane & 31;
  // the wave's 32 output channels; cout is a multiple of 32, so they are
  // all valid or all past the end
  const int cbase = blockIdx.y * kMCols + 32 * wave;
  const bool wok = cbase < g.cout;
  // W^T fragments of every k-step: A operand rows = channels cbase + r32
  const uint16_t* Wt = (blockIdx.z ? g.wb2 : g.wb) + (int64_t)l * g.w_deg_stride;
  constexpr int kKSteps = kMaxCin / 16;
  bf16x8 wv[kKSteps];
  auto load_w = [&]() {
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      wv[s] = (wok && 16 * s < cin)
                  ? *reinterpret_cast<const bf16x8*>(Wt + (size_t)(cbase + r32) * cin + 16 * s + 8 * half)
                  : bf16x8{};
  };
  // with the folded norm the weights load after the rows are staged (their
  // registers would otherwise be live beside the rows and the gains)
  if constexpr (NM != 1) load_w();
  // the tile's rows of x: a lane's 8 k values per step, all loads in flight
  // before the conversions and LDS stores
  constexpr int kSteps = kMRows * (kMaxCin / 8) / 256;
  XT8<XT> xv[kSteps];
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int t = tid + 256 * q;
    const int r = t / kg, k8 = (t % kg) * 8;
    const unsigned row = static_cast<unsigned>(row0) + r;
    if (t < kMRows * kg && row < nrows) {
      const unsigned a = row / w, comp = l * l + row % w;
      xv[q] = load8(static_cast<const XT*>(g.x) + ((size_t)a * g.kx + comp) * cin + k8);
    } else {
      xv[q] = XT8<XT>{};
    }
  }
  if constexpr (NM == 1) scale_rows(g, xv, l, w, static_cast<unsigned>(row0), nrows, tid);
#pragma unroll
  for (int q = 0; q < kSteps; ++q) {
    const int t = tid + 256 * q;
    if (t < kMRows * kg) store8_bf16(xv[q], Xs + (t / kg) * ldk + (t % kg) * 8);
  }
  if constexpr (NM == 1) load_w();
  __syncthreads();
  // B operand = x^T: column j = node row 32 t + r32, k = 16 s + 8 half ..
  f32x16 acc[4] = {};
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) {
    if (!wok || 16 * s >= cin) break;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 xb = *reinterpret_cast<const bf16x8*>(Xs + (32 * t + r32) * ldk + 16 * s + 8 * half);
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[s], xb, acc[t], 0, 0, 0);
    }
  }
  // Epilogue through LDS, 64 rows at a time: a lane's accumulators (node row
  // 32 t + r32, channels 8 q + 4 half + 0..3 of the wave's 32) go to an fp32
  // [row][channel] tile, then each row is read back by 32 consecutive
  // threads, 4 channels each, so residual and gate loads and the stores cover
  // whole rows (512 bytes fp32, 256 bytes bf16).
  float* St = reinterpret_cast<float*>(smem);   // [64][kMCols + 4], over Xs
  float* rsum = reinterpret_cast<float*>(smem + rowsum_offset(cin));   // [kMRows] (mode 2)
  constexpr int lds = kMCols + 4;
  YT* Y = static_cast<YT*>(blockIdx.z ? g.y2 : g.y);
  const int cw = blockIdx.y * kMCols;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    __syncthreads();   // Xs (or the previous half) no longer read
    if (wok) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(St + (32 * tt + r32) * lds + 32 * wave + 8 * q + 4 * half) =
              float4{acc[2 * hh + tt][4 * q], acc[2 * hh + tt][4 * q + 1], acc[2 * hh + tt][4 * q + 2],
                     acc[2 * hh + tt][4 * q + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid + 256 * j;
      const int rr = idx >> 5, c4 = (idx & 31) * 4;
      const unsigned row = static_cast<unsigned>(row0) + 64 * hh + rr;
      const bool ok = row < nrows && cw + c4 < g.cout;
      float4 v = {};
      if (ok) {
      const unsigned a = row / w, comp = l * l + row % w;
      const size_t o = ((size_t)a * g.ky + comp - g.y_comp0) * g.cout + cw + c4;
      v = *reinterpret_cast<const float4*>(St + rr * lds + c4);
      if (g.res) {
        const float4 rv = *reinterpret_cast<const float4*>(g.res + o);
        v.x += rv.x;
        v.y += rv.y;
        v.z += rv.z;
        v.w += rv.w;
      }
      if (g.gate) {
        if (l > 0) {
          const float4 zv = *reinterpret_cast<const float4*>(g.gate_z + (size_t)a * g.z_stride +
                                                             (size_t)(l - 1) * g.cout + cw + c4);
          v = float4{gated(v.x, zv.x), gated(v.y, zv.y), gated(v.z, zv.z), gated(v.w, zv.w)};
        } else {
          v = float4{silu(v.x), silu(v.y), silu(v.z), silu(v.w)};
        }
      }
      store4(Y + o, v);
      }
      if constexpr (NM == 2) {
        // the row's sum of squares of the stored values: its 32 threads are
        // consecutive lanes of one wave
        float sq = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) sq += __shfl_xor(sq, m);
        if ((idx & 31) == 0) rsum[64 * hh + rr] = sq;
      }
    }
  }
  if constexpr (NM == 2) {
    // per atom of the tile (whole atoms): its 2l+1 row sums in row order
    __syncthreads();
    const unsigned nr = nrows - static_cast<unsigned>(row0);
    for (unsigned k = tid; k * w < nr; k += 256) {
      float ss = 0.0f;
      for (unsigned r = 0; r < w; ++r) ss += rsum[k * w + r];
      const float inv = 1.0f / sqrtf(ss / static_cast<float>(static_cast<int>(w) * g.cout) + kNormEps);
      g.stats_out[(size_t)((static_cast<unsigned>(row0) + k * w) / w) * g.stats_ld + l] = inv;
    }
  }
}

// wt[d][n][k] = w[d][k][n] (bf16), for the matrix-core GEMM's k-contiguous
// weight columns.  With w2 set, matrix 1 comes from w2 instead (two separate
// matrices in one launch).
__global__ void k_transpose_bf16(const uint16_t* __restrict__ w, const uint16_t* __restrict__ w2,
                                 uint16_t* __restrict__ wt, int nmat, int rows, int cols) {
  __shared__ uint16_t tile[32][33];
  const int m = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const uint16_t* src = (w2 && m == 1) ? w2 : w + (size_t)m * rows * cols;
  uint16_t* dst = wt + (size_t)m * rows * cols;
  for (int t = threadIdx.x; t < 32 * 32; t += blockDim.x) {
    const int r = t / 32, c = t % 32;
    if (r0 + r < rows && c0 + c < cols) tile[r][c] = src[(size_t)(r0 + r) * cols + c0 + c];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < 32 * 32; t += blockDim.x) {
    const int c = t / 32, r = t % 32;
    if (r0 + r < rows && c0 + c < cols) dst[(size_t)(c0 + c) * rows + r0 + r] = tile[r][c];
  }
  (void)nmat;
}

// fp32 path (fp32 storage, or shapes without a matrix-core tile): the same
// tiles, each thread 4 rows x 4 columns, fp32 throughout.
template <typename XT>
__global__ void __launch_bounds__(256) k_deg_gemm_valu(DegGemm g) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int cin = g.cin;
  float* As = reinterpret_cast<float*>(smem);   // [kRows][cin]
  float* Bs = As + kRows * cin;                 // [cin][kCols]
  int l;
  int64_t row0, nrows;
  tile_degree(g, blockIdx.x, l, row0, nrows);
  const int w = 2 * l + 1;
  const int col0 = blockIdx.y * kCols;
  const int tid = threadIdx.x;
  for (int t = tid; t < kRows * cin; t += 256) {
    const int r = t / cin, k = t % cin;
    const int64_t row = row0 + r;
    float v = 0.0f;
    if (row < nrows) {
      const int64_t a = row / w;
      const int comp = l * l + static_cast<int>(row % w);
      v = load_as_f32(static_cast<const XT*>(g.x), (size_t)(a * g.kx + comp) * cin + k);
    }
    As[t] = v;
  }
  const float* W = g.wf + (int64_t)l * g.w_deg_stride;
  for (int t = tid; t < cin * kCols; t += 256) {
    const int k = t / kCols, nn = t % kCols;
    Bs[t] = col0 + nn < g.cout ? W[(size_t)k * g.cout + col0 + nn] : 0.0f;
  }
  __syncthreads();
  const int tr = (tid / 16) * 4, tc = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int k = 0; k < cin; ++k) {
    float av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = As[(tr + i) * cin + k];
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = Bs[k * kCols + tc + j];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + tr + i;
    if (row >= nrows) continue;
    const int64_t a = row / w;
    const int comp = l * l + static_cast<int>(row % w) - g.y_comp0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = col0 + tc + j;
      if (col >= g.cout) continue;
      const size_t o = (size_t)(a * g.ky + comp) * g.cout + col;
      static_cast<float*>(g.y)[o] = (g.res ? g.res[o] : 0.0f) + acc[i][j];
    }
  }
}

// fp32 copy of bf16 or fp32 weights (the VALU path reads fp32).
template <typename T>
__global__ void k_widen(const T* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) dst[i] = load_as_f32(src, (size_t)i);
}

}  // namespace

bool block_uses_mfma(int C, int dtype) {
  return dtype == E2A_DTYPE_BF16 && C % 32 == 0 && C >= 32 && C <= kMaxCin;
}

BlockWs block_ws_layout(int64_t n, int L, int C, int H, int dtype) {
  BlockWs w{};
  const int K = (L + 1) * (L + 1);
  const size_t s = dtype == E2A_DTYPE_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t nkc = (size_t)n * K * C;
  w.n1 = take(s * nkc);
  w.attn = take(sizeof(float) * nkc);      // the layer's output, later the FFN's hidden u
  w.h1 = take(sizeof(float) * nkc);
  w.n2 = take(s * nkc);                    // Norm2, later the gated activations
  w.z = take(sizeof(float) * (size_t)n * (L > 0 ? L : 1) * C);
  w.inv2 = take(sizeof(float) * (size_t)n * (L + 1));   // Norm2's per-atom inverse RMS (matrix-core path)
  const size_t nw = (size_t)(L + 1) * C * C;
  // node-wise weights: transposed bf16 copies (matrix cores) or fp32 copies (VALU)
  w.wf = block_uses_mfma(C, dtype) ? take(sizeof(uint16_t) * (3 * nw + (size_t)C * L * C))
                                   : take(sizeof(float) * (3 * nw + (size_t)C * L * C));
  w.attn_ws = off;
  w.attn_ws_bytes = 0;   // set by the caller from the attention workspace query
  w.total = off;
  return w;
}

namespace {

e2a_status launch_norm(const float* h, const void* gamma, void* out, int64_t n, int L, int C, int dtype,
                       hipStream_t s) {
  if (n == 0) return E2A_OK;
  const dim3 grid((n + 3) / 4);
  if (dtype == E2A_DTYPE_BF16)
    hipLaunchKernelGGL((k_degree_norm<uint16_t, uint16_t>), grid, dim3(256), 0, s, h,
                       static_cast<const uint16_t*>(gamma), static_cast<uint16_t*>(out), n, L, C);
  else
    hipLaunchKernelGGL((k_degree_norm<float, float>), grid, dim3(256), 0, s, h, static_cast<const float*>(gamma),
                       static_cast<float*>(out), n, L, C);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

// y (+ res) = x W per degree l in [l_lo, l_hi]; x in storage dtype (xbf16) or
// fp32; weights as bf16 (mfma) or fp32 (valu).
e2a_status launch_deg_gemm(DegGemm g, bool mfma, bool x_bf16, hipStream_t s) {
  if (g.n == 0) return E2A_OK;
  g.tile_rows = mfma ? kMRows : kRows;
  g.atom_tiles = mfma && g.stats_out;
  const int tcols = mfma ? kMCols : kCols;
  g.group = g.n;
  int64_t per = 0;
  for (int l = g.l_lo; l <= g.l_hi; ++l) {
    if (per > INT32_MAX) break;
    g.tile_start[l - g.l_lo] = static_cast<int>(per);
    const int64_t tr = g.atom_tiles ? g.tile_rows / (2 * l + 1) * (2 * l + 1) : g.tile_rows;
    per += (g.group * (2 * l + 1) + tr - 1) / tr;
  }
  if (per > INT32_MAX) return fail(E2A_ERR_UNSUPPORTED, "node-wise GEMM: %lld tiles", (long long)per);
  g.tile_start[g.l_hi - g.l_lo + 1] = static_cast<int>(per);
  const int64_t tiles = (g.n + g.group - 1) / g.group * per;
  if (tiles > INT32_MAX) return fail(E2A_ERR_UNSUPPORTED, "node-wise GEMM: %lld tiles", (long long)tiles);
  const dim3 grid(static_cast<unsigned>(tiles), (g.cout + tcols - 1) / tcols, mfma && g.wb2 ? 2 : 1);
  if (mfma) {
    if (g.cin > kMaxCin || g.cin % 32 != 0 || g.cout % 32 != 0)
      return fail(E2A_ERR_UNSUPPORTED, "node-wise GEMM: cin=%d cout=%d on the matrix cores", g.cin, g.cout);
    const size_t smem = rowsum_offset(g.cin) + (g.stats_out ? sizeof(float) * kMRows : 0);
    if ((g.norm_gamma && (x_bf16 || !g.inv_in)) || (g.stats_out && (g.cout > kMCols || g.y_bf16 || g.gate)))
      return fail(E2A_ERR_UNSUPPORTED, "node-wise GEMM: folded norm needs fp32 x and its statistics; statistics "
                                       "need one column block of fp32 output");
    if (x_bf16 && g.y_bf16)
      hipLaunchKernelGGL((k_deg_gemm_mfma<uint16_t, uint16_t, 0>), grid, dim3(256), smem, s, g);
    else if (x_bf16)
      hipLaunchKernelGGL((k_deg_gemm_mfma<uint16_t, float, 0>), grid, dim3(256), smem, s, g);
    else if (g.stats_out)
      hipLaunchKernelGGL((k_deg_gemm_mfma<float, float, 2>), grid, dim3(256), smem, s, g);
    else if (g.norm_gamma && g.y_bf16)
      hipLaunchKernelGGL((k_deg_gemm_mfma<float, uint16_t, 1>), grid, dim3(256), smem, s, g);
    else if (g.norm_gamma)
      hipLaunchKernelGGL((k_deg_gemm_mfma<float, float, 1>), grid, dim3(256), smem, s, g);
    else if (g.y_bf16)
      hipLaunchKernelGGL((k_deg_gemm_mfma<float, uint16_t, 0>), grid, dim3(256), smem, s, g);
    else
      hipLaunchKernelGGL((k_deg_gemm_mfma<float, float, 0>), grid, dim3(256), smem, s, g);
  } else {
    const size_t smem = sizeof(float) * (size_t)(kRows + kCols) * g.cin;
    if (x_bf16) {
      E2A_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_deg_gemm_valu<uint16_t>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
      hipLaunchKernelGGL(k_deg_gemm_valu<uint16_t>, grid, dim3(256), smem, s, g);
    } else {
      E2A_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_deg_gemm_valu<float>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem));
      hipLaunchKernelGGL(k_deg_gemm_valu<float>, grid, dim3(256), smem, s, g);
    }
  }
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

// dst[m][c][r] = src[m][r][c] for nmat bf16 matrices of rows x cols (with
// src2 set: two matrices, the second from src2).
e2a_status launch_transpose(const void* src, uint16_t* dst, int nmat, int rows, int cols, hipStream_t s,
                            const void* src2 = nullptr) {
  if (nmat == 0 || rows == 0 || cols == 0) return E2A_OK;
  const dim3 grid((cols + 31) / 32, (rows + 31) / 32, nmat);
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src),
                     static_cast<const uint16_t*>(src2), dst, nmat, rows, cols);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

e2a_status launch_widen(const void* src, float* dst, int64_t n, int dtype, hipStream_t s) {
  if (n == 0) return E2A_OK;
  const dim3 grid((n + 255) / 256);
  if (dtype == E2A_DTYPE_BF16)
    hipLaunchKernelGGL(k_widen<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), dst, n);
  else
    hipLaunchKernelGGL(k_widen<float>, grid, dim3(256), 0, s, static_cast<const float*>(src), dst, n);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

}  // namespace

e2a_status launch_qk_mfma(const uint16_t* feat, const uint16_t* wq, const uint16_t* wk, uint16_t* wqk_t, int64_t n,
                          int K, int C, float* q, float* k, hipStream_t s) {
  const e2a_status st = launch_transpose(wq, wqk_t, 2, C, C, s, wk);
  if (st != E2A_OK) return st;
  DegGemm g{};
  g.x = feat;
  g.n = n;
  g.kx = K;
  g.ky = 1;
  g.cin = g.cout = C;
  g.l_lo = g.l_hi = 0;
  g.wb = wqk_t;
  g.y = q;
  g.wb2 = wqk_t + (size_t)C * C;
  g.y2 = k;
  return launch_deg_gemm(g, true, true, s);
}

e2a_status launch_block(const BlockPlan& p, hipStream_t s) {
  const e2a_block_args* b = p.b;
  const int L = b->L, C = b->C, dtype = b->dtype;
  const int64_t n = b->n_atoms;
  const int K = (L + 1) * (L + 1);
  char* base = static_cast<char*>(b->workspace);
  const BlockWs& W = p.ws;
  void* n1 = base + W.n1;
  float* attn = reinterpret_cast<float*>(base + W.attn);
  float* h1 = reinterpret_cast<float*>(base + W.h1);
  void* n2 = base + W.n2;
  float* z = reinterpret_cast<float*>(base + W.z);
  const bool mfma = block_uses_mfma(C, dtype);
  const bool bf = dtype == E2A_DTYPE_BF16;
  const int64_t nw = (int64_t)(L + 1) * C * C;
  // fp32 copies of the node-wise weights for the VALU path, transposed bf16
  // copies (k contiguous) for the matrix cores
  const float *wo_f = nullptr, *w1_f = nullptr, *w2_f = nullptr, *wg_f = nullptr;
  const uint16_t *wo_t = nullptr, *w1_t = nullptr, *w2_t = nullptr, *wg_t = nullptr;
  if (mfma) {
    uint16_t* wt = reinterpret_cast<uint16_t*>(base + W.wf);
    e2a_status st = launch_transpose(b->w_o, wt, L + 1, C, C, s);
    if (st == E2A_OK) st = launch_transpose(b->w_1, wt + nw, L + 1, C, C, s);
    if (st == E2A_OK) st = launch_transpose(b->w_2, wt + 2 * nw, L + 1, C, C, s);
    if (st == E2A_OK && L > 0) st = launch_transpose(b->w_gate, wt + 3 * nw, 1, C, L * C, s);
    if (st != E2A_OK) return st;
    wo_t = wt;
    w1_t = wt + nw;
    w2_t = wt + 2 * nw;
    wg_t = wt + 3 * nw;
  } else {
    float* wf = reinterpret_cast<float*>(base + W.wf);
    e2a_status st = launch_widen(b->w_o, wf, nw, dtype, s);
    if (st == E2A_OK) st = launch_widen(b->w_1, wf + nw, nw, dtype, s);
    if (st == E2A_OK) st = launch_widen(b->w_2, wf + 2 * nw, nw, dtype, s);
    if (st == E2A_OK && L > 0) st = launch_widen(b->w_gate, wf + 3 * nw, (int64_t)C * L * C, dtype, s);
    if (st != E2A_OK) return st;
    wo_f = wf;
    w1_f = wf + nw;
    w2_f = wf + 2 * nw;
    wg_f = wf + 3 * nw;
  }
  // n1 = Norm1(h)
  e2a_status st = launch_norm(b->h_in, b->norm1, n1, n, L, C, dtype, s);
  if (st != E2A_OK) return st;
  // a = Attn(n1)
  e2a_attn_args a{};
  a.pos = b->pos;
  a.box = b->box;
  a.n_atoms = n;
  a.row_ptr = b->row_ptr;
  a.col = b->col;
  a.n_edges = b->n_edges;
  a.cutoff = b->cutoff;
  a.L = L;
  a.C = C;
  a.H = b->H;
  a.n_rbf = b->n_rbf;
  a.dtype = dtype;
  a.variant = b->variant;
  a.feat = n1;
  a.w_q = b->w_q;
  a.w_k = b->w_k;
  a.w_rad = b->w_rad;
  a.w_so2 = b->w_so2;
  a.out = attn;
  a.out_lse = nullptr;
  a.w_so2_packed = b->w_so2_packed;
  a.order = b->order;
  a.workspace = base + W.attn_ws;
  a.workspace_bytes = W.attn_ws_bytes;
  st = p.attention(&a, s);
  if (st != E2A_OK) return st;
  // Norm2 on the matrix cores: the projection's epilogue writes each atom's
  // inverse RMS of h1 per degree (inv2), and the products that read
  // Norm2(h1) (gate logits, first FFN product) scale h1's rows by it and the
  // gains as they stage them; with gains off the 16-byte boundary, or on the
  // VALU path, Norm2 is a pass of its own
  const bool fuse_norm2 = mfma && (reinterpret_cast<uintptr_t>(b->norm2) & 15) == 0;
  float* inv2 = reinterpret_cast<float*>(base + W.inv2);
  // h1 = h + a W_o
  DegGemm g{};
  g.n = n;
  g.kx = g.ky = K;
  g.cin = g.cout = C;
  g.l_lo = 0;
  g.l_hi = L;
  g.w_deg_stride = (int64_t)C * C;
  g.x = attn;
  g.wb = wo_t;
  g.wf = wo_f;
  g.y = h1;
  g.res = b->h_in;
  g.stats_out = fuse_norm2 ? inv2 : nullptr;
  g.stats_ld = L + 1;
  st = launch_deg_gemm(g, mfma, false, s);
  if (st != E2A_OK) return st;
  g.stats_out = nullptr;
  if (!fuse_norm2) {
    st = launch_norm(h1, b->norm2, n2, n, L, C, dtype, s);
    if (st != E2A_OK) return st;
  }
  // z = n2[l = 0] W_gate (gate logits of degrees 1..L)
  if (L > 0) {
    DegGemm gz{};
    gz.n = n;
    gz.x = fuse_norm2 ? static_cast<const void*>(h1) : n2;
    gz.norm_gamma = fuse_norm2 ? static_cast<const uint16_t*>(b->norm2) : nullptr;
    gz.inv_in = fuse_norm2 ? inv2 : nullptr;
    gz.stats_ld = L + 1;
    gz.kx = K;
    gz.ky = 1;
    gz.cin = C;
    gz.cout = L * C;
    gz.l_lo = gz.l_hi = 0;
    gz.w_deg_stride = 0;
    gz.wb = wg_t;
    gz.wf = wg_f;
    gz.y = z;
    st = launch_deg_gemm(gz, mfma, bf && !fuse_norm2, s);
    if (st != E2A_OK) return st;
  }
  void* act;
  if (mfma) {
    // act = gate(n2 W1, z) in the GEMM's epilogue, stored bf16 in the
    // attention output's space (its rows are read before any is written:
    // each x row belongs to one tile and cout = C is one column block, but
    // a separate buffer keeps that independent of the tiling)
    act = attn;
    g.x = fuse_norm2 ? static_cast<const void*>(h1) : n2;
    g.norm_gamma = fuse_norm2 ? static_cast<const uint16_t*>(b->norm2) : nullptr;
    g.inv_in = fuse_norm2 ? inv2 : nullptr;
    g.wb = w1_t;
    g.y = act;
    g.y_bf16 = true;
    g.res = nullptr;
    g.gate = true;
    g.gate_z = L > 0 ? z : nullptr;
    g.z_stride = (int64_t)L * C;
    st = launch_deg_gemm(g, true, !fuse_norm2, s);
    if (st != E2A_OK) return st;
    g.norm_gamma = nullptr;
    g.inv_in = nullptr;
    g.y_bf16 = false;
    g.gate = false;
    g.gate_z = nullptr;
  } else {
    // u = n2 W1 (into the attention output's space), then act = gate(u, z)
    // in n2's space (Norm2 is no longer needed)
    float* u = attn;
    g.x = n2;
    g.wf = w1_f;
    g.y = u;
    g.res = nullptr;
    st = launch_deg_gemm(g, false, bf, s);
    if (st != E2A_OK) return st;
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(n, 8192)));
    if (bf)
      hipLaunchKernelGGL(k_gate<uint16_t>, grid, dim3(256), 0, s, u, z, static_cast<uint16_t*>(n2), n, L, C);
    else
      hipLaunchKernelGGL(k_gate<float>, grid, dim3(256), 0, s, u, z, static_cast<float*>(n2), n, L, C);
    E2A_LAUNCH_CHECK();
    act = n2;
  }
  // out = h1 + act W2
  g.x = act;
  g.wb = w2_t;
  g.wf = w2_f;
  g.y = b->h_out;
  g.res = h1;
  return launch_deg_gemm(g, mfma, bf, s);
}

}  // namespace e2a

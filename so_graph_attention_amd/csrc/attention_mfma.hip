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
#include <utility>

#include "e2a_geometry.hpp"
#include "e2a_internal.hpp"

namespace e2a {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
  // weight stream of one chunk: block m has nb(m) output blocks (pairs for
  // m = 0) of ks(m) k-steps; sbase(m) is its first step in the chunk
  static constexpr int ks(int m) { return km(m) / 16; }
  static constexpr int nb(int m) { return m == 0 ? (L + 2) / 2 : L + 1 - m; }
  static constexpr int tot(int m) { return nb(m) * ks(m); }
  static constexpr int sbase(int m) {
    int o = 0;
    for (int k = 0; k < m; ++k) o += tot(k);
    return o;
  }
  static constexpr int stot() { return sbase(L + 1); }
  static constexpr int blk_lo(int m, int b, int f) { return m == 0 ? 2 * b + f : m + b; }
  static constexpr bool has1(int m, int b) { return m > 0 || 2 * b + 1 <= L; }
  // block m of the chunk stream holding chunk step G (0 <= G < stot())
  static constexpr int stream_m(int G) {
    int m = 0;
    while (m < L && G >= sbase(m + 1)) ++m;
    return m;
  }
  // byte offset of fragment f of chunk step G, without the wave's column term
  static constexpr int stream_off(int G, int f) {
    const int m = stream_m(G);
    const int g = G - sbase(m);
    const int b = g / ks(m), st = g % ks(m);
    return m == 0 ? static_cast<int>((woff(0) + (int64_t)(blk_lo(0, b, f) * 4) * wblock(0)) * 16) + st * 1024
                  : static_cast<int>((woff(m) + (int64_t)((blk_lo(m, b, 0) - m) * 4) * wblock(m)) * 16) +
                        st * 2048 + f * 1024;
  }
  static constexpr bool stream_has1(int G) {
    const int m = stream_m(G);
    return has1(m, (G - sbase(m)) / ks(m));
  }
  static constexpr int64_t wave_bytes(int m) { return wblock(m) * 16; }
  // two A regions: even m in A0, odd m in A1 (block m+1 is built while m runs)
  static constexpr int amax_par(int par) {
    int b = 0;
    for (int m = par; m <= L; m += 2) b = abytes(m) > b ? abytes(m) : b;
    return b;
  }
  static constexpr int off_A1 = (amax_par(0) + 255) / 256 * 256;
  // LDS layout (bytes)
  static constexpr int off_D = off_A1 + (amax_par(1) + 255) / 256 * 256;
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

// Calls f(std::integral_constant<int, i>) for i = 0..N-1: every index is a
// compile-time constant, so register arrays indexed by it never spill and
// pipeline decisions resolve statically.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
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
__device__ __forceinline__ f32x4 mfma16_f16(const f16x8 a, const f16x8 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Node accumulator of one degree lo for this wave's 32 channels: two 16x16
// MFMA tiles (rows n = 0..15 >= 2 lo + 1, columns = channels 0-15 and 16-31
// of the wave).  Lane l holds rows 4 (l / 16) + r, column l % 16.
struct NodeAcc {
  f32x4 a;   // channels 32 w + 0..15
  f32x4 b;   // channels 32 w + 16..31
};

// Rotate-out contraction step: acc[n][c] += sum_k G[n][k] U[k][c] over the 16
// (edge, sign) slots this k-step carries.  The 32x32 GEMM result gives lane l
// the values of channel l % 32 for 8 edges (lanes 0-31 and 32-63 hold
// different edges).  In the 16x16x32 MFMA, k-slot group g = l / 16 comes from
// lanes 16 g .. 16 g + 15: groups 0 and 2 carry channels 0-15, groups 1 and 3
// channels 16-31, so each of the two MFMAs keeps its own groups and zeroes
// the others.  G (the D rows) is the same register for both.
__device__ __forceinline__ void rotate_out_step(NodeAcc& acc, const f16x8 g, const f16x8 u, bool grp_odd) {
  const f16x8 zero = {};
  acc.a = mfma16_f16(g, grp_odd ? zero : u, acc.a);
  acc.b = mfma16_f16(g, grp_odd ? u : zero, acc.b);
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
  const int32_t* order;   // destination atoms in spatial (Morton) order
  int64_t n_atoms;
  int64_t per_xcd;        // ceil(n_atoms / 8)
  float* out;
  float* out_lse;
  float box[3];
  int periodic;
  float cutoff;
};

struct Smem {
  uint16_t* A0;    // GEMM operand of even |m| blocks
  uint16_t* A1;    // GEMM operand of odd |m| blocks
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

// Rotate-in task tau of block MN for this thread: degree l = MN + tau / 2,
// edge (tid / 16) + 16 (tau % 2), channels 8 (tid % 16) .. +8:
// x_{l,+-MN}[c] = sum_n D^l[l +- MN][n] h_j[l*l + n][c], written as bf16 to
// the block's GEMM operand (rows: edge, and for MN > 0 the +MN row of edge e
// at 32 (e / 16) + e % 16 with its -MN row 16 below; columns (l - MN) C + c).
// The loads and the arithmetic are separate calls so that the loads can be
// issued well before their use.
template <int L, int MN, int TAU>
__device__ __forceinline__ void task_load(const MfmaParams& p, const Smem& s, int tid, uint4 (&raw)[2 * L + 1]) {
  using S = Shape<L>;
  constexpr int l = MN + (TAU >> 1);
  const int e = (tid >> 4) + 16 * (TAU & 1);
  const uint16_t* hp = p.feat + ((int64_t)s.j[e] * S::K + l * l) * kC + 8 * (tid & 15);
#pragma unroll
  for (int n = 0; n < 2 * l + 1; ++n) raw[n] = *reinterpret_cast<const uint4*>(hp + n * kC);
}

// Term n of rotate-in task TAU: xp += D^l[l+MN][n] h[n], xm += D^l[l-MN][n] h[n].
template <int L, int MN, int TAU, int N>
__device__ __forceinline__ void task_term(const Smem& s, int tid, const uint4 (&raw)[2 * L + 1], float (&xp)[8],
                                          float (&xm)[8]) {
  using S = Shape<L>;
  constexpr int l = MN + (TAU >> 1);
  const int e = (tid >> 4) + 16 * (TAU & 1);
  const float* De = s.D + e * S::DSZ + doff(l);
  float hv[8];
  unpack_bf16x8(raw[N], hv);
  const float dp = De[(l + MN) * dpad(l) + N];
#pragma unroll
  for (int q = 0; q < 8; ++q) xp[q] = (N == 0 ? 0.0f : xp[q]) + dp * hv[q];
  if constexpr (MN > 0) {
    const float dm = De[(l - MN) * dpad(l) + N];
#pragma unroll
    for (int q = 0; q < 8; ++q) xm[q] = (N == 0 ? 0.0f : xm[q]) + dm * hv[q];
  }
}

// Rounds task TAU's result to bf16 and writes it to block MN's GEMM operand.
template <int L, int MN, int TAU>
__device__ __forceinline__ void task_store(uint16_t* A, int tid, const float (&xp)[8], const float (&xm)[8]) {
  using S = Shape<L>;
  constexpr int stride = S::astride(MN);
  constexpr int l = MN + (TAU >> 1);
  const int e = (tid >> 4) + 16 * (TAU & 1);
  const int g = tid & 15;
  if constexpr (MN == 0) {
    *reinterpret_cast<bf16x8*>(A + e * stride + l * kC + 8 * g) = to_vec8<bf16x8>(xp);
  } else {
    const int row = 32 * (e >> 4) + (e & 15);
    const int colk = (l - MN) * kC + 8 * g;
    *reinterpret_cast<bf16x8*>(A + row * stride + colk) = to_vec8<bf16x8>(xp);
    *reinterpret_cast<bf16x8*>(A + (row + 16) * stride + colk) = to_vec8<bf16x8>(xm);
  }
}

template <int L, int MN, int TAU>
__device__ __forceinline__ void task_compute(const Smem& s, uint16_t* A, int tid, const uint4 (&raw)[2 * L + 1]) {
  constexpr int W = 2 * (MN + (TAU >> 1)) + 1;
  float xp[8], xm[8];
  static_for<W>([&](auto nc) { task_term<L, MN, TAU, decltype(nc)::value>(s, tid, raw, xp, xm); });
  task_store<L, MN, TAU>(A, tid, xp, xm);
}

// Stand-alone rotate-in of block 0 (the start of a chunk): the loads of task
// tau+1 are issued before task tau's arithmetic.
template <int L>
__device__ __forceinline__ void build_a0(const MfmaParams& p, const Smem& s, int tid) {
  static_assert(kThreads == 16 * kET / 2, "two edges x 16 channel groups per thread");
  tid = opaque(tid);
  uint4 raw[2][2 * L + 1];
  task_load<L, 0, 0>(p, s, tid, raw[0]);
  static_for<2 * (L + 1)>([&](auto tc) {
    constexpr int tau = decltype(tc)::value;
    if constexpr (tau + 1 < 2 * (L + 1)) task_load<L, 0, tau + 1>(p, s, tid, raw[(tau + 1) & 1]);
    task_compute<L, 0, tau>(s, s.A0, tid, raw[tau & 1]);
  });
}

// Compile-time schedule of block M+1's rotate-in inside block M's k-steps:
// tasks run one after another; task tau issues its loads at start(tau),
// accumulates term n at start(tau) + delta + n, and stores one step later.
template <int L, int M>
struct TaskSched {
  using S = Shape<L>;
  static constexpr int NT = M < L ? 2 * (L - M) : 0;
  static constexpr int W(int tau) { return 2 * (M + 1 + tau / 2) + 1; }
  static constexpr int work() {
    int w = 0;
    for (int t = 0; t < NT; ++t) w += W(t) + 1;
    return w;
  }
  static constexpr int delta() {
    if (NT == 0) return 0;
    const int d = (S::tot(M) - work()) / NT;
    return d > 6 ? 6 : d;
  }
  static constexpr int start(int tau) {
    int o = 0;
    for (int t = 0; t < tau; ++t) o += delta() + W(t) + 1;
    return o;
  }
  // task whose loads are issued at step g (or -1)
  static constexpr int load_at(int g) {
    for (int t = 0; t < NT; ++t)
      if (g == start(t)) return t;
    return -1;
  }
  // task and term accumulated at step g (term == W: store), or task -1
  static constexpr int term_task(int g) {
    for (int t = 0; t < NT; ++t)
      if (g >= start(t) + delta() && g <= start(t) + delta() + W(t)) return t;
    return -1;
  }
  static constexpr int term_n(int g) { return term_task(g) < 0 ? 0 : g - start(term_task(g)) - delta(); }
};

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

// 16-byte load of a B fragment through a buffer resource: the per-lane offset
// stays in one VGPR and the k-step advances a scalar offset.
__device__ __forceinline__ bf16x8 load_b(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return __builtin_bit_cast(bf16x8, v);
}

constexpr int kRing = 8;   // weight k-steps in flight per wave
struct WRing {
  bf16x8 r[kRing][2];
};

// Loads chunk step G of the weight stream into its ring slot G % kRing.
template <int L, int G>
__device__ __forceinline__ void wring_load(WRing& ring, __amdgpu_buffer_rsrc_t wrsrc, int voff, int wave) {
  using S = Shape<L>;
  constexpr int m = S::stream_m(G);
  constexpr int off0 = S::stream_off(G, 0);
  constexpr int off1 = S::stream_off(G, 1);
  const int wo = static_cast<int>(wave * S::wave_bytes(m));
  ring.r[G % kRing][0] = load_b(wrsrc, voff, wo + off0);
  if constexpr (S::stream_has1(G)) ring.r[G % kRing][1] = load_b(wrsrc, voff, wo + off1);
}

// GEMM of block M for this wave's 32 output channels, then the epilogue of
// each output block: y_{+-m} from the W1/W2 products, u = alpha * rho * y
// (rho from one MFMA against the radial basis), and the partial rotate-out
// acc_lo[n][c] += sum_{edges, +-} D^lo[lo +- M][n] u_{+-}[c], itself an MFMA
// contraction over the chunk's edges.
//
// Software pipeline, all fixed at compile time: the weight stream runs kRing
// k-steps ahead (continuing into the next block and the next chunk, whose
// weights are the same), A fragments one step ahead, and the rotate-in of
// block M+1 is spread over the k-steps (TaskSched: one term per step) so that
// its VALU work and feature loads overlap the MFMAs.
// A scheduling barrier after every k-step keeps the compiler from undoing
// this order.
template <int L, int M>
__device__ __forceinline__ void mma_block(const MfmaParams& p, const Smem& s, __amdgpu_buffer_rsrc_t wrsrc,
                                          int tid, int wave, const f16x8 (&arbf)[3], const float (&alpha)[16],
                                          NodeAcc (&nacc)[L + 1], WRing& ring) {
  using S = Shape<L>;
  constexpr int KS = S::ks(M);
  constexpr int stride = S::astride(M);
  using TS = TaskSched<L, M>;
  constexpr int NT = TS::NT;                          // rotate-in tasks of block M+1 per thread
  static_assert(NT == 0 || TS::delta() >= 2, "too few k-steps to hide the next rotate-in");
  uint16_t* const Acur = (M % 2 == 0) ? s.A0 : s.A1;
  uint16_t* const Anext = (M % 2 == 0) ? s.A1 : s.A0;
  tid = opaque(tid);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int c_own = 32 * wave + (lane & 31);
  const int n = lane & 15;                 // D row of the rotate-out A operand
  const bool grp_odd = (lane >> 4) & 1;    // lane group 1 or 3: channels 16-31
  const int voff = lane * 16;
  const f16x8 zero8 = {};
  const uint16_t* ap0 = Acur + (lane & 31) * stride + 8 * half;
  const uint16_t* ap1 = ap0 + 32 * stride;   // second row tile (m > 0 only)
  bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ap0);
  bf16x8 a1 = {};
  if constexpr (M > 0) a1 = *reinterpret_cast<const bf16x8*>(ap1);
  uint4 raw[2 * L + 1];
  float txp[8], txm[8];
  static_for<S::nb(M)>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    f32x16 c00 = {}, c01 = {}, c10 = {}, c11 = {};
    // radial-weight fragments of this block's output degrees, fetched now so
    // that they have landed by the epilogue
    f16x8 brad0 = zero8, brad1 = zero8;
    if (half == 0) {
      brad0 = p.radpk[S::blk_lo(M, b, 0) * kC + c_own];
      if constexpr (M == 0 && S::has1(M, b)) brad1 = p.radpk[S::blk_lo(M, b, 1) * kC + c_own];
    }
    static_for<KS>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      constexpr int g = b * KS + st;
      constexpr int G = S::sbase(M) + g;
      const bf16x8 b0 = ring.r[G % kRing][0];
      const bf16x8 b1 = ring.r[G % kRing][1];
      wring_load<L, (G + kRing) % S::stot()>(ring, wrsrc, voff, wave);
      constexpr int sn = (st + 1) % KS;
      const bf16x8 a0n = *reinterpret_cast<const bf16x8*>(ap0 + sn * 16);
      bf16x8 a1n = {};
      if constexpr (M > 0) a1n = *reinterpret_cast<const bf16x8*>(ap1 + sn * 16);
      c00 = mfma_bf16(a0, b0, c00);
      if constexpr (M == 0) {
        if constexpr (S::has1(M, b)) c01 = mfma_bf16(a0, b1, c01);
      } else {
        c01 = mfma_bf16(a0, b1, c01);
        c10 = mfma_bf16(a1, b0, c10);
        c11 = mfma_bf16(a1, b1, c11);
      }
      a0 = a0n;
      a1 = a1n;
      if constexpr (NT > 0) {
        constexpr int MN = M < L ? M + 1 : L;
        constexpr int tl = TS::load_at(g);
        if constexpr (tl >= 0) task_load<L, MN, tl>(p, s, tid, raw);
        constexpr int tt = TS::term_task(g);
        if constexpr (tt >= 0) {
          constexpr int tn = TS::term_n(g);
          if constexpr (tn < TS::W(tt)) task_term<L, MN, tt, tn>(s, tid, raw, txp, txm);
          else task_store<L, MN, tt>(Anext, tid, txp, txm);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (M == 0) {
      static_for<2>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        if constexpr (f == 0 || S::has1(M, b)) {
          constexpr int lo = S::blk_lo(M, b, f);
          const f32x16& c0 = f == 0 ? c00 : c01;
          const f16x8 brad = f == 0 ? brad0 : brad1;
          const f32x16 rho = mfma_f16(arbf[0], brad, f32x16{});
          float u[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) u[r] = alpha[r] * rho[r] * c0[r];
          const bool nvalid = n < 2 * lo + 1;
          const _Float16* drow = s.DT + wig_off(lo) * kET + (lo * (2 * lo + 1) + n) * kET;
          rotate_out_step(nacc[lo], dt_frag(drow, 0, half, nvalid), to_vec8<f16x8>(u), grp_odd);
          rotate_out_step(nacc[lo], dt_frag(drow, 16, half, nvalid), to_vec8<f16x8>(u + 8), grp_odd);
        }
      });
    } else {
      constexpr int lo = S::blk_lo(M, b, 0);
      const f16x8 brad = brad0;
      const bool nvalid = n < 2 * lo + 1;
      const _Float16* dt_lo = s.DT + wig_off(lo) * kET;
      const _Float16* drow_p = dt_lo + ((lo + M) * (2 * lo + 1) + n) * kET;
      const _Float16* drow_m = dt_lo + ((lo - M) * (2 * lo + 1) + n) * kET;
      auto tile = [&](int t, const f32x16& C1, const f32x16& C2) {
        const f32x16 rho = mfma_f16(arbf[1 + t], brad, f32x16{});
        float up[8], um[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sc = alpha[r + 8 * t] * rho[r];
          up[r] = sc * (C1[r] - C2[r + 8]);
          um[r] = sc * (C2[r] + C1[r + 8]);
        }
        rotate_out_step(nacc[lo], dt_frag(drow_p, 16 * t, half, nvalid), to_vec8<f16x8>(up), grp_odd);
        rotate_out_step(nacc[lo], dt_frag(drow_m, 16 * t, half, nvalid), to_vec8<f16x8>(um), grp_odd);
      };
      tile(0, c00, c01);
      tile(1, c10, c11);
    }
  });
}

// D^l for l = 2..L of all chunk edges, one (edge, row) per thread and level.
template <int L, int l>
__device__ __forceinline__ void wig_level(const Smem& s, int tid) {
  using S = Shape<L>;
  constexpr int w = 2 * l + 1;
#pragma unroll 1
  for (int t = opaque(tid); t < kET * w; t += kThreads) {
    const int e = t / w, mi = t % w;
    float* De = s.D + e * S::DSZ;
    float r1[3][3];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int b = 0; b < 3; ++b) r1[a][b] = De[doff(1) + a * dpad(1) + b];
    const float* Dp = De + doff(l - 1);
    auto rp = [&](int a) { return Dp + (a + l - 1) * dpad(l - 1); };
    float out[w];
    ir_row<l>(mi - l, r1, rp, out);
#pragma unroll
    for (int n = 0; n < w; ++n) {
      De[doff(l) + mi * dpad(l) + n] = out[n];
      s.DT[(wig_off(l) + mi * w + n) * kET + e] = static_cast<_Float16>(out[n]);
    }
  }
  __syncthreads();
  if constexpr (l < L) wig_level<L, l + 1>(s, tid);
}

// Blocks M = 0..L of one chunk: GEMM of M (while block M+1 is rotated in),
// then a barrier so that the next block's operand is complete.
template <int L, int M>
__device__ __forceinline__ void do_block(const MfmaParams& p, const Smem& s, __amdgpu_buffer_rsrc_t wrsrc, int tid,
                                         int wave, const f16x8 (&arbf)[3], const float (&alpha)[16],
                                         NodeAcc (&nacc)[L + 1], WRing& ring) {
  mma_block<L, M>(p, s, wrsrc, tid, wave, arbf, alpha, nacc, ring);
  __syncthreads();
  if constexpr (M < L) do_block<L, M + 1>(p, s, wrsrc, tid, wave, arbf, alpha, nacc, ring);
}

template <int L>
__global__ void __launch_bounds__(kThreads, 1) k_attn_mfma(MfmaParams p) {
  using S = Shape<L>;
  constexpr int K = S::K;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Smem s;
  s.A0 = reinterpret_cast<uint16_t*>(smem);
  s.A1 = reinterpret_cast<uint16_t*>(smem + S::off_A1);
  s.D = reinterpret_cast<float*>(smem + S::off_D);
  s.DT = reinterpret_cast<_Float16*>(smem + S::off_DT);
  s.rbf = reinterpret_cast<float*>(smem + S::off_rbf);
  s.alpha = reinterpret_cast<float*>(smem + S::off_alpha);
  s.q = reinterpret_cast<float*>(smem + S::off_q);
  s.j = reinterpret_cast<int*>(smem + S::off_j);
  s.m_run = reinterpret_cast<float*>(smem + S::off_stat);
  s.l_run = s.m_run + kH;
  s.scale = s.l_run + kH;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16x8*>(p.wpk), (short)0, static_cast<int>(S::wtotal() * 16), 0x00020000);
  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD one
  // contiguous stretch of the spatial order so that neighbouring destinations
  // (which share most neighbours) run on the same L2.
  const int64_t slot = (int64_t)(blockIdx.x & 7) * p.per_xcd + (blockIdx.x >> 3);
  if (slot >= p.n_atoms) return;
  const int64_t i = p.order[slot];

  if (tid < kC) s.q[tid] = p.q[i * kC + tid];
  if (tid < kH) { s.m_run[tid] = -INFINITY; s.l_run[tid] = 0.0f; }
  NodeAcc nacc[L + 1];
#pragma unroll
  for (int l = 0; l <= L; ++l) nacc[l] = NodeAcc{f32x4{}, f32x4{}};
  const float xi[3] = {p.pos[3 * i], p.pos[3 * i + 1], p.pos[3 * i + 2]};
  const int64_t e_beg = p.row_ptr[i], e_end = p.row_ptr[i + 1];
  // the weight stream is the same for every chunk: prime it once
  WRing ring;
  {
    const int voff = opaque(lane) * 16;
    static_for<kRing>([&](auto Gc) { wring_load<L, decltype(Gc)::value>(ring, wrsrc, voff, wave); });
  }

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
    if constexpr (L >= 2) wig_level<L, 2>(s, tid);
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
      // the wave's 32 channels are heads 2w and 2w+1
      const float sa = s.scale[2 * wave], sb = s.scale[2 * wave + 1];
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        nacc[l].a *= sa;
        nacc[l].b *= sb;
      }
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int r = ln & 31;
      arbf[0] = to_vec8<f16x8>(half == 0 ? s.rbf + r * 8 : z);
      arbf[1] = to_vec8<f16x8>(half == 0 ? s.rbf + (r & 15) * 8 : z);
      arbf[2] = to_vec8<f16x8>(half == 0 ? s.rbf + (16 + (r & 15)) * 8 : z);
    }
    build_a0<L>(p, s, tid);
    __syncthreads();
    do_block<L, 0>(p, s, wrsrc, tid, wave, arbf, alpha, nacc, ring);
  }
  __syncthreads();
  {
    const int c0 = 32 * wave + (lane & 15);
    const float la = s.l_run[2 * wave], lb = s.l_run[2 * wave + 1];
    const float ia = la > 0.0f ? 1.0f / la : 0.0f, ib = lb > 0.0f ? 1.0f / lb : 0.0f;
#pragma unroll
    for (int lo = 0; lo <= L; ++lo)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 4 * (lane >> 4) + r;
        if (n < 2 * lo + 1) {
          float* o = p.out + (i * K + lo * lo + n) * kC + c0;
          o[0] = nacc[lo].a[r] * ia;
          o[16] = nacc[lo].b[r] * ib;
        }
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

constexpr int kOrderBits = 6;                       // Morton cells per axis = 64
constexpr int kOrderBins = 1 << (3 * kOrderBits);

__global__ void k_ord_bbox(const float* __restrict__ pos, int64_t n, float* __restrict__ out) {
  __shared__ float smin[3][256], smax[3][256];
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      mn[d] = fminf(mn[d], pos[3 * i + d]);
      mx[d] = fmaxf(mx[d], pos[3 * i + d]);
    }
  for (int d = 0; d < 3; ++d) { smin[d][threadIdx.x] = mn[d]; smax[d][threadIdx.x] = mx[d]; }
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st)
      for (int d = 0; d < 3; ++d) {
        smin[d][threadIdx.x] = fminf(smin[d][threadIdx.x], smin[d][threadIdx.x + st]);
        smax[d][threadIdx.x] = fmaxf(smax[d][threadIdx.x], smax[d][threadIdx.x + st]);
      }
    __syncthreads();
  }
  if (threadIdx.x == 0)
    for (int d = 0; d < 3; ++d) { out[d] = smin[d][0]; out[3 + d] = smax[d][0]; }
}

__device__ __forceinline__ uint32_t spread3(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < kOrderBits; ++b) r |= ((v >> b) & 1u) << (3 * b);
  return r;
}

__global__ void k_ord_keys(const float* __restrict__ pos, int64_t n, const float* __restrict__ bbox,
                           int32_t* __restrict__ key, int32_t* __restrict__ bins) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t c[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    const float ext = fmaxf(bbox[3 + d] - bbox[d], 1e-6f);
    float f = (pos[3 * i + d] - bbox[d]) / ext * float(1 << kOrderBits);
    f = fminf(fmaxf(f, 0.0f), float((1 << kOrderBits) - 1));
    c[d] = static_cast<uint32_t>(f);
  }
  const int32_t k = static_cast<int32_t>(spread3(c[0]) | (spread3(c[1]) << 1) | (spread3(c[2]) << 2));
  key[i] = k;
  atomicAdd(&bins[k], 1);
}

__global__ void k_ord_scatter(int64_t n, const int32_t* __restrict__ key, const int32_t* __restrict__ start,
                              int32_t* __restrict__ cursor, int32_t* __restrict__ order) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int k = key[i];
  order[start[k] + atomicAdd(&cursor[k], 1)] = static_cast<int32_t>(i);
}

struct MfmaWs {
  size_t w, rad, order, key, bins, cursor, bsum, bbox, total;
};

template <int L>
MfmaWs mfma_ws_layout(int64_t n) {
  using S = Shape<L>;
  MfmaWs m{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  m.w = take(S::wtotal() * 16);
  m.rad = take((L + 1) * kC * 16);
  m.order = take(sizeof(int32_t) * n);
  m.key = take(sizeof(int32_t) * n);
  m.bins = take(sizeof(int32_t) * (kOrderBins + 1));
  m.cursor = take(sizeof(int32_t) * kOrderBins);
  m.bsum = take(sizeof(int64_t) * scan_bsum_count(kOrderBins));
  m.bbox = take(8 * sizeof(float));
  m.total = off;
  return m;
}


template <int L>
e2a_status launch_typed(const AttnPlan& pl, hipStream_t st) {
  using S = Shape<L>;
  const e2a_attn_args* a = pl.a;
  const MfmaWs W = mfma_ws_layout<L>(a->n_atoms);
  char* wb = static_cast<char*>(pl.mfma_ws);
  bf16x8* wpk = reinterpret_cast<bf16x8*>(wb + W.w);
  f16x8* radpk = reinterpret_cast<f16x8*>(wb + W.rad);
  int32_t* order = reinterpret_cast<int32_t*>(wb + W.order);
  int32_t* key = reinterpret_cast<int32_t*>(wb + W.key);
  int32_t* bins = reinterpret_cast<int32_t*>(wb + W.bins);
  int32_t* cursor = reinterpret_cast<int32_t*>(wb + W.cursor);
  int64_t* bsum = reinterpret_cast<int64_t*>(wb + W.bsum);
  float* bbox = reinterpret_cast<float*>(wb + W.bbox);
  const int64_t n = a->n_atoms;
  {
    // spatial order of the destination atoms: Morton code of a 64^3 grid over
    // the bounding box, counting-sorted (order only affects locality)
    const int64_t nb = (n + 255) / 256;
    k_ord_bbox<<<1, 256, 0, st>>>(a->pos, n, bbox);
    E2A_HIP_CHECK(hipMemsetAsync(bins, 0, sizeof(int32_t) * (kOrderBins + 1), st));
    E2A_HIP_CHECK(hipMemsetAsync(cursor, 0, sizeof(int32_t) * kOrderBins, st));
    k_ord_keys<<<nb, 256, 0, st>>>(a->pos, n, bbox, key, bins);
    E2A_LAUNCH_CHECK();
    e2a_status ss = exclusive_scan_i32(bins, kOrderBins, cursor, bsum, st);
    if (ss != E2A_OK) return ss;
    // cursor now holds the bin starts; reuse bins as the running cursor
    E2A_HIP_CHECK(hipMemsetAsync(bins, 0, sizeof(int32_t) * (kOrderBins + 1), st));
    k_ord_scatter<<<nb, 256, 0, st>>>(n, key, cursor, bins, order);
    E2A_LAUNCH_CHECK();
  }
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
  p.order = order;
  p.n_atoms = n;
  p.per_xcd = (n + 7) / 8;
  p.out = a->out;
  p.out_lse = a->out_lse;
  for (int d = 0; d < 3; ++d) p.box[d] = pl.box[d];
  p.periodic = pl.periodic;
  p.cutoff = a->cutoff;
  E2A_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_mfma<L>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, S::total));
  hipLaunchKernelGGL(k_attn_mfma<L>, dim3(8 * p.per_xcd), dim3(kThreads), S::total, st, p);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

}  // namespace

bool mfma_supported(int L, int C, int H, int dtype) {
  return L >= 1 && L <= 4 && C == kC && H == kH && dtype == E2A_DTYPE_BF16;
}

size_t mfma_workspace_bytes(int64_t n, int L, int C) {
  if (C != kC) return 0;
  switch (L) {
    case 1: return mfma_ws_layout<1>(n).total;
    case 2: return mfma_ws_layout<2>(n).total;
    case 3: return mfma_ws_layout<3>(n).total;
    case 4: return mfma_ws_layout<4>(n).total;
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

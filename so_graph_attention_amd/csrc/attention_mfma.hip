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
//   * two workgroups of 256 threads share a CU (each under 80 KB of LDS and
//     256 registers per lane), so that one workgroup's latency-bound phases
//     (edge geometry, Wigner-D, softmax, rotate-in) run while the other
//     keeps the matrix cores busy;
//   * per chunk, 32 lanes build the edge frames, D^1 and the radial basis;
//     all 256 threads then extend D^2..D^L level by level (one matrix entry
//     per thread per step, fp32, in the GEMM operand's LDS space, which is
//     free at that point) and compute the 32 x 8 logits; an fp16 copy of D
//     feeds both rotations;
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
//
// The same kernel, instantiated in other modes, computes the EAAS
// convolution stage (section 2.1: every edge weight 1, the messages summed)
// and the two passes of the layer's feature gradient.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 128;      // channels
constexpr int kH = 8;        // heads
constexpr int kDH = 16;      // channels per head
constexpr int kET = 32;      // edges per chunk
constexpr int kThreads = 256;
constexpr int kMinPerWg = 4;       // destinations per workgroup, at least

// Kernel modes: the forward layer, and the two passes of its feature
// gradient.  The query pass recomputes each edge's message and reduces it
// against the destination's cotangent (the softmax gradient ds); the value
// pass carries the cotangents back along the reversed edges through the
// transposed mix.
constexpr int kFwd = 0, kBwdQ = 1, kBwdV = 2;
// Radial pass of the weight gradient: the query pass's recomputation, with
// dW_rad[k][l][c] = sum_edges e_k(r) alpha sum_m y[l,m][c] (D G_i)[l,m][c]
// accumulated per workgroup instead of dalpha.
constexpr int kBwdR = 4;
constexpr int kMaxRadWg = 2048;   // radial pass: at most this many workgroups (partial slots)
// The convolution stage: the forward with every edge weight 1.
constexpr int kConv = 3;
// The query pass with the radial pass's accumulation in the same epilogue:
// both contract y (D G) from one recomputation, so a call that wants ds and
// dW_rad runs the mix once instead of twice.
constexpr int kBwdQR = 5;
__host__ __device__ constexpr bool q_like(int md) { return md == kBwdQ || md == kBwdQR; }
__host__ __device__ constexpr bool r_like(int md) { return md == kBwdR || md == kBwdQR; }

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
  static constexpr int DSZ = doff(L + 1);                       // fp32 D floats per edge (set-up only)
  static constexpr int DT = wig_size(L) * kET;                  // fp16 transposed D, [entry][edge]
  static constexpr int km(int m) { return (L + 1 - m) * kC; }   // GEMM K (= N) of block m
  // query pass: 8-entry slots per (atom, channel) of the fp16 cotangent, one
  // per degree (2 lo + 1 <= 7 entries, zero-padded) and a second for degree 4
  static constexpr int gslots = L >= 4 ? L + 2 : L + 1;
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
  // The last two blocks (m = L-1 and L) are rotated in by one pass over the
  // degree-L feature rows; their operands sit side by side, block L's at
  // a_off(L).
  static constexpr int rup(int x) { return (x + 255) / 256 * 256; }
  static constexpr int a_off(int m) { return m == L && L >= 1 ? rup(abytes(L - 1)) : 0; }
  static constexpr int aregion() {
    int b = amax();
    if (a_off(L) + abytes(L) > b) b = a_off(L) + abytes(L);
    if (kET * DSZ * 4 > b) b = kET * DSZ * 4;
    return rup(b);
  }
  // LDS layout (bytes): the GEMM operand region, which also holds the fp32
  // D of the chunk while the recursion runs
  static constexpr int off_DT = aregion();
  static constexpr int off_rbf = off_DT + DT * 2;
  static constexpr int off_alpha = off_rbf + kET * 8 * 4;
  static constexpr int off_q = off_alpha + kET * kH * 4;
  static constexpr int off_j = off_q + 2 * kC * 4;
  static constexpr int off_stat = off_j + kET * 4;
  static constexpr int total = off_stat + 5 * kH * 4;
  static_assert(total <= 80 * 1024, "two workgroups per CU");
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

// Materialises a running sum where it stands: without it the whole chain of
// additions is sunk to the sum's last use, with every term held live (or
// spilled) until then.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(const f16x8 a, const f16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8 a, const bf16x8 b, const f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Node accumulator of one degree lo for this wave's 32 channels: two 16x16
// MFMA tiles (columns = channels 0-15 and 16-31 of the wave).  Lane l holds
// rows 4 (l / 16) + r, column l % 16.
struct NodeAcc {
  f32x4 a;   // channels 32 w + 0..15
  f32x4 b;   // channels 32 w + 16..31
};

// A chunk carries the edges of at most two destination atoms: A (the first
// nA edge slots) and B (the next nB, starting B's list).  For lo <= 3 both
// share acc[lo]: rows 0-7 hold A's 2 lo + 1 output rows (lanes 0-31) and
// rows 8-15 B's (lanes 32-63).  Degree 4 needs 9 rows, so B's part of it
// goes to `hi`.  B's rows are zero whenever a chunk starts.
template <int L>
struct NodeState {
  NodeAcc acc[L + 1];
  NodeAcc hi;
  float dal[16];   // query pass: dalpha partials of the lane's 16 edges crow(r, half), its channel
  NodeAcc rad[3];  // radial pass: dW_rad of degree pairs (0, 1), (2, 3), (4): rows 0-7 even, 8-15 odd degree
};
template <int LO>
__host__ __device__ constexpr bool packed_lo() { return 2 * LO + 1 <= 8; }

// Rotate-out contraction step: acc[n][c] += sum_k G[n][k] U[k][c] over the 16
// (edge, sign) slots this k-step carries.  The 32x32 GEMM result gives lane l
// the values of channel l % 32 for 8 edges (lanes 0-31 and 32-63 hold
// different edges).  In the 16x16x32 MFMA, k-slot group g = l / 16 comes from
// lanes 16 g .. 16 g + 15: groups 0 and 2 carry channels 0-15, groups 1 and 3
// channels 16-31, so each of the two MFMAs keeps its own groups and zeroes
// the others.  G (the D rows) is the same register for both.
__device__ __forceinline__ void rotate_out_step(NodeAcc& acc, const bf16x8 g, const bf16x8 u, bool grp_odd) {
  const bf16x8 zero = {};
  acc.a = mfma16_bf16(g, grp_odd ? zero : u, acc.a);
  acc.b = mfma16_bf16(g, grp_odd ? u : zero, acc.b);
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
  const bf16x8* radpk;    // W_rad as [(L+1) C] vectors of its 8 basis weights (bf16, exact)
  const int32_t* order;   // destination atoms in spatial (Morton) order
  const int64_t* xcd_lo;  // [9] the XCD ranges of the order, split by edges (null: by atoms)
  const int32_t* sched;   // balanced deal: per workgroup, its slots of `order` in turn (null: cyclic)
  const int32_t* sched_n; // per workgroup, the number of slots in its row of sched
  int64_t sched_len;      // row length of sched
  int64_t n_atoms;
  int wg_per_xcd;
  float* out;
  float* out_lse;
  float box[3];
  int periodic;
  float cutoff;
  // feature gradient
  const float* lse;        // the forward's log-normaliser [N, H]
  const float* delta;      // query pass: sum_{k, c in h} G_i o_i [N, H]
  const f16x8* gpk;        // query pass: scaled fp16 cotangent, [N][gslots][C] vectors of 8
  const float* gsc;        // query pass: per-atom inverse scale of gpk
  const float* gnorm;      // value pass: power of two that brings max |G| into [1, 2)
  float* rad_part;         // radial pass: per-workgroup dW_rad partials [WG][8][(L+1) C], times gnorm
  float* ds;               // query pass: softmax gradient [E, H]
};

struct Smem {
  uint16_t* A;     // GEMM operand of the current |m| block
  float* D;        // fp32 D^0..D^L of the chunk (aliases A; set-up only)
  _Float16* DT;    // fp16 D, [entry][edge]
  float* rbf;
  float* alpha;    // [edge][head]: logits, then softmax weights
  float* q;        // [2][C]: queries of destinations A and B
  int* j;
  float* m_run;    // [2][H] running max of A and B
  float* l_run;    // [2][H] running normaliser of A and B
  float* scale;    // [H] rescale of A's accumulators in this chunk
};

// Per-lane constants of one chunk.
struct Lane {
  float alpha[16];   // softmax weights of the 16 edges whose GEMM rows the lane holds (its head)
  bf16x8 arbf[3];    // radial-basis A operands (all 32 edges; edges 0-15; edges 16-31)
  u32x4 mk[2];       // per fp16 pair of the rotate-out operand: keep A's edges (edge groups 0, 16)
  uint32_t flip;     // ~0 on lanes whose packed rows (n >= 8) belong to B
  int nA;            // query pass: edges 0 .. nA-1 belong to A
  int64_t ia, ib;    // query pass: atom ids of A and B
  float gsA, gsB;    // query pass: inverse cotangent scales of A and B
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
  constexpr int l = MN + (TAU >> 1);
  const int e = (tid >> 4) + 16 * (TAU & 1);
  const _Float16* dl = s.DT + wig_off(l) * kET + e;
  float hv[8];
  unpack_bf16x8(raw[N], hv);
  const float dp = static_cast<float>(dl[((l + MN) * (2 * l + 1) + N) * kET]);
#pragma unroll
  for (int q = 0; q < 8; ++q) xp[q] = (N == 0 ? 0.0f : xp[q]) + dp * hv[q];
  if constexpr (MN > 0) {
    const float dm = static_cast<float>(dl[((l - MN) * (2 * l + 1) + N) * kET]);
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

// Value pass: rho[l][c] = sum_k rbf[e][k] W_rad[k][l][c] for the thread's 8
// channels 8 g .. 8 g + 7 (g = lane % 16) and its two edges (tid / 16 and
// tid / 16 + 16), as 16x16x32 fp16 products whose result lands in exactly
// that layout: row 4 i + r, column g of product h is rho[e_i][8 g + 4 h + r]
// for the wave's edge i = lane / 16.  The k index 8 r' + kb pairs basis
// function kb with channel offset r': A's row 4 i + r holds edge i's basis
// values in group r' = r only, B's column g holds the 8 basis weights of
// channel 8 g + r' + 4 h (one packed vector).  Operands and precision are
// those of the forward's radial product.
template <int L>
__device__ __forceinline__ void rho_pair(const MfmaParams& p, const Smem& s, int tid, int l, float (&rho)[2][8]) {
  // rebuilt in every call (a fresh lane index) rather than kept live across the chunk
  const int lane = opaque(tid) & 63, wave = tid >> 6;
  const int e = 4 * wave + ((lane & 15) >> 2);   // the edge of A's row lane % 16
  const bool diag = (lane & 3) == (lane >> 4);
  bf16x8 a0 = {}, a1 = {};
  if (diag) {
    a0 = to_vec8<bf16x8>(s.rbf + e * 8);
    a1 = to_vec8<bf16x8>(s.rbf + (e + 16) * 8);
  }
  const bf16x8* wl = p.radpk + l * kC + 8 * (lane & 15) + (lane >> 4);
  const bf16x8 b0 = wl[0], b1 = wl[4];
  const f32x4 z = {};
  const f32x4 r00 = mfma16_bf16(a0, b0, z), r01 = mfma16_bf16(a0, b1, z);
  const f32x4 r10 = mfma16_bf16(a1, b0, z), r11 = mfma16_bf16(a1, b1, z);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rho[0][r] = r00[r];
    rho[0][4 + r] = r01[r];
    rho[1][r] = r10[r];
    rho[1][4 + r] = r11[r];
  }
}

template <int L, int MN, int TAU, int MD>
__device__ __forceinline__ void task_compute(const Smem& s, uint16_t* A, int tid, const uint4 (&raw)[2 * L + 1],
                                             const float (&rho)[8]) {
  constexpr int l = MN + (TAU >> 1);
  constexpr int W = 2 * l + 1;
  float xp[8], xm[8];
  static_for<W>([&](auto nc) { task_term<L, MN, TAU, decltype(nc)::value>(s, tid, raw, xp, xm); });
  if constexpr (MD == kBwdV) {
    // value pass: the rotated cotangent is scaled by the edge's weight
    // alpha (its head) and by the radial weights rho[l][c] of this degree
    const int e = (tid >> 4) + 16 * (TAU & 1);
    const float a = s.alpha[e * kH + 8 * (tid & 15) / kDH];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      xp[q] *= a * rho[q];
      xm[q] *= a * rho[q];
    }
  }
  task_store<L, MN, TAU>(A, tid, xp, xm);
}

// Rotate-in of block MN: all its tasks, the loads of task tau+1 issued before
// task tau's arithmetic.
template <int L, int MN, int MD>
__device__ __forceinline__ void rotate_in(const MfmaParams& p, const Smem& s, int tid) {
  using S = Shape<L>;
  static_assert(kThreads == 16 * kET / 2, "two edges x 16 channel groups per thread");
  constexpr int NT = 2 * (L + 1 - MN);
  // for MN = L-1 the last two tasks (degree L) also produce block L
  constexpr bool pair = MN == L - 1;
  tid = opaque(tid);
  uint4 raw[2][2 * L + 1];
  float rho[2][8];   // value pass: rho of the current degree for the thread's two edges
  // the rotate-in runs at a raised wave priority, so that when the two
  // workgroups of a CU are in different phases the issue arbiter does not
  // treat their waves alike (measured: 3.5% less time per launch at 100k
  // atoms; raising the GEMM instead, or both at different levels, gave the
  // same; results are bit-identical)
  __builtin_amdgcn_s_setprio(1);
  task_load<L, MN, 0>(p, s, tid, raw[0]);
  static_for<NT>([&](auto tc) {
    constexpr int tau = decltype(tc)::value;
    if constexpr (tau + 1 < NT) task_load<L, MN, tau + 1>(p, s, tid, raw[(tau + 1) & 1]);
    // tasks 2d and 2d+1 share degree MN + d (one edge each)
    if constexpr (MD == kBwdV && tau % 2 == 0) rho_pair<L>(p, s, tid, MN + tau / 2, rho);
    task_compute<L, MN, tau, MD>(s, s.A + S::a_off(MN) / 2, tid, raw[tau & 1], rho[tau & 1]);
    if constexpr (pair && tau >= NT - 2)
      task_compute<L, L, tau - (NT - 2), MD>(s, s.A + S::a_off(L) / 2, tid, raw[tau & 1], rho[tau & 1]);
  });
  __builtin_amdgcn_s_setprio(0);
}

// A operand of the rotate-out contraction: row n of D^l rows `mrow`, for the
// 8 edges eg + crow(q, h), q = 0..7, read as fp16 and rounded to bf16 (the
// type of the other operand, whose range is fp32's).  Rows n >= 2l+1 are zero.
__device__ __forceinline__ bf16x8 dt_frag(const _Float16* row_base, int eg, int h, bool valid) {
  f16x8 v = {};
  if (valid) {
    const f16x4 a = *reinterpret_cast<const f16x4*>(row_base + eg + 4 * h);
    const f16x4 b = *reinterpret_cast<const f16x4*>(row_base + eg + 8 + 4 * h);
    v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  return __builtin_convertvector(__builtin_convertvector(v, f32x8), bf16x8);
}

// Rotate-out of one fragment: D^LO row `row`, the 8 edges of group eg that
// this lane's k-slots carry, contracted with u into the node accumulators.
// Packed degrees: the lane's D column is n mod 8 and the G entries of the
// other destination's edges are zero.  Degree 4: A's edges go to acc[4] and,
// when the chunk has a B, B's edges to hi.
template <int L, int LO, int ROW, int EG>
__device__ __forceinline__ void rot_out(NodeState<L>& ns, const Smem& s, const Lane& ln, int lane, const bf16x8 u,
                                        bool has_b) {
  constexpr int W = 2 * LO + 1;
  const int n = lane & 15;
  const int ncol = packed_lo<LO>() ? (n & 7) : n;
  const bool grp_odd = (lane >> 4) & 1;    // lane group 1 or 3: channels 16-31
  const _Float16* drow = s.DT + (wig_off(LO) + ROW * W + ncol) * kET;
  const u32x4 g = __builtin_bit_cast(u32x4, dt_frag(drow, EG, lane >> 5, ncol < W));
  const u32x4 mA = ln.mk[EG / 16];
  if constexpr (packed_lo<LO>()) {
    rotate_out_step(ns.acc[LO], __builtin_bit_cast(bf16x8, g & (mA ^ ln.flip)), u, grp_odd);
  } else {
    rotate_out_step(ns.acc[LO], __builtin_bit_cast(bf16x8, g & mA), u, grp_odd);
    if (has_b) rotate_out_step(ns.hi, __builtin_bit_cast(bf16x8, g & ~mA), u, grp_odd);
  }
}

// Radial pass: degree LO's share of the chunk's dW_rad,
// acc[k][c] += sum over the 8 edges EG + crow(q, h) of rbf[edge][k] t[edge][c],
// with the rotate-out's k-slot layout (t in the GEMM result's registers as
// the B operand, the basis values in place of the D rows as A).  Degrees
// share accumulator tiles in pairs: an even degree uses rows 0-7 (k), an odd
// one rows 8-15.
template <int L, int LO, int EG>
__device__ __forceinline__ void rad_acc(NodeState<L>& ns, const Smem& s, int lane, const bf16x8 t) {
  const int row = lane & 15;
  const bool valid = (LO & 1) ? row >= 8 : row < 8;
  const int k = row & 7, h = lane >> 5;
  bf16x8 a = {};
  if (valid) {
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = static_cast<__bf16>(s.rbf[(EG + crow(q, h)) * 8 + k]);
  }
  rotate_out_step(ns.rad[LO / 2], a, t, (lane >> 4) & 1);
}

// 16-byte load of a B fragment through a buffer resource: the per-lane offset
// stays in one VGPR and the k-step advances a scalar offset.
__device__ __forceinline__ bf16x8 load_b(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return __builtin_bit_cast(bf16x8, v);
}

constexpr int kRing = 2;   // weight k-steps in flight per wave
struct WRing {
  bf16x8 r[kRing][2];
};

// Loads chunk step G of the weight stream into its ring slot G % kRing.
template <int L, int G>
__device__ __forceinline__ void wring_load(WRing& ring, __amdgpu_buffer_rsrc_t wrsrc, int voff, int wave) {
  using S = Shape<L>;
  // the ring runs on from one chunk into the next, so the step after the
  // last of a chunk (step 0 again) must land in the slot that step frees
  static_assert(S::stot() % kRing == 0, "chunk step count must be a multiple of the ring depth");
  constexpr int m = S::stream_m(G);
  constexpr int off0 = S::stream_off(G, 0);
  constexpr int off1 = S::stream_off(G, 1);
  // the wave's column term goes into the per-lane offset, so that the scalar
  // offsets are constants (rematerialised, never kept live in SGPRs)
  const int vo = voff + wave * static_cast<int>(S::wave_bytes(m));
  ring.r[G % kRing][0] = load_b(wrsrc, vo, off0);
  if constexpr (S::stream_has1(G)) ring.r[G % kRing][1] = load_b(wrsrc, vo, off1);
}

// Query pass: B operands of degree LO's rotated cotangent, this lane's
// channel 32 wave + lane % 32.  Degrees up to 3 carry A's G in k = 0-7 (lanes
// 0-31) and B's in k = 8-15 (lanes 32-63); degree 4 has one operand per
// destination, k = n (slot 4 holds n = 0-7, slot 5 n = 8).
template <int L, int LO>
__device__ __forceinline__ void grad_frags(const MfmaParams& p, const Lane& ln, int lane, int wave, f16x8& g0,
                                           f16x8& g1) {
  constexpr int NSL = Shape<L>::gslots;
  const int half = lane >> 5;
  const int c = 32 * wave + (lane & 31);
  if constexpr (LO < 4) {
    // arithmetic, not a select: a select here becomes a load through a
    // selected pointer into a private copy of the lane constants
    const int64_t id = ln.ia + half * (ln.ib - ln.ia);
    g0 = p.gpk[(id * NSL + LO) * kC + c];
  } else {
    g0 = p.gpk[(ln.ia * NSL + 4 + half) * kC + c];
    g1 = p.gpk[(ln.ib * NSL + 4 + half) * kC + c];
  }
}

// Query pass: the cotangent of each row's destination in the edge's frame,
// (D^LO G_dest)[row][c] = sum_n D^LO[row][n] G_dest[LO^2 + n][c], for the 32
// rows of one output tile of block M: for M = 0 edge r (0-31) and D row LO;
// for M > 0 edge 16 T + r % 16, D row LO + M (r < 16) or LO - M.  One matrix
// product over k = n per destination, with the D entries (fp16, from LDS) as
// A, the row r = lane % 32 and entries 8 (lane / 32) .. +7; a row keeps only
// the half of k, or the product, that carries its own destination's G.  The
// result is in G's scale (the destination's gsc undoes it).
template <int L, int LO, int M, int T>
__device__ __forceinline__ f32x16 rot_grad(const Smem& s, const Lane& ln, int lane, const f16x8 g0,
                                           const f16x8 g1) {
  constexpr int W = 2 * LO + 1;
  // nothing here depends on the GEMM: a fresh lane index keeps these reads
  // and products after it, instead of hoisted above it with their results
  // held (or spilled) across the k-loop
  lane = opaque(lane);
  const int half = lane >> 5;
  const int r = lane & 31;
  const int e = M == 0 ? r : 16 * T + (r & 15);
  const int mrow = M == 0 ? LO : (r < 16 ? LO + M : LO - M);
  const _Float16* dr = s.DT + (wig_off(LO) + mrow * W) * kET + e;
  const bool in_a = e < ln.nA;
  f16x8 a = {};
  if constexpr (LO < 4) {
#pragma unroll
    for (int q = 0; q < W; ++q) a[q] = dr[q * kET];
    const u32x4 keep = (in_a == (half == 0)) ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
    return mfma_f16(__builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, a) & keep), g0, f32x16{});
  } else {
    // k = 8-15 carry n = 8 in their first entry; the others meet zeros in B
    a[0] = dr[8 * half * kET];
#pragma unroll
    for (int q = 1; q < 8; ++q) a[q] = dr[q * kET];
    const u32x4 av = __builtin_bit_cast(u32x4, a);
    const u32x4 ma = in_a ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
    const f32x16 g = mfma_f16(__builtin_bit_cast(f16x8, av & ma), g0, f32x16{});
    return mfma_f16(__builtin_bit_cast(f16x8, av & ~ma), g1, g);
  }
}

// One exchange step of a reduce-scatter over a row of 16 lanes: the partner
// (through DPP control CTRL) differs from this lane in bit B of the lane
// index; of the 2N values the lane keeps the half that bit selects and adds
// the partner's copy of it.
template <int CTRL, int B, int N>
__device__ __forceinline__ void rs_step(float (&v)[16], int lane) {
  const bool up = (lane & B) != 0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float send = up ? v[k] : v[k + N];
    const float keep = up ? v[k + N] : v[k];
    const int got = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), CTRL, 0xF, 0xF, false);
    v[k] = keep + __builtin_bit_cast(float, got);
  }
}

// Sum of v[r] over the 16 lanes of this lane's row, returned in lane r of the
// row (r = lane % 16).  Partners: 15 - i (row mirror), 7 - i (half mirror),
// i ^ 2 and i ^ 1 (quad permutations); they flip bits 3, 2, 1, 0 in turn.
__device__ __forceinline__ float row_reduce_scatter16(float (&v)[16], int lane) {
  rs_step<0x140, 8, 8>(v, lane);
  rs_step<0x141, 4, 4>(v, lane);
  rs_step<0x4E, 2, 2>(v, lane);
  rs_step<0xB1, 1, 1>(v, lane);
  return v[0];
}

// GEMM of block M for this wave's 32 output channels, then the epilogue of
// each output block: y_{+-m} from the W1/W2 products, u = alpha * rho * y
// (rho from one MFMA against the radial basis), and the partial rotate-out
// acc_lo[n][c] += sum_{edges, +-} D^lo[lo +- M][n] u_{+-}[c], itself an MFMA
// contraction over the chunk's edges.
//
// Software pipeline, all fixed at compile time: the weight stream runs kRing
// k-steps ahead (continuing into the next block and the next chunk, whose
// weights are the same) and A fragments one step ahead.  A scheduling
// barrier after every k-step keeps the compiler from undoing this order.
template <int L, int M, int MD>
__device__ __forceinline__ void mma_block(const MfmaParams& p, const Smem& s, __amdgpu_buffer_rsrc_t wrsrc,
                                          int tid, int wave, const Lane& ln, bool has_b, NodeState<L>& ns,
                                          WRing& ring) {
  using S = Shape<L>;
  constexpr int KS = S::ks(M);
  constexpr int stride = S::astride(M);
  tid = opaque(tid);
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int c_own = 32 * wave + (lane & 31);
  const int voff = lane * 16;
  const f16x8 zero8 = {};
  const uint16_t* ap0 = s.A + S::a_off(M) / 2 + (lane & 31) * stride + 8 * half;
  const uint16_t* ap1 = ap0 + 32 * stride;   // second row tile (m > 0 only)
  bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ap0);
  bf16x8 a1 = {};
  if constexpr (M > 0) a1 = *reinterpret_cast<const bf16x8*>(ap1);
  static_for<S::nb(M)>([&](auto bc) {
    constexpr int b = decltype(bc)::value;
    f32x16 c00 = {}, c01 = {}, c10 = {}, c11 = {};
    // radial-weight fragments of this block's output degrees, fetched now so
    // that they have landed by the epilogue
    bf16x8 brad0 = {}, brad1 = {};
    if (MD != kBwdV && MD != kBwdR && half == 0) {
      brad0 = p.radpk[S::blk_lo(M, b, 0) * kC + c_own];
      if constexpr (M == 0 && S::has1(M, b)) brad1 = p.radpk[S::blk_lo(M, b, 1) * kC + c_own];
    }
    // query pass: the destinations' cotangent of the block's output degrees
    // (a pair of degrees below 4, or degree 4 alone: two operands at most)
    f16x8 gq0 = zero8, gq1 = zero8;
    if constexpr (q_like(MD) || r_like(MD)) {
      if constexpr (M == 0 && S::has1(M, b)) {
        grad_frags<L, S::blk_lo(M, b, 0)>(p, ln, lane, wave, gq0, gq1);
        grad_frags<L, S::blk_lo(M, b, 1)>(p, ln, lane, wave, gq1, gq1);
      } else {
        grad_frags<L, S::blk_lo(M, b, 0)>(p, ln, lane, wave, gq0, gq1);
      }
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
      if constexpr (M == 0 && !S::has1(M, b)) {
        // a single output degree: alternate two accumulators so that
        // consecutive MFMAs do not wait on each other's result
        if constexpr (st % 2 == 0) c00 = mfma_bf16(a0, b0, c00);
        else c01 = mfma_bf16(a0, b0, c01);
      } else {
        c00 = mfma_bf16(a0, b0, c00);
      }
      if constexpr (M == 0) {
        if constexpr (S::has1(M, b)) c01 = mfma_bf16(a0, b1, c01);
      } else {
        c01 = mfma_bf16(a0, b1, c01);
        c10 = mfma_bf16(a1, b0, c10);
        c11 = mfma_bf16(a1, b1, c11);
      }
      a0 = a0n;
      a1 = a1n;
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (M == 0) {
      static_for<2>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        if constexpr (f == 0 || S::has1(M, b)) {
          constexpr int lo = S::blk_lo(M, b, f);
          const f32x16 c0 = f == 0 ? (S::has1(M, b) ? c00 : c00 + c01) : c01;
          if constexpr (MD == kBwdV) {
            // value pass: alpha and rho were applied to the rotated input
            float u[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) u[r] = c0[r];
            rot_out<L, lo, lo, 0>(ns, s, ln, lane, to_vec8<bf16x8>(u), has_b);
            rot_out<L, lo, lo, 16>(ns, s, ln, lane, to_vec8<bf16x8>(u + 8), has_b);
          } else if constexpr (MD == kBwdR) {
            // t = alpha y (D G) per (edge, channel), alpha carrying the edge's scales
            const f32x16 gt = rot_grad<L, lo, 0, 0>(s, ln, lane, f == 0 ? gq0 : gq1, gq1);
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) t[r] = ln.alpha[r] * c0[r] * gt[r];
            rad_acc<L, lo, 0>(ns, s, lane, to_vec8<bf16x8>(t));
            rad_acc<L, lo, 16>(ns, s, lane, to_vec8<bf16x8>(t + 8));
          } else {
            const bf16x8 brad = f == 0 ? brad0 : brad1;
            const f32x16 rho = mfma_bf16(ln.arbf[0], brad, f32x16{});
            if constexpr (q_like(MD)) {
              // the two operands are (lo0, lo1) for a pair, (A, B) for degree 4
              const f32x16 gt = rot_grad<L, lo, 0, 0>(s, ln, lane, f == 0 ? gq0 : gq1, gq1);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                ns.dal[r] += rho[r] * c0[r] * gt[r];
                pin(ns.dal[r]);
              }
              if constexpr (MD == kBwdQR) {
                // the radial pass's t, as that pass forms it
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) t[r] = ln.alpha[r] * c0[r] * gt[r];
                rad_acc<L, lo, 0>(ns, s, lane, to_vec8<bf16x8>(t));
                rad_acc<L, lo, 16>(ns, s, lane, to_vec8<bf16x8>(t + 8));
              }
            } else {
              float u[16];
#pragma unroll
              for (int r = 0; r < 16; ++r) u[r] = ln.alpha[r] * rho[r] * c0[r];
              rot_out<L, lo, lo, 0>(ns, s, ln, lane, to_vec8<bf16x8>(u), has_b);
              rot_out<L, lo, lo, 16>(ns, s, ln, lane, to_vec8<bf16x8>(u + 8), has_b);
            }
          }
        }
      });
    } else {
      constexpr int lo = S::blk_lo(M, b, 0);
      const bf16x8 brad = brad0;
      static_for<2>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const f32x16& C1 = t == 0 ? c00 : c10;
        const f32x16& C2 = t == 0 ? c01 : c11;
        if constexpr (MD == kBwdV) {
          float up[8], um[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            up[r] = C1[r] - C2[r + 8];
            um[r] = C2[r] + C1[r + 8];
          }
          rot_out<L, lo, lo + M, 16 * t>(ns, s, ln, lane, to_vec8<bf16x8>(up), has_b);
          rot_out<L, lo, lo - M, 16 * t>(ns, s, ln, lane, to_vec8<bf16x8>(um), has_b);
        } else if constexpr (MD == kBwdR) {
          // the edge's +M and -M rows summed: drho takes sum over m
          const f32x16 gt = rot_grad<L, lo, M, t>(s, ln, lane, gq0, gq1);
          float ts[8];
#pragma unroll
          for (int r = 0; r < 8; ++r)
            ts[r] = ln.alpha[8 * t + r] * ((C1[r] - C2[r + 8]) * gt[r] + (C2[r] + C1[r + 8]) * gt[r + 8]);
          rad_acc<L, lo, 16 * t>(ns, s, lane, to_vec8<bf16x8>(ts));
        } else {
          const f32x16 rho = mfma_bf16(ln.arbf[1 + t], brad, f32x16{});
          if constexpr (q_like(MD)) {
            // tile rows r and r + 16 are the +M and -M rows of one edge
            const f32x16 gt = rot_grad<L, lo, M, t>(s, ln, lane, gq0, gq1);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              ns.dal[8 * t + r] += rho[r] * ((C1[r] - C2[r + 8]) * gt[r] + (C2[r] + C1[r + 8]) * gt[r + 8]);
              pin(ns.dal[8 * t + r]);
            }
            if constexpr (MD == kBwdQR) {
              float ts[8];
#pragma unroll
              for (int r = 0; r < 8; ++r)
                ts[r] = ln.alpha[8 * t + r] * ((C1[r] - C2[r + 8]) * gt[r] + (C2[r] + C1[r + 8]) * gt[r + 8]);
              rad_acc<L, lo, 16 * t>(ns, s, lane, to_vec8<bf16x8>(ts));
            }
          } else {
            float up[8], um[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              const float sc = ln.alpha[r + 8 * t] * rho[r];
              up[r] = sc * (C1[r] - C2[r + 8]);
              um[r] = sc * (C2[r] + C1[r + 8]);
            }
            rot_out<L, lo, lo + M, 16 * t>(ns, s, ln, lane, to_vec8<bf16x8>(up), has_b);
            rot_out<L, lo, lo - M, 16 * t>(ns, s, ln, lane, to_vec8<bf16x8>(um), has_b);
          }
        }
      });
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

// Blocks M = 0..L of one chunk: rotate-in of M into the operand region, a
// barrier, the GEMM of M, and a barrier before the region is rewritten;
// blocks L-1 and L share one rotate-in pass and run their GEMMs back to back.
template <int L, int M, int MD>
__device__ __forceinline__ void do_block(const MfmaParams& p, const Smem& s, __amdgpu_buffer_rsrc_t wrsrc, int tid,
                                         int wave, const Lane& ln, bool has_b, NodeState<L>& ns, WRing& ring) {
  rotate_in<L, M, MD>(p, s, tid);
  __syncthreads();
  mma_block<L, M, MD>(p, s, wrsrc, tid, wave, ln, has_b, ns, ring);
  if constexpr (M == L - 1) {
    // block L was rotated in with block L-1 and has its own operand space
    mma_block<L, L, MD>(p, s, wrsrc, tid, wave, ln, has_b, ns, ring);
    __syncthreads();
  } else {
    __syncthreads();
    if constexpr (M < L) do_block<L, M + 1, MD>(p, s, wrsrc, tid, wave, ln, has_b, ns, ring);
  }
}

// Writes destination A's output (the normalised node accumulator, lanes of
// rows 0-7 for packed degrees) and its log-normaliser, then moves B's partial
// state into A's place and clears B's.
template <int L>
__device__ __forceinline__ void finish_a(const MfmaParams& p, const Smem& s, NodeState<L>& ns, int64_t i, int tid,
                                         int wave) {
  constexpr int K = Shape<L>::K;
  tid = opaque(tid);
  const int lane = tid & 63;
  __syncthreads();
  {
    const int c0 = 32 * wave + (lane & 15);
    const float la = s.l_run[2 * wave], lb = s.l_run[2 * wave + 1];
    const float ia = la > 0.0f ? 1.0f / la : 0.0f, ib = lb > 0.0f ? 1.0f / lb : 0.0f;
    static_for<L + 1>([&](auto lc) {
      constexpr int lo = decltype(lc)::value;
      if (packed_lo<lo>() ? lane < 32 : true) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 4 * (lane >> 4) + r;
          if (n < 2 * lo + 1) {
            float* o = p.out + (i * K + lo * lo + n) * kC + c0;
            o[0] = ns.acc[lo].a[r] * ia;
            o[16] = ns.acc[lo].b[r] * ib;
          }
        }
      }
    });
  }
  if (p.out_lse && tid < kH)
    p.out_lse[i * kH + tid] = s.l_run[tid] > 0.0f ? s.m_run[tid] + logf(s.l_run[tid]) : -INFINITY;
  __syncthreads();
  if (tid < kH) {
    s.m_run[tid] = s.m_run[kH + tid];
    s.l_run[tid] = s.l_run[kH + tid];
    s.m_run[kH + tid] = -INFINITY;
    s.l_run[kH + tid] = 0.0f;
  }
  static_for<L + 1>([&](auto lc) {
    constexpr int lo = decltype(lc)::value;
    if constexpr (packed_lo<lo>()) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float va = __shfl_down(ns.acc[lo].a[r], 32);
        const float vb = __shfl_down(ns.acc[lo].b[r], 32);
        ns.acc[lo].a[r] = lane < 32 ? va : 0.0f;
        ns.acc[lo].b[r] = lane < 32 ? vb : 0.0f;
      }
    } else {
      ns.acc[lo] = ns.hi;
      ns.hi = NodeAcc{f32x4{}, f32x4{}};
    }
  });
}

// Uniform description of one chunk: nA edge slots of destination A (its
// edges a0 .. a0 + nA - 1), then nB slots of destination B (its first nB).
struct ChunkPlan {
  int64_t sa, a0;     // A's slot in the spatial order, and its first edge in the chunk
  int64_t ia, ib;     // atom ids of A and B (ib = ia without B)
  int64_t ea, eb;     // first neighbour-list entry of A's and B's part
  int64_t sb;         // B's slot
  int nA, nB;
  bool a_done, b_done;
};

// The workgroup's destinations at positions s_lo, s_lo + step, ... (< s_hi)
// of its sequence (the spatial order itself, or its row `seq` of the
// balanced deal): their concatenated neighbour lists in chunks of 32 edge
// slots; a chunk holds the rest of the current atom A and, when A ends inside
// it, the start of the next atom B.  Only the last chunk is padded.
template <int L, int MD>
__device__ __forceinline__ void stretch(const MfmaParams& p, const Smem& s, __amdgpu_buffer_rsrc_t wrsrc, int tid0,
                                        int wave, const int32_t* seq, int64_t s_lo, int64_t s_hi, int64_t step,
                                        NodeState<L>& ns, WRing& ring);

// A persistent workgroup processes its share of its XCD's range of the
// spatial order: every wg_per_xcd-th destination (cyclic deal), or its row of
// the balanced deal.
template <int L, int MD>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) k_attn_mfma(MfmaParams p) {
  using S = Shape<L>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Smem s;
  s.A = reinterpret_cast<uint16_t*>(smem);
  s.D = reinterpret_cast<float*>(smem);
  s.DT = reinterpret_cast<_Float16*>(smem + S::off_DT);
  s.rbf = reinterpret_cast<float*>(smem + S::off_rbf);
  s.alpha = reinterpret_cast<float*>(smem + S::off_alpha);
  s.q = reinterpret_cast<float*>(smem + S::off_q);
  s.j = reinterpret_cast<int*>(smem + S::off_j);
  s.m_run = reinterpret_cast<float*>(smem + S::off_stat);
  s.l_run = s.m_run + 2 * kH;
  s.scale = s.l_run + 2 * kH;

  const int tid0 = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16x8*>(p.wpk), (short)0, static_cast<int>(S::wtotal() * 16), 0x00020000);
  if (tid0 < 2 * kH) { s.m_run[tid0] = -INFINITY; s.l_run[tid0] = 0.0f; }
  NodeState<L> ns;
#pragma unroll
  for (int l = 0; l <= L; ++l) ns.acc[l] = NodeAcc{f32x4{}, f32x4{}};
  ns.hi = NodeAcc{f32x4{}, f32x4{}};
#pragma unroll
  for (int t = 0; t < 3; ++t) ns.rad[t] = NodeAcc{f32x4{}, f32x4{}};
  // the weight stream is the same for every chunk: prime it once
  WRing ring;
  {
    const int voff = opaque(tid0 & 63) * 16;
    static_for<kRing>([&](auto Gc) { wring_load<L, decltype(Gc)::value>(ring, wrsrc, voff, wave); });
  }

  // Workgroups are dealt to the 8 XCDs round-robin.  Each XCD owns one
  // eighth of the spatial order, dealt to its workgroups in rounds of
  // consecutive destinations: at any time they work on neighbouring
  // destinations, which share most of their neighbours' features in the
  // XCD's L2.  The balanced deal (k_deal) chooses which workgroup takes which
  // destination of a round; without it workgroup w takes the w-th.
  const int xcd = blockIdx.x & 7;
  const int64_t x_lo = p.xcd_lo ? p.xcd_lo[xcd] : xcd * p.n_atoms / 8;
  const int64_t x_hi = p.xcd_lo ? p.xcd_lo[xcd + 1] : (xcd + 1) * p.n_atoms / 8;
  const bool dealt = p.sched != nullptr;
  const int32_t* seq = dealt ? p.sched + (int64_t)blockIdx.x * p.sched_len : nullptr;
  const int64_t s_lo = dealt ? 0 : x_lo + (blockIdx.x >> 3);
  const int64_t s_hi = dealt ? p.sched_n[blockIdx.x] : x_hi;
  const int64_t step = dealt ? 1 : p.wg_per_xcd;
  stretch<L, MD>(p, s, wrsrc, tid0, wave, seq, s_lo, s_hi, step, ns, ring);
  if constexpr (r_like(MD)) {
    // lane l holds rows 4 (l / 16) + i (basis k of an even or odd degree),
    // channel 32 wave + l % 16 (a) and + 16 (b)
    const int lane = tid0 & 63;
#pragma unroll
    for (int t = 0; t < (L + 2) / 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        const int lo = 2 * t + (row >= 8 ? 1 : 0);
        if (lo <= L) {
          float* dst = p.rad_part + ((int64_t)blockIdx.x * 8 + (row & 7)) * (L + 1) * kC + lo * kC + 32 * wave +
                       (lane & 15);
          dst[0] = ns.rad[t].a[i];
          dst[16] = ns.rad[t].b[i];
        }
      }
  }
}

template <int L, int MD>
__device__ __forceinline__ void stretch(const MfmaParams& p, const Smem& s, __amdgpu_buffer_rsrc_t wrsrc, int tid0,
                                        int wave, const int32_t* seq, int64_t s_lo, int64_t s_hi, int64_t step,
                                        NodeState<L>& ns, WRing& ring) {
  using S = Shape<L>;
  constexpr int K = S::K;
  // the atom at position sl of the workgroup's sequence
  auto atom_at = [&](int64_t sl) -> int64_t { return p.order[seq ? seq[sl] : sl]; };
  auto degree = [&](int64_t sl) {
    const int64_t i = atom_at(sl);
    return p.row_ptr[i + 1] - p.row_ptr[i];
  };
  // atoms without neighbours: zero output, log-normaliser -inf (the query
  // pass writes no output)
  for (int64_t sl = s_lo + tid0 * step; !q_like(MD) && !r_like(MD) && sl < s_hi; sl += kThreads * step) {
    if (degree(sl) == 0) {
      const int64_t i = atom_at(sl);
      for (int q = 0; q < K * kC; ++q) p.out[i * K * kC + q] = 0.0f;
      if (p.out_lse)
        for (int h = 0; h < kH; ++h) p.out_lse[i * kH + h] = -INFINITY;
    }
  }
  auto next_nz = [&](int64_t sl) {
    while (sl < s_hi && degree(sl) == 0) sl += step;
    return sl;
  };
  auto make_plan = [&](int64_t sa, int64_t a0) {
    ChunkPlan c{};
    c.sa = sa;
    c.a0 = a0;
    c.sb = s_hi;
    if (sa >= s_hi) return c;
    c.ia = atom_at(sa);
    const int64_t deg_a = p.row_ptr[c.ia + 1] - p.row_ptr[c.ia];
    c.nA = static_cast<int>(deg_a - a0 < kET ? deg_a - a0 : kET);
    c.a_done = a0 + c.nA == deg_a;
    c.ib = c.ia;
    if (c.a_done && c.nA < kET) {
      c.sb = next_nz(sa + step);
      if (c.sb < s_hi) {
        c.ib = atom_at(c.sb);
        const int64_t deg_b = p.row_ptr[c.ib + 1] - p.row_ptr[c.ib];
        c.nB = static_cast<int>(deg_b < kET - c.nA ? deg_b : kET - c.nA);
        c.b_done = c.nB == deg_b;
      }
    }
    c.ea = p.row_ptr[c.ia] + a0;
    c.eb = p.row_ptr[c.ib];
    return c;
  };
  // the chunk after c: finish A (and B if it also ended), B becomes A
  auto next_plan = [&](const ChunkPlan& c) {
    if (!c.a_done) return make_plan(c.sa, c.a0 + c.nA);
    if (c.nB == 0) return make_plan(next_nz(c.sa + step), 0);
    if (c.b_done) return make_plan(next_nz(c.sb + step), 0);
    return make_plan(c.sb, c.nB);
  };
  // neighbour index of edge slot t of chunk c (the atom itself for padding)
  auto slot_col = [&](const ChunkPlan& c, int t) {
    if (c.sa >= s_hi || t >= c.nA + c.nB) return static_cast<int>(t >= c.nA ? c.ib : c.ia);
    return p.col[t < c.nA ? c.ea + t : c.eb + (t - c.nA)];
  };
  ChunkPlan cur = make_plan(next_nz(s_lo), 0);
  int jcur = slot_col(cur, static_cast<int>(tid0 & (kET - 1)));
  while (cur.sa < s_hi) {
    // lane-dependent values are derived afresh in every chunk rather than
    // hoisted out of the loop and kept live (or spilled) across it
    const int tid = opaque(tid0);
    const int lane = tid & 63;
    const int64_t ia = cur.ia, ib = cur.ib, ea = cur.ea, eb = cur.eb;
    const int nA = cur.nA, nB = cur.nB;
    const bool a_done = cur.a_done, b_done = cur.b_done;
    const int ne = nA + nB;
    const bool has_b = nB > 0;
    // the next chunk's plan and neighbour indices are fetched now, so that
    // their load latency overlaps this chunk's work
    const ChunkPlan nxt = next_plan(cur);
    const int jnext = slot_col(nxt, tid & (kET - 1));

    // logits s = <q_i, k_j>: the value pass runs over the reversed edges, so
    // its centre supplies the key and its neighbour the query
    const float* qsrc = MD == kBwdV ? p.k : p.q;
    const float* ksrc = MD == kBwdV ? p.q : p.k;
    if (tid < kET) s.j[tid] = jcur;
    if constexpr (MD != kConv) {
      if (tid < kC) s.q[tid] = qsrc[ia * kC + tid];
      else if (has_b) s.q[tid] = qsrc[ib * kC + (tid - kC)];
    }
    __syncthreads();
    // edge frames, D^0, D^1 and the radial basis: one lane per edge
    if (tid < kET) {
      const bool in_b = tid >= nA;
      const int64_t id = in_b ? ib : ia;
      float* De = s.D + tid * S::DSZ;
      float R[3][3] = {{0, 0, 0}, {0, 0, 0}, {0, 0, 0}};
      float d0 = 0.0f;
      float e8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int j = jcur;
      if (tid < ne) {
        float r3[3];
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          // the value pass takes the frame of the edge from its neighbour to
          // its centre: the same fp32 difference the forward computed
          float dx = MD == kBwdV ? p.pos[3 * id + d] - p.pos[3 * (int64_t)j + d]
                                 : p.pos[3 * (int64_t)j + d] - p.pos[3 * id + d];
          if (p.periodic) {
            if (dx > 0.5f * p.box[d]) dx -= p.box[d];
            else if (dx < -0.5f * p.box[d]) dx += p.box[d];
          }
          r3[d] = dx;
        }
        float u[3];
        const float rr = edge_unit(r3, u);
        edge_rotation(u, R);
        d0 = 1.0f;
        radial_basis8(rr, p.cutoff, e8);
      }
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
      if (e < ne && MD != kConv) {
        const int j = s.j[e];
        const float4* kp = reinterpret_cast<const float4*>(ksrc + (int64_t)j * kC + h * kDH);
        const float* qv = s.q + (e >= nA ? kC : 0) + h * kDH;
        float d = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 kv = kp[t];
          d += kv.x * qv[4 * t] + kv.y * qv[4 * t + 1] + kv.z * qv[4 * t + 2] + kv.w * qv[4 * t + 3];
        }
        sv = d * 0.25f;
        if constexpr (q_like(MD) || MD == kBwdV || r_like(MD)) {
          // gradient passes: alpha from the forward's log-normaliser of the
          // destination of the forward edge (the neighbour, in the value
          // pass).  The value pass carries the cotangent times gnorm (alpha
          // scaled by it), so that its rotate-out coefficients sit in fp16's
          // range whatever the cotangent's magnitude; the normaliser
          // divides it out
          const int64_t src = MD != kBwdV ? (e < nA ? ia : ib) : (int64_t)j;
          sv = expf(sv - p.lse[src * kH + h]);
          if constexpr (MD == kBwdV) sv *= *p.gnorm;
        }
      }
      s.alpha[e * kH + h] = sv;
    }
    __syncthreads();
    // online softmax update, one thread per (destination, head), while the
    // others extend D; padding slots get weight 0
    if (tid < 2 * kH) {
      const int d = tid / kH, h = tid % kH;
      const int b0 = d == 0 ? 0 : nA, b1 = d == 0 ? nA : ne;
      if constexpr (q_like(MD) || MD == kBwdV || r_like(MD)) {
        // gradient passes: the weights were formed with the logits; the
        // normaliser is the value pass's cotangent scale, or 1
        const float gs = MD == kBwdV ? *p.gnorm : 1.0f;
        if (b1 > b0) {
          s.l_run[d * kH + h] = gs;
          s.m_run[d * kH + h] = 0.0f;
        }
        if (d == 0) s.scale[h] = 1.0f;
      } else if (MD == kConv) {
        // convolution: weight 1 for every edge, normaliser 1, no rescale
        for (int e = b0; e < b1; ++e) s.alpha[e * kH + h] = 1.0f;
        if (b1 > b0) {
          s.l_run[d * kH + h] = 1.0f;
          s.m_run[d * kH + h] = 0.0f;
        }
        if (d == 0) s.scale[h] = 1.0f;
      }
      if (d == 1)
        for (int e = ne; e < kET; ++e) s.alpha[e * kH + h] = 0.0f;
    }
    if constexpr (MD == kFwd) {
      // forward: wave 0 updates destination A, wave 1 destination B; lane
      // e = lane % 32 holds edge b0 + e and each 32-lane half one head per
      // pass; the chunk's max and sum over the edges are butterfly shuffles
      // within the half (a chunk holds at most 32 edges of a destination)
      static_assert(kET == 32 && kH % 2 == 0, "one lane per edge slot, two heads per pass");
      if (tid < 128) {
        const int d = tid >> 6, e = tid & 31;
        const int b0 = d == 0 ? 0 : nA, b1 = d == 0 ? nA : ne;
        const bool valid = b0 + e < b1;
        if (b1 > b0) {
          for (int h = (tid >> 5) & 1; h < kH; h += 2) {
            const float v = valid ? s.alpha[(b0 + e) * kH + h] : -INFINITY;
            const float m_old = s.m_run[d * kH + h];
            float mx = v;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            mx = fmaxf(mx, m_old);
            const float a = valid ? expf(v - mx) : 0.0f;
            if (valid) s.alpha[(b0 + e) * kH + h] = a;
            float sum = a;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
            if (e == 0) {
              const float sc = expf(m_old - mx);
              s.l_run[d * kH + h] = s.l_run[d * kH + h] * sc + sum;
              s.m_run[d * kH + h] = mx;
              if (d == 0) s.scale[h] = sc;
            }
          }
        }
      }
    }
    if constexpr (L >= 2) wig_level<L, 2>(s, tid);
    __syncthreads();
    // per-lane constants of this chunk, and the rescale of A's running
    // accumulators (B's rows are zero)
    Lane ln;
    {
      const int lnr = opaque(lane);
      const int half = lnr >> 5;
      const int h_own = (32 * wave + (lnr & 31)) / kDH;
#pragma unroll
      for (int q = 0; q < 16; ++q) ln.alpha[q] = s.alpha[crow(q, half) * kH + h_own];
      // the wave's 32 channels are heads 2w and 2w+1
      const float sa_ = s.scale[2 * wave], sb_ = s.scale[2 * wave + 1];
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        ns.acc[l].a *= sa_;
        ns.acc[l].b *= sb_;
      }
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const int rr = lnr & 31;
      ln.arbf[0] = to_vec8<bf16x8>(half == 0 ? s.rbf + rr * 8 : z);
      ln.arbf[1] = to_vec8<bf16x8>(half == 0 ? s.rbf + (rr & 15) * 8 : z);
      ln.arbf[2] = to_vec8<bf16x8>(half == 0 ? s.rbf + (16 + (rr & 15)) * 8 : z);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t0 = 16 * g + 8 * (q >> 1) + 4 * half + 2 * (q & 1);
          ln.mk[g][q] = (t0 < nA ? 0x0000FFFFu : 0u) | (t0 + 1 < nA ? 0xFFFF0000u : 0u);
        }
      ln.flip = (lnr & 8) ? ~0u : 0u;
      if constexpr (q_like(MD) || r_like(MD)) {
        ln.nA = nA;
        ln.ia = ia;
        ln.ib = ib;
        ln.gsA = p.gsc[ia];
        ln.gsB = p.gsc[ib];
      }
      if constexpr (q_like(MD)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ns.dal[r] = 0.0f;
      }
      if constexpr (r_like(MD)) {
        // the rotated cotangent is in its atom's fp16 scale: undo it per
        // edge, then apply the global power of two that keeps alpha y (D G)
        // in fp16's range (divided out when the partials are added)
        const float gn = *p.gnorm;
#pragma unroll
        for (int q = 0; q < 16; ++q) ln.alpha[q] *= (crow(q, half) < nA ? ln.gsA : ln.gsB) * gn;
      }
    }
    do_block<L, 0, MD>(p, s, wrsrc, tid, wave, ln, has_b, ns, ring);
    if constexpr (q_like(MD)) {
      // dalpha[edge][head]: the lane's partials summed over the head's 16
      // channels (a row of 16 lanes), lane r of the row ending with edge
      // crow(r, half); s.q is free since the logits
      {
        const int lane = tid & 63;
        const float v = row_reduce_scatter16(ns.dal, lane);
        const int e = crow(lane & 15, lane >> 5);
        const int head = 2 * wave + ((lane >> 4) & 1);
        s.q[e * kH + head] = v * (e < nA ? ln.gsA : ln.gsB);
      }
      __syncthreads();
      // ds = alpha (dalpha - delta) for the chunk's edges, one (edge, head)
      // per thread, at the edge's place in the neighbour list
      const int e = tid >> 3, h = tid & 7;
      if (e < ne) {
        const bool in_b = e >= nA;
        const int64_t id = in_b ? ib : ia;
        const int64_t g = in_b ? eb + (e - nA) : ea + e;
        p.ds[g * kH + h] = s.alpha[e * kH + h] * (s.q[e * kH + h] - p.delta[id * kH + h]);
      }
      __syncthreads();
    } else if constexpr (MD == kBwdR) {
      // the radial pass only accumulates; the workgroup writes at the end
    } else if (a_done) {
      // finish A (and B if it also ended); B's partial state becomes A's
      finish_a<L>(p, s, ns, ia, tid, wave);
      if (b_done) finish_a<L>(p, s, ns, ib, tid, wave);
    }
    cur = nxt;
    jcur = jnext;
  }
}

// Logical SO(2) weights -> B-fragment image: vector v holds, for lane
// v % 64 of one k-step, the 8 values W[k0 .. k0+7][n] with k0 = 16 s + 8 (lane/32)
// and n = (l_out - m) C + 32 wave + lane % 32.  With TR set, the image of the
// transposed mix the value pass needs: W0^T for m = 0, and W1^T, -W2^T for
// m > 0 (so that the kernel's complex product gives dx_+ = dy_+ W1^T + dy_- W2^T
// and dx_- = -dy_+ W2^T + dy_- W1^T).  With wrad set, the first (L+1) C
// threads also pack W_rad into radout (k_pack_rad's work, in the same launch).
template <int L>
__device__ __forceinline__ void pack_rad_entry(const uint16_t* __restrict__ w, u32x4* __restrict__ out, int v) {
  uint32_t b[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) b[q] = w[q * (L + 1) * kC + v];
  out[v] = u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
}

template <int L, bool TR>
__global__ void k_pack_so2(const uint16_t* __restrict__ w, bf16x8* __restrict__ out,
                           const uint16_t* __restrict__ wrad = nullptr, u32x4* __restrict__ radout = nullptr) {
  using S = Shape<L>;
  const int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (wrad && v < (L + 1) * kC) pack_rad_entry<L>(wrad, radout, static_cast<int>(v));
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
  for (int q = 0; q < 8; ++q) {
    if constexpr (TR) vals[q] = base[n * km + k0 + q] ^ (wsel == 1 ? 0x8000 : 0);
    else vals[q] = base[(k0 + q) * km + n];
  }
  uint4 o;
  o.x = vals[0] | (uint32_t(vals[1]) << 16);
  o.y = vals[2] | (uint32_t(vals[3]) << 16);
  o.z = vals[4] | (uint32_t(vals[5]) << 16);
  o.w = vals[6] | (uint32_t(vals[7]) << 16);
  *reinterpret_cast<uint4*>(out + v) = o;
}

// W_rad [8][L+1][C] -> [(L+1) C] vectors of 8 basis weights (bf16, copied
// bit for bit).
template <int L>
__global__ void k_pack_rad(const uint16_t* __restrict__ w, u32x4* __restrict__ out) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < (L + 1) * kC) pack_rad_entry<L>(w, out, v);
}

// The balanced deal of destinations to the workgroups of an XCD sorts each
// round in one wave, so it serves up to 64 workgroups per XCD (two per CU
// on MI355X's 32 CUs per XCD); beyond that the kernel deals cyclically.
constexpr int kDealMaxWpx = 64;

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Ascending bitonic sort of one key per lane across the 64 lanes of a wave.
__device__ __forceinline__ uint64_t wave_sort64(uint64_t key, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = shfl_xor64(key, j);
      const bool keep_min = ((lane & j) == 0) == ((lane & k) == 0);
      key = keep_min ? (o < key ? o : key) : (o > key ? o : key);
    }
  return key;
}

// The balanced deal, one wave per (round, XCD).  Round r of XCD range
// [x_lo, x_hi) holds the slots x_lo + r wpx + t (t < wpx) of the order, as in
// the cyclic deal, but ranked by degree (most edges first, ties by slot): in
// even rounds the workgroup w takes rank w, in odd rounds rank wpx - 1 - w,
// so that a workgroup's heavy and light destinations alternate and the
// workgroups end with about the same number of edges.  Rounds are
// independent of each other, and the deal depends only on the degrees in
// order, so it (and with it every result) is the same on every launch.  Row
// xcd + 8 w of sched lists workgroup w's slots in round order; only the last
// round can leave a workgroup without one, and sched_n counts them.
__global__ void __launch_bounds__(64) k_deal(const int32_t* __restrict__ order, const int64_t* __restrict__ row_ptr,
                                             const int64_t* __restrict__ xcd_lo, int64_t n, int wpx, int64_t R,
                                             int32_t* __restrict__ sched, int32_t* __restrict__ sched_n) {
  const int64_t r = blockIdx.x;
  const int xcd = blockIdx.y, lane = threadIdx.x;
  const int64_t x_lo = xcd_lo ? xcd_lo[xcd] : xcd * n / 8;
  const int64_t x_hi = xcd_lo ? xcd_lo[xcd + 1] : (xcd + 1) * n / 8;
  const int64_t rounds = (x_hi - x_lo + wpx - 1) / wpx;
  const int64_t slot = x_lo + r * wpx + lane;
  const bool valid = lane < wpx && slot < x_hi;
  uint64_t key = ~0ull;
  if (valid) {
    const int64_t a = order[slot];
    const int64_t d = row_ptr[a + 1] - row_ptr[a];
    key = (static_cast<uint64_t>(0x7fffffff - d) << 32) | static_cast<uint64_t>(slot - x_lo);
  }
  key = wave_sort64(key, lane);
  if (lane < wpx) {
    const int w = (r & 1) ? wpx - 1 - lane : lane;
    const bool got = key != ~0ull;
    sched[(int64_t)(xcd + 8 * w) * R + r] = got ? static_cast<int32_t>(x_lo + (key & 0xffffffffu)) : -1;
    const int64_t last = rounds > 0 ? rounds - 1 : 0;
    if (r == last) sched_n[xcd + 8 * w] = static_cast<int32_t>(last + (got ? 1 : 0));
  }
}

// The XCD ranges of the order split by edges: the degree of every slot of
// the order, their prefix sums (k_scan), and the first slot whose prefix
// reaches x E / 8 for x = 1..7, each kept within n / 16 of the split by atoms
// x n / 8 (so that no range holds more than about a quarter of the atoms).
// Every XCD then streams about the same number of edges.
__global__ void k_slot_degree(const int32_t* __restrict__ order, const int64_t* __restrict__ row_ptr, int64_t n,
                              int32_t* __restrict__ deg) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) {
    const int64_t a = order[t];
    deg[t] = static_cast<int32_t>(row_ptr[a + 1] - row_ptr[a]);
  }
}

__global__ void __launch_bounds__(64) k_xcd_split(const int32_t* __restrict__ pre, int64_t n,
                                                  int64_t* __restrict__ xcd_lo) {
  const int x = threadIdx.x;
  if (x > 8) return;
  int64_t b = x * n / 8;
  if (x > 0 && x < 8) {
    const int64_t target = (int64_t)x * pre[n] / 8;
    int64_t lo = 0, hi = n;   // first t with pre[t] >= target
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (pre[mid] < target) lo = mid + 1;
      else hi = mid;
    }
    const int64_t h = (n + 15) / 16;
    const int64_t c = x * n / 8;
    b = lo < c - h ? c - h : (lo > c + h ? c + h : lo);
    b = b < 0 ? 0 : (b > n ? n : b);
  }
  xcd_lo[x] = b;
}

constexpr int kOrderBits = 6;                       // Morton cells per axis = 64
constexpr int kRadixBits = 9;                        // two radix passes over 18-bit keys
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortBlock = 1024;                     // elements per sort block (4 rounds of 256)

__device__ __forceinline__ uint32_t spread3(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < kOrderBits; ++b) r |= ((v >> b) & 1u) << (3 * b);
  return r;
}

// Morton keys of one sort block (kSortBlock atoms, 256 threads) with the
// first radix pass's digit counts of the block, hist[d * nblk + b].  Each
// block first reduces the bounding box from the nparts partial boxes
// (min and max are exact in any order, so every block gets the same box),
// and the grid clears hist_next, which the first scatter fills.
__global__ void __launch_bounds__(256) k_ord_keys(const float* __restrict__ pos, int64_t n,
                                                  const float* __restrict__ bbox_part, int nparts,
                                                  int32_t* __restrict__ key, int32_t* __restrict__ val,
                                                  int32_t* __restrict__ hist, int32_t* __restrict__ hist_next,
                                                  int64_t nblk) {
  __shared__ float bmin[3][256], bmax[3][256];
  __shared__ int32_t h[kRadix];
  for (int d = threadIdx.x; d < kRadix; d += blockDim.x) h[d] = 0;
  {
    float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
    for (int b = threadIdx.x; b < nparts; b += blockDim.x)
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        mn[d] = fminf(mn[d], bbox_part[8 * b + d]);
        mx[d] = fmaxf(mx[d], bbox_part[8 * b + 3 + d]);
      }
#pragma unroll
    for (int d = 0; d < 3; ++d) { bmin[d][threadIdx.x] = mn[d]; bmax[d][threadIdx.x] = mx[d]; }
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
      if (threadIdx.x < st)
#pragma unroll
        for (int d = 0; d < 3; ++d) {
          bmin[d][threadIdx.x] = fminf(bmin[d][threadIdx.x], bmin[d][threadIdx.x + st]);
          bmax[d][threadIdx.x] = fmaxf(bmax[d][threadIdx.x], bmax[d][threadIdx.x + st]);
        }
      __syncthreads();
    }
  }
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < kRadix * nblk;
       t += (int64_t)gridDim.x * blockDim.x)
    hist_next[t] = 0;
  const int64_t base = blockIdx.x * (int64_t)kSortBlock;
  for (int r = threadIdx.x; r < kSortBlock; r += blockDim.x) {
    const int64_t i = base + r;
    if (i >= n) break;
    uint32_t c[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float lo = bmin[d][0];
      const float ext = fmaxf(bmax[d][0] - lo, 1e-6f);
      float f = (pos[3 * i + d] - lo) / ext * float(1 << kOrderBits);
      f = fminf(fmaxf(f, 0.0f), float((1 << kOrderBits) - 1));
      c[d] = static_cast<uint32_t>(f);
    }
    const int32_t k = static_cast<int32_t>(spread3(c[0]) | (spread3(c[1]) << 1) | (spread3(c[2]) << 2));
    key[i] = k;
    val[i] = static_cast<int32_t>(i);
    atomicAdd(&h[k & (kRadix - 1)], 1);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < kRadix; d += blockDim.x) hist[(int64_t)d * nblk + blockIdx.x] = h[d];
}

// LSD radix sort of (Morton key, atom index) pairs, one kRadixBits digit per
// pass.  The sort is stable, so the order (and with it the way atoms share
// edge chunks in the layer kernel) is the same on every launch.
//
// Stable scatter: element i of block b (digit d) goes to off[d * nblk + b]
// plus the number of earlier elements of the block with digit d.  The block's
// 1024 elements go in 4 rounds of 256 in index order; within a round the waves
// take turns, and inside a wave the lanes holding the same digit are found with
// one ballot per digit bit.
//
// With hist_next set, each element also counts its next digit for the sort
// block it lands in, hist_next[d' * nblk + at / kSortBlock] (the next pass's
// counts, so no separate counting launch is needed; hist_next starts at 0).
__global__ void __launch_bounds__(256) k_radix_scatter(const int32_t* __restrict__ key_in,
                                                       const int32_t* __restrict__ val_in, int64_t n, int shift,
                                                       const int32_t* __restrict__ off, int64_t nblk,
                                                       int32_t* __restrict__ key_out, int32_t* __restrict__ val_out,
                                                       int32_t* __restrict__ hist_next) {
  __shared__ int32_t next[kRadix];
  for (int d = threadIdx.x; d < kRadix; d += blockDim.x) next[d] = off[(int64_t)d * nblk + blockIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = blockIdx.x * (int64_t)kSortBlock;
  for (int round = 0; round < kSortBlock / 256; ++round) {
    const int64_t i = base + round * 256 + threadIdx.x;
    const bool valid = i < n;
    const int32_t k = valid ? key_in[i] : 0;
    const int32_t v = valid ? val_in[i] : 0;
    const int d = (k >> shift) & (kRadix - 1);
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < kRadixBits; ++bit) {
      const uint64_t b = __ballot((d >> bit) & 1);
      same &= ((d >> bit) & 1) ? b : ~b;
    }
    const int rank = __popcll(same & below);
    const int count = __popcll(same);
    for (int w = 0; w < 4; ++w) {
      if (wave == w && valid) {
        const int32_t at = next[d] + rank;
        key_out[at] = k;
        val_out[at] = v;
        if (hist_next)
          atomicAdd(&hist_next[(int64_t)((k >> (shift + kRadixBits)) & (kRadix - 1)) * nblk + at / kSortBlock], 1);
      }
      __syncthreads();
      if (wave == w && valid && rank == 0) next[d] += count;
      __syncthreads();
    }
  }
}

struct MfmaWs {
  size_t w, rad, order, key, key2, val2, hist, hist2, off, bsum, bbox_part;
  size_t sched, sched_n;   // the balanced deal: per-workgroup rows of slots and their lengths
  size_t xdeg, xpre, xbsum, xlo;   // the XCD ranges split by edges
  size_t wt, gbf, delta;   // feature gradient only: transposed image, bf16 cotangent, delta,
  size_t gpk, gsc;         // and the query pass's scaled fp16 cotangent with its scales,
  size_t gnorm;            // and the value pass's cotangent scale,
  size_t radpart;          // and the radial pass's per-workgroup dW_rad partials
  size_t total;
};

inline int64_t sort_blocks(int64_t n) { return (n + kSortBlock - 1) / kSortBlock; }

template <int L>
MfmaWs mfma_ws_layout(int64_t n, bool backward) {
  using S = Shape<L>;
  MfmaWs m{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  m.w = take(S::wtotal() * 16);
  m.rad = take((L + 1) * kC * 16);
  m.order = take(sizeof(int32_t) * n);
  m.key = take(sizeof(int32_t) * n);
  m.key2 = take(sizeof(int32_t) * n);
  m.val2 = take(sizeof(int32_t) * n);
  m.hist = take(sizeof(int32_t) * kRadix * sort_blocks(n));
  m.hist2 = take(sizeof(int32_t) * kRadix * sort_blocks(n));
  m.off = take(sizeof(int32_t) * (kRadix * sort_blocks(n) + 1));   // the scan also writes the total
  m.bsum = take(sizeof(int64_t) * scan_bsum_count(kRadix * sort_blocks(n)));
  m.bbox_part = take(sizeof(float) * kBboxPartialFloats);
  // a range of the edge split holds at most 2 ceil(n / 8) + 2 slots
  m.sched = take(sizeof(int32_t) * (2 * n + 32 + 8 * kDealMaxWpx));
  m.sched_n = take(sizeof(int32_t) * 8 * kDealMaxWpx);
  m.xdeg = take(sizeof(int32_t) * n);
  m.xpre = take(sizeof(int32_t) * (n + 1));
  m.xbsum = take(sizeof(int64_t) * scan_bsum_count(n));
  m.xlo = take(sizeof(int64_t) * 9);
  if (backward) {
    m.wt = take(S::wtotal() * 16);
    m.gbf = take(sizeof(uint16_t) * n * S::K * kC);
    m.delta = take(sizeof(float) * n * kH);
    m.gpk = take(16 * n * S::gslots * kC);
    m.gsc = take(sizeof(float) * n);
    m.gnorm = take(sizeof(float));
    m.radpart = take(sizeof(float) * kMaxRadWg * 8 * (L + 1) * kC);
  }
  m.total = off;
  return m;
}

// The cotangent G in the two forms the feature gradient reads, one atom per
// workgroup: bf16 (the value pass's features) and, for the query pass, fp16
// times a power of two s_i that puts max |G_i| in [2^14, 2^15), so that small
// cotangents keep fp16's precision and none overflows; gsc[i] = 1 / s_i.
// The fp16 form is in 8-entry vectors per (slot, channel): slot lo holds
// G[lo^2 + n], n < 2 lo + 1, zero-padded; degree 4 also fills slot 5 with
// n = 8 (then zeros).
template <int L>
__global__ void __launch_bounds__(256) k_prep_grad(const float* __restrict__ g, uint16_t* __restrict__ gbf,
                                                   f16x8* __restrict__ gpk, float* __restrict__ gsc) {
  using S = Shape<L>;
  constexpr int NSL = S::gslots;
  __shared__ float red[4];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const float* gi = g + i * S::K * kC;
  uint16_t* bi = gbf + i * S::K * kC;
  float mx = 0.0f;
  // four values per access (K C is a multiple of 128): 16-byte reads, 8-byte bf16 writes
  static_assert((S::K * kC) % 4 == 0, "whole vectors of four");
  for (int t = tid; t < S::K * kC / 4; t += 256) {
    const float4 v = reinterpret_cast<const float4*>(gi)[t];
    uint2 b;
    b.x = static_cast<uint32_t>(f32_to_bf16_rne(v.x)) | (static_cast<uint32_t>(f32_to_bf16_rne(v.y)) << 16);
    b.y = static_cast<uint32_t>(f32_to_bf16_rne(v.z)) | (static_cast<uint32_t>(f32_to_bf16_rne(v.w)) << 16);
    reinterpret_cast<uint2*>(bi)[t] = b;
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // max |G_i| < 2^(E - 126) for its biased exponent E: s_i = 2^(141 - E)
  const int E = static_cast<int>((__float_as_uint(mx) >> 23) & 0xffu);
  const int sh = min(100, max(-100, 141 - E));
  const float sc = __uint_as_float(static_cast<uint32_t>(127 + sh) << 23);
  if (tid == 0) gsc[i] = __uint_as_float(static_cast<uint32_t>(127 - sh) << 23);
  for (int t = tid; t < NSL * kC; t += 256) {
    const int slot = t / kC, c = t % kC;
    const int lo = slot <= L ? slot : L;
    const int nb = slot <= L ? 0 : 8;
    f16x8 v = {};
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (nb + q < 2 * lo + 1) v[q] = static_cast<_Float16>(gi[(lo * lo + nb + q) * kC + c] * sc);
    gpk[(i * NSL + slot) * kC + c] = v;
  }
}

// The value pass's cotangent scale from the per-atom ones: gsc[i] = 2^(E_i - 141)
// for the biased exponent E_i of max |G_i|, so the largest gsc marks the
// largest max |G_i| = 1.f 2^(E - 127), and 2^-14 / max gsc = 2^(127 - E)
// brings it into [1, 2).  One workgroup; every value involved is a power of
// two, so the result is exact.
__global__ void __launch_bounds__(1024) k_grad_norm(const float* __restrict__ gsc, int64_t n, float* __restrict__ gnorm) {
  __shared__ float red[16];
  float mx = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 1024) mx = fmaxf(mx, gsc[i]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) mx = fmaxf(mx, red[w]);
    *gnorm = 0x1p-14f / mx;
  }
}

// Spatial order of the destinations: the Morton code of a 64^3 grid over the
// bounding box, stably sorted with the atom index as the tie-break, so the
// order (and with it which atoms share edge chunks) is the same on every
// launch.  `order` and the scratch come from the layout W.
e2a_status spatial_order(const float* pos, int64_t n, const MfmaWs& W, char* wb, int32_t* order, hipStream_t st) {
  if (n == 0) return E2A_OK;
  int32_t* key = reinterpret_cast<int32_t*>(wb + W.key);
  int32_t* key2 = reinterpret_cast<int32_t*>(wb + W.key2);
  int32_t* val2 = reinterpret_cast<int32_t*>(wb + W.val2);
  int32_t* hist = reinterpret_cast<int32_t*>(wb + W.hist);
  int32_t* hist2 = reinterpret_cast<int32_t*>(wb + W.hist2);
  int32_t* off = reinterpret_cast<int32_t*>(wb + W.off);
  int64_t* bsum = reinterpret_cast<int64_t*>(wb + W.bsum);
  float* bbox_part = reinterpret_cast<float*>(wb + W.bbox_part);
  const int64_t nblk = sort_blocks(n);
  const int nparts = launch_bbox_partial(pos, n, bbox_part, st);
  E2A_LAUNCH_CHECK();
  k_ord_keys<<<nblk, 256, 0, st>>>(pos, n, bbox_part, nparts, key, order, hist, hist2, nblk);
  E2A_LAUNCH_CHECK();
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass * kRadixBits;
    const int32_t* kin = pass == 0 ? key : key2;
    const int32_t* vin = pass == 0 ? order : val2;
    int32_t* kout = pass == 0 ? key2 : key;
    int32_t* vout = pass == 0 ? val2 : order;
    e2a_status ss = exclusive_scan_i32(pass == 0 ? hist : hist2, kRadix * nblk, off, bsum, st);
    if (ss != E2A_OK) return ss;
    k_radix_scatter<<<nblk, 256, 0, st>>>(kin, vin, n, shift, off, nblk, kout, vout, pass == 0 ? hist2 : nullptr);
    E2A_LAUNCH_CHECK();
  }
  return E2A_OK;
}

// The destination order (the caller's, or the spatial order computed here)
// and the packed forward weights (the caller's image, or packed here).
template <int L>
e2a_status prepare(const e2a_attn_args* a, const MfmaWs& W, char* wb, hipStream_t st) {
  using S = Shape<L>;
  if (!a->order) {
    const e2a_status so = spatial_order(a->pos, a->n_atoms, W, wb, reinterpret_cast<int32_t*>(wb + W.order), st);
    if (so != E2A_OK) return so;
  }
  const uint16_t* wrad = static_cast<const uint16_t*>(a->w_rad);
  u32x4* radout = reinterpret_cast<u32x4*>(wb + W.rad);
  if (!a->w_so2_packed) {
    static_assert(S::wtotal() >= (L + 1) * kC, "the weight image outnumbers W_rad's vectors");
    const int64_t nv = S::wtotal();
    k_pack_so2<L, false><<<(nv + 255) / 256, 256, 0, st>>>(static_cast<const uint16_t*>(a->w_so2),
                                                            reinterpret_cast<bf16x8*>(wb + W.w), wrad, radout);
  } else {
    k_pack_rad<L><<<((L + 1) * kC + 255) / 256, 256, 0, st>>>(wrad, radout);
  }
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

// Parameters shared by every mode; the persistent grid has two workgroups
// per CU (the LDS and register budget), fewer when the system is small.
template <int L>
e2a_status base_params(const e2a_attn_args* a, const MfmaWs& W, char* wb, const float* box, int periodic,
                       MfmaParams& p) {
  p = MfmaParams{};
  p.pos = a->pos;
  p.row_ptr = a->row_ptr;
  p.col = a->col;
  p.feat = static_cast<const uint16_t*>(a->feat);
  p.wpk = a->w_so2_packed ? static_cast<const bf16x8*>(a->w_so2_packed) : reinterpret_cast<const bf16x8*>(wb + W.w);
  p.radpk = reinterpret_cast<const bf16x8*>(wb + W.rad);
  p.order = a->order ? a->order : reinterpret_cast<const int32_t*>(wb + W.order);
  p.n_atoms = a->n_atoms;
  int dev = 0, n_cu = 0;
  E2A_HIP_CHECK(hipGetDevice(&dev));
  E2A_HIP_CHECK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  const int64_t per_xcd_atoms = (a->n_atoms + 7) / 8;
  int64_t wpx = (2 * (int64_t)n_cu + 7) / 8;
  const int64_t by_size = (per_xcd_atoms + kMinPerWg - 1) / kMinPerWg;
  if (wpx > by_size) wpx = by_size;
  if (wpx < 1) wpx = 1;
  p.wg_per_xcd = static_cast<int>(wpx);
  for (int d = 0; d < 3; ++d) p.box[d] = box[d];
  p.periodic = periodic;
  p.cutoff = a->cutoff;
  return E2A_OK;
}

// The balanced deal for p's workgroups over the destination order p.order
// (from the caller or spatial_order), into the workspace; p then reads it.
// Set p.wg_per_xcd first.  With a mean degree below the 32-edge chunk the
// cyclic deal stays: a chunk holds at most two destinations, so there the
// work follows the number of chunks rather than of edges, and an edge-
// balanced deal pairs light destinations into half-empty chunks (measured
// slower on the drug-like batch, faster on the denser systems).
e2a_status deal(const MfmaWs& W, char* wb, MfmaParams& p, int64_t n_edges, hipStream_t st) {
  const int64_t n = p.n_atoms;
  if (n == 0 || n_edges < (int64_t)kET * n) return E2A_OK;   // cyclic deal, XCD ranges by atoms
  // the XCD ranges split by edges (prefix sums in int32: E < 2^31); below a
  // chunk's mean degree the imbalance is within the XCDs' ranges and the
  // three extra launches did not pay (drug-like batch)
  if (n_edges < INT32_MAX) {
    int32_t* deg = reinterpret_cast<int32_t*>(wb + W.xdeg);
    int32_t* pre = reinterpret_cast<int32_t*>(wb + W.xpre);
    int64_t* xlo = reinterpret_cast<int64_t*>(wb + W.xlo);
    k_slot_degree<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(p.order, p.row_ptr, n, deg);
    E2A_LAUNCH_CHECK();
    const e2a_status e = exclusive_scan_i32(deg, n, pre, reinterpret_cast<int64_t*>(wb + W.xbsum), st);
    if (e != E2A_OK) return e;
    k_xcd_split<<<1, 64, 0, st>>>(pre, n, xlo);
    E2A_LAUNCH_CHECK();
    p.xcd_lo = xlo;
  }
  if (p.wg_per_xcd > kDealMaxWpx) return E2A_OK;   // cyclic deal
  const int wpx = p.wg_per_xcd;
  const int64_t span = p.xcd_lo ? 2 * ((n + 7) / 8) + 2 : (n + 7) / 8;   // slots of the largest range
  const int64_t R = (span + wpx - 1) / wpx;
  int32_t* sched = reinterpret_cast<int32_t*>(wb + W.sched);
  int32_t* sched_n = reinterpret_cast<int32_t*>(wb + W.sched_n);
  k_deal<<<dim3(static_cast<unsigned>(R), 8), 64, 0, st>>>(p.order, p.row_ptr, p.xcd_lo, n, wpx, R, sched,
                                                           sched_n);
  E2A_LAUNCH_CHECK();
  p.sched = sched;
  p.sched_n = sched_n;
  p.sched_len = R;
  return E2A_OK;
}

template <int L, int MD>
e2a_status launch_mode(const MfmaParams& p, hipStream_t st) {
  using S = Shape<L>;
  E2A_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_mfma<L, MD>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, S::total));
  hipLaunchKernelGGL((k_attn_mfma<L, MD>), dim3(8 * p.wg_per_xcd), dim3(kThreads), S::total, st, p);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

template <int L>
e2a_status launch_typed(const AttnPlan& pl, hipStream_t st) {
  const e2a_attn_args* a = pl.a;
  const MfmaWs W = mfma_ws_layout<L>(a->n_atoms, false);
  char* wb = static_cast<char*>(pl.mfma_ws);
  e2a_status e = prepare<L>(a, W, wb, st);
  if (e != E2A_OK) return e;
  MfmaParams p;
  e = base_params<L>(a, W, wb, pl.box, pl.periodic, p);
  if (e != E2A_OK) return e;
  e = deal(W, wb, p, a->n_edges, st);
  if (e != E2A_OK) return e;
  p.q = pl.q;
  p.k = pl.k;
  p.out = a->out;
  p.out_lse = pl.conv ? nullptr : a->out_lse;
  return pl.conv ? launch_mode<L, kConv>(p, st) : launch_mode<L, kFwd>(p, st);
}

// dW_rad[k][l][c] = (sum over workgroups, in order, of their partials) / gnorm.
template <int L>
__global__ void k_rad_reduce(const float* __restrict__ part, int n_wg, const float* __restrict__ gnorm,
                             float* __restrict__ w_rad) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int N = 8 * (L + 1) * kC;
  if (t >= N) return;
  float v = 0.0f;
  for (int g = 0; g < n_wg; ++g) v += part[(int64_t)g * N + t];
  w_rad[t] = v / *gnorm;
}

// Feature gradient on the matrix cores: delta, the query pass (ds), the
// value pass (the transposed messages into grad_feat) and the l = 0 terms.
template <int L>
e2a_status launch_bwd_typed(const BwdPlan& pl, hipStream_t st) {
  using S = Shape<L>;
  const e2a_attn_args* a = pl.a;
  const MfmaWs W = mfma_ws_layout<L>(a->n_atoms, true);
  char* wb = static_cast<char*>(pl.mfma_ws);
  e2a_status e = prepare<L>(a, W, wb, st);
  if (e != E2A_OK) return e;
  {
    const int64_t nv = S::wtotal();
    k_pack_so2<L, true><<<(nv + 255) / 256, 256, 0, st>>>(static_cast<const uint16_t*>(a->w_so2),
                                                           reinterpret_cast<bf16x8*>(wb + W.wt));
    k_prep_grad<L><<<a->n_atoms, 256, 0, st>>>(pl.grad_out, reinterpret_cast<uint16_t*>(wb + W.gbf),
                                               reinterpret_cast<f16x8*>(wb + W.gpk),
                                               reinterpret_cast<float*>(wb + W.gsc));
    E2A_LAUNCH_CHECK();
    k_grad_norm<<<1, 1024, 0, st>>>(reinterpret_cast<const float*>(wb + W.gsc), a->n_atoms,
                                    reinterpret_cast<float*>(wb + W.gnorm));
    E2A_LAUNCH_CHECK();
  }
  float* delta = reinterpret_cast<float*>(wb + W.delta);
  e = launch_bwd_delta(pl, delta, st);
  if (e != E2A_OK) return e;
  MfmaParams p;
  e = base_params<L>(a, W, wb, pl.box, pl.periodic, p);
  if (e != E2A_OK) return e;
  // with dW_rad the partials take one slot per workgroup
  if (pl.w_rad && 8 * p.wg_per_xcd > kMaxRadWg) p.wg_per_xcd = kMaxRadWg / 8;
  e = deal(W, wb, p, a->n_edges, st);
  if (e != E2A_OK) return e;
  p.q = pl.q;
  p.k = pl.k;
  p.lse = a->out_lse;
  // query pass
  p.gpk = reinterpret_cast<const f16x8*>(wb + W.gpk);
  p.gsc = reinterpret_cast<const float*>(wb + W.gsc);
  p.gnorm = reinterpret_cast<const float*>(wb + W.gnorm);
  p.delta = delta;
  p.ds = pl.ds;
  if (pl.ds_later) {
    // the call forms ds from its edge batches and adds the l = 0 terms then
  } else if (pl.w_rad) {
    // dW_rad in the same pass (the radial pass's partials and reduction)
    p.rad_part = reinterpret_cast<float*>(wb + W.radpart);
    e = launch_mode<L, kBwdQR>(p, st);
    if (e != E2A_OK) return e;
    constexpr int N = 8 * (L + 1) * kC;
    k_rad_reduce<L><<<(N + 255) / 256, 256, 0, st>>>(p.rad_part, 8 * p.wg_per_xcd, p.gnorm, pl.w_rad);
    E2A_LAUNCH_CHECK();
  } else {
    e = launch_mode<L, kBwdQ>(p, st);
    if (e != E2A_OK) return e;
  }
  if (!pl.grad_feat) return pl.wdq ? launch_bwd_qk(pl, st) : E2A_OK;
  // value pass: the cotangent in bf16 takes the features' place
  p.feat = reinterpret_cast<const uint16_t*>(wb + W.gbf);
  p.wpk = reinterpret_cast<const bf16x8*>(wb + W.wt);
  p.out = pl.grad_feat;
  e = launch_mode<L, kBwdV>(p, st);
  if (e != E2A_OK) return e;
  return pl.ds_later ? E2A_OK : launch_bwd_qk(pl, st);
}

// dW_rad on the matrix cores: the cotangent's copies, then the radial pass
// and the reduction of its partials.
template <int L>
e2a_status launch_radial_typed(const BwdPlan& pl, float* w_rad, hipStream_t st) {
  const e2a_attn_args* a = pl.a;
  const MfmaWs W = mfma_ws_layout<L>(a->n_atoms, true);
  char* wb = static_cast<char*>(pl.mfma_ws);
  e2a_status e = prepare<L>(a, W, wb, st);
  if (e != E2A_OK) return e;
  k_prep_grad<L><<<a->n_atoms, 256, 0, st>>>(pl.grad_out, reinterpret_cast<uint16_t*>(wb + W.gbf),
                                             reinterpret_cast<f16x8*>(wb + W.gpk),
                                             reinterpret_cast<float*>(wb + W.gsc));
  E2A_LAUNCH_CHECK();
  k_grad_norm<<<1, 1024, 0, st>>>(reinterpret_cast<const float*>(wb + W.gsc), a->n_atoms,
                                  reinterpret_cast<float*>(wb + W.gnorm));
  E2A_LAUNCH_CHECK();
  MfmaParams p;
  e = base_params<L>(a, W, wb, pl.box, pl.periodic, p);
  if (e != E2A_OK) return e;
  if (8 * p.wg_per_xcd > kMaxRadWg) p.wg_per_xcd = kMaxRadWg / 8;
  e = deal(W, wb, p, a->n_edges, st);
  if (e != E2A_OK) return e;
  p.q = pl.q;
  p.k = pl.k;
  p.lse = a->out_lse;
  p.gpk = reinterpret_cast<const f16x8*>(wb + W.gpk);
  p.gsc = reinterpret_cast<const float*>(wb + W.gsc);
  p.gnorm = reinterpret_cast<const float*>(wb + W.gnorm);
  p.rad_part = reinterpret_cast<float*>(wb + W.radpart);
  e = launch_mode<L, kBwdR>(p, st);
  if (e != E2A_OK) return e;
  constexpr int N = 8 * (L + 1) * kC;
  k_rad_reduce<L><<<(N + 255) / 256, 256, 0, st>>>(p.rad_part, 8 * p.wg_per_xcd, p.gnorm, w_rad);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

}  // namespace

const uint16_t* mfma_grad_bf16(const void* mfma_ws, int64_t n, int L) {
  size_t off = 0;
  switch (L) {
    case 1: off = mfma_ws_layout<1>(n, true).gbf; break;
    case 2: off = mfma_ws_layout<2>(n, true).gbf; break;
    case 3: off = mfma_ws_layout<3>(n, true).gbf; break;
    case 4: off = mfma_ws_layout<4>(n, true).gbf; break;
    default: return nullptr;
  }
  return reinterpret_cast<const uint16_t*>(static_cast<const char*>(mfma_ws) + off);
}

const float* mfma_delta(const void* mfma_ws, int64_t n, int L) {
  size_t off = 0;
  switch (L) {
    case 1: off = mfma_ws_layout<1>(n, true).delta; break;
    case 2: off = mfma_ws_layout<2>(n, true).delta; break;
    case 3: off = mfma_ws_layout<3>(n, true).delta; break;
    case 4: off = mfma_ws_layout<4>(n, true).delta; break;
    default: return nullptr;
  }
  return reinterpret_cast<const float*>(static_cast<const char*>(mfma_ws) + off);
}

e2a_status launch_radial_mfma(const BwdPlan& pl, float* w_rad, hipStream_t s) {
  switch (pl.a->L) {
    case 1: return launch_radial_typed<1>(pl, w_rad, s);
    case 2: return launch_radial_typed<2>(pl, w_rad, s);
    case 3: return launch_radial_typed<3>(pl, w_rad, s);
    case 4: return launch_radial_typed<4>(pl, w_rad, s);
    default: return fail(E2A_ERR_UNSUPPORTED, "MFMA radial pass: L=%d", pl.a->L);
  }
}

size_t mfma_packed_bytes(int L) {
  switch (L) {
    case 1: return Shape<1>::wtotal() * 16;
    case 2: return Shape<2>::wtotal() * 16;
    case 3: return Shape<3>::wtotal() * 16;
    case 4: return Shape<4>::wtotal() * 16;
    default: return 0;
  }
}

e2a_status pack_so2_mfma(const void* w_so2, void* out, int L, hipStream_t st) {
  auto go = [&](auto lc) {
    constexpr int LL = decltype(lc)::value;
    const int64_t nv = Shape<LL>::wtotal();
    k_pack_so2<LL, false><<<(nv + 255) / 256, 256, 0, st>>>(static_cast<const uint16_t*>(w_so2),
                                                             static_cast<bf16x8*>(out));
  };
  switch (L) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    default: return fail(E2A_ERR_UNSUPPORTED, "packed SO(2) image: L=%d", L);
  }
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

size_t order_workspace_bytes(int64_t n) { return mfma_ws_layout<1>(n, false).total; }

e2a_status destination_order(const float* pos, int64_t n, int32_t* order, void* ws, hipStream_t st) {
  if (n == 0) return E2A_OK;
  const MfmaWs W = mfma_ws_layout<1>(n, false);
  return spatial_order(pos, n, W, static_cast<char*>(ws), order, st);
}

bool mfma_supported(int L, int C, int H, int dtype) {
  return L >= 1 && L <= 4 && C == kC && H == kH && dtype == E2A_DTYPE_BF16;
}

size_t mfma_workspace_bytes(int64_t n, int L, int C, bool backward) {
  if (C != kC) return 0;
  switch (L) {
    case 1: return mfma_ws_layout<1>(n, backward).total;
    case 2: return mfma_ws_layout<2>(n, backward).total;
    case 3: return mfma_ws_layout<3>(n, backward).total;
    case 4: return mfma_ws_layout<4>(n, backward).total;
    default: return 0;
  }
}

e2a_status launch_backward_mfma(const BwdPlan& pl, hipStream_t s) {
  switch (pl.a->L) {
    case 1: return launch_bwd_typed<1>(pl, s);
    case 2: return launch_bwd_typed<2>(pl, s);
    case 3: return launch_bwd_typed<3>(pl, s);
    case 4: return launch_bwd_typed<4>(pl, s);
    default: return fail(E2A_ERR_UNSUPPORTED, "MFMA backward: L=%d", pl.a->L);
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

/*
 * e2a.h - C ABI of libe2a, an MI355X (gfx950) implementation of the
 * on-the-fly equivariant attention layer of E2Former-V2 (arXiv 2601.16622,
 * "E2Former-V2: On-the-Fly Equivariant Attention with Linear Activation
 * Memory").
 *
 * The pages describe the layer's problem as atom positions, radius
 * neighbourhoods j in N(i), node irrep features and attention heads
 * (English technical summary, section 1 "Problem Statement" and section 2.2
 * "On-the-Fly Equivariant Attention").  This header turns that into these calls:
 *
 *   e2a_build_neighbors  - cell-list radius graph, CSR sorted by destination;
 *   e2a_attention_fwd    - the fused, node-centric layer;
 *   e2a_conv_fwd         - the same messages summed without attention (the
 *                          EAAS convolution stage);
 *   e2a_attention_bwd    - the layer's gradient with respect to the node
 *                          features.
 *
 * Conventions shared by every entry point:
 *   - Pointers named "device" are HIP device pointers owned by the caller.  The
 *     library never frees them and keeps none of them after the call returns.
 *     The library allocates no device memory: scratch comes in through a
 *     caller-owned workspace whose size a *_workspace_bytes() query gives.
 *     The kernels read arrays in 16-byte vectors: every device array of the
 *     layer's argument struct, and the cotangent of the backward calls, must
 *     start on a 16-byte boundary (hipMalloc and PyTorch's allocator give
 *     256); a misaligned one is refused with E2A_ERR_INVALID_ARG.
 *   - "stream" is a hipStream_t passed as void* (NULL = the default stream).
 *     All device work is enqueued on it, in order.
 *   - Every function that can fail returns an e2a_status.  Argument checks run
 *     on the host before anything is launched, so an invalid call touches
 *     neither the device nor the outputs.  e2a_last_error_message() (per host
 *     thread) says what failed.  No C++ exception crosses this boundary.
 *   - Real spherical-harmonic components are stored at index l*l + l + m
 *     (m = -l..l), orthonormal and without the Condon-Shortley phase, so the
 *     l = 1 block is proportional to (y, z, x).
 */
#ifndef E2A_H_
#define E2A_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define E2A_ABI_VERSION 2

typedef int32_t e2a_status;
enum {
  E2A_OK = 0,
  E2A_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad value, coordinates outside [0, box) */
  E2A_ERR_CAPACITY = 2,      /* col_capacity too small; *n_edges holds the required count       */
  E2A_ERR_BOX_TOO_SMALL = 3, /* a periodic box side is shorter than 2 * cutoff                 */
  E2A_ERR_UNSUPPORTED = 4,   /* (L, C, H, dtype, variant) combination not built                 */
  E2A_ERR_HIP = 5            /* a HIP runtime call failed; the message names it                 */
};

enum { E2A_DTYPE_F32 = 0, E2A_DTYPE_BF16 = 1 };

/* Kernel choice for e2a_attention_fwd.  AUTO picks the MFMA kernel when it is
 * built for (L, C, H, dtype) and the scalar reference kernel otherwise. */
enum { E2A_VARIANT_AUTO = 0, E2A_VARIANT_REFERENCE = 1, E2A_VARIANT_MFMA = 2 };

/* ABI version (E2A_ABI_VERSION of the built library). */
int e2a_version(void);

/* Static, human-readable name of a status code. */
const char* e2a_status_string(e2a_status s);

/* Message of the last failing call on this host thread ("" if none). */
const char* e2a_last_error_message(void);

/* ------------------------------------------------------------------------ */
/* Neighbour graph                                                          */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace e2a_build_neighbors needs for n_atoms atoms. */
size_t e2a_neighbors_workspace_bytes(int64_t n_atoms);

/*
 * Radius graph N(i) = { j != i : batch_j == batch_i, 0 < d_ij < cutoff }
 * (technical summary section 1: |E| ~ kN neighbour edges; section 2.2:
 * the kernel iterates j in N(i)).
 *
 * The predicate is evaluated in fp32 with every operation correctly rounded
 * and no fused multiply-add: dx = x_j - x_i per axis; in a periodic box
 * dx -= box if dx > box/2, else dx += box if dx < -box/2; d2 = (dx*dx + dy*dy)
 * + dz*dz; neighbour iff 0 < d2 < cutoff*cutoff.  Two atoms at one point
 * (d2 = 0) have no edge direction and are not each other's neighbours.  The
 * result is exact and deterministic (independent of launch order).
 *
 *   pos          device f32 [n_atoms, 3].  Periodic: each coordinate must lie
 *                in [0, box_d); otherwise E2A_ERR_INVALID_ARG.
 *   batch        device i32 [n_atoms] graph ids, or NULL (one graph).
 *   box          HOST f32 [3] periodic box sides, or NULL for open boundaries.
 *   cutoff       > 0.  Every periodic side must be >= 2*cutoff
 *                (E2A_ERR_BOX_TOO_SMALL).
 *   row_ptr      device i64 [n_atoms + 1]: edges of i are col[row_ptr[i] ..
 *                row_ptr[i+1]), ascending in j.
 *   col          device i32 [col_capacity].
 *   n_edges      HOST out: the number of edges.  If it exceeds col_capacity
 *                the call returns E2A_ERR_CAPACITY with *n_edges set to the
 *                required count and col untouched; retry with more space.
 *   workspace    device scratch of e2a_neighbors_workspace_bytes(n_atoms).
 *
 * Blocks the calling host thread once, until the edge count is known (one
 * device to host copy of the edge count, the longest row and the bounding
 * box, whose coordinate checks are made then; the cell grid of open
 * boundaries is sized on the device).  Rows longer than 4096 neighbours give
 * E2A_ERR_UNSUPPORTED.
 */
e2a_status e2a_build_neighbors(const float* pos, int64_t n_atoms, const int32_t* batch,
                               const float* box, float cutoff, int64_t* row_ptr, int32_t* col,
                               int64_t col_capacity, int64_t* n_edges, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Fused on-the-fly equivariant attention                                   */
/* ------------------------------------------------------------------------ */

/* Number of SO(2) mixing weights for (L, C): ((L+1)C)^2 + 2 sum_{m=1..L} ((L+1-m)C)^2. */
int64_t e2a_so2_param_count(int L, int C);

typedef struct e2a_attn_args {
  /* geometry and graph */
  const float* pos;        /* device f32 [n_atoms, 3]                                 */
  const float* box;        /* HOST f32 [3] or NULL (open); minimum image when set    */
  int64_t n_atoms;
  const int64_t* row_ptr;  /* device i64 [n_atoms + 1] (CSR by destination);
                              row_ptr[0] = 0 and row_ptr[n_atoms] = n_edges            */
  const int32_t* col;      /* device i32 [n_edges], neighbour j of each edge          */
  int64_t n_edges;
  float cutoff;            /* radius used by the radial basis envelope               */
  /* shapes */
  int L;                   /* 0..4: irrep degrees 0..L, (L+1)^2 components           */
  int C;                   /* channels; multiple of H                                 */
  int H;                   /* heads; head h owns channels [h C/H, (h+1) C/H)          */
  int n_rbf;               /* must be 8                                                */
  int dtype;               /* E2A_DTYPE_F32 or E2A_DTYPE_BF16: storage of the inputs  */
  int variant;             /* E2A_VARIANT_*                                            */
  /* inputs, all device, stored in `dtype` */
  const void* feat;        /* [n_atoms, (L+1)^2, C] node irrep features h             */
  const void* w_q;         /* [C, C]  q_i = h_{i,l=0} W_q                              */
  const void* w_k;         /* [C, C]  k_j = h_{j,l=0} W_k                              */
  const void* w_rad;       /* [n_rbf, L+1, C]  rho[l,c] = sum_k e_k(r) W_rad[k,l,c]     */
  const void* w_so2;       /* [e2a_so2_param_count(L,C)] per-m blocks, see below      */
  /* outputs, device */
  float* out;              /* f32 [n_atoms, (L+1)^2, C], fully overwritten            */
  float* out_lse;          /* f32 [n_atoms, H] log-sum-exp of the logits, or NULL     */
  /* scratch */
  void* workspace;         /* device, e2a_attention_workspace_bytes(...) bytes        */
  size_t workspace_bytes;
  /* optional, device (NULL: the call makes its own) */
  const void* w_so2_packed;  /* e2a_pack_so2_weights of w_so2 (matrix-core path only;
                                the scalar path ignores it)                            */
  const int32_t* order;      /* [n_atoms] the order destinations are visited in, a
                                permutation of 0..n_atoms-1 (e2a_destination_order);
                                results depend on it (which atoms share edge tiles)   */
} e2a_attn_args;

/*
 * Packed SO(2) weights, for callers that run the layer many times on the same
 * weights (every forward call otherwise repacks them).  The matrix-core path
 * streams w_so2 as MFMA B fragments: per |m|, output degree, wave column
 * group and k-step, 64 lanes x 8 bf16 (one 16-byte load per lane).
 * e2a_so2_packed_bytes gives the image's size for (L, C, dtype), 0 where no
 * matrix-core build exists (then the packer returns E2A_ERR_UNSUPPORTED).
 * The image is valid for every call with these weights; the library does not
 * check that it matches w_so2.  Asynchronous.
 */
size_t e2a_so2_packed_bytes(int L, int C, int dtype);
e2a_status e2a_pack_so2_weights(const void* w_so2, void* w_packed, int L, int C, int dtype, void* stream);

/*
 * Spatial order of the destinations the layer uses by default (the Morton
 * code of a 64^3 grid over the bounding box of pos, stably sorted, ties by
 * atom index): atoms close in the order are close in space, so workgroups
 * working on neighbouring destinations share neighbour features in cache.
 * For callers that run several layers on one geometry (stacked blocks), or
 * that keep the order between neighbour-list rebuilds.  order: device i32
 * [n_atoms]; workspace of e2a_destination_order_workspace_bytes(n_atoms).
 */
size_t e2a_destination_order_workspace_bytes(int64_t n_atoms);
e2a_status e2a_destination_order(const float* pos, int64_t n_atoms, int32_t* order, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Bytes of device workspace e2a_attention_fwd needs. */
size_t e2a_attention_workspace_bytes(int64_t n_atoms, int L, int C, int H, int dtype);

/*
 * o_i = sum_{j in N(i)} alpha_ij^{h(c)} v_ij for every destination atom i.
 *
 * Logits come from invariant scalars only (technical summary section 2.2,
 * "Node-Centric Factorization", Eq. 6): q_i = h_{i,0} W_q, k_j = h_{j,0} W_k,
 * s_ij^h = <q_i^h, k_j^h> / sqrt(C/H), alpha = softmax over j in N(i),
 * computed with an online (streaming) softmax ("Online Softmax").
 *
 * Geometry enters only the value v_ij (section 2.1, "Equivariant Axis-Aligned
 * Sparsification", and the abstract): r = x_j - x_i (minimum image), R_ij with
 * R_ij r_hat = z, D^l = Wigner-D of R_ij; x^l = D^l h_j^l; per-m SO(2) mix
 *   m = 0: y_{lo,0}  = sum_li x_{li,0} W0[li,lo]
 *   m > 0: y_{lo,+m} = sum_li x_{li,+m} W1_m[li,lo] - x_{li,-m} W2_m[li,lo]
 *          y_{lo,-m} = sum_li x_{li,+m} W2_m[li,lo] + x_{li,-m} W1_m[li,lo]
 * then yhat_{l,m}[c] = rho[l,c] y_{l,m}[c] with the radial basis
 * e_k(r) = exp(-g (r - mu_k)^2) (cos(pi r/cutoff) + 1)/2, mu_k = k cutoff/7,
 * g = 1/(2 (cutoff/7)^2); and v^l = D^l^T yhat^l.  No per-edge tensor is
 * written to device memory ("Elimination of Edge Materialization").
 *
 * w_so2 layout: for m = 0..L in order, a [(L+1-m)C] x [(L+1-m)C] row-major
 * matrix with row (l_in - m)*C + c_in and column (l_out - m)*C + c_out; one
 * such matrix (W0) for m = 0, two (W1 then W2) for each m >= 1.
 *
 * An atom with no neighbours gets o_i = 0 and lse = -inf.  An edge of zero
 * length (two atoms at one point, which e2a_build_neighbors never pairs) has
 * no direction; it takes r_hat = z (the identity frame).  Range: every matrix
 * product takes bf16 operands (fp32's exponent range) and sums in fp32, so
 * inputs of any magnitude within fp32's normal range keep the stated
 * precision; scaling w_so2 or w_rad by a power of two scales o exactly.
 * Asynchronous: no
 * host synchronisation, no device-memory set or copy commands, only kernel
 * launches on the stream (so a caller may record the call into a HIP graph).
 * Deterministic: the same inputs give bit-identical outputs.  Errors: E2A_ERR_INVALID_ARG (null pointer, C % H != 0,
 * cutoff <= 0, n_rbf != 8, L outside 0..4, workspace too small),
 * E2A_ERR_UNSUPPORTED (variant not built for the shape or dtype).
 */
e2a_status e2a_attention_fwd(const e2a_attn_args* args, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as e2a_attention_fwd, with the same arguments, inputs, outputs,
 * results (bit for bit) and errors, but its scratch comes from a fixed array
 * of E2A_NOALLOC_SCRATCH_BYTES that the library keeps on each GPU it runs on
 * (loaded with the library, held until the process ends).  args->workspace
 * and args->workspace_bytes are ignored.  The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  Sizes whose workspace
 * (e2a_attention_workspace_bytes) exceeds E2A_NOALLOC_SCRATCH_BYTES give
 * E2A_ERR_INVALID_ARG before anything runs (64 MiB holds up to about 60,000
 * atoms at L = 4, C = 128).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Nothing in the array needs to start at zero.
 */
#define E2A_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
e2a_status e2a_attention_fwd_noalloc(const e2a_attn_args* args, void* stream);

/*
 * The EAAS convolution stage: o_i = sum_{j in N(i)} v_ij, the same per-edge
 * messages v_ij as e2a_attention_fwd (rotate in, per-m SO(2) mix, radial
 * scale, rotate out) summed over the neighbourhood with no attention weights
 * (technical summary section 2.1, "Equivariant Axis-Aligned Sparsification",
 * whose result is stated for the convolution stage).  A plain sum: no
 * division by the degree.
 *
 * Takes the same e2a_attn_args: w_q and w_k are not read (may be NULL), H
 * only selects the build (the MFMA kernel is built for H = 8), and out_lse is
 * ignored (nothing is written there).  An atom with no neighbours gets
 * o_i = 0.  Same workspace (e2a_attention_workspace_bytes), same asynchrony,
 * determinism and errors as e2a_attention_fwd.
 */
e2a_status e2a_conv_fwd(const e2a_attn_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* One block around the layer                                               */
/* ------------------------------------------------------------------------ */

/*
 * The pages place the fused attention layer inside the E2Former-V2 model
 * (abstract; technical summary section 2, "Methodology") but print none of
 * the block around it.  This is the plainest equivariant reading, a pre-norm
 * residual block on an fp32 residual stream h (K = (L+1)^2 components):
 *
 *   Norm(x)[l,m,c] = g[l,c] x[l,m,c] / sqrt(mean_{m,c} x[l,m,c]^2 + 1e-6)
 *   h1  = h + Proj(Attn(Norm1(h))),  Proj(a)[l,m,:] = a[l,m,:] W_o[l]
 *   u   = Norm2(h1)[l,m,:] W_1[l],   z = Norm2(h1)[0,0,:] W_gate
 *   act = SiLU(u) for l = 0;  u[l,m,c] sigmoid(z[(l-1) C + c]) for l >= 1
 *   out = h1 + act[l,m,:] W_2[l]
 *
 * Attn is e2a_attention_fwd on Norm1(h) stored in `dtype` (bf16 rounds it),
 * with the attention fields of this struct; stacking blocks is calling this
 * once per block with that block's weights (h_out of one is h_in of the next).
 * Node-wise products take bf16 operands on the matrix cores for bf16 storage
 * (C a multiple of 32, at most 128) and fp32 otherwise; sums are fp32.  With
 * bf16 storage the gated activations are rounded to bf16 (Norm1(h), Norm2(h1)
 * likewise); u itself stays fp32 up to the gate.
 */
typedef struct e2a_block_args {
  const float* pos;        /* device f32 [n_atoms, 3]                                 */
  const float* box;        /* HOST f32 [3] or NULL (open)                             */
  int64_t n_atoms;
  const int64_t* row_ptr;  /* device i64 [n_atoms + 1], as for e2a_attention_fwd      */
  const int32_t* col;      /* device i32 [n_edges]                                    */
  int64_t n_edges;
  float cutoff;
  int L, C, H, n_rbf, dtype, variant;   /* as for e2a_attention_fwd                */
  const float* h_in;       /* device f32 [n_atoms, K, C] residual stream in           */
  float* h_out;            /* device f32 [n_atoms, K, C]; may equal h_in              */
  /* weights, device, stored in `dtype` */
  const void* norm1;       /* [L+1, C]                                                */
  const void* w_q;         /* [C, C]          attention, as in e2a_attn_args          */
  const void* w_k;         /* [C, C]                                                  */
  const void* w_rad;       /* [n_rbf, L+1, C]                                         */
  const void* w_so2;       /* [e2a_so2_param_count(L, C)]                             */
  const void* w_o;         /* [L+1, C, C]     projection of the layer's output        */
  const void* norm2;       /* [L+1, C]                                                */
  const void* w_1;         /* [L+1, C, C]     FFN in                                  */
  const void* w_gate;      /* [C, L*C]        gate logits of degrees 1..L (NULL if L=0) */
  const void* w_2;         /* [L+1, C, C]     FFN out                                 */
  void* workspace;         /* device, e2a_block_workspace_bytes(...) bytes            */
  size_t workspace_bytes;
  const void* w_so2_packed;  /* optional, as in e2a_attn_args                          */
  const int32_t* order;      /* optional, as in e2a_attn_args                          */
} e2a_block_args;

/* Bytes of device workspace e2a_block_fwd needs (0 for invalid sizes). */
size_t e2a_block_workspace_bytes(int64_t n_atoms, int L, int C, int H, int dtype);

/* One block (above).  Asynchronous and deterministic; no memory set or copy
 * commands.  Errors as e2a_attention_fwd, plus E2A_ERR_INVALID_ARG for a NULL
 * h_in, h_out or node-wise weight or an h_in, h_out not on a 16-byte boundary,
 * and E2A_ERR_UNSUPPORTED for C not a multiple of 4 or n_atoms (2L+1) >= 2^31. */
e2a_status e2a_block_fwd(const e2a_block_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Feature gradient                                                         */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace e2a_attention_bwd needs. */
size_t e2a_attention_bwd_workspace_bytes(int64_t n_atoms, int64_t n_edges, int L, int C, int H);

/*
 * dL/dh of e2a_attention_fwd for a cotangent grad_out = dL/do: the backward
 * that training the layer needs (technical summary section 2.2: per-edge
 * quantities are recomputed from the per-destination softmax statistics
 * rather than stored).  With G = grad_out, alpha_ij = exp(s_ij - lse_i):
 *   ds_ij = alpha_ij (sum_{k, c in h} G_i v_ij - sum_{k, c in h} G_i o_i),
 *   dh_j  = sum_{i: j in N(i)} D_ij^T SO2^T(rho_ij * D_ij (alpha_ij G_i))
 *           + [l = 0] (sum_j' ds_jj' k_j' W_q^T + sum_i ds_ij q_i W_k^T) / sqrt(C/H),
 * where SO2^T is the transposed per-m mix and D_ij, rho_ij belong to the
 * edge from centre i to neighbour j.  Gradients of the weights and positions
 * are not computed.
 *
 *   args       the forward's arguments, with out = the forward's output o
 *              (f32 [n_atoms, (L+1)^2, C]) and out_lse = its log-normaliser
 *              (f32 [n_atoms, H]), both INPUTS here and both required;
 *              workspace / workspace_bytes as e2a_attention_bwd_workspace_bytes
 *              gives for (n_atoms, n_edges).  The neighbour graph must be
 *              symmetric (j in N(i) iff i in N(j)), as e2a_build_neighbors
 *              builds it, with rows ascending in j.
 *   grad_out   device f32 [n_atoms, (L+1)^2, C].
 *   grad_feat  device f32 [n_atoms, (L+1)^2, C], fully overwritten.
 *
 * Variant REFERENCE runs scalar fp32 kernels (any shape, fp32 or bf16
 * storage).  MFMA runs the matrix-core passes (bf16 storage, C = 128, H = 8,
 * 1 <= L <= 4; other shapes give E2A_ERR_UNSUPPORTED): a query pass and a
 * value pass of the forward's fused kernel with bf16 operands and fp32
 * accumulation, relative L2 error a few 1e-3 against an exact gradient.
 * AUTO takes MFMA where it is built, else REFERENCE.  The matrix-core passes
 * normalise the cotangent by powers of two (per atom, and by its largest
 * entry), so its magnitude does not matter within fp32's normal range.
 * The workspace keeps one float per edge and head (the softmax gradient ds)
 * and, for MFMA, the cotangent's copies.  Asynchronous and deterministic,
 * like the forward.  Errors as e2a_attention_fwd, plus E2A_ERR_INVALID_ARG
 * for a NULL out, out_lse, grad_out or grad_feat.
 */
e2a_status e2a_attention_bwd(const e2a_attn_args* args, const float* grad_out, float* grad_feat, void* stream);

/* Workspace bytes e2a_attention_bwd_weights needs for these sizes (the same
 * for fp32 and bf16 storage); 0 for invalid sizes. */
size_t e2a_attention_bwd_weights_workspace_bytes(int64_t n_atoms, int64_t n_edges, int L, int C, int H);

/*
 * Gradients of e2a_attention_fwd with respect to its weights, and optionally
 * its node features and the atom positions, for a cotangent grad_out =
 * dL/do: what training the layer needs, and the forces of an energy built on
 * it (technical summary section 2.2; the message steps of section 2.1).  With ds_ij, dq_i, dk_j as in e2a_attention_bwd, the edge cotangent
 * alpha_ij G_i, x_ij = D_ij h_j, y = SO2(x), dyhat = D_ij (alpha_ij G_i),
 * rho_ij[l][c] = sum_k e_k(r_ij) W_rad[k][l][c] and dy = rho_ij dyhat:
 *   dW_q = sum_i h_{i,0}^T dq_i,   dW_k = sum_j h_{j,0}^T dk_j,
 *   dW_rad[k][l][c] = sum_ij e_k(r_ij) sum_m y[l,m][c] dyhat[l,m][c],
 *   per m: dW0 = sum X0^T dY0,  dW1 = sum Xp^T dYp + Xm^T dYm,
 *          dW2 = sum Xp^T dYm - Xm^T dYp
 * (X0, Xp, Xm the rows m = 0, +m, -m of x laid out as in w_so2's blocks).
 * Positions (neighbour graph held fixed): each edge vector r_ij = x_j - x_i
 * enters through its length (the radial basis) and its direction (the
 * Wigner blocks); with T_a the derivative along a rotation of r_hat about
 * axis a (the frame turned with it, dD^l = D^l(R(1 - [e_a]x)) - D^l) and
 * s = sum_{l,c} dL/drho[l][c] drho[l][c]/dr,
 *   dL/dr_ij = s r_hat + (T x r_hat) / |r|,   dL/dx_j += dL/dr_ij, dL/dx_i -= dL/dr_ij.
 *
 *   args        as for e2a_attention_bwd (out and out_lse of the forward are
 *               required); workspace / workspace_bytes as
 *               e2a_attention_bwd_weights_workspace_bytes gives.
 *   grad_out    device f32 [n_atoms, (L+1)^2, C].
 *   grad_feat   NULL, or device f32 [n_atoms, (L+1)^2, C]: dL/dh as
 *               e2a_attention_bwd computes it.
 *   grad_w_q, grad_w_k   NULL or device f32 [C, C] (layout of w_q, w_k).
 *   grad_w_rad  NULL or device f32 [8, L+1, C].
 *   grad_w_so2  NULL or device f32 [e2a_so2_param_count(L, C)] (layout of w_so2).
 *   grad_pos    NULL or device f32 [n_atoms, 3] (layout of pos).
 * Every output that is set is overwritten; at least one must be set.
 *
 * dL/dh and ds come from the same kernels as e2a_attention_bwd (variant as
 * there); the query pass runs only when grad_feat, grad_w_q or grad_w_k is
 * set.  One exception: with grad_feat and grad_pos set, neither grad_w_q,
 * grad_w_k nor grad_w_rad, bf16 storage, C = 128, H = 8 and the matrix-core
 * variant, ds_ij is formed from the edge batches instead (the sum over a
 * head's channels and every (l, m) of y dy is alpha_ij dL/dalpha_ij, so
 * ds = sum y dy - alpha delta_i) with y and dy in bf16; then dL/dh's rows
 * l >= 1 equal e2a_attention_bwd's bit for bit and row 0 agrees to within
 * the bf16 rounding of y and dy.  W_rad and W_so2 sum over all edges into
 * matrices too large for a workgroup, so the workspace holds per-edge
 * tensors for one batch of at most 262144 edges at a time: rotated features
 * and cotangents (storage precision), SO2(x) in fp32 (bf16 where the
 * matrix-core kernels read it).  The GEMMs run on the matrix cores for bf16
 * storage (bf16 operands, fp32 sums) and in fp32 otherwise; all sums run in
 * a fixed order, so results are bit-reproducible.  Asynchronous.  Errors as
 * e2a_attention_bwd, plus E2A_ERR_INVALID_ARG when no output is set.
 */
e2a_status e2a_attention_bwd_weights(const e2a_attn_args* args, const float* grad_out, float* grad_feat,
                                     float* grad_w_q, float* grad_w_k, float* grad_w_rad, float* grad_w_so2,
                                     float* grad_pos, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* E2A_H_ */

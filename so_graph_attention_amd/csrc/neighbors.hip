// Cell-list radius graph: CSR sorted by destination atom, rows ascending in j.
//
// The layer streams j in N(i) for every destination i (arXiv 2601.16622,
// English technical summary section 2.2, "Streaming Reduction"; section 1
// gives |E| ~ kN).  The pages do not say how N(i) is built; this is a
// deterministic counting-sort cell list:
//   1. bounding box (and coordinate check), on the device; an open system's
//      cell grid is sized from it there, a periodic one's from the box sides;
//   2. bin atoms into cells of side >= 1.001 * cutoff (counting sort), with
//      each atom's position and batch id copied to its cell-order slot;
//   3. count the neighbours of each atom over its <= 27 stencil cells (one
//      wavefront per atom, the cells' candidates flattened across lanes);
//   4. exclusive scan -> row_ptr; read the edge count, longest row and
//      bounding box back (the call's one wait on the device) and check them;
//   5. one wavefront per atom gathers its neighbours with ballot compaction
//      into LDS and writes the row sorted (rank of each entry for rows of up
//      to 256, an LDS bitonic sort for longer ones).
// The pair predicate is the fp32 rule documented in e2a.h, written with
// explicitly rounded intrinsics so that no multiply-add is ever fused.
#include <climits>
#include <cstring>

#include "e2a_internal.hpp"

namespace e2a {
namespace {

constexpr int kScanBlock = 1024;   // elements per scan block (256 threads x 4)
constexpr int kMaxRow = 4096;      // longest row the LDS sort handles
constexpr int kRowFast = 256;      // rows up to this length take the wave-per-atom fill
constexpr int kCandTab = 1024;     // candidates per atom whose slots a wave tabulates in LDS
constexpr int kBboxBlocks = kBboxPartialFloats / 8;   // first-stage blocks of the bounding box

struct Grid {
  int n[3];
  float origin[3];
  float inv_side[3];
  int periodic;
  float box[3];
  float half[3];
  float rc2;
};

// The grid a kernel runs on: given by value (a periodic box, sized on the
// host from its sides), or in device memory (open boundaries, sized on the
// device from the bounding box so that the host need not read it back first).
struct GridArg {
  Grid g;
  const Grid* dev;
};
__device__ __forceinline__ Grid load_grid(const GridArg& a) { return a.dev ? *a.dev : a.g; }

__device__ __forceinline__ int cell_coord(float x, int d, const Grid& g) {
  int c = static_cast<int>(floorf((x - g.origin[d]) * g.inv_side[d]));
  return c < 0 ? 0 : (c >= g.n[d] ? g.n[d] - 1 : c);
}

// Up to three distinct stencil coordinates along one axis.
__device__ __forceinline__ int stencil(int c, int d, const Grid& g, int out[3]) {
  const int n = g.n[d];
  if (g.periodic) {
    if (n >= 3) {
      out[0] = (c + n - 1) % n; out[1] = c; out[2] = (c + 1) % n;
      return 3;
    }
    out[0] = 0; out[1] = 1;
    return n;
  }
  int k = 0;
  for (int o = -1; o <= 1; ++o) {
    const int cc = c + o;
    if (cc >= 0 && cc < n) out[k++] = cc;
  }
  return k;
}

__device__ __forceinline__ bool pair_ok(const float* pi, const float* pj, const Grid& g) {
  float d2 = 0.0f;
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    float dx = __fsub_rn(pj[d], pi[d]);
    if (g.periodic) {
      if (dx > g.half[d]) dx = __fsub_rn(dx, g.box[d]);
      else if (dx < -g.half[d]) dx = __fadd_rn(dx, g.box[d]);
    }
    const float sq = __fmul_rn(dx, dx);
    d2 = (d == 0) ? sq : __fadd_rn(d2, sq);
  }
  // d2 = 0 (two atoms at one point in fp32) gives no edge: such a pair has no direction
  return d2 > 0.0f && d2 < g.rc2;
}

// ---- bounding box ---------------------------------------------------------
// out[0..2] = min, out[3..5] = max, out[6] = 1 if any coordinate is not finite.
__device__ __forceinline__ void bbox_reduce(float (&mn)[3], float (&mx)[3], int& bad, float (*smin)[256],
                                            float (*smax)[256], int* sbad) {
  for (int d = 0; d < 3; ++d) { smin[d][threadIdx.x] = mn[d]; smax[d][threadIdx.x] = mx[d]; }
  sbad[threadIdx.x] = bad;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) {
      for (int d = 0; d < 3; ++d) {
        smin[d][threadIdx.x] = fminf(smin[d][threadIdx.x], smin[d][threadIdx.x + st]);
        smax[d][threadIdx.x] = fmaxf(smax[d][threadIdx.x], smax[d][threadIdx.x + st]);
      }
      sbad[threadIdx.x] |= sbad[threadIdx.x + st];
    }
    __syncthreads();
  }
}

// Stage 1: block b reduces atoms b, b + gridDim.x, ... (grid-stride by block
// and thread) into partial[b][0..6].
__global__ void __launch_bounds__(256) k_bbox_partial(const float* __restrict__ pos, int64_t n,
                                                      float* __restrict__ partial) {
  __shared__ float smin[3][256], smax[3][256];
  __shared__ int sbad[256];
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  int bad = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float x = pos[3 * i + d];
      if (!isfinite(x)) bad = 1;
      mn[d] = fminf(mn[d], x);
      mx[d] = fmaxf(mx[d], x);
    }
  }
  bbox_reduce(mn, mx, bad, smin, smax, sbad);
  if (threadIdx.x == 0) {
    float* o = partial + 8 * blockIdx.x;
    for (int d = 0; d < 3; ++d) { o[d] = smin[d][0]; o[3 + d] = smax[d][0]; }
    o[6] = sbad[0] ? 1.0f : 0.0f;
  }
}

// Stage 2: out[0..2] = min, out[3..5] = max, out[6] = 1 if any coordinate is
// not finite.
__global__ void __launch_bounds__(256) k_bbox_final(const float* __restrict__ partial, int nparts,
                                                    float* __restrict__ out) {
  __shared__ float smin[3][256], smax[3][256];
  __shared__ int sbad[256];
  float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
  int bad = 0;
  for (int b = threadIdx.x; b < nparts; b += blockDim.x) {
    const float* o = partial + 8 * b;
    for (int d = 0; d < 3; ++d) { mn[d] = fminf(mn[d], o[d]); mx[d] = fmaxf(mx[d], o[3 + d]); }
    bad |= o[6] != 0.0f;
  }
  bbox_reduce(mn, mx, bad, smin, smax, sbad);
  if (threadIdx.x == 0) {
    for (int d = 0; d < 3; ++d) { out[d] = smin[d][0]; out[3 + d] = smax[d][0]; }
    out[6] = sbad[0] ? 1.0f : 0.0f;
  }
}

// Open boundaries: the cell grid from the bounding box bbox[0..6], cells of
// side >= 1.001 cutoff over [min, max], the largest axis halved until at
// most cap cells remain.  Any side of at least the cutoff gives the same
// neighbour lists (the stencil reaches one cell each way), so the grid only
// needs to be safe; for non-finite coordinates (reported by the host after
// the edge-count read-back) it is one cell, and extents are clamped before
// the integer conversion.  One thread.
__global__ void k_grid_open(const float* __restrict__ bbox, float cutoff, int64_t cap, Grid* __restrict__ out,
                            int64_t* __restrict__ ncell) {
  Grid g{};
  g.periodic = 0;
  g.rc2 = cutoff * cutoff;
  const float side_min = cutoff * 1.001f;
  const bool finite = bbox[6] == 0.0f;
  for (int d = 0; d < 3; ++d) {
    const float ext = finite ? bbox[3 + d] - bbox[d] : 0.0f;
    float e = ext / side_min;
    if (!(e < 1048576.0f)) e = 1048576.0f;
    g.n[d] = static_cast<int>(floorf(e)) + 1;
    g.origin[d] = finite ? bbox[d] : 0.0f;
  }
  while ((int64_t)g.n[0] * g.n[1] * g.n[2] > cap) {
    int d = 0;
    if (g.n[1] > g.n[d]) d = 1;
    if (g.n[2] > g.n[d]) d = 2;
    g.n[d] = g.n[d] / 2 > 1 ? g.n[d] / 2 : 1;
  }
  for (int d = 0; d < 3; ++d) {
    const float ext = finite ? bbox[3 + d] - bbox[d] : 0.0f;
    const float side = fmaxf(side_min, ext / g.n[d] * 1.0001f);
    g.inv_side[d] = 1.0f / side;
  }
  *out = g;
  *ncell = (int64_t)g.n[0] * g.n[1] * g.n[2];
}

__global__ void k_bin(const float* __restrict__ pos, int64_t n, GridArg ga, int32_t* __restrict__ cell_of,
                      int32_t* __restrict__ cell_cnt) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const Grid g = load_grid(ga);
  const int cx = cell_coord(pos[3 * i + 0], 0, g);
  const int cy = cell_coord(pos[3 * i + 1], 1, g);
  const int cz = cell_coord(pos[3 * i + 2], 2, g);
  const int c = (cz * g.n[1] + cy) * g.n[0] + cx;
  cell_of[i] = c;
  atomicAdd(&cell_cnt[c], 1);
}

// Atom i to its slot of its cell; the slot also gets i's position and batch
// id (bits in w), so that the pair tests read a candidate by slot in one
// 16-byte load, independent of the load of its atom id.
__global__ void k_scatter(int64_t n, const float* __restrict__ pos, const int32_t* __restrict__ batch,
                          const int32_t* __restrict__ cell_of, const int32_t* __restrict__ cell_start,
                          int32_t* __restrict__ cursor, int32_t* __restrict__ cell_atoms, float4* __restrict__ pos_cell) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int c = cell_of[i];
  const int slot = cell_start[c] + atomicAdd(&cursor[c], 1);
  cell_atoms[slot] = static_cast<int32_t>(i);
  pos_cell[slot] = float4{pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], __int_as_float(batch ? batch[i] : 0)};
}

// ---- exclusive scan (int32 in, T out, total at out[n]) ---------------------
__global__ void k_scan_reduce(const int32_t* __restrict__ in, int64_t n, int64_t* __restrict__ bsum) {
  __shared__ int64_t s[256];
  const int64_t base = blockIdx.x * (int64_t)kScanBlock;
  int64_t acc = 0;
  for (int k = 0; k < 4; ++k) {
    const int64_t t = base + threadIdx.x * 4 + k;
    if (t < n) acc += in[t];
  }
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) s[threadIdx.x] += s[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = s[0];
}

// One block: exclusive scan of nb block sums in place; total to bsum[nb].
__global__ void k_scan_blocks(int64_t* __restrict__ bsum, int64_t nb) {
  __shared__ int64_t s[256];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < nb; base += 256) {
    const int64_t t = base + threadIdx.x;
    const int64_t v = t < nb ? bsum[t] : 0;
    s[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int64_t add = threadIdx.x >= off ? s[threadIdx.x - off] : 0;
      __syncthreads();
      s[threadIdx.x] += add;
      __syncthreads();
    }
    if (t < nb) bsum[t] = carry + s[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 255) carry += s[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[nb] = carry;
}

template <typename T>
// (in and clear may be one array: neither is restrict-qualified)
__global__ void k_scan_apply(const int32_t* in, int64_t n, const int64_t* __restrict__ boff,
                             T* __restrict__ out, int32_t* clear) {
  __shared__ int64_t s[256];
  const int64_t base = blockIdx.x * (int64_t)kScanBlock;
  int64_t v[4];
  int64_t loc = 0;
  for (int k = 0; k < 4; ++k) {
    const int64_t t = base + threadIdx.x * 4 + k;
    v[k] = t < n ? in[t] : 0;
    loc += v[k];
    if (clear && t < n) clear[t] = 0;
  }
  s[threadIdx.x] = loc;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int64_t add = threadIdx.x >= off ? s[threadIdx.x - off] : 0;
    __syncthreads();
    s[threadIdx.x] += add;
    __syncthreads();
  }
  int64_t run = boff[blockIdx.x] + s[threadIdx.x] - loc;
  for (int k = 0; k < 4; ++k) {
    const int64_t t = base + threadIdx.x * 4 + k;
    if (t < n) out[t] = static_cast<T>(run);
    run += v[k];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    const int nb = gridDim.x;
    out[n] = static_cast<T>(boff[nb]);
  }
}

// Inputs up to kScanSingle entries: one block of 1024 threads, in tiles of
// 4096 entries (4 consecutive per thread), each scanned across the block and
// offset by the total of the tiles before it.  One launch instead of three;
// its tiles run one after another, so past about 16k entries the three
// launches are faster (measured).
constexpr int64_t kScanSingle = 16384;

__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int o) {
  const int lo = __shfl_up(static_cast<int>(static_cast<uint64_t>(v)), o);
  const int hi = __shfl_up(static_cast<int>(static_cast<uint64_t>(v) >> 32), o);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}

// n_dev (optional): a length found on the device, at most n, scanned instead.
// clear (optional, the input's address): each entry is set to zero once read.
template <typename T>
__global__ void __launch_bounds__(1024) k_scan_single(const int32_t* in, int64_t n, T* __restrict__ out,
                                                      const int64_t* __restrict__ n_dev, int32_t* clear) {
  __shared__ int64_t wsum[16];
  if (n_dev && *n_dev < n) n = *n_dev;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += 4096) {
    int64_t v[4];
    int64_t loc = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = base + threadIdx.x * 4 + k;
      v[k] = t < n ? in[t] : 0;
      loc += v[k];
      if (clear && t < n) clear[t] = 0;
    }
    int64_t inc = loc;   // inclusive sum over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t u = shfl_up_i64(inc, o);
      if (lane >= o) inc += u;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int64_t before = 0, tile = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int64_t x = wsum[w];
      before += w < wave ? x : 0;
      tile += x;
    }
    __syncthreads();   // wsum is rewritten by the next tile
    int64_t run = carry + before + inc - loc;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = base + threadIdx.x * 4 + k;
      if (t < n) out[t] = static_cast<T>(run);
      run += v[k];
    }
    carry += tile;
  }
  if (threadIdx.x == 0) out[n] = static_cast<T>(carry);
}

// n_dev (optional, one-block scans only): the device holds a shorter length.
// clear (optional, the input's address): the input is left all zero (the
// entries scanned are cleared as they are read; the caller owns the rest).
template <typename T>
e2a_status exclusive_scan(const int32_t* in, int64_t n, T* out, int64_t* bsum, hipStream_t s,
                          const int64_t* n_dev = nullptr, int32_t* clear = nullptr) {
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  if (nb == 0) {
    E2A_HIP_CHECK(hipMemsetAsync(out, 0, sizeof(T), s));
    return E2A_OK;
  }
  if (n <= kScanSingle) {
    k_scan_single<T><<<1, 1024, 0, s>>>(in, n, out, n_dev, clear);
    E2A_LAUNCH_CHECK();
    return E2A_OK;
  }
  k_scan_reduce<<<nb, 256, 0, s>>>(in, n, bsum);
  k_scan_blocks<<<1, 256, 0, s>>>(bsum, nb);
  k_scan_apply<T><<<nb, 256, 0, s>>>(in, n, bsum, out, clear);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

// ---- candidates of one destination atom, one wavefront ---------------------
// The <= 27 stencil cells' atom ranges are flattened: lane l handles
// candidates l, l + 64, ... of the concatenation (cells in stencil order,
// atoms in cell order), so that every pass keeps all 64 lanes busy.
// sh: 64 ints of LDS for this wavefront, tab: kCandTab ints (the slots of
// the first kCandTab candidates, written once per atom by the stencil lanes,
// so that a pass finds its slots in one LDS read; candidates past it search
// the cell starts).  f(valid, j, q) is called once per
// pass by every lane, with the candidate's atom id and its cell-order copy of
// position and batch id (slot 0's when not valid); the next pass's two loads
// are issued before f runs on the current one.
template <typename F>
__device__ __forceinline__ void for_candidates(const float (&pi)[3], const Grid& g,
                                               const int32_t* __restrict__ cell_start,
                                               const int32_t* __restrict__ cell_atoms,
                                               const float4* __restrict__ pos_cell, int lane, int* sh, int* tab,
                                               F&& f) {
  int sx[3], sy[3], sz[3];
  const int nx = stencil(cell_coord(pi[0], 0, g), 0, g, sx);
  const int ny = stencil(cell_coord(pi[1], 1, g), 1, g, sy);
  const int nz = stencil(cell_coord(pi[2], 2, g), 2, g, sz);
  const int ncells = nx * ny * nz;
  int cstart = 0, ccnt = 0;
  if (lane < ncells) {
    const int a = lane / (ny * nx), b = (lane / nx) % ny, c = lane % nx;
    const int cell = (sz[a] * g.n[1] + sy[b]) * g.n[0] + sx[c];
    cstart = cell_start[cell];
    ccnt = cell_start[cell + 1] - cstart;
  }
  int incl = ccnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  const int total = __shfl(incl, 63);
  if (lane < 32) {
    sh[lane] = incl - ccnt;   // first flattened index of the lane's cell
    sh[32 + lane] = cstart;
  }
  for (int k = 0, t = incl - ccnt; k < ccnt && t < kCandTab; ++k, ++t) tab[t] = cstart + k;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // slot of flattened candidate t: from the table, or past it the last cell
  // whose first index is <= t (empty cells never win: the next non-empty
  // cell starts after t)
  auto slot_of = [&](int t) {
    if (t >= total) return 0;
    if (t < kCandTab) return tab[t];
    int lo = 0, hi = ncells;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sh[mid] <= t) lo = mid;
      else hi = mid;
    }
    return sh[32 + lo] + (t - sh[lo]);
  };
  int s = slot_of(lane);
  int j = cell_atoms[s];
  float4 q = pos_cell[s];
  for (int base = 0; base < total; base += 64) {
    const int sn = slot_of(base + 64 + lane);
    const int jn = cell_atoms[sn];
    const float4 qn = pos_cell[sn];
    f(base + lane < total, j, q);
    j = jn;
    q = qn;
  }
}

// ---- neighbour count: one wavefront per destination atom, 4 per block ------
__global__ void __launch_bounds__(256) k_count(const float* __restrict__ pos, int64_t n,
                                               const int32_t* __restrict__ batch, GridArg ga,
                                               const int32_t* __restrict__ cell_start,
                                               const int32_t* __restrict__ cell_atoms,
                                               const float4* __restrict__ pos_cell, const float* __restrict__ bbox,
                                               int32_t* __restrict__ row_cnt) {
  __shared__ int sh[4][64];
  __shared__ int tab[4][kCandTab];
  const int w = threadIdx.x >> 6;
  const int64_t i = blockIdx.x * 4 + w;
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const Grid g = load_grid(ga);
  // coordinates the host will refuse (non-finite, or outside a periodic box)
  // may put every atom into one clamped cell: count nothing instead of
  // testing all pairs on the way to that error
  bool bad = bbox[6] != 0.0f;
  if (g.periodic)
    for (int d = 0; d < 3; ++d) bad = bad || bbox[d] < 0.0f || bbox[3 + d] >= g.box[d];
  if (bad) {
    if (lane == 0) row_cnt[i] = 0;
    return;
  }
  const float pi[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
  const int bi = batch ? batch[i] : 0;
  int cnt = 0;
  for_candidates(pi, g, cell_start, cell_atoms, pos_cell, lane, sh[w], tab[w], [&](bool valid, int j, const float4& q) {
    bool ok = valid && (j != i) && (!batch || __float_as_int(q.w) == bi);
    if (ok) {
      const float pj[3] = {q.x, q.y, q.z};
      ok = pair_ok(pi, pj, g);
    }
    cnt += __popcll(__ballot(ok));
  });
  if (lane == 0) row_cnt[i] = cnt;
}

// out[0] = number of edges, out[1] = longest row (one block of 1024 threads,
// four independent loads in flight per thread).
__global__ void __launch_bounds__(1024) k_readback(const int64_t* __restrict__ row_ptr, int64_t n,
                                                   const int32_t* __restrict__ row_cnt, int64_t* __restrict__ out) {
  __shared__ int32_t sm[1024];
  int32_t m = 0;
  for (int64_t i = threadIdx.x; i < n; i += 4 * (int64_t)blockDim.x) {
    int32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t k = i + u * (int64_t)blockDim.x;
      v[u] = k < n ? row_cnt[k] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) m = max(m, v[u]);
  }
  sm[threadIdx.x] = m;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if (threadIdx.x < st) sm[threadIdx.x] = max(sm[threadIdx.x], sm[threadIdx.x + st]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = row_ptr[n];
    out[1] = sm[0];
  }
}

// ---- fill + sort, rows of at most kRowFast entries: one wavefront per atom,
// 4 per block.  Candidates are compacted into the wave's LDS row with a
// ballot; each entry's position in the sorted row is the number of smaller
// entries (the atom ids of a row are distinct), so the row is written sorted
// straight from registers.
__global__ void __launch_bounds__(256) k_fill_fast(const float* __restrict__ pos, int64_t n,
                                                   const int32_t* __restrict__ batch, GridArg ga,
                                                   const int32_t* __restrict__ cell_start,
                                                   const int32_t* __restrict__ cell_atoms,
                                                   const float4* __restrict__ pos_cell,
                                                   const int64_t* __restrict__ row_ptr, int32_t* __restrict__ col) {
  __shared__ int32_t rows[4][kRowFast];
  __shared__ int sh[4][64];
  __shared__ int tab[4][kCandTab];
  const int w = threadIdx.x >> 6;
  const int64_t i = blockIdx.x * 4 + w;
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const Grid g = load_grid(ga);
  int32_t* buf = rows[w];
  const float pi[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
  const int bi = batch ? batch[i] : 0;
  int cnt = 0;
  for_candidates(pi, g, cell_start, cell_atoms, pos_cell, lane, sh[w], tab[w], [&](bool valid, int j, const float4& q) {
    bool ok = valid && (j != i) && (!batch || __float_as_int(q.w) == bi);
    if (ok) {
      const float pj[3] = {q.x, q.y, q.z};
      ok = pair_ok(pi, pj, g);
    }
    const uint64_t mask = __ballot(ok);
    if (ok) {
      const int slot = cnt + __popcll(mask & ((1ull << lane) - 1ull));
      if (slot < kRowFast) buf[slot] = j;
    }
    cnt += __popcll(mask);
  });
  // The host launches this kernel only when every row fits (count pass).
  // the row was written by other lanes of this wavefront
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int64_t o = row_ptr[i];
  for (int t = lane; t < cnt; t += 64) {
    const int32_t v = buf[t];
    int rank = 0;
    for (int u = 0; u < cnt; ++u) rank += buf[u] < v ? 1 : 0;
    col[o + rank] = v;
  }
}

// ---- fill + sort, any row up to kMaxRow: one wavefront (= one block) per atom
__global__ void __launch_bounds__(64) k_fill(const float* __restrict__ pos, int64_t n,
                                             const int32_t* __restrict__ batch, GridArg ga,
                                             const int32_t* __restrict__ cell_start,
                                             const int32_t* __restrict__ cell_atoms,
                                             const float4* __restrict__ pos_cell,
                                             const int64_t* __restrict__ row_ptr, int32_t* __restrict__ col) {
  __shared__ int32_t buf[kMaxRow];
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x;
  const Grid g = load_grid(ga);
  const float pi[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
  const int bi = batch ? batch[i] : 0;
  int sx[3], sy[3], sz[3];
  const int nx = stencil(cell_coord(pi[0], 0, g), 0, g, sx);
  const int ny = stencil(cell_coord(pi[1], 1, g), 1, g, sy);
  const int nz = stencil(cell_coord(pi[2], 2, g), 2, g, sz);
  int cnt = 0;
  for (int a = 0; a < nz; ++a)
    for (int b = 0; b < ny; ++b)
      for (int c = 0; c < nx; ++c) {
        const int cell = (sz[a] * g.n[1] + sy[b]) * g.n[0] + sx[c];
        const int t0 = cell_start[cell], t1 = cell_start[cell + 1];
        for (int base = t0; base < t1; base += 64) {
          const int t = base + lane;
          bool ok = false;
          int j = 0;
          if (t < t1) {
            j = cell_atoms[t];
            const float4 q = pos_cell[t];
            ok = (j != i) && (!batch || __float_as_int(q.w) == bi);
            if (ok) {
              const float pj[3] = {q.x, q.y, q.z};
              ok = pair_ok(pi, pj, g);
            }
          }
          const uint64_t mask = __ballot(ok);
          if (ok) {
            const int slot = cnt + __popcll(mask & ((1ull << lane) - 1ull));
            if (slot < kMaxRow) buf[slot] = j;
          }
          cnt += __popcll(mask);
        }
      }
  // The host has already checked cnt <= kMaxRow from the count pass.
  int P = 1;
  while (P < cnt) P <<= 1;
  for (int t = cnt + lane; t < P; t += 64) buf[t] = INT_MAX;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int t = lane; t < P; t += 64) {
        const int u = t ^ jj;
        if (u > t) {
          const int x = buf[t], y = buf[u];
          const bool up = (t & k) == 0;
          if ((x > y) == up) { buf[t] = y; buf[u] = x; }
        }
      }
      __syncthreads();
    }
  }
  const int64_t o = row_ptr[i];
  for (int t = lane; t < cnt; t += 64) col[o + t] = buf[t];
}

struct WsLayout {
  size_t cell_of, cell_cnt, cursor, cell_atoms, pos_cell, row_cnt, bsum, small, bbox_part, total;
  int64_t cap_cells;
};

WsLayout ws_layout(int64_t n) {
  WsLayout w{};
  const int64_t cap = 4 * n + 4096;
  const int64_t nb = (std::max<int64_t>(n, cap + 1) + kScanBlock - 1) / kScanBlock + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  w.cell_of = take(sizeof(int32_t) * n);
  w.cell_cnt = take(sizeof(int32_t) * (cap + 1));
  w.cursor = take(sizeof(int32_t) * cap);
  w.cell_atoms = take(sizeof(int32_t) * n);
  w.pos_cell = take(sizeof(float) * 4 * n);
  w.row_cnt = take(sizeof(int32_t) * n);
  w.bsum = take(sizeof(int64_t) * nb);
  w.small = take(256);
  w.bbox_part = take(sizeof(float) * kBboxPartialFloats);
  w.total = off;
  w.cap_cells = cap;
  return w;
}

}  // namespace

size_t neighbors_workspace_bytes(int64_t n) { return ws_layout(n).total; }

int launch_bbox_partial(const float* pos, int64_t n, float* partial, hipStream_t s) {
  const int nparts = static_cast<int>(std::min<int64_t>(kBboxBlocks, (n + 255) / 256));
  k_bbox_partial<<<nparts, 256, 0, s>>>(pos, n, partial);
  return nparts;
}

e2a_status launch_bbox(const float* pos, int64_t n, float* partial, float* out, hipStream_t s) {
  const int nparts = launch_bbox_partial(pos, n, partial, s);
  k_bbox_final<<<1, 256, 0, s>>>(partial, nparts, out);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

e2a_status exclusive_scan_i32(const int32_t* in, int64_t n, int32_t* out, int64_t* bsum, hipStream_t s) {
  return exclusive_scan<int32_t>(in, n, out, bsum, s);
}

int64_t scan_bsum_count(int64_t n) { return (n + kScanBlock - 1) / kScanBlock + 1; }

e2a_status build_neighbors_impl(const float* pos, int64_t n, const int32_t* batch, const float* box,
                                float cutoff, int64_t* row_ptr, int32_t* col, int64_t cap_edges,
                                int64_t* n_edges, void* ws, size_t ws_bytes, hipStream_t s) {
  const WsLayout L = ws_layout(n);
  if (ws_bytes < L.total) return fail(E2A_ERR_INVALID_ARG, "workspace_bytes %zu < required %zu", ws_bytes, L.total);
  char* base = static_cast<char*>(ws);
  int32_t* cell_of = reinterpret_cast<int32_t*>(base + L.cell_of);
  int32_t* cell_cnt = reinterpret_cast<int32_t*>(base + L.cell_cnt);
  int32_t* cursor = reinterpret_cast<int32_t*>(base + L.cursor);
  int32_t* cell_atoms = reinterpret_cast<int32_t*>(base + L.cell_atoms);
  float4* pos_cell = reinterpret_cast<float4*>(base + L.pos_cell);
  int32_t* row_cnt = reinterpret_cast<int32_t*>(base + L.row_cnt);
  int64_t* bsum = reinterpret_cast<int64_t*>(base + L.bsum);
  float* bbox = reinterpret_cast<float*>(base + L.small);
  float* bbox_part = reinterpret_cast<float*>(base + L.bbox_part);
  int64_t* rb = reinterpret_cast<int64_t*>(base + L.small + 128);

  if (n == 0) {
    E2A_HIP_CHECK(hipMemsetAsync(row_ptr, 0, sizeof(int64_t), s));
    *n_edges = 0;
    return E2A_OK;
  }

  // 1. bounding box and coordinate check, read back with the edge count, so
  // the call waits on the device once.  Until then every kernel is safe on
  // any coordinates: cell indices are clamped into the grid, a non-finite
  // coordinate fails the pair test, and an open grid is sized on the device.
  {
    const e2a_status st = launch_bbox(pos, n, bbox_part, bbox, s);
    if (st != E2A_OK) return st;
  }
  float hb[8] = {};
  auto check_coords = [&]() -> e2a_status {
    if (hb[6] != 0.0f) return fail(E2A_ERR_INVALID_ARG, "positions contain a non-finite value");
    if (box)
      for (int d = 0; d < 3; ++d)
        if (hb[d] < 0.0f || hb[3 + d] >= box[d])
          return fail(E2A_ERR_INVALID_ARG, "periodic coordinate on axis %d outside [0, %g): range [%g, %g]", d,
                      (double)box[d], (double)hb[d], (double)hb[3 + d]);
    return E2A_OK;
  };
  GridArg ga{};
  int64_t ncell = 1;
  int64_t* ncell_dev = nullptr;   // open boundaries: the grid's cell count, on the device
  if (!box) {
    // sized on the device: the host clears and copies the cell counts over
    // the workspace's cell capacity (zeros past the grid), and a one-block
    // scan reads the grid's cell count from the device
    static_assert(32 + sizeof(Grid) <= 104, "grid and cell count overlap in the small region");
    Grid* gdev = reinterpret_cast<Grid*>(base + L.small + 32);
    ncell_dev = reinterpret_cast<int64_t*>(base + L.small + 104);
    k_grid_open<<<1, 1, 0, s>>>(bbox, cutoff, L.cap_cells, gdev, ncell_dev);
    E2A_LAUNCH_CHECK();
    ga.dev = gdev;
    ncell = L.cap_cells;
  } else {
    // periodic: sized on the host from the box sides
    Grid& g = ga.g;
    g.periodic = 1;
    g.rc2 = cutoff * cutoff;
    const float side_min = cutoff * 1.001f;
    for (int d = 0; d < 3; ++d) {
      g.n[d] = std::max(1, static_cast<int>(floorf(box[d] / side_min)));
      g.origin[d] = 0.0f;
      g.box[d] = box[d];
      g.half[d] = 0.5f * box[d];
    }
    // keep the cell count within the workspace by coarsening the largest axis
    for (;;) {
      ncell = (int64_t)g.n[0] * g.n[1] * g.n[2];
      if (ncell <= L.cap_cells) break;
      int d = 0;
      if (g.n[1] > g.n[d]) d = 1;
      if (g.n[2] > g.n[d]) d = 2;
      g.n[d] = std::max(1, g.n[d] / 2);
    }
    for (int d = 0; d < 3; ++d) g.inv_side[d] = 1.0f / (box[d] / g.n[d]);
  }

  const int tpb = 256;
  const int64_t nblk = (n + tpb - 1) / tpb;
  // 2. counting sort into cells: counts in `cursor`, scanned into the cell
  // starts (cell_cnt), the scan leaving `cursor` zero for the scatter's
  // per-cell counters
  E2A_HIP_CHECK(hipMemsetAsync(cursor, 0, sizeof(int32_t) * ncell, s));
  k_bin<<<nblk, tpb, 0, s>>>(pos, n, ga, cell_of, cursor);
  E2A_LAUNCH_CHECK();
  {
    e2a_status st = exclusive_scan<int32_t>(cursor, ncell, cell_cnt, bsum, s, ncell_dev, cursor);
    if (st != E2A_OK) return st;
  }
  k_scatter<<<nblk, tpb, 0, s>>>(n, pos, batch, cell_of, cell_cnt, cursor, cell_atoms, pos_cell);
  E2A_LAUNCH_CHECK();

  // 3-4. count, scan, read back
  const int64_t nwblk = (n + 3) / 4;   // wave-per-atom kernels: 4 atoms per block
  k_count<<<nwblk, 256, 0, s>>>(pos, n, batch, ga, cell_cnt, cell_atoms, pos_cell, bbox, row_cnt);
  E2A_LAUNCH_CHECK();
  {
    e2a_status st = exclusive_scan<int64_t>(row_cnt, n, row_ptr, bsum, s);
    if (st != E2A_OK) return st;
  }
  k_readback<<<1, 1024, 0, s>>>(row_ptr, n, row_cnt, rb);
  E2A_LAUNCH_CHECK();
  // one copy of the small region: the bounding box at its start, the edge
  // count and longest row 128 bytes in
  static_assert(7 * sizeof(float) <= 128, "bounding box and read-back slots overlap");
  unsigned char small[128 + 2 * sizeof(int64_t)];
  E2A_HIP_CHECK(hipMemcpyAsync(small, bbox, sizeof(small), hipMemcpyDeviceToHost, s));
  E2A_HIP_CHECK(hipStreamSynchronize(s));
  int64_t hr[2];
  std::memcpy(hr, small + 128, sizeof(hr));
  std::memcpy(hb, small, 7 * sizeof(float));
  {
    const e2a_status st = check_coords();
    if (st != E2A_OK) return st;
  }
  *n_edges = hr[0];
  if (hr[1] > kMaxRow)
    return fail(E2A_ERR_UNSUPPORTED, "an atom has %lld neighbours; rows longer than %d are not supported",
                (long long)hr[1], kMaxRow);
  if (hr[0] > cap_edges)
    return fail(E2A_ERR_CAPACITY, "need %lld edges, col_capacity is %lld", (long long)hr[0], (long long)cap_edges);

  // 5. fill and sort rows
  if (hr[1] <= kRowFast)
    k_fill_fast<<<nwblk, 256, 0, s>>>(pos, n, batch, ga, cell_cnt, cell_atoms, pos_cell, row_ptr, col);
  else
    k_fill<<<n, 64, 0, s>>>(pos, n, batch, ga, cell_cnt, cell_atoms, pos_cell, row_ptr, col);
  E2A_LAUNCH_CHECK();
  return E2A_OK;
}

}  // namespace e2a

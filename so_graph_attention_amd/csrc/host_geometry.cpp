// Host-only build of the per-edge geometry routines, so that the Wigner-D
// recursion, the edge rotation and the radial basis can be checked on a CPU.
#include "e2a_geometry.hpp"

namespace {

// Blocks l .. L of one tangent, row by row, from its blocks below l.
template <int l>
void tangent_blocks(int L, const float* D, float* dD) {
  for (int m = -l; m <= l; ++m) e2a::wigner_tangent_row<l>(m, D, dD, dD + e2a::wig_off(l) + (m + l) * (2 * l + 1));
  if constexpr (l < 4) {
    if (l < L) tangent_blocks<l + 1>(L, D, dD);
  }
}

}  // namespace

extern "C" {

// Unit vectors and lengths of edge vectors r [n][3] (zero-length edges take z).
void e2a_host_edge_unit(const float* r, int n, float* u_out, float* len_out) {
  for (int e = 0; e < n; ++e) len_out[e] = e2a::edge_unit(r + 3 * e, u_out + 3 * e);
}

void e2a_host_edge_rotation(const float* rhat, int n, float* R_out) {
  for (int e = 0; e < n; ++e) {
    float R[3][3];
    e2a::edge_rotation(rhat + 3 * e, R);
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b) R_out[9 * e + 3 * a + b] = R[a][b];
  }
}

void e2a_host_wigner(int L, const float* R_in, int n, float* D_out) {
  const int sz = e2a::wig_size(L);
  for (int e = 0; e < n; ++e) {
    float R[3][3];
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b) R[a][b] = R_in[9 * e + 3 * a + b];
    e2a::wigner_blocks_rt(L, R, D_out + (size_t)sz * e);
  }
}

// Same blocks built row by row with ir_row (the form the matrix-core kernel uses).
void e2a_host_wigner_rows(int L, const float* R_in, int n, float* D_out) {
  const int sz = e2a::wig_size(L);
  for (int e = 0; e < n; ++e) {
    float R[3][3];
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b) R[a][b] = R_in[9 * e + 3 * a + b];
    float* D = D_out + (size_t)sz * e;
    D[0] = 1.0f;
    if (L < 1) continue;
    float r1[3][3];
    e2a::wigner_l1(R, &r1[0][0], 3);
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b) D[1 + 3 * a + b] = r1[a][b];
    for (int l = 2; l <= L; ++l) {
      const float* Dp = D + e2a::wig_off(l - 1);
      float* Dl = D + e2a::wig_off(l);
      for (int m = -l; m <= l; ++m) {
        auto rp = [&](int a) { return Dp + (a + l - 1) * (2 * l - 1); };
        float* out = Dl + (m + l) * (2 * l + 1);
        switch (l) {
          case 2: e2a::ir_row<2>(m, r1, rp, out); break;
          case 3: e2a::ir_row<3>(m, r1, rp, out); break;
          default: e2a::ir_row<4>(m, r1, rp, out); break;
        }
      }
    }
  }
}

void e2a_host_radial_basis8(const float* r, int n, float rc, float* out) {
  for (int e = 0; e < n; ++e) e2a::radial_basis8(r[e], rc, out + 8 * e);
}

void e2a_host_radial_basis8_deriv(const float* r, int n, float rc, float* out) {
  for (int e = 0; e < n; ++e) e2a::radial_basis8_deriv(r[e], rc, out + 8 * e);
}

// The three tangents of the Wigner blocks for the frame turned about x, y, z
// (the position gradient's form): dD_out[(e * 3 + a) * wig_size(L) + ...].
void e2a_host_wigner_tangents(int L, const float* R_in, int n, float* dD_out) {
  const int sz = e2a::wig_size(L);
  float D[e2a::wig_size(4)];
  for (int e = 0; e < n; ++e) {
    float R[3][3];
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b) R[a][b] = R_in[9 * e + 3 * a + b];
    e2a::wigner_blocks_rt(L, R, D);
    for (int a = 0; a < 3; ++a) {
      float* dD = dD_out + (size_t)(e * 3 + a) * sz;
      dD[0] = 0.0f;
      if (L < 1) continue;
      float dR[3][3];
      e2a::frame_tangent(R, a, dR);
      e2a::wigner_l1(dR, dD + e2a::wig_off(1), 3);
      if (L >= 2) tangent_blocks<2>(L, D, dD);
    }
  }
}

}

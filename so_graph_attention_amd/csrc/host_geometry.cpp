// Host-only build of the per-edge geometry routines, so that the Wigner-D
// recursion, the edge rotation and the radial basis can be checked on a CPU.
#include "e2a_geometry.hpp"

extern "C" {

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

void e2a_host_radial_basis8(const float* r, int n, float rc, float* out) {
  for (int e = 0; e < n; ++e) e2a::radial_basis8(r[e], rc, out + 8 * e);
}

}

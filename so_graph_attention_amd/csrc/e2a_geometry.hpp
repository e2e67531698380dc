// Per-edge geometry of the on-the-fly equivariant attention layer
// (arXiv 2601.16622, English technical summary section 2.1, "Equivariant
// Axis-Aligned Sparsification"): the rotation that aligns an edge with z, the
// real Wigner-D blocks of that rotation, and the radial basis.
//
// Everything here is plain fp32 arithmetic usable from device code and from a
// host-only build, so the recursion can be checked on a CPU.
#pragma once

#include <math.h>

#if defined(__HIPCC__)
#define E2A_HD __host__ __device__ inline
#else
#define E2A_HD inline
#endif

namespace e2a {

// Offset of block l inside a packed set of Wigner-D blocks D^0, D^1, ...:
// sum_{k<l} (2k+1)^2 = l (4 l^2 - 1) / 3.
E2A_HD constexpr int wig_off(int l) { return l * (4 * l * l - 1) / 3; }
E2A_HD constexpr int wig_size(int L) { return wig_off(L + 1); }

// Length of the edge vector r3 and its unit vector u.  An edge of zero length
// has no direction; it takes u = z (the identity frame), so that every value
// derived from it stays finite.  The neighbour build never pairs two atoms at
// one point, so such an edge only occurs in a caller-built graph.
E2A_HD float edge_unit(const float r3[3], float u[3]) {
  const float rr = sqrtf(r3[0] * r3[0] + r3[1] * r3[1] + r3[2] * r3[2]);
  if (rr > 0.0f) {
    u[0] = r3[0] / rr;
    u[1] = r3[1] / rr;
    u[2] = r3[2] / rr;
  } else {
    u[0] = 0.0f;
    u[1] = 0.0f;
    u[2] = 1.0f;
  }
  return rr;
}

// Rotation R with R r_hat = z: R = R_y(-theta) R_z(-phi) for r_hat =
// (sin t cos p, sin t sin p, cos t).  Rows: (ct cp, ct sp, -st), (-sp, cp, 0),
// (st cp, st sp, ct).  At the poles phi = 0.
E2A_HD void edge_rotation(const float u[3], float R[3][3]) {
  const float st = sqrtf(u[0] * u[0] + u[1] * u[1]);
  const float ct = u[2];
  float cp = 1.0f, sp = 0.0f;
  if (st > 0.0f) {
    cp = u[0] / st;
    sp = u[1] / st;
  }
  R[0][0] = ct * cp; R[0][1] = ct * sp; R[0][2] = -st;
  R[1][0] = -sp;     R[1][1] = cp;      R[1][2] = 0.0f;
  R[2][0] = st * cp; R[2][1] = st * sp; R[2][2] = ct;
}

// One entry D^l[m][n] (l >= 2) of the Ivanic-Ruedenberg recursion (J. Phys.
// Chem. 100, 6342 (1996); erratum 102, 9099 (1998)), which builds D^l from
// D^{l-1} and D^1.  r1(i, j) returns D^1[i][j] and rp(a, b) returns
// D^{l-1}[a][b], both with signed indices.
template <typename R1, typename RP>
E2A_HD float ir_entry(int l, int m, int n, const R1& r1, const RP& rp) {
  // P(i, a, b): a in [-(l-1), l-1], b in [-l, l]
  auto P = [&](int i, int a, int b) {
    if (b == l) return r1(i, 1) * rp(a, l - 1) - r1(i, -1) * rp(a, 1 - l);
    if (b == -l) return r1(i, 1) * rp(a, 1 - l) + r1(i, -1) * rp(a, l - 1);
    return r1(i, 0) * rp(a, b);
  };
  const int am = m < 0 ? -m : m;
  const int an = n < 0 ? -n : n;
  const float d = (m == 0) ? 1.0f : 0.0f;
  const float denom = (an == l) ? float((2 * l) * (2 * l - 1)) : float((l + n) * (l - n));
  const float u = sqrtf(float((l + m) * (l - m)) / denom);
  const float v = 0.5f * sqrtf((1.0f + d) * float((l + am - 1) * (l + am)) / denom) * (1.0f - 2.0f * d);
  const float w = -0.5f * sqrtf(float((l - am - 1) * (l - am)) / denom) * (1.0f - d);
  float acc = 0.0f;
  if (am < l) acc += u * P(0, m, n);
  if (m == 0) {
    acc += v * (P(1, 1, n) + P(-1, -1, n));
  } else if (m > 0) {
    const float t1 = P(1, m - 1, n) * (m == 1 ? 1.41421356237f : 1.0f);
    const float t2 = (m == 1) ? 0.0f : P(-1, 1 - m, n);
    acc += v * (t1 - t2);
    if (am < l - 1) acc += w * (P(1, m + 1, n) + P(-1, -m - 1, n));
  } else {
    const float t1 = (m == -1) ? 0.0f : P(1, m + 1, n);
    const float t2 = P(-1, -m - 1, n) * (m == -1 ? 1.41421356237f : 1.0f);
    acc += v * (t1 + t2);
    if (am < l - 1) acc += w * (P(1, m - 1, n) - P(-1, -m + 1, n));
  }
  return acc;
}

// Row m of D^l (compile-time l >= 2) by the same recursion as ir_entry,
// grouped per row: the U, V and W terms use at most five (i, a) pairs whose
// coefficients depend on m alone, and every column n carries the factor
// 1/sqrt(denominator(n)).  r1[i+1][j+1] = D^1[i][j]; rp(a) points at row a of
// D^{l-1} (column b at index b + l - 1).  Writes out[n + l], n = -l..l.
template <int l, typename RP>
E2A_HD void ir_row(int m, const float r1[3][3], const RP& rp, float* out) {
  const int am = m < 0 ? -m : m;
  const float d = (m == 0) ? 1.0f : 0.0f;
  const float cu = (am < l) ? sqrtf(float((l + m) * (l - m))) : 0.0f;
  const float cv = 0.5f * sqrtf((1.0f + d) * float((l + am - 1) * (l + am))) * (1.0f - 2.0f * d);
  const float cw = (am < l - 1) ? -0.5f * sqrtf(float((l - am - 1) * (l - am))) : 0.0f;
  const float s2 = 1.41421356237f;
  int ii[5], aa[5];
  float cc[5];
  ii[0] = 0; aa[0] = (am < l) ? m : 0; cc[0] = cu;
  if (m == 0) {
    ii[1] = 1;  aa[1] = 1;  cc[1] = cv;
    ii[2] = -1; aa[2] = -1; cc[2] = cv;
    ii[3] = 1;  aa[3] = 0;  cc[3] = 0.0f;
    ii[4] = -1; aa[4] = 0;  cc[4] = 0.0f;
  } else if (m > 0) {
    ii[1] = 1;  aa[1] = m - 1;                   cc[1] = cv * (m == 1 ? s2 : 1.0f);
    ii[2] = -1; aa[2] = (m == 1) ? 0 : 1 - m;    cc[2] = (m == 1) ? 0.0f : -cv;
    ii[3] = 1;  aa[3] = (am < l - 1) ? m + 1 : 0;  cc[3] = cw;
    ii[4] = -1; aa[4] = (am < l - 1) ? -m - 1 : 0; cc[4] = cw;
  } else {
    ii[1] = 1;  aa[1] = (m == -1) ? 0 : m + 1;   cc[1] = (m == -1) ? 0.0f : cv;
    ii[2] = -1; aa[2] = -m - 1;                  cc[2] = cv * (m == -1 ? s2 : 1.0f);
    ii[3] = 1;  aa[3] = (am < l - 1) ? m - 1 : 0;  cc[3] = cw;
    ii[4] = -1; aa[4] = (am < l - 1) ? -m + 1 : 0; cc[4] = -cw;
  }
  float g0[5], gp[5], gm[5];   // r1(i_k, 0), r1(i_k, +1), r1(i_k, -1)
  float row[5][2 * l - 1];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int i = ii[k] + 1;
    g0[k] = i == 0 ? r1[0][1] : (i == 1 ? r1[1][1] : r1[2][1]);
    gp[k] = i == 0 ? r1[0][2] : (i == 1 ? r1[1][2] : r1[2][2]);
    gm[k] = i == 0 ? r1[0][0] : (i == 1 ? r1[1][0] : r1[2][0]);
    const float* rk = rp(aa[k]);
#pragma unroll
    for (int b = 0; b < 2 * l - 1; ++b) row[k][b] = rk[b];
  }
#pragma unroll
  for (int n = -l; n <= l; ++n) {
    const int an = n < 0 ? -n : n;
    const float inv = 1.0f / sqrtf(an == l ? float((2 * l) * (2 * l - 1)) : float((l + n) * (l - n)));
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      float pk;
      if (n == l) pk = gp[k] * row[k][2 * l - 2] - gm[k] * row[k][0];
      else if (n == -l) pk = gp[k] * row[k][0] + gm[k] * row[k][2 * l - 2];
      else pk = g0[k] * row[k][n + l - 1];
      acc += cc[k] * pk;
    }
    out[n + l] = acc * inv;
  }
}

// D^1 in the harmonic order (y, z, x) <- index m + 1, written with row stride ld.
E2A_HD void wigner_l1(const float R[3][3], float* D1, int ld) {
  const int p[3] = {1, 2, 0};
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 3; ++b) D1[a * ld + b] = R[p[a]][p[b]];
}

// Real Wigner-D blocks D^0..D^L of rotation R, defined by Y^l(R v) = D^l Y^l(v)
// for real harmonics without the Condon-Shortley phase stored at m = -l..l.
// D^1 is R in (y, z, x) order; higher blocks follow ir_entry.  Block l sits at
// D + wig_off(l), row-major [(m + l)(2l + 1) + (n + l)].
template <int L>
E2A_HD void wigner_blocks(const float R[3][3], float* D) {
  D[0] = 1.0f;
  if (L < 1) return;
  float* D1 = D + wig_off(1);
  wigner_l1(R, D1, 3);
  auto r1 = [&](int i, int j) { return D1[(i + 1) * 3 + (j + 1)]; };
#pragma unroll
  for (int l = 2; l <= L; ++l) {
    const float* Dp = D + wig_off(l - 1);
    float* Dl = D + wig_off(l);
    const int wp = 2 * l - 1;
    auto rp = [&](int a, int b) { return Dp[(a + l - 1) * wp + (b + l - 1)]; };
#pragma unroll
    for (int m = -l; m <= l; ++m)
#pragma unroll
      for (int n = -l; n <= l; ++n) Dl[(m + l) * (2 * l + 1) + (n + l)] = ir_entry(l, m, n, r1, rp);
  }
}

// The frame's change when r_hat turns about axis a and the frame turns with
// it: R -> R (1 - t [e_a]x), so dR/dt = -R [e_a]x with ([e_a]x)[k][c] = eps(k, a, c).
E2A_HD void frame_tangent(const float R[3][3], int a, float dR[3][3]) {
  const int a1 = (a + 1) % 3, a2 = (a + 2) % 3;
  for (int r = 0; r < 3; ++r) {
    // (R [e_a]x)[r][c] = sum_k R[r][k] eps(k, a, c): +R[r][a2] at c = a1, -R[r][a1] at c = a2
    dR[r][a] = 0.0f;
    dR[r][a1] = -R[r][a2];
    dR[r][a2] = R[r][a1];
  }
}

// Row m of block l >= 2 of a tangent of the Wigner blocks.  The recursion is
// bilinear in D^1 and D^{l-1}, so the tangent row is ir(dD^1, D^{l-1}) +
// ir(D^1, dD^{l-1}); D and dD hold blocks 0 .. l-1 at wig_off.  Writes
// out[n + l], n = -l..l.
template <int l>
E2A_HD void wigner_tangent_row(int m, const float* D, const float* dD, float* out) {
  constexpr int w = 2 * l + 1, wp = 2 * l - 1;
  float r1[3][3], d1[3][3];
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 3; ++b) {
      r1[a][b] = D[wig_off(1) + a * 3 + b];
      d1[a][b] = dD[wig_off(1) + a * 3 + b];
    }
  const float* pv = D + wig_off(l - 1);
  const float* pd = dD + wig_off(l - 1);
  auto rpv = [&](int a) { return pv + (a + l - 1) * wp; };
  auto rpd = [&](int a) { return pd + (a + l - 1) * wp; };
  float o1[w], o2[w];
  ir_row<l>(m, d1, rpv, o1);
  ir_row<l>(m, r1, rpd, o2);
  for (int n = 0; n < w; ++n) out[n] = o1[n] + o2[n];
}

// Runtime-L front end of wigner_blocks.
E2A_HD void wigner_blocks_rt(int L, const float R[3][3], float* D) {
  switch (L) {
    case 0: wigner_blocks<0>(R, D); break;
    case 1: wigner_blocks<1>(R, D); break;
    case 2: wigner_blocks<2>(R, D); break;
    case 3: wigner_blocks<3>(R, D); break;
    default: wigner_blocks<4>(R, D); break;
  }
}

// Radial basis: 8 Gaussians with centres mu_k = k rc/7, width = spacing, times
// the cosine envelope (cos(pi r / rc) + 1) / 2.
E2A_HD void radial_basis8(float r, float rc, float e[8]) {
  const float delta = rc / 7.0f;
  const float gamma = 0.5f / (delta * delta);
  const float env = 0.5f * (cosf(3.14159265358979f * r / rc) + 1.0f);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float t = r - float(k) * delta;
    e[k] = expf(-gamma * t * t) * env;
  }
}

// d e_k / d r of radial_basis8: the Gaussian's slope times the envelope plus
// the Gaussian times the envelope's slope, -(pi / 2 rc) sin(pi r / rc).
E2A_HD void radial_basis8_deriv(float r, float rc, float de[8]) {
  const float delta = rc / 7.0f;
  const float gamma = 0.5f / (delta * delta);
  const float a = 3.14159265358979f / rc;
  const float env = 0.5f * (cosf(a * r) + 1.0f);
  const float denv = -0.5f * a * sinf(a * r);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float t = r - float(k) * delta;
    const float g = expf(-gamma * t * t);
    de[k] = g * (-2.0f * gamma * t * env + denv);
  }
}

}  // namespace e2a

// Compile-time coupling tables for the channelwise tensor-product convolution.
//
// Paths (FlashCart paper, section 2 "Irreducible Cartesian tensors"): a path
// (l1, l2) -> l3 is admissible when |l1-l2| <= l3 <= l1+l2 and l1+l2+l3 is even
// (natural parity).  Node irreps are l1 = 0..L1, edge harmonics l2 = 0..L2,
// outputs l3 = 0..L3; paths are ordered lexicographically by (l1, l2, l3).
//
// Coefficients: for an admissible path the equivariant bilinear maps form a
// one-dimensional space (same section), so any non-zero equivariant coupling
// fixes them up to a scale.  This file builds the real Gaunt coefficients
//   integral of S_{l1 m1} S_{l2 m2} S_{l3 m3} over the sphere
// of the real harmonics S (z polar axis, m<0 <-> sin(|m| phi), m>0 <-> cos(m phi),
// no Condon-Shortley phase) from the closed form of the complex Gaunt integral
// as a product of two Wigner 3j symbols, each evaluated with the Racah sum, and
// the unitary map from complex to real harmonics.  Each path's tensor is then
// scaled to unit Frobenius norm (sign fixed by the integral).
//
// Everything is constexpr: the kernels unroll over the non-zero pattern with the
// coefficients as literals, and the host exposes the same tables for inspection.
#pragma once

#include <cstdint>

namespace tpc {

constexpr int kMaxL = 3;
constexpr int kMaxPaths = 32;

constexpr double cx_sqrt(double x) {
  if (x <= 0.0) return 0.0;
  double g = x > 1.0 ? x : 1.0;
  for (int i = 0; i < 200; ++i) {
    double n = 0.5 * (g + x / g);
    if (n == g) break;
    g = n;
  }
  // one correction step toward the correctly rounded root
  double r = g;
  double e1 = r * r - x;
  double up = r + r * 2.220446049250313e-16, dn = r - r * 2.220446049250313e-16;
  double e_up = up * up - x, e_dn = dn * dn - x;
  auto ab = [](double v) { return v < 0 ? -v : v; };
  if (ab(e_up) < ab(e1)) r = up;
  if (ab(e_dn) < ab(r * r - x)) r = dn;
  return r;
}

constexpr double cx_fact(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; ++i) f *= double(i);
  return f;
}

// Wigner 3j symbol (j1 j2 j3; m1 m2 m3) by the Racah formula.
constexpr double wigner3j(int j1, int j2, int j3, int m1, int m2, int m3) {
  if (m1 + m2 + m3 != 0) return 0.0;
  if (j3 < (j1 > j2 ? j1 - j2 : j2 - j1) || j3 > j1 + j2) return 0.0;
  if (m1 < -j1 || m1 > j1 || m2 < -j2 || m2 > j2 || m3 < -j3 || m3 > j3) return 0.0;
  double tri = cx_fact(j1 + j2 - j3) * cx_fact(j1 - j2 + j3) * cx_fact(-j1 + j2 + j3) /
               cx_fact(j1 + j2 + j3 + 1);
  double pre = cx_sqrt(tri * cx_fact(j1 + m1) * cx_fact(j1 - m1) * cx_fact(j2 + m2) *
                       cx_fact(j2 - m2) * cx_fact(j3 + m3) * cx_fact(j3 - m3));
  double sum = 0.0;
  for (int k = 0; k <= j1 + j2 + j3; ++k) {
    int a = j3 - j2 + k + m1, b = j3 - j1 + k - m2, c = j1 + j2 - j3 - k, d = j1 - k - m1,
        e = j2 - k + m2;
    if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
    double t = 1.0 / (cx_fact(k) * cx_fact(a) * cx_fact(b) * cx_fact(c) * cx_fact(d) * cx_fact(e));
    sum += (k % 2 ? -t : t);
  }
  int ph = j1 - j2 - m3;
  double sgn = ((ph % 2) + 2) % 2 ? -1.0 : 1.0;
  return sgn * pre * sum;
}

struct cplx {
  double re, im;
};
constexpr cplx cmul(cplx a, cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }

// Coefficient of the complex harmonic Y_l^mu in the real harmonic S_{l m}.
constexpr cplx u_real(int m, int mu) {
  const double r2 = 0.70710678118654752440;  // 1/sqrt(2)
  int a = m < 0 ? -m : m;
  double sa = (a % 2) ? -1.0 : 1.0;           // (-1)^a
  if (m == 0) return {mu == 0 ? 1.0 : 0.0, 0.0};
  if (m > 0) {
    if (mu == m) return {sa * r2, 0.0};
    if (mu == -m) return {r2, 0.0};
    return {0.0, 0.0};
  }
  if (mu == -a) return {0.0, r2};
  if (mu == a) return {0.0, -sa * r2};
  return {0.0, 0.0};
}

// Real Gaunt integral (up to a common positive factor per path).
constexpr double real_gaunt(int l1, int l2, int l3, int m1, int m2, int m3) {
  double w000 = wigner3j(l1, l2, l3, 0, 0, 0);
  double re = 0.0;
  for (int a = -l1; a <= l1; ++a)
    for (int b = -l2; b <= l2; ++b) {
      int c = -a - b;
      if (c < -l3 || c > l3) continue;
      cplx u = cmul(cmul(u_real(m1, a), u_real(m2, b)), u_real(m3, c));
      if (u.re == 0.0 && u.im == 0.0) continue;
      double g = w000 * wigner3j(l1, l2, l3, a, b, c);
      re += u.re * g;
    }
  return re;
}

struct Path {
  int l1, l2, l3;
  int q;         // rank among the paths with the same l3
  int nq;        // number of paths with this l3
  int out_base;  // first output row of the l3 block
};

struct Table {
  int L1, L2, L3;
  bool summed;  // paths of one output rank share one (m3, channel) block
  int np;
  int din, dsh, dout;
  int nnz;
  int nm;    // non-zero (p, m1, m3) entries of the per-edge coupling matrices
  int nms;   // row stride of the per-edge coupling-matrix buffer (nm rounded up to 4)
  Path path[kMaxPaths];
  double cg[kMaxPaths][7][7][7];
  // index of entry (p, m1, m3) in an edge's coupling-matrix row, -1 if zero;
  // entries are ordered path-major, then m3, then m1
  int midx[kMaxPaths][7][7];

  constexpr int out_row(int p, int m3) const {
    return path[p].out_base + m3 * path[p].nq + path[p].q;
  }
  // does any C^p[m1][m2][m3] differ from zero for this (m1, m2)
  constexpr bool m12nz(int p, int m1, int m2) const {
    for (int c = 0; c < 7; ++c)
      if (cg[p][m1][m2][c] != 0.0) return true;
    return false;
  }
};

constexpr bool admissible(int l1, int l2, int l3) {
  int d = l1 > l2 ? l1 - l2 : l2 - l1;
  return d <= l3 && l3 <= l1 + l2 && ((l1 + l2 + l3) % 2 == 0);
}

// Output rows: l3 blocks ascending; inside a block (m3, q, channel) with q
// the rank of the path among those with that l3, or, summed (FlashCart
// section 3, "Generating Cartesian tensor products": paths with the same
// output rank may be summed), one (m3, channel) block per l3 that occurs.
constexpr Table make_table(int L1, int L2, int L3, bool summed = false) {
  Table t{};
  t.L1 = L1;
  t.L2 = L2;
  t.L3 = L3;
  t.summed = summed;
  t.din = (L1 + 1) * (L1 + 1);
  t.dsh = (L2 + 1) * (L2 + 1);
  int np = 0;
  for (int l1 = 0; l1 <= L1; ++l1)
    for (int l2 = 0; l2 <= L2; ++l2)
      for (int l3 = 0; l3 <= L3; ++l3)
        if (admissible(l1, l2, l3) && np < kMaxPaths) {
          t.path[np] = Path{l1, l2, l3, 0, 0, 0};
          ++np;
        }
  t.np = np;
  int base = 0;
  for (int l3 = 0; l3 <= L3; ++l3) {
    int nq = 0;
    for (int p = 0; p < np; ++p)
      if (t.path[p].l3 == l3) ++nq;
    int q = 0;
    for (int p = 0; p < np; ++p)
      if (t.path[p].l3 == l3) {
        t.path[p].q = summed ? 0 : q++;
        t.path[p].nq = summed ? 1 : nq;
        t.path[p].out_base = base;
      }
    base += (summed ? (nq > 0 ? 1 : 0) : nq) * (2 * l3 + 1);
  }
  t.dout = base;
  int nnz = 0;
  for (int p = 0; p < np; ++p) {
    const int l1 = t.path[p].l1, l2 = t.path[p].l2, l3 = t.path[p].l3;
    double nrm = 0.0;
    for (int a = 0; a < 7; ++a)
      for (int b = 0; b < 7; ++b)
        for (int c = 0; c < 7; ++c) t.cg[p][a][b][c] = 0.0;
    for (int a = 0; a <= 2 * l1; ++a)
      for (int b = 0; b <= 2 * l2; ++b)
        for (int c = 0; c <= 2 * l3; ++c) {
          double g = real_gaunt(l1, l2, l3, a - l1, b - l2, c - l3);
          t.cg[p][a][b][c] = g;
          nrm += g * g;
        }
    nrm = cx_sqrt(nrm);
    for (int a = 0; a <= 2 * l1; ++a)
      for (int b = 0; b <= 2 * l2; ++b)
        for (int c = 0; c <= 2 * l3; ++c) {
          double v = t.cg[p][a][b][c] / nrm;
          double av = v < 0 ? -v : v;
          t.cg[p][a][b][c] = av < 1e-12 ? 0.0 : v;
          if (av >= 1e-12) ++nnz;
        }
  }
  t.nnz = nnz;
  int nm = 0;
  for (int p = 0; p < np; ++p)
    for (int c = 0; c < 7; ++c)
      for (int a = 0; a < 7; ++a) t.midx[p][a][c] = -1;
  for (int p = 0; p < np; ++p)
    for (int c = 0; c <= 2 * t.path[p].l3; ++c)
      for (int a = 0; a <= 2 * t.path[p].l1; ++a) {
        bool any = false;
        for (int b = 0; b <= 2 * t.path[p].l2; ++b)
          if (t.cg[p][a][b][c] != 0.0) any = true;
        if (any) t.midx[p][a][c] = nm++;
      }
  t.nm = nm;
  t.nms = (nm + 3) / 4 * 4;
  return t;
}

template <int L1, int L2, int L3, bool SUM = false>
inline constexpr Table kTable = make_table(L1, L2, L3, SUM);

// Split of the paths over NG waves of one receiver row: by whole l1 classes
// when that balances well enough, else greedy by descending per-wave work
// (coupling-matrix terms plus per-channel FMAs).
struct Groups {
  int group[kMaxPaths];
};

constexpr Groups make_groups(const Table& t, int ng, int cpl) {
  Groups g{};
  int cost[kMaxPaths] = {};
  bool done[kMaxPaths] = {};
  int load[8] = {};
  for (int p = 0; p < t.np; ++p) {
    int m13 = 0, nnz = 0;
    for (int a = 0; a < 7; ++a)
      for (int c = 0; c < 7; ++c) {
        if (t.midx[p][a][c] >= 0) ++m13;
        for (int b = 0; b < 7; ++b)
          if (t.cg[p][a][b][c] != 0.0) ++nnz;
      }
    cost[p] = cpl * (m13 + 2 * t.path[p].l1 + 1) + nnz;
  }
  // With separate outputs, whole l1 classes go to one wave when some split of
  // the classes keeps the busiest wave within 5/4 of an even share: each
  // wave then loads only its classes' rows of the sender features.
  if (!t.summed && ng > 1) {
    int ccost[4] = {};
    for (int p = 0; p < t.np; ++p) ccost[t.path[p].l1] += cost[p];
    int total = 0;
    for (int l = 0; l <= t.L1; ++l) total += ccost[l];
    int best_max = -1, best_code = -1;
    int n_codes = 1;
    for (int l = 0; l <= t.L1; ++l) n_codes *= ng;
    for (int code = 0; code < n_codes; ++code) {
      int ld[8] = {}, x = code;
      for (int l = 0; l <= t.L1; ++l) {
        ld[x % ng] += ccost[l];
        x /= ng;
      }
      int mx = 0, empty = 0;
      for (int k = 0; k < ng; ++k) {
        if (ld[k] > mx) mx = ld[k];
        if (ld[k] == 0) empty = 1;
      }
      if (!empty && (best_max < 0 || mx < best_max)) {
        best_max = mx;
        best_code = code;
      }
    }
    if (best_code >= 0 && 4 * best_max * ng <= 5 * total) {
      for (int p = 0; p < t.np; ++p) {
        int x = best_code;
        for (int l = 0; l < t.path[p].l1; ++l) x /= ng;
        g.group[p] = x % ng;
      }
      return g;
    }
  }
  // with summed outputs a wave owns whole output blocks: the paths of one l3
  // move together, at the cost of the class
  if (t.summed) {
    int cls[kMaxPaths] = {};
    for (int p = 0; p < t.np; ++p)
      for (int q = 0; q < t.np; ++q)
        if (t.path[q].l3 == t.path[p].l3) cls[p] += cost[q];
    for (int p = 0; p < t.np; ++p) cost[p] = cls[p];
  }
  for (int it = 0; it < t.np; ++it) {
    int best = -1;
    for (int p = 0; p < t.np; ++p)
      if (!done[p] && (best < 0 || cost[p] > cost[best])) best = p;
    if (best < 0) break;  // summed: whole classes already placed
    int gl = 0;
    for (int k = 1; k < ng; ++k)
      if (load[k] < load[gl]) gl = k;
    if (t.summed) {
      for (int q = 0; q < t.np; ++q)
        if (t.path[q].l3 == t.path[best].l3) {
          g.group[q] = gl;
          done[q] = true;
        }
    } else {
      g.group[best] = gl;
      done[best] = true;
    }
    load[gl] += cost[best];
  }
  return g;
}

template <int L1, int L2, int L3, bool SUM, int NG, int CPL>
inline constexpr Groups kGroups = make_groups(kTable<L1, L2, L3, SUM>, NG, CPL);

// Does wave group g use the sender-feature rows of rank l1?
constexpr bool group_uses_l1(const Table& t, const Groups& gr, int g, int l1) {
  for (int p = 0; p < t.np; ++p)
    if (gr.group[p] == g && t.path[p].l1 == l1) return true;
  return false;
}

// Non-zero test for the pattern (m1, m3) of path p: is any C[m1][m2][m3] != 0.
constexpr bool m13_nonzero(const Table& t, int p, int a, int c) {
  for (int b = 0; b <= 2 * t.path[p].l2; ++b)
    if (t.cg[p][a][b][c] != 0.0) return true;
  return false;
}

// Path groups of the fused backward: NG waves of one receiver row and one
// channel slice own whole l1 classes, so the sender-gradient rows (dh) that
// different waves accumulate never overlap.  Among the ways to place the
// classes on NG non-empty waves, the one with the smallest busiest wave is
// taken (cost per edge: the per-channel multiply-adds of dR, dY and dh plus
// the coupling matrix of the edge).  kofs[p] is the offset of path p's
// entries in its wave's per-row coupling array K[(m1, m2)] (the non-zero
// (m1, m2) pairs of the path, m1-major); nk[g] is that array's length.
struct BwdGroups {
  int ng;
  int group[kMaxPaths];
  int kofs[kMaxPaths];
  int nk[8];
  bool ok;  // every group non-empty
};

constexpr int m12_count(const Table& t, int p) {
  int n = 0;
  for (int a = 0; a <= 2 * t.path[p].l1; ++a)
    for (int b = 0; b <= 2 * t.path[p].l2; ++b)
      if (t.m12nz(p, a, b)) ++n;
  return n;
}

// index of (m1, m2) among the non-zero pairs of path p (m1-major), -1 if zero
constexpr int m12_index(const Table& t, int p, int m1, int m2) {
  int n = 0;
  for (int a = 0; a <= 2 * t.path[p].l1; ++a)
    for (int b = 0; b <= 2 * t.path[p].l2; ++b)
      if (t.m12nz(p, a, b)) {
        if (a == m1 && b == m2) return n;
        ++n;
      }
  return -1;
}

constexpr int bwd_path_cost(const Table& t, int p) {
  int m13 = 0, nnz = 0;
  for (int a = 0; a < 7; ++a)
    for (int c = 0; c < 7; ++c) {
      if (t.midx[p][a][c] >= 0) ++m13;
      for (int b = 0; b < 7; ++b)
        if (t.cg[p][a][b][c] != 0.0) ++nnz;
    }
  const int n2 = 2 * t.path[p].l2 + 1, n3 = 2 * t.path[p].l3 + 1;
  return m12_count(t, p) + 2 * n2 + n3 + m13 + nnz;
}

constexpr BwdGroups make_bwd_groups(const Table& t, int ng) {
  BwdGroups g{};
  g.ng = ng;
  int ccost[4] = {};
  for (int p = 0; p < t.np; ++p) ccost[t.path[p].l1] += bwd_path_cost(t, p);
  int n_codes = 1;
  for (int l = 0; l <= t.L1; ++l) n_codes *= ng;
  int best_max = -1, best_code = -1;
  for (int code = 0; code < n_codes; ++code) {
    int ld[8] = {}, used[8] = {}, x = code;
    for (int l = 0; l <= t.L1; ++l) {
      ld[x % ng] += ccost[l];
      used[x % ng] = 1;
      x /= ng;
    }
    int mx = 0, empty = 0;
    for (int k = 0; k < ng; ++k) {
      if (ld[k] > mx) mx = ld[k];
      if (!used[k]) empty = 1;
    }
    if (!empty && (best_max < 0 || mx < best_max)) {
      best_max = mx;
      best_code = code;
    }
  }
  g.ok = best_code >= 0;
  if (!g.ok) return g;
  for (int p = 0; p < t.np; ++p) {
    int x = best_code;
    for (int l = 0; l < t.path[p].l1; ++l) x /= ng;
    g.group[p] = x % ng;
  }
  for (int p = 0; p < t.np; ++p) {
    g.kofs[p] = g.nk[g.group[p]];
    g.nk[g.group[p]] += m12_count(t, p);
  }
  return g;
}

template <int L1, int L2, int L3, bool SUM, int NG>
inline constexpr BwdGroups kBwdGroups = make_bwd_groups(kTable<L1, L2, L3, SUM>, NG);

// Does backward group g own the l1 class l (its sender-gradient rows)?
constexpr bool bwd_group_owns_l1(const Table& t, const BwdGroups& gr, int g, int l1) {
  for (int p = 0; p < t.np; ++p)
    if (gr.group[p] == g && t.path[p].l1 == l1) return true;
  return false;
}

// Does backward group g read output row o (of G) for any of its paths?
constexpr bool bwd_group_reads_row(const Table& t, const BwdGroups& gr, int g, int o) {
  for (int p = 0; p < t.np; ++p)
    if (gr.group[p] == g)
      for (int m3 = 0; m3 <= 2 * t.path[p].l3; ++m3)
        if (t.out_row(p, m3) == o) return true;
  return false;
}

}  // namespace tpc

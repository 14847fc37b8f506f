// Host check of the packed input of the device vector phase.  It factors a seeded symmetric
// matrix with the host eigensolver, packs the rotation log (runs, groups, (c, s) pairs), the
// reflector blocks and the wanted positions as a compression does, and applies them the way
// the rotation kernel and the reflector products do (the same grouping, wavefront schedule,
// identity padding and chunking, with every row and LDS index bounds-checked), then compares
// the result with the host's own eigenvectors.  With parts > 1 the groups are cut into pieces as
// a compression cuts them: piece 0 applied to the wanted unit vectors, every later piece to the
// identity, and the pieces' products multiplied together before the reflectors.  The kernel's
// constants come in as -D flags.
//   usage: ritz_pack_check n r power [run_cap] [spread] [parts]
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
extern "C" {
#include "host_eigh.h"
}

static void bail(const char* what, long v) {
  std::printf("FAIL %s %ld\n", what, v);
  std::exit(3);
}

int main(int argc, char** argv) {
  if (argc < 4) return 2;
  const int n = std::atoi(argv[1]), r = std::atoi(argv[2]);
  const double pw = std::atof(argv[3]);
  const int run_cap = argc > 4 ? std::atoi(argv[4]) : KRUNCAP;
  const int spread = argc > 5 ? std::atoi(argv[5]) : KSPREAD;
  const int parts = argc > 6 ? std::atoi(argv[6]) : 1;
  if (parts < 1 || parts > 4) bail("parts", parts);
  const int kB = KB, CH = KCH, kSlot = spread + KRUNCAP + spread + 2 * KCH, kPadLo = 2 * KCH + KB, kPadHi = KB;
  // H = G diag(k^pw) G^T, symmetric positive semi-definite with a graded spectrum
  std::mt19937_64 g(n * 1000003ull + r);
  std::normal_distribution<double> N;
  std::vector<double> G((size_t)n * n), H((size_t)n * n);
  std::vector<double> sc_k(n);
  for (auto& x : G) x = N(g);
  for (int k = 0; k < n; ++k) sc_k[k] = std::pow(k + 1.0, pw);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j <= i; ++j) {
      double s = 0;
      for (int k = 0; k < n; ++k) s += G[(size_t)i * n + k] * G[(size_t)j * n + k] * sc_k[k];
      H[(size_t)i * n + j] = H[(size_t)j * n + i] = s;
    }
  xkv_eigh_scratch sc;
  std::memset(&sc, 0, sizeof(sc));
  std::vector<double> w(n), Z((size_t)n * r);
  if (xkv_eigh_values(n, H.data(), r, w.data(), &sc) || xkv_eigh_vectors(&sc, 0, r, Z.data(), &sc)) bail("eigh", 0);
  const int nruns = xkv_eigh_runs(&sc, run_cap);
  std::vector<int> runs(4 * (size_t)nruns + 4), groups(2 * (size_t)nruns + 2), pos(r);
  std::vector<double> cs(2 * (size_t)sc.log.n + 2), refl(xkv_eigh_refl_doubles(n) + 1);
  xkv_eigh_pack_log(&sc, run_cap, runs.data(), cs.data());
  const int ng = xkv_eigh_group_runs(runs.data(), nruns, kB, spread, KRUNCAP + spread, groups.data());
  xkv_eigh_pack_reflectors(&sc, refl.data());
  xkv_eigh_positions(&sc, pos.data());
  long covered = 0;
  for (int q = 0; q < nruns; ++q) {
    const int* R = &runs[4 * q];
    if (R[1] - R[0] + 1 > run_cap || R[0] != (q ? runs[4 * (q - 1) + 1] + 1 : 0)) bail("run", q);
    covered += R[1] - R[0] + 1;
  }
  if (covered != sc.log.n) bail("runs cover the log", covered);
  for (int gq = 0, next = nruns - 1; gq < ng; ++gq) {
    if (groups[2 * gq] != next || groups[2 * gq + 1] < 1 || groups[2 * gq + 1] > kB) bail("group", gq);
    next -= groups[2 * gq + 1];
    if (gq + 1 == ng && next != -1) bail("groups cover the runs", next);
  }
  // the pieces: bounds[q] .. bounds[q + 1] - 1 are piece q's groups, together every group once
  std::vector<int> bounds(parts + 1, 0);
  if (parts > 1) xkv_eigh_split_groups(runs.data(), groups.data(), ng, KOVERHEAD, parts, bounds.data());
  else bounds[1] = ng;
  if (bounds[0] != 0 || bounds[parts] != ng) bail("pieces cover the groups", bounds[parts]);
  for (int q = 0; q < parts; ++q)
    if (bounds[q + 1] < bounds[q]) bail("piece bounds", q);
  const int rows = kPadLo + n + kPadHi;
  std::vector<double> Zd((size_t)n * r), csc((size_t)kB * kSlot), css((size_t)kB * kSlot), sr(rows);
  // column(start, g0, g1, out): the unit vector at row `start` with groups [g0, g1) applied, out[i]
  // for rows i < n at stride `ldo`
  auto column = [&](int start, int g_begin, int g_end, double* out, long ldo) {
    auto zl = [&](int row) {
      if (row + kPadLo < 0 || row + kPadLo >= rows) bail("row load", row);
      return sr[row + kPadLo];
    };
    auto zs = [&](int row, double v) {
      if (row + kPadLo < 0 || row + kPadLo >= rows) bail("row store", row);
      sr[row + kPadLo] = v;
    };
    for (int i = -kPadLo; i < n + kPadHi; ++i) zs(i, i == start ? 1.0 : 0.0);
    for (int gq = g_begin; gq < g_end; ++gq) {
      const int gx = groups[2 * gq], gy = groups[2 * gq + 1];
      std::vector<int> kt(kB), len(kB, 0);
      int f0 = INT_MIN, f1 = INT_MAX;
      for (int b = 0; b < gy; ++b) {
        const int* R = &runs[4 * (gx - b)];
        kt[b] = R[2];
        len[b] = R[1] - R[0] + 1;
        f0 = std::max(f0, R[2] - b);
        f1 = std::min(f1, R[2] - len[b] + 1 - b);
      }
      for (int b = gy; b < kB; ++b) kt[b] = f0 + b;
      for (int b = 0; b < kB; ++b) {
        const double* src = b < gy ? &cs[2 * (size_t)runs[4 * (gx - b)]] : cs.data();
        for (int idx = 0; idx < kSlot; ++idx) {
          const int m = idx - spread;
          const bool in = m >= 0 && m < len[b];
          csc[(size_t)b * kSlot + idx] = in ? src[2 * (len[b] - 1 - m)] : 1.0;
          css[(size_t)b * kSlot + idx] = in ? src[2 * (len[b] - 1 - m) + 1] : 0.0;
        }
      }
      std::vector<double> y(kB);
      for (int b = 0; b < kB; ++b) y[b] = zl(f0 + b + 1);
      std::vector<int> gi(kB);
      for (int b = 0; b < kB; ++b) gi[b] = spread + kt[b] - b - f0;
      const int steps = f0 - f1 + 1, nf = steps / CH, rem = steps % CH;
      int f = f0;
      std::vector<double> xa(CH), xb(CH);
      auto load = [&](std::vector<double>& x, int ff) {
        for (int u = 0; u < CH; ++u) x[u] = zl(ff - u);
      };
      auto apply = [&](const std::vector<double>& x, int ff, int cnt) {
        for (int u = 0; u < cnt; ++u) {
          double v = x[u];
          for (int b = 0; b < kB; ++b) {
            const int ix = gi[b] + u;
            if (ix < 0 || ix >= kSlot) bail("pair index", ix);
            const double c = csc[(size_t)b * kSlot + ix], s = css[(size_t)b * kSlot + ix], cx = c * v;
            v = std::fma(s, v, c * y[b]);
            y[b] = std::fma(-s, y[b], cx);
          }
          zs(ff - u + kB, v);
        }
      };
      load(xa, f);
      int c = 0;
      for (; c + 1 < nf; c += 2) {
        load(xb, f - CH);
        apply(xa, f, CH);
        f -= CH;
        for (int b = 0; b < kB; ++b) gi[b] += CH;
        load(xa, f - CH);
        apply(xb, f, CH);
        f -= CH;
        for (int b = 0; b < kB; ++b) gi[b] += CH;
      }
      if (c < nf) {
        load(xb, f - CH);
        apply(xa, f, CH);
        f -= CH;
        for (int b = 0; b < kB; ++b) gi[b] += CH;
        if (rem) apply(xb, f, rem);
      } else if (rem) {
        apply(xa, f, rem);
      }
      for (int b = 0; b < kB; ++b) zs(f1 + b, y[b]);
    }
    for (int i = 0; i < n; ++i) out[(size_t)i * ldo] = zl(i);
  };
  for (int j = 0; j < r; ++j) column(pos[j], bounds[0], bounds[1], Zd.data() + j, r);
  // Z <- S_q Z for the later pieces, S_q = piece q applied to the identity
  std::vector<double> Sq((size_t)n * n), Zt((size_t)n * r);
  for (int q = 1; q < parts; ++q) {
    for (int j = 0; j < n; ++j) column(j, bounds[q], bounds[q + 1], Sq.data() + j, n);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < r; ++j) {
        double t = 0;
        for (int k = 0; k < n; ++k) t += Sq[(size_t)i * n + k] * Zd[(size_t)k * r + j];
        Zt[(size_t)i * r + j] = t;
      }
    Zd.swap(Zt);
  }
  // the reflector blocks, last first: S2 -= Y (T (Y^T S2))
  const int NBG = XKV_EIGH_NBG, nref = n - 2;
  if (nref > 0) {
    const int nblk = (nref + NBG - 1) / NBG;
    const size_t ytot = xkv_eigh_refl_doubles(n) - (size_t)nblk * NBG * NBG;
    for (int b = nblk - 1; b >= 0; --b) {
      const int r0 = NBG * b + 1, M = n - r0;
      const double* Y = refl.data() + (size_t)NBG * ((size_t)b * (n - 1) - (size_t)NBG * b * (b - 1) / 2);
      const double* T = refl.data() + ytot + (size_t)b * NBG * NBG;
      for (int j = 0; j < r; ++j) {
        double d[64] = {0}, w2[64];
        for (int i = 0; i < M; ++i)
          for (int a = 0; a < NBG; ++a) d[a] += Y[(size_t)i * NBG + a] * Zd[(size_t)(r0 + i) * r + j];
        for (int a = 0; a < NBG; ++a) {
          double t = 0;
          for (int c2 = a; c2 < NBG; ++c2) t += T[a * NBG + c2] * d[c2];
          w2[a] = t;
        }
        for (int i = 0; i < M; ++i) {
          double t = 0;
          for (int a = 0; a < NBG; ++a) t += Y[(size_t)i * NBG + a] * w2[a];
          Zd[(size_t)(r0 + i) * r + j] -= t;
        }
      }
    }
  }
  double md = 0;
  for (size_t i = 0; i < Z.size(); ++i) md = std::fmax(md, std::fabs(Z[i] - Zd[i]));
  long full = 0;
  for (int q = 0; q < ng; ++q) full += groups[2 * q + 1] == kB;
  std::printf("n %d r %d rotations %ld runs %d groups %d full %ld parts %d (first groups", n, r, sc.log.n, nruns, ng,
              full, parts);
  for (int q = 0; q < parts; ++q) std::printf(" %d", bounds[q]);
  std::printf(") maxdiff %.3g\n", md);
  xkv_eigh_scratch_release(&sc);
  return md <= 1e-12 ? 0 : 4;
}

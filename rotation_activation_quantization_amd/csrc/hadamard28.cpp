// The library's order-28 Hadamard factor, built on the host from its
// definition: Paley's first construction for the prime power q = 27.
//
// Field: GF(27) represented as polynomials c0 + c1 t + c2 t^2 over GF(3),
// reduced modulo t^3 + 2t + 1 (so t^3 = t + 2).  An element is indexed
// e = c0 + 3 c1 + 9 c2.  The quadratic character chi(a) is 0 for a = 0, +1
// for the 13 nonzero squares and -1 for the other 13 elements.  With
// Q[i][j] = chi(e_i - e_j), S is Q with a border (S[0][0] = 0, S[0][j] = +1,
// S[i][0] = -1) and H28 = I + S.  Since q = 3 mod 4, chi(-1) = -1, Q and S are
// antisymmetric and H28 H28^T = 28 I.
#include <cstring>

#include "internal.h"

namespace signrot {
namespace {

struct Gf27 {
  int c[3];
};

Gf27 from_index(int e) { return Gf27{{e % 3, (e / 3) % 3, (e / 9) % 3}}; }
int to_index(const Gf27& a) { return a.c[0] + 3 * a.c[1] + 9 * a.c[2]; }

Gf27 sub(const Gf27& a, const Gf27& b) {
  Gf27 r;
  for (int i = 0; i < 3; ++i) r.c[i] = ((a.c[i] - b.c[i]) % 3 + 3) % 3;
  return r;
}

Gf27 mul(const Gf27& a, const Gf27& b) {
  int p[5] = {0, 0, 0, 0, 0};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) p[i + j] += a.c[i] * b.c[j];
  // t^4 = t * t^3 = t^2 + 2t ; t^3 = t + 2
  p[2] += p[4];
  p[1] += 2 * p[4];
  p[1] += p[3];
  p[0] += 2 * p[3];
  return Gf27{{p[0] % 3, p[1] % 3, p[2] % 3}};
}

H28Table build() {
  bool square[27];
  std::memset(square, 0, sizeof(square));
  for (int e = 1; e < 27; ++e) {
    Gf27 a = from_index(e);
    square[to_index(mul(a, a))] = true;
  }
  auto chi = [&](const Gf27& a) -> int {
    int idx = to_index(a);
    if (idx == 0) return 0;
    return square[idx] ? 1 : -1;
  };
  H28Table t;
  for (int i = 0; i < 28; ++i) {
    for (int j = 0; j < 28; ++j) {
      int s;
      if (i == 0 && j == 0) s = 0;
      else if (i == 0) s = 1;
      else if (j == 0) s = -1;
      else s = chi(sub(from_index(i - 1), from_index(j - 1)));
      t.h[i][j] = static_cast<int8_t>((i == j ? 1 : 0) + s);
    }
  }
  for (int i = 0; i < 28; ++i) {
    uint32_t m = 0;
    for (int j = 0; j < 28; ++j)
      if (t.h[i][j] < 0) m |= 1u << j;
    t.rowmask[i] = m;
  }
  return t;
}

}  // namespace

const H28Table& h28() {
  static const H28Table table = build();
  return table;
}

H28Masks h28_masks() {
  H28Masks r;
  for (int i = 0; i < 28; ++i) r.m[i] = h28().rowmask[i];
  return r;
}

}  // namespace signrot

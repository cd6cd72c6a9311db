// Outer Hadamard factors H_m of n = m * 2^k beyond order 28, built on the host
// from Paley's constructions.  The pages only require that the rotation be a
// Hadamard matrix; the choice of factor is the library's:
//   n = o * 2^v (o odd).  o = 1: no outer factor (Sylvester alone).  Else
//   m = o * 2^j for the smallest j >= 2 with a Paley matrix of order
//   m <= kMaxOuter:
//   - construction I when q = m - 1 is a prime power, q = 3 (mod 4):
//     S = [[0, 1^T], [-1, Q]], H = I + S;
//   - otherwise construction II when q = m/2 - 1 is a prime power, q = 1
//     (mod 4): C = [[0, 1^T], [1, Q]] and H = C (x) [[1, 1], [1, -1]] +
//     I (x) [[1, -1], [-1, -1]] (index 2 i + s);
//   with Q[i][j] = chi(e_i - e_j), chi the quadratic character of GF(q).
// GF(p^e) is GF(p)[t] modulo the first monic irreducible polynomial of degree
// e in lexicographic order of (a_{e-1}, ..., a_0); element e has base-p
// digits (c_0, c_1, ...) = polynomial coefficients.  For q = 27 this gives
// t^3 + 2t + 1, the modulus of h28(), and the same matrix.
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "internal.h"

namespace signrot {
namespace {

bool is_prime(int p) {
  if (p < 2) return false;
  for (int d = 2; d * d <= p; ++d)
    if (p % d == 0) return false;
  return true;
}

// q = p^e with p prime: returns true and sets p, e.
bool prime_power(int q, int* p, int* e) {
  if (q < 2) return false;
  int f = 2;
  while (q % f) ++f;  // smallest prime factor
  int x = q, k = 0;
  while (x % f == 0) {
    x /= f;
    ++k;
  }
  if (x != 1 || !is_prime(f)) return false;
  *p = f;
  *e = k;
  return true;
}

struct Field {
  int q = 0, p = 0, e = 0;
  std::vector<int> mod;  // a_0 .. a_{e-1}, 1
  std::vector<int> digit(int x) const {
    std::vector<int> d(e);
    for (int t = 0; t < e; ++t) {
      d[t] = x % p;
      x /= p;
    }
    return d;
  }
  int index(const std::vector<int>& d) const {
    int x = 0;
    for (int t = e - 1; t >= 0; --t) x = x * p + ((d[t] % p) + p) % p;
    return x;
  }
  int sub(int a, int b) const {
    std::vector<int> da = digit(a), db = digit(b), r(e);
    for (int t = 0; t < e; ++t) r[t] = ((da[t] - db[t]) % p + p) % p;
    return index(r);
  }
  int mul(int a, int b) const {
    std::vector<int> da = digit(a), db = digit(b), pr(2 * e - 1, 0);
    for (int i = 0; i < e; ++i)
      for (int j = 0; j < e; ++j) pr[i + j] += da[i] * db[j];
    for (int d = 2 * e - 2; d >= e; --d) {  // t^d = -(a_0 + ... + a_{e-1} t^{e-1}) t^{d-e}
      const int c = pr[d] % p;
      pr[d] = 0;
      for (int t = 0; t < e; ++t) pr[d - e + t] -= c * mod[t];
    }
    pr.resize(e);
    return index(pr);
  }
};

// true when the monic polynomial g (low first) divides f over GF(p)
bool divides(std::vector<int> f, const std::vector<int>& g, int p) {
  const int dg = static_cast<int>(g.size()) - 1;
  for (int d = static_cast<int>(f.size()) - 1; d >= dg; --d) {
    const int c = ((f[d] % p) + p) % p;
    if (c)
      for (int t = 0; t <= dg; ++t) f[d - dg + t] = ((f[d - dg + t] - c * g[t]) % p + p) % p;
  }
  for (int t = 0; t < dg; ++t)
    if (f[t] % p) return false;
  return true;
}

// coefficient list [a_0 .. a_{deg-1}, 1] of the i-th monic polynomial of
// degree deg in lexicographic order of (a_{deg-1}, ..., a_0)
std::vector<int> monic(int i, int deg, int p) {
  std::vector<int> f(deg + 1, 0);
  f[deg] = 1;
  for (int t = 0; t < deg; ++t) {  // a_0 is the last (fastest) digit
    f[t] = i % p;
    i /= p;
  }
  return f;
}

Field make_field(int q) {
  Field fl;
  prime_power(q, &fl.p, &fl.e);
  fl.q = q;
  if (fl.e == 1) {
    fl.mod = {0, 1};
    return fl;
  }
  int total = 1;
  for (int t = 0; t < fl.e; ++t) total *= fl.p;
  for (int i = 0; i < total; ++i) {
    std::vector<int> f = monic(i, fl.e, fl.p);
    bool irreducible = true;
    for (int d = 1; d <= fl.e / 2 && irreducible; ++d) {
      int cnt = 1;
      for (int t = 0; t < d; ++t) cnt *= fl.p;
      for (int g = 0; g < cnt && irreducible; ++g)
        if (divides(f, monic(g, d, fl.p), fl.p)) irreducible = false;
    }
    if (irreducible) {
      fl.mod = f;
      return fl;
    }
  }
  return fl;  // not reached for a prime power
}

// Paley construction type for order m: 1 (I), 2 (II) or 0; q set
int paley_kind(int m, int* q) {
  int p, e;
  if (m % 4) return 0;
  if ((m - 1) % 4 == 3 && prime_power(m - 1, &p, &e)) {
    *q = m - 1;
    return 1;
  }
  const int q2 = m / 2 - 1;
  if (q2 >= 5 && q2 % 4 == 1 && prime_power(q2, &p, &e)) {
    *q = q2;
    return 2;
  }
  return 0;
}

bool build(int m, OuterTable* out) {
  int q = 0;
  const int kind = paley_kind(m, &q);
  if (!kind) return false;
  const Field f = make_field(q);
  std::vector<int> chi(q, -1);
  chi[0] = 0;
  for (int x = 1; x < q; ++x) chi[f.mul(x, x)] = 1;
  auto jac = [&](int i, int j) { return chi[f.sub(i, j)]; };
  out->m = m;
  out->words = (m + 31) / 32;
  out->h.assign(static_cast<size_t>(m) * m, 0);
  if (kind == 1) {
    for (int i = 0; i < m; ++i)
      for (int j = 0; j < m; ++j) {
        int s;
        if (i == 0 && j == 0) s = 0;
        else if (i == 0) s = 1;
        else if (j == 0) s = -1;
        else s = jac(i - 1, j - 1);
        out->h[static_cast<size_t>(i) * m + j] = static_cast<int8_t>((i == j ? 1 : 0) + s);
      }
  } else {
    const int c = q + 1;
    auto conf = [&](int i, int j) {
      if (i == 0 && j == 0) return 0;
      if (i == 0 || j == 0) return 1;
      return jac(i - 1, j - 1);
    };
    const int a2[2][2] = {{1, 1}, {1, -1}};
    const int b2[2][2] = {{1, -1}, {-1, -1}};
    for (int i = 0; i < c; ++i)
      for (int s = 0; s < 2; ++s)
        for (int j = 0; j < c; ++j)
          for (int u = 0; u < 2; ++u)
            out->h[static_cast<size_t>(2 * i + s) * m + 2 * j + u] =
                static_cast<int8_t>(conf(i, j) * a2[s][u] + (i == j ? b2[s][u] : 0));
  }
  out->mask.assign(static_cast<size_t>(m) * out->words, 0u);
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < m; ++j)
      if (out->h[static_cast<size_t>(i) * m + j] < 0) out->mask[static_cast<size_t>(i) * out->words + j / 32] |= 1u << (j % 32);
  out->mask_t.assign(static_cast<size_t>(m) * out->words, 0u);
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < m; ++j)
      if (out->h[static_cast<size_t>(i) * m + j] < 0) out->mask_t[static_cast<size_t>(j) * out->words + i / 32] |= 1u << (i % 32);
  return true;
}

}  // namespace

int outer_order_for(int odd, int v) {
  for (int j = 2; j <= v; ++j) {
    const int64_t m = static_cast<int64_t>(odd) << j;
    if (m > kMaxOuter) break;
    int q;
    if (paley_kind(static_cast<int>(m), &q)) return static_cast<int>(m);
  }
  return 0;
}

const OuterTable* outer_table(int m) {
  static std::mutex mu;
  static std::map<int, OuterTable> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(m);
  if (it != cache.end()) return &it->second;
  OuterTable t;
  if (!build(m, &t)) return nullptr;
  return &cache.emplace(m, std::move(t)).first->second;
}

const OuterTable* outer_table_folded(int m, int j) {
  if (j == 0 && m > 1 && m != 28) return outer_table(m);
  const int64_t mm = static_cast<int64_t>(m) << j;
  if (m < 1 || j < 0 || mm > kMaxOuter || mm < 2) return nullptr;
  static std::mutex mu;
  static std::map<std::pair<int, int>, OuterTable> cache;
  // the factor H_m: Sylvester's [[1]] for m = 1, the order-28 table, or Paley
  std::vector<int8_t> base;
  if (m == 1) {
    base.assign(1, 1);
  } else if (m == 28) {
    base.assign(&h28().h[0][0], &h28().h[0][0] + 28 * 28);
  } else {
    const OuterTable* t = outer_table(m);
    if (!t) return nullptr;
    base = t->h;
  }
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({m, j});
  if (it != cache.end()) return &it->second;
  // H_m (x) Syl_{2^j}: entry (a 2^j + u, a' 2^j + v) = H_m[a][a'] (-1)^popcount(u & v)
  OuterTable t;
  t.m = static_cast<int>(mm);
  t.words = (t.m + 31) / 32;
  t.h.assign(static_cast<size_t>(t.m) * t.m, 0);
  const int B = 1 << j;
  for (int r = 0; r < t.m; ++r)
    for (int c = 0; c < t.m; ++c) {
      const int syl = (__builtin_popcount(static_cast<unsigned>((r % B) & (c % B))) & 1) ? -1 : 1;
      t.h[static_cast<size_t>(r) * t.m + c] = static_cast<int8_t>(base[static_cast<size_t>(r / B) * m + c / B] * syl);
    }
  t.mask.assign(static_cast<size_t>(t.m) * t.words, 0u);
  t.mask_t.assign(static_cast<size_t>(t.m) * t.words, 0u);
  for (int r = 0; r < t.m; ++r)
    for (int c = 0; c < t.m; ++c)
      if (t.h[static_cast<size_t>(r) * t.m + c] < 0) {
        t.mask[static_cast<size_t>(r) * t.words + c / 32] |= 1u << (c % 32);
        t.mask_t[static_cast<size_t>(c) * t.words + r / 32] |= 1u << (r % 32);
      }
  return &cache.emplace(std::make_pair(m, j), std::move(t)).first->second;
}

}  // namespace signrot

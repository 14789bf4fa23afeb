// Host permutation generators: Gilbert curve, cuboid order, inverse.
//
// Video-BLADE "Preprocessing" reorders tokens along a Gilbert space-filling
// curve before blocking; the pages name the curve only.  The curve built here
// is a corner-to-corner generalised Hilbert walk over the T x H x W box:
//
//   walk(o; a, b, c): visit every cell of the box spanned from corner o by
//   the axis-aligned signed extents a (major), b, c; start at o and finish on
//   the neighbouring corner along a.  Rules, first match wins:
//     |b| = |c| = 1          line along a
//     |a| = 1                (b, c) plane walked from o, then reversed
//     |c| = 1 / |b| = 1      the 2D walk of (a, b) / (a, c)
//     |a| >= 4, 2|a| > 3|b|, 2|a| > 3|c|
//                            cut a at h = half(|a|, 2); walk(o; a[:h], b, c),
//                            walk(o + a[:h]; a[h:], b, c)
//     |a| = |b| = |c| = 2    Gray order 000 001 011 010 110 111 101 100 (a b c)
//     otherwise              "U" across a and the longer minor x (ties: b),
//                            y the other: with X1 = half(|x|, 1), A1 = |a|/2,
//                            walk(o; x[:X1], y, a[:A1]);
//                            walk(o + x[:X1]; a, y, x[X1:]);
//                            walk(o + (|a|-1)^a + (X1-1)^x; -x[:X1], y, -a[A1:])
//   walk2(o; a, b) for planes: |b| = 1 line a; |a| = 1 line b reversed;
//     |a| >= 4 and 2|a| > 3|b| cut a at half(|a|, 2); otherwise the "U" with
//     B1 = half(|b|, 1), A1 = |a|/2: walk2(o; b[:B1], a[:A1]);
//     walk2(o + b[:B1]; a, b[B1:]); walk2(o + (|a|-1)^a + (B1-1)^b; -b[:B1], -a[A1:]).
//   half(L, r) = L/2, plus one when that is odd and L minus it stays >= r.
//   Top level: the major axis is the longest side of even length if one
//   exists (else the longest), then the longer remaining side; ties prefer
//   w, then h, then t.  Starting from (0, 0, 0).
// Choosing the even side as the root's major keeps every piece of the
// recursion "balanced" (even major side, or all sides odd), which is the
// condition for a corner-to-corner walk with unit steps; every step of the
// resulting curve therefore moves to a face-adjacent cell.
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "../dbs_internal.h"

namespace dbs {
namespace {

struct Ext {      // axis-aligned signed extent
  int axis;       // 0 = t, 1 = h, 2 = w
  int len;        // signed length, |len| >= 1
  int size() const { return len < 0 ? -len : len; }
  int dir() const { return len < 0 ? -1 : 1; }
  Ext take(int n) const { return Ext{axis, dir() * n}; }          // first n cells
  Ext rest(int n) const { return Ext{axis, dir() * (size() - n)}; }  // after the first n
  Ext flip() const { return Ext{axis, -len}; }
};

struct Pt {
  int c[3];
  Pt step(const Ext& e, int n) const {
    Pt p = *this;
    p.c[e.axis] += e.dir() * n;
    return p;
  }
};

int half(int L, int rest_min) {
  int h = L / 2;
  if ((h & 1) && L - (h + 1) >= rest_min) ++h;
  return h;
}

class CurveBuilder {
 public:
  CurveBuilder(int H, int W, int prefix, int32_t* out) : H_(H), W_(W), prefix_(prefix), out_(out) {}

  void walk3(Pt o, Ext a, Ext b, Ext c) {
    const int A = a.size(), B = b.size(), C = c.size();
    if (B == 1 && C == 1) { line(o, a); return; }
    if (A == 1) { plane_reversed(o, b, c); return; }
    if (C == 1) { walk2(o, a, b); return; }
    if (B == 1) { walk2(o, a, c); return; }
    if (A >= 4 && 2 * A > 3 * B && 2 * A > 3 * C) {
      const int h = half(A, 2);
      walk3(o, a.take(h), b, c);
      walk3(o.step(a, h), a.rest(h), b, c);
      return;
    }
    if (A == 2 && B == 2 && C == 2) {
      static const int gray[8][3] = {{0, 0, 0}, {0, 0, 1}, {0, 1, 1}, {0, 1, 0},
                                     {1, 1, 0}, {1, 1, 1}, {1, 0, 1}, {1, 0, 0}};
      for (const auto& gcode : gray) emit(o.step(a, gcode[0]).step(b, gcode[1]).step(c, gcode[2]));
      return;
    }
    const Ext x = (B >= C) ? b : c;
    const Ext y = (B >= C) ? c : b;
    const int X1 = half(x.size(), 1), A1 = A / 2;
    walk3(o, x.take(X1), y, a.take(A1));
    walk3(o.step(x, X1), a, y, x.rest(X1));
    walk3(o.step(a, A - 1).step(x, X1 - 1), x.take(X1).flip(), y, a.rest(A1).flip());
  }

  void walk2(Pt o, Ext a, Ext b) {
    const int A = a.size(), B = b.size();
    if (B == 1) { line(o, a); return; }
    if (A == 1) { line(o.step(b, B - 1), b.flip()); return; }
    if (A >= 4 && 2 * A > 3 * B) {
      const int h = half(A, 2);
      walk2(o, a.take(h), b);
      walk2(o.step(a, h), a.rest(h), b);
      return;
    }
    const int B1 = half(B, 1), A1 = A / 2;
    walk2(o, b.take(B1), a.take(A1));
    walk2(o.step(b, B1), a, b.rest(B1));
    walk2(o.step(a, A - 1).step(b, B1 - 1), b.take(B1).flip(), a.rest(A1).flip());
  }

 private:
  void emit(const Pt& p) { out_[pos_++] = prefix_ + (p.c[0] * H_ + p.c[1]) * W_ + p.c[2]; }
  void line(Pt o, Ext a) {
    for (int i = 0; i < a.size(); ++i) emit(o.step(a, i));
  }
  void plane_reversed(Pt o, Ext b, Ext c) {
    std::vector<int32_t> tmp((size_t)b.size() * c.size());
    CurveBuilder sub(H_, W_, prefix_, tmp.data());
    if (b.size() >= c.size()) sub.walk2(o, b, c); else sub.walk2(o, c, b);
    for (size_t i = tmp.size(); i-- > 0;) out_[pos_++] = tmp[i];
  }

  int H_, W_, prefix_;
  int32_t* out_;
  int64_t pos_ = 0;
};

}  // namespace

void gilbert3d(int T, int H, int W, int prefix, int32_t* out) {
  for (int i = 0; i < prefix; ++i) out[i] = i;
  struct Side { int len, rank, axis; };
  Side s[3] = {{W, 0, 2}, {H, 1, 1}, {T, 2, 0}};
  auto before = [](const Side& p, const Side& q) {   // longer first, then w, h, t
    return p.len != q.len ? p.len > q.len : p.rank < q.rank;
  };
  int major = -1;
  for (int i = 0; i < 3; ++i)
    if (s[i].len % 2 == 0 && (major < 0 || before(s[i], s[major]))) major = i;
  if (major < 0) {
    major = 0;
    for (int i = 1; i < 3; ++i)
      if (before(s[i], s[major])) major = i;
  }
  int r0 = -1, r1 = -1;
  for (int i = 0; i < 3; ++i) {
    if (i == major) continue;
    if (r0 < 0) r0 = i; else r1 = i;
  }
  if (before(s[r1], s[r0])) { const int t = r0; r0 = r1; r1 = t; }
  CurveBuilder cb(H, W, prefix, out + prefix);
  Pt o{{0, 0, 0}};
  cb.walk3(o, Ext{s[major].axis, s[major].len}, Ext{s[r0].axis, s[r0].len},
           Ext{s[r1].axis, s[r1].len});
}

void cuboid_order(int T, int H, int W, int ct, int ch, int cw, int prefix, int32_t* out) {
  int64_t pos = 0;
  for (int i = 0; i < prefix; ++i) out[pos++] = i;
  for (int t0 = 0; t0 < T; t0 += ct)
    for (int h0 = 0; h0 < H; h0 += ch)
      for (int w0 = 0; w0 < W; w0 += cw)
        for (int t = t0; t < T && t < t0 + ct; ++t)
          for (int h = h0; h < H && h < h0 + ch; ++h)
            for (int w = w0; w < W && w < w0 + cw; ++w)
              out[pos++] = prefix + (t * H + h) * W + w;
}

}  // namespace dbs

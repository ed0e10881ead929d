// Host builder of the E8 codebook (QuIP#, abstract: codebooks built on the E8
// lattice). The lattice is D8 (integer vectors with an even coordinate sum)
// together with D8 + (1/2, ..., 1/2). The codebook keeps its 65536 points of
// smallest squared norm, ordered by squared norm and then by the coordinates
// read as real numbers from the first to the last.
//
// Enumeration works in doubled coordinates v = 2x (all even for D8, all odd
// for the shifted coset); a depth-first walk over the 8 coordinates prunes on
// the running squared norm (|x|^2 <= 12 is enough: the first 65536 points end
// inside the shell of squared norm 12).
#include <algorithm>
#include <array>
#include <vector>

#include "common.h"

namespace quip {
namespace {

struct Pt {
  int norm4;  // 4 |x|^2
  std::array<int8_t, 8> v;
};

void walk(int depth, int norm4, int sum2, bool odd, std::array<int8_t, 8>& cur, std::vector<Pt>& out,
          int limit4) {
  if (depth == 8) {
    // coordinate sum x = sum2 / 2 must be even  <=>  sum2 % 4 == 0
    if (((sum2 % 4) + 4) % 4 == 0) out.push_back(Pt{norm4, cur});
    return;
  }
  for (int v = -7; v <= 7; ++v) {
    if (((v & 1) != 0) != odd) continue;
    int nn = norm4 + v * v;
    if (nn > limit4) continue;
    cur[depth] = int8_t(v);
    walk(depth + 1, nn, sum2 + v, odd, cur, out, limit4);
  }
}

}  // namespace

void e8_build_codebook(float* host_out) {
  std::vector<Pt> pts;
  pts.reserve(200000);
  std::array<int8_t, 8> cur{};
  const int limit4 = 4 * 12;
  walk(0, 0, 0, false, cur, pts, limit4);
  walk(0, 0, 0, true, cur, pts, limit4);
  std::sort(pts.begin(), pts.end(), [](const Pt& a, const Pt& b) {
    if (a.norm4 != b.norm4) return a.norm4 < b.norm4;
    return a.v < b.v;  // lexicographic on the doubled coordinates = on the reals
  });
  for (size_t i = 0; i < 65536; ++i)
    for (int k = 0; k < 8; ++k) host_out[i * 8 + k] = 0.5f * float(pts[i].v[k]);
}

}  // namespace quip

// Workgroup placement of the many-row GEMM launches: a plain constexpr
// function with no HIP types, so the kernels call it and the host tests
// check it.
#pragma once

namespace sdm {

// Work units are (weight tile group, K split) pairs; activation groups go in
// bands of eight.  Inside a band of g groups, g dividing 8, workgroup L takes
// group L % g and unit L / g: workgroups go to the eight XCDs round robin, so
// each XCD keeps one activation group (L2-resident), and the groups reading
// one weight tile run at the same time (the tile comes from HBM once).  A
// band whose group count does not divide 8 runs group by group.  Over
// L in [0, units * groups) every (unit, group) pair comes out exactly once.
struct ManyRowPlace {
  int unit, group;
};
constexpr ManyRowPlace many_row_place(int L, int units, int groups) {
  const int band = L / (units * 8);
  const int r = L - band * units * 8;
  const int gb = (groups - 8 * band) < 8 ? (groups - 8 * band) : 8;
  if (8 % gb == 0) return ManyRowPlace{r / gb, 8 * band + r % gb};
  return ManyRowPlace{r % units, 8 * band + r / units};
}

}  // namespace sdm

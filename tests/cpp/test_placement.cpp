// Host check of the many-row GEMM workgroup placement (placement.hpp):
// every (unit, activation group) pair exactly once, and inside a band whose
// group count divides 8, one activation group per XCD (workgroups reach the
// XCDs round robin: XCD = L % 8).
#include <cstdio>
#include <vector>

#include "placement.hpp"

int main() {
  int fails = 0, cases = 0;
  const int unit_counts[] = {1, 2, 7, 64, 96, 256, 384, 544, 2374};
  for (int units : unit_counts)
    for (int groups = 1; groups <= 40; ++groups) {
      ++cases;
      std::vector<int> seen((size_t)units * groups, 0);
      std::vector<int> xcd_group(8 * ((groups + 7) / 8), -1);  // per (band, XCD)
      for (int L = 0; L < units * groups; ++L) {
        const sdm::ManyRowPlace p = sdm::many_row_place(L, units, groups);
        if (p.unit < 0 || p.unit >= units || p.group < 0 || p.group >= groups) {
          std::printf("out of range: units %d groups %d L %d -> (%d, %d)\n", units, groups, L, p.unit, p.group);
          ++fails;
          break;
        }
        ++seen[(size_t)p.group * units + p.unit];
        const int band = p.group / 8, gb = groups - 8 * band < 8 ? groups - 8 * band : 8;
        if (8 % gb == 0) {
          int& g = xcd_group[band * 8 + L % 8];
          if (g < 0) g = p.group;
          else if (g != p.group) {
            std::printf("XCD %d of band %d sees groups %d and %d (units %d groups %d)\n", L % 8, band, g, p.group,
                        units, groups);
            ++fails;
          }
        }
      }
      for (size_t i = 0; i < seen.size(); ++i)
        if (seen[i] != 1) {
          std::printf("pair %zu covered %d times (units %d groups %d)\n", i, seen[i], units, groups);
          ++fails;
          break;
        }
    }
  if (fails) return 1;
  std::printf("all checks passed (%d configurations)\n", cases);
  return 0;
}

// Host check of the shared-prefix launch's workgroup -> wave mapping
// (pa_launch_map.h, the header the device kernel includes).  For every
// tail / prefix wave count in a range it checks that each tail index
// 0..waves-1 and each prefix index 0..pf_waves-1 is given to exactly one
// workgroup of the grid, and that indices keep their workgroup's XCD
// (id mod 8) where the header promises it.  Prints "launch map: ok".
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "pa_launch_map.h"

static int failures = 0;
#define CHECK(c, ...)                      \
  do {                                     \
    if (!(c)) {                            \
      if (failures++ < 20) {               \
        fprintf(stderr, __VA_ARGS__);      \
        fprintf(stderr, "\n");             \
      }                                    \
    }                                      \
  } while (0)

static void check(int waves, int pf_waves) {
  std::vector<int> seen_tail(waves, 0), seen_pf(pf_waves, 0);
  const int alt = pa::mixed_alternating(waves, pf_waves);
  for (int b = 0; b < waves + pf_waves; ++b) {
    const pa::MixedWave w = pa::mixed_wave(b, waves, pf_waves);
    if (w.tail) {
      CHECK(w.index >= 0 && w.index < waves, "waves %d pf %d: b %d -> tail %d out of range",
            waves, pf_waves, b, w.index);
      if (w.index >= 0 && w.index < waves) ++seen_tail[w.index];
      CHECK(w.index % 8 == b % 8, "waves %d pf %d: b %d -> tail %d changes XCD", waves,
            pf_waves, b, w.index);
    } else {
      CHECK(w.index >= 0 && w.index < pf_waves, "waves %d pf %d: b %d -> prefix %d out of range",
            waves, pf_waves, b, w.index);
      if (w.index >= 0 && w.index < pf_waves) ++seen_pf[w.index];
      if (b < alt || waves % 8 == 0)
        CHECK(w.index % 8 == b % 8, "waves %d pf %d: b %d -> prefix %d changes XCD", waves,
              pf_waves, b, w.index);
    }
  }
  for (int i = 0; i < waves; ++i)
    CHECK(seen_tail[i] == 1, "waves %d pf %d: tail %d runs %d times", waves, pf_waves, i,
          seen_tail[i]);
  for (int i = 0; i < pf_waves; ++i)
    CHECK(seen_pf[i] == 1, "waves %d pf %d: prefix %d runs %d times", waves, pf_waves, i,
          seen_pf[i]);
}

int main() {
  for (int w = 0; w <= 300; ++w)
    for (int p = 0; p <= 300; ++p) check(w, p);
  // Launch sizes of the 256-CU part: tails get what the prefix waves leave.
  const int sizes[] = {64, 256, 700, 1536, 1792, 2048, 4096};
  for (int w : sizes)
    for (int p : {1, 7, 8, 9, 12, 16, 100, 768, 1000, 3000}) check(w, p);
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("launch map: ok\n");
  return 0;
}

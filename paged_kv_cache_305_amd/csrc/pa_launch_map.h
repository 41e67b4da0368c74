// Workgroup -> wave mapping of the shared-prefix launch, as a pure integer
// function that the device kernel and a host test both compile.
//
// One launch holds `waves` tail waves (the balanced split over each
// sequence's own tokens) and `pf_waves` prefix waves (the shared blocks).
// Workgroups are dealt in runs of 8, alternating tail / prefix, while both
// kinds have a whole run left; the rest follows, first the remaining tail
// waves, then the remaining prefix waves.  Every tail index 0..waves-1 and
// every prefix index 0..pf_waves-1 is given to exactly one workgroup of the
// 0..waves+pf_waves-1.  In the alternating part, and for the remaining tail
// waves, a wave's index within its kind equals its workgroup id mod 8, so
// both kinds keep their XCD placement (workgroups go round-robin to the 8
// XCDs); the remaining prefix waves keep it when `waves` is a multiple of 8.
#pragma once

#if defined(__HIPCC__)
#define PA_HOST_DEVICE __host__ __device__
#else
#define PA_HOST_DEVICE
#endif

namespace pa {

struct MixedWave {
  bool tail;   // a tail wave (else a prefix wave)
  int index;   // its index among the waves of its kind
};

// Workgroups at the start of the launch dealt alternately, 8 of each kind
// at a time: twice the smaller count, rounded down to whole runs of 8.
PA_HOST_DEVICE inline int mixed_alternating(int waves, int pf_waves) {
  int m = waves < pf_waves ? waves : pf_waves;
  m -= m % 8;
  return 2 * m;
}

PA_HOST_DEVICE inline MixedWave mixed_wave(int b, int waves, int pf_waves) {
  const int alt = mixed_alternating(waves, pf_waves), m = alt / 2;
  MixedWave w;
  if (b < alt) {
    w.tail = ((b >> 3) & 1) == 0;
    w.index = ((b >> 4) << 3) | (b & 7);
    return w;
  }
  const int r = b - alt;
  if (r < waves - m) {
    w.tail = true;
    w.index = m + r;
  } else {
    w.tail = false;
    w.index = m + (r - (waves - m));
  }
  return w;
}

}  // namespace pa

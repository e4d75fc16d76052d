// pow_f32.h -- the f64 power of the device math library rounded to f32, by a
// shorter route.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace per {

// f32(pow(y, a)): the f64 pow rounded once to f32, bit for bit what
// (float)pow(y, a) gives on the device, in a fraction of its time.  With
// z = a log2(y), r = exp2(z) in f64 lies within 4 + 3.5|z| units in the last
// place of y^a (log2 and exp2 each within 2 units, the product within half a
// unit, and an error dz in z moves r by ln2 dz relatively), so r rounds to the
// same f32 as y^a -- and as the f64 pow, within a unit of y^a -- unless it
// lies that close to a point halfway between two f32 values.  The 29 low bits
// of r's significand are what rounding to f32 drops, and such a point sits
// where they read 2^28; within twice that distance (plus 2|a| units, for a
// log2 near y = 1 that is only absolutely accurate), and wherever the result
// leaves the f32 normal range or z is NaN (y <= 0 included), the f64 pow
// itself is taken.  That is about one case in 10^6 at |z| ~ 20.
__device__ __forceinline__ float pow_f32(double y, double a) {
  const double z = a * log2(y);
  if (z > -125.0 && z < 127.0) {
    const double r = exp2(z);
    const int64_t d = (int64_t)(__double_as_longlong(r) & 0x1FFFFFFFll) - 0x10000000ll;
    const double margin = 8.0 + 8.0 * fabs(z) + 2.0 * fabs(a);
    if ((double)(d < 0 ? -d : d) > margin) return (float)r;
  }
  return (float)pow(y, a);
}

}  // namespace per

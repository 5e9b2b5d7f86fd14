// Instantiations of the gather + rebuild + RoPE + attention kernel for F32 with d = 64
// (see select_attend.inc).
#include "select_attend.inc"
#include "select_attend_variants.h"

namespace sals {
namespace sa {

#define SALS_CASE(RR)                       \
  case RR:                                  \
    launch_shape<F32, RR, 64>(a, st);       \
    return true;
bool f32_d64_launch(int r, const SAArgs& a, hipStream_t st) {
  switch (r) { SALS_CASE(32) SALS_CASE(64) SALS_CASE(128) SALS_CASE(256) SALS_CASE(384) SALS_CASE(512) }
  return false;
}
#undef SALS_CASE

#define SALS_CASE(RR) \
  case RR:            \
    return max_split_t<F32, RR, 64>(nqh);
int f32_d64_max_split(int r, int nqh) {
  switch (r) { SALS_CASE(32) SALS_CASE(64) SALS_CASE(128) SALS_CASE(256) SALS_CASE(384) SALS_CASE(512) }
  return 0;
}
#undef SALS_CASE

}  // namespace sa
}  // namespace sals

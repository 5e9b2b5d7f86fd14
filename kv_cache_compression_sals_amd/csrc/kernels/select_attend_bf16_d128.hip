// Instantiations of the gather + rebuild + RoPE + attention kernel for BF16 with d = 128
// (see select_attend.inc).
#include "select_attend.inc"
#include "select_attend_variants.h"

namespace sals {
namespace sa {

#define SALS_CASE(RR)                       \
  case RR:                                  \
    launch_shape<BF16, RR, 128>(a, st);       \
    return true;
bool bf16_d128_launch(int r, const SAArgs& a, hipStream_t st) {
  switch (r) { SALS_CASE(32) SALS_CASE(64) SALS_CASE(128) SALS_CASE(256) SALS_CASE(384) SALS_CASE(512) }
  return false;
}
#undef SALS_CASE

#define SALS_CASE(RR) \
  case RR:            \
    return max_split_t<BF16, RR, 128>(nqh);
int bf16_d128_max_split(int r, int nqh) {
  switch (r) { SALS_CASE(32) SALS_CASE(64) SALS_CASE(128) SALS_CASE(256) SALS_CASE(384) SALS_CASE(512) }
  return 0;
}
#undef SALS_CASE

#define SALS_CASE(RR) \
  case RR:            \
    return rank_fits_t<BF16, RR, 128>(nqh, split_len, nc, kp);
bool bf16_d128_rank_fits(int r, int nqh, int split_len, int nc, int kp) {
  switch (r) { SALS_CASE(32) SALS_CASE(64) SALS_CASE(128) SALS_CASE(256) SALS_CASE(384) SALS_CASE(512) }
  return false;
}
#undef SALS_CASE

}  // namespace sa
}  // namespace sals

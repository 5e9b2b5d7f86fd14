// Per-(dtype, head dimension) entry points of the gather + rebuild + RoPE + attention kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sals {
namespace sa {

struct SAArgs;

bool bf16_d128_launch(int r, const SAArgs& a, hipStream_t st);
bool bf16_d64_launch(int r, const SAArgs& a, hipStream_t st);
bool f32_d128_launch(int r, const SAArgs& a, hipStream_t st);
bool f32_d64_launch(int r, const SAArgs& a, hipStream_t st);
int bf16_d128_max_split(int r, int nqh);
int bf16_d64_max_split(int r, int nqh);
int f32_d128_max_split(int r, int nqh);
int f32_d64_max_split(int r, int nqh);
bool bf16_d128_rank_fits(int r, int nqh, int split_len, int nc, int kp);

}  // namespace sa
}  // namespace sals

// Instantiations of the attention mainloop (the native kernel catalog's
// kernels, one per physical tile shape and head dimension).
#include "attn_fwd.h"

namespace bsa {

AttnLauncher attn_launcher(int tq, int tkv, int d) {
#define BSA_CASE(TQ_, TKV_, D_) \
  if (tq == TQ_ && tkv == TKV_ && d == D_) return &launch_attn<TQ_, TKV_, D_>;
  BSA_CASE(64, 64, 128)
  BSA_CASE(128, 32, 128)
  BSA_CASE(128, 64, 128)
  BSA_CASE(128, 128, 128)
  BSA_CASE(256, 64, 128)
  BSA_CASE(64, 32, 64)
  BSA_CASE(64, 64, 64)
  BSA_CASE(128, 32, 64)
  BSA_CASE(128, 64, 64)
  BSA_CASE(64, 32, 32)
  BSA_CASE(64, 64, 32)
  BSA_CASE(128, 64, 32)
  BSA_CASE(128, 128, 32)
  BSA_CASE(64, 32, 256)
  BSA_CASE(128, 32, 256)
#undef BSA_CASE
  return nullptr;
}

template <int TQ, int TKV, int D, bool STREAM>
static int wg_per_cu_as() {
  int n = 0;
  hipError_t e;
  if constexpr (use_w3<TQ, TKV, D>())
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_kernel_w3<TQ, TKV, D, STREAM>, TQ * 2, 0);
  else if constexpr (use_w2<TQ, TKV, D>())
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_kernel_w2<TQ, TKV, D, STREAM>, TQ * 2, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_kernel<TQ, TKV, D, STREAM>, TQ * 2, 0);
  return e == hipSuccess ? n : 0;
}
template <int TQ, int TKV, int D>
static int wg_per_cu(bool stream) {
  return stream ? wg_per_cu_as<TQ, TKV, D, true>() : wg_per_cu_as<TQ, TKV, D, false>();
}

int attn_wg_per_cu(int tq, int tkv, int d, bool stream) {
#define BSA_CASE(TQ_, TKV_, D_) \
  if (tq == TQ_ && tkv == TKV_ && d == D_) return wg_per_cu<TQ_, TKV_, D_>(stream);
  BSA_CASE(64, 64, 128)
  BSA_CASE(128, 32, 128)
  BSA_CASE(128, 64, 128)
  BSA_CASE(128, 128, 128)
  BSA_CASE(256, 64, 128)
  BSA_CASE(64, 32, 64)
  BSA_CASE(64, 64, 64)
  BSA_CASE(128, 32, 64)
  BSA_CASE(128, 64, 64)
  BSA_CASE(64, 32, 32)
  BSA_CASE(64, 64, 32)
  BSA_CASE(128, 64, 32)
  BSA_CASE(128, 128, 32)
  BSA_CASE(64, 32, 256)
  BSA_CASE(128, 32, 256)
#undef BSA_CASE
  return 0;
}

}  // namespace bsa

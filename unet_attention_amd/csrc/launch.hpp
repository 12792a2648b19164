// launch.hpp -- internal launchers between the C ABI (sdattn_api.hip) and
// the kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_common.hpp"

namespace sdattn {

// Launch a kernel whose one parameter is `arg` and return this launch's own
// status: an error left on the thread by earlier, unrelated work is neither
// reported nor cleared.
template <typename A>
hipError_t launch_kernel(void (*kernel)(A), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, A arg) {
  void *args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, lds, stream);
}

// Largest key count the short-key (all keys in LDS) bf16 kernel takes for
// head dimension d.
int short_path_max_keys(int d);

// 16-bit kernels (bf16, or fp16 when half).  a.qblocks and a.nwg are filled
// in by the launcher.
hipError_t launch_16(const Args16 &a, int BH, bool short_path, bool out_f32, bool half,
                     hipStream_t stream);

// The same for one head-dim class DK (head dim rounded up to 16).
template <int DK>
hipError_t launch_16_dk(const Args16 &a, int BH, bool short_path, bool out_f32, bool half,
                        hipStream_t stream);

// GroupNorm (+ SiLU); elem: 0 fp32, 1 bf16, 2 fp16 (x, and y unless out_f32).
hipError_t launch_group_norm(const GnArgs &a, int elem, bool out_f32, hipStream_t stream);

// Largest group (elements) the register-resident GroupNorm kernel holds.
int group_norm_max_resident();

// Most channels per group (their gamma and beta are staged in LDS).
int group_norm_max_channels_per_group();

// fp32 kernel (any Lk).
hipError_t launch_f32(const F32Args &a, int BH, hipStream_t stream);

}  // namespace sdattn

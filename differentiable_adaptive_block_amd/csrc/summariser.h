// Launchers of the learned Stage-0 summariser (summariser.hip).
#pragma once

#include "common.h"

hipError_t launch_pool_attn(const void* k, const float* w, void* kbar, int BH, int H, int T, int D, int dtype,
                            hipStream_t st);
// dk_in: null (dk holds the other dK terms and is updated in place) or the
// other terms unrounded (fp32, dk's layout; dk is then written once).
hipError_t launch_pool_attn_bwd(const void* k, const float* w, const float* dkbar, void* dk, float* dw,
                                float* dw_part, int B, int H, int T, int D, int dtype, hipStream_t st,
                                const float* dk_in = nullptr);

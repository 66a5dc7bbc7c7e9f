// Row padding for a causal prefill of a length that is not a multiple of 64 (ragged.hip).
#pragma once

#include "common.h"

hipError_t launch_pad_rows(const void* src, void* dst, int BH, int T, int Tp, int row_bytes, hipStream_t st);
hipError_t launch_unpad_rows(const void* src, void* dst, int BH, int T, int Tp, int row_bytes, hipStream_t st);
hipError_t launch_pad_f32(const float* src, float* dst, int BH, int T, int Tp, float fill, hipStream_t st);
hipError_t launch_unpad_f32(const float* src, float* dst, int BH, int T, int Tp, hipStream_t st);

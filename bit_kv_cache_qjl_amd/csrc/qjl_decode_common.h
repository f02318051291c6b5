// Device helpers shared by the two decode paths (byte tables, matrix cores).
#pragma once

#include "qjl_common.h"

namespace qjl {

template <typename QT>
__device__ __forceinline__ float load_elem(const QT* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }

// dot of one JL row (d = 128 values, bf16 or fp32) with the masked query in LDS, fp32 in channel order
__device__ __forceinline__ float row_dot(const uint16_t* row, const float* q) {
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < kD / 8; ++v) {
        const uint4 x = reinterpret_cast<const uint4*>(row)[v];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(__uint_as_float(w[e] << 16), q[8 * v + 2 * e], acc);
            acc = fmaf(__uint_as_float(w[e] & 0xFFFF0000u), q[8 * v + 2 * e + 1], acc);
        }
    }
    return acc;
}
__device__ __forceinline__ float row_dot(const float* row, const float* q) {
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < kD / 4; ++v) {
        const float4 x = reinterpret_cast<const float4*>(row)[v];
        acc = fmaf(x.x, q[4 * v], acc);
        acc = fmaf(x.y, q[4 * v + 1], acc);
        acc = fmaf(x.z, q[4 * v + 2], acc);
        acc = fmaf(x.w, q[4 * v + 3], acc);
    }
    return acc;
}

}  // namespace qjl

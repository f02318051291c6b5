// Token-wise value quantization (memory-bound: 256 B read, 36 B written per token and KV head).
//
// Method: "2 numbers out of 128 destroy the entire KV cache", "The Obvious Fix: Use Fewer Bits"
// (take the range of the vector, divide it into 2^b equally spaced values, round each number to the
// nearest) and the QJL summary, "Limitations" (values use token-wise quantization).
//
// Sixteen threads own one value vector (8 channels each): a 16-lane min/max butterfly, then every
// thread emits 8 codes (nbits bytes).  The decisions are IEEE fp32 operations with no contraction:
// subtract, correctly rounded divide, fp16 round-to-nearest-even, rint (ties to even).
#include "qjl_common.h"

namespace qjl {
namespace {

constexpr int kRowsPerBlock = 16;

template <typename VT>
__device__ __forceinline__ void load8(const VT* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const float4 x = reinterpret_cast<const float4*>(p)[0];
    const float4 y = reinterpret_cast<const float4*>(p)[1];
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

template <typename VT, int NBITS>
__global__ __launch_bounds__(256) void quantize_values_kernel(ValueQuantArgs a) {
#pragma clang fp contract(off)
    const int tid = threadIdx.x;
    const int sub = tid & 15;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (tid >> 4);
    const int64_t rows = (int64_t)a.B * a.T * a.Hkv;
    const bool valid = row < rows;
    const int h = (int)(row % a.Hkv);
    const int64_t bt = row / a.Hkv;
    const int64_t t = bt % a.T;
    const int64_t b = bt / a.T;

    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (valid) load8<VT>(static_cast<const VT*>(a.V) + b * a.sVb + t * a.sVt + h * a.sVh + 8 * sub, v);
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int q = 1; q < 8; ++q) {
        mn = fminf(mn, v[q]);
        mx = fmaxf(mx, v[q]);
    }
    mn = row16_min(mn);   // the 16 lanes of a vector are one DPP row; min/max are exact
    mx = row16_max(mx);
    constexpr int L = (1 << NBITS) - 1;
    const float range = mx - mn;
    const float stepf = range / (float)L;
    const _Float16 step16 = (_Float16)stepf;
    const _Float16 mn16 = (_Float16)mn;
    const float step = (float)step16;
    const float base = (float)mn16;
    uint32_t packed = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t code = 0;
        if (step != 0.f) {
            const float diff = v[q] - base;
            const float r = rintf(diff / step);
            code = (uint32_t)fminf(fmaxf(r, 0.f), (float)L);
        }
        packed |= code << (NBITS * q);
    }
    if (!valid) return;
    const int64_t cache_row = ((int64_t)b * a.Hkv + h) * a.Ncap + a.t0 + t;
    uint8_t* dst = a.codes + cache_row * (16 * NBITS) + sub * NBITS;
    if (NBITS == 2) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
    } else if (NBITS == 4) {
        *reinterpret_cast<uint32_t*>(dst) = packed;
    } else {
#pragma unroll
        for (int q = 0; q < NBITS; ++q) dst[q] = (uint8_t)(packed >> (8 * q));
    }
    if (sub == 0) {
        reinterpret_cast<uint32_t*>(a.meta)[cache_row] =
            (uint32_t)__builtin_bit_cast(uint16_t, mn16) | ((uint32_t)__builtin_bit_cast(uint16_t, step16) << 16);
    }
}

template <typename VT>
hipError_t launch_typed(const ValueQuantArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.T * a.Hkv;
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    switch (a.nbits) {
        case 2: hipLaunchKernelGGL((quantize_values_kernel<VT, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((quantize_values_kernel<VT, 3>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((quantize_values_kernel<VT, 4>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_values(const ValueQuantArgs& a, int vdt, hipStream_t s) {
    return vdt == 0 ? launch_typed<uint16_t>(a, s) : launch_typed<float>(a, s);
}

}  // namespace qjl

// Checks of the gfx950 instruction forms the library's kernels rely on, for the GPU tests in
// tests/test_gpu_instructions.py (test infrastructure: built beside the tests, loaded only by them).
// Each kernel runs one form on inputs the test chooses; the test compares the outputs with an exact
// model of the operand layout and number formats written on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef float v32f_t __attribute__((ext_vector_type(32)));
typedef uint32_t v6u_t __attribute__((ext_vector_type(6)));

// v_mfma_scale_f32_16x16x128_f8f6f4 with A in fp6 e2m3 (format 2) and B in fp4 e2m1 (format 4): lane
// l supplies the 8 words a[8 l ..], b[8 l ..] and the scale word sc[l], whose byte OP is the E8M0 scale
// of the lane's A slice; d[4 l + i] = D element i of lane l.
template <int OP>
__global__ void mfma_f6f4_kernel(const uint32_t* a, const uint32_t* b, const uint32_t* sc, float* d) {
    const int l = threadIdx.x;
    v8i_t A, B;
    for (int i = 0; i < 8; ++i) {
        A[i] = (int)a[8 * l + i];
        B[i] = (int)b[8 * l + i];
    }
    v4f_t C = {0.f, 0.f, 0.f, 0.f};
    C = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, 2, 4, OP, (int)sc[l], 0, 127);
    for (int i = 0; i < 4; ++i) d[4 * l + i] = C[i];
}

// v_cvt_scalef32_2xpk16_fp6_f32 of lane l's 32 values x[32 l ..] (the first 16 as the first source, the
// next 16 as the second) at scale s[l], the six packed words in p[6 l ..], and
// v_cvt_scalef32_pk32_f32_fp6 of those words back to 32 values in y[32 l ..].  The sources and the
// scale stay live across each conversion (the compiler may otherwise give the destination their
// registers, which these instructions do not allow).
__global__ void cvt_fp6_kernel(const float* x, const float* s, uint32_t* p, float* y) {
    const int l = threadIdx.x;
    v16f_t lo, hi;
    for (int i = 0; i < 16; ++i) {
        lo[i] = x[32 * l + i];
        hi[i] = x[32 * l + 16 + i];
    }
    const float scale = s[l];
    const v6u_t pk = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, scale);
    asm volatile("" :: "v"(lo), "v"(hi), "v"(scale));
    const v32f_t back = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(pk, scale);
    asm volatile("" :: "v"(pk), "v"(scale));
    for (int i = 0; i < 6; ++i) p[6 * l + i] = pk[i];
    for (int i = 0; i < 32; ++i) y[32 * l + i] = back[i];
}

// Buffer loads with an LDS destination: lane l loads `size` bytes at byte offset off[l] of src (1 KB)
// into LDS; the LDS image of one instruction is copied to out (size * 64 bytes).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}
__global__ void lds_dma_kernel(const uint32_t* src, const int* off, int size, uint32_t* out) {
    __shared__ __attribute__((aligned(16))) uint32_t img[64 * 4];
    const int l = threadIdx.x;
    for (int i = l; i < 64 * 4; i += 64) img[i] = 0xFFFFFFFFu;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(src), (short)0, 1024, 0x00020000);
    if (size == 16) dma16(r, img, off[l]);
    else dma4(r, img, off[l]);
    // the loads write LDS behind the compiler's back: wait for them, and keep img escaping
    asm volatile("s_waitcnt vmcnt(0)" :: "s"(img) : "memory");
    __syncthreads();
    for (int i = l; i < 64 * size / 4; i += 64) out[i] = img[i];
}

// A streaming read of n 16-byte words (grid-stride), folded into one word per thread so the loads stay.
__global__ void stream_read_kernel(const uint4* src, int64_t n, uint32_t* sink) {
    uint32_t acc = 0u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int probe_mfma_f6f4(const uint32_t* a, const uint32_t* b, const uint32_t* sc, int opsel, float* d, hipStream_t s) {
    switch (opsel) {
        case 0: hipLaunchKernelGGL(mfma_f6f4_kernel<0>, dim3(1), dim3(64), 0, s, a, b, sc, d); break;
        case 1: hipLaunchKernelGGL(mfma_f6f4_kernel<1>, dim3(1), dim3(64), 0, s, a, b, sc, d); break;
        case 2: hipLaunchKernelGGL(mfma_f6f4_kernel<2>, dim3(1), dim3(64), 0, s, a, b, sc, d); break;
        case 3: hipLaunchKernelGGL(mfma_f6f4_kernel<3>, dim3(1), dim3(64), 0, s, a, b, sc, d); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int probe_cvt_fp6(const float* x, const float* scale, uint32_t* packed, float* back, hipStream_t s) {
    hipLaunchKernelGGL(cvt_fp6_kernel, dim3(1), dim3(64), 0, s, x, scale, packed, back);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int probe_lds_dma(const uint32_t* src, const int* off, int size, uint32_t* out, hipStream_t s) {
    if (size != 4 && size != 16) return -1;
    hipLaunchKernelGGL(lds_dma_kernel, dim3(1), dim3(64), 0, s, src, off, size, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int probe_stream_read(const void* src, int64_t n16, uint32_t* sink, int blocks, hipStream_t s) {
    if (blocks <= 0 || n16 <= 0) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const uint4*>(src), n16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

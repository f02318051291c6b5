// Outlier-channel selection: for every KV head, the n_out channels whose keys have the largest mean
// magnitude over all prefill tokens of every sequence.
//
// Method: "2 numbers out of 128 destroy the entire KV cache", "The Real Problem: Outlier Channels"
// (a few coordinates carry values 10-100x the rest) and "Why Compressing the KV Cache Is Hard",
// "The Third Problem: Magnitude Outliers" (such channels have to be detected); the QJL summary
// ("Approach") gives them a separate quantizer copy.  The statistic is the mean of |k_c|; equal
// means are ordered by the lower channel, and the result lists the chosen channels in ascending
// order.
//
// Phase 1 (memory-bound, one pass over the keys): workgroup = (token range, KV head, sequence);
// 16 lanes of 8 channels x 16 token lanes add |k_c| in fp64 (bf16 magnitudes are exact in fp64;
// the sums are exact until they exceed 2^53 ulps of the smallest term) and reduce the 16 token lanes
// in a fixed order into one partial per channel.  Phase 2: one workgroup per head adds the partials
// in a fixed order (8 strided lanes per channel, then the lanes in order; the result does not
// depend on scheduling), ranks the channels, writes the chosen ones.  Comparing sums is comparing means: every channel of a head has the same count.
#include "qjl_common.h"

namespace qjl {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelTokLanes = kSelThreads / 16;     // token lanes per workgroup

// 8 channels of one key row as raw words (zeros when the token is past the range)
template <typename KT> struct Row8;
template <> struct Row8<uint16_t> { uint4 x; };
template <> struct Row8<float> { float4 x, y; };

template <typename KT>
__device__ __forceinline__ Row8<KT> load8(const KT* p, bool ok);
template <>
__device__ __forceinline__ Row8<uint16_t> load8<uint16_t>(const uint16_t* p, bool ok) {
    return Row8<uint16_t>{ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u)};
}
template <>
__device__ __forceinline__ Row8<float> load8<float>(const float* p, bool ok) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    return Row8<float>{ok ? reinterpret_cast<const float4*>(p)[0] : z, ok ? reinterpret_cast<const float4*>(p)[1] : z};
}

// acc[e] += |channel e| (bf16 and fp32 magnitudes are exact in fp64)
__device__ __forceinline__ void add_abs8(const Row8<uint16_t>& r, double (&acc)[8]) {
    const uint32_t w[4] = {r.x.x, r.x.y, r.x.z, r.x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] += (double)__uint_as_float((w[q] << 16) & 0x7FFFFFFFu);
        acc[2 * q + 1] += (double)__uint_as_float(w[q] & 0x7FFF0000u);
    }
}
__device__ __forceinline__ void add_abs8(const Row8<float>& r, double (&acc)[8]) {
    acc[0] += (double)fabsf(r.x.x); acc[1] += (double)fabsf(r.x.y); acc[2] += (double)fabsf(r.x.z); acc[3] += (double)fabsf(r.x.w);
    acc[4] += (double)fabsf(r.y.x); acc[5] += (double)fabsf(r.y.y); acc[6] += (double)fabsf(r.y.z); acc[7] += (double)fabsf(r.y.w);
}
constexpr int kSelUnroll = 4;                      // rows in flight per thread

template <typename KT>
__global__ __launch_bounds__(kSelThreads) void outlier_partials_kernel(OutlierArgs a) {
    __shared__ double red[kSelTokLanes][kD + 1];
    const int tid = threadIdx.x;
    const int cg = tid & 15, tl = tid >> 4;
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t t0 = (int64_t)blockIdx.x * a.tokens_per_block;
    const int64_t t1 = min(a.T, t0 + (int64_t)a.tokens_per_block);
    const KT* K = static_cast<const KT*>(a.K) + b * a.sKb + h * a.sKh + 8 * cg;
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t t = t0 + tl; t < t1; t += kSelUnroll * kSelTokLanes) {
        Row8<KT> r[kSelUnroll];
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) {
            const int64_t tu = t + u * kSelTokLanes;
            r[u] = load8<KT>(K + (tu < t1 ? tu : t) * a.sKt, tu < t1);
        }
#pragma unroll
        for (int u = 0; u < kSelUnroll; ++u) add_abs8(r[u], acc);   // zeros past the range add nothing
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tl][8 * cg + e] = acc[e];
    __syncthreads();
    if (tid < kD) {
        double s = 0.0;
#pragma unroll
        for (int l = 0; l < kSelTokLanes; ++l) s += red[l][tid];
        // partial index: sequence-major, then token block
        const int64_t p = (int64_t)b * gridDim.x + blockIdx.x;
        a.partial[(p * a.Hkv + h) * kD + tid] = s;
    }
}

constexpr int kPartLanes = 8;                      // partial lanes per channel in the selection kernel

__global__ __launch_bounds__(kD * kPartLanes) void outlier_select_kernel(OutlierArgs a, int64_t nparts) {
    __shared__ double lsum[kPartLanes][kD];
    __shared__ double sum[kD];
    const int c = threadIdx.x & (kD - 1), pl = threadIdx.x / kD, h = blockIdx.x;
    // lane pl adds partials pl, pl + 8, ... (four loads in flight), then the lanes in order 0..7
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    const double* src = a.partial + (size_t)h * kD + c;
    const int64_t stride = (int64_t)a.Hkv * kD;
    int64_t p = pl;
    for (; p + 3 * kPartLanes < nparts; p += 4 * kPartLanes) {
        s0 += src[p * stride];
        s1 += src[(p + kPartLanes) * stride];
        s2 += src[(p + 2 * kPartLanes) * stride];
        s3 += src[(p + 3 * kPartLanes) * stride];
    }
    for (; p < nparts; p += kPartLanes) s0 += src[p * stride];
    lsum[pl][c] = (s0 + s1) + (s2 + s3);
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int l = 0; l < kPartLanes; ++l) s += lsum[l][c];     // every lane of channel c: the same sum
    if (pl == 0) sum[c] = s;
    __syncthreads();
    // rank: channels ahead of c (larger sum, or equal sum and lower index); lane 0 of each channel
    // writes, in ascending channel order (channels 0..63 are wave 0, 64..127 wave 1)
    int rank = 0;
    for (int o = 0; o < kD; ++o) rank += (sum[o] > s || (sum[o] == s && o < c)) ? 1 : 0;
    const bool chosen = pl == 0 && rank < a.n_out;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(chosen);
    __shared__ uint64_t wmask[2];
    if (threadIdx.x < kD && (c & 63) == 0) wmask[c >> 6] = mask;
    __syncthreads();
    if (chosen) {
        const int lane = c & 63;
        int pos = __popcll(mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (c >= 64) pos += __popcll(wmask[0]);
        a.outlier_idx[h * a.n_out + pos] = c;
    }
}

}  // namespace

int64_t outlier_token_blocks(int B, int64_t T, int Hkv) {
    // ~1024 workgroups over (sequence, head, token block), at least 256 tokens each
    const int64_t units = (int64_t)B * Hkv;
    if (units <= 0 || T <= 0) return 0;
    int64_t nb = (1024 + units - 1) / units;
    const int64_t max_nb = (T + 255) / 256;
    if (nb > max_nb) nb = max_nb;
    return nb < 1 ? 1 : nb;
}

hipError_t launch_select_outliers(const OutlierArgs& a, int B, int kdt, hipStream_t s) {
    const int64_t nb = outlier_token_blocks(B, a.T, a.Hkv);
    if (nb > 0) {
        OutlierArgs p = a;
        p.tokens_per_block = (a.T + nb - 1) / nb;
        const dim3 grid((unsigned)nb, (unsigned)a.Hkv, (unsigned)B);
        if (kdt == 0) hipLaunchKernelGGL(outlier_partials_kernel<uint16_t>, grid, dim3(kSelThreads), 0, s, p);
        else hipLaunchKernelGGL(outlier_partials_kernel<float>, grid, dim3(kSelThreads), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(outlier_select_kernel, dim3((unsigned)a.Hkv), dim3(kD * kPartLanes), 0, s, a, nb * (int64_t)B);
    return hipGetLastError();
}

}  // namespace qjl

// Token-wise value quantization (256 B read and, at 2 bits, 36 B written per token and KV head; the
// kernel is bound by its vector instructions more than by HBM).
//
// Method: "2 numbers out of 128 destroy the entire KV cache", "The Obvious Fix: Use Fewer Bits"
// (take the range of the vector, divide it into 2^b equally spaced values, round each number to the
// nearest) and the QJL summary, "Limitations" (values use token-wise quantization).
//
// One workgroup per (32-token code tile touched by the append, KV head, sequence).  Phase 1: eight
// threads own one value vector (16 channels each): an 8-lane min/max butterfly, the (min, step)
// meta, and the codes of 16 channels into LDS, one byte per code.  Phase 2: one thread per stream
// slot p packs the tile's 32 codes of channel code_channel(p) into nbits words (the channel-major
// tile the decode kernels read as matrix-core operands; channel c is stream slot 8 (c % 16) + c / 16
// of the tile; token j sits in field code_field(j, nbits), or for 3-bit codes in the two planes
// described with code_field).  LDS row p holds slot p (the 8 lanes of a token then write 8 rows that
// fall on distinct banks).  In a row, token j = 16 a + 4 e + f is byte 16 a + 4 f + e: 2-bit words
// then come from three shift-or operations on the row's words (byte e of word f holds token 4 e + f,
// so w0 | w1 << 2 | (w2 | w3 << 2) << 4 puts token 4 e + f at bits 8 e + 2 f).  A tile wholly inside the
// append is stored; a tile the append covers only in part is merged bit-exactly with two atomics per
// word (clear the appended fields, then set them), so tokens outside [t0, t0 + T) keep their codes.
//
// The decisions are those of IEEE fp32 operations with no contraction: subtract, correctly rounded
// divide, fp16 round-to-nearest-even, rint (ties to even); value_codes reaches the same codes with
// reciprocal products and falls back to the divides near rounding boundaries.
#include "qjl_common.h"

namespace qjl {
namespace {

constexpr int kValThreads = kCodeTile * 8;    // 256: 8 threads per token, 16 channels each
constexpr int kRowPitch = kCodeTile + 4;      // bytes per channel row of the LDS code tile

// byte of token j in a channel's LDS row, and the token held by byte p
__host__ __device__ constexpr int code_byte(int j) { return 16 * (j >> 4) + 4 * (j & 3) + ((j & 15) >> 2); }
__host__ __device__ constexpr int byte_token(int p) { return 16 * (p >> 4) + 4 * (p & 3) + ((p & 15) >> 2); }
static_assert(byte_token(code_byte(13)) == 13 && byte_token(code_byte(22)) == 22, "inverse permutations");

// 2-bit fields [a, b) of a 16-field word (a, b clamped to 0..16)
__device__ __forceinline__ uint32_t field_mask2(int a, int b) {
    a = a < 0 ? 0 : (a > 16 ? 16 : a);
    b = b < 0 ? 0 : (b > 16 ? 16 : b);
    const uint32_t hi = b >= 16 ? 0xFFFFFFFFu : ((1u << (2 * b)) - 1u);
    const uint32_t lo = a >= 16 ? 0xFFFFFFFFu : ((1u << (2 * a)) - 1u);
    return hi & ~lo;
}

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

// grid: x = code tile of the append (from tile_first), y = KV head, z = sequence
template <typename VT, int NBITS>
__global__ __launch_bounds__(kValThreads) void quantize_values_kernel(ValueQuantArgs a, int64_t tile_first) {
#pragma clang fp contract(off)
    __shared__ __attribute__((aligned(16))) uint8_t cs[kD * kRowPitch];   // [channel][token of the tile]
    const int tid = threadIdx.x;
    const int sub = tid & 7;
    const int tk = tid >> 3;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t bh = b * a.Hkv + h;
    const int64_t tile = tile_first + blockIdx.x;
    const int64_t p0 = tile * kCodeTile;
    // tokens of the tile inside the append: [ia, ib) (uniform), so a lane's test is on its 32-bit index
    const int ia = (int)(a.t0 > p0 ? a.t0 - p0 : 0);
    const int ib = (int)(a.t0 + a.T - p0 < kCodeTile ? a.t0 + a.T - p0 : kCodeTile);
    const int64_t pos = p0 + tk;                      // cache position of this thread's token
    const bool valid = tk >= ia && tk < ib;

    float v[16], lo[8], hi[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) lo[q] = hi[q] = 0.f;
    if (valid) {
        // the tile's first row in the value tensor (uniform), then this lane's row and channels
        const VT* tile_row0 = static_cast<const VT*>(a.V) + b * a.sVb + h * a.sVh + (p0 - a.t0) * a.sVt;
        const VT* src = tile_row0 + tk * a.sVt + 16 * sub;
        load8<VT>(src, lo);
        load8<VT>(src + 8, hi);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        v[q] = lo[q];
        v[8 + q] = hi[q];
    }
    uint32_t code[16];
    const uint32_t mt = value_codes<NBITS, 16>(v, code);
#pragma unroll
    for (int q = 0; q < 16; ++q) cs[code_slot(16 * sub + q) * kRowPitch + code_byte(tk)] = (uint8_t)code[q];
    if (valid && sub == 0) reinterpret_cast<uint32_t*>(a.meta)[bh * a.Ncap + pos] = mt;
    __syncthreads();

    if (tid >= kD) return;
    const int slot = tid;
    const uint32_t* row = reinterpret_cast<const uint32_t*>(cs + slot * kRowPitch);
    uint32_t* dst = a.codes + ((size_t)bh * code_tiles(a.Ncap) + tile) * (kD * NBITS) + slot * NBITS;
    const bool full = ia == 0 && ib == kCodeTile;
    uint32_t wd[NBITS], msk[NBITS];
    if constexpr (NBITS == 2) {
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = row[k];
        wd[0] = (w[0] | (w[1] << 2)) | ((w[2] | (w[3] << 2)) << 4);
        wd[1] = (w[4] | (w[5] << 2)) | ((w[6] | (w[7] << 2)) << 4);
        msk[0] = field_mask2(ia, ib);
        msk[1] = field_mask2(ia - 16, ib - 16);
    } else {
#pragma unroll
        for (int k = 0; k < NBITS; ++k) wd[k] = msk[k] = 0u;
#pragma unroll
        for (int q = 0; q < kCodeTile / 4; ++q) {
            const uint32_t four = row[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = byte_token(4 * q + e);
                const uint32_t code = (four >> (8 * e)) & 0xFFu;
                const bool in = i >= ia && i < ib;
                if constexpr (NBITS == 3) {
                    // two planes: the low two bits where a 2-bit stream keeps its code, the high bit in word 2
                    const int bl = 2 * i;
                    wd[bl >> 5] |= (code & 3u) << (bl & 31);
                    if (in) msk[bl >> 5] |= 3u << (bl & 31);
                    wd[2] |= (code >> 2) << hi3_bit(i);
                    if (in) msk[2] |= 1u << hi3_bit(i);
                } else {
                    constexpr uint32_t fm = (1u << NBITS) - 1u;
                    const int bp = NBITS * code_field(i, NBITS);   // a 4-bit field never crosses a word
                    wd[bp >> 5] |= code << (bp & 31);
                    if (in) msk[bp >> 5] |= fm << (bp & 31);
                }
            }
        }
    }
    if (full) {
#pragma unroll
        for (int k = 0; k < NBITS; ++k) dst[k] = wd[k];
    } else {
#pragma unroll
        for (int k = 0; k < NBITS; ++k) {
            if (msk[k]) {
                atomicAnd(dst + k, ~msk[k]);
                atomicOr(dst + k, wd[k] & msk[k]);
            }
        }
    }
}

template <typename VT>
hipError_t launch_typed(const ValueQuantArgs& a, hipStream_t s) {
    const int64_t first = a.t0 / kCodeTile;
    const int64_t last = (a.t0 + a.T - 1) / kCodeTile;
    const int ntiles = (int)(last - first + 1);
    const dim3 grid((unsigned)ntiles, (unsigned)a.Hkv, (unsigned)a.B);
    switch (a.nbits) {
        case 2: hipLaunchKernelGGL((quantize_values_kernel<VT, 2>), grid, dim3(kValThreads), 0, s, a, first); break;
        case 3: hipLaunchKernelGGL((quantize_values_kernel<VT, 3>), grid, dim3(kValThreads), 0, s, a, first); break;
        default: hipLaunchKernelGGL((quantize_values_kernel<VT, 4>), grid, dim3(kValThreads), 0, s, a, first); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_values(const ValueQuantArgs& a, int vdt, hipStream_t s) {
    return vdt == 0 ? launch_typed<uint16_t>(a, s) : launch_typed<float>(a, s);
}

}  // namespace qjl

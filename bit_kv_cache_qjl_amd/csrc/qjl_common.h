// Internal definitions shared by the libqjl HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qjl {

constexpr int kD = 128;              // supported head dimension
constexpr int kMaxOutliers = 16;     // outlier channels per KV head (one bf16 MFMA K step)
constexpr int kMaxBits = 1024;       // m + m_out
constexpr float kSqrtHalfPi = 1.2533141373155002f;   // sqrt(pi / 2)
constexpr float kLog2e = 1.4426950408889634f;

// ---- cross-lane reductions on the VALU (DPP row permutes and gfx950 permlane swaps; no LDS
//      crossbar round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over each row of 16 lanes, result in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return v;
}
__device__ __forceinline__ float row16_min(float v) {
    v = fminf(v, dpp_mov<0xB1>(v));
    v = fminf(v, dpp_mov<0x4E>(v));
    v = fminf(v, dpp_mov<0x141>(v));
    v = fminf(v, dpp_mov<0x140>(v));
    return v;
}
// value held by lane l ^ 16 (neighbouring row) and by lane l ^ 32 (other half-wave)
__device__ __forceinline__ uint32_t lane_xor16(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((__lane_id() >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() >= 32) ? r[0] : r[1];
}
__device__ __forceinline__ float wave64_sum(float v) {
    v = row16_sum(v);
    v += __uint_as_float(lane_xor16(__float_as_uint(v)));
    v += __uint_as_float(lane_xor32(__float_as_uint(v)));
    return v;
}
__device__ __forceinline__ float wave64_max(float v) {
    v = row16_max(v);
    v = fmaxf(v, __uint_as_float(lane_xor16(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(lane_xor32(__float_as_uint(v))));
    return v;
}

// Launch descriptors filled by the host layer (qjl_api.hip) and consumed by the kernels.
struct KeyQuantArgs {
    const void* K;
    int64_t sKb, sKt, sKh;           // element strides
    const void* S_in;
    const void* S_out;
    const int32_t* oidx;
    uint32_t* bits;
    uint16_t* norms;
    int64_t T, Ncap, t0;
    int Hkv, m, m_out, n_out, W;
    int tokens_per_block;            // multiple of 32
};

// Value codes live in tiles of kCodeTile consecutive positions: for each channel, the codes of the
// tile's tokens as an LSB-first bit stream of nbits 32-bit words.
constexpr int kCodeTile = 32;
__host__ __device__ constexpr int64_t code_tiles(int64_t Ncap) { return (Ncap + kCodeTile - 1) / kCodeTile; }

struct ValueQuantArgs {
    const void* V;
    int64_t sVb, sVt, sVh;
    uint32_t* codes;                 // [B*Hkv][code_tiles(Ncap)][kD][nbits]
    uint16_t* meta;
    int64_t T, Ncap, t0;
    int B, Hkv, nbits;
};

struct DecodeArgs {
    const void* Q;
    const void* S_in;
    const void* S_out;
    const int32_t* oidx;
    const uint32_t* bits;
    const uint16_t* norms;
    const uint32_t* codes;            // 2-bit code tiles [B*Hkv][code_tiles(Ncap)][kD][2]
    const uint16_t* meta;
    const float* V_f32;
    float* out;
    float* scores_dbg;
    float* sq;                        // workspace: projected queries [B*Hq][m + m_out]
    float* part;                      // workspace: partials [B*Hq][nsplit][d + 2]
    int64_t N, Ncap;
    int B, Hq, Hkv, g, m, m_out, n_out, nsplit;
    int64_t chunk;                    // tokens per split (multiple of the tile)
    float z_scale;                    // sm_scale * log2(e)
};

// Kernel ids of the launch timer.
enum TimedKernel { TK_QUANT_KEYS = 0, TK_QUANT_VALUES, TK_QPROJ, TK_DECODE, TK_COMBINE, TK_COUNT };

// Host-side launchers (defined next to their kernels). They return hipSuccess or the launch error.
hipError_t launch_quantize_keys_bf16(const KeyQuantArgs& a, int B, hipStream_t s);
hipError_t launch_quantize_keys_f32(const KeyQuantArgs& a, int B, hipStream_t s);
hipError_t launch_quantize_values(const ValueQuantArgs& a, int vdt, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int qdt, int vmode, hipStream_t s);

// Decode geometry shared by the workspace-size query and the launcher.
constexpr int kDecodeTile = 512;     // tokens per tile = threads per decode block
int decode_pick_nsplit(int B, int Hkv, int g, int64_t N, int m, int m_out);
int64_t decode_chunk(int64_t N, int nsplit);

// Launch timer hooks (no-ops unless enabled).
void timer_begin(TimedKernel k, hipStream_t s);
void timer_end(TimedKernel k, hipStream_t s);

}  // namespace qjl

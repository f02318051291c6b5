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

struct ValueQuantArgs {
    const void* V;
    int64_t sVb, sVt, sVh;
    uint8_t* codes;
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
    const uint8_t* codes;
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

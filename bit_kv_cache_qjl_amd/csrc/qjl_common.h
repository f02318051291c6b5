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

// Sign words of a token row: natural word w holds projections 32 w .. 32 w + 31 (inlier words
// 0 .. win-1, outlier words win .. win+wout-1).  The row is stored as 4 groups of (win + wout)/4
// words; group j holds inlier words j win/4 .. (j+1) win/4 - 1, then outlier words
// win + j wout/4 .. win + (j+1) wout/4 - 1 (win and wout multiples of 4).  One 4-, 8- or 16-byte load
// then gives each lane group of a matrix-core operand its inlier and outlier words.
__host__ __device__ constexpr int bits_slot(int w, int win, int wout) {
    return w < win ? (w / (win >> 2)) * ((win + wout) >> 2) + w % (win >> 2)
                   : ((w - win) / (wout >> 2)) * ((win + wout) >> 2) + (win >> 2) + (w - win) % (wout >> 2);
}
// natural word held by stored slot s (inverse of bits_slot)
__host__ __device__ constexpr int bits_word(int s, int win, int wout) {
    return (s % ((win + wout) >> 2)) < (win >> 2)
               ? (s / ((win + wout) >> 2)) * (win >> 2) + s % ((win + wout) >> 2)
               : win + (s / ((win + wout) >> 2)) * (wout >> 2) + (s % ((win + wout) >> 2)) - (win >> 2);
}

// Value codes live in tiles of kCodeTile consecutive positions: for each channel, the codes of the
// tile's tokens as an LSB-first bit stream of nbits 32-bit words.  The 128 channel streams of a tile
// are stored in the order slot p = 8 (c % 16) + c / 16 (channel c = 16 (p % 8) + p / 8), so the
// channels 16 cg + t (cg = 0..7) of one matrix-core column t are 8 consecutive streams.
constexpr int kCodeTile = 32;
__host__ __device__ constexpr int64_t code_tiles(int64_t Ncap) { return (Ncap + kCodeTile - 1) / kCodeTile; }
__host__ __device__ constexpr int code_slot(int c) { return 8 * (c & 15) + (c >> 4); }
__host__ __device__ constexpr int code_channel(int p) { return 16 * (p & 7) + (p >> 3); }

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
    float* sq;                        // workspace: projected queries [B*Hq][m + m_out] (table path), or
                                      // the matrix-core query operand, 4 (m + m_out) bytes per head
    float* qconst;                    // workspace: per-head constants [B*Hq][4] of the matrix-core path
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
// query operand + matrix-core decode kernel (partials only; launch_decode adds the merge)
hipError_t launch_decode_mfma(const DecodeArgs& a, int qdt, hipStream_t s);

// Decode geometry shared by the workspace-size query and the launcher.
constexpr int kDecodeTile = 512;     // tokens per tile = threads per decode block
constexpr int kMaxSplits = 4096;     // context chunks per (sequence, query head)
int decode_pick_nsplit(int B, int Hkv, int g, int64_t N, int m, int m_out);
int64_t decode_chunk(int64_t N, int nsplit);
// True when decode runs on the matrix-core path (2-bit value codes, W = (m + m_out)/32 <= 16).
bool decode_uses_mfma(int m, int m_out, int vmode, int nbits);
// Row groups of 4 query heads per matrix-core workgroup: 2 (8 heads) when a KV head serves more than 4.
__host__ __device__ constexpr int decode_mfma_rowgroups(int g) { return g > 4 ? 2 : 1; }

// Launch timer hooks (no-ops unless enabled).
void timer_begin(TimedKernel k, hipStream_t s);
void timer_end(TimedKernel k, hipStream_t s);

}  // namespace qjl

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
//      crossbar round trip).  The row permutes read lanes of the same row only, so bound_ctrl (zero for
//      invalid lanes) changes nothing and lets the compiler fold the move into the consuming instruction.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// sum over each row of 16 lanes, result in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    return v;
}
// max / min: the IEEE maximum and minimum (v_maximum3 / v_minimum3), which agree with fmaxf / fminf
// on non-NaN values and need no canonicalizing of the permuted operand
__device__ __forceinline__ float row16_max(float v) {
    v = __builtin_elementwise_maximum(v, dpp_mov<0xB1>(v));
    v = __builtin_elementwise_maximum(v, dpp_mov<0x4E>(v));
    v = __builtin_elementwise_maximum(v, dpp_mov<0x141>(v));
    v = __builtin_elementwise_maximum(v, dpp_mov<0x140>(v));
    return v;
}
__device__ __forceinline__ float row16_min(float v) {
    v = __builtin_elementwise_minimum(v, dpp_mov<0xB1>(v));
    v = __builtin_elementwise_minimum(v, dpp_mov<0x4E>(v));
    v = __builtin_elementwise_minimum(v, dpp_mov<0x141>(v));
    v = __builtin_elementwise_minimum(v, dpp_mov<0x140>(v));
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

// Raw buffer resource over [base, base + bytes): loads at or past the end return zero, which is how
// the kernels treat ragged ends (no branches, no clamped addresses).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---- per-token arithmetic of small appends, shared by the quantize kernels and the decode-step
//      append so that every path writes the same norms, codes and meta

// Eight bf16 channels c0 .. c0 + 7 of a key (kv), split into the inlier part (outlier channels
// zeroed) and the outlier part (the other channels zeroed), and the squares of each part added in
// channel order.  Bit i of om flags channel c0 + i as an outlier channel.
__device__ __forceinline__ void split_key8(uint4 kv, uint32_t om, uint4& kin, uint4& kout, float& ss_in, float& ss_out) {
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
    uint32_t wi[4], wo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = kw[q] & 0xFFFFu, hi = kw[q] >> 16;
        const float flo = __uint_as_float(lo << 16), fhi = __uint_as_float(hi << 16);
        const bool olo = (om >> (2 * q)) & 1u, ohi = (om >> (2 * q + 1)) & 1u;
        if (olo) ss_out = fmaf(flo, flo, ss_out); else ss_in = fmaf(flo, flo, ss_in);
        if (ohi) ss_out = fmaf(fhi, fhi, ss_out); else ss_in = fmaf(fhi, fhi, ss_in);
        wi[q] = (olo ? 0u : lo) | ((ohi ? 0u : hi) << 16);
        wo[q] = (olo ? lo : 0u) | ((ohi ? hi : 0u) << 16);
    }
    kin = make_uint4(wi[0], wi[1], wi[2], wi[3]);
    kout = make_uint4(wo[0], wo[1], wo[2], wo[3]);
}

// (|k_in|, |k_out|) as IEEE binary16 (round to nearest even) in one word, from the sums of squares
__device__ __forceinline__ uint32_t norm_pair(float ss_in, float ss_out) {
    const _Float16 ni = (_Float16)sqrtf(ss_in);
    const _Float16 no = (_Float16)sqrtf(ss_out);
    return (uint32_t)__builtin_bit_cast(uint16_t, ni) | ((uint32_t)__builtin_bit_cast(uint16_t, no) << 16);
}

__device__ __forceinline__ float row8_max(float v) {
    v = __builtin_elementwise_maximum(v, dpp_mov<0xB1>(v));
    v = __builtin_elementwise_maximum(v, dpp_mov<0x4E>(v));
    v = __builtin_elementwise_maximum(v, dpp_mov<0x141>(v));
    return v;
}
__device__ __forceinline__ float row8_min(float v) {
    v = __builtin_elementwise_minimum(v, dpp_mov<0xB1>(v));
    v = __builtin_elementwise_minimum(v, dpp_mov<0x4E>(v));
    v = __builtin_elementwise_minimum(v, dpp_mov<0x141>(v));
    return v;
}

// Token-wise quantization of one value vector held by 128 / NV consecutive lanes (16 or 8, aligned),
// NV channels per lane (v): min and max over those lanes, step = fp16((max - min) / L),
// mn16 = fp16(min), and the codes clamp(rint((v - mn16) / step), 0, L) of the lane's channels (all 0
// when step is 0).  IEEE fp32 operations with no contraction.  Returns the meta word
// (mn16 | step16 << 16).
// The quotient x / step is first taken as y = x * rcp(step) (v_rcp_f32, within 1 ulp; the product
// rounded: y is within 2^-22 |y| of the exact quotient, the correctly rounded quotient within 2^-24),
// so for |y| <= L + 1 rint(y) is the code unless y lies within 2^-20 (L + 2) of a half-integer (beyond
// that range both quotients clamp to the same code).  A lane with such a value takes the correctly
// rounded divides for all its values (one branch, rarely entered).  A step of 0 gives a reciprocal of
// 0, so every code is 0 without a branch.
template <int NBITS, int NV>
__device__ __forceinline__ uint32_t value_codes(const float (&v)[NV], uint32_t (&code)[NV]) {
#pragma clang fp contract(off)
    static_assert(NV == 8 || NV == 16, "a vector of 128 channels over 16 or 8 lanes");
    // IEEE minimum / maximum (three-input instructions, no canonicalizing), in any order: exact
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int q = 1; q + 1 < NV; q += 2) {
        mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, v[q]), v[q + 1]);
        mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, v[q]), v[q + 1]);
    }
    mn = __builtin_elementwise_minimum(mn, v[NV - 1]);
    mx = __builtin_elementwise_maximum(mx, v[NV - 1]);
    if constexpr (NV == 8) {
        mn = row16_min(mn);
        mx = row16_max(mx);
    } else {
        mn = row8_min(mn);
        mx = row8_max(mx);
    }
    constexpr int L = (1 << NBITS) - 1;
    // fp16(fl32((mx - mn) / L)): the product with fl32(1 / L) is within 3 fp32 ulps of the correctly
    // rounded quotient, so both round to the same fp16 unless their 13 dropped bits lie within 4 of
    // the halfway pattern 0x1000, or the step is below the fp16 normal range; then divide.
    const float rng = mx - mn;
    float stepf = rng * (1.0f / (float)L);
    const uint32_t dropped = __float_as_uint(stepf) & 0x1FFFu;
    if (stepf < 0x1p-14f || (dropped >= 0x1000u - 4u && dropped <= 0x1000u + 4u)) stepf = rng / (float)L;
    const _Float16 step16 = (_Float16)stepf;
    const _Float16 mn16 = (_Float16)mn;
    const float step = (float)step16;
    const float base = (float)mn16;
    const float rstep = step != 0.f ? __builtin_amdgcn_rcpf(step) : 0.f;
    // y = v rstep + (1/2 - base rstep) in two fused multiply-adds approximates Q + 1/2, with Q the
    // recipe's fl(fl(v - base) / step); the code is rint(Q) = floor(Q + 1/2) clamped to [0, L] unless Q
    // is a tie.  Over the quotients that decide a code (0 <= Q <= L), |y - (Q + 1/2)| is below
    // 2^-21 (L + 2 + |base rstep|): the two roundings of Q and the one-ulp reciprocal scale with Q, the
    // offset's rounding with |base rstep|, the last fma's with |y|.  Outside twice that margin of an
    // integer, floor(y) is the code; within it (exact ties: bf16 values over an fp16 step land on them
    // often enough that some lane of a wave has one about every other wave) the quotient is recomputed
    // with the divide, one value at a time, each behind a branch of its own.
    const float off = fmaf(-base, rstep, 0.5f);
    const float marg = 0x1p-20f * ((float)(L + 2) + fabsf(base * rstep));
    float y[NV], f[NV];
    float fmin = 1.f, fmax = 0.f;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        y[q] = fmaf(v[q], rstep, off);
        f[q] = __builtin_amdgcn_fractf(y[q]);
        fmin = __builtin_elementwise_minimum(fmin, f[q]);
        fmax = __builtin_elementwise_maximum(fmax, f[q]);
    }
    if (fmin <= marg || fmax >= 1.f - marg) {
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            if (f[q] <= marg || f[q] >= 1.f - marg) {
                asm volatile("");                // keeps the divide behind its branch
                y[q] = rintf((v[q] - base) / step) + 0.5f;
            }
        }
    }
    // floor of y clamped to [0, L + 1/2] (med3 of values that are never NaN: no canonicalizing)
#pragma unroll
    for (int q = 0; q < NV; ++q) code[q] = (uint32_t)__builtin_amdgcn_fmed3f(y[q], 0.f, (float)L + 0.5f);
    return (uint32_t)__builtin_bit_cast(uint16_t, mn16) | ((uint32_t)__builtin_bit_cast(uint16_t, step16) << 16);
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
// Field of token j (0..31) in a channel stream: fields are nbits wide, LSB first.  2-bit streams are
// in token order; a 4-bit stream holds in word w the tokens 16 (w / 2) + 2 e + (w % 2) (nibble e), so
// the two 2-bit planes of each word follow the token order of a 2-bit stream.  3-bit streams are two
// planes instead: words 0 and 1 hold the low two bits of every code where a 2-bit stream holds its
// code (field j), word 2 the high bits, token j at bit hi3_bit(j); then nibble n of
// (word 2 >> k) & 0x11111111 belongs to the same token as nibble n of the k-th 2-bit plane word
// (word 0 & 0x33333333, (word 0 >> 2) & .., word 1 & .., (word 1 >> 2) & ..).
__host__ __device__ constexpr int code_field(int j, int nbits) {
    return nbits == 4 ? 8 * (2 * (j >> 4) + (j & 1)) + ((j & 15) >> 1) : j;
}
__host__ __device__ constexpr int hi3_bit(int j) { return 4 * ((j & 15) >> 1) + 2 * (j >> 4) + (j & 1); }
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
    const uint32_t* codes;            // code tiles [B*Hkv][code_tiles(Ncap)][kD][nbits]
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
    int nbits;                        // value code width (2, 3 or 4 on the matrix-core path)
    int64_t chunk;                    // tokens per split (multiple of the tile)
    float z_scale;                    // sm_scale * log2(e)
    int estimator;                    // 0: one-sided (query unquantized); 1: two-sided (query signs)
    int path;                         // qjl_decode_path: 0 auto, 1 matrix cores, 2 vector units
    size_t ws_need;                   // workspace bytes these sizes need (host-side check)
};

// The new token of a decode step (one per sequence, bf16, model layout) and the cache it goes to.
struct AppendArgs {
    const uint16_t* K;
    int64_t sKb, sKh;                 // element strides of the new keys
    const uint16_t* V;
    int64_t sVb, sVh;                 // element strides of the new values
    uint32_t* bits;
    uint16_t* norms;
    uint32_t* codes;                  // 2-, 3- or 4-bit code tiles
    uint16_t* meta;
    int64_t pos;                      // cache position of the new token (N - 1)
};

// Outlier-channel selection over prefill keys (model layout, element strides).
struct OutlierArgs {
    const void* K;
    int64_t sKb, sKt, sKh;
    double* partial;                  // workspace: per-channel sums [B * token blocks][Hkv][kD]
    int32_t* outlier_idx;             // [Hkv][n_out]
    int64_t T;
    int64_t tokens_per_block;
    int Hkv, n_out;
};

// Kernel ids of the launch timer.
enum TimedKernel { TK_QUANT_KEYS = 0, TK_QUANT_VALUES, TK_QPROJ, TK_DECODE, TK_COMBINE, TK_STEP, TK_SELECT, TK_COUNT };

// Host-side launchers (defined next to their kernels). They return hipSuccess or the launch error.
hipError_t launch_quantize_keys_bf16(const KeyQuantArgs& a, int B, hipStream_t s);
// True when bf16 keys of this sketch shape take the kernel that keeps the JL matrices in LDS
// (m and m_out in {0, 128, 256, 512} with m_out in {0, m}; one workgroup per CU).
inline bool quantize_keys_lds_shape(int m, int m_out) {
    return (m == 128 || m == 256 || m == 512) && (m_out == 0 || m_out == m);
}
hipError_t launch_quantize_keys_f32(const KeyQuantArgs& a, int B, hipStream_t s);
hipError_t launch_quantize_values(const ValueQuantArgs& a, int vdt, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int qdt, int vmode, hipStream_t s);
// query operand + matrix-core decode kernel + split merge
hipError_t launch_decode_mfma(const DecodeArgs& a, int qdt, hipStream_t s);
// decode step on the matrix-core path: append of the new token + query operand in one launch, then
// the decode kernel and the split merge
hipError_t launch_decode_step_mfma(const DecodeArgs& a, const AppendArgs& ap, hipStream_t s);
// log-sum-exp merge of the chunk partials into out
hipError_t launch_combine(const DecodeArgs& a, hipStream_t s);
// outlier-channel selection (kdt 0: bf16 keys, 1: fp32) and its token blocks per (sequence, head)
hipError_t launch_select_outliers(const OutlierArgs& a, int B, int kdt, hipStream_t s);
int64_t outlier_token_blocks(int B, int64_t T, int Hkv);

// Decode geometry shared by the workspace-size query and the launcher.
constexpr int kDecodeTile = 512;     // tokens per tile = threads per decode block
constexpr int kMaxSplits = 4096;     // context chunks per (sequence, query head)
int decode_pick_nsplit(int B, int Hkv, int g, int64_t N, int m, int m_out);
int64_t decode_chunk(int64_t N, int nsplit);
// True when decode runs on the matrix-core path (2-, 3- or 4-bit value codes, W = (m + m_out)/32 <= 16).
bool decode_uses_mfma(int m, int m_out, int vmode, int nbits);
// Row groups of 4 query heads per matrix-core workgroup: 2 (8 heads) when a KV head serves more than 4.
__host__ __device__ constexpr int decode_mfma_rowgroups(int g) { return g > 4 ? 2 : 1; }

// Launch timer hooks (no-ops unless enabled).
void timer_begin(TimedKernel k, hipStream_t s);
void timer_end(TimedKernel k, hipStream_t s);

}  // namespace qjl

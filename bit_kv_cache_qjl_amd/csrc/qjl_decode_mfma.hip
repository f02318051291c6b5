// Decode attention on the matrix cores: estimator scores and the value aggregation of up to four
// query heads per instruction.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero Overhead",
// "Approach" (asymmetric estimator sqrt(pi/2)/m * |k| * <S q, sign(S k)> with the query projected
// unquantized) and softmax attention over the estimated scores with the dequantized values ("Your
// Brain Already Runs on 1-Bit Keys", "Keys Select. Values Deliver.").
//
// Scores on v_mfma_scale_f32_16x16x128_f8f6f4 (A fp6 e2m3, B fp4 e2m1; with no 8-bit operand the
// instruction is faster: the fp8 x fp4 form takes 1.2x the time under full load): 16 tokens x 4 query heads per
// instruction, 128 sign positions of one kind (inlier or outlier) per instruction.
//   B (sign bits): with b = 1 for a non-negative projection, a 32-bit sign word x gives four fp4
//     operand words, one instruction each: x & 0x11111111, x & 0x22222222, x & 0x44444444 (nibble n
//     holds bit 4n + i with the value 0.5 b, b, 2 b: e2m1 0001, 0010, 0100) and
//     (x & 0x88888888) | 0x11111111 (e2m1 0001 or 1001: the value 0.5 - b of bit 4n + 3).
//   A (query): x_k = 2 z_scale sqrt(pi/2)/m (S q)_k divided by its plane's bit coefficient (0.5, 1,
//     2, -1), split into four e2m3 pieces, each with its own power of two per 32 K indices (the
//     E8M0 scale a lane supplies for its slice of the operand, 2^(s0 - 4 piece)); rows = (query
//     head, piece).  After four pieces a value's error is at most 2^(s0 - 16), below 2^-17.9 of the
//     largest magnitude of its 32-value slice.
//   sign = 2b - 1, so <S q, sign> = 2 <S q, b> - sum (S q).  The plane-3 positions contribute
//     x_k b_k - x_k / 2 by themselves; the accumulator starts at -sum x_k / 2 over the other
//     positions, so z = |k_in| D_in + |k_out| D_out is the token's base-2 softmax logit.
// Values on the same instruction: rows = (query head, piece) of the weight p * step, columns = 16
// channels, K = 128 tokens; B = the 2-bit codes of a code tile as x & 0x33333333 and
// (x >> 2) & 0x33333333 (e2m1 nibble 00cc = code / 2); 4-bit codes as their two 2-bit planes, the
// high one through a B scale of 4.  The weights of a 128-token block are scaled
// by 2^(8 - E), 2^E > the block's largest step, split into three e4m3 pieces, and transposed to the
// A-operand order through LDS.  Each wave is an independent online-softmax stream over 128-token
// blocks; the waves of a workgroup merge at the end of the chunk.  Two kernels: decode_mfma_kernel
// (four waves, each streaming its blocks through registers; one or two row groups of four heads) and,
// for more than four heads per KV head with 2-bit values, decode_mfma8_kernel (eight waves, two per
// SIMD, block data staged through LDS by LDS-destination loads, score rows holding piece pairs of all
// eight heads).
#include <math.h>

#include "qjl_decode_common.h"

namespace qjl {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef short v2s_t __attribute__((ext_vector_type(2)));

constexpr int kMThreads = 256;               // 4 waves
constexpr int kMWaves = kMThreads / 64;
constexpr int kMBlock = 128;                 // tokens per wave step
constexpr int kWPitch = 144;                 // bytes per row of a wave's weight tile (16-byte aligned;
                                             // rows of different heads land on different LDS banks)
// cache policy of the loads that stream the cache (sign words, norms, meta, codes): non-temporal,
// each byte is read once per launch (measured 4-5% faster on the Llama-2 and Llama-3 decodes)
constexpr int kStream = 2;

// 4 fp8 e4m3 bytes: a, b in the low half-word and c, d in the high one, rounded to nearest even
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)r, true);
}
// The three e4m3 pieces of 4 values v: k[0] = e4m3(v), k[1] = e4m3(16 r1), k[2] = e4m3(256 r2), with
// r1 = v - k[0] and r2 = r1 - k[1] / 16 exact in fp32, so v = k[0] + k[1] / 16 + k[2] / 256 + residual.
// The scaled conversions of gfx950 divide by the scale's power of two before rounding and multiply by
// it after decoding, two values per instruction.
__device__ __forceinline__ void fp8_pieces(const float (&v)[4], uint32_t (&k)[3]) {
    k[0] = fp8x4(v[0], v[1], v[2], v[3]);
    v2f_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)k[0], 1.0f, false);
    v2f_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)k[0], 1.0f, true);
    float r0 = v[0] - lo[0], r1 = v[1] - lo[1], r2 = v[2] - hi[0], r3 = v[3] - hi[1];
    v2s_t q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s_t{0, 0}, r0, r1, 0.0625f, false);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q, r2, r3, 0.0625f, true);
    k[1] = (uint32_t)(uint16_t)q[0] | ((uint32_t)(uint16_t)q[1] << 16);
    lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)k[1], 0.0625f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)k[1], 0.0625f, true);
    r0 -= lo[0]; r1 -= lo[1]; r2 -= hi[0]; r3 -= hi[1];
    q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s_t{0, 0}, r0, r1, 0.00390625f, false);
    q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q, r2, r3, 0.00390625f, true);
    k[2] = (uint32_t)(uint16_t)q[0] | ((uint32_t)(uint16_t)q[1] << 16);
}

// The four fp4 operand words of a sign word (plane i = bit 4n + i of x in nibble n).  m8 and o1 hold
// 0x88888888 and 0x11111111 in VGPRs (VOP3 takes no literals), so the last word is one v_and_or_b32;
// the code stays plain C, so the compiler sees every instruction that feeds the matrix core and
// inserts its wait states.
__device__ __forceinline__ v8i_t sign_planes(uint32_t x, uint32_t m8, uint32_t o1) {
    return v8i_t{(int)(x & 0x11111111u), (int)(x & 0x22222222u), (int)(x & 0x44444444u),
                 (int)((x & m8) | o1), 0, 0, 0, 0};
}

// Score instruction: A = the query operand (fp6 e2m3) with the E8M0 scale in byte kb of sc, B = a
// sign plane (fp4 e2m1).  The byte select is an instruction field, so kb is a constant once the
// caller's loop over K blocks is unrolled.
template <int KB>
__device__ __forceinline__ v4f_t mfma_query_kb(const v8i_t& qa, const v8i_t& sb, v4f_t acc, int sc) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, sb, acc, 2, 4, KB, sc, 0, 127);
}
__device__ __forceinline__ v4f_t mfma_query(int kb, const v8i_t& qa, const v8i_t& sb, v4f_t acc, int sc) {
    switch (kb) {
        case 0: return mfma_query_kb<0>(qa, sb, acc, sc);
        case 1: return mfma_query_kb<1>(qa, sb, acc, sc);
        case 2: return mfma_query_kb<2>(qa, sb, acc, sc);
        default: return mfma_query_kb<3>(qa, sb, acc, sc);
    }
}

// ---------------------------------------------------------------------------- query operand
// The smallest power-of-two exponent s with mx <= 7.5 2^s (0 for mx = 0), at least -126 (a normal
// fp32 scale for the conversions, a valid E8M0 byte for the instruction).
__device__ __forceinline__ int e2m3_scale_exp(float mx) {
    if (!(mx > 0.f)) return 0;
    const int e = __builtin_amdgcn_frexp_expf(mx);                // mx = f 2^e, f in [0.5, 1)
    const int s = __builtin_amdgcn_frexp_mantf(mx) <= 0.9375f ? e - 3 : e - 2;
    return s < -126 ? -126 : s;
}

// The matrix-core operand of a query head from its projections x_j = 2 z_scale sqrt(pi/2)/m (S q)_j
// (inlier j < m, then outlier, natural order, in LDS; for the two-sided estimator
// x_j = 2 z_scale |q_part|/m sign((S q)_j) instead).  One lane per 32-value slice: a row of 16 lanes
// (one DPP row) serves one head, lane slice = 4 kb + ga covers lane group ga of K block kb (one
// instruction's 128 K indices; lane group ga supplies K indices 32 ga .. 32 ga + 31, which pair with
// the sign word of B lane group ga: K index 32 ga + j is bit 4 (j % 8) + j / 8 of that word, plane
// j / 8).  The 32 values of a slice are one sign word's projections, divided by their plane's bit
// coefficient (0.5, 1, 2, -1) and split into four fp6 e2m3 pieces: piece p is the residual after
// pieces 0 .. p-1 at the power of two 2^(s0 - 4 p) (the instruction's E8M0 scale of that lane),
// where 2^s0 takes the slice's largest magnitude into (3.75, 7.5].  The residual after piece p is at
// most 2^(s0 - 2), 2^(s0 - 7), 2^(s0 - 12) (half a step of e2m3 at the piece's largest scaled value
// 7.5, 4, 2), so the next piece's scaled values are at most 4, 2, 1, and the error after the four
// pieces is at most 2^(s0 - 16).  The pieces come from gfx950's packed conversions (32 values in one
// instruction, nearest even; element 2i from the first source's i, 2i + 1 from the second's).
// Output, per K block: [piece][lane group][8 words] = the 32 e2m3 codes packed from bit 0 (6 words),
// the E8M0 byte 127 + s (word 6) and a zero word; then the per-head constants [-sum x_in / 2,
// -sum x_out / 2 (both over the positions outside plane 3), 0, 0] (written by the lane of slice 0).
// Every lane of the row takes part (the sums are DPP row reductions); active is uniform per row.
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef float v32f_t __attribute__((ext_vector_type(32)));
typedef uint32_t v6u_t __attribute__((ext_vector_type(6)));
__device__ void query_operand_slices(const float* xs, int win4, int wout4, int slice, bool active, uint32_t* dst,
                                     float* qc) {
    const int W4 = win4 + wout4;
    const int kb = slice >> 2, ga = slice & 3;
    const bool live = active && slice < 4 * W4;
    const bool out = kb >= win4;
    const int word = out ? 4 * win4 + ga * wout4 + (kb - win4) : ga * win4 + kb;
    float x[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 v = live ? reinterpret_cast<const float4*>(xs + 32 * word)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
    // position 4 n + plane; plane-3 positions carry their own -x/2 and stay out of the sums
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q)
        if ((q & 3) != 3) part += x[q];
    const float s_in = row16_sum(out ? 0.f : part), s_out = row16_sum(out ? part : 0.f);
    if (active && slice == 0) {
        qc[0] = -0.5f * s_in;
        qc[1] = -0.5f * s_out;
        qc[2] = 0.f;
        qc[3] = 0.f;
    }
    // K order j = 8 plane + n: element 2 i of the slice in ev[i], 2 i + 1 in od[i]
    v16f_t ev, od;
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const int plane = j >> 3, n = j & 7;
        const float v = x[4 * n + plane] * (plane == 0 ? 2.f : (plane == 1 ? 1.f : (plane == 2 ? 0.5f : -1.f)));
        mx = fmaxf(mx, fabsf(v));
        if (j & 1) od[j >> 1] = v;
        else ev[j >> 1] = v;
    }
    const int s0 = e2m3_scale_exp(mx);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int sc = s0 - 4 * p < -126 ? -126 : s0 - 4 * p;
        const float scale = ldexpf(1.f, sc);
        const v6u_t pk = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, scale);
        // the sources (and the scale) stay live across each conversion, so its destination cannot share
        // their registers (the compiler would otherwise allow it, and the conversions read their
        // sources after writing part of the destination)
        asm volatile("" :: "v"(ev), "v"(od), "v"(scale));
        const v32f_t d = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(pk, scale);
        asm volatile("" :: "v"(pk), "v"(scale));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            ev[i] -= d[2 * i];                   // exact: the piece holds the leading bits of the residual
            od[i] -= d[2 * i + 1];
        }
        if (live) {
            uint4* o = reinterpret_cast<uint4*>(dst + kb * 128 + p * 32 + ga * 8);
            o[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            o[1] = make_uint4(pk[4], pk[5], (uint32_t)(127 + sc), 0u);
        }
    }
}

// fp32 queries and JL matrices: one workgroup per (sequence, query head), S q in fp32 on the VALU in
// channel order, then the operand (wave 0).
__global__ __launch_bounds__(256) void qproj_f32_kernel(DecodeArgs a, int win4, int wout4) {
    __shared__ float qin[kD];
    __shared__ float qo[kMaxOutliers];
    __shared__ int so[kMaxOutliers];
    __shared__ __attribute__((aligned(16))) float xs[kMaxBits];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int hq = bh % a.Hq;
    const int h = hq / a.g;
    const float* Q = static_cast<const float*>(a.Q);
    if (tid < a.n_out) so[tid] = a.oidx[h * a.n_out + tid] & (kD - 1);   // never index outside a row
    if (tid < kD) qin[tid] = Q[(size_t)bh * kD + tid];
    __syncthreads();
    if (tid < a.n_out) qo[tid] = qin[so[tid]];
    __syncthreads();
    if (tid < a.n_out) qin[so[tid]] = 0.f;
    __syncthreads();
    const float* Sin = static_cast<const float*>(a.S_in);
    const float* Sout = static_cast<const float*>(a.S_out);
    // two-sided estimator: the sign of each projection times the norm of the query part (sign(0) = +1)
    const bool two = a.estimator != 0;
    float qn_in = 0.f, qn_out = 0.f;
    if (two) {
        for (int c = 0; c < kD; ++c) qn_in = fmaf(qin[c], qin[c], qn_in);
        for (int i = 0; i < a.n_out; ++i) qn_out = fmaf(qo[i], qo[i], qn_out);
        qn_in = sqrtf(qn_in);
        qn_out = sqrtf(qn_out);
    }
    const float c_in = 2.f * a.z_scale * (two ? qn_in : kSqrtHalfPi) / (float)a.m;
    for (int j = tid; j < a.m; j += 256) {
        const float p = row_dot(Sin + (size_t)j * kD, qin);
        xs[j] = two ? (p >= 0.f ? c_in : -c_in) : p * c_in;
    }
    if (a.m_out) {
        const float c_out = 2.f * a.z_scale * (two ? qn_out : kSqrtHalfPi) / (float)a.m_out;
        for (int j = tid; j < a.m_out; j += 256) {
            float acc = 0.f;
            for (int i = 0; i < a.n_out; ++i) acc = fmaf(Sout[(size_t)j * kD + so[i]], qo[i], acc);
            xs[a.m + j] = two ? (acc >= 0.f ? c_out : -c_out) : acc * c_out;
        }
    }
    __syncthreads();
    if (tid < 64)
        query_operand_slices(xs, win4, wout4, tid & 15, tid < 16,
                             reinterpret_cast<uint32_t*>(a.sq) + (size_t)bh * (128 * (win4 + wout4)), a.qconst + (size_t)bh * 4);
}

// ---------------------------------------------------------------------------- query projection (bf16)
constexpr int kVRow = kD + 8;                // LDS row of a staged vector (bf16), 272 B
constexpr int kMaxMfmaBits = 512;            // m + m_out on the matrix-core path
constexpr int kXPitch = kMaxMfmaBits + 4;    // LDS row of a head's projections (floats)

// LDS of the projection phase: the staged vectors (outlier channels zeroed / outlier channels only),
// their projections, the KV head's outlier mask and the vectors' part norms (two-sided estimator).
struct ProjLds {
    __attribute__((aligned(16))) uint16_t vin[16 * kVRow];
    __attribute__((aligned(16))) uint16_t vout[16 * kVRow];
    __attribute__((aligned(16))) float xs[16 * kXPitch];
    uint32_t mask[4];
    float qn[16][2];
};

// The new value of a decode step (sequence, KV head vunit) into its code tile and meta at ap.pos: one
// wave, a row of 16 lanes with 8 channels per lane; the 2- or 4-bit fields are merged into the tile
// words with atomic and/or (the rest of the tile is kept), 3-bit codes into their two planes.
__device__ __forceinline__ void append_value(const DecodeArgs& a, const AppendArgs& ap, int vunit, int lane) {
    const int vb = vunit / a.Hkv, vh = vunit - vb * a.Hkv;
    uint4 vv = make_uint4(0u, 0u, 0u, 0u);
    if (lane < 16) vv = *reinterpret_cast<const uint4*>(ap.V + vb * ap.sVb + vh * ap.sVh + 8 * lane);
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
    float v[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
    const int nb = a.nbits;
    uint32_t code[8];
    const uint32_t mt = nb == 4 ? value_codes<4, 8>(v, code) : (nb == 3 ? value_codes<3, 8>(v, code) : value_codes<2, 8>(v, code));
    if (lane < 16) {
        if (lane == 0) reinterpret_cast<uint32_t*>(ap.meta)[(size_t)vunit * a.Ncap + ap.pos] = mt;
        const int64_t tile = ap.pos / kCodeTile;
        const int j = (int)(ap.pos % kCodeTile);
        // a 2- or 4-bit field never crosses a word; 3-bit codes: the low two bits at the 2-bit
        // field, the high bit in word 2 (two planes)
        const int bit = nb == 3 ? 2 * j : nb * code_field(j, nb);
        uint32_t* tw = ap.codes + ((size_t)vunit * code_tiles(a.Ncap) + tile) * (kD * nb);
        const int sh = bit & 31;
        const uint32_t fm = nb == 3 ? 3u : (1u << nb) - 1u;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint32_t* dst = tw + code_slot(8 * lane + q) * nb;
            atomicAnd(dst + (bit >> 5), ~(fm << sh));
            atomicOr(dst + (bit >> 5), (code[q] & fm) << sh);
            if (nb == 3) {
                atomicAnd(dst + 2, ~(1u << hi3_bit(j)));
                atomicOr(dst + 2, (code[q] >> 2) << hi3_bit(j));
            }
        }
    }
}

// One (sequence, KV head) on the matrix cores: D (16 vectors x 16 projections) = A (vectors x channels,
// from LDS) . B (S rows, straight from global memory), v_mfma_f32_16x16x32_bf16 (exact bf16 products,
// fp32 sums).  The vectors are the KV head's g query heads, preceded by the new key when app; the key's
// signs are the sign bits of its cache row (ballot of the D column), its norms are computed as in the
// quantize kernels.  Wave w < NPW owns sign words w WPW .. (w + 1) WPW - 1 (two 16-projection tiles per
// word), so WPW = W / NPW.  The query projections go to LDS, then one wave per head builds its operand
// at sq_dst + head (128 W/4) words and its constants at qc_dst + 4 head.  Threads 0..255 stage the
// vectors and build the operands; every thread of the workgroup calls this (it holds the workgroup's
// barriers).
template <int WPW, int NPW>
__device__ __forceinline__ void project_unit(const DecodeArgs& a, const AppendArgs& ap, int unit, bool app, ProjLds& L,
                                             uint32_t* sq_dst, float* qc_dst) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool worker = tid < 256;               // staging and operands
    const bool proj = wave < NPW;                // projections
    const int b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int Win = a.m >> 5, Wout = a.m_out >> 5, W = Win + Wout;
    const int win4 = a.m >> 7, wout4 = a.m_out >> 7;
    const int ncol = a.g + (app ? 1 : 0);
    const int64_t head0 = (int64_t)b * a.Hq + (int64_t)h * a.g;

    // ---- every global load that does not depend on another is issued first: the KV head's outlier
    //      channels (one entry per lane of wave 0) and the first pass's vectors, then this wave's S tiles
    //      (B operands: projection row 16 hf + lane % 16 of word wn, channels 32 s + 8 (lane / 16) ..).
    //      Loads complete in order for the wait counter, so in this order the mask and the staging below
    //      wait for their own loads while the S tiles are still in flight.
    // (the raw entry, read only after the S tiles are issued: arithmetic on it next to its load would
    // wait for the load there; the unused default is the lane index, not a constant that would let the
    // compiler fold the arithmetic into the load's branch)
    const bool has_oc = wave == 0 && lane < a.n_out;
    int oc_raw = lane;
    if (has_oc) oc_raw = a.oidx[h * a.n_out + lane];
    const int sv = (tid >> 4) & 15, cg = tid & 15;   // staging: vector sv of a pass, channels 8 cg .. 8 cg + 7
    auto load_vector = [&](int col) {
        if (!worker || col >= ncol) return make_uint4(0u, 0u, 0u, 0u);
        if (app && col == 0) return *reinterpret_cast<const uint4*>(ap.K + b * ap.sKb + h * ap.sKh + 8 * cg);
        return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Q) + (head0 + col - (app ? 1 : 0)) * kD + 8 * cg);
    };
    uint4 xv = load_vector(sv);
    uint4 sb[WPW][2][4];
#pragma unroll
    for (int u = 0; u < WPW; ++u) {
        const int wn = proj ? WPW * wave + u : 0;
        const uint16_t* S = wn < Win ? static_cast<const uint16_t*>(a.S_in) + (size_t)(32 * wn) * kD
                                     : static_cast<const uint16_t*>(a.S_out) + (size_t)(32 * (wn - Win)) * kD;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sb[u][hf][s] = proj ? *reinterpret_cast<const uint4*>(S + (size_t)(16 * hf + (lane & 15)) * kD + 32 * s + 8 * (lane >> 4))
                                      : make_uint4(0u, 0u, 0u, 0u);
    }
    if (wave == 0) {
        // outlier mask of the KV head (bit c % 32 of word c / 32): the LDS operations of a wave complete
        // in order, so the words are cleared before the entries set their bits
        if (lane < 4) L.mask[lane] = 0u;
        const int oc = oc_raw & (kD - 1);        // never index outside a row
        if (has_oc) atomicOr(&L.mask[oc >> 5], 1u << (oc & 31));
    }
    __syncthreads();

    const float c_in = 2.f * a.z_scale * kSqrtHalfPi / (float)a.m;
    const float c_out = a.m_out ? 2.f * a.z_scale * kSqrtHalfPi / (float)a.m_out : 0.f;
    const float c2_in = 2.f * a.z_scale / (float)a.m;
    const float c2_out = a.m_out ? 2.f * a.z_scale / (float)a.m_out : 0.f;
    // one pass per 16 vectors; the first pass is its own copy, so that its staging waits only for the
    // vector loaded before the S tiles (a wait at a join with later passes would wait for all loads)
    auto pass = [&](const int c0, const uint4 xv) {
        const bool key_pass = app && c0 == 0;
        // ---- stage 16 vectors, split at the outlier channels
        if (worker) {
            const uint32_t om = (L.mask[cg >> 2] >> (8 * (cg & 3))) & 0xFFu;
            uint4 xi, xo;
            float ss_in = 0.f, ss_out = 0.f;
            split_key8(xv, om, xi, xo, ss_in, ss_out);
            *reinterpret_cast<uint4*>(L.vin + sv * kVRow + 8 * cg) = xi;
            *reinterpret_cast<uint4*>(L.vout + sv * kVRow + 8 * cg) = xo;
            if (key_pass || a.estimator) {
                // squared norms of each vector's two parts: one DPP row of 16 lanes per vector
                ss_in = row16_sum(ss_in);
                ss_out = row16_sum(ss_out);
            }
            // the key is vector 0: lanes 0..15 of wave 0
            if (key_pass && tid == 0) reinterpret_cast<uint32_t*>(ap.norms)[(size_t)unit * a.Ncap + ap.pos] = norm_pair(ss_in, ss_out);
            if (a.estimator && cg == 0) {
                L.qn[sv][0] = sqrtf(ss_in);
                L.qn[sv][1] = sqrtf(ss_out);
            }
        }
        __syncthreads();

        // ---- projections: sign word wn = WPW wave + u is the pair of 16-projection tiles 2 wn, 2 wn + 1;
        //      D lane l holds projection 32 wn + 16 hf + l % 16 of vectors 4 (l / 16) + i
        if (proj) {
#pragma unroll
            for (int u = 0; u < WPW; ++u) {
                const int wn = WPW * wave + u;
                const bool inl = wn < Win;
                const uint16_t* vsrc = (inl ? L.vin : L.vout) + (lane & 15) * kVRow + 8 * (lane >> 4);
                uint32_t word = 0;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    v4f_t acc = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(vsrc + 32 * s)),
                                                                      __builtin_bit_cast(bf16x8_t, sb[u][hf][s]), acc, 0, 0, 0);
                    if (key_pass) word |= ((uint32_t)__builtin_amdgcn_ballot_w64(acc[0] >= 0.f) & 0xFFFFu) << (16 * hf);
                    const int j = (inl ? 32 * wn : a.m + 32 * (wn - Win)) + 16 * hf + (lane & 15);
                    const float cs = inl ? c_in : c_out;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int vec = 4 * (lane >> 4) + i;
                        // two-sided estimator: the projection's sign times the norm of the query part
                        const float t = a.estimator ? L.qn[vec][inl ? 0 : 1] * (inl ? c2_in : c2_out) : 0.f;
                        L.xs[vec * kXPitch + j] = a.estimator ? (acc[i] >= 0.f ? t : -t) : acc[i] * cs;
                    }
                }
                if (key_pass && lane == 0) ap.bits[((size_t)unit * a.Ncap + ap.pos) * W + bits_slot(wn, Win, Wout)] = word;
            }
        }
        __syncthreads();

        // ---- operands of this pass's query heads: wave w serves columns w, w + 4, w + 8, w + 12, one
        //      row of 16 lanes each
        if (worker) {
            const int v = wave + 4 * (lane >> 4);
            const int col = c0 + v;
            const bool active = col < ncol && !(app && col == 0);
            const int hl = active ? col - (app ? 1 : 0) : 0;
            query_operand_slices(L.xs + v * kXPitch, win4, wout4, lane & 15, active, sq_dst + hl * (128 * (win4 + wout4)),
                                 qc_dst + hl * 4);
        }
        __syncthreads();
    };
    pass(0, xv);
    for (int c0 = 16; c0 < ncol; c0 += 16) pass(c0, load_vector(c0 + sv));
}

// bf16: one workgroup per (sequence, KV head) projects the KV head's g query heads (and, for a decode
// step, the new key) into the workspace; for a decode step, workgroups of their own append the new
// values, one (sequence, KV head) per wave (their atomic round trips overlap the projections).
template <int WPW, bool APPEND>
__global__ __launch_bounds__(256) void prologue_kernel(DecodeArgs a, AppendArgs ap) {
    __shared__ ProjLds L;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nunits = a.B * a.Hkv;
    if (APPEND && (int)blockIdx.x >= nunits) {
        const int vunit = 4 * ((int)blockIdx.x - nunits) + wave;
        if (vunit >= nunits) return;
        append_value(a, ap, vunit, tid & 63);
        return;
    }
    const int unit = blockIdx.x;                 // b * Hkv + h
    const int b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int64_t head0 = (int64_t)b * a.Hq + (int64_t)h * a.g;
    project_unit<WPW, 4>(a, ap, unit, APPEND, L, reinterpret_cast<uint32_t*>(a.sq) + head0 * (128 * ((a.m + a.m_out) >> 7)),
                      a.qconst + head0 * 4);
}

// ---------------------------------------------------------------------------- decode
// Token of sub-step s (0..7) of a 128-token block in B column t, chosen so that the four sub-steps
// 4q..4q+3 of one column land on four consecutive bytes of the value operand (one 32-bit LDS store
// per piece): tau = 32 (2q + t3) + 16 t2 + 2 (4 t1 + i) + t0 for s = 4q + i, t = (t3 t2 t1 t0) in bits.
__device__ __forceinline__ int mfma_token(int s, int t) {
    return 32 * (2 * (s >> 2) + ((t >> 3) & 1)) + 16 * ((t >> 2) & 1) + 2 * (4 * ((t >> 1) & 1) + (s & 3)) + (t & 1);
}

// Token data of one 128-token block for one lane: the stored quarter-row (lane group hh) of the sign
// words of its token for each sub-step, the (norm, meta) pairs of tokens 2 lane and 2 lane + 1 (staged
// through LDS before use), and the NB code words of channels 16 cg + t in code tile s0/32 + hh.
template <int WIN4, int WOUT4, int NB>
struct MBlock {
    uint32_t w[8][WIN4 + WOUT4];
    uint32_t nm[4];
    uint32_t cx[8][NB];
};

// Per-lane parts of the block loads (the block start enters as a scalar offset).
struct MOffsets {
    int bits;    // sign quarter-row of sub-step 0
    int nm;      // (norm, meta) of tokens 2 lane, 2 lane + 1
    int codes;   // channel streams 8 t .. 8 t + 7 of code tile hh (2-bit codes: piece hh of stream group t)
};

template <int WIN4, int WOUT4, int NB>
__device__ __forceinline__ void load_mblock(MBlock<WIN4, WOUT4, NB>& bl, __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rn,
                                            __amdgpu_buffer_rsrc_t rm, __amdgpu_buffer_rsrc_t rc, const MOffsets& o, int s0) {
    constexpr int Q = WIN4 + WOUT4;              // words per quarter-row
    constexpr int WB = 4 * Q;
    // one address add per stream and block; the sub-step offsets are instruction immediates
    const int vb0 = o.bits + s0 * WB * 4;                       // sub-steps 0..3
    const int vb1 = vb0 + 64 * WB * 4;                          // sub-steps 4..7
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        // token of sub-step s = token of sub-step 0 + 64 (s / 4) + 2 (s % 4)
        const int voff = (s < 4 ? vb0 : vb1) + 2 * (s & 3) * WB * 4;
        if constexpr (Q == 1) {
            bl.w[s][0] = __builtin_amdgcn_raw_buffer_load_b32(rb, voff, 0, kStream);
        } else if constexpr (Q == 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(rb, voff, 0, kStream);
            bl.w[s][0] = x[0]; bl.w[s][1 % Q] = x[1];
        } else {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, kStream);
            bl.w[s][0] = x[0]; bl.w[s][1 % Q] = x[1]; bl.w[s][2 % Q] = x[2]; bl.w[s][3 % Q] = x[3];
        }
    }
    const int vn = o.nm + s0 * 4;
    const auto n2 = __builtin_amdgcn_raw_buffer_load_b64(rn, vn, 0, kStream);
    const auto m2 = __builtin_amdgcn_raw_buffer_load_b64(rm, vn, 0, kStream);
    bl.nm[0] = n2[0]; bl.nm[1] = m2[0]; bl.nm[2] = n2[1]; bl.nm[3] = m2[1];
    const int vc = o.codes + s0 * (kD * NB * 4 / kCodeTile);
    // the 8 channels' NB words each are 8 NB consecutive words: word 4 q + e is word (4 q + e) % NB of
    // channel group (4 q + e) / NB.  2-bit codes: load q is all of code tile q (lane 16 p + u: piece p of
    // stream group u), and transpose_code_pieces later hands each lane its own pieces
    // 3- and 4-bit codes keep the per-lane pieces, 96 or 128 bytes apart: each load takes 16 bytes of a line
    // whose other pieces follow in the next loads, so they are cached loads (non-temporal ones let the
    // lines go before those pieces arrive: 1.5x the time at 4 bits)
    constexpr int kCodePolicy = NB == 2 ? kStream : 0;
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rc, vc + (NB == 2 ? q * (kD * NB * 4) : 16 * q), 0, kCodePolicy);
#pragma unroll
        for (int e = 0; e < 4; ++e) bl.cx[(4 * q + e) / NB][(4 * q + e) % NB] = x[e];
    }
}

// 2-bit codes loaded a whole tile per load: lane row p (lanes 16 p ..) holds in load q's four words
// piece p of its stream group in tile q, which lane row q needs as its piece p.  Two exchange stages
// transpose the 4 x 4 (row, load) blocks: v_permlane32_swap swaps the upper two rows of one register
// with the lower two rows of another (row and load index exchange their high bits), v_permlane16_swap
// the odd rows of one with the even rows of another (the low bits).  Afterwards register group p of
// lane row hh is piece p of its stream group in tile hh, as the strided loads would have left it.
__device__ __forceinline__ void transpose_code_pieces(uint32_t (&cx)[8][2]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = cx[(4 * q + e) / 2][(4 * q + e) % 2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const auto x = __builtin_amdgcn_permlane32_swap(r[q], r[q + 2], false, false);
            r[q] = x[0];
            r[q + 2] = x[1];
        }
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
            const auto x = __builtin_amdgcn_permlane16_swap(r[q], r[q + 1], false, false);
            r[q] = x[0];
            r[q + 1] = x[1];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) cx[(4 * q + e) / 2][(4 * q + e) % 2] = r[q];
    }
}

// R = 1: one workgroup serves 4 query heads of a KV head; R = 2: 8 query heads as two row groups of
// the same instructions' B operands (the sign and code planes are built once for both).
// Two workgroups per CU for 4 query heads and 2-bit codes; one (the whole register file) otherwise.
// FUSED: as in the eight-wave kernel, the workgroup projects the KV head's query heads (g <= HPG: one
// head group) into LDS, and the workgroup whose chunk holds the new token (ap.pos; -1 for none)
// appends it first; no projection launch precedes the decode.
template <int WIN4, int WOUT4, int R, bool DBG, int NB, bool FUSED>
__global__ __launch_bounds__(kMThreads, (R == 1 && NB == 2) ? 2 : 1) void decode_mfma_kernel(DecodeArgs a, AppendArgs ap, int groups,
                                                                                             int hgroups) {
    constexpr int W4 = WIN4 + WOUT4;             // instructions (K blocks of 128 sign positions) per token
    constexpr int WB = 4 * W4;                   // sign words per token
    constexpr int HPG = 4 * R;                   // query heads per workgroup
    // projection phase (FUSED): ProjLds, the query operands (HPG x 128 W4 words), the per-head constants
    constexpr int PJ_BYTES = (int)sizeof(ProjLds) + HPG * 128 * W4 * 4 + HPG * 4 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t pj[FUSED ? PJ_BYTES : 16];
    uint32_t* const s_sq = reinterpret_cast<uint32_t*>(pj + sizeof(ProjLds));
    float* const s_qc = reinterpret_cast<float*>(pj + sizeof(ProjLds) + HPG * 128 * W4 * 4);
    __shared__ __attribute__((aligned(16))) uint8_t wtile[kMWaves][R][16 * kWPitch];   // weight pieces
    __shared__ __attribute__((aligned(16))) uint32_t nmt[kMWaves][2 * kMBlock];        // (norm, meta) per token
    __shared__ float red_m[kMWaves][HPG], red_l[kMWaves][HPG], red_mn[kMWaves][HPG];
    __shared__ __attribute__((aligned(16))) float red_o[kMWaves][HPG][kD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = lane & 15;                     // B column: token slot (scores) / channel (values)
    const int hh = lane >> 4;                    // lane group: D rows 4 hh .. 4 hh + 3 = head hh of a row group

    // XCD-aware placement: the head groups of one (KV head, chunk) run on one XCD (shared L2)
    const int lin = blockIdx.x;
    const int xcd = lin & 7;
    const int slot = lin >> 3;
    const int hg = slot % hgroups;
    const int64_t us = (int64_t)(slot / hgroups) * 8 + xcd;
    if (us >= (int64_t)groups) return;
    const int split = (int)(us % a.nsplit);
    const int unit = (int)(us / a.nsplit);       // b * Hkv + h
    const int b = unit / a.Hkv;
    const int h = unit - b * a.Hkv;
    const int t_begin = (int)((int64_t)split * a.chunk);
    const int t_end = (int)min(a.N, (int64_t)t_begin + a.chunk);
    const int head0 = b * a.Hq + h * a.g;        // (b, first query head of KV head h)
    if constexpr (FUSED) {
        // wave 3 appends the new value first when this chunk holds the new token; all four waves project
        const bool app = ap.pos >= t_begin && ap.pos < t_end;
        if (app && wave == 3) append_value(a, ap, unit, lane);
        project_unit<W4, 4>(a, ap, unit, app, *reinterpret_cast<ProjLds*>(pj), s_sq, s_qc);
        // the appended row is in memory before any load of this workgroup's blocks
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    const uint8_t* sq_base = FUSED ? reinterpret_cast<const uint8_t*>(s_sq)
                                   : reinterpret_cast<const uint8_t*>(a.sq) + (size_t)head0 * (128 * WB);
    const float* qc_base = FUSED ? s_qc : a.qconst + (size_t)head0 * 4;

    // ---- score A operands and scales: this lane's A row in row group rg is (head 4 rg + rh, piece pc),
    //      K slice hh
    const int rh = t >> 2, pc = lane & 3;
    v8i_t sA[R][W4];
    int sc[R];                                   // E8M0 scale of K block kb in byte kb
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const int qa_head = HPG * hg + 4 * rg + rh;
        sc[rg] = 0x7F7F7F7F;
        if (qa_head < a.g) {
            const uint4* src = reinterpret_cast<const uint4*>(sq_base + (size_t)qa_head * (128 * WB));
            uint32_t bytes = 0u;
#pragma unroll
            for (int kb = 0; kb < W4; ++kb) {
                const uint4 lo = src[kb * 32 + (pc * 4 + hh) * 2], hi = src[kb * 32 + (pc * 4 + hh) * 2 + 1];
                sA[rg][kb] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, 0, 0};
                bytes |= (hi.z & 0xFFu) << (8 * kb);
            }
            sc[rg] = (int)bytes;
        } else {
#pragma unroll
            for (int kb = 0; kb < W4; ++kb) sA[rg][kb] = v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    // ---- D-side constants: lane group hh is query head HPG hg + 4 rg + hh of the KV head
    float cin[R], cout[R];
    float* sdbg[R];
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const int dhead = HPG * hg + 4 * rg + hh;
        const bool ok = dhead < a.g;
        cin[rg] = ok ? qc_base[dhead * 4] : 0.f;
        cout[rg] = ok ? qc_base[dhead * 4 + 1] : 0.f;
        sdbg[rg] = (DBG && ok) ? a.scores_dbg + (size_t)(head0 + dhead) * a.N : nullptr;
    }

    // zero this wave's weight tiles once (the rows of piece 3 are never written again)
    uint8_t* wt = &wtile[wave][0][0];
    for (int i = lane; i < R * 16 * kWPitch / 16; i += 64) reinterpret_cast<uint4*>(wt)[i] = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();

    // this lane's byte offset in a weight tile for sub-steps 4q..4q+3 (row and 16 q added later)
    const int woff = 32 * (2 * ((t >> 3) & 1) + ((t >> 2) & 1)) + 8 * (t & 1) + 4 * ((t >> 1) & 1);

    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(a.bits + (size_t)unit * a.Ncap * WB, (uint32_t)t_end * WB * 4u);
    const __amdgpu_buffer_rsrc_t rn = buffer_rsrc(reinterpret_cast<const uint32_t*>(a.norms) + (size_t)unit * a.Ncap,
                                                  (uint32_t)t_end * 4u);
    const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(reinterpret_cast<const uint32_t*>(a.meta) + (size_t)unit * a.Ncap,
                                                  (uint32_t)t_end * 4u);
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(a.codes + (size_t)unit * code_tiles(a.Ncap) * (kD * NB),
                                                  (uint32_t)code_tiles(t_end) * (kD * NB * 4u));
    const MOffsets offs{(mfma_token(0, t) * WB + hh * W4) * 4, 8 * lane,
                        NB == 2 ? (8 * NB * 4) * t + 16 * hh : hh * (kD * NB * 4) + t * (8 * NB * 4)};
    const float inv_z = 1.0f / a.z_scale;

    float m_run[R], l_acc[R], mn_acc[R];
    v4f_t dv[R][8];
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        m_run[rg] = -INFINITY;
        l_acc[rg] = mn_acc[rg] = 0.f;
#pragma unroll
        for (int cg = 0; cg < 8; ++cg) dv[rg][cg] = v4f_t{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t* nmw = nmt[wave];
    // plane-3 masks in VGPRs; the empty asm only hides the constants from constant folding
    uint32_t m8 = 0x88888888u, o1 = 0x11111111u;
    asm volatile("" : "+v"(m8), "+v"(o1));

    // ---- one 128-token block
    auto process = [&](const MBlock<WIN4, WOUT4, NB>& cur, int s0) {
        // (norm, meta) of the block's tokens to LDS (the previous block's reads are done: LDS
        // operations of a wave complete in order)
        *reinterpret_cast<uint4*>(nmw + 4 * lane) = make_uint4(cur.nm[0], cur.nm[1], cur.nm[2], cur.nm[3]);
        __builtin_amdgcn_wave_barrier();
        uint32_t nrm[8], mt[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint2 v = *reinterpret_cast<const uint2*>(nmw + 2 * mfma_token(s, t));
            nrm[s] = v.x;
            mt[s] = v.y;
        }

        // scores (base-2 logits) of the 8 sub-steps
        float z[R][8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float n_in = (float)__builtin_bit_cast(_Float16, (uint16_t)(nrm[s] & 0xFFFFu));
            const float n_out = (float)__builtin_bit_cast(_Float16, (uint16_t)(nrm[s] >> 16));
            v8i_t bin[WIN4], bout[WOUT4 > 0 ? WOUT4 : 1];
#pragma unroll
            for (int kb = 0; kb < WIN4; ++kb) bin[kb] = sign_planes(cur.w[s][kb], m8, o1);
#pragma unroll
            for (int kb = 0; kb < WOUT4; ++kb) bout[kb] = sign_planes(cur.w[s][WIN4 + kb], m8, o1);
#pragma unroll
            for (int rg = 0; rg < R; ++rg) {
                v4f_t din = v4f_t{cin[rg], 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < WIN4; ++kb)
                    din = mfma_query(kb, sA[rg][kb], bin[kb], din, sc[rg]);
                float zz = n_in * ((din[0] + din[1]) + (din[2] + din[3]));
                if constexpr (WOUT4 > 0) {
                    v4f_t dout = v4f_t{cout[rg], 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < WOUT4; ++kb)
                        dout = mfma_query(WIN4 + kb, sA[rg][WIN4 + kb], bout[kb], dout, sc[rg]);
                    zz = fmaf(n_out, (dout[0] + dout[1]) + (dout[2] + dout[3]), zz);
                }
                if constexpr (DBG) {
                    const int P = s0 + mfma_token(s, t);
                    if (sdbg[rg] && P < t_end) sdbg[rg][P] = zz * inv_z;
                }
                z[rg][s] = zz;
            }
        }
        if (s0 + kMBlock > t_end) {
            // the chunk's last block: tokens past its end take no part in the softmax
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bool past = s0 + mfma_token(s, t) >= t_end;
#pragma unroll
                for (int rg = 0; rg < R; ++rg) z[rg][s] = past ? -INFINITY : z[rg][s];
            }
        }

        // step scale of the block (shared by the row groups): every step of the block < 2^E
        float mxs = 0.f, stp[8], mnv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            mnv[s] = (float)__builtin_bit_cast(_Float16, (uint16_t)(mt[s] & 0xFFFFu));
            stp[s] = (float)__builtin_bit_cast(_Float16, (uint16_t)(mt[s] >> 16));
            mxs = fmaxf(mxs, stp[s]);
        }
        mxs = row16_max(mxs);
        const int E = mxs > 0.f ? __builtin_amdgcn_frexp_expf(mxs) : 0;
        float stpf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) stpf[s] = ldexpf(stp[s], 8 - E);
        bool rescale = false;
        float alpha[R];

        // online softmax per row group (per head = per row of 16 lanes), weights to the LDS tile
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            float mx = z[rg][0];
#pragma unroll
            for (int s = 1; s < 8; ++s) mx = fmaxf(mx, z[rg][s]);
            mx = row16_max(mx);
            const float m_new = fmaxf(m_run[rg], mx);    // finite: token s0 of the block is valid
            alpha[rg] = __builtin_amdgcn_exp2f(m_run[rg] - m_new);
            rescale |= alpha[rg] != 1.f;
            m_run[rg] = m_new;
            l_acc[rg] *= alpha[rg];
            mn_acc[rg] *= alpha[rg];
            uint8_t* row0 = wt + rg * 16 * kWPitch + (4 * hh) * kWPitch + woff;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 4 * q + i;
                    const float p = __builtin_amdgcn_exp2f(z[rg][s] - m_new);
                    l_acc[rg] += p;
                    mn_acc[rg] = fmaf(p, mnv[s], mn_acc[rg]);
                    w[i] = p * stpf[s];                   // in [0, 256)
                }
                uint32_t k[3];
                fp8_pieces(w, k);
                uint8_t* row = row0 + 16 * q;
                *reinterpret_cast<uint32_t*>(row) = k[0];
                *reinterpret_cast<uint32_t*>(row + kWPitch) = k[1];
                *reinterpret_cast<uint32_t*>(row + 2 * kWPitch) = k[2];
            }
        }
        if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
            for (int rg = 0; rg < R; ++rg)
#pragma unroll
                for (int cg = 0; cg < 8; ++cg) dv[rg][cg] *= alpha[rg];
        }
        __builtin_amdgcn_wave_barrier();   // the weight tiles written above are read across lanes below

        // values: A = weight pieces (row t = (head, piece), K slice hh), B = code tile hh (built once)
        v8i_t aw[R];
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            const uint8_t* src = wt + rg * 16 * kWPitch + t * kWPitch + 32 * hh;
            const uint4 alo = *reinterpret_cast<const uint4*>(src);
            const uint4 ahi = *reinterpret_cast<const uint4*>(src + 16);
            aw[rg] = v8i_t{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
        }
        const int sc_w = 120 + E - 4 * pc;   // 2^(E - 8 - 4 piece), times 2 for the nibble = code / 2
        uint32_t cx2[8][2];
        if constexpr (NB == 2) {
#pragma unroll
            for (int cg = 0; cg < 8; ++cg) {
                cx2[cg][0] = cur.cx[cg][0];
                cx2[cg][1] = cur.cx[cg][1 % NB];
            }
            transpose_code_pieces(cx2);
        }
#pragma unroll
        for (int cg = 0; cg < 8; ++cg) {
            if constexpr (NB == 2) {
                const uint32_t x0 = cx2[cg][0], x1 = cx2[cg][1];
                const v8i_t bv = v8i_t{(int)(x0 & 0x33333333u), (int)((x0 >> 2) & 0x33333333u), (int)(x1 & 0x33333333u),
                                       (int)((x1 >> 2) & 0x33333333u), 0, 0, 0, 0};
#pragma unroll
                for (int rg = 0; rg < R; ++rg)
                    dv[rg][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[rg], bv, dv[rg][cg], 0, 4, 0, sc_w, 0, 127);
            } else if constexpr (NB == 3) {
                // 3-bit codes: the 2-bit planes of words 0 and 1 as above, the high bits of word 2 as
                // four 1-bit planes in the same token order; code = low + 4 high (B scale 2^2)
                const uint32_t x0 = cur.cx[cg][0], x1 = cur.cx[cg][1 % NB], hb = cur.cx[cg][2 % NB];
                const v8i_t blo = v8i_t{(int)(x0 & 0x33333333u), (int)((x0 >> 2) & 0x33333333u), (int)(x1 & 0x33333333u),
                                        (int)((x1 >> 2) & 0x33333333u), 0, 0, 0, 0};
                const v8i_t bhi = v8i_t{(int)(hb & 0x11111111u), (int)((hb >> 1) & 0x11111111u),
                                        (int)((hb >> 2) & 0x11111111u), (int)((hb >> 3) & 0x11111111u), 0, 0, 0, 0};
#pragma unroll
                for (int rg = 0; rg < R; ++rg) {
                    dv[rg][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[rg], blo, dv[rg][cg], 0, 4, 0, sc_w, 0, 127);
                    dv[rg][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[rg], bhi, dv[rg][cg], 0, 4, 0, sc_w, 0, 129);
                }
            } else {
                // 4-bit codes: word w holds the same tokens in its two 2-bit planes as the 2-bit
                // planes above; code = low + 4 high, the high plane through a B scale of 2^2
                const uint32_t x0 = cur.cx[cg][0], x1 = cur.cx[cg][1 % NB], x2 = cur.cx[cg][2 % NB], x3 = cur.cx[cg][3 % NB];
                const v8i_t blo = v8i_t{(int)(x0 & 0x33333333u), (int)(x1 & 0x33333333u), (int)(x2 & 0x33333333u),
                                        (int)(x3 & 0x33333333u), 0, 0, 0, 0};
                const v8i_t bhi = v8i_t{(int)((x0 >> 2) & 0x33333333u), (int)((x1 >> 2) & 0x33333333u),
                                        (int)((x2 >> 2) & 0x33333333u), (int)((x3 >> 2) & 0x33333333u), 0, 0, 0, 0};
#pragma unroll
                for (int rg = 0; rg < R; ++rg) {
                    dv[rg][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[rg], blo, dv[rg][cg], 0, 4, 0, sc_w, 0, 127);
                    dv[rg][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[rg], bhi, dv[rg][cg], 0, 4, 0, sc_w, 0, 129);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();   // the next block rewrites the weight tiles
    };

    // ---- the block loop, software-pipelined over two buffers: block i + 1 is in flight while block i
    //      is computed (loads past the chunk end fall outside the buffer ranges and return zeros)
    constexpr int kStep = kMBlock * kMWaves;
    MBlock<WIN4, WOUT4, NB> ba, bb;
    const int s_first = t_begin + kMBlock * wave;
    load_mblock(ba, rb, rn, rm, rc, offs, s_first);
    for (int s0 = s_first; s0 < t_end; s0 += 2 * kStep) {
        load_mblock(bb, rb, rn, rm, rc, offs, s0 + kStep);
        process(ba, s0);
        if (s0 + kStep >= t_end) break;
        load_mblock(ba, rb, rn, rm, rc, offs, s0 + 2 * kStep);
        process(bb, s0 + kStep);
    }

    // ---- merge the four wave streams of each head
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const float l_sum = row16_sum(l_acc[rg]), mn_sum = row16_sum(mn_acc[rg]);
        if (t == 0) {
            red_m[wave][4 * rg + hh] = m_run[rg];
            red_l[wave][4 * rg + hh] = l_sum;
            red_mn[wave][4 * rg + hh] = mn_sum;
        }
#pragma unroll
        for (int cg = 0; cg < 8; ++cg) red_o[wave][4 * rg + hh][16 * cg + t] = (dv[rg][cg][0] + dv[rg][cg][1]) + dv[rg][cg][2];
    }
    __syncthreads();
    const int c0 = 2 * (tid & 63);           // channels c0, c0 + 1
    for (int oh = tid >> 6; oh < HPG; oh += kMWaves) {
        if (HPG * hg + oh >= a.g) break;
        float M = red_m[0][oh];
#pragma unroll
        for (int w = 1; w < kMWaves; ++w) M = fmaxf(M, red_m[w][oh]);
        float L = 0.f, o0 = 0.f, o1 = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kMWaves; ++w) {
                const float mw = red_m[w][oh];
                if (mw == -INFINITY) continue;
                const float sc = exp2f(mw - M);
                L = fmaf(sc, red_l[w][oh], L);
                o0 = fmaf(sc, red_o[w][oh][c0] + red_mn[w][oh], o0);
                o1 = fmaf(sc, red_o[w][oh][c0 + 1] + red_mn[w][oh], o1);
            }
        }
        if (a.nsplit == 1) {                 // the whole context: the output itself (no merge launch)
            float* o = a.out + (size_t)(head0 + HPG * hg + oh) * kD;
            o[c0] = L > 0.f ? o0 / L : 0.f;
            o[c0 + 1] = L > 0.f ? o1 / L : 0.f;
            continue;
        }
        float* dst = a.part + ((size_t)(head0 + HPG * hg + oh) * a.nsplit + split) * (kD + 2);
        dst[2 + c0] = o0;
        dst[3 + c0] = o1;
        if ((tid & 63) == 0) {
            dst[0] = M;
            dst[1] = L;
        }
    }

}

// ---------------------------------------------------------------------------- eight-wave decode
// The same computation for 8 query heads per workgroup (two row groups) and 2-bit codes, with eight
// waves, two per SIMD: one wave's vector instructions run while the other's matrix instructions do.
// Registers allow that only without the two block buffers of decode_mfma_kernel, so a block's sign
// quarter-rows, norms, meta and code words go from HBM straight into LDS (buffer loads with the LDS as
// destination), one buffer per wave (norms and meta two), and are read from there when used:
//   after the weight-tile stores of block i:  sign quarter-rows, norms and meta of block i + 1 (8 + 4 loads);
//   after the values of block i:              code words of block i + 1 (4 loads).
// Loads complete in issue order, so block i + 1 may start once at most the 4 code loads are
// outstanding (vmcnt 4), and its values once at most the 12 loads issued after its weight stores are
// (vmcnt 12).  These loads write no register, so the waits are explicit; the empty asm statements
// that carry them also make the buffers escape, so the compiler does not take their contents as
// never written.  Tokens past the chunk end read as zero (buffer bounds) and are masked as before.
constexpr int kM8Waves = 8;
constexpr int kM8Threads = 64 * kM8Waves;

// 16 or 4 bytes per lane from a buffer into LDS (lane l at byte 16 l, or 4 l, of the destination), in
// plain functions: with the size inside a kernel template the compiler's host pass drops the
// kernel's launch stub
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, kStream);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, uint32_t* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, 0, 0, kStream);
}

typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));

// The LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// The (norm, meta) words of this lane's token in each of the eight sub-steps of a staged block: token
// mfma_token(s, t) sits f(s) = 64 (s / 4) + 2 (s % 4) words after that of sub-step 0, the meta words 128
// words after the norms.  The reads are waited for in the same statement.  They go through asm because
// the compiler cannot tell this buffer from those that the block's code loads are still writing, and
// would otherwise wait for every outstanding load (those of the next code words included) first; the
// caller has waited for the loads into this buffer.
__device__ __forceinline__ void read_nm8(uint32_t addr, v2u_t (&nm)[8]) {
    asm volatile(
        "ds_read2_b32 %0, %8 offset0:0 offset1:128\n\t"
        "ds_read2_b32 %1, %8 offset0:2 offset1:130\n\t"
        "ds_read2_b32 %2, %8 offset0:4 offset1:132\n\t"
        "ds_read2_b32 %3, %8 offset0:6 offset1:134\n\t"
        "ds_read2_b32 %4, %8 offset0:64 offset1:192\n\t"
        "ds_read2_b32 %5, %8 offset0:66 offset1:194\n\t"
        "ds_read2_b32 %6, %8 offset0:68 offset1:196\n\t"
        "ds_read2_b32 %7, %8 offset0:70 offset1:198\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(nm[0]), "=&v"(nm[1]), "=&v"(nm[2]), "=&v"(nm[3]), "=&v"(nm[4]), "=&v"(nm[5]), "=&v"(nm[6]), "=&v"(nm[7])
        : "v"(addr)
        : "memory");
}

// The three e4m3 piece words of a weight quadruple into rows r, r + 1, r + 2 of a wave's weight tile.
// Through asm for the same reason as read_nm8: the tile is not written by any load, but the compiler
// would wait for every outstanding load into LDS before a store it can see.  The stores are in order
// with the wave's later LDS reads of the tile.
static_assert(kWPitch == 144, "row offsets of store_pieces");
__device__ __forceinline__ void store_pieces(uint32_t addr, const uint32_t (&k)[3]) {
    asm volatile(
        "ds_write_b32 %0, %1\n\t"
        "ds_write_b32 %0, %2 offset:144\n\t"
        "ds_write_b32 %0, %3 offset:288"
        :
        : "v"(addr), "v"(k[0]), "v"(k[1]), "v"(k[2])
        : "memory");
}

// FUSED: the workgroup projects its query heads itself (the KV head's g <= 8 heads: one head group),
// into LDS, and the workgroup whose chunk holds the new token of a decode step (ap.pos; -1 for none)
// appends it to the cache first; no projection launch precedes the decode.
template <int WIN4, int WOUT4, bool DBG, bool FUSED>
__global__ __launch_bounds__(kM8Threads, 1) void decode_mfma8_kernel(DecodeArgs a, AppendArgs ap, int groups, int hgroups) {
    constexpr int R = 2, NB = 2;
    constexpr int W4 = WIN4 + WOUT4;
    constexpr int WB = 4 * W4;
    constexpr int HPG = 4 * R;
    static_assert(W4 == 1 || W4 == 4, "a sign quarter-row of 4 or 16 bytes: one LDS-destination load");
    // projection phase (FUSED): ProjLds, then the query operands (HPG x 128 W4 words) and the per-head
    // constants (HPG x 4); with 16-byte sign quarter-rows it lies over the sign buffers, which the
    // block loads fill only after it
    constexpr bool PJ_OVER = W4 == 4;
    constexpr int PJ_BYTES = (int)sizeof(ProjLds) + HPG * 128 * W4 * 4 + HPG * 4 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t s_pj[(FUSED && !PJ_OVER) ? PJ_BYTES : 16];
    // separate arrays, so that the compiler's own wait analysis can tell the load destinations apart
    __shared__ __attribute__((aligned(16))) uint8_t s_wtile[kM8Waves][2][16 * kWPitch];   // weight pieces
    __shared__ __attribute__((aligned(16))) uint32_t s_sgn[kM8Waves][8][64][W4];         // sign quarter-rows
    __shared__ __attribute__((aligned(16))) uint32_t s_cod[kM8Waves][4][64][4];          // code words
    __shared__ __attribute__((aligned(16))) uint32_t s_nm[kM8Waves][2][2][kMBlock];      // [buffer][norm, meta][token]
    __shared__ float s_red_m[kM8Waves][8], s_red_l[kM8Waves][8], s_red_mn[kM8Waves][8];
    static_assert(!FUSED || !PJ_OVER || sizeof(s_sgn) >= PJ_BYTES, "the projection phase fits the sign buffers");
    uint8_t* const pj = PJ_OVER ? reinterpret_cast<uint8_t*>(&s_sgn[0][0][0][0]) : s_pj;
    uint32_t* const s_sq = reinterpret_cast<uint32_t*>(pj + sizeof(ProjLds));
    float* const s_qc = reinterpret_cast<float*>(pj + sizeof(ProjLds) + HPG * 128 * W4 * 4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = lane & 15;
    const int hh = lane >> 4;

    const int lin = blockIdx.x;
    const int xcd = lin & 7;
    const int slot = lin >> 3;
    const int hg = slot % hgroups;
    const int64_t us = (int64_t)(slot / hgroups) * 8 + xcd;
    if (us >= (int64_t)groups) return;
    const int split = (int)(us % a.nsplit);
    const int unit = (int)(us / a.nsplit);
    const int b = unit / a.Hkv;
    const int h = unit - b * a.Hkv;
    const int t_begin = (int)((int64_t)split * a.chunk);
    const int t_end = (int)min(a.N, (int64_t)t_begin + a.chunk);
    const int head0 = b * a.Hq + h * a.g;
    if constexpr (FUSED) {
        // wave 4 appends the new value while waves 0..3 project (the key first, when this chunk holds it)
        const bool app = ap.pos >= t_begin && ap.pos < t_end;
        if (app && wave == 4) append_value(a, ap, unit, lane);
        // eight projecting waves for 16 sign words per token (half the S tiles per wave), four for 4
        project_unit<W4 == 4 ? 2 : 1, W4 == 4 ? 8 : 4>(a, ap, unit, app, *reinterpret_cast<ProjLds*>(pj), s_sq, s_qc);
        // the appended row is in memory before any load of this workgroup's blocks
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    const uint8_t* sq_base = FUSED ? reinterpret_cast<const uint8_t*>(s_sq)
                                   : reinterpret_cast<const uint8_t*>(a.sq) + (size_t)head0 * (128 * WB);
    const float* qc_base = FUSED ? s_qc : a.qconst + (size_t)head0 * 4;

    // ---- score operands: A row t of both instructions is (head t / 2, slot t % 2) of the eight heads;
    //      instruction pp carries piece 2 pp + slot, and both accumulate into the same rows, so D row
    //      (head, slot) ends with pieces slot and 2 + slot summed.  Lane group hh then holds the rows of
    //      heads 2 hh and 2 hh + 1 (the score heads of the lane, index j); its value rows stay those of
    //      heads hh and 4 + hh (row group rg of the value instructions).
    const int ah = t >> 1, aslot = t & 1;
    const int pc = lane & 3;                     // value instructions: A row t is (head t / 4, piece t % 4)
    v8i_t sA[2][W4];
    int sc[2];                                   // E8M0 scale of K block kb in byte kb
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
        const int qa_head = HPG * hg + ah;
        const int piece = 2 * pp + aslot;
        sc[pp] = 0x7F7F7F7F;
        if (qa_head < a.g) {
            const uint4* src = reinterpret_cast<const uint4*>(sq_base + (size_t)qa_head * (128 * WB));
            uint32_t bytes = 0u;
#pragma unroll
            for (int kb = 0; kb < W4; ++kb) {
                const uint4 lo = src[kb * 32 + (piece * 4 + hh) * 2], hi = src[kb * 32 + (piece * 4 + hh) * 2 + 1];
                sA[pp][kb] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, 0, 0};
                bytes |= (hi.z & 0xFFu) << (8 * kb);
            }
            sc[pp] = (int)bytes;
        } else {
#pragma unroll
            for (int kb = 0; kb < W4; ++kb) sA[pp][kb] = v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    float cin[2], cout[2];
    float* sdbg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int dhead = HPG * hg + 2 * hh + j;
        const bool ok = dhead < a.g;
        cin[j] = ok ? qc_base[dhead * 4] : 0.f;
        cout[j] = ok ? qc_base[dhead * 4 + 1] : 0.f;
        sdbg[j] = (DBG && ok) ? a.scores_dbg + (size_t)(head0 + dhead) * a.N : nullptr;
    }
    // every wave has its operands in registers before any block load writes over the projection phase
    if constexpr (FUSED) __syncthreads();
    // the lane group whose score heads include value head 4 rg + hh, as a ds_bpermute byte address
    const int perm_addr[2] = {4 * (16 * (hh >> 1) + t), 4 * (16 * (2 + (hh >> 1)) + t)};

    uint8_t* wt = &s_wtile[wave][0][0];
    for (int i = lane; i < R * 16 * kWPitch / 16; i += 64) reinterpret_cast<uint4*>(wt)[i] = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    const int woff = 32 * (2 * ((t >> 3) & 1) + ((t >> 2) & 1)) + 8 * (t & 1) + 4 * ((t >> 1) & 1);

    const uint32_t* bits_u = a.bits + (size_t)unit * a.Ncap * WB;
    const uint32_t* norms_u = reinterpret_cast<const uint32_t*>(a.norms) + (size_t)unit * a.Ncap;
    const uint32_t* meta_u = reinterpret_cast<const uint32_t*>(a.meta) + (size_t)unit * a.Ncap;
    const uint32_t* codes_u = a.codes + (size_t)unit * code_tiles(a.Ncap) * (kD * NB);
    const int off_bits = (mfma_token(0, t) * WB + hh * W4) * 4;        // sign quarter-row of sub-step 0
    // code words: lane (t, hh) needs the 64 bytes of channel streams 8 t .. of code tile hh, as four
    // 16-byte pieces.  Load q brings in all of tile q, 1 KB, so every cache line is whole within one load:
    // its lane 16 p + u reads piece p of stream group u, which lands at slot 16 p + u of buffer q (for a
    // given piece the 16 lanes of a lane group then read 16 consecutive slots, without bank conflicts)
    const int off_codes = (8 * NB * 4) * (lane & 15) + 16 * (lane >> 4);
    const float inv_z = 1.0f / a.z_scale;

    // the loads of a block into this wave's LDS buffers.  The block start s0 is wave-uniform: each
    // block gets buffer descriptors based at its first token (scalar work), sized to the tokens left
    // before t_end (none once s0 >= t_end: every load returns zeros), so the lane offsets stay the same
    // from block to block and no vector instruction computes an address.
    auto load_signs_nm = [&](int s0, int nb) {
        const uint32_t left = s0 < t_end ? (uint32_t)(t_end - s0) : 0u;
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(bits_u + (size_t)s0 * WB, left * WB * 4u);
        const __amdgpu_buffer_rsrc_t rn = buffer_rsrc(norms_u + s0, left * 4u);
        const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(meta_u + s0, left * 4u);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int voff = off_bits + (64 * (s >> 2) + 2 * (s & 3)) * WB * 4;
            if constexpr (W4 == 4) lds_load16(rb, &s_sgn[wave][s][0][0], voff);
            else lds_load4(rb, &s_sgn[wave][s][0][0], voff);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            lds_load4(rn, &s_nm[wave][nb][0][64 * q], (64 * q + lane) * 4);
            lds_load4(rm, &s_nm[wave][nb][1][64 * q], (64 * q + lane) * 4);
        }
    };
    auto load_codes = [&](int s0) {
        // s0 is a multiple of the block, so the block starts a code tile
        const int tile0 = s0 / kCodeTile, tiles = code_tiles(t_end);
        const uint32_t left = tile0 < tiles ? (uint32_t)(tiles - tile0) : 0u;
        const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(codes_u + (size_t)tile0 * (kD * NB), left * (kD * NB * 4u));
#pragma unroll
        for (int q = 0; q < 2 * NB; ++q) lds_load16(rc, &s_cod[wave][q][0][0], off_codes + q * (kD * NB * 4));
    };

    float m_run[R], l_acc[R], mn_acc[R];
    v4f_t dv[R][8];
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        m_run[rg] = -INFINITY;
        l_acc[rg] = mn_acc[rg] = 0.f;
#pragma unroll
        for (int cg = 0; cg < 8; ++cg) dv[rg][cg] = v4f_t{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t m8 = 0x88888888u, o1 = 0x11111111u;
    asm volatile("" : "+v"(m8), "+v"(o1));

    constexpr int kStep = kMBlock * kM8Waves;
    const int s_first = t_begin + kMBlock * wave;
    int nb = 0;
    load_signs_nm(s_first, nb);
    load_codes(s_first);
    for (int s0 = s_first; s0 < t_end; s0 += kStep) {
        // this block's sign quarter-rows, norms and meta have landed (only the 4 code loads may be pending)
        if constexpr (DBG) asm volatile("s_waitcnt vmcnt(0)" ::"s"(s_sgn), "s"(s_cod), "s"(s_nm) : "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::"s"(s_sgn), "s"(s_cod), "s"(s_nm) : "memory");
        __builtin_amdgcn_wave_barrier();

        float z[R][8];
        uint32_t mtw[8];                               // meta of the 8 sub-steps, read before its buffer is reloaded
        v2u_t nmw[8];
        read_nm8(lds_addr(&s_nm[wave][nb][0][mfma_token(0, t)]), nmw);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            mtw[s] = nmw[s][1];
            const uint32_t nrm = nmw[s][0];
            const float n_in = (float)__builtin_bit_cast(_Float16, (uint16_t)(nrm & 0xFFFFu));
            const float n_out = (float)__builtin_bit_cast(_Float16, (uint16_t)(nrm >> 16));
            uint32_t w[W4];
            if constexpr (W4 == 4) {
                const uint4 x = *reinterpret_cast<const uint4*>(&s_sgn[wave][s][lane][0]);
                w[0] = x.x; w[1 % W4] = x.y; w[2 % W4] = x.z; w[3 % W4] = x.w;
            } else {
                w[0] = s_sgn[wave][s][lane][0];
            }
            v8i_t bin[WIN4], bout[WOUT4 > 0 ? WOUT4 : 1];
#pragma unroll
            for (int kb = 0; kb < WIN4; ++kb) bin[kb] = sign_planes(w[kb], m8, o1);
#pragma unroll
            for (int kb = 0; kb < WOUT4; ++kb) bout[kb] = sign_planes(w[WIN4 + kb], m8, o1);
            v4f_t din = v4f_t{cin[0], 0.f, cin[1], 0.f};
#pragma unroll
            for (int kb = 0; kb < WIN4; ++kb) {
                din = mfma_query(kb, sA[0][kb], bin[kb], din, sc[0]);
                din = mfma_query(kb, sA[1][kb], bin[kb], din, sc[1]);
            }
            float zz[2] = {n_in * (din[0] + din[1]), n_in * (din[2] + din[3])};
            if constexpr (WOUT4 > 0) {
                v4f_t dout = v4f_t{cout[0], 0.f, cout[1], 0.f};
#pragma unroll
                for (int kb = 0; kb < WOUT4; ++kb) {
                    dout = mfma_query(WIN4 + kb, sA[0][WIN4 + kb], bout[kb], dout, sc[0]);
                    dout = mfma_query(WIN4 + kb, sA[1][WIN4 + kb], bout[kb], dout, sc[1]);
                }
                zz[0] = fmaf(n_out, dout[0] + dout[1], zz[0]);
                zz[1] = fmaf(n_out, dout[2] + dout[3], zz[1]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (DBG) {
                    const int P = s0 + mfma_token(s, t);
                    if (sdbg[j] && P < t_end) sdbg[j][P] = zz[j] * inv_z;
                }
                z[j][s] = zz[j];
            }
        }
        if (s0 + kMBlock > t_end) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bool past = s0 + mfma_token(s, t) >= t_end;
#pragma unroll
                for (int rg = 0; rg < R; ++rg) z[rg][s] = past ? -INFINITY : z[rg][s];
            }
        }

        float mxs = 0.f, stp[8], mnv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t mt = mtw[s];
            mnv[s] = (float)__builtin_bit_cast(_Float16, (uint16_t)(mt & 0xFFFFu));
            stp[s] = (float)__builtin_bit_cast(_Float16, (uint16_t)(mt >> 16));
            mxs = fmaxf(mxs, stp[s]);
        }
        mxs = row16_max(mxs);
        const int E = mxs > 0.f ? __builtin_amdgcn_frexp_expf(mxs) : 0;
        float stpf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) stpf[s] = ldexpf(stp[s], 8 - E);
        bool rescale = false;
        float alpha[R];
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            float mx = z[rg][0];
#pragma unroll
            for (int s = 1; s < 8; ++s) mx = fmaxf(mx, z[rg][s]);
            mx = row16_max(mx);
            const float m_new = fmaxf(m_run[rg], mx);
            alpha[rg] = __builtin_amdgcn_exp2f(m_run[rg] - m_new);
            rescale |= alpha[rg] != 1.f;
            m_run[rg] = m_new;
            l_acc[rg] *= alpha[rg];
            mn_acc[rg] *= alpha[rg];
            // score head 2 hh + rg: value row group hh / 2, rows 4 (2 (hh % 2) + rg) ..
            uint8_t* row0 = wt + (hh >> 1) * 16 * kWPitch + (4 * (2 * (hh & 1) + rg)) * kWPitch + woff;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float wgt[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 4 * q + i;
                    const float p = __builtin_amdgcn_exp2f(z[rg][s] - m_new);
                    l_acc[rg] += p;
                    mn_acc[rg] = fmaf(p, mnv[s], mn_acc[rg]);
                    wgt[i] = p * stpf[s];
                }
                uint32_t k[3];
                fp8_pieces(wgt, k);
                store_pieces(lds_addr(row0 + 16 * q), k);
            }
        }
        // the sign buffer is free once its reads are done: the next block's signs, norms and meta.  Issued
        // after this block's LDS stores (the weight tiles above): the compiler waits for every load into
        // LDS before an LDS store, whatever its address
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        load_signs_nm(s0 + kStep, nb ^ 1);
        if (__builtin_amdgcn_ballot_w64(rescale)) {
            // the value rows of head 4 rg + hh take that head's factor from the lane group scoring it
            // (slot hh % 2 of group 2 rg + hh / 2)
#pragma unroll
            for (int rg = 0; rg < R; ++rg) {
                const float f0 = __int_as_float(__builtin_amdgcn_ds_bpermute(perm_addr[rg], __float_as_int(alpha[0])));
                const float f1 = __int_as_float(__builtin_amdgcn_ds_bpermute(perm_addr[rg], __float_as_int(alpha[1])));
                const float av = (hh & 1) ? f1 : f0;
#pragma unroll
                for (int cg = 0; cg < 8; ++cg) dv[rg][cg] *= av;
            }
        }
        // this block's code words have landed (the 12 loads issued after the weight stores may be pending)
        if constexpr (DBG) asm volatile("s_waitcnt vmcnt(0)" ::"s"(s_sgn), "s"(s_cod), "s"(s_nm) : "memory");
        else asm volatile("s_waitcnt vmcnt(12)" ::"s"(s_sgn), "s"(s_cod), "s"(s_nm) : "memory");
        __builtin_amdgcn_wave_barrier();

        v8i_t aw[R];
#pragma unroll
        for (int rg = 0; rg < R; ++rg) {
            const uint8_t* src = wt + rg * 16 * kWPitch + t * kWPitch + 32 * hh;
            const uint4 alo = *reinterpret_cast<const uint4*>(src);
            const uint4 ahi = *reinterpret_cast<const uint4*>(src + 16);
            aw[rg] = v8i_t{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
        }
        uint32_t cx[8][NB];
#pragma unroll
        for (int q = 0; q < 2 * NB; ++q) {
            const uint4 x = *reinterpret_cast<const uint4*>(&s_cod[wave][hh][16 * q + t][0]);
            const uint32_t xe[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) cx[(4 * q + e) / NB][(4 * q + e) % NB] = xe[e];
        }
        const int sc_w = 120 + E - 4 * pc;
#pragma unroll
        for (int cg = 0; cg < 8; ++cg) {
            const uint32_t x0 = cx[cg][0], x1 = cx[cg][1];
            const v8i_t bv = v8i_t{(int)(x0 & 0x33333333u), (int)((x0 >> 2) & 0x33333333u), (int)(x1 & 0x33333333u),
                                   (int)((x1 >> 2) & 0x33333333u), 0, 0, 0, 0};
#pragma unroll
            for (int rg = 0; rg < R; ++rg)
                dv[rg][cg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[rg], bv, dv[rg][cg], 0, 4, 0, sc_w, 0, 127);
        }
        // the code buffer and the weight tiles are free once their reads are done: the next block's codes
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        load_codes(s0 + kStep);
        nb ^= 1;
    }
    // no load may still write this wave's buffers when the merge below reuses the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::"s"(s_sgn), "s"(s_cod), "s"(s_nm) : "memory");

    // ---- merge the eight wave streams of each head (the output rows go through the weight tiles)
    float* red_o = reinterpret_cast<float*>(&s_wtile[0][0][0]);        // [wave][head][kD]
    static_assert(sizeof(s_wtile) >= kM8Waves * HPG * kD * sizeof(float), "merge rows fit the weight tiles");
    __syncthreads();
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const float l_sum = row16_sum(l_acc[rg]), mn_sum = row16_sum(mn_acc[rg]);
        if (t == 0) {                            // score head 2 hh + rg
            s_red_m[wave][2 * hh + rg] = m_run[rg];
            s_red_l[wave][2 * hh + rg] = l_sum;
            s_red_mn[wave][2 * hh + rg] = mn_sum;
        }
#pragma unroll
        for (int cg = 0; cg < 8; ++cg)
            red_o[(wave * HPG + 4 * rg + hh) * kD + 16 * cg + t] = (dv[rg][cg][0] + dv[rg][cg][1]) + dv[rg][cg][2];
    }
    __syncthreads();
    const int c0 = 2 * (tid & 63);
    for (int oh = tid >> 6; oh < HPG; oh += kM8Waves) {
        if (HPG * hg + oh >= a.g) break;
        float M = s_red_m[0][oh];
#pragma unroll
        for (int w = 1; w < kM8Waves; ++w) M = fmaxf(M, s_red_m[w][oh]);
        float Ls = 0.f, o0 = 0.f, o1v = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kM8Waves; ++w) {
                const float mw = s_red_m[w][oh];
                if (mw == -INFINITY) continue;
                const float sc = exp2f(mw - M);
                Ls = fmaf(sc, s_red_l[w][oh], Ls);
                o0 = fmaf(sc, red_o[(w * HPG + oh) * kD + c0] + s_red_mn[w][oh], o0);
                o1v = fmaf(sc, red_o[(w * HPG + oh) * kD + c0 + 1] + s_red_mn[w][oh], o1v);
            }
        }
        if (a.nsplit == 1) {
            float* o = a.out + (size_t)(head0 + HPG * hg + oh) * kD;
            o[c0] = Ls > 0.f ? o0 / Ls : 0.f;
            o[c0 + 1] = Ls > 0.f ? o1v / Ls : 0.f;
            continue;
        }
        float* dst = a.part + ((size_t)(head0 + HPG * hg + oh) * a.nsplit + split) * (kD + 2);
        dst[2 + c0] = o0;
        dst[3 + c0] = o1v;
        if ((tid & 63) == 0) {
            dst[0] = M;
            dst[1] = Ls;
        }
    }
}

template <int WIN4, int WOUT4, int R, int NB>
hipError_t launch_decode_mfma_r(const DecodeArgs& a, const AppendArgs* ap, hipStream_t s) {
    const int hgroups = (a.g + 4 * R - 1) / (4 * R);
    const int groups = a.B * a.Hkv * a.nsplit;
    const int slots = (groups + 7) / 8;
    const unsigned nblocks = (unsigned)slots * 8u * (unsigned)hgroups;
    timer_begin(TK_DECODE, s);
    if constexpr (R == 2 && NB == 2 && (WIN4 + WOUT4 == 4 || WIN4 + WOUT4 == 1)) {
        // eight waves (two per SIMD), block data through LDS; with ap, the projection (and the append of
        // ap->pos, if >= 0) inside the kernel
        const AppendArgs apv = ap ? *ap : AppendArgs{};
        if (ap) {
            if (a.scores_dbg)
                hipLaunchKernelGGL((decode_mfma8_kernel<WIN4, WOUT4, true, true>), dim3(nblocks), dim3(kM8Threads), 0, s, a, apv, groups,
                                   hgroups);
            else
                hipLaunchKernelGGL((decode_mfma8_kernel<WIN4, WOUT4, false, true>), dim3(nblocks), dim3(kM8Threads), 0, s, a, apv, groups,
                                   hgroups);
        } else if (a.scores_dbg)
            hipLaunchKernelGGL((decode_mfma8_kernel<WIN4, WOUT4, true, false>), dim3(nblocks), dim3(kM8Threads), 0, s, a, apv, groups,
                               hgroups);
        else
            hipLaunchKernelGGL((decode_mfma8_kernel<WIN4, WOUT4, false, false>), dim3(nblocks), dim3(kM8Threads), 0, s, a, apv, groups,
                               hgroups);
    } else {
        const AppendArgs apv = ap ? *ap : AppendArgs{};
        if (ap) {
            if (a.scores_dbg)
                hipLaunchKernelGGL((decode_mfma_kernel<WIN4, WOUT4, R, true, NB, true>), dim3(nblocks), dim3(kMThreads), 0, s, a, apv,
                                   groups, hgroups);
            else
                hipLaunchKernelGGL((decode_mfma_kernel<WIN4, WOUT4, R, false, NB, true>), dim3(nblocks), dim3(kMThreads), 0, s, a, apv,
                                   groups, hgroups);
        } else if (a.scores_dbg)
            hipLaunchKernelGGL((decode_mfma_kernel<WIN4, WOUT4, R, true, NB, false>), dim3(nblocks), dim3(kMThreads), 0, s, a, apv,
                               groups, hgroups);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<WIN4, WOUT4, R, false, NB, false>), dim3(nblocks), dim3(kMThreads), 0, s, a, apv,
                               groups, hgroups);
    }
    timer_end(TK_DECODE, s);
    return hipGetLastError();
}

template <int WIN4, int WOUT4>
hipError_t launch_decode_mfma_t(const DecodeArgs& a, const AppendArgs* ap, hipStream_t s) {
    const bool r2 = decode_mfma_rowgroups(a.g) == 2;
    if (a.nbits == 4) return r2 ? launch_decode_mfma_r<WIN4, WOUT4, 2, 4>(a, ap, s) : launch_decode_mfma_r<WIN4, WOUT4, 1, 4>(a, ap, s);
    if (a.nbits == 3) return r2 ? launch_decode_mfma_r<WIN4, WOUT4, 2, 3>(a, ap, s) : launch_decode_mfma_r<WIN4, WOUT4, 1, 3>(a, ap, s);
    return r2 ? launch_decode_mfma_r<WIN4, WOUT4, 2, 2>(a, ap, s) : launch_decode_mfma_r<WIN4, WOUT4, 1, 2>(a, ap, s);
}

template <bool APPEND>
hipError_t launch_prologue(const DecodeArgs& a, const AppendArgs& ap, hipStream_t s) {
    const int wpw = (a.m + a.m_out) / 128;       // sign words per wave
    const int nunits = a.B * a.Hkv;              // + workgroups of 4 value appends
    const dim3 grid((unsigned)(nunits + (APPEND ? (nunits + 3) / 4 : 0)));
    if (wpw == 1) hipLaunchKernelGGL((prologue_kernel<1, APPEND>), grid, dim3(256), 0, s, a, ap);
    else if (wpw == 2) hipLaunchKernelGGL((prologue_kernel<2, APPEND>), grid, dim3(256), 0, s, a, ap);
    else if (wpw == 4) hipLaunchKernelGGL((prologue_kernel<4, APPEND>), grid, dim3(256), 0, s, a, ap);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode_kernel(const DecodeArgs& a, const AppendArgs* ap, hipStream_t s) {
    const int win4 = a.m >> 7, wout4 = a.m_out >> 7;
    if (win4 == 1 && wout4 == 0) return launch_decode_mfma_t<1, 0>(a, ap, s);
    if (win4 == 1 && wout4 == 1) return launch_decode_mfma_t<1, 1>(a, ap, s);
    if (win4 == 2 && wout4 == 0) return launch_decode_mfma_t<2, 0>(a, ap, s);
    if (win4 == 2 && wout4 == 2) return launch_decode_mfma_t<2, 2>(a, ap, s);
    if (win4 == 4 && wout4 == 0) return launch_decode_mfma_t<4, 0>(a, ap, s);
    return hipErrorInvalidValue;
}

// With at most 8 query heads per KV head a workgroup serves all of them (one head group), and the
// decode kernels project the queries (and append a decode step's token) themselves.
bool decode_fuses_projection(const DecodeArgs& a) { return a.g <= 8; }

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int qdt, hipStream_t s) {
    const int win4 = a.m >> 7, wout4 = a.m_out >> 7;
    if (qdt == 0 && decode_fuses_projection(a)) {
        AppendArgs none{};
        none.pos = -1;
        hipError_t e = launch_decode_kernel(a, &none, s);
        if (e != hipSuccess || a.nsplit == 1) return e;
        return launch_combine(a, s);
    }
    timer_begin(TK_QPROJ, s);
    if (qdt == 0)
        (void)launch_prologue<false>(a, AppendArgs{}, s);
    else
        hipLaunchKernelGGL(qproj_f32_kernel, dim3(a.B * a.Hq), dim3(256), 0, s, a, win4, wout4);
    timer_end(TK_QPROJ, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_decode_kernel(a, nullptr, s);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_combine(a, s);
}

hipError_t launch_decode_step_mfma(const DecodeArgs& a, const AppendArgs& ap, hipStream_t s) {
    if (decode_fuses_projection(a)) {
        hipError_t e = launch_decode_kernel(a, &ap, s);
        if (e != hipSuccess || a.nsplit == 1) return e;
        return launch_combine(a, s);
    }
    timer_begin(TK_STEP, s);
    hipError_t e = launch_prologue<true>(a, ap, s);
    timer_end(TK_STEP, s);
    if (e != hipSuccess) return e;
    e = launch_decode_kernel(a, nullptr, s);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_combine(a, s);
}

}  // namespace qjl

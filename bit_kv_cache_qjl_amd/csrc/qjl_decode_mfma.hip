// Decode attention on the matrix cores: estimator scores and the value aggregation of up to four
// query heads per instruction.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero Overhead",
// "Approach" (asymmetric estimator sqrt(pi/2)/m * |k| * <S q, sign(S k)> with the query projected
// unquantized) and softmax attention over the estimated scores with the dequantized values ("Your
// Brain Already Runs on 1-Bit Keys", "Keys Select. Values Deliver.").
//
// Scores on v_mfma_scale_f32_16x16x128_f8f6f4 (A fp8 e4m3, B fp4 e2m1): 16 tokens x 4 query heads
// per instruction, 128 sign positions of one kind (inlier or outlier) per instruction.
//   B (sign bits): with b = 1 for a non-negative projection, a 32-bit sign word x gives four fp4
//     operand words, one instruction each: x & 0x11111111, x & 0x22222222, x & 0x44444444 (nibble n
//     holds bit 4n + i with the value 0.5 b, b, 2 b: e2m1 0001, 0010, 0100) and
//     (x & 0x88888888) | 0x11111111 (e2m1 0001 or 1001: the value 0.5 - b of bit 4n + 3).
//   A (query): x_k = 2 z_scale sqrt(pi/2)/m (S q)_k divided by its plane's bit coefficient (0.5, 1,
//     2, -1) and scaled by a per-head power of two, split into three e4m3 pieces (each rounded to
//     nearest, 4 significant bits, so the residual is below 2^-12 of the value); rows = (query head,
//     piece), the fourth row of a head is zero, and the instruction's E8M0 row scales undo the powers
//     of two.
//   sign = 2b - 1, so <S q, sign> = 2 <S q, b> - sum (S q).  The plane-3 positions contribute
//     x_k b_k - x_k / 2 by themselves; the accumulator starts at -sum x_k / 2 over the other
//     positions, so z = |k_in| D_in + |k_out| D_out is the token's base-2 softmax logit.
// Values on the same instruction: rows = (query head, piece) of the weight p * step, columns = 16
// channels, K = 128 tokens; B = the 2-bit codes of a code tile as x & 0x33333333 and
// (x >> 2) & 0x33333333 (e2m1 nibble 00cc = code / 2); 4-bit codes as their two 2-bit planes, the
// high one through a B scale of 4.  The weights of a 128-token block are scaled
// by 2^(8 - E), 2^E > the block's largest step, split into three e4m3 pieces, and transposed to the
// A-operand order through LDS.  Each wave is an independent online-softmax stream over 128-token
// blocks; the four waves of a workgroup merge at the end of the chunk.
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

// ---------------------------------------------------------------------------- query operand
// The matrix-core operand of one query head, built by one wave from the head's projections
// x_j = 2 z_scale sqrt(pi/2)/m (S q)_j (inlier j < m, then outlier, natural order, in LDS; for the
// two-sided estimator x_j = 2 z_scale |q_part|/m sign((S q)_j) instead): the
// A-operand bytes in the order the decode kernel loads them, [K block kb][piece][lane group ga][32
// bytes] (byte ea of lane group ga is K index k = 16 ga + ea % 16 + 64 (ea / 16) of the instruction,
// and K index k pairs with bit 4n + i, n = (k % 32) % 8, i = (k % 32) / 8, of the sign word that B
// lane group k / 32 supplies), and the per-head constants [-sum x_in / 2, -sum x_out / 2 (both over
// the positions outside plane 3), e_in, e_out].
__device__ void query_operand_wave(const float* xs, int m, int m_out, int win4, int wout4, uint32_t* dst, float* qc,
                                   int lane) {
    // |x| divided by its plane's bit coefficient (0.5, 1, 2, -1 for position % 4 = 0, 1, 2, 3)
    auto plane_abs = [](float x, int pos) {
        const int i = pos & 3;
        return fabsf(x) * (i == 0 ? 2.f : (i == 2 ? 0.5f : 1.f));
    };
    float sum_in = 0.f, sum_out = 0.f, mx_in = 0.f, mx_out = 0.f;
    for (int j = lane; j < m; j += 64) {
        const float x = xs[j];
        if ((j & 3) != 3) sum_in += x;           // plane-3 positions carry their own -x/2
        mx_in = fmaxf(mx_in, plane_abs(x, j));
    }
    for (int j = lane; j < m_out; j += 64) {   // m is a multiple of 4: position m + j is in plane j % 4
        const float x = xs[m + j];
        if ((j & 3) != 3) sum_out += x;
        mx_out = fmaxf(mx_out, plane_abs(x, j));
    }
    sum_in = wave64_sum(sum_in);
    sum_out = wave64_sum(sum_out);
    mx_in = wave64_max(mx_in);
    mx_out = wave64_max(mx_out);
    // the power of two that takes the largest operand value into [128, 256), kept within the E8M0
    // range of the row scales 127 - e - 4 piece
    auto pick_exp = [](float mx) {
        if (!(mx > 0.f)) return 0;
        const int e = 8 - __builtin_amdgcn_frexp_expf(mx);
        return e > 114 ? 114 : (e < -120 ? -120 : e);
    };
    const int e_in = pick_exp(mx_in), e_out = pick_exp(mx_out);
    if (lane == 0) {
        qc[0] = -0.5f * sum_in;
        qc[1] = -0.5f * sum_out;
        qc[2] = __int_as_float(e_in);
        qc[3] = __int_as_float(e_out);
    }
    // one task = 4 consecutive bytes e0 .. e0 + 3 of lane group ga in K block kb, all three pieces
    // (words kb 128 + piece 32 + ga 8 + e0 / 4; the fourth piece's word is zero)
    const int W = 4 * (win4 + wout4);
    for (int task = lane; task < 8 * W; task += 64) {
        const int kb = task >> 5;
        const int ga = (task >> 3) & 3;
        const int e0 = (task & 7) * 4;
        const bool out = kb >= win4;
        const int e = out ? e_out : e_in;
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ea = e0 + q;
            const int k = 16 * ga + (ea & 15) + 64 * (ea >> 4);
            const int gb = k >> 5, eb = k & 31;
            const int plane = eb >> 3, n = eb & 7;
            const int word = out ? 4 * win4 + gb * wout4 + (kb - win4) : gb * win4 + kb;
            // divided by the plane's bit coefficient and scaled by the head's power of two (exact)
            const float v = ldexpf(xs[32 * word + 4 * n + plane], e + (plane == 0 ? 1 : (plane == 2 ? -1 : 0)));
            y[q] = plane == 3 ? -v : v;
        }
        uint32_t k[3];
        fp8_pieces(y, k);
        uint32_t* d = dst + kb * 128 + ga * 8 + (task & 7);
        d[0] = k[0];
        d[32] = k[1];
        d[64] = k[2];
        d[96] = 0u;
    }
}

// fp32 queries and JL matrices: one workgroup per (sequence, query head), S q in fp32 on the VALU in
// channel order, then the operand (wave 0).
__global__ __launch_bounds__(256) void qproj_f32_kernel(DecodeArgs a, int win4, int wout4) {
    __shared__ float qin[kD];
    __shared__ float qo[kMaxOutliers];
    __shared__ int so[kMaxOutliers];
    __shared__ float xs[kMaxBits];
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
        query_operand_wave(xs, a.m, a.m_out, win4, wout4, reinterpret_cast<uint32_t*>(a.sq) + (size_t)bh * (128 * (win4 + wout4)),
                           a.qconst + (size_t)bh * 4, tid);
}

// bf16: one workgroup per (sequence, KV head) projects the KV head's g query heads (and, for a decode
// step, the new key) on the matrix cores: D (16 vectors x 16 projections) = A (vectors x channels,
// from LDS) . B (S rows, straight from global memory), v_mfma_f32_16x16x32_bf16 (exact bf16 products,
// fp32 sums).  Vector 0 of the first pass is the new key when APPEND; its signs are the sign bits of
// the cache row (ballot of the D column), its norms and its value codes are computed as in the
// quantize kernels.  Wave w owns sign words w WPW .. (w + 1) WPW - 1 (two 16-projection tiles per
// word), so WPW = W / 4.  The query projections go to LDS, then one wave per head builds the operand.
constexpr int kVRow = kD + 8;                // LDS row of a staged vector (bf16), 272 B
constexpr int kMaxMfmaBits = 512;            // m + m_out on the matrix-core path
constexpr int kXPitch = kMaxMfmaBits + 4;    // LDS row of a head's projections (floats)

template <int WPW, bool APPEND>
__global__ __launch_bounds__(256) void prologue_kernel(DecodeArgs a, AppendArgs ap) {
    __shared__ __attribute__((aligned(16))) uint16_t vin[16 * kVRow];    // vectors, outlier channels zeroed
    __shared__ __attribute__((aligned(16))) uint16_t vout[16 * kVRow];   // vectors on the outlier channels only
    __shared__ float xs[16 * kXPitch];
    __shared__ uint32_t s_mask[4];
    __shared__ float s_qn[16][2];                                         // vector norms (two-sided)
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nunits = a.B * a.Hkv;
    if (APPEND && (int)blockIdx.x >= nunits) {
        // ---- the new values, one (sequence, KV head) per wave in workgroups of their own (their atomic
        //      round trips overlap the projections): a row of 16 lanes, 8 channels per lane; the 2- or
        //      4-bit fields are merged into the tile words of position pos with atomic and/or, the rest
        //      of the tile is kept
        const int vunit = 4 * ((int)blockIdx.x - nunits) + wave;
        if (vunit >= nunits) return;
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
        return;
    }
    const int unit = blockIdx.x;                 // b * Hkv + h
    const int b = unit / a.Hkv, h = unit - b * a.Hkv;
    const int Win = a.m >> 5, Wout = a.m_out >> 5, W = Win + Wout;
    const int win4 = a.m >> 7, wout4 = a.m_out >> 7;
    const int ncol = a.g + (APPEND ? 1 : 0);
    const int64_t head0 = (int64_t)b * a.Hq + (int64_t)h * a.g;

    // ---- every global load that does not depend on another is issued first: this wave's S tiles
    //      (B operands: projection row 16 hf + lane % 16 of word wn, channels 32 s + 8 (lane / 16) ..),
    //      the outlier channels and the first pass's vectors
    uint4 sb[WPW][2][4];
#pragma unroll
    for (int u = 0; u < WPW; ++u) {
        const int wn = WPW * wave + u;
        const uint16_t* S = wn < Win ? static_cast<const uint16_t*>(a.S_in) + (size_t)(32 * wn) * kD
                                     : static_cast<const uint16_t*>(a.S_out) + (size_t)(32 * (wn - Win)) * kD;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sb[u][hf][s] = *reinterpret_cast<const uint4*>(S + (size_t)(16 * hf + (lane & 15)) * kD + 32 * s + 8 * (lane >> 4));
    }
    // the KV head's outlier channels: one entry per lane of wave 0, all in one round trip
    const int oc = (wave == 0 && lane < a.n_out) ? (a.oidx[h * a.n_out + lane] & (kD - 1)) : -1;
    const int sv = tid >> 4, cg = tid & 15;      // staging: vector sv of a pass, channels 8 cg .. 8 cg + 7
    auto load_vector = [&](int col) {
        if (col >= ncol) return make_uint4(0u, 0u, 0u, 0u);
        if (APPEND && col == 0) return *reinterpret_cast<const uint4*>(ap.K + b * ap.sKb + h * ap.sKh + 8 * cg);
        return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Q) + (head0 + col - (APPEND ? 1 : 0)) * kD + 8 * cg);
    };
    uint4 xv = load_vector(sv);
    if (wave == 0) {
        // outlier mask of the KV head (bit c % 32 of word c / 32): the LDS operations of a wave complete
        // in order, so the words are cleared before the entries set their bits
        if (lane < 4) s_mask[lane] = 0u;
        if (oc >= 0) atomicOr(&s_mask[oc >> 5], 1u << (oc & 31));
    }
    __syncthreads();

    const float c_in = 2.f * a.z_scale * kSqrtHalfPi / (float)a.m;
    const float c_out = a.m_out ? 2.f * a.z_scale * kSqrtHalfPi / (float)a.m_out : 0.f;
    const float c2_in = 2.f * a.z_scale / (float)a.m;
    const float c2_out = a.m_out ? 2.f * a.z_scale / (float)a.m_out : 0.f;
    for (int c0 = 0; c0 < ncol; c0 += 16) {
        const bool key_pass = APPEND && c0 == 0;
        // ---- stage 16 vectors, split at the outlier channels
        {
            if (c0) xv = load_vector(c0 + sv);
            const uint32_t om = (s_mask[cg >> 2] >> (8 * (cg & 3))) & 0xFFu;
            uint4 xi, xo;
            float ss_in = 0.f, ss_out = 0.f;
            split_key8(xv, om, xi, xo, ss_in, ss_out);
            *reinterpret_cast<uint4*>(vin + sv * kVRow + 8 * cg) = xi;
            *reinterpret_cast<uint4*>(vout + sv * kVRow + 8 * cg) = xo;
            if (key_pass || a.estimator) {
                // squared norms of each vector's two parts: one DPP row of 16 lanes per vector
                ss_in = row16_sum(ss_in);
                ss_out = row16_sum(ss_out);
            }
            // the key is vector 0: lanes 0..15 of wave 0
            if (key_pass && tid == 0) reinterpret_cast<uint32_t*>(ap.norms)[(size_t)unit * a.Ncap + ap.pos] = norm_pair(ss_in, ss_out);
            if (a.estimator && cg == 0) {
                s_qn[sv][0] = sqrtf(ss_in);
                s_qn[sv][1] = sqrtf(ss_out);
            }
        }
        __syncthreads();

        // ---- projections: sign word wn = WPW wave + u is the pair of 16-projection tiles 2 wn, 2 wn + 1;
        //      D lane l holds projection 32 wn + 16 hf + l % 16 of vectors 4 (l / 16) + i
#pragma unroll
        for (int u = 0; u < WPW; ++u) {
            const int wn = WPW * wave + u;
            const bool inl = wn < Win;
            const uint16_t* vsrc = (inl ? vin : vout) + (lane & 15) * kVRow + 8 * (lane >> 4);
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
                    const float t = a.estimator ? s_qn[vec][inl ? 0 : 1] * (inl ? c2_in : c2_out) : 0.f;
                    xs[vec * kXPitch + j] = a.estimator ? (acc[i] >= 0.f ? t : -t) : acc[i] * cs;
                }
            }
            if (key_pass && lane == 0) ap.bits[((size_t)unit * a.Ncap + ap.pos) * W + bits_slot(wn, Win, Wout)] = word;
        }
        __syncthreads();

        // ---- operands of this pass's query heads, one wave per head
        for (int v = wave; v < 16; v += 4) {
            const int col = c0 + v;
            if (col >= ncol) break;
            if (APPEND && col == 0) continue;
            const int64_t hq = head0 + col - (APPEND ? 1 : 0);
            query_operand_wave(xs + v * kXPitch, a.m, a.m_out, win4, wout4,
                               reinterpret_cast<uint32_t*>(a.sq) + hq * (128 * (win4 + wout4)), a.qconst + hq * 4, lane);
        }
        __syncthreads();
    }
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
    int codes;   // channel streams 8 t .. 8 t + 7 of code tile hh
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
            bl.w[s][0] = __builtin_amdgcn_raw_buffer_load_b32(rb, voff, 0, 0);
        } else if constexpr (Q == 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(rb, voff, 0, 0);
            bl.w[s][0] = x[0]; bl.w[s][1 % Q] = x[1];
        } else {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0);
            bl.w[s][0] = x[0]; bl.w[s][1 % Q] = x[1]; bl.w[s][2 % Q] = x[2]; bl.w[s][3 % Q] = x[3];
        }
    }
    const int vn = o.nm + s0 * 4;
    const auto n2 = __builtin_amdgcn_raw_buffer_load_b64(rn, vn, 0, 0);
    const auto m2 = __builtin_amdgcn_raw_buffer_load_b64(rm, vn, 0, 0);
    bl.nm[0] = n2[0]; bl.nm[1] = m2[0]; bl.nm[2] = n2[1]; bl.nm[3] = m2[1];
    const int vc = o.codes + s0 * (kD * NB * 4 / kCodeTile);
    // the 8 channels' NB words each are 8 NB consecutive words: word 4 q + e is word (4 q + e) % NB of
    // channel group (4 q + e) / NB
#pragma unroll
    for (int q = 0; q < 2 * NB; ++q) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rc, vc + 16 * q, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) bl.cx[(4 * q + e) / NB][(4 * q + e) % NB] = x[e];
    }
}

// R = 1: one workgroup serves 4 query heads of a KV head; R = 2: 8 query heads as two row groups of
// the same instructions' B operands (the sign and code planes are built once for both).
// Two workgroups per CU for 4 query heads and 2-bit codes; one (the whole register file) otherwise.
template <int WIN4, int WOUT4, int R, bool DBG, int NB>
__global__ __launch_bounds__(kMThreads, (R == 1 && NB == 2) ? 2 : 1) void decode_mfma_kernel(DecodeArgs a, int groups, int hgroups) {
    constexpr int W4 = WIN4 + WOUT4;             // instructions (K blocks of 128 sign positions) per token
    constexpr int WB = 4 * W4;                   // sign words per token
    constexpr int HPG = 4 * R;                   // query heads per workgroup
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

    // ---- score A operands and scales: this lane's A row in row group rg is (head 4 rg + rh, piece pc),
    //      K slice hh
    const int rh = t >> 2, pc = lane & 3;
    v8i_t sA[R][W4];
    int sc_in[R], sc_out[R];
#pragma unroll
    for (int rg = 0; rg < R; ++rg) {
        const int qa_head = HPG * hg + 4 * rg + rh;
        sc_in[rg] = sc_out[rg] = 127;
        if (qa_head < a.g) {
            const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.sq) +
                                                              (size_t)(head0 + qa_head) * (128 * WB));
#pragma unroll
            for (int kb = 0; kb < W4; ++kb) {
                const uint4 lo = src[kb * 32 + (pc * 4 + hh) * 2], hi = src[kb * 32 + (pc * 4 + hh) * 2 + 1];
                sA[rg][kb] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            const float* c = a.qconst + (size_t)(head0 + qa_head) * 4;
            sc_in[rg] = 127 - __float_as_int(c[2]) - 4 * pc;
            sc_out[rg] = 127 - __float_as_int(c[3]) - 4 * pc;
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
        cin[rg] = ok ? a.qconst[(size_t)(head0 + dhead) * 4] : 0.f;
        cout[rg] = ok ? a.qconst[(size_t)(head0 + dhead) * 4 + 1] : 0.f;
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
    const MOffsets offs{(mfma_token(0, t) * WB + hh * W4) * 4, 8 * lane, hh * (kD * NB * 4) + t * (8 * NB * 4)};
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
                    din = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sA[rg][kb], bin[kb], din, 0, 4, 0, sc_in[rg], 0, 127);
                float zz = n_in * ((din[0] + din[1]) + din[2]);
                if constexpr (WOUT4 > 0) {
                    v4f_t dout = v4f_t{cout[rg], 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < WOUT4; ++kb)
                        dout = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sA[rg][WIN4 + kb], bout[kb], dout, 0, 4, 0,
                                                                                sc_out[rg], 0, 127);
                    zz = fmaf(n_out, (dout[0] + dout[1]) + dout[2], zz);
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
#pragma unroll
        for (int cg = 0; cg < 8; ++cg) {
            if constexpr (NB == 2) {
                const uint32_t x0 = cur.cx[cg][0], x1 = cur.cx[cg][1 % NB];
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

template <int WIN4, int WOUT4, int R, int NB>
hipError_t launch_decode_mfma_r(const DecodeArgs& a, hipStream_t s) {
    const int hgroups = (a.g + 4 * R - 1) / (4 * R);
    const int groups = a.B * a.Hkv * a.nsplit;
    const int slots = (groups + 7) / 8;
    const unsigned nblocks = (unsigned)slots * 8u * (unsigned)hgroups;
    timer_begin(TK_DECODE, s);
    if (a.scores_dbg)
        hipLaunchKernelGGL((decode_mfma_kernel<WIN4, WOUT4, R, true, NB>), dim3(nblocks), dim3(kMThreads), 0, s, a, groups, hgroups);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<WIN4, WOUT4, R, false, NB>), dim3(nblocks), dim3(kMThreads), 0, s, a, groups, hgroups);
    timer_end(TK_DECODE, s);
    return hipGetLastError();
}

template <int WIN4, int WOUT4>
hipError_t launch_decode_mfma_t(const DecodeArgs& a, hipStream_t s) {
    const bool r2 = decode_mfma_rowgroups(a.g) == 2;
    if (a.nbits == 4) return r2 ? launch_decode_mfma_r<WIN4, WOUT4, 2, 4>(a, s) : launch_decode_mfma_r<WIN4, WOUT4, 1, 4>(a, s);
    if (a.nbits == 3) return r2 ? launch_decode_mfma_r<WIN4, WOUT4, 2, 3>(a, s) : launch_decode_mfma_r<WIN4, WOUT4, 1, 3>(a, s);
    return r2 ? launch_decode_mfma_r<WIN4, WOUT4, 2, 2>(a, s) : launch_decode_mfma_r<WIN4, WOUT4, 1, 2>(a, s);
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

hipError_t launch_decode_kernel(const DecodeArgs& a, hipStream_t s) {
    const int win4 = a.m >> 7, wout4 = a.m_out >> 7;
    if (win4 == 1 && wout4 == 0) return launch_decode_mfma_t<1, 0>(a, s);
    if (win4 == 1 && wout4 == 1) return launch_decode_mfma_t<1, 1>(a, s);
    if (win4 == 2 && wout4 == 0) return launch_decode_mfma_t<2, 0>(a, s);
    if (win4 == 2 && wout4 == 2) return launch_decode_mfma_t<2, 2>(a, s);
    if (win4 == 4 && wout4 == 0) return launch_decode_mfma_t<4, 0>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int qdt, hipStream_t s) {
    const int win4 = a.m >> 7, wout4 = a.m_out >> 7;
    timer_begin(TK_QPROJ, s);
    if (qdt == 0)
        (void)launch_prologue<false>(a, AppendArgs{}, s);
    else
        hipLaunchKernelGGL(qproj_f32_kernel, dim3(a.B * a.Hq), dim3(256), 0, s, a, win4, wout4);
    timer_end(TK_QPROJ, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_decode_kernel(a, s);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_combine(a, s);
}

hipError_t launch_decode_step_mfma(const DecodeArgs& a, const AppendArgs& ap, hipStream_t s) {
    timer_begin(TK_STEP, s);
    hipError_t e = launch_prologue<true>(a, ap, s);
    timer_end(TK_STEP, s);
    if (e != hipSuccess) return e;
    e = launch_decode_kernel(a, s);
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_combine(a, s);
}

}  // namespace qjl

// Decode attention over the 1-bit key sketch: query projection, estimator scores, online softmax,
// dequantized-value aggregation, split-context log-sum-exp merge.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero Overhead",
// "Approach" (the query is JL-projected without quantization; the asymmetric estimator
// sqrt(pi/2)/m * |k| * <S q, sign(S k)> is unbiased); softmax attention with a weighted sum of the
// dequantized values ("Your Brain Already Runs on 1-Bit Keys", "Keys Select. Values Deliver.").
//
// Kernels
//   qproj   one workgroup per (sequence, query head): Sq = S q (fp32) pre-multiplied by
//           sqrt(pi/2)/m (inlier part) and sqrt(pi/2)/m_out (outlier part); for the two-sided
//           estimator (both sides as signs: "Surprising findings" of the QJL summary) sign(Sq) times
//           |q_in|/m and |q_out|/m_out instead.
//   decode  one workgroup (8 waves) per (sequence, KV head, query head, context chunk).  The
//           projected query is expanded in LDS into byte tables: entry [p][beta] is the signed sum of
//           the 8 Sq values of byte position p under sign pattern beta, so one LDS read replaces
//           eight +-1 accumulations.  Each wave is an independent online-softmax stream over
//           64-token slabs:
//             score  lane = token: buffer loads of the token's sign words, one table read per byte
//                    (offset from one SDWA shift), s = |k_in| * sum_in + |k_out| * sum_out;
//             softmax wave-wide running max (log2 domain), p = 2^(z - M), running sums;
//             value  lane = two channels: one 16-byte load per 32-token code tile brings the code
//                    words of both channel streams; the 2-bit codes of tokens (t, t + 8) of a word become
//                    an fp16 pair 1 + code/4 with one shift and one and-or, and v_dot2_f32_f16
//                    accumulates p*step for both tokens at once; the constant 1 is removed at the
//                    end (sum p*step*(1 + code/4) - sum p*step = sum p*step*code/4), and the min
//                    term sum p*min is carried separately.
//           The eight wave states merge into the chunk's partial (max, sum, unnormalized output).
//   combine one workgroup per (sequence, query head): log-sum-exp merge of the chunk partials.
#include <math.h>

#include "qjl_decode_common.h"

namespace qjl {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = kDecodeTile;   // 512
constexpr int kWaves = kThreads / 64;

// ------------------------------------------------------------------------------------ qproj
template <typename QT>
__global__ __launch_bounds__(256) void qproj_kernel(DecodeArgs a) {
    __shared__ float qin[kD];
    __shared__ float qo[kMaxOutliers];
    __shared__ int so[kMaxOutliers];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int hq = bh % a.Hq;
    const int h = hq / a.g;
    const QT* Q = static_cast<const QT*>(a.Q);
    if (tid < a.n_out) so[tid] = a.oidx[h * a.n_out + tid] & (kD - 1);   // never index outside a row
    if (tid < kD) qin[tid] = load_elem<QT>(Q, (size_t)bh * kD + tid);
    __syncthreads();
    if (tid < a.n_out) qo[tid] = qin[so[tid]];
    __syncthreads();
    if (tid < a.n_out) qin[so[tid]] = 0.f;
    __syncthreads();
    const QT* Sin = static_cast<const QT*>(a.S_in);
    const QT* Sout = static_cast<const QT*>(a.S_out);
    float* dst = a.sq + (size_t)bh * (a.m + a.m_out);
    // one-sided: Sq scaled by sqrt(pi/2)/m; two-sided: only the sign of each projection is kept, scaled
    // by the norm of the query part over m (sign(0) = +1)
    const bool two = a.estimator != 0;
    float qn_in = 0.f, qn_out = 0.f;
    if (two) {
        for (int c = 0; c < kD; ++c) qn_in = fmaf(qin[c], qin[c], qn_in);
        for (int i = 0; i < a.n_out; ++i) qn_out = fmaf(qo[i], qo[i], qn_out);
        qn_in = sqrtf(qn_in);
        qn_out = sqrtf(qn_out);
    }
    const float c_in = (two ? qn_in : kSqrtHalfPi) / (float)a.m;
    for (int j = tid; j < a.m; j += 256) {
        const float p = row_dot(Sin + (size_t)j * kD, qin);
        dst[j] = two ? (p >= 0.f ? c_in : -c_in) : p * c_in;
    }
    if (a.m_out) {
        const float c_out = (two ? qn_out : kSqrtHalfPi) / (float)a.m_out;
        for (int j = tid; j < a.m_out; j += 256) {
            float acc = 0.f;
            for (int i = 0; i < a.n_out; ++i) acc = fmaf(load_elem<QT>(Sout, (size_t)j * kD + so[i]), qo[i], acc);
            dst[a.m + j] = two ? (acc >= 0.f ? c_out : -c_out) : acc * c_out;
        }
    }
}

// ------------------------------------------------------------------------------------ decode
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
    uint32_t r;
    asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(o));
    return r;
}

// Byte k of x, times 4 (a table offset in bytes) in one SDWA instruction.
template <int K>
__device__ __forceinline__ uint32_t byte_x4(uint32_t x) {
    uint32_t r;
    if (K == 0) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(x));
    if (K == 1) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(x));
    if (K == 2) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(x));
    if (K == 3) asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(x));
    return r;
}

__device__ __forceinline__ float wave_max(float v) { return wave64_max(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave64_sum(v); }

constexpr int kSlab = 64;                    // tokens per wave step

// Token data of one wave step.
template <int WB, int VM>
struct Slab {
    uint32_t w[WB];      // sign words of this lane's token
    uint32_t nrm;        // (|k_in|, |k_out|) fp16 pair
    uint32_t mt;         // (min, step) fp16 pair
    uint32_t xv[8];      // value role: code words of this lane's two channel streams in the slab's two tiles
};

template <int WB, int VM>
__device__ __forceinline__ void load_slab(Slab<WB, VM>& sl, __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rn,
                                          __amdgpu_buffer_rsrc_t rm, __amdgpu_buffer_rsrc_t rc, int s0, int lane) {
    const int t = s0 + lane;
#pragma unroll
    for (int q = 0; q < WB / 4; ++q) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rb, (t * WB + 4 * q) * 4, 0, 0);
        sl.w[4 * q] = x[0]; sl.w[4 * q + 1] = x[1]; sl.w[4 * q + 2] = x[2]; sl.w[4 * q + 3] = x[3];
    }
    sl.nrm = __builtin_amdgcn_raw_buffer_load_b32(rn, t * 4, 0, 0);
    if (VM == 0) {
        sl.mt = __builtin_amdgcn_raw_buffer_load_b32(rm, t * 4, 0, 0);
        // tile = [128 stream slots][2 words] (1 KiB); this lane's stream slots 2 lane, 2 lane + 1
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rc, (s0 / kCodeTile + q) * 1024 + lane * 16, 0, 0);
            sl.xv[4 * q] = x[0]; sl.xv[4 * q + 1] = x[1]; sl.xv[4 * q + 2] = x[2]; sl.xv[4 * q + 3] = x[3];
        }
    } else {
        sl.mt = 0u;
    }
}

// VM = 0: 2-bit codes + (min, step) meta;  VM = 1: fp32 values.
//
// Each wave is an independent online-softmax stream over 64-token slabs (slab i of the chunk goes
// to wave i mod 8); the waves share only the read-only byte tables, so there is no workgroup
// barrier inside the token loop.  The eight partial (max, sum, output) states are merged once at
// the end of the chunk.
template <int WIN, int WOUT, int VM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeArgs a, int groups) {
    constexpr int WB = WIN + WOUT;
    constexpr int P = 4 * WB;                    // byte positions = tables
    constexpr int LUT_FLOATS = P * 256 > (kThreads / 8) * kD ? P * 256 : (kThreads / 8) * kD;
    __shared__ __attribute__((aligned(16))) float lut[LUT_FLOATS];   // [P][256]; reused for the final reduction
    __shared__ float sq_s[8 * P];
    __shared__ __attribute__((aligned(16))) float wts[kWaves][kSlab];   // per-wave weights of one slab
    __shared__ float red[kWaves][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // XCD-aware placement: blocks L, L+8, L+16, ... share an XCD (and its L2); the query heads of one
    // (KV head, chunk) are consecutive slots of the same XCD so their re-reads of the chunk hit L2.
    const int lin = blockIdx.x;
    const int xcd = lin & 7;
    const int slot = lin >> 3;
    const int hg = slot % a.g;
    const int64_t us = (int64_t)(slot / a.g) * 8 + xcd;
    if (us >= (int64_t)groups) return;
    const int split = (int)(us % a.nsplit);
    const int unit = (int)(us / a.nsplit);       // b * Hkv + h
    const int b = unit / a.Hkv;
    const int h = unit - b * a.Hkv;
    const int hq = h * a.g + hg;
    const int bhq = b * a.Hq + hq;

    // token range of this chunk, as 32-bit offsets inside the (sequence, KV head) rows
    const int t_begin = (int)((int64_t)split * a.chunk);
    const int t_end = (int)min(a.N, (int64_t)t_begin + a.chunk);

    // ---- byte tables of the projected query: entry [p][beta] = sum_i (+-) Sq[8p' + i] for stored
    //      byte p of a row (slot p/4, natural word w = bits_word(p/4), p' = 4 w + p % 4)
    for (int i = tid; i < 8 * P; i += kThreads) sq_s[i] = a.sq[(size_t)bhq * (8 * P) + i];
    __syncthreads();
    // one task = (position p, high nibble): 16 entries from the high-nibble sum and two
    // 4-entry tables of the low bit pairs
    for (int idx = tid; idx < P * 16; idx += kThreads) {
        const int p = idx >> 4, bh = idx & 15;
        const float* sv = sq_s + 32 * bits_word(p >> 2, WIN, WOUT) + 8 * (p & 3);
        float hi = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) hi += ((bh >> i) & 1) ? sv[4 + i] : -sv[4 + i];
        const float t01[4] = {-sv[0] - sv[1], sv[0] - sv[1], -sv[0] + sv[1], sv[0] + sv[1]};
        const float t23[4] = {-sv[2] - sv[3], sv[2] - sv[3], -sv[2] + sv[3], sv[2] + sv[3]};
        float4* dst = reinterpret_cast<float4*>(lut + p * 256 + bh * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float h2 = hi + t23[q];
            dst[q] = make_float4(h2 + t01[0], h2 + t01[1], h2 + t01[2], h2 + t01[3]);
        }
    }
    __syncthreads();

    // the (sequence, KV head) rows, bounded at the end of this chunk
    const uint32_t* bits = a.bits + (size_t)unit * a.Ncap * WB;
    const uint32_t* norms = reinterpret_cast<const uint32_t*>(a.norms) + (size_t)unit * a.Ncap;
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(bits, (uint32_t)t_end * WB * 4u);
    const __amdgpu_buffer_rsrc_t rn = buffer_rsrc(norms, (uint32_t)t_end * 4u);
    const __amdgpu_buffer_rsrc_t rm = VM == 0 ? buffer_rsrc(reinterpret_cast<const uint32_t*>(a.meta) + (size_t)unit * a.Ncap,
                                                            (uint32_t)t_end * 4u) : rn;
    // code tiles of this (sequence, KV head), bounded at the tile holding the chunk's last token
    const __amdgpu_buffer_rsrc_t rc = VM == 0 ? buffer_rsrc(a.codes + (size_t)unit * code_tiles(a.Ncap) * (kD * 2),
                                                            (uint32_t)code_tiles(t_end) * 1024u) : rn;
    const float* vf = VM == 1 ? a.V_f32 + (size_t)unit * a.Ncap * kD : nullptr;
    float* sdbg = a.scores_dbg ? a.scores_dbg + (size_t)bhq * a.N : nullptr;

    const int jv = lane & 7;         // fp32 value role: 16-channel slice
    const int pg = lane >> 3;        // fp32 value role: token-pair group of the slab (0..7)
    float* wl = wts[wave];
    // code role: the weight of token tau sits in fp16 pair 8 (tau / 16) + tau % 8, half (tau / 8) % 2,
    // next to the token 8 positions away that shares its code word
    const int wslot = 2 * (8 * (lane >> 4) + (lane & 7)) + ((lane >> 3) & 1);

    float m_run = -INFINITY;
    float l_t = 0.f, mn_t = 0.f, sw_t = 0.f;   // per-lane partial sums (score role)
    constexpr int NACC = VM == 0 ? 8 : 16;      // codes: 2 channels x 4 partial sums; fp32: 16 channels
    float acc[NACC];
#pragma unroll
    for (int c = 0; c < NACC; ++c) acc[c] = 0.f;

    const char* lut_b = reinterpret_cast<const char*>(lut);
    for (int s0 = t_begin + kSlab * wave; s0 < t_end; s0 += kSlab * kWaves) {
        Slab<WB, VM> cur;
        load_slab<WB, VM>(cur, rb, rn, rm, rc, s0, lane);
        const int t = s0 + lane;
        const bool valid = t < t_end;

        // ---- score of this lane's token: one table read per byte of its sign words
        float s_in = 0.f, s_out = 0.f;
#pragma unroll
        for (int w = 0; w < WB; ++w) {
            const uint32_t x = cur.w[w];
            const char* tb = lut_b + (4 * w) * 1024;
            float part = *reinterpret_cast<const float*>(tb + byte_x4<0>(x));
            part += *reinterpret_cast<const float*>(tb + 1024 + byte_x4<1>(x));
            part += *reinterpret_cast<const float*>(tb + 2048 + byte_x4<2>(x));
            part += *reinterpret_cast<const float*>(tb + 3072 + byte_x4<3>(x));
            if (w % (WB / 4) < WIN / 4) s_in += part; else s_out += part;   // stored slot w
        }
        const float n_in = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.nrm & 0xFFFFu));
        const float n_out = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.nrm >> 16));
        const float score = WOUT ? fmaf(n_out, s_out, n_in * s_in) : n_in * s_in;
        if (sdbg && valid) sdbg[t] = score;
        const float z = valid ? score * a.z_scale : -INFINITY;

        // ---- online softmax of this wave's stream (log2 domain)
        const float m_new = fmaxf(m_run, wave_max(z));
        // v_exp_f32 directly: weights below 2^-126 contribute nothing to the sums
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // m_new is finite: lane 0 of a slab is valid
        const float p = valid ? __builtin_amdgcn_exp2f(z - m_new) : 0.f;
        m_run = m_new;
        l_t = fmaf(l_t, alpha, p);
        if (VM == 0) {
            const float mn = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.mt & 0xFFFFu));
            const float step = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.mt >> 16));
            const _Float16 w16 = (_Float16)(p * step);
            mn_t = fmaf(mn_t, alpha, p * mn);
            sw_t = fmaf(sw_t, alpha, (float)w16);
            reinterpret_cast<_Float16*>(wl)[wslot] = w16;
        } else {
            wl[lane] = p;
        }
        if (alpha != 1.f) {
#pragma unroll
            for (int c = 0; c < NACC; ++c) acc[c] *= alpha;
        }
        __builtin_amdgcn_wave_barrier();   // the weights written above are read by other lanes below

        // ---- values
        if (VM == 0) {
            // lane = channels 2 lane, 2 lane + 1; word G % 2 of tile G / 2 holds tokens 16 G .. 16 G + 15
            const uint32_t base = 0x3C003C00u, mask = 0x03000300u;
            const uint4* wq = reinterpret_cast<const uint4*>(wl);
#pragma unroll
            for (int G = 0; G < 4; ++G) {
                const uint4 wa = wq[2 * G], wb = wq[2 * G + 1];   // pairs (t, t + 8), t = 0..7
                const uint32_t wpair[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    const uint32_t x = cur.xv[4 * (G >> 1) + 2 * ch + (G & 1)];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const uint32_t y = t <= 4 ? (x << (8 - 2 * t)) : (x >> (2 * t - 8));
                        acc[4 * ch + (t & 3)] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, and_or(y, mask, base)),
                                                                       __builtin_bit_cast(half2_t, wpair[t]),
                                                                       acc[4 * ch + (t & 3)], false);
                    }
                }
            }
        } else {
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int tl = 2 * (pg + 8 * pass) + e;
                    const int tt = s0 + tl;
                    if (tt < t_end) {
                        const float wgt = wl[tl];
                        const float4* src = reinterpret_cast<const float4*>(vf + (size_t)tt * kD + 16 * jv);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 x = src[q];
                            acc[4 * q] = fmaf(wgt, x.x, acc[4 * q]);
                            acc[4 * q + 1] = fmaf(wgt, x.y, acc[4 * q + 1]);
                            acc[4 * q + 2] = fmaf(wgt, x.z, acc[4 * q + 2]);
                            acc[4 * q + 3] = fmaf(wgt, x.w, acc[4 * q + 3]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();   // next slab rewrites the weights
    }

    // ---- merge the eight wave streams: common max, then sums and the channel reduction
    if (lane == 0) red[wave][3] = m_run;
    __syncthreads();
    float m_blk = red[0][3];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m_blk = fmaxf(m_blk, red[i][3]);
    const float sc = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_blk);
    const float l_sum = wave_sum(l_t) * sc, mn_sum = wave_sum(mn_t) * sc, sw_sum = wave_sum(sw_t) * sc;
    if (lane == 0) {
        red[wave][0] = l_sum;
        red[wave][1] = mn_sum;
        red[wave][2] = sw_sum;
    }
    float* rbuf = lut;
    int nrows;
    if (VM == 0) {   // [8 waves][128 channels]
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
            rbuf[wave * kD + code_channel(2 * lane + ch)] = ((acc[4 * ch] + acc[4 * ch + 1]) + (acc[4 * ch + 2] + acc[4 * ch + 3])) * sc;
        nrows = kWaves;
    } else {         // [64 = wave x pair group][128 channels]
#pragma unroll
        for (int c = 0; c < 16; ++c) rbuf[(wave * 8 + pg) * kD + 16 * jv + c] = acc[c] * sc;
        nrows = kThreads / 8;
    }
    __syncthreads();
    if (tid < kD) {
        float tot = 0.f;
        for (int i = 0; i < nrows; ++i) tot += rbuf[i * kD + tid];
        float L = 0.f, MN = 0.f, SW = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            L += red[i][0];
            MN += red[i][1];
            SW += red[i][2];
        }
        const float o = VM == 0 ? fmaf(4.f, tot - SW, MN) : tot;
        float* dst = a.part + ((size_t)bhq * a.nsplit + split) * (kD + 2);
        dst[2 + tid] = o;
        if (tid == 0) {
            dst[0] = m_blk;
            dst[1] = L;
        }
    }
}

// ------------------------------------------------------------------------------------ combine
// One workgroup per (sequence, query head), one thread per channel: the log-sum-exp merge of the
// head's nsplit chunk partials (max, sum, unnormalized output) in one pass with a running maximum,
// so a thread's loads do not wait on each other or on a barrier and the merge costs one round trip
// to memory.  A separate launch: merging inside the decode kernel would need a device-scope
// release/acquire per workgroup, which on MI355X writes back and invalidates the XCD's whole L2.
// One chunk's partials into the running (M, L, O); a chunk with no valid token (mi = -inf) leaves them
// as they are.  Branch-free, so that the loads of every chunk can be in flight before the first merge.
__device__ __forceinline__ void merge_chunk(float mi, float li, float oi, float& M, float& L, float& O) {
    const bool skip = mi == -INFINITY;
    const float Mn = fmaxf(M, mi);
    const float keep = exp2f(M - Mn);            // 0 while M is still -inf
    const float f = exp2f(mi - Mn);
    L = skip ? L : fmaf(f, li, L * keep);
    O = skip ? O : fmaf(f, oi, O * keep);
    M = skip ? M : Mn;
}

__global__ __launch_bounds__(kD) void combine_kernel(DecodeArgs a) {
    constexpr int kFew = 16;                     // chunks whose partials are all requested before the merge
    const int c = threadIdx.x;
    const int bhq = blockIdx.x;
    const int ns = a.nsplit;
    const float* src = a.part + (size_t)bhq * ns * (kD + 2);
    float M = -INFINITY, L = 0.f, O = 0.f;
    if (ns <= kFew) {
        // one round trip: every chunk's (max, sum, value) is loaded first, then merged in chunk order
        float mi[kFew], li[kFew], oi[kFew];
#pragma unroll
        for (int i = 0; i < kFew; ++i) {
            const float* pi = src + (size_t)(i < ns ? i : ns - 1) * (kD + 2);   // past ns: a repeat, skipped
            const float m_ld = pi[0];
            mi[i] = i < ns ? m_ld : -INFINITY;
            li[i] = pi[1];
            oi[i] = pi[2 + c];
        }
#pragma unroll
        for (int i = 0; i < kFew; ++i) merge_chunk(mi[i], li[i], oi[i], M, L, O);
    } else {
#pragma unroll 4
        for (int i = 0; i < ns; ++i)
            merge_chunk(src[(size_t)i * (kD + 2)], src[(size_t)i * (kD + 2) + 1], src[(size_t)i * (kD + 2) + 2 + c], M, L, O);
    }
    a.out[(size_t)bhq * kD + c] = L > 0.f ? O / L : 0.f;
}

}  // namespace

namespace {

template <int WIN, int WOUT, int VM>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    const int groups = a.B * a.Hkv * a.nsplit;
    const int slots = (groups + 7) / 8;
    const unsigned nblocks = (unsigned)slots * 8u * (unsigned)a.g;
    timer_begin(TK_DECODE, s);
    hipLaunchKernelGGL((decode_kernel<WIN, WOUT, VM>), dim3(nblocks), dim3(kThreads), 0, s, a, groups);
    timer_end(TK_DECODE, s);
    return hipGetLastError();
}

template <int WIN, int WOUT>
hipError_t launch_decode_v(const DecodeArgs& a, int vmode, hipStream_t s) {
    return vmode == 0 ? launch_decode_t<WIN, WOUT, 0>(a, s) : launch_decode_t<WIN, WOUT, 1>(a, s);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
    timer_begin(TK_COMBINE, s);
    hipLaunchKernelGGL(combine_kernel, dim3(a.B * a.Hq), dim3(kD), 0, s, a);
    timer_end(TK_COMBINE, s);
    return hipGetLastError();
}

bool decode_uses_mfma(int m, int m_out, int vmode, int nbits) {
    const int win = m >> 5, wout = m_out >> 5;
    return vmode == 0 && (nbits >= 2 && nbits <= 4) && (win == 4 || win == 8 || win == 16) && (wout == 0 || wout == win) &&
           win + wout <= 16;
}

int decode_pick_nsplit(int B, int Hkv, int g, int64_t N, int m, int m_out) {
    (void)m;
    (void)m_out;
    // Work units: (sequence, KV head, group of 4 or 8 query heads); each context chunk of a unit is
    // one workgroup.  The chunks stream from HBM at the same rate when every CU holds the same number
    // of them, so a step lasts about ceil(units ns / 256) chunk lengths of N / ns tokens: pick the ns
    // that minimizes ceil(units ns / 256) / ns (the smallest such ns, for the fewest partials).
    constexpr int64_t kCUs = 256;
    const int hpg = 4 * decode_mfma_rowgroups(g);
    const int64_t units = (int64_t)B * Hkv * ((g + hpg - 1) / hpg);
    if (units <= 0) return 1;                          // empty batch: nothing is launched
    int64_t max_ns = (N + kDecodeTile - 1) / kDecodeTile;
    if (max_ns > 1024) max_ns = 1024;
    int64_t best = 1, best_rounds = (units + kCUs - 1) / kCUs;
    for (int64_t ns = 2; ns <= max_ns; ++ns) {
        const int64_t rounds = (units * ns + kCUs - 1) / kCUs;
        if (rounds * best < best_rounds * ns) {        // rounds / ns < best_rounds / best
            best = ns;
            best_rounds = rounds;
        }
    }
    return (int)best;
}

int64_t decode_chunk(int64_t N, int nsplit) {
    const int64_t per = (N + nsplit - 1) / nsplit;
    return ((per + kDecodeTile - 1) / kDecodeTile) * kDecodeTile;
}

hipError_t launch_decode(const DecodeArgs& a, int qdt, int vmode, hipStream_t s) {
    const int win = a.m >> 5, wout = a.m_out >> 5;
    if (a.path != 2 && decode_uses_mfma(a.m, a.m_out, vmode, vmode == 0 ? a.nbits : 2)) return launch_decode_mfma(a, qdt, s);
    timer_begin(TK_QPROJ, s);
    if (qdt == 0) hipLaunchKernelGGL(qproj_kernel<uint16_t>, dim3(a.B * a.Hq), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(qproj_kernel<float>, dim3(a.B * a.Hq), dim3(256), 0, s, a);
    timer_end(TK_QPROJ, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (win == 4 && wout == 0) e = launch_decode_v<4, 0>(a, vmode, s);
    else if (win == 4 && wout == 4) e = launch_decode_v<4, 4>(a, vmode, s);
    else if (win == 8 && wout == 0) e = launch_decode_v<8, 0>(a, vmode, s);
    else if (win == 8 && wout == 8) e = launch_decode_v<8, 8>(a, vmode, s);
    else if (win == 16 && wout == 0) e = launch_decode_v<16, 0>(a, vmode, s);
    else if (win == 16 && wout == 16) e = launch_decode_v<16, 16>(a, vmode, s);
    else return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
    return launch_combine(a, s);
}

bool decode_shape_supported(int m, int m_out) {
    const int win = m >> 5, wout = m_out >> 5;
    return (win == 4 || win == 8 || win == 16) && (wout == 0 || wout == win);
}

}  // namespace qjl

// Key quantization: JL projection on the matrix cores, sign extraction and bit packing fused into
// the epilogue, fp16 norms.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero Overhead",
// "Approach" (Gaussian JL transform of each key, keep the signs plus the key norm, outlier channels
// through a separate quantizer copy); 16-bit norm from "Your Brain Already Runs on 1-Bit Keys",
// "But Wait. Don't the Small Dims Overpower?".
//
// bf16 kernel layout (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//   * one workgroup = 8 waves; it owns one (sequence, KV head) and a range of tokens, walked in
//     chunks of 32 tokens (the MFMA N dimension);
//   * the JL matrix is stationary: each wave keeps its share of 32-row tiles of S_in (K = 128, eight
//     K steps) and of the outlier-channel columns of S_out (K = 16, one step) in VGPRs for the whole
//     workgroup lifetime;
//   * the key chunk is staged in LDS with the outlier channels zeroed (inlier operand) and the
//     outlier channels gathered into a 16-wide row (outlier operand); the loader threads also form
//     the two sums of squares for the norms;
//   * D = S_tile x K_chunk^T puts 16 projections of one token in each lane; the sign bits are shifted
//     into a word with v_alignbit, the two half-waves are merged with one cross-lane exchange, and
//     the S rows are permuted when loaded so that bit b of the word is projection 32*tile + b;
//   * words are staged in LDS and written with coalesced stores.
#include "qjl_common.h"


namespace qjl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTok = 32;        // tokens per chunk
constexpr int kKRow = 136;      // LDS row of one key in bf16 elements (272 B: conflict-free b128 reads)
constexpr int kGRow = 24;       // LDS row of the gathered outlier channels (48 B)
constexpr int64_t kSmallAppend = 16;   // tokens per sequence at or below which the flattened-row kernel runs

__device__ __forceinline__ float bf16_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// MFMA output row i (0..31) of a 32x32 tile holds projection tile_row(i) of that tile.  Lane l
// holds rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15; the packing loop leaves the sign of
// register r in bit 15 - r of the lane's half-word, and the half-wave l >= 32 supplies bits 16..31.
__device__ __forceinline__ int tile_row(int i) {
    const int half = (i >> 2) & 1;
    const int r = 4 * (i >> 3) + (i & 3);
    return 15 - r + 16 * half;
}

// Signs of one 32x32 tile -> one packed word per token (valid in lanes 0..31, lane = token).
// Bit = 1 iff the projection is >= 0: the sign bit of each accumulator is shifted in, then inverted.
__device__ __forceinline__ uint32_t pack_signs(const f32x16& acc, int lane) {
    uint32_t w = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) w = __builtin_amdgcn_alignbit(w, __float_as_uint(acc[r]), 31);
    const uint32_t other = lane_xor32(w);
    const uint32_t lo = lane < 32 ? w : other;
    const uint32_t hi = lane < 32 ? other : w;
    return ~(lo | (hi << 16));
}

// Signs of two 32x32 tiles at once: lane l < 32 gets tile a's word for token l, lane l + 32 tile b's
// word for token l (same bit order as pack_signs).  The lane's 32 sign bits (b's in the upper half)
// are swapped across the lane halves and one byte permute (sel: 0x05040100 in lanes 0..31,
// 0x07060302 in lanes 32..63) joins each tile's two half-words.
__device__ __forceinline__ uint32_t pack_sign_pair(const f32x16& a, const f32x16& b, uint32_t sel) {
    uint32_t w = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) w = __builtin_amdgcn_alignbit(w, __float_as_uint(b[r]), 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) w = __builtin_amdgcn_alignbit(w, __float_as_uint(a[r]), 31);
    // x[0]: the word of lane l % 32, x[1]: the word of lane l % 32 + 32
    const auto x = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return ~__builtin_amdgcn_perm(x[1], x[0], sel);
}

template <int N>
__device__ __forceinline__ void store_words(uint32_t* dst, const uint32_t (&w)[N]) {
    if constexpr (N == 1) dst[0] = w[0];
    else if constexpr (N == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    else {
        static_assert(N == 4, "one, two or four words per lane");
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Waves per SIMD the register budget must allow: two workgroups per CU for up to 512 inlier
// projections (TPW <= 2), one for more.
template <int TPW>
struct QKOccupancy { static constexpr int waves = TPW <= 2 ? 4 : 2; };

// One workgroup = one (sequence, KV head) and a token range.  The outlier columns of the
// stationary S_in fragments are zeroed once, so S_in k = S_in k_in and the key chunk is staged in
// LDS unmasked; the outlier operand (k gathered on the head's outlier channels, K = 16) is read
// back from the staged chunk.
constexpr int kTokH = 64;        // tokens per chunk of the per-head kernel (two MFMA N tiles)

template <int TPW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(QKOccupancy<TPW>::waves)))
void quantize_keys_bf16_kernel(KeyQuantArgs a) {
    constexpr int NW = kWaves;
    constexpr int NT = kThreads;
    __shared__ __attribute__((aligned(16))) uint16_t kl[2][kTokH * kKRow];
    __shared__ uint32_t ol[2][kTokH * (kMaxBits / 32 + 1)];
    __shared__ int s_oidx[kMaxOutliers];
    __shared__ uint4 sout_l[TPW][NW][64];                            // gathered S_out fragments

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_block;
    const int64_t t_end = min(a.T, t_begin + (int64_t)a.tokens_per_block);
    const int n_out = a.n_out;
    const int Win = a.m >> 5;
    const int Wout = a.m_out >> 5;
    const int W = a.W;
    const int orow = W + 1;

    if (tid < n_out) s_oidx[tid] = a.oidx[h * n_out + tid] & (kD - 1);   // never index outside a row
    __syncthreads();

    // loader role: tokens tt and tt + 32 of the chunk, channels 8*cg .. 8*cg+7
    const int tt = tid >> 4;
    const int cg = tid & 15;
    uint32_t keep_out[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < n_out; ++i) {
        const int c = s_oidx[i];
        if ((c >> 3) == cg) keep_out[(c & 7) >> 1] |= (c & 1) ? 0xFFFF0000u : 0x0000FFFFu;
    }

    const uint16_t* K = static_cast<const uint16_t*>(a.K);
    const int64_t head_row0 = ((int64_t)b * a.Hkv + h) * a.Ncap + a.t0;
    const uint16_t* krow = K + b * a.sKb + h * a.sKh + 8 * cg;
    uint32_t* norms32 = reinterpret_cast<uint32_t*>(a.norms);

    // first chunk in flight while the stationary JL fragments load
    uint4 kv0 = make_uint4(0u, 0u, 0u, 0u), kv1 = make_uint4(0u, 0u, 0u, 0u);
    if (t_begin + tt < t_end) kv0 = *reinterpret_cast<const uint4*>(krow + (t_begin + tt) * a.sKt);
    if (t_begin + tt + 32 < t_end) kv1 = *reinterpret_cast<const uint4*>(krow + (t_begin + tt + 32) * a.sKt);

    const uint16_t* Sin = static_cast<const uint16_t*>(a.S_in);
    const uint16_t* Sout = static_cast<const uint16_t*>(a.S_out);
    const int prow = tile_row(lane & 31);
    const int khalf = (lane >> 5) * 8;
    uint4 sin_frag[TPW][8];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int j = wave + NW * i;
        if (j < Win) {
            const uint16_t* row = Sin + (size_t)(32 * j + prow) * kD + khalf;
#pragma unroll
            for (int s = 0; s < 8; ++s) sin_frag[i][s] = *reinterpret_cast<const uint4*>(row + 16 * s);
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) sin_frag[i][s] = make_uint4(0u, 0u, 0u, 0u);
        }
        uint32_t g[4] = {0u, 0u, 0u, 0u};
        if (j < Wout) {
            const uint16_t* row = Sout + (size_t)(32 * j + prow) * kD;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = khalf + e;
                const uint32_t v = k < n_out ? row[s_oidx[k]] : 0u;
                g[e >> 1] |= v << (16 * (e & 1));
            }
        }
        sout_l[i][wave][lane] = make_uint4(g[0], g[1], g[2], g[3]);
    }
    for (int i = 0; i < n_out; ++i) {       // S_in k = S_in k_in: zero the outlier columns
        const int c = s_oidx[i];
        const int s = c >> 4, off = c & 15;
        if ((off >> 3) == (khalf >> 3)) {
            const int e = off & 7;
            const uint32_t m = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int ss = 0; ss < 8; ++ss)
                    if (ss == s) {
                        uint32_t* f = reinterpret_cast<uint32_t*>(&sin_frag[t][ss]);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (q == (e >> 1)) f[q] &= m;
                    }
        }
    }

    // stage one token row: unmasked key to LDS, the two sums of squares, its norms
    auto stage = [&](uint4 v, uint16_t* dst, int tok, int64_t tglob) {
        *reinterpret_cast<uint4*>(dst + tok * kKRow + 8 * cg) = v;
        const uint32_t kw[4] = {v.x, v.y, v.z, v.w};
        float ss_in = 0.f, ss_out = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t o = kw[q] & keep_out[q];
            const uint32_t n = kw[q] & ~keep_out[q];
            ss_out = dot2_bf16(o, o, ss_out);
            ss_in = dot2_bf16(n, n, ss_in);
        }
        ss_in = row16_sum(ss_in);       // the 16 loader lanes of a token are one DPP row
        ss_out = row16_sum(ss_out);
        if (cg == 0 && tglob < t_end) norms32[head_row0 + tglob] = norm_pair(ss_in, ss_out);
    };

    stage(kv0, kl[0], tt, t_begin + tt);
    stage(kv1, kl[0], tt + 32, t_begin + tt + 32);
    __syncthreads();

    const int my_tok = lane & 31;
    int buf = 0;
    for (int64_t c0 = t_begin; c0 < t_end; c0 += kTokH) {
        const int nvalid = (int)min((int64_t)kTokH, t_end - c0);
        const int64_t cn = c0 + kTokH;

        // next chunk's keys in flight during this chunk's matrix work
        uint4 kn0 = make_uint4(0u, 0u, 0u, 0u), kn1 = make_uint4(0u, 0u, 0u, 0u);
        if (cn + tt < t_end) kn0 = *reinterpret_cast<const uint4*>(krow + (cn + tt) * a.sKt);
        if (cn + tt + 32 < t_end) kn1 = *reinterpret_cast<const uint4*>(krow + (cn + tt + 32) * a.sKt);

        // ---- projections on the matrix cores
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int j = wave + NW * i;
            if (j < Win) {
                {
#pragma unroll
                    for (int nh = 0; nh < 2; ++nh) {
                        const uint16_t* klb = kl[buf] + (32 * nh + my_tok) * kKRow + khalf;
                        f32x16 acc = {};
#pragma unroll
                        for (int s = 0; s < 8; ++s)
                            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sin_frag[i][s]),
                                                                          as_bf16x8(*reinterpret_cast<const uint4*>(klb + 16 * s)), acc, 0, 0, 0);
                        const uint32_t w = pack_signs(acc, lane);
                        if (lane < 32) ol[buf][(32 * nh + lane) * orow + j] = w;
                    }
                }
            }
        }
        if (Wout > wave) {
#pragma unroll
            for (int nh = 0; nh < 2; ++nh) {
                // outlier operand: this lane's token, gathered on the head's outlier channels
                uint32_t g[4] = {0u, 0u, 0u, 0u};
                const uint16_t* krw = kl[buf] + (32 * nh + my_tok) * kKRow;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = khalf + e;
                    if (k < n_out) g[e >> 1] |= (uint32_t)krw[s_oidx[k]] << (16 * (e & 1));
                }
                const uint4 gfrag = make_uint4(g[0], g[1], g[2], g[3]);
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int j = wave + NW * i;
                    if (j < Wout) {
                        f32x16 ao = {};
                        ao = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(sout_l[i][wave][lane]), as_bf16x8(gfrag), ao, 0, 0, 0);
                        const uint32_t w = pack_signs(ao, lane);
                        if (lane < 32) ol[buf][(32 * nh + lane) * orow + Win + j] = w;
                    }
                }
            }
        }
        // ---- stage the next chunk into the other buffer (its last readers passed the previous barrier)
        if (cn < t_end) {
            stage(kn0, kl[buf ^ 1], tt, cn + tt);
            stage(kn1, kl[buf ^ 1], tt + 32, cn + tt + 32);
        }
        __syncthreads();

        // ---- coalesced store of this chunk's packed words
        uint32_t* dst = a.bits + (head_row0 + c0) * W;
        const uint32_t* olb = ol[buf];
        const int w = tid & 31;
        if (w < W) {
            const int slot = bits_slot(w, Win, Wout);
            for (int tok = tid >> 5; tok < nvalid; tok += NT / 32) dst[tok * W + slot] = olb[tok * orow + w];
        }
        buf ^= 1;
    }
}

// Sketches with m <= 512 and m_out <= 512: the JL matrices stay in LDS for the whole workgroup (S_in
// with its outlier columns zeroed; S_out gathered on the head's outlier channels in rank order, 16
// per row), loaded once.  Each wave then streams its own 32-token blocks with no further barrier:
// the keys of a block go from global memory straight into the MFMA B operand (lane l: token l % 32,
// channels 16 s + 8 (l / 32) .. + 7), the A operands (32 projections x 16 channels) come from LDS,
// and the two lanes of a token store its sign words quarter-row group by group (the group's words
// are consecutive slots of the stored row).  The norms come from the same registers: |k_in|^2 with the
// outlier channels masked out (S_in has zero columns there, so the projections need no masking),
// |k_out|^2 from the gathered operand.
constexpr int kOGRow = 16;                   // gathered S_out row (bf16)
// S_in row in LDS (bf16, 272 B): the 16-byte A-fragment reads of a wave, in the MFMA's row order,
// fall on distinct banks (measured: such a 64-lane b128 read runs at the full LDS rate)
constexpr int kSRowL = kD + 8;


constexpr int kLWaves = 16;                  // one workgroup per CU: 4 waves per SIMD
constexpr int kLThreads = 64 * kLWaves;

template <int WIN, int WOUT>
__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(4)))
void quantize_keys_lds_kernel(KeyQuantArgs a) {
    constexpr int W = WIN + WOUT;
    __shared__ __attribute__((aligned(16))) uint16_t sl[WIN * 32 * kSRowL];
    __shared__ __attribute__((aligned(16))) uint16_t so[(WOUT > 0 ? WOUT : 1) * 32 * kOGRow];
    __shared__ int s_oidx[kMaxOutliers];
    __shared__ uint32_t s_keep[2 * 32];          // keep masks of the 32 key words of each lane half
    __shared__ uint32_t s_goff[2 * 8];           // byte offsets of the gathered channels of each lane half
    __shared__ int s_next;                       // next unclaimed 32-token block of the workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_block;
    const int64_t t_end = min(a.T, t_begin + (int64_t)a.tokens_per_block);
    const int n_out = a.n_out;

    if (tid < n_out) s_oidx[tid] = a.oidx[h * n_out + tid] & (kD - 1);   // never index outside a row
    if (tid == 0) s_next = kLWaves;              // blocks 0 .. kLWaves - 1 go to waves 0 .. kLWaves - 1
    __syncthreads();
    if (tid < 64) {
        // word w = 4 s + q of lane half hf holds channels 16 s + 8 hf + 2 q, + 1
        const int hf = tid >> 5, w = tid & 31;
        const int c0 = 16 * (w >> 2) + 8 * hf + 2 * (w & 3);
        uint32_t keep = 0xFFFFFFFFu;
        for (int k = 0; k < n_out; ++k) {
            if (s_oidx[k] == c0) keep &= 0xFFFF0000u;
            if (s_oidx[k] == c0 + 1) keep &= 0x0000FFFFu;
        }
        s_keep[tid] = keep;
    } else if (tid < 80) {
        // rank r = 8 hf + e of the gathered operand: its channel, or an offset past any buffer (reads 0)
        const int r = tid - 64;
        s_goff[r] = r < n_out ? 2u * (uint32_t)s_oidx[r] : 0x7FFFFF00u;
    }
    {
        // every load of a thread is issued before the first LDS store: one round trip to L2, not one
        // per element
        constexpr int NSI = WIN * 32 * 16 / kLThreads, NSO = WOUT * 32 * kOGRow / kLThreads;
        static_assert(NSI * kLThreads == WIN * 32 * 16 && NSO * kLThreads == WOUT * 32 * kOGRow, "whole rounds");
        const uint16_t* Sin = static_cast<const uint16_t*>(a.S_in);
        const uint16_t* Sout = static_cast<const uint16_t*>(a.S_out);
        uint4 v[NSI > 0 ? NSI : 1];
        uint16_t go[NSO > 0 ? NSO : 1];
#pragma unroll
        for (int u = 0; u < NSI; ++u) {
            const int i = tid + u * kLThreads;
            v[u] = *reinterpret_cast<const uint4*>(Sin + (size_t)(i >> 4) * kD + 8 * (i & 15));
        }
#pragma unroll
        for (int u = 0; u < NSO; ++u) {
            const int i = tid + u * kLThreads;
            const int j = i / kOGRow, r = i % kOGRow;
            go[u] = r < n_out ? Sout[(size_t)j * kD + s_oidx[r]] : (uint16_t)0;
        }
        // this thread's 8 channels 8 cgi .. 8 cgi + 7 are the same in every round: their keep masks
        // (outlier channels zeroed) are built once, per lane, with no branch on the channel list
        const int cgi = tid & 15;
        uint32_t outl = 0;                               // bit e: channel 8 cgi + e is an outlier
        for (int k = 0; k < n_out; ++k) {
            const int c = s_oidx[k];
            outl |= ((c >> 3) == cgi ? 1u : 0u) << (c & 7);
        }
        uint32_t keepw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            keepw[q] = (((outl >> (2 * q)) & 1u) ? 0xFFFF0000u : 0xFFFFFFFFu) & (((outl >> (2 * q + 1)) & 1u) ? 0x0000FFFFu : 0xFFFFFFFFu);
#pragma unroll
        for (int u = 0; u < NSI; ++u) {
            const int i = tid + u * kLThreads;
            const int r = i >> 4;
            *reinterpret_cast<uint4*>(sl + r * kSRowL + 8 * cgi) =
                make_uint4(v[u].x & keepw[0], v[u].y & keepw[1], v[u].z & keepw[2], v[u].w & keepw[3]);
        }
#pragma unroll
        for (int u = 0; u < NSO; ++u) {
            const int i = tid + u * kLThreads;
            const int j = i / kOGRow, r = i % kOGRow;
            // the two 8-rank halves of row j swap places when bit 4 of the row is set
            so[j * kOGRow + (r ^ (((j >> 4) & 1) << 3))] = go[u];
        }
    }
    __syncthreads();

    const int tcol = lane & 31;
    const int hf = lane >> 5;
    const int khalf = hf * 8;
    const int prow = tile_row(lane & 31);
    const uint32_t psel = hf ? 0x07060302u : 0x05040100u;
    // this (sequence, head)'s key rows up to the end of the last valid token: loads of tokens past
    // t_end (and of the unused gathered ranks) fall outside and return zeros
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(static_cast<const uint16_t*>(a.K) + b * a.sKb + h * a.sKh,
                                                  (uint32_t)((t_end - 1) * a.sKt * 2 + kD * 2));
    const int64_t head_row0 = ((int64_t)b * a.Hkv + h) * a.Ncap + a.t0;
    uint32_t* norms32 = reinterpret_cast<uint32_t*>(a.norms);
    // A fragment of tile j, K step s: arow + 32 j kSRowL + 16 s
    const uint16_t* arow = sl + prow * kSRowL + khalf;
    // gathered S_out fragment of tile j: orow + 32 j kOGRow
    const uint16_t* orow = so + prow * kOGRow + 8 * ((khalf >> 3) ^ ((prow >> 4) & 1));
    const uint32_t* keep = s_keep + (lane >> 5) * 32;
    const uint32_t* goff = s_goff + (lane >> 5) * 8;

    auto load_keys = [&](int64_t tk, const uint32_t* goffb, uint4 (&bk)[8], uint4& bg) {
        const uint32_t voff = (uint32_t)(tk * a.sKt * 2);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 2 * khalf + 32 * s, 0, 0);
            bk[s] = make_uint4(x[0], x[1], x[2], x[3]);
        }
        uint32_t g[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rk, voff + goffb[2 * q], 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rk, voff + goffb[2 * q + 1], 0, 0);
            g[q] = lo | (hi << 16);
        }
        bg = make_uint4(g[0], g[1], g[2], g[3]);
    };

    // Blocks are claimed one at a time from an LDS counter: the four waves of a SIMD progress at
    // different rates, and with a fixed share per wave the workgroup would end with its slowest wave
    // while the others sit idle (measured: 4 blocks per wave took 38 to 74 us).
    const int64_t nblk = (t_end - t_begin + 31) / 32;
    for (int64_t blk = wave; blk < nblk;) {
        const int64_t t0b = t_begin + 32 * blk;
        const int64_t tk = t0b + tcol;
        // the mask tables are read per block, not held in registers across the loop
        int opaque = 0;
        asm volatile("" : "+v"(opaque));
        const uint32_t* keepb = keep + opaque;
        const uint32_t* goffb = goff + opaque;
        uint4 bk[8], bg;
        load_keys(tk, goffb, bk, bg);

        // norms: |k_in|^2 over this lane's channels outside the outlier set, |k_out|^2 over its gathered ranks
        float si = 0.f, sg = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint4 m = *reinterpret_cast<const uint4*>(keepb + 4 * q);
            si = dot2_bf16(bk[q].x & m.x, bk[q].x, si);
            si = dot2_bf16(bk[q].y & m.y, bk[q].y, si);
            si = dot2_bf16(bk[q].z & m.z, bk[q].z, si);
            si = dot2_bf16(bk[q].w & m.w, bk[q].w, si);
        }
        sg = dot2_bf16(bg.x, bg.x, sg);
        sg = dot2_bf16(bg.y, bg.y, sg);
        sg = dot2_bf16(bg.z, bg.z, sg);
        sg = dot2_bf16(bg.w, bg.w, sg);
        si += __uint_as_float(lane_xor32(__float_as_uint(si)));
        sg += __uint_as_float(lane_xor32(__float_as_uint(sg)));
        if (lane < 32 && tk < t_end) norms32[head_row0 + tk] = norm_pair(si, sg);

        // projections by quarter-row group g of the stored row (inlier words g WIN/4 .., then outlier
        // words g WOUT/4 ..: consecutive slots g W/4 ..), two independent MFMA chains at a time.  Tiles
        // are packed in pairs: lanes 0..31 keep the first tile's word, lanes 32..63 the second's.  With
        // an outlier sketch, inlier tile p pairs with outlier tile p, so for token t of the block lane t
        // holds the group's inlier words and lane t + 32 its outlier words: one store per lane.
        constexpr int GI = WIN / 4, GO = WOUT / 4;
        static_assert(GO == 0 || GO == GI, "outlier tiles pair with inlier tiles");
        uint32_t* row = a.bits + (head_row0 + tk) * W;
        const bool live = tk < t_end;
#pragma unroll 1
        for (int g = 0; g < 4; ++g) {
            uint32_t* dst = row + g * (W / 4);
            if constexpr (GO > 0) {
                uint32_t wd[GI];
#pragma unroll
                for (int p = 0; p < GI; p += 2) {
                    const uint16_t* a0p = arow + 32 * (g * GI + p) * kSRowL;
                    const uint16_t* o0p = orow + 32 * (g * GO + p) * kOGRow;
                    if constexpr (GI >= 2) {
                        f32x16 a0 = {}, a1 = {};
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(a0p + 16 * s)),
                                                                         as_bf16x8(bk[s]), a0, 0, 0, 0);
                            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                as_bf16x8(*reinterpret_cast<const uint4*>(a0p + 32 * kSRowL + 16 * s)), as_bf16x8(bk[s]), a1, 0, 0, 0);
                        }
                        const f32x16 o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(*reinterpret_cast<const uint4*>(o0p)), as_bf16x8(bg), f32x16{}, 0, 0, 0);
                        const f32x16 o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(*reinterpret_cast<const uint4*>(o0p + 32 * kOGRow)), as_bf16x8(bg), f32x16{}, 0, 0, 0);
                        wd[p] = pack_sign_pair(a0, o0, psel);
                        wd[p + 1] = pack_sign_pair(a1, o1, psel);
                    } else {
                        f32x16 a0 = {};
#pragma unroll
                        for (int s = 0; s < 8; ++s)
                            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(a0p + 16 * s)),
                                                                         as_bf16x8(bk[s]), a0, 0, 0, 0);
                        const f32x16 o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(*reinterpret_cast<const uint4*>(o0p)), as_bf16x8(bg), f32x16{}, 0, 0, 0);
                        wd[p] = pack_sign_pair(a0, o0, psel);
                    }
                }
                if (live) store_words<GI>(dst + hf * GI, wd);
            } else if constexpr (GI >= 2) {
                // pairs (p, p + GI/2): lanes 0..31 hold words 0 .. GI/2 - 1 of the group, 32..63 the rest
                uint32_t wi[GI / 2];
#pragma unroll
                for (int p = 0; p < GI / 2; ++p) {
                    const uint16_t* a0p = arow + 32 * (g * GI + p) * kSRowL;
                    const uint16_t* a1p = a0p + 32 * (GI / 2) * kSRowL;
                    f32x16 a0 = {}, a1 = {};
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(a0p + 16 * s)),
                                                                     as_bf16x8(bk[s]), a0, 0, 0, 0);
                        a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(a1p + 16 * s)),
                                                                     as_bf16x8(bk[s]), a1, 0, 0, 0);
                    }
                    wi[p] = pack_sign_pair(a0, a1, psel);
                }
                if (live) store_words<GI / 2>(dst + hf * (GI / 2), wi);
            } else {
                f32x16 a0 = {};
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(*reinterpret_cast<const uint4*>(arow + 32 * g * kSRowL + 16 * s)), as_bf16x8(bk[s]), a0, 0, 0, 0);
                const uint32_t w = pack_signs(a0, lane);
                if (lane < 32 && live) dst[0] = w;
            }
        }
        int claim = 0;
        if (lane == 0) claim = atomicAdd(&s_next, 1);
        blk = __builtin_amdgcn_readfirstlane(claim);
    }
}

// Small appends (a few new tokens per sequence, e.g. one per decode step): every 32 key rows of any
// (sequence, KV head, token) form one MFMA chunk.  The outlier sketch is computed with the
// full-width S_out on the outlier-only key (zeros on the other channels), so the JL operands are
// the same for every row and one workgroup covers rows of all heads: the JL matrices are read once
// per 32 rows instead of once per (sequence, head).
constexpr int kMaxTilesPerWave = 4;          // (m + m_out) / 32 / 8 waves

template <int TT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void quantize_keys_rows_kernel(KeyQuantArgs a, int64_t rows) {
    __shared__ __attribute__((aligned(16))) uint16_t kl[kTok * kKRow];   // inlier channels
    __shared__ __attribute__((aligned(16))) uint16_t ko[kTok * kKRow];   // outlier channels
    __shared__ uint32_t ol[kTok * (kMaxBits / 32 + 1)];
    __shared__ int64_t s_dst[kTok];
    extern __shared__ uint32_t s_mask[];                                   // [Hkv][4] outlier masks

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Win = a.m >> 5, Wout = a.m_out >> 5, W = a.W, orow = W + 1;
    const int64_t r0 = (int64_t)blockIdx.x * kTok;

    for (int hh = tid; hh < a.Hkv; hh += kThreads) {
        // the head's outlier list as independent loads (one round trip), then its 128-bit mask
        int cl[kMaxOutliers];
#pragma unroll
        for (int i = 0; i < kMaxOutliers; ++i) cl[i] = i < a.n_out ? (a.oidx[hh * a.n_out + i] & (kD - 1)) : -1;
        uint32_t mk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kMaxOutliers; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (cl[i] >= 0 && (cl[i] >> 5) == q) mk[q] |= 1u << (cl[i] & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) s_mask[hh * 4 + q] = mk[q];
    }

    // stationary JL tiles of this wave: global tile gt = wave + 8 i over [inlier tiles, outlier tiles]
    const int prow = tile_row(lane & 31);
    const int khalf = (lane >> 5) * 8;
    uint4 frag[TT][8];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int gt = wave + kWaves * i;
        const uint16_t* row = nullptr;
        if (gt < Win) row = static_cast<const uint16_t*>(a.S_in) + (size_t)(32 * gt + prow) * kD + khalf;
        else if (gt < Win + Wout) row = static_cast<const uint16_t*>(a.S_out) + (size_t)(32 * (gt - Win) + prow) * kD + khalf;
#pragma unroll
        for (int s = 0; s < 8; ++s) frag[i][s] = row ? *reinterpret_cast<const uint4*>(row + 16 * s) : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    // ---- stage 32 rows: split into inlier / outlier halves, norms
    const int tt = tid >> 4, cg = tid & 15;
    const int64_t r = r0 + tt;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
    uint32_t om = 0;
    if (r < rows) {
        const int64_t t = r % a.T, bh = r / a.T;
        const int h = (int)(bh % a.Hkv);
        const int64_t b = bh / a.Hkv;
        kv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.K) + b * a.sKb + t * a.sKt + h * a.sKh + 8 * cg);
        om = (s_mask[h * 4 + (cg >> 2)] >> (8 * (cg & 3))) & 0xFFu;
        if (cg == 0) s_dst[tt] = ((int64_t)b * a.Hkv + h) * a.Ncap + a.t0 + t;
    }
    {
        uint4 kin, kout;
        float ss_in = 0.f, ss_out = 0.f;
        split_key8(kv, om, kin, kout, ss_in, ss_out);
        *reinterpret_cast<uint4*>(kl + tt * kKRow + 8 * cg) = kin;
        *reinterpret_cast<uint4*>(ko + tt * kKRow + 8 * cg) = kout;
        ss_in = row16_sum(ss_in);
        ss_out = row16_sum(ss_out);
        __syncthreads();
        if (cg == 0 && r < rows) reinterpret_cast<uint32_t*>(a.norms)[s_dst[tt]] = norm_pair(ss_in, ss_out);
    }

    // ---- projections and sign packing
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        const int gt = wave + kWaves * i;
        if (gt < Win + Wout) {
            const uint16_t* src = (gt < Win ? kl : ko) + (lane & 31) * kKRow + khalf;
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < 8; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(frag[i][s]),
                                                              as_bf16x8(*reinterpret_cast<const uint4*>(src + 16 * s)), acc, 0, 0, 0);
            const uint32_t w = pack_signs(acc, lane);
            if (lane < 32) ol[lane * orow + gt] = w;
        }
    }
    __syncthreads();
    const int nvalid = (int)min((int64_t)kTok, rows - r0);
    for (int i = tid; i < nvalid * W; i += kThreads) {
        const int tok = i / W, w = i - tok * W;
        a.bits[s_dst[tok] * W + bits_slot(w, Win, Wout)] = ol[tok * orow + w];
    }
}

// fp32 keys and JL matrix (VALU, one wave per key): exact fp32 fused multiply-adds in channel order.
constexpr int kF32Tok = 4;

__global__ __launch_bounds__(256) void quantize_keys_f32_kernel(KeyQuantArgs a) {
    __shared__ float kin[kF32Tok][kD];
    __shared__ float kout[kF32Tok][kD];
    __shared__ int s_oidx[kMaxOutliers];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t t = (int64_t)blockIdx.x * kF32Tok + wave;
    const bool valid = t < a.T;
    if (tid < a.n_out) s_oidx[tid] = a.oidx[h * a.n_out + tid] & (kD - 1);
    __syncthreads();
    const float* K = static_cast<const float*>(a.K);
    float ss_in = 0.f, ss_out = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = 2 * lane + q;
        const float v = valid ? K[b * a.sKb + t * a.sKt + h * a.sKh + c] : 0.f;
        bool is_out = false;
        for (int i = 0; i < a.n_out; ++i) is_out |= (s_oidx[i] == c);
        kin[wave][c] = is_out ? 0.f : v;
        kout[wave][c] = is_out ? v : 0.f;
        if (is_out) ss_out = fmaf(v, v, ss_out); else ss_in = fmaf(v, v, ss_in);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        ss_in += __shfl_xor(ss_in, o);
        ss_out += __shfl_xor(ss_out, o);
    }
    __syncthreads();
    if (!valid) return;
    const int64_t row = ((int64_t)b * a.Hkv + h) * a.Ncap + a.t0 + t;
    if (lane == 0) {
        const _Float16 ni = (_Float16)sqrtf(ss_in), no = (_Float16)sqrtf(ss_out);
        reinterpret_cast<uint32_t*>(a.norms)[row] =
            (uint32_t)__builtin_bit_cast(uint16_t, ni) | ((uint32_t)__builtin_bit_cast(uint16_t, no) << 16);
    }
    const float* Sin = static_cast<const float*>(a.S_in);
    const float* Sout = static_cast<const float*>(a.S_out);
    const int total = a.m + a.m_out;
    for (int g = 0; 64 * g < total; ++g) {
        const int r = 64 * g + lane;
        float p = 0.f;
        if (r < a.m) {
            const float* srow = Sin + (size_t)r * kD;
            for (int c = 0; c < kD; ++c) p = fmaf(srow[c], kin[wave][c], p);
        } else if (r < total) {
            const float* srow = Sout + (size_t)(r - a.m) * kD;
            for (int c = 0; c < kD; ++c) p = fmaf(srow[c], kout[wave][c], p);
        }
        const uint64_t bal = __ballot(r < total && p >= 0.f);
        if (lane == 0) {
            uint32_t* dst = a.bits + row * a.W;
            const int win = a.m >> 5, wout = a.m_out >> 5;
            if (2 * g < a.W) dst[bits_slot(2 * g, win, wout)] = (uint32_t)bal;
            if (2 * g + 1 < a.W) dst[bits_slot(2 * g + 1, win, wout)] = (uint32_t)(bal >> 32);
        }
    }
}

}  // namespace

hipError_t launch_quantize_keys_bf16(const KeyQuantArgs& a, int B, hipStream_t s) {
    if (a.T <= kSmallAppend) {
        // few tokens per sequence: flattened rows, one JL load per 32 rows of all heads
        const int64_t rows = (int64_t)B * a.Hkv * a.T;
        const int tt = ((a.m >> 5) + (a.m_out >> 5) + kWaves - 1) / kWaves;
        const dim3 grid((unsigned)((rows + kTok - 1) / kTok));
        const size_t lds = (size_t)a.Hkv * 4 * sizeof(uint32_t);
        if (tt <= 1) hipLaunchKernelGGL(quantize_keys_rows_kernel<1>, grid, dim3(kThreads), lds, s, a, rows);
        else if (tt == 2) hipLaunchKernelGGL(quantize_keys_rows_kernel<2>, grid, dim3(kThreads), lds, s, a, rows);
        else hipLaunchKernelGGL(quantize_keys_rows_kernel<4>, grid, dim3(kThreads), lds, s, a, rows);
        return hipGetLastError();
    }
    const int tiles = (a.m >> 5) > (a.m_out >> 5) ? (a.m >> 5) : (a.m_out >> 5);
    dim3 grid((unsigned)((a.T + a.tokens_per_block - 1) / a.tokens_per_block), (unsigned)a.Hkv, (unsigned)B);
    // the LDS-resident kernel addresses one (sequence, head)'s key rows with 32-bit buffer offsets
    if (quantize_keys_lds_shape(a.m, a.m_out) && a.T * a.sKt * 2 + 256 < ((int64_t)1 << 31)) {
        const int wi = a.m >> 5, wo = a.m_out >> 5;
#define QK_LDS(WI, WO) hipLaunchKernelGGL((quantize_keys_lds_kernel<WI, WO>), grid, dim3(kLThreads), 0, s, a)
        if (wi == 16 && wo == 16) QK_LDS(16, 16);
        else if (wi == 16 && wo == 0) QK_LDS(16, 0);
        else if (wi == 8 && wo == 8) QK_LDS(8, 8);
        else if (wi == 8 && wo == 0) QK_LDS(8, 0);
        else if (wi == 4 && wo == 4) QK_LDS(4, 4);
        else QK_LDS(4, 0);
#undef QK_LDS
        return hipGetLastError();
    }
    if (tiles <= 8) hipLaunchKernelGGL(quantize_keys_bf16_kernel<1>, grid, dim3(kThreads), 0, s, a);
    else if (tiles <= 16) hipLaunchKernelGGL(quantize_keys_bf16_kernel<2>, grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(quantize_keys_bf16_kernel<4>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_quantize_keys_f32(const KeyQuantArgs& a, int B, hipStream_t s) {
    dim3 grid((unsigned)((a.T + kF32Tok - 1) / kF32Tok), (unsigned)a.Hkv, (unsigned)B);
    hipLaunchKernelGGL(quantize_keys_f32_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace qjl

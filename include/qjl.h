/*
 * qjl.h - C ABI of libqjl: 1-bit QJL KV-cache key compression and decode attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (page "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero
 * Overhead", sections "Approach" and "Surprising findings"): every key k is projected with a
 * Gaussian JL matrix S (m x d) and only the signs of S k are kept, plus the key norm; outlier
 * channels go through a separate copy of the quantizer; the query is projected without
 * quantization, and the inner product is estimated by the unbiased asymmetric estimator
 *
 *     score(q, k) = sqrt(pi/2)/m * |k_in| * <S_in q_in, sign(S_in k_in)>
 *                 + sqrt(pi/2)/m_out * |k_out| * <S_out q_out, sign(S_out k_out)>
 *
 * where x_in / x_out are x with its outlier channels / its other channels set to zero.  Values use
 * token-wise min/max quantization (same page, "Limitations"; page "2 numbers out of 128 destroy the
 * entire KV cache", section "The Obvious Fix: Use Fewer Bits").  Decode attention is softmax over
 * sm_scale * score followed by the weighted sum of the dequantized values.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller; the library never allocates,
 *     frees, or synchronizes.  Work is enqueued on `stream` (0 = the null stream) and returns
 *     immediately; results are valid once the stream reaches that point.
 *   - Argument errors are detected on the host before anything is enqueued and returned as a
 *     negative qjl_status; nothing is written then.  A failed launch returns QJL_ERR_HIP.
 *     qjl_last_error() gives a human-readable detail of the last error on the calling thread.
 *   - Supported shapes: head dimension d = 128; m and m_out multiples of 128 with 128 <= m,
 *     0 <= m_out, m + m_out <= 1024; 0 <= n_out <= 16 outlier channels per KV head, n_out > 0 only
 *     with m_out > 0; Hq a multiple of Hkv.  Query head hq reads KV head hq / (Hq / Hkv).
 *   - Every device pointer must be 16-byte aligned, and the model-layout strides must keep every
 *     d-vector 16-byte aligned (QJL_ERR_MISALIGNED otherwise).
 *   - Stateless and thread-safe; calls on different streams may overlap.
 *
 * Cache layout in HBM (per sequence b, KV head h, token position t < Ncap):
 *   bits  uint32 [B][Hkv][Ncap][W], W = (m + m_out) / 32.  Sign word w (w < W) has bit i set iff
 *         projection 32 w + i is >= 0 (sign(0) taken as +1); words 0 .. Win-1 (Win = m/32) hold the
 *         inlier sketch, words Win .. W-1 (Wout = m_out/32 of them) the outlier sketch.  A token's
 *         row stores its W words as 4 groups of W/4: group j (j = 0..3) holds inlier words
 *         j Win/4 .. (j+1) Win/4 - 1 followed by outlier words Win + j Wout/4 .. Win + (j+1) Wout/4 - 1,
 *         so row slot j W/4 + r holds inlier word j Win/4 + r for r < Win/4 and outlier word
 *         Win + j Wout/4 + r - Win/4 otherwise.  (Each quarter of a row is what one lane group of a
 *         matrix-core operand consumes; one load per token and lane.)
 *   norms fp16  [B][Hkv][Ncap][2]: (|k_in|, |k_out|) as IEEE binary16 round-to-nearest-even.
 *   codes uint32 [B][Hkv][Ncap32/32][d][nbits], Ncap32 = Ncap rounded up to a multiple of 32: the
 *         positions are grouped in tiles of 32 (tile i covers positions 32 i .. 32 i + 31).  For each
 *         channel c a tile holds the codes of its 32 positions in nbits words: for nbits 2, position
 *         32 i + j in bits [2j, 2j + 2) of the LSB-first 64-bit stream; for nbits 4, word w holds
 *         positions 32 i + 16 floor(w/2) + 2 e + (w mod 2) in its nibbles e = 0..7 (so each 2-bit
 *         plane of a 4-bit word lists its positions in the same order as a 2-bit stream); for nbits 3,
 *         words 0 and 1 hold the low two bits of every code exactly as a 2-bit stream holds its code
 *         and word 2 the high bits, position 32 i + j at bit 4 floor((j mod 16)/2) + 2 floor(j/16) +
 *         (j mod 2) (so (word 2 >> k) & 0x11111111 lists the same positions, nibble by nibble, as the
 *         k-th 2-bit plane of words 0 and 1).  The stream of channel c is stream slot 8 (c mod 16) + floor(c / 16) of
 *         the tile (slot p holds channel 16 (p mod 8) + floor(p / 8)).  Channel-major tiles let the
 *         decode kernels feed the codes to the matrix cores directly, 8 channels per load.
 *   meta  fp16  [B][Hkv][Ncap][2]: (min, step) of the token's value vector.
 */
#ifndef QJL_H
#define QJL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QJL_OK = 0,
    QJL_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent shapes, bad enum   */
    QJL_ERR_UNSUPPORTED = -2,  /* valid request outside the supported shapes listed above      */
    QJL_ERR_MISALIGNED = -3,   /* a pointer or stride breaks the 16-byte alignment rule       */
    QJL_ERR_WORKSPACE = -4,    /* decode workspace missing or smaller than required            */
    QJL_ERR_HIP = -5           /* the HIP runtime reported an error at launch                  */
} qjl_status;

typedef enum { QJL_BF16 = 0, QJL_F32 = 1 } qjl_dtype;

typedef enum {
    QJL_V_CODES = 0,  /* values as token-wise codes + (min, step) meta                         */
    QJL_V_F32 = 1     /* values kept unquantized, fp32 [B][Hkv][Ncap][d]                       */
} qjl_vmode;

/* The inner-product estimate the decode scores with (the key sketch is the same for both). */
typedef enum {
    QJL_EST_ONE_SIDED = 0,  /* query unquantized: sqrt(pi/2)/m |k| <S q, sign(S k)>, unbiased     */
    QJL_EST_TWO_SIDED = 1   /* query reduced to its signs as well: |q| |k| / m <sign(S q), sign(S k)>
                               per part, a biased estimate (expectation |q||k|(1 - 2 theta/pi))  */
} qjl_estimator;

/*
 * Which decode kernels score the keys and aggregate the values (both compute the same attention; see
 * qjl_decode_attention for their operand formats).
 */
typedef enum {
    QJL_PATH_AUTO = 0,    /* the matrix cores where the shape allows it, else the vector units          */
    QJL_PATH_MATRIX = 1,  /* matrix cores: value codes of 2, 3 or 4 bits, m + m_out <= 512 with m in
                             {128, 256, 512} and m_out in {0, m}; QJL_ERR_UNSUPPORTED otherwise          */
    QJL_PATH_VECTOR = 2   /* vector units (byte tables of the projected query): 2-bit value codes or
                             fp32 values, any supported sketch; QJL_ERR_UNSUPPORTED for 3- and 4-bit codes */
} qjl_decode_path;

/*
 * qjl_quantize_keys - sketch T new keys per (sequence, KV head) into the cache at positions
 * [t0, t0 + T).
 *
 * Defined by "QJL: 1-Bit Quantized JL Transform ..." ("Approach"): Gaussian JL transform, keep the
 * sign bits plus the key norm; outlier channels through a separate quantizer copy; the norm is
 * 16-bit (page "Your Brain Already Runs on 1-Bit Keys", "But Wait. Don't the Small Dims
 * Overpower?").  Per key k of KV head h with outlier set O_h:
 *     bits  = sign(S_in k_in) then sign(S_out k_out), packed as described above;
 *     norms = fp16(|k_in|), fp16(|k_out|).
 *
 *   K           keys in the model layout, element (b, t, h, c) at K[b*sK_b + t*sK_t + h*sK_h + c]
 *               (element strides; the d channels are contiguous); dtype kdt (bf16 or fp32).
 *   S_in        [m][d] row-major, dtype kdt.  S_out [m_out][d] row-major, dtype kdt (may be NULL
 *               when m_out == 0).  The caller draws S (i.i.d. N(0,1)) and keeps it for decode.
 *   outlier_idx int32 [Hkv][n_out]: distinct channels in [0, d) per KV head (NULL if n_out == 0).
 *   bits, norms the cache arrays (layout above) with capacity Ncap tokens; t0 + T <= Ncap.
 * Projections accumulate in fp32 (bf16 keys on the matrix cores); a sign bit can differ from the
 * exact sign only where |S k| is within fp32 accumulation error of zero.  T == 0 or B == 0 is a
 * no-op.
 */
int qjl_quantize_keys(const void* K, int kdt, int B, int64_t T, int Hkv, int d,
                      int64_t sK_b, int64_t sK_t, int64_t sK_h,
                      const void* S_in, int m, const void* S_out, int m_out,
                      const int32_t* outlier_idx, int n_out,
                      uint32_t* bits, uint16_t* norms, int64_t Ncap, int64_t t0,
                      hipStream_t stream);

/*
 * qjl_quantize_values - token-wise min/max quantization of T new values per (sequence, KV head)
 * into the cache at positions [t0, t0 + T).
 *
 * Defined by "2 numbers out of 128 destroy the entire KV cache" ("The Obvious Fix: Use Fewer Bits":
 * find the range, divide it into equally spaced values, round to the nearest) and the QJL summary
 * ("Limitations": values use token-wise quantization).  Per value vector v (d channels), in IEEE
 * fp32 with L = 2^nbits - 1:
 *     mn = min v; mx = max v; step = fp16_rne((mx - mn) / L); mn16 = fp16_rne(mn);
 *     code_c = clamp(rint((v_c - mn16) / step), 0, L)   (rint ties to even; all 0 if step == 0);
 *     dequantized value = mn16 + step * code.
 *   V      values in the model layout with element strides (sV_b, sV_t, sV_h), dtype vdt.
 *   nbits  2, 3 or 4.
 *   codes  the code tiles (layout above) of a cache with capacity Ncap; meta fp16 [B][Hkv][Ncap][2]
 *          = (mn16, step).  Only the code fields and meta of positions [t0, t0 + T) are written;
 *          every other position keeps its contents (a tile the append covers in part is merged
 *          with atomic and/or on its words, so appends to disjoint positions of one tile must not
 *          run concurrently on different streams).
 */
int qjl_quantize_values(const void* V, int vdt, int B, int64_t T, int Hkv, int d,
                        int64_t sV_b, int64_t sV_t, int64_t sV_h, int nbits,
                        uint32_t* codes, uint16_t* meta, int64_t Ncap, int64_t t0,
                        hipStream_t stream);

/*
 * qjl_decode_workspace_size - bytes of device workspace qjl_decode_attention needs for these
 * sizes and this nsplit (nsplit <= 0: the library's own choice, the same one the decode call makes).
 */
size_t qjl_decode_workspace_size(int B, int Hq, int Hkv, int d, int64_t N, int m, int m_out,
                                 int nsplit);

/*
 * qjl_decode_attention - one decode step: each query attends over the first N cached tokens of
 * its KV head.
 *
 * Defined by the QJL summary ("Approach": the query is JL-projected without quantization, and the
 * asymmetric estimator is unbiased for the inner product) and by softmax attention over the
 * estimated scores with a weighted sum of the dequantized values (page "Your Brain Already Runs on
 * 1-Bit Keys", "Keys Select. Values Deliver.").  Per (b, hq) with h = hq / (Hq/Hkv):
 *     Sq_in = S_in q_in, Sq_out = S_out q_out                         (fp32 sums of exact products)
 *     s_t   = score(q, k_t) from the sketch bits and fp16 norms      (formula at the top)
 *     out   = sum_t softmax(sm_scale * s)_t * v_t                    (fp32 accumulation)
 * where v_t = mn16 + step * code (QJL_V_CODES) or the fp32 value itself (QJL_V_F32).
 * Operand formats (`path`):
 *   matrix cores   each projected query value, times sm_scale log2(e) sqrt(pi/2)/m and divided by its
 *                  sign plane's coefficient, is carried as the sum of four fp6 e2m3 pieces with a power
 *                  of two per 32 values (piece p at 2^(s - 4p), where 2^s takes the largest magnitude
 *                  of the 32 into (3.75, 7.5]; round to nearest), so its error is at most 2^(s - 16),
 *                  below 2^-17.9 of that largest magnitude; multiplied exactly with the sign bits as
 *                  fp4 operands and summed in fp32, a score is within 5.9e-4 of its magnitude scale
 *                  sqrt(pi/2) (|k_in| |Sq_in|_1/m + |k_out| |Sq_out|_1/m_out) plus fp32 rounding; each
 *                  softmax weight times its token's step is carried as three fp8 e4m3 pieces (round
 *                  to nearest, residual below 2^-12 of the value) against the codes, so the value
 *                  term is within 2^-12 of the largest value range;
 *   vector units   Sq in fp32, summed through byte tables in fp32; weights times step in fp16 against
 *                  the codes (2^-11 relative).
 *   Q           [B][Hq][d] contiguous, dtype qdt; S_in / S_out / outlier_idx as for quantize (S in
 *               dtype qdt).
 *   bits, norms the key cache (capacity Ncap >= N).
 *   vmode       QJL_V_CODES: codes + meta (nbits 2, or 3 or 4 with m + m_out <= 512), V_f32 ignored;
 *               QJL_V_F32: V_f32 [B][Hkv][Ncap][d] fp32, codes/meta ignored.
 *   sm_scale    softmax scale; <= 0 selects 1/sqrt(d).
 *   path        a qjl_decode_path.
 *   estimator   a qjl_estimator.  QJL_EST_TWO_SIDED is the variant the QJL summary contrasts with the
 *               one-sided estimator ("Surprising findings": quantizing both sides gives a biased
 *               estimate of the cosine): s_t = |q_in| n_in / m <sign(Sq_in), s_in> + |q_out| n_out /
 *               m_out <sign(Sq_out), s_out>, with sign(0) = +1 on the query side as on the key side.
 *               Rotate-then-sign keys ("Your Brain Already Runs on 1-Bit Keys", "The 1-Bit
 *               Breakthrough": sign after a rotation, key = norm x signs) are the one-sided estimator
 *               with m = d, m_out = 0 and S_in = sqrt(2d/pi) R for an orthogonal R: the score is then
 *               <R q, |k| sign(R k) / sqrt(d)>.
 *   out         fp32 [B][Hq][d].  N == 0 writes zeros.
 *   scores_dbg  optional fp32 [B][Hq][N] receiving the raw estimator scores s_t (NULL to skip).
 *   nsplit      number of context chunks per (b, KV head) merged by log-sum-exp (<= 0: auto).
 *   workspace   device scratch of at least qjl_decode_workspace_size(...) bytes (same nsplit);
 *               owned by the caller, contents undefined on return, must not be shared by calls
 *               that overlap in time.
 */
int qjl_decode_attention(const void* Q, int qdt, int B, int Hq, int Hkv, int d, int64_t N,
                         const void* S_in, int m, const void* S_out, int m_out,
                         const int32_t* outlier_idx, int n_out,
                         const uint32_t* bits, const uint16_t* norms, int64_t Ncap,
                         int vmode, const uint32_t* codes, const uint16_t* meta, const float* V_f32,
                         int nbits, float sm_scale, int estimator, int path, float* out, float* scores_dbg, int nsplit,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qjl_decode_step - one step of autoregressive decoding: append the new token of every sequence to
 * the cache at position N - 1, then decode attention over the first N positions.
 *
 * The operations are the ones above, in this order: qjl_quantize_keys and qjl_quantize_values with
 * T = 1 and t0 = N - 1, then qjl_decode_attention over N tokens (the new token is quantized on the
 * fly before the step's query attends to it, as the QJL summary describes for generated tokens,
 * "Approach"; the cache then holds the same bits, norms, codes and meta as after the separate calls).
 * On the matrix-core path (dt = QJL_BF16, 2-, 3- or 4-bit values, (m, m_out) in {(128, 0), (128, 128),
 * (256, 0), (256, 256), (512, 0)}) the decode kernel itself appends the token and projects the queries
 * when a KV head serves at most 8 query heads (one launch, plus the chunk merge when the context is
 * split), and one launch does the appends and projections before the decode kernel when it serves more;
 * otherwise the three operations are enqueued one after the other.
 *   Q           [B][Hq][d] contiguous, dtype dt.
 *   K_new       new keys, element (b, h, c) at K_new[b*sK_b + h*sK_h + c] (the model layout of one
 *               token: [B][1][Hkv][d] with its strides), dtype dt; V_new likewise with (sV_b, sV_h).
 *   S_in, S_out, outlier_idx, n_out, m, m_out  as for qjl_quantize_keys (S in dtype dt).
 *   bits, norms, codes, meta  the cache (layout at the top) of capacity Ncap >= N; nbits 2, 3 or 4 (as
 *               for qjl_decode_attention).
 *   N           context length after the append (N >= 1).
 *   sm_scale, estimator, path, out, scores_dbg, nsplit, workspace  as for qjl_decode_attention (same
 *               workspace size; QJL_PATH_VECTOR runs the three operations as separate launches).
 * Every argument is checked before anything is enqueued.
 */
int qjl_decode_step(const void* Q, const void* K_new, const void* V_new, int dt, int B, int Hq, int Hkv, int d,
                    int64_t N, int64_t sK_b, int64_t sK_h, int64_t sV_b, int64_t sV_h,
                    const void* S_in, int m, const void* S_out, int m_out,
                    const int32_t* outlier_idx, int n_out,
                    uint32_t* bits, uint16_t* norms, uint32_t* codes, uint16_t* meta, int64_t Ncap, int nbits,
                    float sm_scale, int estimator, int path, float* out, float* scores_dbg, int nsplit,
                    void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qjl_decode_step_no_alloc - qjl_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, operations, results and errors as qjl_decode_step, except that there is no
 * workspace argument: the workspace is a fixed device array inside the library of
 * QJL_NO_ALLOC_SCRATCH_BYTES bytes, one per GPU, resolved on the first call on a device and held until
 * the process ends.  A call whose workspace need (qjl_decode_workspace_size with the same sizes and
 * nsplit) exceeds QJL_NO_ALLOC_SCRATCH_BYTES returns QJL_ERR_WORKSPACE before anything is enqueued.
 * The call allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *   - The array belongs to the device that is current on the calling thread, which must be the
 *     device of `stream`.
 *   - Every call on one GPU uses the same array: calls that overlap in time on one GPU (different
 *     streams, or threads) race on it and give undefined results; calls ordered on one stream are
 *     safe.  The array keeps the last call's contents; no part of it needs to start at zero (every
 *     byte a call reads was written earlier in the same call).
 * For the Llama-3.1-70B decode shape (B = 16, Hq = 64, m = m_out = 256, library split choice) the
 * workspace is about 3.2 MB.
 */
#define QJL_NO_ALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int qjl_decode_step_no_alloc(const void* Q, const void* K_new, const void* V_new, int dt, int B, int Hq, int Hkv, int d,
                             int64_t N, int64_t sK_b, int64_t sK_h, int64_t sV_b, int64_t sV_h,
                             const void* S_in, int m, const void* S_out, int m_out,
                             const int32_t* outlier_idx, int n_out,
                             uint32_t* bits, uint16_t* norms, uint32_t* codes, uint16_t* meta, int64_t Ncap, int nbits,
                             float sm_scale, int estimator, int path, float* out, float* scores_dbg, int nsplit,
                             hipStream_t stream);

/*
 * qjl_select_outliers - the outlier channels of every KV head, from prefill keys.
 *
 * The pages describe outlier channels as the few coordinates whose values are 10-100x those of the
 * rest ("2 numbers out of 128 destroy the entire KV cache", "The Real Problem: Outlier Channels";
 * "Why Compressing the KV Cache Is Hard", "The Third Problem: Magnitude Outliers", which asks for
 * detecting them); the QJL summary ("Approach") routes them through a separate quantizer copy.
 * Here: for KV head h, the n_out channels with the largest mean |k_c| over all B*T keys of the
 * head; equal means are ordered by the lower channel; written to outlier_idx[h][0..n_out) in
 * ascending channel order, ready for qjl_quantize_keys / qjl_decode_attention.
 *   K           keys in the model layout (as for qjl_quantize_keys), dtype kdt; keys must be finite.
 *   n_out       0..16 (0 writes nothing).  B*T == 0 selects channels 0..n_out-1.
 *   outlier_idx int32 [Hkv][n_out].
 *   workspace   device scratch of at least qjl_select_outliers_workspace_size(B, T, Hkv, d) bytes.
 * The magnitudes are summed in fp64 in a fixed order, so the result is deterministic; bf16 keys are
 * summed exactly unless a channel's sum spans more than 53 bits.
 */
size_t qjl_select_outliers_workspace_size(int B, int64_t T, int Hkv, int d);
int qjl_select_outliers(const void* K, int kdt, int B, int64_t T, int Hkv, int d,
                        int64_t sK_b, int64_t sK_t, int64_t sK_h, int n_out, int32_t* outlier_idx,
                        void* workspace, size_t ws_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* qjl_status_string(int status);

/* Detail of the last error reported on the calling thread ("" if none). */
const char* qjl_last_error(void);

/*
 * Kernel timing for measurement harnesses.  While enabled, every launch of the named kernel
 * ("decode", "quantize_keys", "quantize_values", "query_project", "combine", "append_project": the
 * append + query-projection launch of qjl_decode_step where it is a launch of its own, "select_outliers";
 * where the decode kernel projects the queries itself, "decode" includes that work) is bracketed by HIP
 * events recorded on the launch stream.  qjl_timer_read synchronizes on the recorded events and
 * returns the number of launches timed and their total duration in milliseconds, then clears the
 * record.  Disabled by default; enabling it does not change results.
 */
int qjl_timer_enable(int on);
int qjl_timer_read(const char* kernel, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* QJL_H */

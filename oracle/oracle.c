/*
 * oracle.c -- plain, slow, obviously correct CPU reference for FSDP2's
 * mixed-dtype gradient pack for reduce-scatter and its all-gather staging.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no source with the HIP
 * path: conversions, index math and layout are written here from the pages'
 * statement of the method, one element at a time, with no blocking, fusion
 * or reordering.
 *
 * Sources (web pages on FSDP2 per-parameter mixed precision):
 *  - "PyTorch adds per-parameter mixed precision to FSDP2" (ainewsletter.today),
 *    paragraphs 1-2: grads of mixed compute dtypes are chunked, padded and cast
 *    straight into one buffer of the reduction dtype (the _chunk_cat.out
 *    extension); one bucket per effective reduction dtype; the all-gather
 *    copy-in groups staging copies by (source, target) dtype and keeps one
 *    all-gather per fully_shard unit.
 *  - "The unit you wrapped" (kernels.rudrite.com), the shard-slicing
 *    paragraphs: a rank's shard is a contiguous row-major slice; right-hand
 *    padding makes every rank's shard the same size.
 *  - "Mixed-Precision Training" (NVIDIA NeMo AutoModel docs), table "Storage
 *    Dtype Compared to Compute Dtype": param_dtype is the compute dtype,
 *    reduce_dtype the dtype of the gradient reduce-scatter; bf16 keeps 7
 *    explicit mantissa bits.
 *
 * Parity status of each function (what pins it, from outside this file):
 *  - oracle_f32_to_bf16_bits: every non-NaN binary32 input is compared with
 *    torch's CPU float32->bfloat16 conversion (round to nearest even).  The
 *    NaN rule (keep sign and top payload bits, set the quiet bit) is a
 *    reading the pages do not fix: parity unpinned for NaN payloads beyond
 *    "the result is a NaN of the same sign".
 *  - oracle_bf16_to_f32_bits: exact widening; pinned by torch's conversion.
 *  - oracle_pack: the Linear(4,4), W=2 printed shard and printed grad shard;
 *    the Linear(3,3), W=4 padding count; closed-form layouts; torch's
 *    homogeneous _chunk_cat on pre-cast inputs.
 *  - oracle_unpack, oracle_copy_out: round-trip identities with oracle_pack /
 *    oracle_copy_in.
 *  - oracle_copy_in: the round trip copy-out(all-gather(copy-in)) equals the
 *    cast of the full parameter.  The byte offsets of the segments (16-byte
 *    aligned, in unit order, zero gap bytes) are a reading the pages leave
 *    open: parity unpinned for the layout beyond that round trip and the
 *    closed-form offsets.
 *  - oracle_rs_copy_out: torch's CPU division of the reduced row by a tensor
 *    of the divide factor, then its cast to the storage dtype, on every
 *    non-NaN element (the two operations FSDP2 applies to a reduce-scatter
 *    output); with no divide, the unpacked pack cast to the storage dtype;
 *    the divide of W summed identical rows by a power-of-two W gives the row
 *    back exactly.  The NaN rule of the divide (not divided, quiet bit set) is
 *    a reading: parity unpinned for NaN payloads there.
 *  - oracle_pack_flat, oracle_rs_copy_out_flat, oracle_copy_in_flat,
 *    oracle_copy_out_flat (the FSDP1 flat-parameter layout): the printed
 *    36/18/9 shard sizes and the Linear(3,3) padding count; torch's
 *    concatenate-pad-split of the cast gradients; the per-parameter pieces
 *    put back together give the rank's flat shard; copy-out of the gathered
 *    copy-ins gives the cast parameters back.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* dtype codes: the same numbers the library header uses, restated here */
#define ORACLE_BF16 1
#define ORACLE_FP32 2

static int64_t elem_size(int32_t dtype) { return dtype == ORACLE_BF16 ? 2 : 4; }

/*
 * bfloat16 is the upper half of an IEEE-754 binary32 (same sign and 8-bit
 * exponent, 7 explicit mantissa bits), so widening appends 16 zero bits.
 * Exact for every input, NaN and infinities included.
 */
uint32_t oracle_bf16_to_f32_bits(uint16_t h) { return ((uint32_t)h) << 16; }

/*
 * binary32 -> bfloat16 with round-to-nearest, ties-to-even on the 16
 * discarded mantissa bits.  A carry out of the kept mantissa moves into the
 * exponent, which is exactly what rounding up to the next binade (or to
 * infinity past the largest finite value) requires.  Subnormals are rounded
 * like any other value (no flush to zero).  NaN inputs keep their sign and
 * top payload bits and get the quiet bit set, so they stay NaN.
 */
uint16_t oracle_f32_to_bf16_bits(uint32_t u)
{
    uint32_t exponent = (u >> 23) & 0xFFu;
    uint32_t mantissa = u & 0x7FFFFFu;
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (exponent == 0xFFu && mantissa != 0u)
        return (uint16_t)(kept | 0x0040u);
    if (dropped > 0x8000u)
        kept += 1u;                      /* above the halfway point: round up */
    else if (dropped == 0x8000u && (kept & 1u))
        kept += 1u;                      /* exactly halfway: round to even */
    return (uint16_t)kept;
}

/* Read element i of a bf16 or fp32 array and return it as the bit pattern of
 * the target dtype. */
static uint32_t load_as(const void *base, int32_t src_dtype, int64_t i, int32_t dst_dtype)
{
    if (src_dtype == ORACLE_BF16) {
        uint16_t h = ((const uint16_t *)base)[i];
        return dst_dtype == ORACLE_BF16 ? (uint32_t)h : oracle_bf16_to_f32_bits(h);
    }
    uint32_t f = ((const uint32_t *)base)[i];
    return dst_dtype == ORACLE_FP32 ? f : (uint32_t)oracle_f32_to_bf16_bits(f);
}

static void store_as(void *base, int32_t dtype, int64_t i, uint32_t bits)
{
    if (dtype == ORACLE_BF16)
        ((uint16_t *)base)[i] = (uint16_t)bits;
    else
        ((uint32_t *)base)[i] = bits;
}

/* An element's bit pattern cast from one dtype to another. */
static uint32_t cast_bits(uint32_t bits, int32_t from, int32_t to)
{
    if (from == to) return bits;
    if (from == ORACLE_BF16) return oracle_bf16_to_f32_bits((uint16_t)bits);
    return (uint32_t)oracle_f32_to_bf16_bits(bits);
}

/* An element of `dtype` divided by d in that dtype: the quotient of the
 * element's binary32 value by d, correctly rounded to binary32 (the host
 * compiler's IEEE single-precision division), then rounded once more to
 * bfloat16 when that is the dtype.  A NaN is not divided; it keeps its sign
 * and payload and gets the quiet bit. */
static uint32_t divide_in(uint32_t bits, int32_t dtype, float d)
{
    uint32_t f = cast_bits(bits, dtype, ORACLE_FP32);
    if (((f >> 23) & 0xFFu) == 0xFFu && (f & 0x7FFFFFu) != 0u) {
        f |= 0x00400000u;
    } else {
        float x;
        memcpy(&x, &f, sizeof x);
        x = x / d;
        memcpy(&f, &x, sizeof f);
    }
    return cast_bits(f, ORACLE_FP32, dtype);
}

/* Number of source elements that land in rank r's chunk of a tensor with
 * numel elements and padded chunk size P (the rest of the chunk is padding). */
static int64_t valid_in_chunk(int64_t numel, int64_t P, int64_t r)
{
    int64_t v = numel - r * P;
    if (v < 0) v = 0;
    if (v > P) v = P;
    return v;
}

/*
 * Reduce-scatter input pack for one bucket (all tensors share the bucket's
 * reduction dtype dst_dtype).  Tensor t has numel[t] elements in grad_dtype[t],
 * padded chunk size P[t] and column offset O[t] in each of the W rows of S
 * columns.  Element j of rank r's chunk of tensor t is the tensor's flat
 * element r*P[t]+j when that exists, cast to the reduction dtype, and +0
 * otherwise:
 *     out[r*S + O[t] + j] = cast(g_t[r*P[t] + j])   if r*P[t] + j < numel[t]
 *                         = +0                       otherwise
 * Returns 0, or -1 if a column range leaves [0, S).
 */
int oracle_pack(int32_t W, int32_t n, const void *const *grads, const int32_t *grad_dtype,
                const int64_t *numel, const int64_t *P, const int64_t *O, int64_t S,
                int32_t dst_dtype, void *out)
{
    for (int32_t t = 0; t < n; ++t)
        if (O[t] < 0 || P[t] < 0 || O[t] + P[t] > S) return -1;
    for (int64_t r = 0; r < W; ++r) {
        for (int32_t t = 0; t < n; ++t) {
            for (int64_t j = 0; j < P[t]; ++j) {
                int64_t s = r * P[t] + j;
                uint32_t bits = 0u;
                if (s < numel[t]) bits = load_as(grads[t], grad_dtype[t], s, dst_dtype);
                store_as(out, dst_dtype, r * S + O[t] + j, bits);
            }
        }
    }
    return 0;
}

/*
 * Inverse layout of oracle_pack: write back every real (non-padding) element
 * of each rank chunk into a flat per-tensor array of the packed dtype.
 *     g_t[r*P[t] + j] = packed[r*S + O[t] + j]   for j < valid_r(t)
 */
int oracle_unpack(int32_t W, int32_t n, const void *packed, int32_t dtype, int64_t S,
                  const int64_t *numel, const int64_t *P, const int64_t *O, void *const *dst)
{
    for (int32_t t = 0; t < n; ++t) {
        for (int64_t r = 0; r < W; ++r) {
            int64_t v = valid_in_chunk(numel[t], P[t], r);
            for (int64_t j = 0; j < v; ++j)
                store_as(dst[t], dtype, r * P[t] + j,
                         load_as(packed, dtype, r * S + O[t] + j, dtype));
        }
    }
    return 0;
}

/*
 * All-gather copy-in for one rank: row `rank` of the [W, B]-byte all-gather
 * buffer receives, for each parameter t in unit order, its padded local shard
 * (P[t] elements in storage_dtype[t]) cast to the compute dtype param_dtype[t],
 * starting at byte A[t] of the row.  Bytes of the row not covered by a
 * segment are zero.
 */
int oracle_copy_in(int32_t rank, int32_t n, const void *const *shards, const int32_t *storage_dtype,
                   const int32_t *param_dtype, const int64_t *P, const int64_t *A, int64_t B,
                   void *ag)
{
    unsigned char *row = (unsigned char *)ag + (int64_t)rank * B;
    for (int32_t t = 0; t < n; ++t)
        if (A[t] < 0 || A[t] + P[t] * elem_size(param_dtype[t]) > B) return -1;
    memset(row, 0, (size_t)B);
    for (int32_t t = 0; t < n; ++t) {
        void *seg = row + A[t];
        for (int64_t j = 0; j < P[t]; ++j)
            store_as(seg, param_dtype[t], j, load_as(shards[t], storage_dtype[t], j, param_dtype[t]));
    }
    return 0;
}

/*
 * All-gather copy-out: rebuild each full parameter (numel[t] elements in
 * param_dtype[t]) from the gathered [W, B]-byte buffer, dropping padding.
 *     x_t[r*P[t] + j] = segment t of row r, element j    for j < valid_r(t)
 */
int oracle_copy_out(int32_t W, int32_t n, const void *ag, int64_t B, const int64_t *A,
                    const int64_t *P, const int64_t *numel, const int32_t *param_dtype,
                    void *const *params)
{
    for (int32_t t = 0; t < n; ++t) {
        for (int64_t r = 0; r < W; ++r) {
            const unsigned char *seg = (const unsigned char *)ag + r * B + A[t];
            int64_t v = valid_in_chunk(numel[t], P[t], r);
            for (int64_t j = 0; j < v; ++j)
                store_as(params[t], param_dtype[t], r * P[t] + j,
                         load_as(seg, param_dtype[t], j, param_dtype[t]));
        }
    }
    return 0;
}

/*
 * Reduce-scatter output write-back for one rank: the step after the
 * reduce-scatter on the gradient path, where each rank keeps the gradient
 * slice of the parameters it owns ("The unit you wrapped", the paragraphs on
 * the collectives FSDP issues), in the resident parameter's dtype
 * ("Mixed-Precision Training": reduce_dtype only sets how gradients are
 * summed; the gradient buffer follows the resident parameter dtype).
 *
 * `row` holds the rank's S reduced elements of one bucket in the reduction
 * dtype.  When divide_factor is not 1 each element is first divided by it in
 * the reduction dtype (divide_in).  Member t then receives the real
 * (non-padding) elements of its rank chunk, cast to its storage dtype:
 *     grad_t[j] = cast(div(row[O[t] + j]))     for j < valid_rank(t)
 * Returns 0, or -1 if a member's columns leave [0, S).
 */
int oracle_rs_copy_out(int32_t rank, int32_t n, const void *row, int32_t reduce_dtype, int64_t S,
                       float divide_factor, const int64_t *numel, const int64_t *P, const int64_t *O,
                       const int32_t *storage_dtype, void *const *grads)
{
    for (int32_t t = 0; t < n; ++t)
        if (O[t] < 0 || P[t] < 0 || O[t] + P[t] > S) return -1;
    for (int32_t t = 0; t < n; ++t) {
        int64_t v = valid_in_chunk(numel[t], P[t], rank);
        for (int64_t j = 0; j < v; ++j) {
            uint32_t x = load_as(row, reduce_dtype, O[t] + j, reduce_dtype);
            if (divide_factor != 1.0f) x = divide_in(x, reduce_dtype, divide_factor);
            store_as(grads[t], storage_dtype[t], j, cast_bits(x, reduce_dtype, storage_dtype[t]));
        }
    }
    return 0;
}

/*
 * FSDP1 flat-parameter layout ("The unit you wrapped", the auto_wrap_policy
 * paragraphs and the padding paragraph): a unit's parameters, flattened and
 * concatenated in unit order, form one 1-D flat parameter of N elements;
 * it is padded on the right to W*c elements, c = ceil(N / W), and rank r
 * holds flat positions [r*c, (r+1)*c).  Parameter t sits at flat offset F[t]
 * (the exclusive prefix sum of numel); its piece on rank r is the part of
 * [F[t], F[t] + numel[t]) inside the rank's positions.
 */

/* Parameter t's piece on rank r, as flat positions [*lo, *hi) (empty when
 * *lo >= *hi). */
static void flat_piece(int64_t F, int64_t numel, int64_t c, int64_t r, int64_t *lo, int64_t *hi)
{
    int64_t a = F, b = F + numel, s0 = r * c, s1 = (r + 1) * c;
    *lo = a > s0 ? a : s0;
    *hi = b < s1 ? b : s1;
}

/* Reduce-scatter input: out (W*c elements of dst_dtype) = the concatenated
 * gradients cast to the reduction dtype, then +0 up to W*c. */
int oracle_pack_flat(int32_t W, int32_t n, const void *const *grads, const int32_t *grad_dtype,
                     const int64_t *numel, int64_t c, int32_t dst_dtype, void *out)
{
    int64_t F = 0;
    for (int32_t t = 0; t < n; ++t) {
        for (int64_t j = 0; j < numel[t]; ++j)
            store_as(out, dst_dtype, F + j, load_as(grads[t], grad_dtype[t], j, dst_dtype));
        F += numel[t];
    }
    if (F > (int64_t)W * c) return -1;
    for (int64_t k = F; k < (int64_t)W * c; ++k) store_as(out, dst_dtype, k, 0u);
    return 0;
}

/* Write-back for rank r from its reduced row (c elements of reduce_dtype):
 * each parameter's piece, divided as in oracle_rs_copy_out, cast to its
 * storage dtype:  grads[t][f - lo_t] = cast(div(row[f - r*c])), f in the piece. */
int oracle_rs_copy_out_flat(int32_t rank, int32_t n, const void *row, int32_t reduce_dtype, int64_t c,
                            float divide_factor, const int64_t *numel, const int32_t *storage_dtype,
                            void *const *grads)
{
    int64_t F = 0;
    for (int32_t t = 0; t < n; ++t) {
        int64_t lo, hi;
        flat_piece(F, numel[t], c, rank, &lo, &hi);
        for (int64_t f = lo; f < hi; ++f) {
            uint32_t x = load_as(row, reduce_dtype, f - (int64_t)rank * c, reduce_dtype);
            if (divide_factor != 1.0f) x = divide_in(x, reduce_dtype, divide_factor);
            store_as(grads[t], storage_dtype[t], f - lo, cast_bits(x, reduce_dtype, storage_dtype[t]));
        }
        F += numel[t];
    }
    return 0;
}

/* All-gather copy-in for rank r: `row` (c elements of param_dtype) receives
 * each parameter's piece (shards[t]: the piece's elements in the storage
 * dtype) cast to param_dtype at its flat position minus r*c; positions past
 * N are +0. */
int oracle_copy_in_flat(int32_t rank, int32_t n, const void *const *shards, const int32_t *storage_dtype,
                        int32_t param_dtype, const int64_t *numel, int64_t c, void *row)
{
    for (int64_t k = 0; k < c; ++k) store_as(row, param_dtype, k, 0u);
    int64_t F = 0;
    for (int32_t t = 0; t < n; ++t) {
        int64_t lo, hi;
        flat_piece(F, numel[t], c, rank, &lo, &hi);
        for (int64_t f = lo; f < hi; ++f)
            store_as(row, param_dtype, f - (int64_t)rank * c,
                     load_as(shards[t], storage_dtype[t], f - lo, param_dtype));
        F += numel[t];
    }
    return 0;
}

/* All-gather copy-out: params[t][j] = flat[F[t] + j], flat = the gathered
 * W*c elements of param_dtype. */
int oracle_copy_out_flat(int32_t n, const void *flat, int32_t param_dtype, const int64_t *numel, void *const *params)
{
    int64_t F = 0;
    for (int32_t t = 0; t < n; ++t) {
        for (int64_t j = 0; j < numel[t]; ++j)
            store_as(params[t], param_dtype, j, load_as(flat, param_dtype, F + j, param_dtype));
        F += numel[t];
    }
    return 0;
}

/* Element-wise conversion of a whole array (used by the exhaustive
 * conversion pins and the bf16 parity cases). */
void oracle_convert(const void *src, int32_t src_dtype, void *dst, int32_t dst_dtype, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        store_as(dst, dst_dtype, i, load_as(src, src_dtype, i, dst_dtype));
}

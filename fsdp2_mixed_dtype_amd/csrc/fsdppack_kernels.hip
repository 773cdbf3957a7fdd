// fsdppack_kernels.hip -- the grouped multi-tensor kernels of libfsdppack
// for gfx950 (MI355X).
//
// One launch moves a whole operation: the reduce-scatter pack of a bucket
// (every (rank, tensor) chunk, cast to the reduction dtype and zero-padded:
// "PyTorch adds per-parameter mixed precision to FSDP2", paragraph 2), the
// write-back of a rank's reduced row into its sharded gradients ("The unit
// you wrapped", the paragraphs on the collectives FSDP issues), the
// all-gather copy-in of one rank (every shard cast to its compute dtype,
// paragraph 1) or the all-gather copy-out (every gathered segment back into
// its full parameter, padding dropped); each in the per-parameter layout or
// the FSDP1 flat layout.
//
// The work is pure data movement with a handful of integer operations per
// element (plus one division per element in a dividing write-back), so the
// design aims at HBM bandwidth, not at the matrix cores:
//  * each workgroup (one wave64) owns one 2 KiB window, finds the ranges it
//    overlaps from its index and the plan's small tables, and walks them; a
//    pack window inside a single member's chunk with no padding (nearly all
//    of them in large layouts) skips the walk and copies directly, a copy-in
//    window is always one range of one parameter's segment (copied directly
//    when whole), and a copy-out window over many small rank chunks gathers
//    its elements in one pass instead of one round trip of loads and stores
//    per chunk;
//  * every whole 16-byte destination vector is written by one 16-byte vector
//    store (element stores only at a range's unaligned head and tail),
//    64-lane wavefronts covering 1 KiB per store instruction;
//  * source vectors come from 8- or 16-byte loads that need only dword
//    alignment; a bf16 source sitting 2 bytes past a dword boundary loads
//    one extra dword and shifts adjacent dwords by 16 bits, so no load ever
//    touches a dword that holds no byte of the source;
//  * bf16 -> fp32 widening and fp32 -> bf16 round-to-nearest-even happen in
//    registers with integer operations (bit exact, independent of the
//    floating-point mode registers);
//  * padding is produced by stores of zero vectors, never by reads.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "fsdppack_internal.h"

// Device scratch of the allocation-free pack (fsdppack_pack_reduce_scatter_
// input_noalloc): the plan's pack tables are copied here, when it does not
// already hold them, instead of living in memory the library allocates.
// Each GPU holds its own copy until the process ends; host code reaches it
// only through the address scratch_address() looks up per device, never
// through this name.
static __device__ __align__(256) unsigned char scratch[fsdppack::kScratchBytes];

namespace fsdppack {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One wavefront per workgroup, two destination vectors per lane: a window
// of kBlock * kUnroll * 16 = 2 KiB is one pass (loads issued, then stores),
// and a launch has tens of thousands of short workgroups.  On MI355X this
// shape kept the most bytes in flight once each wave's table reads are paid
// (about a microsecond of dependent scalar loads and index arithmetic before
// its first data load): one vector per lane, in one- to four-wave
// workgroups, leaves too few bytes per wave behind those reads (25-35 %
// slower even at full occupancy), and more vectors per lane, wider
// workgroups or persistent workgroups measured no better.
constexpr int kBlock = 64;    // threads per workgroup (one wave64)
constexpr int kUnroll = 2;    // destination vectors per thread per pass
static_assert(kBlock * kUnroll * 16 == kWindowBytes, "one window is one pass of the workgroup");
// The pack's workgroup shape.  A plain bf16 -> fp32 cast of the 50.3M-element
// layout's bytes streams faster on MI355X as 128-thread workgroups of one
// vector per lane (44.9-45.2 us) than as one wave of two (46.7-47.3 us), but
// the pack in that shape took 59.8 us against 48.1 us: every wave still pays
// its launch-argument and stretch-record reads before its first data load,
// behind half the bytes.
constexpr int kPackBlock = 64;
constexpr int kPackUnroll = 2;
static_assert(kPackBlock * kPackUnroll * 16 == kWindowBytes, "one window is one pass of the workgroup");

template <int DT> struct ElemT;
template <> struct ElemT<kBF16> { using T = uint16_t; };
template <> struct ElemT<kFP32> { using T = uint32_t; };

// binary32 bits -> bfloat16 bits.  Adding 0x7FFF plus the lowest kept bit
// and dropping the low half rounds to nearest with ties to even (a carry
// runs into the exponent, reaching infinity past the largest finite value).
// NaNs are selected separately: quiet bit set, sign and top payload kept.
__device__ __forceinline__ uint32_t f32_to_bf16(uint32_t u)
{
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const bool is_nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
    return is_nan ? ((u >> 16) | 0x0040u) : rounded;
}

template <int S, int D>
__device__ __forceinline__ uint32_t convert1(uint32_t bits)
{
    if constexpr (S == kBF16 && D == kFP32) return bits << 16;
    else if constexpr (S == kFP32 && D == kBF16) return f32_to_bf16(bits);
    else return bits;
}

// Division by the write-back's divide factor in the source (reduction)
// dtype: a correctly rounded binary32 division (the compiler's IEEE divide
// sequence; fp32 denormals are kept), rounded once more to bfloat16 when that
// is the dtype.  A NaN is not divided: it keeps sign and payload and gets the
// quiet bit.
__device__ __forceinline__ uint32_t div_f32(uint32_t u, float d)
{
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return u | 0x00400000u;
    return __float_as_uint(__uint_as_float(u) / d);
}

template <int S>
__device__ __forceinline__ uint32_t divide_in(uint32_t bits, float d)
{
    if constexpr (S == kBF16) return f32_to_bf16(div_f32(bits << 16, d));
    else return div_f32(bits, d);
}

// One element of S cast to D, divided first when DIV.
template <int S, int D, bool DIV>
__device__ __forceinline__ uint32_t convert1_div(uint32_t bits, float d)
{
    if constexpr (DIV) bits = divide_in<S>(bits, d);
    return convert1<S, D>(bits);
}

template <int S, int D>
struct Path {
    using ST = typename ElemT<S>::T;
    using DT = typename ElemT<D>::T;
    static constexpr int V = 16 / (int)sizeof(DT);             // elements per 16 B store
    static constexpr int NSRC = V * (int)sizeof(ST) / 4;        // source dwords per vector
};

// ---------------------------------------------------------------- loads
//
// Caller tensors arrive through the pointer table as plain addresses; they
// are global memory, so every access is made through address-space-1
// pointers (global_load / global_store rather than flat instructions).
// (C-style casts: C++ casts may not change the address space.)  Multi-dword
// loads need only dword alignment; the vector types below say so.

#define FSDPPACK_GLOBAL __attribute__((address_space(1)))
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));

template <typename T>
__device__ __forceinline__ const FSDPPACK_GLOBAL T *gin(const char *p) { return (const FSDPPACK_GLOBAL T *)p; }
template <typename T>
__device__ __forceinline__ FSDPPACK_GLOBAL T *gout(char *p) { return (FSDPPACK_GLOBAL T *)p; }

// Global loads of 16, 8 and 4 bytes from dword-aligned addresses,
// non-temporal when NT (a source read exactly once).  One function per width,
// so that each load assumes the 4-byte alignment its pointer type declares
// (a template would deduce the naturally aligned vector type).
template <bool NT>
__device__ __forceinline__ u32x4 gload4(const FSDPPACK_GLOBAL u32x4_a4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ u32x2 gload2(const FSDPPACK_GLOBAL u32x2_a4 *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ uint32_t gload1(const FSDPPACK_GLOBAL uint32_t *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// N consecutive dwords from a 4-byte aligned global address.
template <int N, bool NT>
__device__ __forceinline__ void load_dwords(const char *p, uint32_t *w)
{
    const FSDPPACK_GLOBAL uint32_t *g = gin<uint32_t>(p);
    int i = 0;
#pragma unroll
    for (; i + 4 <= N; i += 4) {
        const u32x4 v = gload4<NT>((const FSDPPACK_GLOBAL u32x4_a4 *)(g + i));
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
    }
    if constexpr (N % 4 >= 2) {
        const u32x2 v = gload2<NT>((const FSDPPACK_GLOBAL u32x2_a4 *)(g + (N / 4) * 4));
        w[(N / 4) * 4] = v.x; w[(N / 4) * 4 + 1] = v.y;
    }
    if constexpr (N % 2 == 1) w[N - 1] = gload1<NT>(g + N - 1);
}

// Source vector of NSRC dwords starting 2 bytes past a dword boundary (a
// bf16 source whose element offset is odd): load NSRC + 1 dwords from the
// boundary below and shift every adjacent pair down by 16 bits.  The first
// and last dword each still hold a byte of the vector, so no load touches a
// dword the source does not own part of.
template <int NSRC, bool NT>
__device__ __forceinline__ void load_half_shifted(const char *p_minus_2, uint32_t (&o)[NSRC])
{
    uint32_t w[NSRC + 1];
    load_dwords<NSRC + 1, NT>(p_minus_2, w);
#pragma unroll
    for (int k = 0; k < NSRC; ++k) o[k] = (w[k] >> 16) | (w[k + 1] << 16);
}

// ---------------------------------------------------------------- convert + store

template <int S, int D>
__device__ __forceinline__ u32x4 convert_vec(const uint32_t (&w)[Path<S, D>::NSRC])
{
    u32x4 r;
    if constexpr (S == kBF16 && D == kFP32) {          // 4 bf16 -> 4 fp32
        r.x = w[0] << 16; r.y = w[0] & 0xFFFF0000u;
        r.z = w[1] << 16; r.w = w[1] & 0xFFFF0000u;
    } else if constexpr (S == kFP32 && D == kBF16) {   // 8 fp32 -> 8 bf16
        r.x = f32_to_bf16(w[0]) | (f32_to_bf16(w[1]) << 16);
        r.y = f32_to_bf16(w[2]) | (f32_to_bf16(w[3]) << 16);
        r.z = f32_to_bf16(w[4]) | (f32_to_bf16(w[5]) << 16);
        r.w = f32_to_bf16(w[6]) | (f32_to_bf16(w[7]) << 16);
    } else {                                           // same dtype: bit copy
        r.x = w[0]; r.y = w[1]; r.z = w[2]; r.w = w[3];
    }
    return r;
}

// Divide every source element of a vector's dwords (two per dword for bf16).
template <int S, int N>
__device__ __forceinline__ void divide_words(uint32_t (&w)[N], float d)
{
#pragma unroll
    for (int k = 0; k < N; ++k) {
        if constexpr (S == kBF16)
            w[k] = divide_in<kBF16>(w[k] & 0xFFFFu, d) | (divide_in<kBF16>(w[k] >> 16, d) << 16);
        else
            w[k] = divide_in<kFP32>(w[k], d);
    }
}

// Cache-policy bits of a gfx950 memory instruction.
constexpr int kNT = 2, kSC1 = 16;   // (sc0 is bit 0)
// Whole destination vectors: device scope, non-temporal.  The written
// buffer is read next by a collective or another kernel, never by this one,
// so the stores stream out past the XCD's L2 instead of waiting there, dirty,
// for the write-back at the kernel's end (on MI355X this measured ahead of
// plain non-temporal stores and of system scope).
constexpr int kStorePolicy = kSC1 | kNT;
// Buffer resource word 3 (untyped 32-bit data) for the gfx9 family.
constexpr int kRsrcWord3 = 0x00020000;

// The whole 16-byte destination vectors of one range, written through a
// buffer resource that spans exactly those vectors: the store instruction
// carries the cache policy, and the hardware drops any store that would
// fall outside the resource.
struct VecOut {
    __amdgpu_buffer_rsrc_t rsrc;
    __device__ __forceinline__ VecOut(char *base, int64_t nvec)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(nvec * 16), kRsrcWord3)) {}
    // vector q of the span
    __device__ __forceinline__ void put(int64_t q, u32x4 v) const
    {
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, static_cast<int>(q * 16), 0, kStorePolicy);
    }
    // half vector p (8 bytes) of the span
    __device__ __forceinline__ void put8(int64_t p, u32x2 v) const
    {
        __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, static_cast<int>(p * 8), 0, kStorePolicy);
    }
};

// One element: dst[i] = i < valid ? cast(src[i]) : +0.
template <int S, int D, bool DIV>
__device__ __forceinline__ void copy_one(const char *src, char *dst, int64_t i, int64_t valid, float d)
{
    using P = Path<S, D>;
    uint32_t v = 0;
    if (i < valid) v = convert1_div<S, D, DIV>(gin<typename P::ST>(src)[i], d);
    gout<typename P::DT>(dst)[i] = static_cast<typename P::DT>(v);
}

// A destination vector (vector q of `out`, element i0 of the chunk) that
// straddles the end of the valid prefix (at most one per range): element-wise
// loads of the valid part only.
template <int S, int D, bool DIV>
__device__ __forceinline__ void copy_straddle(const char *src, const VecOut &out, int64_t q, int64_t i0,
                                              int64_t valid, float d)
{
    using P = Path<S, D>;
    typename P::DT e[P::V];
#pragma unroll
    for (int k = 0; k < P::V; ++k) {
        uint32_t v = 0;
        if (i0 + k < valid) v = convert1_div<S, D, DIV>(gin<typename P::ST>(src)[i0 + k], d);
        e[k] = static_cast<typename P::DT>(v);
    }
    u32x4 r;
    __builtin_memcpy(&r, e, 16);
    out.put(q, r);
}

// Elements [lo, hi) of one range: dst[i] = i < valid ? cast(src[i]) : +0,
// where src / dst address element 0 of the range's chunk.  All threads of the
// workgroup take part; no two threads write the same byte.  NT: the whole
// source vectors are loaded non-temporally.  DIV: every element is divided
// by d (in S) before the cast.
template <int S, int D, bool NT, bool DIV, int BLK = kBlock, int UNR = kUnroll>
__device__ void copy_range(const char *__restrict__ src, char *__restrict__ dst, int64_t lo,
                           int64_t hi, int64_t valid, float d)
{
    using P = Path<S, D>;
    constexpr int64_t SB = sizeof(typename P::ST), DB = sizeof(typename P::DT);
    const int tid = threadIdx.x;

    // head: elements before the first 16-byte aligned destination address
    const uint32_t dmis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst + lo * DB) & 15u);
    int64_t head = static_cast<int64_t>(((16u - dmis) & 15u) / DB);
    if (head > hi - lo) head = hi - lo;
    if (tid < head) copy_one<S, D, DIV>(src, dst, lo + tid, valid, d);

    const int64_t v0 = lo + head;                 // first aligned vector
    const int64_t nvec = (hi - v0) / P::V;
    int64_t nfull = valid > v0 ? (valid - v0) / P::V : 0;
    if (nfull > nvec) nfull = nvec;
    const VecOut out(dst + v0 * DB, nvec);

    if (nfull > 0) {
        const char *s0 = src + v0 * SB;
        constexpr int64_t SV = P::V * SB;       // source bytes per vector
        // element alignment makes the source 4-byte aligned, or 2 bytes past
        // a dword boundary for a bf16 source at an odd element offset
        if ((reinterpret_cast<uintptr_t>(s0) & 3u) == 0) {
            for (int64_t q = tid; q < nfull; q += BLK * UNR) {
                uint32_t w[UNR][P::NSRC];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int64_t qq = q + u * BLK;
                    if (qq < nfull) load_dwords<P::NSRC, NT>(s0 + qq * SV, w[u]);
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int64_t qq = q + u * BLK;
                    if (qq < nfull) {
                        if constexpr (DIV) divide_words<S>(w[u], d);
                        out.put(qq, convert_vec<S, D>(w[u]));
                    }
                }
            }
        } else if constexpr (S == kBF16) {
            const char *a0 = s0 - 2;
            for (int64_t q = tid; q < nfull; q += BLK * UNR) {
                uint32_t w[UNR][P::NSRC];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int64_t qq = q + u * BLK;
                    if (qq < nfull) load_half_shifted<P::NSRC, NT>(a0 + qq * SV, w[u]);
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int64_t qq = q + u * BLK;
                    if (qq < nfull) {
                        if constexpr (DIV) divide_words<S>(w[u], d);
                        out.put(qq, convert_vec<S, D>(w[u]));
                    }
                }
            }
        }
    }

    // the straddling vector (if any) and the all-padding vectors
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int64_t q = nfull + tid; q < nvec; q += BLK) {
        const int64_t i0 = v0 + q * P::V;
        if (i0 >= valid) out.put(q, zero);
        else copy_straddle<S, D, DIV>(src, out, q, i0, valid, d);
    }

    // tail: elements after the last whole vector
    const int64_t t0 = v0 + nvec * P::V;
    if (tid < hi - t0) copy_one<S, D, DIV>(src, dst, t0 + tid, valid, d);
}

// Source loads: plain for the pack's general ranges (its line-aligned direct
// windows load non-temporally, above), non-temporal for the all-gather copies
// and the write-back (sources read once).  On MI355X non-temporal loads sped
// the copies up by 2-6 %, but moved the pack by -3 % to +5 % depending on the
// layout.  DIV: divide every element by d before the cast (write-back only).
// SAME: the range never casts (the copy-out moves a parameter's own dtype),
// so only the two plain copies are compiled in.
template <bool NT, bool DIV, bool SAME = false, int BLK = kBlock, int UNR = kUnroll>
__device__ __forceinline__ void run_range(const RangeRef &g, char *base, float d)
{
    char *tp = reinterpret_cast<char *>(g.ptr);
    const char *src;
    char *dst;
    if (g.table_side == kTableIsSource) { src = tp + g.src_off; dst = base + g.dst_off; }
    else { src = (g.src_ptr ? reinterpret_cast<const char *>(g.src_ptr) : base) + g.src_off; dst = tp + g.dst_off; }
    if constexpr (SAME) {
        if (g.dst_dt == kBF16) copy_range<kBF16, kBF16, NT, DIV, BLK, UNR>(src, dst, g.lo, g.hi, g.valid, d);
        else copy_range<kFP32, kFP32, NT, DIV, BLK, UNR>(src, dst, g.lo, g.hi, g.valid, d);
        return;
    }
    switch (g.src_dt * 4 + g.dst_dt) {
    case kBF16 * 4 + kFP32: copy_range<kBF16, kFP32, NT, DIV, BLK, UNR>(src, dst, g.lo, g.hi, g.valid, d); break;
    case kFP32 * 4 + kFP32: copy_range<kFP32, kFP32, NT, DIV, BLK, UNR>(src, dst, g.lo, g.hi, g.valid, d); break;
    case kFP32 * 4 + kBF16: copy_range<kFP32, kBF16, NT, DIV, BLK, UNR>(src, dst, g.lo, g.hi, g.valid, d); break;
    case kBF16 * 4 + kBF16: copy_range<kBF16, kBF16, NT, DIV, BLK, UNR>(src, dst, g.lo, g.hi, g.valid, d); break;
    default: break;   // the planner only emits the four pairs above
    }
}

// A whole window of one member's chunk (pack_direct): each lane loads its
// kUnroll source vectors, converts them and stores them; no range walk.  A
// bf16 source 2 bytes past a dword boundary loads through the shifted path.
// A source that starts on a cache line covers whole lines that no other
// window reads, so it is loaded non-temporally (on MI355X 2 % faster for the
// 445- and 32-tensor layouts); otherwise the lines at its two ends are shared
// with the neighbouring windows and plain loads let the cache serve the
// second read (non-temporal loads there cost 8 % on rows that start off a
// line).
// COPY: a source read exactly once whatever its alignment (the all-gather
// copy-in), loaded non-temporally everywhere.
// fp32 -> bf16 reads 32 source bytes per 16-byte destination vector; rather
// than two 16-byte loads per lane 32 bytes apart (each wave instruction then
// touching half of every line it spans), each lane converts four 16-byte
// source pieces into four 8-byte halves, so every load instruction reads
// 1 KiB and every store writes 512 B contiguously (on MI355X the copy-in of
// the 218M-element block 5 % faster; the pack unchanged).
template <int S, int D, bool COPY, int BLK = kBlock, int UNR = kUnroll>
__device__ __forceinline__ void copy_window_direct(const char *src, char *dst)
{
    using P = Path<S, D>;
    constexpr int64_t SV = P::V * static_cast<int64_t>(sizeof(typename P::ST));
    const VecOut out(dst, BLK * UNR);
    const int tid = threadIdx.x;
    if constexpr (S == kFP32 && D == kBF16) {
        uint32_t h[2 * UNR][4];
        if (COPY || (reinterpret_cast<uintptr_t>(src) & (kLineBytes - 1)) == 0) {
#pragma unroll
            for (int u = 0; u < 2 * UNR; ++u) load_dwords<4, true>(src + (tid + u * BLK) * 16, h[u]);
        } else {
#pragma unroll
            for (int u = 0; u < 2 * UNR; ++u) load_dwords<4, false>(src + (tid + u * BLK) * 16, h[u]);
        }
#pragma unroll
        for (int u = 0; u < 2 * UNR; ++u) {
            u32x2 r;
            r.x = f32_to_bf16(h[u][0]) | (f32_to_bf16(h[u][1]) << 16);
            r.y = f32_to_bf16(h[u][2]) | (f32_to_bf16(h[u][3]) << 16);
            out.put8(tid + u * BLK, r);
        }
        return;
    }
    uint32_t w[UNR][P::NSRC];
    if (COPY || (reinterpret_cast<uintptr_t>(src) & (kLineBytes - 1)) == 0) {
        if (S != kBF16 || (reinterpret_cast<uintptr_t>(src) & 3u) == 0) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) load_dwords<P::NSRC, true>(src + (tid + u * BLK) * SV, w[u]);
        } else {
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                load_half_shifted<P::NSRC, true>(src - 2 + (tid + u * BLK) * SV, w[u]);
        }
    } else if (S != kBF16 || (reinterpret_cast<uintptr_t>(src) & 3u) == 0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) load_dwords<P::NSRC, false>(src + (tid + u * BLK) * SV, w[u]);
    } else {
#pragma unroll
        for (int u = 0; u < UNR; ++u) load_half_shifted<P::NSRC, false>(src - 2 + (tid + u * BLK) * SV, w[u]);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) out.put(tid + u * BLK, convert_vec<S, D>(w[u]));
}

template <bool COPY, int BLK = kBlock, int UNR = kUnroll>
__device__ __forceinline__ void run_direct(const DirectWindow &d, char *base)
{
    const char *src = reinterpret_cast<const char *>(d.src);
    char *dst = base + d.dst_off;
    switch (d.src_dt * 4 + d.dst_dt) {
    case kBF16 * 4 + kFP32: copy_window_direct<kBF16, kFP32, COPY, BLK, UNR>(src, dst); break;
    case kFP32 * 4 + kFP32: copy_window_direct<kFP32, kFP32, COPY, BLK, UNR>(src, dst); break;
    case kFP32 * 4 + kBF16: copy_window_direct<kFP32, kBF16, COPY, BLK, UNR>(src, dst); break;
    case kBF16 * 4 + kBF16: copy_window_direct<kBF16, kBF16, COPY, BLK, UNR>(src, dst); break;
    default: break;
    }
}

// A copy-out window over many small rank chunks (copy_out_gathered): each
// lane fetches its elements one by one from wherever their chunks sit in the
// gathered buffer, so the whole window is one round of loads and one of
// stores.  Copy-out moves bits (same dtype on both sides); lanes take
// consecutive elements, so every store instruction writes one contiguous
// run, and a load instruction reads one contiguous run per rank chunk its
// elements fall in.
template <typename T>
__device__ __forceinline__ void copy_out_gather(const WindowArgs &a, const CopyOutTensor &t, int64_t e0, int64_t e1)
{
    constexpr int kPerLane = static_cast<int>(kWindowBytes / sizeof(T)) / kBlock;
    FSDPPACK_GLOBAL T *dst = gout<T>(reinterpret_cast<char *>(table_entry(a, t.slot)));
    // the tensor has fewer than 2^32 elements (copy_out_gathered); element
    // i0 + j*kBlock is the lane's j-th, present while j*kBlock < left
    const uint32_t i0 = static_cast<uint32_t>(e0) + threadIdx.x;
    const int32_t left = static_cast<int32_t>(e1 - e0) - static_cast<int32_t>(threadIdx.x);
    T v[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
        if (j * kBlock < left) v[j] = __builtin_nontemporal_load(gin<T>(a.base + copy_out_source(a, t, i0 + j * kBlock)));
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
        if (j * kBlock < left) dst[i0 + j * kBlock] = v[j];
}

// The reduce-scatter pack: one workgroup of kPackBlock threads per window,
// on a 2-D grid (x: the windows of a row group, y: the row group).  A window
// the stretch records (or, in a bucket without them, the column map) show to
// lie inside one member's rank chunk is copied directly; any other window
// walks its ranges.
// A launch's pointer table of up to N entries, passed by value: it lives in
// the kernel argument segment, and the waves read its entries with scalar
// loads straight from there.  N = 1: the table is a device table (a.table).
template <int N> struct PtrTab {
    uint64_t p[N];
};

template <int N>
__device__ __forceinline__ void use_inline_table(WindowArgs &a, const PtrTab<N> &t)
{
    if constexpr (N > 1) a.table = (const uint64_t *)&t.p[0];
}

// The direct test's inputs come first, as scalar arguments (st: the stretch
// records; rb: row bytes; glg: group_lg, log2 of the rows per row group), so
// that they can be preloaded into scalar registers.
template <int N>
__global__ void __launch_bounds__(kPackBlock) pack_kernel(const PackStretch *st, uint32_t rb, uint32_t shift,
                                                          uint32_t map_lg, uint32_t glg, WindowArgs a, PtrTab<N> t)
{
    use_inline_table(a, t);
    const int32_t k = static_cast<int32_t>(blockIdx.x >> glg);
    const int32_t r = static_cast<int32_t>((blockIdx.y << glg) | (blockIdx.x & ((1u << glg) - 1)));
    DirectWindow d;
    if (st != nullptr) {
        if (pack_direct_stretch_s(st, a.table, rb, shift, map_lg, r, k, d)) {
            run_direct<false, kPackBlock, kPackUnroll>(d, a.base);
            return;
        }
    } else if (pack_direct_rk(a, r, k, d)) {
        run_direct<false, kPackBlock, kPackUnroll>(d, a.base);
        return;
    }
    pack_window_rk(a, r, k,
                   [&](const RangeRef &g) { run_range<false, false, false, kPackBlock, kPackUnroll>(g, a.base, 1.0f); });
}

// The all-gather copy-in: one workgroup per window of a parameter's segment
// of the row.  The window's group-map entry, then its segment record with
// the shard's pointer, are the only reads before its data; their table
// addresses and the row's line offset come first among the arguments, so
// that they are preloaded into scalar registers.  A whole window of real
// elements is copied directly, a segment's first and last window as a range.
template <int N>
__global__ void __launch_bounds__(kBlock) copy_in_kernel(const ColumnWindow *groups, const CopyInSeg *segs,
                                                        uint32_t shift, WindowArgs a, PtrTab<N> t)
{
    use_inline_table(a, t);
    const CopyInWindow c = copy_in_span(groups, segs, a.table, static_cast<int32_t>(shift),
                                        static_cast<int32_t>(blockIdx.x));
    if (c.y1 <= c.y0) return;                       // the segment's spare window
    DirectWindow d;
    if (copy_in_direct(c, static_cast<int32_t>(shift), d)) run_direct<true>(d, a.base);
    else run_range<true, false>(copy_in_range(c), a.base, 1.0f);
}

// One workgroup per window; the window's ranges come from its index and the
// plan's (cache-resident) record tables.
template <int OP, int N>
__global__ void __launch_bounds__(kBlock) window_kernel(WindowArgs a, PtrTab<N> t)
{
    use_inline_table(a, t);
    const int32_t w = static_cast<int32_t>(blockIdx.x);
    auto body = [&](const RangeRef &g) { run_range<true, false>(g, a.base, 1.0f); };
    if constexpr (OP == kOpCopyOut) {
        const CopyOutTensor t = find_tensor(a, w);
        int64_t e0, e1;
        copy_out_span(t, w, e0, e1);
        if (!copy_out_gathered(t, e0, e1))
            copy_out_chunks(a, t, w, [&](const RangeRef &g) { run_range<true, false, true>(g, a.base, 1.0f); });
        else if (t.dt == kBF16) copy_out_gather<uint16_t>(a, t, e0, e1);
        else copy_out_gather<uint32_t>(a, t, e0, e1);
    } else if constexpr (OP == kOpCopyInFlat) {
        DirectWindow d;
        if (flat_copy_in_direct(a, w, d)) run_direct<true>(d, a.base);
        else flat_window<true>(a, w, body);
    } else if constexpr (OP == kOpWriteBackFlat) {
        if (a.divisor != 1.0f)     // uniform across the launch
            flat_window<false>(a, w, [&](const RangeRef &g) { run_range<true, true>(g, a.base, a.divisor); });
        else
            flat_window<false>(a, w, body);
    } else if (a.divisor != 1.0f)
        write_back_window(a, w, [&](const RangeRef &g) { run_range<true, true>(g, a.base, a.divisor); });
    else
        write_back_window(a, w, body);
}

// A kernel that does nothing (the floor of a launch of its grid).
__global__ void empty_kernel() {}

}  // namespace

int scratch_address(void **out)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return static_cast<int>(e);
        addr[dev] = p;
    }
    *out = addr[dev];
    return static_cast<int>(hipSuccess);
}

int launch_empty(int32_t workgroups, int32_t threads, void *stream, void *start_event, void *stop_event)
{
    hipExtLaunchKernelGGL(empty_kernel, dim3(static_cast<uint32_t>(workgroups)), dim3(static_cast<uint32_t>(threads)), 0,
                          static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                          static_cast<hipEvent_t>(stop_event), 0);
    return static_cast<int>(hipGetLastError());
}

namespace {

template <int N>
int launch_sized(const WindowArgs &args, const uint64_t *inline_ptrs, int32_t n, hipStream_t st, hipEvent_t e0,
                 hipEvent_t e1)
{
    PtrTab<N> t{};
    if (N > 1)
        for (int32_t i = 0; i < n; ++i) t.p[i] = inline_ptrs[i];
    const dim3 grid(static_cast<uint32_t>(args.n_windows)), block(kBlock);
    if (args.op == kOpPack) {
        // x: the windows of a row group, y: the row groups
        const dim3 grid2(static_cast<uint32_t>((args.gx + 1) << args.group_lg),
                         static_cast<uint32_t>(args.W >> args.group_lg));
        const uint32_t lg = args.reduce_dt == kBF16 ? 1u : 2u;
        const uint32_t rb = args.stretches ? static_cast<uint32_t>(args.S) << lg : 0u;
        hipExtLaunchKernelGGL(pack_kernel<N>, grid2, dim3(kPackBlock), 0, st, e0, e1, 0, args.stretches, rb,
                              static_cast<uint32_t>(args.shift), static_cast<uint32_t>(args.map_lg),
                              static_cast<uint32_t>(args.group_lg), args, t);
    } else if (args.op == kOpCopyIn) {
        hipExtLaunchKernelGGL(copy_in_kernel<N>, grid, block, 0, st, e0, e1, 0,
                              static_cast<const ColumnWindow *>(args.columns), static_cast<const CopyInSeg *>(args.members),
                              static_cast<uint32_t>(args.shift), args, t);
    } else if (args.op == kOpCopyOut) {
        hipExtLaunchKernelGGL(window_kernel<kOpCopyOut, N>, grid, block, 0, st, e0, e1, 0, args, t);
    } else if (args.op == kOpWriteBack) {
        hipExtLaunchKernelGGL(window_kernel<kOpWriteBack, N>, grid, block, 0, st, e0, e1, 0, args, t);
    } else if (args.op == kOpWriteBackFlat) {
        hipExtLaunchKernelGGL(window_kernel<kOpWriteBackFlat, N>, grid, block, 0, st, e0, e1, 0, args, t);
    } else {
        hipExtLaunchKernelGGL(window_kernel<kOpCopyInFlat, N>, grid, block, 0, st, e0, e1, 0, args, t);
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_windows(const WindowArgs &args, const uint64_t *inline_ptrs, int32_t n, void *stream, void *start_event,
                   void *stop_event)
{
    if (args.n_windows <= 0) return static_cast<int>(hipSuccess);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
    // hipExtLaunchKernelGGL: when events are given they are stamped by the
    // dispatch itself, so they bracket exactly this kernel's execution
    if (inline_ptrs == nullptr) return launch_sized<1>(args, nullptr, 0, st, e0, e1);
    if (n <= kInlineSmall) return launch_sized<kInlineSmall>(args, inline_ptrs, n, st, e0, e1);
    return launch_sized<kInlineLarge>(args, inline_ptrs, n, st, e0, e1);
}

}  // namespace fsdppack

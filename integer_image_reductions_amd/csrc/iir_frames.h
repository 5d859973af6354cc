// iir_frames.h -- the gfx950 frames kernel (templates) for the integer motion (blurred-luma SAD)
// and PSNR (per-plane SSE) sums of 4:2:0 video. Each iir_frames_*.hip translation unit
// instantiates the kernels of one sample type; iir_kernels.hip picks among them.
//
// What is computed (readings stated in include/iir.h):
//   V[i][j]  = (sum_k g_k x[m(i+k-2)][j] + 2^(bpc-1)) >> bpc            vertical pass
//   Bl[i][j] = (sum_l g_l V[i][m(j+l-2)] + 2^15) >> 16                  horizontal pass
//   SAD_t    = sum |Bl_t - Bl_(t-1)|,  SSE_c = sum (ref_c - dist_c)^2
// with g = (3571, 16004, 26386, 16004, 3571) and m the whole-sample mirror ("ADR-1392: CUDA
// motion, PSNR and moment kernels add one atomic per block ...", Decision 4: vertical pass once per
// output row and column, rounded by the bit depth, then five horizontal taps shifted by 16;
// "Research-0735: CUDA motion kernel ncu hotpath analysis (576x324)": a 5x5 separable Gaussian).
//
// Design (MI355X-first; the CUDA tiles on the pages are prior art only):
//   * One wavefront per workgroup owns one tile: 256 luma columns x TH rows, its rows starting
//     on a 256-column boundary, so every row a wavefront loads is whole, aligned cache lines that
//     no other wavefront touches (chroma: 128 samples per row). Lane l holds luma columns
//     4l .. 4l+3 of the tile. Each lane slides down its columns with the whole 5-row window in
//     registers, so every vertical value is computed exactly once and reused by the five
//     horizontal taps through two DPP lane shifts per row (no LDS round trip, no barrier).
//   * The two columns left and right of the tile (horizontal halo) arrive transposed: one load
//     per frame gives lane k the halo samples of tile row k-2 (lanes 0-31 the left side, lanes
//     32-63 the right side), their vertical pass runs once per frame across lanes, and two copies
//     of the result rotated one lane per row bring each row's pairs to lane 0 and lane 63 (motion
//     v2, with twice the halo values, gathers them with ds_bpermute instead).
//   * The separable filter runs on packed 16-bit pairs: v_perm_b32 builds (row r, row r+1) pairs
//     per column, v_dot2_u32_u16 applies two taps per instruction with the rounding constant as
//     the accumulator, and v_perm_b32 extracts the 16-bit result of a byte-aligned shift. 10-bit
//     input is pre-scaled by 64 so its vertical shift (10) also becomes a 16-bit byte shift.
//   * SAD on packed blurred pairs: one v_sad_u16 adds both columns' |a - b| to the lane's sum.
//   * SSE: 8-bit as sum(r^2 + d^2) - 2 sum(r d) with v_dot4_u32_u8 (exact in 32-bit modular
//     arithmetic, since the true per-lane value is far below 2^32); 10-bit as v_pk_sub_i16 then
//     v_dot2_i32_i16 of the difference with itself.
//   * A workgroup loops over the frames of its time chunk, keeping the previous blurred tile in
//     registers; the blurred state crosses launches through a small tiled plane (ring).
//   * Per frame, per workgroup: one 64-bit atomic per sum ("ADR-1392", Decision 1), into one of
//     kSumSlots partial slots; the last workgroup of each of 8 slot groups folds its group's slots
//     and the host adds the 8 group totals.
//   * Workgroup ids are remapped so each XCD (and its L2) gets a contiguous run of vertically
//     adjacent tiles, which share their halo rows.
#pragma once

#include <algorithm>
#include <type_traits>

#include "iir_internal.h"

namespace iir {
namespace {

constexpr uint32_t G0 = 3571, G1 = 16004, G2 = 26386;
static_assert(2 * G0 + 2 * G1 + G2 == 65536u, "taps must sum to 2^16 so flat planes stay flat");

// (lo, hi) 16-bit tap pairs for v_dot2_u32_u16
constexpr uint32_t T01 = G0 | (G1 << 16);
constexpr uint32_t T21 = G2 | (G1 << 16);
constexpr uint32_t T0z = G0;
constexpr uint32_t Tz0 = G0 << 16;
constexpr uint32_t T12 = G1 | (G2 << 16);
constexpr uint32_t T10 = G1 | (G0 << 16);

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t dot2u(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b), c,
                                  false);
}

__device__ __forceinline__ uint32_t dot4u(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_udot4(a, b, c, false);
}

// square of the packed signed 16-bit difference a - b, summed over both halves, added to c
__device__ __forceinline__ uint32_t sqdiff2(uint32_t a, uint32_t b, uint32_t c)
{
    const i16x2 d = __builtin_bit_cast(i16x2, a) - __builtin_bit_cast(i16x2, b);
    return (uint32_t)__builtin_amdgcn_sdot2(d, d, (int)c, false);
}

// byte permute of the 8-byte value {hi:lo}: selector bytes 0-3 pick lo, 4-7 pick hi, 12 gives 0
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// acc + |a.lo - b.lo| + |a.hi - b.hi| of the unsigned 16-bit halves, in one instruction
// (v_sad_u16)
__device__ __forceinline__ uint32_t sad16x2(uint32_t a, uint32_t b, uint32_t acc)
{
    return __builtin_amdgcn_sad_u16(a, b, acc);
}

// lane i receives lane i-1's value (wave_shr:1); lane 0 receives 0 (bound_ctrl, so no register
// has to be zeroed for the lane without a source)
__device__ __forceinline__ uint32_t from_left(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xf, 0xf, true);
}

// lane i receives lane i+1's value (wave_shl:1); lane 63 receives 0
__device__ __forceinline__ uint32_t from_right(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xf, 0xf, true);
}

// As from_left / from_right, but the lane without a source keeps `edge` (bound_ctrl off: the DPP
// leaves that lane's old value). A select around a plain shift would let the compiler run the
// shift with that lane masked off, and a DPP read from a masked-off lane returns 0 to its
// neighbour.
__device__ __forceinline__ uint32_t from_left_or(uint32_t v, uint32_t edge)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)edge, (int)v, 0x138, 0xf, 0xf, false);
}

__device__ __forceinline__ uint32_t from_right_or(uint32_t v, uint32_t edge)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)edge, (int)v, 0x130, 0xf, 0xf, false);
}

// lane i receives lane (i + 1) mod 64's value (wave_rol:1; every lane has a source, so
// bound_ctrl only spares the copy of an unused old value)
__device__ __forceinline__ uint32_t rotate_down(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x134, 0xf, 0xf, true);
}

// lane i receives lane (i + 32) mod 64's value: the halves of the wave swapped
__device__ __forceinline__ uint32_t swap_halves(uint32_t v, int lane)
{
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return lane < kWave / 2 ? h[1] : h[0];
}

// whole-sample mirror into [0, n), exact for -2 <= i <= n + 1, clamped beyond (never used there)
__device__ __forceinline__ int mirror_clamp(int i, int n)
{
    i = i < 0 ? -i : i;
    i = i >= n ? 2 * n - 2 - i : i;
    return min(max(i, 0), n - 1);
}

// XCD-aware tile order: hardware places workgroup b on XCD b % 8; give each XCD one contiguous
// run of the linear (chunk, row tile, strip) order. A bijection on [0, G) for any G. With strips
// fastest, the wavefronts resident together cover whole rows of the frame, so HBM sees long
// contiguous runs instead of a scatter of 256-byte pieces.
__device__ __forceinline__ int xcd_linear(int b, int G)
{
    const int x = b & 7, j = b >> 3;
    const int q = G >> 3, r = G & 7;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// Sum of a per-lane u32 over the wavefront as u64. DPP row shifts fold each row of 16 lanes into
// its lane 15 (4 adds, no LDS round trip); the four row sums are added in 64 bits on the scalar
// unit, so a wavefront total may exceed 2^32 while each row sum stays below it.
template <int CTRL>
__device__ __forceinline__ uint32_t row_shr_add(uint32_t v)
{
    return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ unsigned long long wave_sum(uint32_t v)
{
    v = row_shr_add<0x111>(v);  // row_shr:1
    v = row_shr_add<0x112>(v);  // row_shr:2
    v = row_shr_add<0x114>(v);  // row_shr:4
    v = row_shr_add<0x118>(v);  // row_shr:8
    const unsigned long long r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const unsigned long long r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const unsigned long long r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const unsigned long long r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    return (r0 + r1) + (r2 + r3);
}

// Wavefront sum of per-lane 64-bit values below 2^40 (the squares of 16-bit samples): the low 24
// bits and the rest are summed apart, each fitting the 32-bit lanes of wave_sum.
__device__ __forceinline__ unsigned long long wave_sum_sq(unsigned long long v)
{
    return wave_sum((uint32_t)v & 0xffffffu) + (wave_sum((uint32_t)(v >> 24)) << 24);
}

__device__ __forceinline__ unsigned long long wave_sum_sq(uint32_t v)
{
    return wave_sum(v);
}

// Wavefront totals of NS (4 or 8) per-lane u32 sums at once, for sums whose every wavefront total
// stays below 2^32 (8-bit samples). Each butterfly step takes two registers and one lane bit: the
// lanes where the bit is clear keep the first register's sum, the others the second's, each plus
// the same sum from a partner lane (lane bits 0 and 1 through quad permutations; bit 2 through a
// rotation by 4 within each row of 16, which pairs every lane with one of the other half of its
// group of 8, so each value is still counted once). Every step halves the registers. A rotation
// by 8 then completes each row, and the two permlane swaps of gfx950 add the four rows, after
// which every lane holds the total of sum (lane mod NS). 8 sums: 36 VALU instead of 64.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}

template <int CTRL>
__device__ __forceinline__ uint32_t pair_step(uint32_t a, uint32_t b, bool bit_set)
{
    return (bit_set ? b : a) + dpp_mov<CTRL>(bit_set ? a : b);
}

template <int NS>
__device__ __forceinline__ void wave_sums_u32(const uint32_t (&x)[NS], int lane,
                                              unsigned long long (&out)[NS])
{
    static_assert(NS == 4 || NS == 8, "four or eight sums");
    constexpr int kSwap1 = 0xB1, kSwap2 = 0x4E;   // quad_perm [1,0,3,2] and [2,3,0,1]
    constexpr int kRor4 = 0x124, kRor8 = 0x128;   // row_ror:4 and row_ror:8
    const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
    uint32_t r;
    if constexpr (NS == 8) {
        const uint32_t p0 = pair_step<kSwap1>(x[0], x[1], b0);
        const uint32_t p1 = pair_step<kSwap1>(x[2], x[3], b0);
        const uint32_t p2 = pair_step<kSwap1>(x[4], x[5], b0);
        const uint32_t p3 = pair_step<kSwap1>(x[6], x[7], b0);
        r = pair_step<kRor4>(pair_step<kSwap2>(p0, p1, b1), pair_step<kSwap2>(p2, p3, b1),
                             (lane & 4) != 0);
    } else {
        r = pair_step<kSwap2>(pair_step<kSwap1>(x[0], x[1], b0),
                              pair_step<kSwap1>(x[2], x[3], b0), b1);
        r += dpp_mov<kRor4>(r);
    }
    r += dpp_mov<kRor8>(r);
    const auto h = __builtin_amdgcn_permlane32_swap(r, r, false, false);  // halves of the wave
    r = h[0] + h[1];
    const auto q = __builtin_amdgcn_permlane16_swap(r, r, false, false);  // rows 0-1 and 2-3
    r = q[0] + q[1];
#pragma unroll
    for (int k = 0; k < NS; ++k)
        out[k] = (uint32_t)__builtin_amdgcn_readlane((int)r, k);
}

__device__ __forceinline__ void add_sum(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-frame wavefront sums waiting for their atomics. Lane q of v[] holds queued frame q's NS
// 64-bit sums (low and high halves); a flush issues every queued frame's atomics at once, one
// frame per lane. On gfx9 stores and atomics share the in-order
// vmcnt counter with loads, so an atomic issued right after a frame would make the next frame's
// first load wait for the atomic's round trip; batching keeps them off the frame loop.
template <int NS>
struct Pending {
    uint32_t v[2 * NS];
    int first;  // frame of queue slot 0 (wave-uniform)
    int count;  // queued frames (wave-uniform)
};

template <int NS>
__device__ __forceinline__ void flush_sums(const KernelArgs &a, Pending<NS> &P, int lane)
{
    if (lane < P.count) {
        unsigned long long *o = a.sums + (size_t)(P.first + lane) * (NS * kSumSlots) +
                                (blockIdx.x & (kSumSlots - 1));
#pragma unroll
        for (int k = 0; k < NS; ++k)
            add_sum(o + k * kSumSlots,
                    ((unsigned long long)P.v[2 * k + 1] << 32) | (unsigned long long)P.v[2 * k]);
    }
    P.first += P.count;
    P.count = 0;
}

template <int NS>
__device__ __forceinline__ void push_sums(const KernelArgs &a, Pending<NS> &P, int lane,
                                          const unsigned long long (&s)[NS])
{
    const bool mine = lane == P.count;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        P.v[2 * k] = mine ? (uint32_t)s[k] : P.v[2 * k];
        P.v[2 * k + 1] = mine ? (uint32_t)(s[k] >> 32) : P.v[2 * k + 1];
    }
    if (++P.count == kWave)
        flush_sums(a, P, lane);
}

template <int BPC>
struct Px;
template <>
struct Px<8> {
    typedef uint32_t Luma;  // 4 luma samples
    static constexpr int kBytes = 1;
};
template <>
struct Px<10> {
    typedef u32x2 Luma;  // 4 luma samples, 2 per dword
    static constexpr int kBytes = 2;
};
// 16-bit storage at any depth from 9 to 16 bits other than 10: samples are scaled to 16 bits by a
// runtime shift, and squares are summed per lane in 64 bits (two 16-bit squares overflow 32)
template <>
struct Px<16> : Px<10> {};

// Per-lane accumulator of squares: 32 bits up to 10-bit samples, 64 bits beyond.
template <int BPC>
using Sq = typename std::conditional<BPC == 16, unsigned long long, uint32_t>::type;

typedef __amdgpu_buffer_rsrc_t Rsrc;

// A buffer resource over one plane: base in SGPRs, `bytes` as its range. Loads then take the
// row offset in an SGPR (soffset) and the lane's column offset in one VGPR (voffset), so no
// per-row VALU address arithmetic and no 64-bit address registers are needed.
__device__ __forceinline__ Rsrc plane_rsrc(const uint8_t *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of a load (the buffer instructions' cache-policy operand): kKeep allocates in L2
// normally; kStream sets the non-temporal bit, so the line is among the first L2 evicts. Samples
// only this wavefront reads (distorted luma, chroma) stream; reference luma rows, which the
// vertically and horizontally neighbouring tiles also read as their halo, are kept so that the
// second reader finds them in L2.
constexpr int kKeep = 0;
constexpr int kStream = 2;

template <int POL = kKeep>
__device__ __forceinline__ uint32_t ld32(Rsrc r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, POL);
}

template <int BPC, int POL = kKeep>
__device__ __forceinline__ typename Px<BPC>::Luma ld_luma(Rsrc r, uint32_t voff, uint32_t soff)
{
    if constexpr (BPC == 8) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, POL);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, POL);
        return u32x2{v[0], v[1]};
    }
}

__device__ __forceinline__ int uni(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

// A value the compiler must treat as changed on every frame, so per-row products of it are not
// hoisted out of the frame loop into dozens of live scalar registers.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+s"(v));
    return v;
}

// Plane k of frame t (wave-uniform; scalar loads when it comes from the frame table).
__device__ __forceinline__ const uint8_t *frame_plane(const KernelArgs &a, int t, int k)
{
    if (a.table) {
        typedef __attribute__((address_space(4))) const FramePtrs cFramePtrs;
        const cFramePtrs *tb = (const cFramePtrs *)(uintptr_t)a.table;
        return tb[t].p[k];
    }
    return a.base[k] + (int64_t)t * a.fstride[k];
}

// Both 16-bit halves of v shifted left by 6. Takes the dword by value: __builtin_bit_cast must
// not be applied to a vector element expression such as a.y (clang reads element 0 there).
__device__ __forceinline__ uint32_t scale64(uint32_t v)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, v) << 6);
}

// 16-bit samples of bit depth bpc scaled to 16 bits (shift 16 - bpc): 10-bit by the constant,
// other depths by the launch's shift. The vertical pass then rounds and shifts by 16 at every
// depth: (sum g x 2^s + 2^15) >> 16 = (sum g x + 2^(bpc-1)) >> bpc with s = 16 - bpc.
template <int BPC>
__device__ __forceinline__ uint32_t to16(uint32_t v, uint32_t shift)
{
    if constexpr (BPC == 10)
        return scale64(v);
    else
        return __builtin_bit_cast(uint32_t,
                                  __builtin_bit_cast(u16x2, v) << (u16x2){(unsigned short)shift,
                                                                          (unsigned short)shift});
}

// (row a, row b) 16-bit pairs of the lane's 4 columns, the vertical filter's operands.
template <int BPC>
__device__ __forceinline__ void column_pairs(typename Px<BPC>::Luma a, typename Px<BPC>::Luma b,
                                             uint32_t p[4], uint32_t shift)
{
    if constexpr (BPC == 8) {
        p[0] = perm(b, a, 0x0c040c00u);
        p[1] = perm(b, a, 0x0c050c01u);
        p[2] = perm(b, a, 0x0c060c02u);
        p[3] = perm(b, a, 0x0c070c03u);
    } else {
        // samples scaled to 16 bits (10-bit: by 64): the vertical shift by bpc becomes >> 16
        const uint32_t ax = to16<BPC>(a.x, shift), ay = to16<BPC>(a.y, shift);
        const uint32_t bx = to16<BPC>(b.x, shift), by = to16<BPC>(b.y, shift);
        p[0] = perm(bx, ax, 0x05040100u);
        p[1] = perm(bx, ax, 0x07060302u);
        p[2] = perm(by, ay, 0x05040100u);
        p[3] = perm(by, ay, 0x07060302u);
    }
}

// |a - b| of both unsigned 16-bit halves
__device__ __forceinline__ uint32_t absdiff16x2(uint32_t a, uint32_t b)
{
    const u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(x, y) - __builtin_elementwise_min(x, y));
}

// acc + the squares of both 16-bit halves of v (each square < 2^32, the sum needs 64 bits)
__device__ __forceinline__ unsigned long long sq16x2(uint32_t v, unsigned long long acc)
{
    const uint32_t lo = v & 0xffffu, hi = v >> 16;
    return acc + (unsigned long long)(lo * lo) + (unsigned long long)(hi * hi);
}

// Squared-error accumulation of one luma group (4 samples) or one chroma dword. 8-bit keeps
// sum(r^2 + d^2) in s and sum(r d) in s2; deeper samples keep the sum of squared differences
// in s (32 bits up to 10-bit samples, 64 bits beyond) and leave s2 alone.
template <int BPC>
__device__ __forceinline__ void sse_luma(typename Px<BPC>::Luma r, typename Px<BPC>::Luma d,
                                         Sq<BPC> &s, uint32_t &s2)
{
    if constexpr (BPC == 8) {
        s = dot4u(d, d, dot4u(r, r, s));
        s2 = dot4u(r, d, s2);
    } else if constexpr (BPC == 10) {
        s = sqdiff2(r.y, d.y, sqdiff2(r.x, d.x, s));
    } else {
        s = sq16x2(absdiff16x2(r.y, d.y), sq16x2(absdiff16x2(r.x, d.x), s));
    }
}

template <int BPC>
__device__ __forceinline__ void sse_chroma(uint32_t r, uint32_t d, Sq<BPC> &s, uint32_t &s2)
{
    if constexpr (BPC == 8) {
        s = dot4u(d, d, dot4u(r, r, s));
        s2 = dot4u(r, d, s2);
    } else if constexpr (BPC == 10) {
        s = sqdiff2(r, d, s);
    } else {
        s = sq16x2(absdiff16x2(r, d), s);
    }
}

// Luma moments of one sample group: m1 += samples, m2 += squares, for ref (r) and dist (d). The
// squared error goes where sse_luma puts it: at 8 bits only the cross term s2 += r . d is added
// (the error is m2r + m2d - 2 s2), deeper samples add their difference squares to s.
template <int BPC>
__device__ __forceinline__ void moments_luma(typename Px<BPC>::Luma r, typename Px<BPC>::Luma d,
                                             uint32_t &m1r, uint32_t &m1d, Sq<BPC> &m2r,
                                             Sq<BPC> &m2d, Sq<BPC> &s, uint32_t &s2)
{
    if constexpr (BPC == 8) {
        m1r = dot4u(r, 0x01010101u, m1r);
        m1d = dot4u(d, 0x01010101u, m1d);
        m2r = dot4u(r, r, m2r);
        m2d = dot4u(d, d, m2d);
        s2 = dot4u(r, d, s2);
    } else {
        m1r = dot2u(r.y, 0x00010001u, dot2u(r.x, 0x00010001u, m1r));
        m1d = dot2u(d.y, 0x00010001u, dot2u(d.x, 0x00010001u, m1d));
        if constexpr (BPC == 10) {
            m2r = dot2u(r.y, r.y, dot2u(r.x, r.x, m2r));
            m2d = dot2u(d.y, d.y, dot2u(d.x, d.x, m2d));
        } else {
            m2r = sq16x2(r.y, sq16x2(r.x, m2r));
            m2d = sq16x2(d.y, sq16x2(d.x, m2d));
        }
        sse_luma<BPC>(r, d, s, s2);
    }
}

// r with the samples outside a per-lane validity mask cleared
template <int BPC>
__device__ __forceinline__ typename Px<BPC>::Luma masked(typename Px<BPC>::Luma r, uint32_t m0,
                                                         uint32_t m1)
{
    if constexpr (BPC == 8) {
        return r & m0;
    } else {
        return u32x2{r.x & m0, r.y & m1};
    }
}

// Everything one wavefront knows about its tile, fixed for the whole launch. Scalars are
// wave-uniform (kept in SGPRs); the rest are per lane.
struct Tile {
    int tile, chunk, strip, r0;  // scalar
    int rows_valid;              // scalar: output rows of the tile inside the frame
    int lane;
    uint32_t luma_off;           // byte offset of the lane's 4 luma samples in a row
    uint32_t m0, m1;             // 16-bit masks of the lane's blurred pairs (0xffff = valid)
    bool out_lane;               // lane owns output columns
    uint32_t coff[4];            // byte offsets of the lane's chroma dword in ref U, dist U,
                                 // ref V, dist V (column, plus one row for the upper half-wave
                                 // at 8 bits)
    int crow0;                   // scalar: first chroma row of the tile
    bool c_on;                   // lane reads chroma
    // horizontal halo, transposed: lane k of each half-wave loads bytes of reference luma row
    // r0 - 2 + (k mod 32) around the tile's left (lanes 0-31) or right (lanes 32-63) edge;
    // hsel picks the two halo columns out of a dword of them as a 16-bit pair, mirrored at a
    // frame edge. Registers: 8 bytes at hvoff. Staged: the aligned 16 bytes at hvoff go to LDS
    // and the dword hlds (LDS dword index) is read back.
    uint32_t hvoff;              // byte offset of the lane's halo load in the plane
    uint32_t hsel;               // byte permutation: (column -2, column -1) or (+256, +257)
    uint32_t hlds;               // staged: LDS dword index of the lane's halo dword
    // motion v2: ds_bpermute byte addresses of row 0's halo values: lane 0 reads lane 2 (left
    // halo), lane 63 reads lane 34 (right halo); row i adds 4 i. Other lanes' gathers are unused.
    int hl_addr, hr_addr;
    // parity of the wavefront's slot on its SIMD (hardware wave id, HW_ID bits 3:0)
    uint32_t slot;
    bool halo_fix;               // staged, generic: lane 63 when column e+1 = W mirrors e-1
    // right frame edge inside the last strip (W % 256 != 0), fast path: the lane whose first
    // column is W loads the group before it and permutes it into the mirror image
    bool edge_tile;              // scalar: the last strip, with W inside it
    bool cmask;                  // scalar, staged: the chroma needs its per-byte masks (cmk)
    bool mirror_right;           // lane whose first column is W: columns W, W+1 from W-2, W-3
    uint32_t msel;               // 8-bit: the byte permutation doing the above (identity else)
    // edges (generic path only)
    bool right_fix;              // lane holding column W-1: mirror the columns right of it
    int right_rem;               // scalar: W % 4
    uint32_t ym0, ym1;           // luma sample masks for SSE (valid columns)
    uint32_t cm;                 // chroma sample mask for SSE (valid columns)
    bool c_upper;                // 8-bit: lane reads the second chroma row of each step
    // staged: byte masks of the lane's 16-byte chroma groups (load q, dword j): the columns
    // inside the plane, on rows of the tile inside the plane
    uint32_t cmk[2][4];
};

// The loaded samples of one frame for one tile: reference luma rows r0-2 .. r0+TH+1, distorted
// luma rows r0 .. r0+TH-1, and the chroma dwords (ref U, dist U, ref V, dist V) of each step
// (8-bit steps cover two chroma rows, one per half-wave).
template <int BPC, int TH>
struct FrameData {
    typedef typename Px<BPC>::Luma Luma;
    static constexpr int kChromaSteps = BPC == 8 ? TH / 4 : TH / 2;
    static constexpr int kChromaStep = BPC == 8 ? 2 : 1;
    static_assert(TH + 4 <= kWave / 2, "the transposed halo gives each tile row one lane per side");
    Luma R[TH + 4];
    Luma D[TH];
    uint32_t cu[kChromaSteps], du[kChromaSteps], cv[kChromaSteps], dv[kChromaSteps];
    u32x2 HL;  // the lane's 8 halo bytes (see Tile::hvoff)
};

// LDS staging of one 8-bit frame's luma (one wavefront per workgroup, so the workgroup's LDS is
// the wave's), in rows of 256 bytes (one dword per lane). Loads write LDS directly, 16 bytes per
// lane, so one instruction moves 1 KB: four luma rows of the tile (16 lanes per row). Two stages
// alternate, so the luma of frames t+1 and t+2 is in flight while frame t is computed. Chroma,
// which only feeds the squared error, skips LDS: 16-byte register loads, the same lane layout for
// the reference and distorted planes (8 lanes per 128-byte chroma row, eight rows per load).
template <int TH>
struct Stage {
    static constexpr int kRefLoads = (TH + 4) / 4;    // 16-byte loads of reference luma
    static constexpr int kDistLoads = TH / 4;         // of distorted luma
    static constexpr int kChromaLoads = (TH + 15) / 16;  // per chroma plane (8 rows each)
    static constexpr int kRef = 0;
    static constexpr int kDist = TH + 4;
    static constexpr int kHalo = kDist + TH;  // four rows: 16 bytes per lane
    static constexpr int kRows = kHalo + 4;
    // staged loads of an accumulated frame, all counted by vmcnt in issue order
    static constexpr int kDmaLoads = kRefLoads + 1 + kDistLoads;
    static_assert(TH % 4 == 0, "whole 16-byte luma loads");
    static_assert(kDmaLoads < 16, "the frame wait encodes the count in vmcnt's low bits");
};

// A frame's chroma for the staged path: ref U, dist U, ref V, dist V, 16 bytes per lane per load.
template <int TH>
struct ChromaX4 {
    u32x4 p[4][Stage<TH>::kChromaLoads];
};

// Per-lane byte offsets of a tile's staged loads, fixed for the whole launch: one per reference
// luma load (rows mirrored at the frame's top and bottom edges), the distorted luma's and the
// four chroma planes' (their rows advance through the scalar offset). Rows past the bottom of a
// plane fall outside its buffer range and read as zero; they are never counted.
template <int TH>
struct StageOffsets {
    uint32_t ref[Stage<TH>::kRefLoads];
    uint32_t dist;
    uint32_t chroma[4];
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS row `row` of a stage whose first row is at LDS byte address `base`. The base is passed
// through opaque() once per frame, so each load's M0 is one scalar add instead of one of dozens
// of precomputed addresses the compiler would otherwise keep (and spill) across the loop.
__device__ __forceinline__ lds_void *lds_row(uint32_t base, int row)
{
    return (lds_void *)(uintptr_t)(base + (uint32_t)row * (kWave * 4u));
}

__device__ __forceinline__ uint32_t lds_addr(uint32_t (*lds)[kWave])
{
    return (uint32_t)(uintptr_t)(lds_void *)&lds[0][0];
}

// Issue every load of frame t for this tile into registers (the distorted planes and chroma only
// when the frame is accumulated; a chunk's prologue frame is only blurred).
template <int BPC, int TH, bool GENERIC>
__device__ __forceinline__ void load_frame(const KernelArgs &a, const Tile &T, int t,
                                           bool accumulate, FrameData<BPC, TH> &F)
{
    typedef FrameData<BPC, TH> FD;
    const int H = a.H;
    Rsrc rs[6];
    uint32_t pitch[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        rs[k] = plane_rsrc(frame_plane(a, t, k), a.span[k]);
        pitch[k] = opaque((uint32_t)a.pitch[k]);
    }
#pragma unroll
    for (int k = 0; k < TH + 4; ++k) {
        // only the two rows above and below the tile can fall outside the frame on the fast path
        const int row = (GENERIC || k < 2 || k >= TH + 2) ? mirror_clamp(T.r0 - 2 + k, H)
                                                          : T.r0 - 2 + k;
        F.R[k] = ld_luma<BPC>(rs[0], T.luma_off, (uint32_t)row * pitch[0]);
    }
    F.HL = ld_luma<10>(rs[0], T.hvoff, 0u);
    if (!accumulate)
        return;
#pragma unroll
    for (int i = 0; i < TH; ++i) {
        // rows past the frame re-read the last row; they are not counted
        const int row = GENERIC ? min(T.r0 + i, H - 1) : T.r0 + i;
        F.D[i] = ld_luma<BPC, kStream>(rs[3], T.luma_off, (uint32_t)row * pitch[3]);
    }
#pragma unroll
    for (int k = 0; k < FD::kChromaSteps; ++k) {
        // the upper half-wave's row is one further down (its coff adds a pitch); at a ragged
        // bottom every lane whose row is past the plane re-reads the last row instead
        const int row = T.crow0 + FD::kChromaStep * k;
        const int rl = GENERIC ? min(row, a.Hc - 1) : row;
        const bool back = GENERIC && T.c_upper && row + 1 >= a.Hc;
        F.cu[k] = ld32<kStream>(rs[1], T.coff[0] - (back ? pitch[1] : 0u), (uint32_t)rl * pitch[1]);
        F.du[k] = ld32<kStream>(rs[4], T.coff[1] - (back ? pitch[4] : 0u), (uint32_t)rl * pitch[4]);
        F.cv[k] = ld32<kStream>(rs[2], T.coff[2] - (back ? pitch[2] : 0u), (uint32_t)rl * pitch[2]);
        F.dv[k] = ld32<kStream>(rs[5], T.coff[3] - (back ? pitch[5] : 0u), (uint32_t)rl * pitch[5]);
    }
}

// Issue every load of 8-bit frame t for this tile into the wavefront's LDS stage: 16 bytes per
// lane per instruction, the reference luma and its halo always, the distorted luma and chroma
// when the frame is accumulated.
template <int TH>
__device__ __forceinline__ void load_frame_staged(const KernelArgs &a, const Tile &T,
                                                  const StageOffsets<TH> &O, int t,
                                                  bool accumulate, uint32_t (*stage)[kWave])
{
    typedef Stage<TH> ST;
    const uint32_t lds = opaque(lds_addr(stage));
    auto dma16 = [&](Rsrc r, int lds_row0, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_row(lds, lds_row0), 16, voff, soff, 0,
                                                 kKeep);
    };
    auto dma16_stream = [&](Rsrc r, int lds_row0, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_row(lds, lds_row0), 16, voff, soff, 0,
                                                 kStream);
    };
    const Rsrc ry = plane_rsrc(frame_plane(a, t, 0), a.span[0]);
#pragma unroll
    for (int q = 0; q < ST::kRefLoads; ++q)
        dma16(ry, ST::kRef + 4 * q, O.ref[q], 0u);
    // transposed halo: one aligned 16-byte load per lane (lane k of each half-wave: tile row k-2)
    dma16(ry, ST::kHalo, T.hvoff, 0u);
    if (!accumulate)
        return;
    const Rsrc rd = plane_rsrc(frame_plane(a, t, 3), a.span[3]);
    const uint32_t pd = opaque((uint32_t)a.pitch[3]);
#pragma unroll
    for (int q = 0; q < ST::kDistLoads; ++q)
        dma16_stream(rd, ST::kDist + 4 * q, O.dist, (uint32_t)(T.r0 + 4 * q) * pd);
}

// Issue frame t's chroma loads into registers (staged path).
template <int TH>
__device__ __forceinline__ void load_chroma_x4(const KernelArgs &a, const Tile &T,
                                               const StageOffsets<TH> &O, int t, ChromaX4<TH> &C)
{
    constexpr int pk[4] = {1, 4, 2, 5};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const Rsrc rc = plane_rsrc(frame_plane(a, t, pk[p]), a.span[pk[p]]);
        const uint32_t pc = opaque((uint32_t)a.pitch[pk[p]]);
#pragma unroll
        for (int q = 0; q < Stage<TH>::kChromaLoads; ++q) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                rc, (int)O.chroma[p], (int)((uint32_t)(T.crow0 + 8 * q) * pc), kStream);
            C.p[p][q] = u32x4{v[0], v[1], v[2], v[3]};
        }
    }
}

// The staged 8-bit frame's luma, from LDS into registers.
template <int TH>
__device__ __forceinline__ void read_stage(bool with_dist, uint32_t (*lds)[kWave], int lane,
                                           uint32_t hlds, FrameData<8, TH> &F)
{
    typedef Stage<TH> ST;
#pragma unroll
    for (int k = 0; k < TH + 4; ++k)
        F.R[k] = lds[ST::kRef + k][lane];
    F.HL = u32x2{(&lds[0][0])[hlds], 0u};
    if (!with_dist)
        return;
#pragma unroll
    for (int i = 0; i < TH; ++i)
        F.D[i] = lds[ST::kDist + i][lane];
}

// Fast path, last strip with the frame's right edge inside it: the lane whose first column is W
// loaded the group of columns W-4..W-1; it becomes (x[W-2], x[W-3], -, -) for columns W..W+3,
// the mirror image the horizontal taps of the lane before it need. Columns W+2 and W+3 feed no
// output.
template <int BPC, int TH, bool STAGED>
__device__ __forceinline__ void mirror_rows(const Tile &T, typename Px<BPC>::Luma (&R)[TH + 4])
{
#pragma unroll
    for (int k = 0; k < TH + 4; ++k) {
        if constexpr (STAGED) {
            // staged rows hold the lane's own columns W..W+3; the group W-4..W-1 comes from the
            // lane to the left (every lane runs the shift; only the edge lane's selector uses it)
            R[k] = perm(from_left(R[k]), R[k], T.msel);
        } else if constexpr (BPC == 8) {
            R[k] = perm(R[k], R[k], T.msel);
        } else {
            // (x[W-2] | x[W-3] << 16) from the second dword's low and the first dword's high half
            const uint32_t m = perm(R[k].x, R[k].y, 0x07060100u);
            R[k] = u32x2{T.mirror_right ? m : R[k].x, R[k].y};
        }
    }
}

template <int BPC, int TH, bool STAGED>
__device__ __forceinline__ void mirror_halo(const Tile &T, FrameData<BPC, TH> &F)
{
    mirror_rows<BPC, TH, STAGED>(T, F.R);
}

// Register-path source of the lane's two horizontal halo columns: the first column `col` of an
// 8-byte load of the halo row and the byte permutation `sel` that makes the 16-bit pair of them
// (8-bit: bytes, 0x0c = zero; 16-bit samples: halves), mirrored at the frame edges.
template <int BPC>
__device__ __forceinline__ void halo_source(int lane, int strip, int s, int W, int &col,
                                            uint32_t &sel)
{
    const int e = s + kStripCols;  // first column right of the tile
    if (lane < kWave / 2) {
        if (strip == 0) {  // columns -2, -1 mirror 2, 1
            col = 0;
            sel = BPC == 8 ? 0x0c010c02u : 0x03020504u;
        } else {  // columns s-2, s-1
            col = s - 4;
            sel = BPC == 8 ? 0x0c030c02u : 0x07060504u;
        }
    } else if (e < W - 1) {  // columns e, e+1
        col = BPC == 8 ? e - 4 : e;
        sel = BPC == 8 ? 0x0c050c04u : 0x03020100u;
    } else if (e == W - 1) {  // column e, then e+1 = W mirrors W-2 = e-1
        col = BPC == 8 ? e - 4 : e - 2;
        sel = BPC == 8 ? 0x0c030c04u : 0x03020504u;
    } else if (e == W) {  // columns W, W+1 mirror W-2, W-3
        col = BPC == 8 ? W - 8 : W - 4;
        sel = BPC == 8 ? 0x0c050c06u : 0x03020504u;
    } else {  // the frame ends inside the tile: unused
        col = 0;
        sel = 0u;
    }
}

// Vertical pass of the transposed halo. Lane k holds the two halo columns of tile row k - 2 (of
// its side) as a 16-bit pair; rows k-2 .. k+2 come from the lanes around it. Lane i + 2 returns
// the vertical values of output row i for the left side, lane i + 34 for the right side.
template <int BPC>
__device__ __forceinline__ uint32_t halo_vertical(u32x2 h, uint32_t hsel, uint32_t shift)
{
    constexpr uint32_t kVRound = BPC == 8 ? 128u : 32768u;
    constexpr uint32_t kVSel = BPC == 8 ? 0x06050201u : 0x07060302u;
    uint32_t x0 = perm(h.y, h.x, hsel);
    if constexpr (BPC != 8)
        x0 = to16<BPC>(x0, shift);
    const uint32_t m1 = from_left(x0), m2 = from_left(m1);    // rows k-1, k-2
    const uint32_t p1 = from_right(x0), p2 = from_right(p1);  // rows k+1, k+2
    const uint32_t va = dot2u(p2 & 0xffffu, T0z,
                              dot2u(perm(p1, x0, 0x05040100u), T21,
                                    dot2u(perm(m1, m2, 0x05040100u), T01, kVRound)));
    const uint32_t vb = dot2u(p2 >> 16, T0z,
                              dot2u(perm(p1, x0, 0x07060302u), T21,
                                    dot2u(perm(m1, m2, 0x07060302u), T01, kVRound)));
    return perm(vb, va, kVSel);
}

// Squared error of the frame's chroma tiles (8-bit: sums of squares in su/sv and cross terms in
// su2/sv2; deeper samples: difference squares in su/sv).
template <int BPC, int TH, bool GENERIC>
__device__ __forceinline__ void chroma_sse(const KernelArgs &a, const Tile &T,
                                           const FrameData<BPC, TH> &F, Sq<BPC> &su, uint32_t &su2,
                                           Sq<BPC> &sv, uint32_t &sv2)
{
    typedef FrameData<BPC, TH> FD;
#pragma unroll
    for (int k = 0; k < FD::kChromaSteps; ++k) {
        uint32_t ru = F.cu[k], rdu = F.du[k], rv = F.cv[k], rdv = F.dv[k];
        if constexpr (GENERIC) {
            const int row = T.crow0 + FD::kChromaStep * k + (T.c_upper ? 1 : 0);
            const uint32_t m = row < a.Hc ? T.cm : 0u;
            ru &= m;
            rdu &= m;
            rv &= m;
            rdv &= m;
        }
        sse_chroma<BPC>(ru, rdu, su, su2);
        sse_chroma<BPC>(rv, rdv, sv, sv2);
    }
}

// Per-lane accumulators of the luma and chroma statistics of one frame.
template <int BPC>
struct FrameStats {
    Sq<BPC> sy = 0, su = 0, sv = 0, m2r = 0, m2d = 0;
    uint32_t sy2 = 0, su2 = 0, sv2 = 0, m1r = 0, m1d = 0;
};

// Squared error of the staged path's chroma (16 bytes per lane per load, masked to the tile).
template <int TH, bool MASK>
__device__ __forceinline__ void chroma_sse_x4(const Tile &T, const ChromaX4<TH> &C,
                                              FrameStats<8> &S)
{
#pragma unroll
    for (int q = 0; q < Stage<TH>::kChromaLoads; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t m = MASK ? T.cmk[q][j] : 0xffffffffu;
            sse_chroma<8>(C.p[0][q][j] & m, C.p[1][q][j] & m, S.su, S.su2);
            sse_chroma<8>(C.p[2][q][j] & m, C.p[3][q][j] & m, S.sv, S.sv2);
        }
}

// Squared error (and moments) of output row i's luma samples.
template <int BPC, int TH, bool GENERIC, bool MOM>
__device__ __forceinline__ void luma_row_stats(const Tile &T, const FrameData<BPC, TH> &F, int i,
                                               FrameStats<BPC> &S)
{
    typename Px<BPC>::Luma r = F.R[i + 2], d = F.D[i];
    if constexpr (GENERIC) {
        r = masked<BPC>(r, T.ym0, T.ym1);
        d = masked<BPC>(d, T.ym0, T.ym1);
    }
    if constexpr (MOM)
        moments_luma<BPC>(r, d, S.m1r, S.m1d, S.m2r, S.m2d, S.sy, S.sy2);
    else
        sse_luma<BPC>(r, d, S.sy, S.sy2);
}

// One wavefront reduction per sum of the frame, queued for the frame's atomics.
template <int BPC, bool MOM>
__device__ __forceinline__ void push_frame_sums(const KernelArgs &a, const Tile &T,
                                                Pending<MOM ? kMaxSums : kSums> &P, uint32_t sad,
                                                const FrameStats<BPC> &S)
{
    // squared errors: 8-bit sy (or, with moments, m2r + m2d) holds sum r^2 + d^2 and sy2
    // sum r d; deeper samples keep the difference squares in sy (su, sv likewise)
    Sq<BPC> ey = S.sy, eu = S.su, ev = S.sv;
    if constexpr (BPC == 8) {
        ey = (MOM ? S.m2r + S.m2d : S.sy) - 2u * S.sy2;
        eu = S.su - 2u * S.su2;
        ev = S.sv - 2u * S.sv2;
    }
    const Sq<BPC> zero = 0;
    if constexpr (MOM && BPC == 8) {
        // every 8-bit total fits 32 bits: at most 20 rows x 4 samples x 255^2 per lane, x 64 lanes
        const uint32_t x[kMaxSums] = {T.out_lane ? sad : 0u,
                                      T.out_lane ? ey : 0u,
                                      T.c_on ? eu : 0u,
                                      T.c_on ? ev : 0u,
                                      T.out_lane ? S.m1r : 0u,
                                      T.out_lane ? S.m1d : 0u,
                                      T.out_lane ? S.m2r : 0u,
                                      T.out_lane ? S.m2d : 0u};
        unsigned long long sums[kMaxSums];
        wave_sums_u32<kMaxSums>(x, T.lane, sums);
        push_sums(a, P, T.lane, sums);
    } else if constexpr (MOM) {
        const unsigned long long sums[kMaxSums] = {
            wave_sum(T.out_lane ? sad : 0u),
            wave_sum_sq(T.out_lane ? ey : zero),
            wave_sum_sq(T.c_on ? eu : zero),
            wave_sum_sq(T.c_on ? ev : zero),
            wave_sum(T.out_lane ? S.m1r : 0u),
            wave_sum(T.out_lane ? S.m1d : 0u),
            wave_sum_sq(T.out_lane ? S.m2r : zero),
            wave_sum_sq(T.out_lane ? S.m2d : zero)};
        push_sums(a, P, T.lane, sums);
    } else if constexpr (BPC == 8) {
        // the four 8-bit totals fit 32 bits too (20 rows x 4 samples x 65535 per lane for the SAD)
        const uint32_t x[kSums] = {T.out_lane ? sad : 0u, T.out_lane ? ey : 0u,
                                   T.c_on ? eu : 0u, T.c_on ? ev : 0u};
        unsigned long long sums[kSums];
        wave_sums_u32<kSums>(x, T.lane, sums);
        push_sums(a, P, T.lane, sums);
    } else {
        const unsigned long long sums[kSums] = {wave_sum(T.out_lane ? sad : 0u),
                                                wave_sum_sq(T.out_lane ? ey : zero),
                                                wave_sum_sq(T.c_on ? eu : zero),
                                                wave_sum_sq(T.c_on ? ev : zero)};
        push_sums(a, P, T.lane, sums);
    }
}

// Row i's halo value for lane 0 (addr = T.hl_addr: hv of lane i + 2) or lane 63 (T.hr_addr: hv of
// lane i + 34), gathered across lanes by ds_bpermute; it only feeds the DPP edge operand below.
__device__ __forceinline__ uint32_t halo_gather(uint32_t hv, int addr, int i)
{
    return (uint32_t)__builtin_amdgcn_ds_bpermute(addr + 4 * i, (int)hv);
}

// The gather addresses for one frame. The empty asm makes them a value of this frame, so the
// compiler does not hoist the per-row sums addr + 4 i out of the frame loop (32 registers held);
// each sum then folds into the gather's immediate offset.
__device__ __forceinline__ void halo_addrs(const Tile &T, int &hl, int &hr)
{
    hl = T.hl_addr;
    hr = T.hr_addr;
    asm volatile("" : "+v"(hl), "+v"(hr));
}

// The horizontal neighbours of one row's packed vertical values. q0, q1 hold the lane's columns
// (c, c+1) and (c+2, c+3) as 16-bit pairs; ql receives (c-2, c-1) from the lane to the left or,
// for lane 0, the left halo hl; qr receives (c+4, c+5) from the lane to the right or, for lane
// 63, the right halo hr. The generic path then mirrors the columns past the right frame edge.
template <bool GENERIC, bool ROWSTAGE>
__device__ __forceinline__ void neighbours(const Tile &T, uint32_t hl, uint32_t hr, uint32_t &q0,
                                           uint32_t &q1, uint32_t &ql, uint32_t &qr)
{
    ql = from_left_or(q1, hl);
    // generic path: (V(c+2), V(c+1)), the mirror image of the lane's own columns, stands for
    // columns W, W+1 at the right frame edge when W % 4 == 0
    const uint32_t mirrored = GENERIC ? perm(q0, q1, 0x07060100u) : 0u;
    if constexpr (GENERIC) {
        if (T.right_rem == 1) {  // columns W, W+1 -> W-2, W-3
            q0 = T.right_fix ? perm(ql, q0, 0x07060100u) : q0;
            q1 = T.right_fix ? ql : q1;
        } else if (T.right_rem == 2) {
            q1 = T.right_fix ? perm(ql, q0, 0x07060100u) : q1;
        } else if (T.right_rem == 3) {
            q1 = T.right_fix ? perm(q0, q1, 0x07060100u) : q1;
        }
    }
    qr = from_right_or(q0, hr);
    if constexpr (GENERIC && ROWSTAGE)
        qr = T.halo_fix ? perm(q1, qr, 0x07060100u) : qr;  // (V(e), V(e-1))
    if constexpr (GENERIC) {
        if (T.right_rem == 0)
            qr = T.right_fix ? mirrored : qr;
        else if (T.right_rem == 3)
            qr = T.right_fix ? q0 : qr;
    }
}

// ---------------------------------------------------------------------------------------------
// Motion v2: the separable filter applied to the difference prev - cur of consecutive reference
// luma frames ("ADR-1392", Decision 4: the kernel stages prev - cur, runs the vertical pass once,
// rounded by the bit depth, then the five horizontal taps shifted by 16). Shifts of negative
// sums floor. The kernel works on the biased difference d' = d + 2^bpc, which is positive, so
// every product is an unsigned 16-bit dot product: the taps sum to 2^16, so the vertical value
// of d' is exactly V' = V + 2^16 (the bias is a multiple of the shift), in [0, 2^17). V' travels
// split into its top bit Vb = floor(V' / 2^16) and its low half Vlo = V' mod 2^16. The horizontal
// sum S' = sum g V' = S + 2^32 is 33 bits wide ("ADR-1392", the alternative of 32-bit horizontal
// sums), so it is taken as two 32-bit sums Q = sum g Vb and L = sum g Vlo + 2^15 (below 2^32):
//   F + 2^16 = floor((S' + 2^15) / 2^16) = Q + floor(L / 2^16).

// The constants of motion v2 at bit depth bpc: the difference bias 2^bpc in both 16-bit halves,
// the vertical rounding term 2^(bpc - 1) and the vertical shift bpc. 8 and 10 bits are
// compile-time; 16-bit storage takes its depth, 9 to 15, from the launch's scale shift
// (16 - depth). At 16 bits the biased difference needs 17 bits: that depth has its own kernel
// variant on halved differences (WideDiff below), which does not use these constants.
struct V2Depth {
    uint32_t bias, round, vshift;
};

template <int BPC>
__device__ __forceinline__ V2Depth v2_depth(const KernelArgs &a)
{
    if constexpr (BPC == 8) {
        return V2Depth{0x01000100u, 128u, 8u};
    } else if constexpr (BPC == 10) {
        return V2Depth{0x04000400u, 512u, 10u};
    } else {
        const uint32_t b = 16u - (uint32_t)a.shift;
        return V2Depth{(1u << b) * 0x10001u, 1u << (b - 1u), b};
    }
}

// prev - cur + 2^bpc of one row's 4 samples as two 16-bit pairs: columns (c, c+1), (c+2, c+3).
// Each half lies in [1, 2^(bpc+1) - 1], so whole-dword arithmetic never carries between halves
// (prev < 2^bpc, so OR-ing the bias in adds it).
template <int BPC>
__device__ __forceinline__ u32x2 diff_row(typename Px<BPC>::Luma p, typename Px<BPC>::Luma r,
                                          const V2Depth &D)
{
    if constexpr (BPC == 8) {
        // bytes of prev widened to 16 bits with 0x01 as the high byte: prev + 256
        return u32x2{perm(0x01010101u, p, 0x04010400u) - perm(0u, r, 0x0c010c00u),
                     perm(0x01010101u, p, 0x04030402u) - perm(0u, r, 0x0c030c02u)};
    } else {
        return u32x2{(p.x | D.bias) - r.x, (p.y | D.bias) - r.y};
    }
}

// (row a, row b) pairs of the 4 columns of two difference rows
__device__ __forceinline__ void diff_pairs(u32x2 da, u32x2 db, uint32_t p[4])
{
    p[0] = perm(db.x, da.x, 0x05040100u);
    p[1] = perm(db.x, da.x, 0x07060302u);
    p[2] = perm(db.y, da.y, 0x05040100u);
    p[3] = perm(db.y, da.y, 0x07060302u);
}

// Two columns' vertical sums of biased differences (rounding term included) -> packed top bits
// (Vb, Vb') and low halves (Vlo, Vlo'). 8-bit: V' = s >> 8 < 2^17, so Vlo is bits 8-23 of s and
// Vb its byte 3; deeper: V' = s >> bpc first (s < 2^32 up to 15 bits).
template <int BPC>
__device__ __forceinline__ void split_pack(uint32_t s0, uint32_t s1, uint32_t &h, uint32_t &l,
                                           const V2Depth &D)
{
    if constexpr (BPC == 8) {
        h = perm(s1, s0, 0x0c070c03u);
        l = perm(s1, s0, 0x06050201u);
    } else {
        const uint32_t v0 = s0 >> D.vshift, v1 = s1 >> D.vshift;
        h = perm(v1, v0, 0x0c060c02u);
        l = perm(v1, v0, 0x05040100u);
    }
}

// Vertical pass of the transposed halo's biased differences (lane k: the two halo columns of
// tile row k - 2 as a pair), split as above; lane i + 2 (left) and i + 34 (right) serve row i.
template <int BPC>
__device__ __forceinline__ void halo_vertical_v2(uint32_t dh, uint32_t &hvh, uint32_t &hvl,
                                                 const V2Depth &D)
{
    const uint32_t m1 = from_left(dh), m2 = from_left(m1);    // rows k-1, k-2
    const uint32_t p1 = from_right(dh), p2 = from_right(p1);  // rows k+1, k+2
    const uint32_t sa = dot2u(p2, T0z,
                              dot2u(perm(p1, dh, 0x05040100u), T21,
                                    dot2u(perm(m1, m2, 0x05040100u), T01, D.round)));
    const uint32_t sb = dot2u(p2 >> 16, T0z,
                              dot2u(perm(p1, dh, 0x07060302u), T21,
                                    dot2u(perm(m1, m2, 0x07060302u), T01, D.round)));
    split_pack<BPC>(sa, sb, hvh, hvl, D);
}

// 16 bits ("wide"): the biased difference d' = d + 2^16 needs 17 bits, so it travels halved:
// dh = floor(d / 2) + 2^15 (16 bits) and dl = d mod 2, d' = 2 dh + dl. With y1 = sum g dh and
// y2 = sum g dl + 2^15, the vertical value is V' = (2 y1 + y2) >> 16 = (y1 + (y2 >> 1)) >> 15 =
// V + 2^16, every sum below 2^32 (y1 + (y2 >> 1) <= 4,294,950,912); the horizontal pass is then
// the one above.
struct WideDiff {
    uint32_t h, l;  // dh and dl of two columns, as 16-bit pairs
};

// dh and dl of one dword of prev and cur samples (two 16-bit columns): floor((p - r) / 2) =
// (p >> 1) - (r >> 1) - (~p & r & 1) per half, plus 2^15, never below 0 or above 65535, so the
// whole-dword arithmetic does not borrow between halves; d mod 2 = (p ^ r) & 1.
__device__ __forceinline__ WideDiff wide_diff(uint32_t p, uint32_t r)
{
    const uint32_t half_p = ((p >> 1) & 0x7fff7fffu) | 0x80008000u;
    const uint32_t half_r = (r >> 1) & 0x7fff7fffu;
    return WideDiff{half_p - half_r - (~p & r & 0x00010001u), (p ^ r) & 0x00010001u};
}

// One dword of V' for the halved representation: the two sums of a column's chain
__device__ __forceinline__ uint32_t wide_vertical(uint32_t y1, uint32_t y2)
{
    return y1 + (y2 >> 1);
}

// halo_vertical_v2 for the halved differences (dh, dl of the halo pair, one lane per tile row)
__device__ __forceinline__ void halo_vertical_v2_wide(WideDiff d, uint32_t &hvh, uint32_t &hvl)
{
    uint32_t s[2][2];  // [dh, dl][column s-2, s-1]
    const uint32_t src[2] = {d.h, d.l};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t x = src[k];
        const uint32_t m1 = from_left(x), m2 = from_left(m1);
        const uint32_t p1 = from_right(x), p2 = from_right(p1);
        const uint32_t start = k == 0 ? 0u : 32768u;
        s[k][0] = dot2u(p2, T0z, dot2u(perm(p1, x, 0x05040100u), T21,
                                       dot2u(perm(m1, m2, 0x05040100u), T01, start)));
        s[k][1] = dot2u(p2 >> 16, T0z, dot2u(perm(p1, x, 0x07060302u), T21,
                                             dot2u(perm(m1, m2, 0x07060302u), T01, start)));
    }
    const V2Depth D{0u, 0u, 15u};
    split_pack<16>(wide_vertical(s[0][0], s[1][0]), wide_vertical(s[0][1], s[1][1]), hvh, hvl, D);
}

// F + 2^16 = Q + floor(L / 2^16) of one output in one instruction: v_mad_u32_u16 multiplies the
// high half of L (op_sel) by 1 and adds Q. |F| = |(F + 2^16) - 2^16|.
constexpr uint32_t kV2Zero = 1u << 16;
__device__ __forceinline__ uint32_t biased_f(uint32_t q, uint32_t l)
{
    uint32_t d;
    asm("v_mad_u32_u16 %0, %1, 1, %2 op_sel:[1,0,0,0]" : "=v"(d) : "v"(l), "v"(q));
    return d;
}

// acc + |x - y| in one instruction (v_sad_u32)
__device__ __forceinline__ uint32_t add_absdiff(uint32_t x, uint32_t y, uint32_t acc)
{
    uint32_t d;
    asm("v_sad_u32 %0, %1, %2, %3" : "=v"(d) : "v"(x), "v"(y), "v"(acc));
    return d;
}

// One frame of one tile from its loaded samples: blur the reference luma (vertical pass once per
// column and row, horizontal taps through DPP neighbours), SAD against the previous blurred tile
// held in registers, SSE of the luma and chroma tiles, one wavefront reduction and one atomic per
// sum. GENERIC adds the frame-edge mirror fix-ups, ragged rows and masked tails; interior tiles
// (the vast majority) run without any of it. MOM also sums the luma moments of ref and dist.
template <int BPC, int TH, bool GENERIC, bool ROWSTAGE, bool MOM>
__device__ __forceinline__ void compute_frame(const KernelArgs &a, const Tile &T, int t,
                                              bool accumulate, FrameData<BPC, TH> &F,
                                              FrameStats<BPC> &S,
                                              const uint32_t (&prev0)[TH],
                                              const uint32_t (&prev1)[TH], uint32_t (&next0)[TH],
                                              uint32_t (&next1)[TH], bool &have_prev,
                                              Pending<MOM ? kMaxSums : kSums> &P)
{
    typedef typename Px<BPC>::Luma Luma;
    typedef FrameData<BPC, TH> FD;
    constexpr uint32_t kVRound = BPC == 8 ? 128u : 32768u;
    constexpr uint32_t kVSel = BPC == 8 ? 0x06050201u : 0x07060302u;

    if constexpr (!GENERIC) {
        if (T.edge_tile)
            mirror_halo<BPC, TH, ROWSTAGE>(T, F);
    }
    const uint32_t shift = (uint32_t)a.shift;
    const uint32_t hv = halo_vertical<BPC>(F.HL, T.hsel, shift);
    // Row i's halo pairs are hv of lane i + 2 (left) and lane i + 34 (right). Two copies of hv
    // rotated one lane per row bring them to the edge lanes: lane 0 of xl holds the left pair of
    // the current row, lane 63 of xr its right pair; each then serves as the DPP edge operand.
    uint32_t xl = rotate_down(rotate_down(hv));
    uint32_t xr = rotate_down(swap_halves(xl, T.lane));

    // SSE of the chroma tiles first, which frees their registers before the blur (the staged
    // path has already summed its chroma into S)
    if constexpr (!ROWSTAGE) {
        if (accumulate)
            chroma_sse<BPC, TH, GENERIC>(a, T, F, S.su, S.su2, S.sv, S.sv2);
    }

    // blur, SAD against the previous blurred tile, and SSE of the luma rows as they go by. A lane
    // whose columns all lie right of the frame drops its sums at the reduction. The generic path
    // (which also has lanes with only some columns inside, and rows below the frame) clears every
    // blurred value it keeps outside the frame, so the previous tile's are clear too and those
    // places add nothing to the SAD; a per-row branch around the SAD instead measured 60 more
    // VGPRs and spilled at 20 rows.
    uint32_t sad = 0;
#pragma unroll
    for (int i = 0; i < TH; ++i) {
        uint32_t pa[4], pb[4], pc[4];
        const Luma zero{};
        column_pairs<BPC>(F.R[i], F.R[i + 1], pa, shift);      // rows i-2, i-1
        column_pairs<BPC>(F.R[i + 2], F.R[i + 3], pb, shift);  // rows i,   i+1
        column_pairs<BPC>(F.R[i + 4], i + 5 < TH + 4 ? F.R[i + 5] : zero, pc,
                          shift);  // rows i+2 (tap 0 on i+3)
        uint32_t v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            v[b] = dot2u(pc[b], T0z, dot2u(pb[b], T21, dot2u(pa[b], T01, kVRound)));
        uint32_t q0 = perm(v[1], v[0], kVSel);  // V of columns c, c+1
        uint32_t q1 = perm(v[3], v[2], kVSel);  // V of columns c+2, c+3
        // halo V of this row: columns s-2, s-1 in lane 0 of xl and e, e+1 in lane 63 of xr (a
        // ds_bpermute gather, as in motion v2, measured slower here: the staged frame's LDS is
        // busy with its own reads)
        const uint32_t hl = xl, hr = xr;
        xl = rotate_down(xl);
        xr = rotate_down(xr);
        uint32_t ql, qr;
        neighbours<GENERIC, ROWSTAGE>(T, hl, hr, q0, q1, ql, qr);
        const uint32_t h0 = dot2u(q1, T0z, dot2u(q0, T21, dot2u(ql, T01, 32768u)));
        const uint32_t h1 = dot2u(q1, T10, dot2u(q0, T12, dot2u(ql, Tz0, 32768u)));
        const uint32_t h2 = dot2u(qr, T0z, dot2u(q1, T21, dot2u(q0, T01, 32768u)));
        const uint32_t h3 = dot2u(qr, T10, dot2u(q1, T12, dot2u(q0, Tz0, 32768u)));
        uint32_t c0 = perm(h1, h0, 0x07060302u);  // Bl of columns c, c+1
        uint32_t c1 = perm(h3, h2, 0x07060302u);  // Bl of columns c+2, c+3
        if constexpr (GENERIC) {
            c0 = i < T.rows_valid ? c0 & T.m0 : 0u;
            c1 = i < T.rows_valid ? c1 & T.m1 : 0u;
        }
        sad = sad16x2(c1, prev1[i], sad16x2(c0, prev0[i], sad));
        if (!GENERIC || i < T.rows_valid) {
            // with moments, staged frames always hold distorted rows (staged_frame's ALL_DIST)
            if ((ROWSTAGE && MOM) || accumulate)
                luma_row_stats<BPC, TH, GENERIC, MOM>(T, F, i, S);
        }
        next0[i] = c0;
        next1[i] = c1;
    }

    if (accumulate)
        push_frame_sums<BPC, MOM>(a, T, P, have_prev ? sad : 0u, S);
    have_prev = true;
}

// One frame of one tile for motion v2: the filter of prev - cur and the sum of its absolute
// values, plus the same squared errors (and moments) as compute_frame. pin holds the previous
// frame's reference luma rows (mirrored like F.R) and pxin its halo pair; on return pout and
// pxout hold this frame's, for the next. WIDE: 16-bit samples, halved differences (above).
template <int BPC, int TH, bool GENERIC, bool ROWSTAGE, bool MOM, bool WIDE>
__device__ __forceinline__ void compute_frame_v2(const KernelArgs &a, const Tile &T,
                                                 bool accumulate, FrameData<BPC, TH> &F,
                                                 FrameStats<BPC> &S,
                                                 const typename Px<BPC>::Luma (&pin)[TH + 4],
                                                 uint32_t pxin,
                                                 typename Px<BPC>::Luma (&pout)[TH + 4],
                                                 uint32_t &pxout, bool &have_prev,
                                                 Pending<MOM ? kMaxSums : kSums> &P)
{
    if constexpr (!GENERIC) {
        if (T.edge_tile)
            mirror_halo<BPC, TH, ROWSTAGE>(T, F);
    }
    const uint32_t x0 = perm(F.HL.y, F.HL.x, T.hsel);  // this frame's halo pair
    if (accumulate) {
        if constexpr (!ROWSTAGE)
            chroma_sse<BPC, TH, GENERIC>(a, T, F, S.su, S.su2, S.sv, S.sv2);
        uint32_t sad = 0;
        if (have_prev) {
            uint32_t hvh, hvl;
            const V2Depth D = WIDE ? V2Depth{0u, 0u, 15u} : v2_depth<BPC>(a);
            if constexpr (WIDE)
                halo_vertical_v2_wide(wide_diff(pxin, x0), hvh, hvl);
            else
                halo_vertical_v2<BPC>((pxin + D.bias) - x0, hvh, hvl, D);
            int hla, hra;
            halo_addrs(T, hla, hra);
            const u32x2 zero{};
#pragma unroll
            for (int i = 0; i < TH; ++i) {
                uint32_t v[4];
                if constexpr (WIDE) {
                    // rows k of the halved differences: (dh, dl) of columns (c, c+1), (c+2, c+3)
                    auto wd = [&](int k, u32x2 &h, u32x2 &l) {
                        if (k >= TH + 4) {
                            h = zero;
                            l = zero;
                        } else {
                            const WideDiff d0 = wide_diff(pin[k].x, F.R[k].x);
                            const WideDiff d1 = wide_diff(pin[k].y, F.R[k].y);
                            h = u32x2{d0.h, d1.h};
                            l = u32x2{d0.l, d1.l};
                        }
                    };
                    u32x2 h[6], l[6];
#pragma unroll
                    for (int k = 0; k < 6; ++k)
                        wd(i + k, h[k], l[k]);
                    uint32_t ph[3][4], pl[3][4];
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        diff_pairs(h[2 * k], h[2 * k + 1], ph[k]);
                        diff_pairs(l[2 * k], l[2 * k + 1], pl[k]);
                    }
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        v[b] = wide_vertical(
                            dot2u(ph[2][b], T0z, dot2u(ph[1][b], T21, dot2u(ph[0][b], T01, 0u))),
                            dot2u(pl[2][b], T0z,
                                  dot2u(pl[1][b], T21, dot2u(pl[0][b], T01, 32768u))));
                } else {
                    uint32_t pa[4], pb[4], pc[4];
                    diff_pairs(diff_row<BPC>(pin[i], F.R[i], D),
                               diff_row<BPC>(pin[i + 1], F.R[i + 1], D), pa);  // rows i-2, i-1
                    diff_pairs(diff_row<BPC>(pin[i + 2], F.R[i + 2], D),
                               diff_row<BPC>(pin[i + 3], F.R[i + 3], D), pb);  // rows i, i+1
                    diff_pairs(diff_row<BPC>(pin[i + 4], F.R[i + 4], D),
                               i + 5 < TH + 4 ? diff_row<BPC>(pin[i + 5], F.R[i + 5], D) : zero,
                               pc);  // rows i+2 (tap 0 on i+3)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        v[b] = dot2u(pc[b], T0z, dot2u(pb[b], T21, dot2u(pa[b], T01, D.round)));
                }
                uint32_t q0h, q0l, q1h, q1l;
                split_pack<BPC>(v[0], v[1], q0h, q0l, D);  // columns c, c+1
                split_pack<BPC>(v[2], v[3], q1h, q1l, D);  // columns c+2, c+3
                const uint32_t hlh = halo_gather(hvh, hla, i);
                const uint32_t hll = halo_gather(hvl, hla, i);
                const uint32_t hrh = halo_gather(hvh, hra, i);
                const uint32_t hrl = halo_gather(hvl, hra, i);
                uint32_t qlh, qrh, qll, qrl;
                neighbours<GENERIC, ROWSTAGE>(T, hlh, hrh, q0h, q1h, qlh, qrh);
                neighbours<GENERIC, ROWSTAGE>(T, hll, hrl, q0l, q1l, qll, qrl);
                uint32_t f[4];  // F + 2^16 of columns c .. c+3
                f[0] = biased_f(dot2u(q1h, T0z, dot2u(q0h, T21, dot2u(qlh, T01, 0u))),
                                dot2u(q1l, T0z, dot2u(q0l, T21, dot2u(qll, T01, 32768u))));
                f[1] = biased_f(dot2u(q1h, T10, dot2u(q0h, T12, dot2u(qlh, Tz0, 0u))),
                                dot2u(q1l, T10, dot2u(q0l, T12, dot2u(qll, Tz0, 32768u))));
                f[2] = biased_f(dot2u(qrh, T0z, dot2u(q1h, T21, dot2u(q0h, T01, 0u))),
                                dot2u(qrl, T0z, dot2u(q1l, T21, dot2u(q0l, T01, 32768u))));
                f[3] = biased_f(dot2u(qrh, T10, dot2u(q1h, T12, dot2u(q0h, Tz0, 0u))),
                                dot2u(qrl, T10, dot2u(q1l, T12, dot2u(q0l, Tz0, 32768u))));
                if constexpr (GENERIC) {
                    // a column outside the frame counts as F = 0
                    if (i < T.rows_valid) {
                        sad = add_absdiff((T.m0 & 1u) ? f[0] : kV2Zero, kV2Zero, sad);
                        sad = add_absdiff((T.m0 >> 16) ? f[1] : kV2Zero, kV2Zero, sad);
                        sad = add_absdiff((T.m1 & 1u) ? f[2] : kV2Zero, kV2Zero, sad);
                        sad = add_absdiff((T.m1 >> 16) ? f[3] : kV2Zero, kV2Zero, sad);
                    }
                } else {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        sad = add_absdiff(f[b], kV2Zero, sad);
                }
                if (!GENERIC || i < T.rows_valid)
                    luma_row_stats<BPC, TH, GENERIC, MOM>(T, F, i, S);
            }
        } else {
#pragma unroll
            for (int i = 0; i < TH; ++i)
                if (!GENERIC || i < T.rows_valid)
                    luma_row_stats<BPC, TH, GENERIC, MOM>(T, F, i, S);
        }
        push_frame_sums<BPC, MOM>(a, T, P, sad, S);
    }
#pragma unroll
    for (int k = 0; k < TH + 4; ++k)
        pout[k] = F.R[k];
    pxout = x0;
    have_prev = true;
}

// s_setprio takes an immediate
__device__ __forceinline__ void set_prio(uint32_t p)
{
    if (p == 3u)
        __builtin_amdgcn_s_setprio(3);
    else if (p == 2u)
        __builtin_amdgcn_s_setprio(2);
    else if (p == 1u)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Staged path, frame t of a chunk's loop: wait until its luma (in the stage `lds`) and its chroma
// (in C) have landed, read the luma out and sum the chroma, then issue frame t+1's chroma into C
// and frame t+2's luma into the stage just read, so two frames of loads stay in flight while
// frame t is computed. Loads complete in issue order (vmcnt): ... luma t, chroma t, luma t+1,
// chroma t+1, luma t+2 ..., so frame t has landed once only the kDmaLoads loads of the luma
// group after its chroma may still be outstanding. Every chroma group is followed by exactly one
// luma group on every path (the chunk's last one reloads its last frame into the free stage, an
// L2 hit), so that one wait is always right and the compiler's own count for the chroma registers
// agrees with it. The wavefront raises its priority from the wait to the last load issued, so a
// wavefront whose data has landed refills the memory pipe ahead of its SIMD's computing waves.
// At equal priority a SIMD's arbiter favours its older wavefront: with two per SIMD, per-wave
// timestamps showed the younger finishing a 50-frame launch about 40% after the older, the SIMD
// then running one wavefront alone. So the two slots take turns, frame by frame, at the higher
// of two priority levels, in the load window (3 or 2) and in the compute that follows (1 or 0).
// ALL_DIST reads the distorted rows out of a frame that is not accumulated too (its stage then
// holds stale rows), so that the luma sums can run for every frame without a branch per row.
template <int TH, bool ALL_DIST, bool ONE = false>
__device__ __forceinline__ void staged_frame(const KernelArgs &a, const Tile &T,
                                             const StageOffsets<TH> &O, int t, int f_begin,
                                             int f_end, uint32_t (*lds)[kWave], ChromaX4<TH> &C,
                                             FrameData<8, TH> &F, FrameStats<8> &S)
{
    const uint32_t favoured = ((uint32_t)t + T.slot) & 1u;
    set_prio(2u + favoured);
    if constexpr (ONE)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): a one-frame launch has no second group
    else
        __builtin_amdgcn_s_waitcnt(0x0F70 | Stage<TH>::kDmaLoads);  // vmcnt(one luma group)
    read_stage<TH>(ALL_DIST || t >= f_begin, lds, T.lane, T.hlds, F);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read out before it is overwritten
    if (t >= f_begin) {
        if (T.cmask)
            chroma_sse_x4<TH, true>(T, C, S);
        else
            chroma_sse_x4<TH, false>(T, C, S);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < f_end) {
        load_chroma_x4<TH>(a, T, O, t + 1, C);
        load_frame_staged<TH>(a, T, O, min(t + 2, f_end - 1), true, lds);
    }
    set_prio(favoured);
}

// The first loads of a chunk's loop: luma and chroma of its first frame, then the luma of the
// second (of the first again for a one-frame chunk). The frame loop waits for all of its loads
// before the chunk's sums are published (vmcnt(0)), so no load into LDS outlives the wavefront.
// ONE: a launch of one frame (one chunk). Its only luma group and chroma are followed by `mid`,
// the previous state's loads, so those are in flight with the frame's instead of one memory
// round trip ahead of them, and no second luma group is loaded.
struct NoLoads {
    __device__ void operator()() const {}
};

template <int TH, bool ONE = false, typename Mid = NoLoads>
__device__ __forceinline__ void staged_start(const KernelArgs &a, const Tile &T,
                                             const StageOffsets<TH> &O, int t0, int f_begin,
                                             int f_end, uint32_t (*lds)[kWave], ChromaX4<TH> &C,
                                             Mid mid = {})
{
    load_frame_staged<TH>(a, T, O, t0, t0 >= f_begin, lds);
    if (t0 >= f_begin)
        load_chroma_x4<TH>(a, T, O, t0, C);
    if constexpr (ONE)
        mid();
    else
        load_frame_staged<TH>(a, T, O, min(t0 + 1, f_end - 1), true, lds + Stage<TH>::kRows);
}

// The previous launch's blurred tile of this wavefront (its rows in the tiled state plane).
template <int TH>
__device__ __forceinline__ void load_prev_tile(const KernelArgs &a, const Tile &T,
                                               uint32_t (&prev0)[TH], uint32_t (&prev1)[TH])
{
    const uint2 *rin = reinterpret_cast<const uint2 *>(a.ring_in);
#pragma unroll
    for (int i = 0; i < TH; ++i) {
        const uint2 v = rin[(T.tile * TH + i) * kWave + T.lane];
        prev0[i] = v.x;
        prev1[i] = v.y;
    }
}

// The frames of this workgroup's time chunk. Chunks after the first start by re-blurring the
// frame before them. STAGED keeps the next frame's loads in flight while the current one is
// computed: the loads of frame t+1 write the wave's LDS stage (no registers held), issued as soon
// as frame t has been read out of it. Frames go in pairs that swap the roles of two blurred-tile
// register sets (prev -> alt -> prev), so no frame ends by copying its blurred tile back.
template <int BPC, int TH, bool GENERIC, bool STAGED, bool MOM, bool ONE = false>
__device__ __forceinline__ void frame_loop(const KernelArgs &a, const Tile &T,
                                           const StageOffsets<TH> &O, uint32_t (&prev0)[TH],
                                           uint32_t (&prev1)[TH], bool have_prev,
                                           uint32_t (*lds)[kWave])
{
    const int f_begin = uni(T.chunk * a.chunk_len);
    const int f_end = uni(min(f_begin + a.chunk_len, a.nframes));
    const int t0 = T.chunk > 0 ? f_begin - 1 : f_begin;
    constexpr int NS = MOM ? kMaxSums : kSums;
    Pending<NS> P;
#pragma unroll
    for (int k = 0; k < 2 * NS; ++k)
        P.v[k] = 0;
    P.first = f_begin;
    P.count = 0;
    ChromaX4<TH> C;
    if constexpr (STAGED && ONE) {
        // the previous blurred tile's loads go out behind the frame's own
        const bool load_prev = T.chunk == 0 && a.has_prev != 0;
        staged_start<TH, true>(a, T, O, t0, f_begin, f_end, lds, C, [&]() {
            if (load_prev)
                load_prev_tile<TH>(a, T, prev0, prev1);
        });
        if (load_prev)
            have_prev = true;
    } else if constexpr (STAGED) {
        staged_start<TH>(a, T, O, t0, f_begin, f_end, lds, C);
    }
    // one frame: blurred tile in (i0, i1), out to (o0, o1); staged, its luma in stage `sidx`
    auto step = [&](int t, int sidx, const uint32_t(&i0)[TH], const uint32_t(&i1)[TH],
                    uint32_t(&o0)[TH], uint32_t(&o1)[TH]) {
        // a fresh frame per step: no sample register is carried from one frame to the next
        FrameData<BPC, TH> F;
        FrameStats<BPC> S;
        if constexpr (STAGED)
            staged_frame<TH, MOM, ONE>(a, T, O, t, f_begin, f_end,
                                       lds + sidx * Stage<TH>::kRows, C, F, S);
        else {
            // 10-bit: the highest priority while the frame's loads issue, the lowest after, so
            // the SIMD's two wavefronts advance alike and vertically adjacent tiles still share
            // their halo rows in L2 (16-bit measured slower with it)
            if constexpr (BPC == 10)
                set_prio(3u);
            load_frame<BPC, TH, GENERIC>(a, T, t, t >= f_begin, F);
            if constexpr (BPC == 10)
                set_prio(0u);
        }
        compute_frame<BPC, TH, GENERIC, STAGED, MOM>(a, T, t, t >= f_begin, F, S, i0, i1, o0,
                                                     o1, have_prev, P);
    };
    uint32_t alt0[TH], alt1[TH];
    for (int t = t0; t < f_end; t += 2) {
        step(t, 0, prev0, prev1, alt0, alt1);
        if (t + 1 < f_end) {
            step(t + 1, 1, alt0, alt1, prev0, prev1);
        } else {
#pragma unroll
            for (int i = 0; i < TH; ++i) {
                prev0[i] = alt0[i];
                prev1[i] = alt1[i];
            }
        }
    }
    flush_sums(a, P, T.lane);
}

// The frames of this workgroup's time chunk for motion v2. The state carried from frame to frame
// is the previous frame's reference luma rows and halo pair, in two register sets whose roles
// swap every frame; chunks after the first load the frame before them as their first state.
template <int BPC, int TH, bool GENERIC, bool STAGED, bool MOM, bool WIDE>
__device__ __forceinline__ void frame_loop_v2(const KernelArgs &a, const Tile &T,
                                              const StageOffsets<TH> &O,
                                              typename Px<BPC>::Luma (&prev)[TH + 4],
                                              uint32_t &pxprev, bool have_prev,
                                              uint32_t (*lds)[kWave])
{
    typedef typename Px<BPC>::Luma Luma;
    const int f_begin = uni(T.chunk * a.chunk_len);
    const int f_end = uni(min(f_begin + a.chunk_len, a.nframes));
    const int t0 = T.chunk > 0 ? f_begin - 1 : f_begin;
    constexpr int NS = MOM ? kMaxSums : kSums;
    Pending<NS> P;
#pragma unroll
    for (int k = 0; k < 2 * NS; ++k)
        P.v[k] = 0;
    P.first = f_begin;
    P.count = 0;
    ChromaX4<TH> C;
    if constexpr (STAGED)
        staged_start<TH>(a, T, O, t0, f_begin, f_end, lds, C);
    auto step = [&](int t, int sidx, const Luma(&pin)[TH + 4], uint32_t pxin,
                    Luma(&pout)[TH + 4], uint32_t &pxout) {
        FrameData<BPC, TH> F;
        FrameStats<BPC> S;
        if constexpr (STAGED)
            staged_frame<TH, false>(a, T, O, t, f_begin, f_end, lds + sidx * Stage<TH>::kRows, C,
                                    F, S);
        else {
            if constexpr (BPC == 10)  // as in frame_loop: the two wavefronts advance alike
                set_prio(3u);
            load_frame<BPC, TH, GENERIC>(a, T, t, t >= f_begin, F);
            if constexpr (BPC == 10)
                set_prio(0u);
        }
        compute_frame_v2<BPC, TH, GENERIC, STAGED, MOM, WIDE>(a, T, t >= f_begin, F, S, pin,
                                                              pxin, pout, pxout, have_prev, P);
    };
    Luma alt[TH + 4];
    uint32_t pxalt = 0;
    for (int t = t0; t < f_end; t += 2) {
        step(t, 0, prev, pxprev, alt, pxalt);
        if (t + 1 < f_end) {
            step(t + 1, 1, alt, pxalt, prev, pxprev);
        } else {
#pragma unroll
            for (int k = 0; k < TH + 4; ++k)
                prev[k] = alt[k];
            pxprev = pxalt;
        }
    }
    flush_sums(a, P, T.lane);
}

// Motion v2 state across launches: the last frame's reference luma, saved as a plane of
// strips * 256 samples per row (ring_out, read back through ring_in by the next launch).
template <int BPC>
__device__ __forceinline__ uint32_t saved_pitch(const KernelArgs &a)
{
    return (uint32_t)(a.strips * kStripCols * Px<BPC>::kBytes);
}

// The previous frame's rows and halo pair from the saved plane, as the frame loop would have
// left them: rows mirrored at the top and bottom, the lane's columns as its loads take them
// (staged: its own four; registers: T.luma_off), the halo pair through the register-path source.
template <int BPC, int TH, bool GENERIC, bool STAGED>
__device__ __forceinline__ void load_saved(const KernelArgs &a, const Tile &T, int s,
                                           typename Px<BPC>::Luma (&prev)[TH + 4],
                                           uint32_t &pxprev)
{
    constexpr int B = Px<BPC>::kBytes;
    const uint32_t pitch = saved_pitch<BPC>(a);
    const Rsrc rs = plane_rsrc(reinterpret_cast<const uint8_t *>(a.ring_in), pitch * (uint32_t)a.H);
    const uint32_t col = STAGED ? (uint32_t)((s + kLumaCols * T.lane) * B) : T.luma_off;
#pragma unroll
    for (int k = 0; k < TH + 4; ++k)
        prev[k] = ld_luma<BPC>(rs, col, (uint32_t)mirror_clamp(T.r0 - 2 + k, a.H) * pitch);
    int hcol;
    uint32_t hsel;
    halo_source<BPC>(T.lane, T.strip, s, a.W, hcol, hsel);
    const int hrow = mirror_clamp(T.r0 - 2 + min(T.lane & (kWave / 2 - 1), TH + 3), a.H);
    const u32x2 h = ld_luma<10>(rs, (uint32_t)(hcol * B) + (uint32_t)hrow * pitch, 0u);
    pxprev = perm(h.y, h.x, hsel);
    if constexpr (!GENERIC) {
        if (T.edge_tile)
            mirror_rows<BPC, TH, STAGED>(T, prev);
    }
}

// The tile's rows of the launch's last frame into the saved plane: exactly TH store
// instructions (rows of a ragged last tile past the frame land in the plane's padding rows,
// which nothing reads).
template <int BPC, int TH>
__device__ __forceinline__ void store_saved(const KernelArgs &a, const Tile &T, int s,
                                            const typename Px<BPC>::Luma (&prev)[TH + 4])
{
    constexpr int B = Px<BPC>::kBytes;
    const uint32_t pitch = saved_pitch<BPC>(a);
    uint8_t *base = reinterpret_cast<uint8_t *>(a.ring_out) + (size_t)(s + kLumaCols * T.lane) * B;
#pragma unroll
    for (int i = 0; i < TH; ++i) {  // non-temporal, like the blurred state's stores
        auto *row = reinterpret_cast<typename Px<BPC>::Luma *>(base + (size_t)(T.r0 + i) * pitch);
        __builtin_nontemporal_store(prev[i + 2], row);
    }
}

// Each workgroup adds its per-frame sums into slot blockIdx mod kSumSlots, so a slot takes the
// atomics of 1/64 of the workgroups: with fewer slots the atomics of the whole grid, all issued
// when the workgroups finish their last frames, queue on the same few addresses (8 slots cost
// ~20 us more per 4K launch than 64). The slots form kSumGroups groups by blockIdx mod 8; the last
// workgroup of a group to finish (found by the two-level count below) folds its group's slots of
// every sum of every frame and writes the group totals straight to the caller-visible pinned
// buffer [frame][sum][group]; the host adds the group totals. No workgroup waits for another,
// and no readback copy follows the kernel. Launches alternate between two slot buffers; each
// launch's workgroups clear the other one (the previous launch's) with plain stores as they
// start, so the fold does not zero anything. Ordering: the sum atomics are device-scope
// read-modify-writes; each workgroup waits until its own have completed (vmcnt(0)) before
// counting itself, and the last one reads them back with device-scope atomic loads after an
// acquire fence. A release fence per workgroup would write back every XCD's L2 once per
// workgroup, which costs far more than the copy it replaces.

// Clear this workgroup's share of the previous launch's slot buffer.
__device__ __forceinline__ void clear_idle_slots(const KernelArgs &a, int lane)
{
    const int64_t step = (int64_t)gridDim.x * kWave;
    for (int64_t i = (int64_t)blockIdx.x * kWave + lane; i < a.zero_n; i += step)
        a.zero[i] = 0ull;
}

// s_waitcnt immediate for vmcnt(n), 0 <= n < 64 (low four bits, then bits 15:14)
constexpr int vmcnt_imm(int n)
{
    return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}

// Count this workgroup as finished, once its sum atomics have completed: they precede the
// YOUNGER vector memory instructions the caller issued last (its state stores), which may still be
// in flight, so the stores drain while the count makes its round trip. Counting takes two levels,
// so that no counter takes more than about 32 arrivals: device-scope atomics on one address are
// performed one after another at memory, and one counter per slot group (253 arrivals each at 4K)
// made the last workgroups of a launch wait up to 18 us for their turn. A workgroup counts into
// its slot's counter (blockIdx mod kSumSlots); the last member of a slot resets it and counts the
// slot into its group's counter (slot mod kSumGroups); the last slot of a group publishes the
// group. Returns (wave-uniform) whether this workgroup publishes.
template <int YOUNGER>
__device__ __forceinline__ bool count_arrival(const KernelArgs &a, int lane)
{
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(YOUNGER));  // the sum atomics have completed
    const unsigned int n = gridDim.x;
    const unsigned int slot = blockIdx.x % kSumSlots;
    const unsigned int g = blockIdx.x % kSumGroups;
    const unsigned int slot_members = n / kSumSlots + (slot < n % kSumSlots ? 1u : 0u);
    // slots of group g with members: g, g + 8, ..., below min(n, kSumSlots)
    const unsigned int used = min(n, (unsigned int)kSumSlots);
    const unsigned int group_slots = used / kSumGroups + (g < used % kSumGroups ? 1u : 0u);
    unsigned int last = 0;
    if (lane == 0) {
        const unsigned int s = __hip_atomic_fetch_add(a.arrivals + slot, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        if (s == slot_members - 1u) {
            // every member of the slot has counted (each after its own sums completed)
            __hip_atomic_store(a.arrivals + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned int q = __hip_atomic_fetch_add(a.arrivals + kSumSlots + g, 1u,
                                                          __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
            last = q == group_slots - 1u ? 1u : 0u;
        }
    }
    return uni((int)last) != 0;
}

template <int NS>
__device__ __forceinline__ void publish_if_last(const KernelArgs &a, int lane, bool last)
{
    constexpr int kPerGroup = kSumSlots / kSumGroups;  // slots g, g + 8, ..., g + 56
    const unsigned int g = blockIdx.x % kSumGroups;
    if (!last)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // kPer totals per lane per pass, all of their slot loads issued before any is added, so a
    // pass costs one memory round trip (a 64-frame launch is one pass)
    constexpr int kPer = 4;
    const int n = a.nframes * NS;
    for (int base = 0; base < n; base += kPer * kWave) {
        unsigned long long v[kPer][kPerGroup];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = min(base + q * kWave + lane, n - 1);
#pragma unroll
            for (int j = 0; j < kPerGroup; ++j)
                v[q][j] = __hip_atomic_load(a.sums + (size_t)i * kSumSlots + g + kSumGroups * j,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = base + q * kWave + lane;
            if (i < n) {
                unsigned long long total = 0;
#pragma unroll
                for (int j = 0; j < kPerGroup; ++j)
                    total += v[q][j];
                __hip_atomic_store(a.publish + (size_t)i * kSumGroups + g, total,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
    }
    if (lane == 0)
        __hip_atomic_store(a.arrivals + kSumSlots + g, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    // the end of the kernel releases these stores to the host before its completion signal
}

// V2: 0 the blurred-frame SAD, 1 motion v2, 2 motion v2 of 16-bit samples (halved differences).
// ONE: the kernel of a one-frame launch (8-bit staged, blurred-frame SAD): the previous state's
// loads go out behind the frame's own.
template <int BPC, int TH, bool STAGED, bool GENERIC, int WPE, bool MOM, int V2, bool ONE = false>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(WPE))) void
frames_kernel(const KernelArgs a)
{
    __shared__ uint32_t stage[STAGED ? 2 * Stage<TH>::kRows : 1][kWave];  // two stages
    static_assert(TH % 4 == 0, "tile height must be a multiple of 4 (two chroma rows per step)");
    static_assert(!STAGED || BPC == 8, "LDS staging is laid out for 8-bit samples");
    constexpr int B = Px<BPC>::kBytes;
    const int lane = threadIdx.x;

    clear_idle_slots(a, lane);

    Tile T;
    const int L = uni(xcd_linear(blockIdx.x, gridDim.x));
    T.chunk = uni(L / a.tiles);
    T.tile = uni(L - T.chunk * a.tiles);
    const int rt = uni(T.tile / a.strips);
    T.strip = uni(T.tile - rt * a.strips);
    T.r0 = uni(rt * TH);                     // first output row of the tile
    const int s = uni(T.strip * kStripCols);  // first column of the tile
    T.lane = lane;
    const int W = a.W, H = a.H;
    T.rows_valid = uni(min(TH, H - T.r0));

    // lane roles; every load offset stays inside its row's pitch (a lane whose first column is
    // outside [0, W) reads column 0 and its values are never used)
    const int c = s + kLumaCols * lane;
    T.luma_off = c < W ? (uint32_t)(c * B)
                 : (!GENERIC && c == W) ? (uint32_t)((W - kLumaCols) * B)
                                        : 0u;
    T.out_lane = c < W;
    if constexpr (STAGED)
        T.slot = (uint32_t)__builtin_amdgcn_s_getreg(0xF804) & 1u;  // hwreg(HW_REG_HW_ID)
    if constexpr (V2) {
        T.hl_addr = lane == 0 ? 4 * 2 : 4 * lane;
        T.hr_addr = lane == kWave - 1 ? 4 * (kWave / 2 + 2) : 4 * lane;
    }
    T.m0 = (c < W ? 0xffffu : 0u) | (c + 1 < W ? 0xffff0000u : 0u);
    T.m1 = (c + 2 < W ? 0xffffu : 0u) | (c + 3 < W ? 0xffff0000u : 0u);
    T.edge_tile = T.strip == a.strips - 1 && W % kStripCols != 0;
    T.mirror_right = c == W;
    // byte permutation building columns W, W+1 from W-2, W-3: staged, from the left neighbour's
    // group (the perm's high operand); else from the lane's own reload of W-4..W-1
    T.msel = T.mirror_right ? (STAGED ? 0x04040506u : 0x00000102u) : 0x03020100u;
    T.right_rem = W & 3;
    // the lane holding column W-1 (on the fast path W % 4 == 0, so its columns end at W-1)
    T.right_fix = c <= W - 1 && W - 1 < c + kLumaCols;
    if constexpr (BPC == 8) {
        T.ym0 = (c < W ? 0xffu : 0u) | (c + 1 < W ? 0xff00u : 0u) | (c + 2 < W ? 0xff0000u : 0u) |
                (c + 3 < W ? 0xff000000u : 0u);
        T.ym1 = 0u;
    } else {
        T.ym0 = (c < W ? 0xffffu : 0u) | (c + 1 < W ? 0xffff0000u : 0u);
        T.ym1 = (c + 2 < W ? 0xffffu : 0u) | (c + 3 < W ? 0xffff0000u : 0u);
    }

    // transposed horizontal halo: 8 bytes of row r0 - 2 + k per lane, inside the row's pitch.
    // Selectors give (column a, column b) as a 16-bit pair: 8-bit picks bytes (0x0c = zero),
    // 10-bit picks 16-bit samples.
    {
        const int k = min(lane & (kWave / 2 - 1), TH + 3);
        const int hrow = mirror_clamp(T.r0 - 2 + k, H);
        const int e = s + kStripCols;  // first column right of the tile
        int col;
        uint32_t sel;
        halo_source<BPC>(lane, T.strip, s, W, col, sel);
        T.hvoff = (uint32_t)(col * B) + (uint32_t)hrow * (uint32_t)a.pitch[0];
        T.hsel = sel;
        T.hlds = 0u;
        T.halo_fix = false;
        if constexpr (STAGED) {
            // 16-byte aligned chunks: left, the chunk ending at s (its last dword holds columns
            // s-4..s-1) or at the frame edge the first chunk (columns 0..3); right, the chunk
            // starting at e, or the one ending at W when the frame ends at e
            int chunk, dw;
            if (lane < kWave / 2) {
                chunk = T.strip == 0 ? 0 : s - 16;
                dw = T.strip == 0 ? 0 : 3;
                sel = T.strip == 0 ? 0x0c010c02u : 0x0c030c02u;
            } else if (e < W) {
                chunk = e;
                dw = 0;
                sel = 0x0c010c00u;  // columns e, e+1 (e+1 = W is fixed up by halo_fix)
            } else if (e == W) {
                chunk = W - 16;
                dw = 3;
                sel = 0x0c010c02u;
            } else {
                chunk = 0;
                dw = 0;
                sel = 0u;
            }
            T.hvoff = (uint32_t)chunk + (uint32_t)hrow * (uint32_t)a.pitch[0];
            T.hsel = sel;
            T.hlds = (uint32_t)(Stage<TH>::kHalo * kWave + 4 * lane + dw);
            T.halo_fix = lane == kWave - 1 && e == W - 1;
        }
    }

    // chroma split: 8-bit, 32 lanes (one dword each) per chroma row and two rows per step (the
    // upper half-wave takes the second); 10-bit, one row per step, 64 dwords
    const int cs = s / 2;  // first chroma sample of the tile
    int ccol;
    if constexpr (BPC == 8) {
        ccol = cs + 4 * (lane & 31);
        T.c_upper = lane >= 32;
        T.c_on = ccol < a.Wc;
        T.cm = (ccol < a.Wc ? 0xffu : 0u) | (ccol + 1 < a.Wc ? 0xff00u : 0u) |
               (ccol + 2 < a.Wc ? 0xff0000u : 0u) | (ccol + 3 < a.Wc ? 0xff000000u : 0u);
    } else {
        ccol = cs + 2 * lane;
        T.c_upper = false;
        T.c_on = ccol < a.Wc;
        T.cm = (ccol < a.Wc ? 0xffffu : 0u) | (ccol + 1 < a.Wc ? 0xffff0000u : 0u);
    }
    T.crow0 = uni(T.r0 / 2);
    if constexpr (STAGED) {
        // staged chroma: lane l reads the 16 bytes at column cs + 16 (l mod 8) of tile chroma row
        // 8q + l / 8; rows past the tile's TH / 2 or past the plane, and columns past Wc, are
        // masked out. On the fast path only the last strip's tiles (W inside them) reach past
        // the plane, since H is a multiple of TH; with one load per plane the rows past TH / 2
        // are whole lanes, left out of the chroma sums through c_on. So the byte masks are
        // applied only on the generic path, on edge tiles and with two loads per plane (20 rows).
        const int c16 = cs + 16 * (lane & 7);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = 8 * q + (lane >> 3);
            const bool row_ok = row < TH / 2 && T.crow0 + row < a.Hc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t m = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    m |= c16 + 4 * j + b < a.Wc ? 0xffu << (8 * b) : 0u;
                T.cmk[q][j] = row_ok ? m : 0u;
            }
        }
        T.cmask = GENERIC || T.edge_tile || Stage<TH>::kChromaLoads > 1;
        T.c_on = T.cmask || (lane >> 3) < TH / 2;
    }
    {
        const uint32_t col = T.c_on ? (uint32_t)(ccol * B) : 0u;
        const int pk[4] = {1, 4, 2, 5};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            T.coff[k] = col + (T.c_upper ? (uint32_t)a.pitch[pk[k]] : 0u);
    }

    // every tile of a launch takes the same path, so wavefronts cost the same and none trails
    // staged: per-lane offsets of the 16-byte loads (16 lanes per luma row, 8 per chroma row)
    StageOffsets<TH> O;
    if constexpr (STAGED) {
        // a 16-byte group wholly right of the frame (the last strip of a width that is not a
        // multiple of 256) loads the strip's first group instead: the same bytes as another lane
        // of the row, so the request coalesces and no row padding is fetched from HBM. Those
        // columns feed no output (the right-edge mirror takes the lane to the left's group).
        const int g = s + 16 * (lane & 15), gc = s / 2 + 16 * (lane & 7);
        const uint32_t col = (uint32_t)(g < W ? g : s);
        const uint32_t ccol16 = (uint32_t)(gc < a.Wc ? gc : s / 2);
#pragma unroll
        for (int q = 0; q < Stage<TH>::kRefLoads; ++q) {
            const int row = mirror_clamp(T.r0 - 2 + 4 * q + (lane >> 4), H);
            O.ref[q] = col + (uint32_t)row * (uint32_t)a.pitch[0];
        }
        O.dist = col + (uint32_t)(lane >> 4) * (uint32_t)a.pitch[3];
        const int pk[4] = {1, 4, 2, 5};
#pragma unroll
        for (int p = 0; p < 4; ++p)
            O.chroma[p] = ccol16 + (uint32_t)(lane >> 3) * (uint32_t)a.pitch[pk[p]];
    }

    if constexpr (V2) {
        // previous reference luma: from the launch before (saved plane), else none (chunk 0), or
        // loaded by the chunk's prologue (later chunks)
        typename Px<BPC>::Luma prev[TH + 4];
        uint32_t pxprev = 0;
        bool have_prev = false;
        if (T.chunk == 0 && a.has_prev) {
            load_saved<BPC, TH, GENERIC, STAGED>(a, T, s, prev, pxprev);
            have_prev = true;
        } else {
#pragma unroll
            for (int k = 0; k < TH + 4; ++k)
                prev[k] = typename Px<BPC>::Luma{};
        }
        frame_loop_v2<BPC, TH, GENERIC, STAGED, MOM, V2 == 2>(a, T, O, prev, pxprev, have_prev,
                                                             stage);
        // the state stores drain while the group count is in flight
        bool arrived;
        if (T.chunk == a.chunks - 1 && a.ring_out) {
            store_saved<BPC, TH>(a, T, s, prev);
            arrived = count_arrival<TH>(a, lane);
        } else {
            arrived = count_arrival<0>(a, lane);
        }
        publish_if_last<MOM ? kMaxSums : kSums>(a, lane, arrived);
    } else {
        // previous blurred tile: from the launch before, else none (chunk 0), or re-blurred by
        // the chunk's prologue (later chunks)
        uint32_t prev0[TH], prev1[TH];
        bool have_prev = false;
        if (!ONE && T.chunk == 0 && a.has_prev) {
            load_prev_tile<TH>(a, T, prev0, prev1);
            have_prev = true;
        } else {
#pragma unroll
            for (int i = 0; i < TH; ++i)
                prev0[i] = prev1[i] = 0;
        }

        frame_loop<BPC, TH, GENERIC, STAGED, MOM, ONE>(a, T, O, prev0, prev1, have_prev, stage);

        // the state stores (TH instructions) drain while the group count is in flight; they are
        // non-temporal, so the launch's end does not find 16 MB (at 4K) of them dirty in L2
        // (measured 2.6 us per 4K 8-bit launch)
        bool arrived;
        if (T.chunk == a.chunks - 1 && a.ring_out) {
            unsigned long long *rout = reinterpret_cast<unsigned long long *>(a.ring_out);
#pragma unroll
            for (int i = 0; i < TH; ++i)
                __builtin_nontemporal_store(((unsigned long long)prev1[i] << 32) | prev0[i],
                                            rout + (T.tile * TH + i) * kWave + lane);
            arrived = count_arrival<TH>(a, lane);
        } else {
            arrived = count_arrival<0>(a, lane);
        }
        publish_if_last<MOM ? kMaxSums : kSums>(a, lane, arrived);
    }
}


#ifndef IIR_STAGE8
#define IIR_STAGE8 1
#endif
#ifndef IIR_STAGE10
#define IIR_STAGE10 0
#endif
#ifndef IIR_WPE12
#define IIR_WPE12 3
#endif
#ifndef IIR_WPE16
#define IIR_WPE16 2
#endif
#ifndef IIR_WPE20
#define IIR_WPE20 2
#endif

// Every (bit depth, tile height, path) the host may pick. The fast path needs W % 8 == 0 and
// H % TH == 0 (no ragged tile, no partial sample group); the generic path takes any size.
// Motion v2 of 16-bit storage carries the previous frame's 16-bit rows beside the 64-bit squared
// error sums: it only has the 12-row tile, at two wavefronts per SIMD (taller tiles spill).
template <int BPC, bool GENERIC, bool MOM, int V2 = 0>
FramesFn frames_fn(int th)
{
    constexpr bool P = BPC == 8 ? IIR_STAGE8 : IIR_STAGE10;
    if constexpr (BPC == 16 && V2) {
        return th == 12 ? frames_kernel<BPC, 12, P, GENERIC, 2, MOM, V2> : nullptr;
    } else if constexpr (BPC == 10 && V2 && MOM) {
        // 10-bit motion v2 with moments holds two frames' rows beside the moment sums: the 12-row
        // tile spills at three wavefronts per SIMD and the 20-row tile at two, so it has the 12-
        // and 16-row tiles at two wavefronts per SIMD, without scratch
        switch (th) {
        case 12:
            return frames_kernel<BPC, 12, P, GENERIC, 2, MOM, V2>;
        case 16:
            return frames_kernel<BPC, 16, P, GENERIC, IIR_WPE16, MOM, V2>;
        default:
            return nullptr;
        }
    } else {
        switch (th) {
        case 12:
            return frames_kernel<BPC, 12, P, GENERIC, IIR_WPE12, MOM, V2>;
        case 16:
            return frames_kernel<BPC, 16, P, GENERIC, IIR_WPE16, MOM, V2>;
        case 20:
            return frames_kernel<BPC, 20, P, GENERIC, IIR_WPE20, MOM, V2>;
        default:
            return nullptr;
        }
    }
}

// The one-frame kernels (8-bit staged, blurred-frame SAD), or nullptr.
template <bool GENERIC, bool MOM>
FramesFn frames_fn_one(int th)
{
    switch (th) {
    case 12:
        return frames_kernel<8, 12, true, GENERIC, IIR_WPE12, MOM, 0, true>;
    case 16:
        return frames_kernel<8, 16, true, GENERIC, IIR_WPE16, MOM, 0, true>;
    case 20:
        return frames_kernel<8, 20, true, GENERIC, IIR_WPE20, MOM, 0, true>;
    default:
        return nullptr;
    }
}

}  // namespace
}  // namespace iir

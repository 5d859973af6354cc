// iir_kernels.hip -- gfx950 kernels for the integer motion (blurred-luma SAD) and PSNR (per-plane
// SSE) sums of 4:2:0 video, 8 and 10 bits per sample.
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
//   * One wavefront per workgroup owns one tile: 4 * lanes_out luma columns x kRowsPerTile rows.
//     Lane l holds 4 adjacent luma columns; lanes 0 and lanes_out + 1 only feed the horizontal
//     halo. Each lane slides down its columns with the whole 5-row window in registers, so every
//     vertical value is computed exactly once and reused by the five horizontal taps through two
//     DPP lane shifts per row (no LDS round trip, no barrier).
//   * The separable filter runs on packed 16-bit pairs: v_perm_b32 builds (row r, row r+1) pairs
//     per column, v_dot2_u32_u16 applies two taps per instruction with the rounding constant as
//     the accumulator, and v_perm_b32 extracts the 16-bit result of a byte-aligned shift. 10-bit
//     input is pre-scaled by 64 so its vertical shift (10) also becomes a 16-bit byte shift.
//   * SAD on packed blurred pairs: |a - b| = a + b - 2 min(a, b), with sum(b) kept from the
//     previous frame, so each pair costs one v_pk_min_u16 and two v_dot2 accumulations.
//   * SSE: 8-bit as sum(r^2 + d^2) - 2 sum(r d) with v_dot4_u32_u8 (exact in 32-bit modular
//     arithmetic, since the true per-lane value is far below 2^32); 10-bit as v_pk_sub_i16 then
//     v_dot2_i32_i16 of the difference with itself.
//   * A workgroup loops over the frames of its time chunk, keeping the previous blurred tile in
//     registers; the blurred state crosses launches through a small tiled plane (ring).
//   * Per frame, per workgroup: one 64-bit atomic per sum ("ADR-1392", Decision 1), into one of
//     kSumSlots partial slots chosen by XCD; the host adds the slots.
//   * Workgroup ids are remapped so each XCD (and its L2) gets a contiguous run of vertically
//     adjacent tiles, which share their halo rows.
#include <algorithm>

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

__device__ __forceinline__ uint32_t pkmin(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// lane i receives lane i-1's value (wave_shr:1); lane 0 receives 0
__device__ __forceinline__ uint32_t from_left(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xf, 0xf, false);
}

// lane i receives lane i+1's value (wave_shl:1); lane 63 receives 0
__device__ __forceinline__ uint32_t from_right(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xf, 0xf, false);
}

// whole-sample mirror into [0, n), exact for -2 <= i <= n + 1, clamped beyond (never used there)
__device__ __forceinline__ int mirror_clamp(int i, int n)
{
    i = i < 0 ? -i : i;
    i = i >= n ? 2 * n - 2 - i : i;
    return min(max(i, 0), n - 1);
}

// XCD-aware tile order: hardware places workgroup b on XCD b % 8; give each XCD one contiguous
// run of the linear (chunk, strip, row tile) order. A bijection on [0, G) for any G.
__device__ __forceinline__ int xcd_linear(int b, int G)
{
    const int x = b & 7, j = b >> 3;
    const int q = G >> 3, r = G & 7;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// Sum of a per-lane u32 over the wavefront as u64: butterflies inside each 32-lane half (each half
// sum stays below 2^32 for every accumulator here), then the two halves added in 64 bits.
__device__ __forceinline__ unsigned long long wave_sum(uint32_t v)
{
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    const uint32_t lo = __builtin_amdgcn_readlane(v, 0);
    const uint32_t hi = __builtin_amdgcn_readlane(v, 32);
    return (unsigned long long)lo + hi;
}

__device__ __forceinline__ void add_sum(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    typedef uint2 Luma;  // 4 luma samples, 2 per dword
    static constexpr int kBytes = 2;
};

// 4 samples at columns c..c+3 of a luma row, mirrored at the left and right edges.
template <int BPC>
__device__ __forceinline__ typename Px<BPC>::Luma load_luma(const uint8_t *row, int c, int W,
                                                            bool on, bool fast)
{
    typedef typename Px<BPC>::Luma L;
    L v = {};
    if (on) {
        if (fast) {
            v = *reinterpret_cast<const L *>(row + c * Px<BPC>::kBytes);
        } else if constexpr (BPC == 8) {
            uint32_t u = 0;
            for (int b = 0; b < 4; ++b)
                u |= (uint32_t)row[mirror_clamp(c + b, W)] << (8 * b);
            v = u;
        } else {
            const uint16_t *r16 = reinterpret_cast<const uint16_t *>(row);
            uint32_t e[4];
            for (int b = 0; b < 4; ++b)
                e[b] = r16[mirror_clamp(c + b, W)];
            v.x = e[0] | (e[1] << 16);
            v.y = e[2] | (e[3] << 16);
        }
    }
    return v;
}

// Distorted luma of an output lane. Columns at or past W take the reference sample instead, so
// their squared difference is 0.
template <int BPC>
__device__ __forceinline__ typename Px<BPC>::Luma load_dist(const uint8_t *row, int c, int W,
                                                            bool on, bool full,
                                                            typename Px<BPC>::Luma ref)
{
    typedef typename Px<BPC>::Luma L;
    L v = ref;
    if (on) {
        if (full) {
            v = *reinterpret_cast<const L *>(row + c * Px<BPC>::kBytes);
        } else if constexpr (BPC == 8) {
            uint32_t u = ref;
            for (int b = 0; b < 4; ++b)
                if (c + b < W)
                    u = (u & ~(0xffu << (8 * b))) | ((uint32_t)row[c + b] << (8 * b));
            v = u;
        } else {
            const uint16_t *r16 = reinterpret_cast<const uint16_t *>(row);
            uint32_t e[4] = {ref.x & 0xffffu, ref.x >> 16, ref.y & 0xffffu, ref.y >> 16};
            for (int b = 0; b < 4; ++b)
                if (c + b < W)
                    e[b] = r16[c + b];
            v.x = e[0] | (e[1] << 16);
            v.y = e[2] | (e[3] << 16);
        }
    }
    return v;
}

// One chroma dword (4 samples at 8 bits, 2 at 10 bits) starting at sample cb; samples at or past
// wc read as 0 in both ref and dist.
template <int BPC>
__device__ __forceinline__ uint32_t load_chroma(const uint8_t *row, int cb, int wc, bool on)
{
    constexpr int per = 4 / Px<BPC>::kBytes;
    uint32_t v = 0;
    if (on) {
        if (cb + per <= wc) {
            v = *reinterpret_cast<const uint32_t *>(row + cb * Px<BPC>::kBytes);
        } else if constexpr (BPC == 8) {
            for (int b = 0; b < 4; ++b)
                if (cb + b < wc)
                    v |= (uint32_t)row[cb + b] << (8 * b);
        } else {
            const uint16_t *r16 = reinterpret_cast<const uint16_t *>(row);
            if (cb < wc)
                v = r16[cb];
        }
    }
    return v;
}

// (row a, row b) 16-bit pairs of the lane's 4 columns, the vertical filter's operands.
template <int BPC>
__device__ __forceinline__ void column_pairs(typename Px<BPC>::Luma a, typename Px<BPC>::Luma b,
                                             uint32_t p[4])
{
    if constexpr (BPC == 8) {
        p[0] = perm(b, a, 0x0c040c00u);
        p[1] = perm(b, a, 0x0c050c01u);
        p[2] = perm(b, a, 0x0c060c02u);
        p[3] = perm(b, a, 0x0c070c03u);
    } else {
        // 10-bit samples scaled by 64 (still < 2^16): the vertical shift by 10 becomes >> 16
        const uint32_t ax = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a.x) << 6);
        const uint32_t ay = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a.y) << 6);
        const uint32_t bx = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, b.x) << 6);
        const uint32_t by = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, b.y) << 6);
        p[0] = perm(bx, ax, 0x05040100u);
        p[1] = perm(bx, ax, 0x07060302u);
        p[2] = perm(by, ay, 0x05040100u);
        p[3] = perm(by, ay, 0x07060302u);
    }
}

template <int BPC>
__global__ __launch_bounds__(kWave) void frames_kernel(const KernelArgs a)
{
    typedef typename Px<BPC>::Luma Luma;
    constexpr int TH = kRowsPerTile;
    // vertical rounding constant, and the selector taking the 16-bit vertical value out of the
    // 32-bit sums of columns (0, 1): bytes 1-2 (>> 8) at 8 bits, bytes 2-3 (>> 16) for scaled 10
    constexpr uint32_t kVRound = BPC == 8 ? 128u : 32768u;
    constexpr uint32_t kVSel = BPC == 8 ? 0x06050201u : 0x07060302u;

    const int lane = threadIdx.x;

    // clear the other sum buffer for the next submission
    for (int i = blockIdx.x * kWave + lane; i < a.zero_n; i += gridDim.x * kWave)
        a.zero[i] = 0ull;

    const int L = xcd_linear(blockIdx.x, gridDim.x);
    const int chunk = L / a.tiles;
    const int tile = L - chunk * a.tiles;
    const int strip = tile / a.row_tiles;
    const int rt = tile - strip * a.row_tiles;
    const int s = strip * kLumaCols * a.lanes_out;  // first output column of the tile
    const int r0 = rt * TH;                         // first output row of the tile
    const int slot = blockIdx.x & (kSumSlots - 1);
    const int W = a.W, H = a.H;

    // lane roles and column validity
    const int c = s - kLumaCols + kLumaCols * lane;  // first luma column of this lane
    const int need_end = min(s + kLumaCols * a.lanes_out, W) + 2;
    const bool luma_on = lane <= a.lanes_out + 1 && c + kLumaCols > s - 2 && c < need_end;
    const bool luma_fast = c >= 0 && c + kLumaCols <= W;
    const bool out_lane = lane >= 1 && lane <= a.lanes_out && c < W;
    const bool out_full = out_lane && c + kLumaCols <= W;
    // per-column weights of the two blurred pairs: 1 in each valid 16-bit half
    const uint32_t w0 = out_lane ? ((c < W ? 1u : 0u) | (c + 1 < W ? 0x10000u : 0u)) : 0u;
    const uint32_t w1 = out_lane ? ((c + 2 < W ? 1u : 0u) | (c + 3 < W ? 0x10000u : 0u)) : 0u;

    // chroma work split: 8-bit, 32 lanes per chroma row (lanes_out / 2 dwords used), two rows per
    // step; 10-bit, one row per step with lanes_out dwords
    const int cs = s / 2;  // first chroma sample of the tile
    int ccol, crow_sub, csteps, crow_step;
    bool c_on;
    if constexpr (BPC == 8) {
        ccol = cs + 4 * (lane & 31);
        crow_sub = lane >> 5;
        c_on = (lane & 31) < a.lanes_out / 2;
        csteps = TH / 4;
        crow_step = 2;
    } else {
        ccol = cs + 2 * lane;
        crow_sub = 0;
        c_on = lane < a.lanes_out;
        csteps = TH / 2;
        crow_step = 1;
    }
    const int crow0 = r0 / 2 + crow_sub;

    // time chunk of this workgroup; chunks after the first re-blur the frame before them
    const int f_begin = chunk * a.chunk_len;
    const int f_end = min(f_begin + a.chunk_len, a.nframes);
    const int t_start = chunk > 0 ? f_begin - 1 : f_begin;

    uint32_t prev0[TH], prev1[TH];
    uint32_t sum_prev = 0;
    bool have_prev = false;
    if (chunk == 0 && a.has_prev) {
        const uint2 *rin = reinterpret_cast<const uint2 *>(a.ring_in);
#pragma unroll
        for (int i = 0; i < TH; ++i) {
            const uint2 v = rin[(tile * TH + i) * kWave + lane];
            prev0[i] = v.x;
            prev1[i] = v.y;
            if (r0 + i < H)
                sum_prev = dot2u(v.y, w1, dot2u(v.x, w0, sum_prev));
        }
        have_prev = true;
    } else {
#pragma unroll
        for (int i = 0; i < TH; ++i)
            prev0[i] = prev1[i] = 0;
    }

    for (int t = t_start; t < f_end; ++t) {
        const bool prologue = t < f_begin;
        const uint8_t *fp[6];
#pragma unroll
        for (int k = 0; k < 6; ++k)
            fp[k] = a.table ? a.table[t].p[k] : a.base[k] + (int64_t)t * a.fstride[k];

        // reference luma rows r0-2 .. r0+TH+1, mirrored at the top and bottom
        Luma R[TH + 5];
#pragma unroll
        for (int k = 0; k < TH + 4; ++k) {
            const int row = mirror_clamp(r0 - 2 + k, H);
            R[k] = load_luma<BPC>(fp[0] + (int64_t)row * a.pitch[0], c, W, luma_on, luma_fast);
        }
        R[TH + 4] = Luma{};

        // blur, and the SAD against the previous blurred tile
        uint32_t acc_c = 0, acc_min = 0;
#pragma unroll
        for (int i = 0; i < TH; ++i) {
            uint32_t pa[4], pb[4], pc[4];
            column_pairs<BPC>(R[i], R[i + 1], pa);      // rows i-2, i-1
            column_pairs<BPC>(R[i + 2], R[i + 3], pb);  // rows i,   i+1
            column_pairs<BPC>(R[i + 4], R[i + 5], pc);  // rows i+2 (i+3 has tap 0)
            uint32_t v[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                v[b] = dot2u(pc[b], T0z, dot2u(pb[b], T21, dot2u(pa[b], T01, kVRound)));
            const uint32_t q0 = perm(v[1], v[0], kVSel);  // V of columns c, c+1
            const uint32_t q1 = perm(v[3], v[2], kVSel);  // V of columns c+2, c+3
            const uint32_t ql = from_left(q1);            // V of columns c-2, c-1
            const uint32_t qr = from_right(q0);           // V of columns c+4, c+5
            const uint32_t h0 = dot2u(q1, T0z, dot2u(q0, T21, dot2u(ql, T01, 32768u)));
            const uint32_t h1 = dot2u(q1, T10, dot2u(q0, T12, dot2u(ql, Tz0, 32768u)));
            const uint32_t h2 = dot2u(qr, T0z, dot2u(q1, T21, dot2u(q0, T01, 32768u)));
            const uint32_t h3 = dot2u(qr, T10, dot2u(q1, T12, dot2u(q0, Tz0, 32768u)));
            const uint32_t c0 = perm(h1, h0, 0x07060302u);  // Bl of columns c, c+1
            const uint32_t c1 = perm(h3, h2, 0x07060302u);  // Bl of columns c+2, c+3
            if (r0 + i < H) {
                acc_c = dot2u(c1, w1, dot2u(c0, w0, acc_c));
                if (have_prev)
                    acc_min = dot2u(pkmin(c1, prev1[i]), w1, dot2u(pkmin(c0, prev0[i]), w0, acc_min));
            }
            prev0[i] = c0;
            prev1[i] = c1;
        }

        if (!prologue) {
            // SSE of the luma tile
            uint32_t sy = 0, sy2 = 0;
#pragma unroll
            for (int i = 0; i < TH; ++i) {
                const int row = r0 + i;
                if (row < H) {
                    const Luma r = R[i + 2];
                    const Luma d = load_dist<BPC>(fp[3] + (int64_t)row * a.pitch[3], c, W, out_lane,
                                                  out_full, r);
                    if (out_lane) {
                        if constexpr (BPC == 8) {
                            sy = dot4u(d, d, dot4u(r, r, sy));
                            sy2 = dot4u(r, d, sy2);
                        } else {
                            sy = sqdiff2(r.y, d.y, sqdiff2(r.x, d.x, sy));
                        }
                    }
                }
            }
            // SSE of the chroma tiles
            uint32_t su = 0, su2 = 0, sv = 0, sv2 = 0;
#pragma unroll
            for (int k = 0; k < TH / 2; ++k) {
                if (k < csteps) {
                    const int row = crow0 + crow_step * k;
                    const bool on = c_on && row < a.Hc;
                    const int64_t ro = (int64_t)(on ? row : 0);
                    const uint32_t ru = load_chroma<BPC>(fp[1] + ro * a.pitch[1], ccol, a.Wc, on);
                    const uint32_t du = load_chroma<BPC>(fp[4] + ro * a.pitch[4], ccol, a.Wc, on);
                    const uint32_t rv = load_chroma<BPC>(fp[2] + ro * a.pitch[2], ccol, a.Wc, on);
                    const uint32_t dv = load_chroma<BPC>(fp[5] + ro * a.pitch[5], ccol, a.Wc, on);
                    if constexpr (BPC == 8) {
                        su = dot4u(du, du, dot4u(ru, ru, su));
                        su2 = dot4u(ru, du, su2);
                        sv = dot4u(dv, dv, dot4u(rv, rv, sv));
                        sv2 = dot4u(rv, dv, sv2);
                    } else {
                        su = sqdiff2(ru, du, su);
                        sv = sqdiff2(rv, dv, sv);
                    }
                }
            }
            const uint32_t sad = have_prev ? acc_c + sum_prev - 2u * acc_min : 0u;
            const unsigned long long t_sad = wave_sum(sad);
            const unsigned long long t_y = wave_sum(sy - 2u * sy2);
            const unsigned long long t_u = wave_sum(su - 2u * su2);
            const unsigned long long t_v = wave_sum(sv - 2u * sv2);
            if (lane == 0) {
                unsigned long long *o = a.sums + (size_t)t * (kSums * kSumSlots) + slot;
                add_sum(o, t_sad);
                add_sum(o + kSumSlots, t_y);
                add_sum(o + 2 * kSumSlots, t_u);
                add_sum(o + 3 * kSumSlots, t_v);
            }
        }
        sum_prev = acc_c;
        have_prev = true;
    }

    if (chunk == a.chunks - 1) {
        uint2 *rout = reinterpret_cast<uint2 *>(a.ring_out);
#pragma unroll
        for (int i = 0; i < TH; ++i)
            rout[(tile * TH + i) * kWave + lane] = make_uint2(prev0[i], prev1[i]);
    }
}

// Tiled blurred state -> W x H uint16 plane.
__global__ void export_kernel(const uint32_t *ring, uint16_t *dst, int64_t pitch, int W, int H,
                              int lanes_out, int row_tiles)
{
    const int pairs = (W + 1) / 2;
    const int64_t n = (int64_t)pairs * H;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int row = (int)(idx / pairs);
        const int j = 2 * (int)(idx - (int64_t)row * pairs);
        const int sw = kLumaCols * lanes_out;
        const int strip = j / sw;
        const int in = j - strip * sw;
        const int lane = in / kLumaCols + 1;
        const int half = (in % kLumaCols) / 2;
        const int tile = strip * row_tiles + row / kRowsPerTile;
        const uint32_t w = ring[(((int64_t)tile * kRowsPerTile + row % kRowsPerTile) * kWave + lane) * 2 + half];
        uint16_t *d = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(dst) + row * pitch);
        d[j] = (uint16_t)(w & 0xffffu);
        if (j + 1 < W)
            d[j + 1] = (uint16_t)(w >> 16);
    }
}

// Memory-ceiling probes: read-only (xor-reduced, written only if a runtime flag asks), write-only,
// copy. 16-byte accesses, grid-stride.
__global__ __launch_bounds__(256) void probe_read(const uint4 *src, int64_t n, uint4 *sink, int keep)
{
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint4 v = src[i];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    if (keep)
        sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void probe_write(uint4 *dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = make_uint4((uint32_t)i, (uint32_t)(i >> 32), 0x9e3779b9u, 0u);
}

__global__ __launch_bounds__(256) void probe_copy(const uint4 *src, uint4 *dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

}  // namespace

hipError_t launch_frames(int bpc, const KernelArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.tiles * a.chunks)), block(kWave);
    if (bpc == 8)
        hipLaunchKernelGGL(frames_kernel<8>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(frames_kernel<10>, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_export(const uint32_t *ring, uint16_t *dst, int64_t pitch, int W, int H,
                         int lanes_out, int row_tiles, hipStream_t stream)
{
    const int64_t n = (int64_t)((W + 1) / 2) * H;
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(export_kernel, dim3(blocks), dim3(256), 0, stream, ring, dst, pitch, W, H,
                       lanes_out, row_tiles);
    return hipGetLastError();
}

// The probe's sink (mode 0) is dst; it must hold blocks * 256 * 16 bytes, which bytes covers.
hipError_t launch_probe(int mode, const void *src, void *dst, int64_t bytes, hipStream_t stream)
{
    const int64_t n = bytes / 16;
    const unsigned blocks = (unsigned)std::min<int64_t>(std::max<int64_t>(n / (256 * 4), 1), 256 * 16);
    if (mode == 0)
        hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint4 *>(src), n, static_cast<uint4 *>(dst), 0);
    else if (mode == 1)
        hipLaunchKernelGGL(probe_write, dim3(blocks), dim3(256), 0, stream,
                           static_cast<uint4 *>(dst), n);
    else
        hipLaunchKernelGGL(probe_copy, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace iir

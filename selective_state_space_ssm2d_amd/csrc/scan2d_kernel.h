// libssm2d: 2DMamba 2D selective scan (forward) for MI355X / gfx950 -- the
// kernel and its launch, shared by the translation units of the library.
//
// Method (juejin.cn "2DMamba 精读", part 四 section 5; papernotes.org "2DMamba" 关键设计):
//   Abar = exp(delta*A), Bx = delta*B*x
//   hh[i,j] = Abar*hh[i,j-1] + Bx         horizontal scan, zero before column 0
//   h[i,j]  = Abar*h[i-1,j]  + hh[i,j]    vertical scan of the horizontal results
//   y = sum_n C*h + D*x                   state dims reduced on chip, only y stored
//
// Work decomposition (gfx950-specific; the pages' CUDA tiling is prior art):
//   * One wave = 64 lanes = 16 channels d x 4 state groups g. All lanes of a
//     wave work on the same cell at the same time, so B and C (shared by all
//     channels) and x / delta (one row segment per channel) arrive together.
//     Each lane keeps NPL states (n = g*NPL + k).
//   * A lane walks a strip of K columns from the top row to the bottom row.
//     Along a row it runs the horizontal recurrence sequentially; the vertical
//     state of its K columns stays in registers. Only the strip's last
//     columns are masked: nothing is padded to the wavefront width.
//   * Inputs: a wave's whole input for one row (x and delta of 16 channels,
//     B and C of 4*NPL states, K cells each) is a packet of 16-byte chunks,
//     one coalesced load per lane. Packets are prefetched P rows ahead into a
//     register ring and staged through a per-wave LDS packet buffer, from
//     which each lane reads its operands (B and C reads are broadcasts).
//   * The horizontal carry (hh at the strip's right edge, per row) flows to
//     the next strip. Strips of one (batch, channel block) form a chain:
//     waves of a workgroup hand carries on through an LDS ring, workgroups
//     through tagged 64-bit words (epoch, row | value) written and polled with
//     relaxed device-scope atomics, so no cache flush or invalidate is needed.
//     A strip only waits for the row it is about to process: the chain is a
//     pipeline, one row deep per strip.
//   * Multi-workgroup chains take tickets from an atomic counter; ticket order
//     puts every producer before its consumer, so a waiting workgroup's
//     producer is resident or done. The global ring is bounded, with
//     back-pressure, and followed by overflow rows: a producer waits for a
//     consumer only once that consumer has reported progress, and otherwise
//     moves on to the overflow rows, so none waits on a consumer that has not
//     started (bound_ring below).
//   * The sum over n: each lane holds K partial sums over its NPL states; two
//     permlane swaps (32- and 16-lane) transpose-reduce them across the 4 state
//     groups, leaving each lane with K/4 finished cells.
// Modes (compile time, kMode* below) reuse this structure for the other scan
// directions and orders (pages: papernotes 消融实验要点 and 局限与展望; juejin
// part 七 section 4), for accumulating and gated outputs (Mamba's operator
// options), and for the backward pass: a forward that stores every state and
// an adjoint pass that scans right to left and bottom to top.
// No MFMA: the scan is not a dense contraction.

#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "ssm2d.h"

namespace ssm2d_impl {

constexpr int kWave = 64;
constexpr int kMaxWaves = 10;                  // waves per workgroup (strips + couriers)

// Kernel modes (bits, fixed at compile time):
//   kModeFlipW       rows are scanned right to left
//   kModeVFirst      the column recurrence runs before the row recurrence
//   kModeAccumulate  the result is added to y instead of stored
//   kModeStates      forward pass that writes every state h and no y
//   kModeBackward    adjoint pass of the backward (with kModeFlipW and rows
//                    bottom to top): gradients from the stored states
//   kModeGate        the result is multiplied by SiLU(z) before it is stored
//   kModeEdges       (with kModeBackward) chains cross workgroups without
//                    courier waves: boundary strips use the global ring
//                    themselves
//   kModeRowCarry    (not accumulating or gated) carried horizontal states:
//                    each row's recurrence starts from hh_init and its state
//                    after the last column goes to hh_last (a band of columns
//                    continuing a scan; in the adjoint pass dL/dhh_last in,
//                    dL/dhh_init out)
constexpr int kModeFlipW = 1;
constexpr int kModeVFirst = 2;
constexpr int kModeAccumulate = 4;
constexpr int kModeStates = 8;
constexpr int kModeBackward = 16;
constexpr int kModeGate = 32;
constexpr int kModeEdges = 64;
constexpr int kModeRowCarry = 128;

// Waves per workgroup: 10 (up to 3 per SIMD) when a lane's register state is
// small (8 state groups, K * NPL <= 16; K * NPL <= 8 for the stored-state
// pass; never for the adjoint pass), else 8, which leaves a wave 256 VGPRs.
// A chain cut into more workgroups than the chip holds at once waits for the
// first ones to finish, so the larger workgroup pays even at lower occupancy.
constexpr int max_waves(int K, int NPL, int G, int MODE = 0)
{
    if (MODE & kModeBackward) return 8;
    if (MODE & kModeStates) return (G == 8 && K * NPL <= 8) ? 10 : 8;
    return (G == 8 && K * NPL <= 16) ? 10 : 8;
}
constexpr int kCourierBatch = 4;               // rows a courier requests per poll
constexpr int kMaxSlots = 16;                   // rows of a workgroup's shared row ring
constexpr int kSpinPolls = 64;                  // polls of an LDS counter before sleeping between polls
constexpr int kSkipWaits = 1 << 30;             // above every row index and counter
constexpr float kLog2e = 1.4426950408889634f;

struct Params {
    const void *x, *delta, *B, *C;
    const float *A, *D;
    void *y;
    const void *zeros;                 // zero page, >= H*W*4 bytes
    void *sink;                        // write target of masked-off output lanes
    unsigned int *ticket, *done, *err;
    // Tag epoch of the carry words, kept on the device so that every launch
    // (a replayed graph's too) tags its words differently: each workgroup
    // reads it at its start, the last one to finish advances it. Stored
    // values run 0 .. 65534; a launch's tags use stored + 1.
    unsigned int *epoch;
    unsigned int *herr;                // host-visible timeout flag (may be null)
    unsigned long long *gring;         // [n_bound][qg (+ H)][NPL][64] tagged carries
    unsigned long long *cons;          // [n_bound][2]: consumer progress, first overflow row (epoch<<32 | row)
    long gring_words, cons_words;      // cleared when the epoch wraps
    int batch, d_inner, d_state, H, W;
    int nstrips, s_local, groups, n_dblk, n_chains, total_wg;
    int tblk;                          // chains per block of tickets
    int ring_rows;                     // LDS ring depth between waves
    int qg;                            // global ring depth (== H: no reuse)
    int ovf;                           // bounded ring: 0 no overflow rows, 1 overflow rows for a
                                       // consumer that has not started, 2 (test) every producer
                                       // moves to them after its first 8 rows
    int use_ticket;                    // chains span workgroups
    int xcd_remap;                     // spread chains over XCDs in contiguous blocks
    int vec_store;                     // gather each channel's cells and store whole chunks
    int coop_slots;                    // rows in the workgroup's shared row ring (cooperative loads)
    int coop_shift;                    // log2 of coop_slots
    int flip_h;                        // rows in scan order run bottom to top
    // Stored states (kModeStates writes, kModeBackward reads), fp32, as the
    // waves hold them: one tile per (chain, strip, row) of NPL x 64 lanes x 4
    // cells, [chain][strip][row][k][lane][cell]. Strips are counted from the
    // left over the map padded on the left by `states_pad` columns (to a
    // multiple of 4), so the right-to-left backward meets the same strips.
    float *states;
    int states_pad;
    // backward: upstream gradient, d delta (dx goes to y), and the sums of dB
    // and dC over each wave's 8 channels, [channel block][batch][d_state][H][ld]
    // (rows of ld = 4 * nstrips columns, the map starting at states_pad)
    const void *dy;
    void *ddelta;
    float *dBp, *dCp, *dA, *dD;
    long part_stride;                  // floats per channel block
    const void *z;                     // gate input, shaped like y (kModeGate)
    // carried vertical states, fp32 [batch][d_inner][d_state][W] (may be
    // null): before the first row in scan order, and after the last row
    const float *h_init;
    float *h_last;
    const float *hh_init;              // carried horizontal states [b][d][n][H] (kModeRowCarry)
    float *hh_last;
    long long spin_limit;
};

constexpr unsigned int kEpochs = 65535;  // tag epochs 1 .. 65535 (zero never matches)

// A wait that gave up: the device error word, and the host-visible flag that
// the library's next call on this workspace reports.
__device__ __forceinline__ void report_timeout(const Params &p)
{
    atomicOr(p.err, 1u);
    if (p.herr) __hip_atomic_store(p.herr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float quiet_nan() { return __uint_as_float(0x7fc00000u); }

template <typename T> struct ChunkOf;
template <> struct ChunkOf<float> { using type = float4; };      // 4 fp32
template <> struct ChunkOf<uint16_t> { using type = uint2; };    // 4 bf16

__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Element type of the per-wave input packets in LDS: fp32 for both input
// types. A bf16 chunk is widened (exactly) once, by the lane that stages
// it, instead of by each of the lanes that read its elements (a B or C
// element is read by every channel lane of its state group).
template <typename T, bool COOP> struct PacketOf { using type = float; };
template <> struct PacketOf<uint16_t, true> { using type = uint16_t; };  // (the shared row ring keeps bf16)
__device__ __forceinline__ float4 to_packet(const float4 &c) { return c; }
__device__ __forceinline__ float4 to_packet(uint2 c)
{
    // (widened here, where the chunk is staged: hoisted to where it is
    // loaded, the widened chunks would double the prefetch buffers' registers)
    asm volatile("" : "+v"(c.x), "+v"(c.y));
    return make_float4(bf16_lo(c.x), bf16_hi(c.x), bf16_lo(c.y), bf16_hi(c.y));
}
__device__ __forceinline__ uint2 to_packet_ring(const uint2 &c) { return c; }
__device__ __forceinline__ float4 to_packet_ring(const float4 &c) { return c; }

// One 4-element chunk, read as 4/ALIGN unconditional loads of ALIGN elements.
// Sub-loads that fall past the end of a row were pointed at the zero page when
// the pointers were set up, so no load needs a mask.
template <int ALIGN> struct Sub;
template <> struct Sub<4> { using f = float4; using h = uint2; };
template <> struct Sub<2> { using f = float2; using h = unsigned; };
template <> struct Sub<1> { using f = float; using h = uint16_t; };

template <int ALIGN>
__device__ __forceinline__ float4 load_chunk(const float *const (&sp)[4 / ALIGN], long off)
{
    float4 v;
    if constexpr (ALIGN == 4) {
        v = *reinterpret_cast<const float4 *>(sp[0] + off);
    } else if constexpr (ALIGN == 2) {
        float2 a = *reinterpret_cast<const float2 *>(sp[0] + off);
        float2 b = *reinterpret_cast<const float2 *>(sp[1] + off);
        v.x = a.x; v.y = a.y; v.z = b.x; v.w = b.y;
    } else {
        v.x = sp[0][off]; v.y = sp[1][off]; v.z = sp[2][off]; v.w = sp[3][off];
    }
    return v;
}

template <int ALIGN>
__device__ __forceinline__ uint2 load_chunk(const uint16_t *const (&sp)[4 / ALIGN], long off)
{
    uint2 v;
    if constexpr (ALIGN == 4) {
        v = *reinterpret_cast<const uint2 *>(sp[0] + off);
    } else if constexpr (ALIGN == 2) {
        v.x = *reinterpret_cast<const unsigned *>(sp[0] + off);
        v.y = *reinterpret_cast<const unsigned *>(sp[1] + off);
    } else {
        v.x = static_cast<unsigned>(sp[0][off]) | (static_cast<unsigned>(sp[1][off]) << 16);
        v.y = static_cast<unsigned>(sp[2][off]) | (static_cast<unsigned>(sp[3][off]) << 16);
    }
    return v;
}

// N consecutive packet elements (N % 4 == 0) starting at element offset `off`.
// REV: each chunk holds its 4 cells in reverse order (rows scanned right to
// left are loaded in memory order), so element m of a chunk is cell 3 - m.
template <int N, bool REV = false>
__device__ __forceinline__ void read_packet(const float *pk, int off, float (&v)[N])
{
    constexpr int X = REV ? 3 : 0;
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        float4 t = *reinterpret_cast<const float4 *>(pk + off + 4 * q);
        v[4 * q + (0 ^ X)] = t.x; v[4 * q + (1 ^ X)] = t.y; v[4 * q + (2 ^ X)] = t.z; v[4 * q + (3 ^ X)] = t.w;
    }
}
template <int N, bool REV = false>
__device__ __forceinline__ void read_packet(const uint16_t *pk, int off, float (&v)[N])
{
    constexpr int X = REV ? 3 : 0;
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        uint2 t = *reinterpret_cast<const uint2 *>(pk + off + 4 * q);
        v[4 * q + (0 ^ X)] = bf16_lo(t.x); v[4 * q + (1 ^ X)] = bf16_hi(t.x);
        v[4 * q + (2 ^ X)] = bf16_lo(t.y); v[4 * q + (3 ^ X)] = bf16_hi(t.y);
    }
}
// Cells c0 .. c0+N-1 of a packet row one by one (chunk order as above).
template <int N, bool REV = false>
__device__ __forceinline__ void read_packet_scalar(const float *pk, int off, int c0, float (&v)[N])
{
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = pk[off + (REV ? ((c0 + c) ^ 3) : (c0 + c))];
}
template <int N, bool REV = false>
__device__ __forceinline__ void read_packet_scalar(const uint16_t *pk, int off, int c0, float (&v)[N])
{
#pragma unroll
    for (int c = 0; c < N; ++c)
        v[c] = __uint_as_float(static_cast<unsigned>(pk[off + (REV ? ((c0 + c) ^ 3) : (c0 + c))]) << 16);
}

__device__ __forceinline__ void store_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ unsigned bf16_bits(float v);
__device__ __forceinline__ void store_elem(uint16_t *p, float v) { *p = static_cast<uint16_t>(bf16_bits(v)); }

__device__ __forceinline__ float elem_value(float v) { return v; }
__device__ __forceinline__ float elem_value(uint16_t v) { return __uint_as_float(static_cast<unsigned>(v) << 16); }

__device__ __forceinline__ float perm_sum32(float a, float b)
{
    // v_permlane32_swap: the upper 32 lanes of `a` trade places with the
    // lower 32 lanes of `b`; the sum leaves lanes 0-31 with a(lanes 0-31) +
    // a(lanes 32-63) and lanes 32-63 with b(lanes 0-31) + b(lanes 32-63).
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float perm_sum16(float a, float b)
{
    // v_permlane16_swap: odd 16-lane rows of `a` trade with even rows of `b`.
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane value of the lane 8 places away in the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float row_ror8(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}

// Sum over the 8 lanes of an aligned group of 8 (the 8 channels that share a
// state group in the 8-group layout); every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float v)
{
    // every lane has a source lane here, so bound_ctrl (zero for lanes
    // without one) changes nothing and lets the move fold into the add
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, true));   // quad_perm 2,3,0,1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, true));  // row_half_mirror
    return v;
}

__device__ __forceinline__ float chunk_elem(const float4 &v, int m)
{
    return m == 0 ? v.x : (m == 1 ? v.y : (m == 2 ? v.z : v.w));
}

// Sum over the G state groups of a wave. Lane l holds partial sums p[0..K) of
// K cells; state group g = l / (64 / G). Each halving level pairs groups that
// are 32, 16 (and, for G = 8, 8) lanes apart and keeps half of the cells on
// each side, so lanes end with K / G finished cells: cells [g*K/G, (g+1)*K/G).
// For G = 8 and K = 4 the last level cannot halve: both lanes of a pair end
// with the full sum of cell g / 2.
template <int K, int G>
__device__ __forceinline__ void reduce_groups(const float (&p)[K], float (&out)[(K / G) > 0 ? K / G : 1], int g)
{
    static_assert(G == 4 || G == 8, "4 or 8 state groups");
    float q[K / 2];
#pragma unroll
    for (int c = 0; c < K / 2; ++c) q[c] = perm_sum32(p[c], p[c + K / 2]);
    float r[K / 4];
#pragma unroll
    for (int c = 0; c < K / 4; ++c) r[c] = perm_sum16(q[c], q[c + K / 4]);
    if constexpr (G == 4) {
#pragma unroll
        for (int c = 0; c < K / 4; ++c) out[c] = r[c];
    } else if constexpr (K / 4 == 1) {
        out[0] = r[0] + row_ror8(r[0]);
    } else {
        // even groups keep the first half of their cells, odd groups the second
        const bool odd = (g & 1) != 0;
#pragma unroll
        for (int c = 0; c < K / 8; ++c) {
            const float send = odd ? r[c] : r[c + K / 8];
            const float keep = odd ? r[c + K / 8] : r[c];
            out[c] = keep + row_ror8(send);
        }
    }
}

// Value of `x` held by the lane in 16-lane row r (0..3) at the same position
// within its row, delivered to the lanes of row 0.
__device__ __forceinline__ float from_row(float x, int r)
{
    if (r == 0) return x;
    if (r == 1) return __uint_as_float(__builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false)[1]);
    const float x2 = __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)[1]);
    if (r == 2) return x2;
    return __uint_as_float(__builtin_amdgcn_permlane16_swap(__float_as_uint(x2), __float_as_uint(x2), false, false)[1]);
}

__device__ __forceinline__ unsigned bf16_bits(float v)
{
    const unsigned u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                    // nearest even
}
__device__ __forceinline__ unsigned row_word(unsigned w, int r) { return __float_as_uint(from_row(__uint_as_float(w), r)); }

// Whole-row store of a strip. After reduce_groups the K finished cells of a
// channel sit in the four 16-lane rows (KO per lane). They are converted to the
// output type first (bf16 cells packed in pairs where a lane holds two), then
// collected, in column order, in the channel's lane of row 0 (lane < 64 / G),
// which stores them as whole chunks: K floats, or K bf16 values.
// Exception, 4-column strips (row r holds cell r, in 4 or 8 groups): one swap
// of odd and even rows leaves cells 0, 1 in row 0 and cells 2, 3 in row 2, and
// the channel's lane in each of those rows stores its two cells (pair_lane and
// pair_offset say which lanes and where).
template <int K, int G>
constexpr bool pair_store() { return K == 4; }
template <int K, int G>
__device__ __forceinline__ int pair_lane(int lane) { return pair_store<K, G>() ? (lane & ~32) : lane; }
template <int K, int G, bool REV>
__device__ __forceinline__ int pair_offset(int lane)
{
    // columns left to right: row 2's pair is the chunk's second half;
    // right to left: row 0's pair is
    return (pair_store<K, G>() && ((lane >> 5) & 1) != (REV ? 1 : 0)) ? 2 : 0;
}
template <bool REV>
__device__ __forceinline__ void store_pair(float *p, float v, bool storer)
{
    // after the swap, lo holds cells 0 and 2 in rows 0 and 2, hi cells 1 and 3
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float lo = __uint_as_float(s[0]), hi = __uint_as_float(s[1]);
    if (storer) *reinterpret_cast<float2 *>(p) = REV ? make_float2(hi, lo) : make_float2(lo, hi);
}
template <bool REV>
__device__ __forceinline__ void store_pair(uint16_t *p, float v, bool storer)
{
    // one cell per lane; pairs as for fp32, packed in one word
    const unsigned h = bf16_bits(v);
    const auto s = __builtin_amdgcn_permlane16_swap(h, h, false, false);
    if (storer) *reinterpret_cast<unsigned *>(p) = REV ? (s[1] | (s[0] << 16)) : (s[0] | (s[1] << 16));
}
template <int K, int G, bool REV = false>
__device__ __forceinline__ void store_chunks(float *p, const float (&v)[(K / G) > 0 ? K / G : 1], bool storer)
{
    constexpr int KO = (K / G) > 0 ? K / G : 1;
    float cells[K];
    if constexpr (G == 4) {
        // row r = group r holds cells [r*KO, (r+1)*KO)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < KO; ++c) cells[r * KO + c] = from_row(v[c], r);
    } else {
        // K = 8: in row r, lanes 0-7 (group 2r) hold cell 2r and lanes 8-15
        // (group 2r+1) cell 2r+1, which comes over 8 lanes.
        static_assert(K == 8, "8-group layout stores 4- or 8-column strips");
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            cells[2 * r] = from_row(v[0], r);
            cells[2 * r + 1] = row_ror8(cells[2 * r]);
        }
    }
    if (storer) {
        // REV: the strip's columns run right to left in memory
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
            if constexpr (REV)
                *reinterpret_cast<float4 *>(p + 4 * q) = make_float4(cells[K - 1 - 4 * q], cells[K - 2 - 4 * q],
                                                                     cells[K - 3 - 4 * q], cells[K - 4 - 4 * q]);
            else
                *reinterpret_cast<float4 *>(p + 4 * q) = make_float4(cells[4 * q], cells[4 * q + 1], cells[4 * q + 2], cells[4 * q + 3]);
        }
    }
}
template <int K, int G, bool REV = false>
__device__ __forceinline__ void store_chunks(uint16_t *p, const float (&v)[(K / G) > 0 ? K / G : 1], bool storer)
{
    constexpr int KO = (K / G) > 0 ? K / G : 1;
    unsigned words[K / 2];  // two bf16 cells per word, column order
    if constexpr (G == 4 && KO >= 2) {
        unsigned w[KO / 2];
#pragma unroll
        for (int c = 0; c < KO / 2; ++c) w[c] = bf16_bits(v[2 * c]) | (bf16_bits(v[2 * c + 1]) << 16);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < KO / 2; ++c) words[r * KO / 2 + c] = row_word(w[c], r);
    } else {
        static_assert(G == 8 && K == 8, "bf16 row store layouts");
        const unsigned h = bf16_bits(v[0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const unsigned t = row_word(h, r);
            words[r] = t | (__float_as_uint(row_ror8(__uint_as_float(t))) << 16);
        }
    }
    if constexpr (REV) {
        // columns right to left in memory: word order reversed, halves swapped
        unsigned t[K / 2];
#pragma unroll
        for (int c = 0; c < K / 2; ++c) t[c] = (words[K / 2 - 1 - c] >> 16) | (words[K / 2 - 1 - c] << 16);
#pragma unroll
        for (int c = 0; c < K / 2; ++c) words[c] = t[c];
    }
    if (storer) *reinterpret_cast<uint4 *>(p) = make_uint4(words[0], words[1], words[2], words[3]);
}
template <int K, int G, bool REV = false, typename T>
__device__ __forceinline__ void store_row(T *p, const float (&v)[(K / G) > 0 ? K / G : 1], bool storer)
{
    if constexpr (pair_store<K, G>()) store_pair<REV>(p, v[0], storer);
    else store_chunks<K, G, REV>(p, v, storer);
}

__device__ __forceinline__ void sleep_a_bit() { __builtin_amdgcn_s_sleep(2); }

// Wave-uniform read of an LDS progress counter (kept in a scalar register so
// the waits below compile to scalar branches, not exec-mask juggling).
__device__ __forceinline__ int lds_counter(const int *c)
{
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
}
__device__ __forceinline__ void lds_publish(int *c, int v)
{
    __hip_atomic_store(c, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Relaxed LDS counter access. A wave's LDS accesses execute in order, so a
// counter written after a ring slot (or read before it) orders the two without
// a hardware wait; signal_fence() keeps the compiler from reordering them.
__device__ __forceinline__ int lds_peek(const int *c)
{
    return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_poke(int *c, int v)
{
    __hip_atomic_store(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void signal_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Tile of a ticket. Tickets are dealt in blocks of tblk chains: within a
// block, strip group by strip group, chain by chain. Workgroups start (and take
// tickets) in the order they are dealt to the 8 XCDs round-robin, so with a
// multiple of 8 chains a block each chain's workgroups share one XCD. With the
// bounded ring (back-pressure) tblk is small: only the chains of the last
// block begun can wait on a consumer that has not started, every earlier block
// is wholly running or done and drains, so the grid finishes while other work
// holds part of the device. With one slot a row tblk = n_chains.
__device__ __forceinline__ void ticket_tile(const Params &p, int wg, int &chain, int &grp)
{
    const int per_blk = p.tblk * p.groups;
    const int blk = wg / per_blk;
    const int c0 = blk * p.tblk;
    const int nb = min(p.tblk, p.n_chains - c0);   // chains in this block (the last may hold fewer)
    const int r = wg - blk * per_blk;
    grp = r / nb;
    chain = c0 + r % nb;
}

// Polls counter *c until it exceeds `need` (returns the value seen), or
// until `limit` polls have failed (sets `timed_out`).
__device__ __forceinline__ int wait_counter_above(const int *c, int need, long long limit, bool &timed_out)
{
    long long spins = 0;
    int v;
    while ((v = lds_counter(c)) <= need) {
        if (++spins > limit) {
            timed_out = true;
            break;
        }
        sleep_a_bit();
    }
    return v;
}

__device__ __forceinline__ unsigned long long ld_relaxed(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Packet rows of a wave: x and delta of 64/G channels, B and C of G*NPL states.
// The backward's packet also carries dy (64/G more rows). Its adjoint pass
// prefetches one row per buffer: its rows are long enough to hide the loads,
// and the registers saved keep it free of spills.
template <int NPL, int G, int MODE = 0>
constexpr int packet_rows() { return 2 * (kWave / G) + 2 * G * NPL + ((MODE & kModeBackward) ? kWave / G : 0); }
template <int NPL, int G, int MODE = 0>
constexpr int passes_for(int K) { return (packet_rows<NPL, G, MODE>() * (K / 4) + kWave - 1) / kWave; }
// The stored-state pass with the shared row ring prefetches 8 rows per
// buffer: its state stores share the in-order vector-memory counter with the
// row loads, so a row's load is waited for only after every store issued
// before it, and the longer distance lets those stores drain first. (With
// per-wave packets the extra registers would spill.)
template <int NPL, int G, int MODE = 0, bool COOP = false>
constexpr int prefetch_rows(int K)
{
    if constexpr ((MODE & kModeBackward) != 0) return 1;
    if (passes_for<NPL, G, MODE>(K) != 1) return 2;
    return ((MODE & kModeStates) && COOP) ? 8 : 4;
}


// End of a launch whose chains span workgroups: the last workgroup to
// finish resets the tickets and advances the tag epoch for the next launch.
// When the epoch wraps, the next launch's tags repeat those of a launch 65535
// launches back, whose words may still sit in slots nobody has rewritten
// since (another shape lays the ring out differently): every ring and
// consumer word is cleared first (zero never matches a tag).
__device__ __forceinline__ void finish_launch(const Params &p, const unsigned int s_epoch, int &s_last)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned int old = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old + 1 == static_cast<unsigned int>(p.total_wg)) ? 1 : 0;
        if (s_last) {
            __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (s_last) {
        const unsigned int next = s_epoch % kEpochs;  // stored value of the next launch
        if (next == 0) {
            for (long k = threadIdx.x; k < p.gring_words; k += blockDim.x) st_relaxed(p.gring + k, 0ull);
            for (long k = threadIdx.x; k < p.cons_words; k += blockDim.x) st_relaxed(p.cons + k, 0ull);
        }
        if (threadIdx.x == 0) __hip_atomic_store(p.epoch, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Courier waves of a workgroup whose chain spans workgroups: wave s_local
// brings the left workgroup's carries into LDS ring 0; wave s_local + 1 sends
// LDS ring s_local to the right workgroup. They are separate waves so that
// waiting for loads never also waits for the write-through of stores (one
// counter tracks both). Carries between workgroups are tagged 64-bit words
// (epoch << 16 | row, value) in the global ring, written and polled with
// relaxed device-scope atomics; s_done / s_used are the LDS rings' published
// and consumed row counts.
template <int NPL>
__device__ __forceinline__ void courier_wave(const Params &p, const int wave, const int lane, const int chain, const int grp,
                             float *lring, int *s_done, int *s_used, const unsigned int s_epoch, const long ring_floats,
                             const int RM)
{
    const int H = p.H;
    const long nb_per_chain = p.groups - 1;
    // a boundary's slots: qg ring rows, then (bounded ring with overflow) a
    // row per map row
    const long gstride = static_cast<long>(p.qg + (p.ovf ? H : 0)) * NPL * kWave;
    const unsigned int etag = s_epoch << 16;
    const unsigned long long ctag = static_cast<unsigned long long>(s_epoch) << 32;
    long idle = 0;
    bool timed_out = false;
    // rows at or past ovf_from sit in the overflow rows (as last seen)
    int ovf_from = H;
    auto slot_of = [&](int row) __attribute__((always_inline)) {
        return row >= ovf_from ? p.qg + row : row % p.qg;
    };
    if (wave == p.s_local && grp > 0) {
        const long bound_in = chain * nb_per_chain + (grp - 1);
        const unsigned long long *gin = p.gring + bound_in * gstride + lane;
        float *ring0 = lring;
        int in_next = 0;
        while (in_next < H) {
            const int used0 = lds_counter(&s_used[0]);
            const int nb = min(min(kCourierBatch, H - in_next), used0 + p.ring_rows - in_next);
            int v = 0;
            if (nb > 0) {
                unsigned long long w[kCourierBatch][NPL];
#pragma unroll
                for (int r = 0; r < kCourierBatch; ++r)
                    if (r < nb)
#pragma unroll
                        for (int k = 0; k < NPL; ++k)
                            w[r][k] = ld_relaxed(gin + (static_cast<long>(slot_of(in_next + r)) * NPL + k) * kWave);
#pragma unroll
                for (int r = 0; r < kCourierBatch; ++r) {
                    if (r < nb && v == r) {
                        const unsigned long long want = static_cast<unsigned long long>(etag | static_cast<unsigned>(in_next + r)) << 32;
                        bool ok = true;
#pragma unroll
                        for (int k = 0; k < NPL; ++k) ok = ok && ((w[r][k] & 0xffffffff00000000ull) == want);
                        if (__all(ok)) {
                            float *dst = ring0 + (static_cast<long>((in_next + r) & RM) * kWave + lane) * NPL;
#pragma unroll
                            for (int k = 0; k < NPL; ++k) dst[k] = __uint_as_float(static_cast<unsigned>(w[r][k] & 0xffffffffu));
                            v = r + 1;
                        }
                    }
                }
            }
            if (v > 0) {
                in_next += v;
                lds_publish(&s_done[0], in_next);
                if (p.qg < H) st_relaxed(p.cons + 2 * bound_in, ctag | static_cast<unsigned>(in_next));
                idle = 0;
            } else {
                // nothing new: has the producer moved to the overflow rows?
                if (p.ovf && ovf_from == H) {
                    const unsigned long long f = ld_relaxed(p.cons + 2 * bound_in + 1);
                    if ((f & 0xffffffff00000000ull) == ctag)
                        ovf_from = __builtin_amdgcn_readfirstlane(static_cast<int>(f & 0xffffffffu));
                }
                if (++idle > p.spin_limit) { timed_out = true; break; }
                sleep_a_bit();
            }
        }
        if (timed_out) {
            // Let wave 0 run to the end on NaN carries: every output it
            // and the strips after it compute from here on is NaN.
            for (long k = lane; k < static_cast<long>(p.ring_rows) * kWave * NPL; k += kWave) ring0[k] = quiet_nan();
            lds_publish(&s_done[0], H);
        }
    } else if (wave == p.s_local + 1 && (grp + 1) * p.s_local < p.nstrips) {
        const long bound_out = chain * nb_per_chain + grp;
        unsigned long long *gout = p.gring + bound_out * gstride + lane;
        const float *ringS = lring + static_cast<long>(p.s_local) * ring_floats;
        int out_next = 0, cons_seen = 0;
        bool started = false;  // the consumer has reported progress
        while (out_next < H) {
            const int avail = lds_counter(&s_done[p.s_local]);
            int nb = min(kCourierBatch, avail - out_next);
            if (p.ovf == 2 && ovf_from == H && out_next >= 8) {
                // (test of the overflow rows: every producer moves there
                // after its first 8 rows)
                ovf_from = out_next;
                st_relaxed(p.cons + 2 * bound_out + 1, ctag | static_cast<unsigned>(ovf_from));
            }
            if (p.qg < H && nb > 0 && out_next < ovf_from && out_next + nb > cons_seen + p.qg) {
                const unsigned long long c = ld_relaxed(p.cons + 2 * bound_out);
                if ((c & 0xffffffff00000000ull) == ctag) {
                    cons_seen = static_cast<int>(c & 0xffffffffu);
                    started = true;
                }
                const int room = cons_seen + p.qg - out_next;
                if (room < nb && p.ovf != 0 && !started) {
                    // The ring is full and the consumer may not be able to
                    // start (other work holds the GPU): rather than wait,
                    // write the rows from here on to the overflow rows.
                    ovf_from = out_next + room;
                    st_relaxed(p.cons + 2 * bound_out + 1, ctag | static_cast<unsigned>(ovf_from));
                } else {
                    nb = min(nb, room);
                }
            }
            if (nb > 0) {
#pragma unroll
                for (int r = 0; r < kCourierBatch; ++r) {
                    if (r < nb) {
                        const int row = out_next + r;
                        const float *src_c = ringS + (static_cast<long>(row & RM) * kWave + lane) * NPL;
                        const unsigned long long tagw = static_cast<unsigned long long>(etag | static_cast<unsigned>(row)) << 32;
#pragma unroll
                        for (int k = 0; k < NPL; ++k)
                            st_relaxed(gout + (static_cast<long>(slot_of(row)) * NPL + k) * kWave,
                                       tagw | __float_as_uint(src_c[k]));
                    }
                }
                out_next += nb;
                lds_publish(&s_used[p.s_local], out_next);
                idle = 0;
            } else {
                if (++idle > p.spin_limit) { timed_out = true; break; }
                sleep_a_bit();
            }
        }
        if (timed_out) lds_publish(&s_used[p.s_local], H);  // let the last wave run to the end
    }
    if (timed_out) report_timeout(p);
}

template <typename T, int K, int NPL, int ALIGN, int G, bool COOP, int MODE>
__global__ __launch_bounds__(kWave * max_waves(K, NPL, G, MODE)) void scan2d_fwd_kernel(Params p)
{
    static_assert(K % 4 == 0, "strip width must be a multiple of 4");
    constexpr bool FW = (MODE & kModeFlipW) != 0;
    constexpr bool VF = (MODE & kModeVFirst) != 0;
    constexpr bool ACC = (MODE & kModeAccumulate) != 0;
    constexpr bool STATES = (MODE & kModeStates) != 0;
    constexpr bool BWD = (MODE & kModeBackward) != 0;
    constexpr bool GATE = (MODE & kModeGate) != 0;
    constexpr bool EDGES = (MODE & kModeEdges) != 0;
    constexpr bool RC = (MODE & kModeRowCarry) != 0;
    static_assert(!EDGES || BWD, "courier-free chains: adjoint pass only");
    static_assert(!RC || (!ACC && !GATE), "carried row states: not accumulated or gated");
    static_assert(!GATE || (!ACC && !STATES && !BWD), "gate: plain output only");
    static_assert(!BWD || (!VF && !ACC && !STATES && K == 4 && G == 8), "backward: one layout");
    static_assert(!BWD || !COOP || EDGES, "backward with the shared row ring: courier-free chains only");
    static_assert(!STATES || (!VF && !ACC), "stored states: horizontal-first order");
    using Chunk = typename ChunkOf<T>::type;
    using LT = typename PacketOf<T, COOP>::type;      // element type of the input rows in LDS
    using LChunk = typename ChunkOf<LT>::type;
    constexpr int CPW = kWave / G;                    // channels per wave
    constexpr int KO = K / G > 0 ? K / G : 1;         // finished cells per lane and row
    constexpr int SEG_X = 0, SEG_DT = CPW, SEG_B = 2 * CPW, SEG_C = 2 * CPW + G * NPL;
    constexpr int SEG_DY = SEG_C + G * NPL;           // backward only
    constexpr int SEGROWS = packet_rows<NPL, G, MODE>();  // packet rows of K elements
    constexpr int CPR = K / 4;                        // chunks per packet row
    constexpr int NCHUNK = SEGROWS * CPR;
    constexpr int PASSES = passes_for<NPL, G, MODE>(K);
    constexpr int P = prefetch_rows<NPL, G, MODE, COOP>(K);  // rows per prefetch buffer

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_done[kMaxWaves + 1];   // rows published into LDS ring b
    __shared__ int s_used[kMaxWaves + 1];   // rows consumed from LDS ring b
    __shared__ unsigned int s_ticket;
    __shared__ unsigned int s_epoch;        // this launch's tag epoch, 1 .. kEpochs
    __shared__ int s_last;                  // this workgroup finished last
    __shared__ int s_arrive[kMaxSlots];     // shares written into row-ring slot

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    if (p.use_ticket && threadIdx.x == 0) {
        s_ticket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // (the previous launch's last workgroup advanced it before that
        // launch completed)
        s_epoch = __hip_atomic_load(p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) % kEpochs + 1;
    }
    if (threadIdx.x <= kMaxWaves) {
        s_done[threadIdx.x] = 0;
        s_used[threadIdx.x] = 0;
    }
    if (threadIdx.x < kMaxSlots) {
        s_arrive[threadIdx.x] = 0;
    }
    __syncthreads();

    int wg;
    if (p.use_ticket) {
        wg = static_cast<int>(s_ticket);
    } else if (p.xcd_remap) {
        // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
        // contiguous run of chains so chains sharing a batch entry (and its
        // B, C) share that XCD's L2.
        const int per = p.total_wg / 8;
        wg = (blockIdx.x % 8) * per + blockIdx.x / 8;
    } else {
        wg = blockIdx.x;
    }
    int chain, grp;
    ticket_tile(p, wg, chain, grp);
    const int b = chain / p.n_dblk;
    const int dblk = chain % p.n_dblk;
    const int H = p.H, W = p.W;
    const int RM = p.ring_rows - 1;                   // ring depth is a power of two
    const long ring_floats = static_cast<long>(p.ring_rows) * kWave * NPL;
    // LDS: the input rows (per-wave packets, or the workgroup's row ring), then
    // the carry rings.
    const long in_bytes = COOP ? static_cast<long>(p.coop_slots) * p.s_local * (NCHUNK + 1) * sizeof(LChunk)
                               : static_cast<long>(p.s_local) * 2 * PASSES * kWave * sizeof(LChunk);
    float *lring = reinterpret_cast<float *>(smem + in_bytes);

    if (wave >= p.s_local) {
        courier_wave<NPL>(p, wave, lane, chain, grp, lring, s_done, s_used, s_epoch, ring_floats, RM);
    } else if (grp * p.s_local + wave < p.nstrips) {
        // ---------------- compute wave: one strip
        const int strip = grp * p.s_local + wave;
        const int j0 = strip * K;
        const int valid = min(K, W - j0);
        const int g = lane / CPW;
        const int dl = lane % CPW;
        const int d = dblk * CPW + dl;
        const bool d_ok = d < p.d_inner;
        const long HW = static_cast<long>(H) * W;
        // Rows in scan order: the map's rows top to bottom, or bottom to top.
        // Row t of the scan sits at row0 + t * rs.
        const int rs = p.flip_h ? -W : W;  // |W| <= 65535
        const long row0 = p.flip_h ? HW - W : 0;
        const T *zeros = static_cast<const T *>(p.zeros);
        // Two packet buffers of PASSES x 64 chunks (chunks past NCHUNK are
        // padding, so every lane stores its chunk without a mask): row i is
        // read from buffer i % 2 while row i + 1 is staged into the other.
        LT *packets = reinterpret_cast<LT *>(smem) + static_cast<long>(wave) * 2 * PASSES * kWave * 4;
        // Cooperative loads: the workgroup's nact strips share one ring of
        // rows in LDS. A row of the ring holds every strip's packet (strip s
        // at chunk s * (NCHUNK + 1): the pad chunk spreads the strips over the
        // LDS banks). Each wave loads an equal share of the row, taken in
        // column order (NCHUNK chunks: packet row r of strips 0, 1, ...), so a
        // load instruction reads whole cache lines instead of one 16-byte
        // piece of each of NCHUNK lines, and scatters it into the packets.
        const int nact = min(p.s_local, p.nstrips - grp * p.s_local);  // strips of this workgroup
        const int slot_elems = nact * (NCHUNK + 1) * 4;
        const int XA = p.coop_slots / 2 - 2;  // rows a share is written ahead of its first reader
        LT *ring_rows = reinterpret_cast<LT *>(smem);

        // Chunk sources of this lane: packet row r, chunk q of that row, split
        // into 4/ALIGN sub-loads; a sub-load past the row end reads the zero page.
        // Scanning right to left, cell u of the scan is memory column W-1-u:
        // a chunk of cells u..u+3 is loaded as memory columns W-4-u..W-1-u,
        // in memory order (the packet reads reverse it).
        constexpr int NSUB = 4 / ALIGN;
        const T *src[PASSES][NSUB];
        int wpos[PASSES];  // ring-row chunk this lane's share chunk goes to
#pragma unroll
        for (int pp = 0; pp < PASSES; ++pp) {
            const int c = pp * kWave + lane;
            int r = c / CPR, q = c % CPR, jc = j0;
            wpos[pp] = 0;
            if constexpr (COOP) {
                const int cw = wave * NCHUNK + c;  // chunk of the workgroup row, column order
                r = cw / (nact * CPR);
                const int rem = cw % (nact * CPR);
                jc = (grp * p.s_local + rem / CPR) * K;
                q = rem % CPR;
                // padding lanes (c >= NCHUNK) write the strip's unused pad chunk
                wpos[pp] = (c < NCHUNK) ? (rem / CPR) * (NCHUNK + 1) + r * CPR + q : wave * (NCHUNK + 1) + NCHUNK;
            }
            const T *base = zeros;
            if (c < NCHUNK) {
                if (r < SEG_DT) {
                    const int dd = dblk * CPW + r;
                    if (dd < p.d_inner) base = static_cast<const T *>(p.x) + (static_cast<long>(b) * p.d_inner + dd) * HW;
                } else if (r < SEG_B) {
                    const int dd = dblk * CPW + r - SEG_DT;
                    if (dd < p.d_inner) base = static_cast<const T *>(p.delta) + (static_cast<long>(b) * p.d_inner + dd) * HW;
                } else if (r < SEG_C) {
                    const int n = r - SEG_B;
                    if (n < p.d_state) base = static_cast<const T *>(p.B) + (static_cast<long>(b) * p.d_state + n) * HW;
                } else if (r < SEG_DY) {
                    const int n = r - SEG_C;
                    if (n < p.d_state) base = static_cast<const T *>(p.C) + (static_cast<long>(b) * p.d_state + n) * HW;
                } else {
                    const int dd = dblk * CPW + r - SEG_DY;
                    if (dd < p.d_inner) base = static_cast<const T *>(p.dy) + (static_cast<long>(b) * p.d_inner + dd) * HW;
                }
            }
#pragma unroll
            for (int e = 0; e < NSUB; ++e) {
                // (the stored-state pass counts strips over the map padded to a
                // multiple of 4 columns at the end it scans last: on the left
                // scanning left to right, on the right scanning right to left;
                // columns outside the map read zeros)
                if constexpr (FW) {
                    const int col = (STATES ? W + p.states_pad : W) - jc - 4 * q - 4 + e * ALIGN;
                    src[pp][e] = (col >= 0 && col + ALIGN <= W) ? base + col + row0 : zeros + row0;
                } else {
                    const int col = jc + 4 * q + e * ALIGN - (STATES ? p.states_pad : 0);
                    src[pp][e] = (col >= 0 && col + ALIGN <= W) ? base + col + row0 : zeros + row0;
                }
            }
        }

        float Ap[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int n = g * NPL + k;
            Ap[k] = (n < p.d_state && d_ok) ? p.A[d * p.d_state + n] * kLog2e : 0.0f;
        }
        const float Dd = d_ok ? p.D[d] : 0.0f;
        // Wait for these loads here, once: used inside the row loop they
        // would make the compiler wait for every load in flight (the row
        // prefetches too) at each use, since it cannot tell at the loop head
        // whether they have completed.
#pragma unroll
        for (int k = 0; k < NPL; ++k) asm volatile("" ::"v"(Ap[k]));
        asm volatile("" ::"v"(Dd));
        // Backward: A itself (d delta takes g_a A Abar).
        float At[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) At[k] = 0.0f;
        if constexpr (BWD) {
#pragma unroll
            for (int k = 0; k < NPL; ++k) {
                const int n = g * NPL + k;
                At[k] = (n < p.d_state && d_ok) ? p.A[d * p.d_state + n] : 0.0f;
                asm volatile("" ::"v"(At[k]));
            }
        }
        // Stored-state tiles: the forward writes its strip's tile of each row
        // (whole 1 KB blocks per state slot, every lane, no masks: lanes and
        // cells outside the map hold exact zeros), and first a tile for row
        // -1, the carried state above the map (zeros without one); the
        // backward's strip s and scan row t read the forward's strip
        // nstrips-1-s, row H-1-t (its cells in reverse order), row -1 at
        // t = H; rows past that read the zero page.
        constexpr long TILE = static_cast<long>(NPL) * kWave * 4;   // floats per (chain, strip, row)
        const int fstrip = BWD ? p.nstrips - 1 - strip : strip;     // strip in the forward's numbering
        const long tile0 = (static_cast<long>(chain) * p.nstrips + fstrip) * (H + 1) + 1;  // tile of row 0
        float *hrow = p.states + tile0 * TILE + lane * 4;            // + row * TILE + k * 256
        const float *hlast = p.states + (tile0 + H - 1) * TILE + lane * 4;
        // backward: 8-channel sums of dB, dC for this lane's group, memory row
        // H-1 - t, the strip's 4 cells at padded column 4 * fstrip
        // (rows of 4 * nstrips columns: the map starts at states_pad when the
        // adjoint runs right to left, at 0 when it runs left to right)
        const long pld = 4L * p.nstrips;
        const long pcol = FW ? 4L * fstrip : 4L * strip;
        const long prow0 = p.flip_h ? H - 1 : 0;  // memory row of scan row 0
        const long part0 = dblk * p.part_stride + ((static_cast<long>(b) * p.d_state + g * NPL) * H + prow0) * pld + pcol;
        float *pbrow = p.dBp + part0;
        float *pcrow = p.dCp + part0;
        const float *zeros_f = static_cast<const float *>(p.zeros);
        bool hok[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) hok[k] = d_ok && (g * NPL + k < p.d_state);
        const bool part_lane = (dl == 0);  // stores the 8-channel sums of its state group
        // First of this lane's finished cells (for G = 8 and K = 4 the two
        // lanes of a pair hold the same cell and the odd one does not store).
        const int c_out = (K >= G) ? g * KO : g / 2;
        const bool storer = (K >= G) || (g % 2 == 0);
        // Output cells of this lane; cells outside the map go to the sink.
        // The pointers advance one row per processed row.
        T *ydst[KO];
        long ystep[KO];
#pragma unroll
        for (int c = 0; c < KO; ++c) {
            const bool ok = d_ok && storer && (c_out + c < valid);
            const int u = j0 + c_out + c;  // column in scan order
            ydst[c] = ok ? static_cast<T *>(p.y) + (static_cast<long>(b) * p.d_inner + d) * HW + row0 + (FW ? W - 1 - u : u)
                         : static_cast<T *>(p.sink) + lane * KO + c;
            ystep[c] = ok ? rs : 0;
        }
        T *ybase[KO];  // row 0 of the scan (accumulating calls read y there)
#pragma unroll
        for (int c = 0; c < KO; ++c) ybase[c] = ydst[c];
        // Whole-strip stores: with 4-aligned rows and a full 4-column strip,
        // each channel's cells are gathered into one lane of row 0 and stored
        // as chunks; other strips, and accumulating calls, store cell by cell.
        // (8-column strips store cell by cell at compile time: a second store
        // form under a branch makes the compiler's wait counts after the
        // stores pessimistic, and gathering 8 cells costs more than it saves.)
        const bool vec_store = K == 4 && !ACC && (ALIGN == 4) && (valid == K) && p.vec_store;
        const bool vec_lane = (pair_lane<K, G>(lane) < CPW) && d_ok;
        T *yvec = static_cast<T *>(p.y) + (static_cast<long>(b) * p.d_inner + (vec_lane ? d : 0)) * HW + row0 +
                  (FW ? W - j0 - K : j0) + pair_offset<K, G, FW>(lane);
        // Backward: d delta goes where dx goes, in its own tensor: the same
        // addresses moved by the distance between the two tensors (zero for
        // lanes writing the sink). Offsets keep the stores on global pointers.
        long ddoff[KO], dvoff = 0;
        if constexpr (BWD) {
            const long dist = static_cast<long>(reinterpret_cast<uintptr_t>(p.ddelta) - reinterpret_cast<uintptr_t>(p.y)) /
                              static_cast<long>(sizeof(T));
#pragma unroll
            for (int c = 0; c < KO; ++c) ddoff[c] = (ystep[c] != 0) ? dist : 0;
            dvoff = dist;
        }
        // Gate: z of this lane's output cells, at the same place in its tensor
        // (offset zero for lanes writing the sink, which read it instead).
        long zoff[KO];
        if constexpr (GATE) {
            const long dist = static_cast<long>(reinterpret_cast<uintptr_t>(p.z) - reinterpret_cast<uintptr_t>(p.y)) /
                              static_cast<long>(sizeof(T));
#pragma unroll
            for (int c = 0; c < KO; ++c) zoff[c] = (ystep[c] != 0) ? dist : 0;
        }
        // backward: this lane's parts of dA and dD. Each row's terms are summed
        // in fp32 and the row sums in fp64, so the rounding of these long sums
        // (every cell of the strip) does not grow with the map's height.
        double dAacc[NPL], dDacc = 0.0;
#pragma unroll
        for (int k = 0; k < NPL; ++k) dAacc[k] = 0.0;

        const bool has_left = strip > 0;
        const bool has_right = strip + 1 < p.nstrips;
        const float *ring_in = lring + static_cast<long>(wave) * ring_floats;
        float *ring_out = lring + static_cast<long>(wave + 1) * ring_floats;
        bool timed_out = false;
        // 0, or kSkipWaits once a wait has timed out: the per-row checks
        // compare max(counter, skip) with the row, so later waits are skipped
        // without a separate test of timed_out on the fast path.
        int skip = 0;

        float hv[K][NPL];
#pragma unroll
        for (int c = 0; c < K; ++c)
#pragma unroll
            for (int k = 0; k < NPL; ++k) hv[c][k] = 0.0f;
        // Carried vertical state (a band of rows continuing a scan): the
        // register state of the strip's columns starts from h_init and is
        // written to h_last after the last row.
        // (the stored-state pass counts its strips over the map padded by
        // states_pad columns at the end it scans last: column u of its scan is
        // j0 + c - states_pad)
        auto carry_index = [&](const int c, const int k, long &idx) -> bool {
            const int n = g * NPL + k, u = j0 + c - (STATES ? p.states_pad : 0);
            idx = ((static_cast<long>(b) * p.d_inner + d) * p.d_state + n) * W + (FW ? W - 1 - u : u);
            return d_ok && n < p.d_state && u >= 0 && u < W;
        };
        // Carried horizontal state of scan row t (kModeRowCarry): element
        // [b][d][n][memory row] of hh_init / hh_last.
        auto row_carry_index = [&](const int t, const int k, long &idx) -> bool {
            const int n = g * NPL + k;
            idx = ((static_cast<long>(b) * p.d_inner + d) * p.d_state + n) * H + (p.flip_h ? H - 1 - t : t);
            return d_ok && n < p.d_state && t < H;
        };
        // the chain's first strip reads the rows' carried states, its last
        // strip writes them (with the row's inputs / after the row's chain)
        const bool rc_in = RC && p.hh_init && strip == 0;
        const bool rc_out = RC && p.hh_last && strip + 1 == p.nstrips;
        // (the adjoint pass: h_init is dL/dh_last, the carry its vertical
        // adjoint starts from; h_last receives dL/dh_init, its final carry)
        {
            if (p.h_init) {
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        long idx;
                        if (carry_index(c, k, idx)) hv[c][k] = p.h_init[idx];
                    }
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int k = 0; k < NPL; ++k) asm volatile("" : "+v"(hv[c][k]));  // loaded before the row loop
            }
            if constexpr (STATES) {
                // row -1's tile: the carried state (or zeros)
#pragma unroll
                for (int k = 0; k < NPL; ++k)
                    *reinterpret_cast<float4 *>(hrow - TILE + k * kWave * 4) =
                        make_float4(hv[0][k], hv[1][k], hv[2][k], hv[3][k]);
            }
        }

        // Operands of row t live at row_base(t) + roff(packet row).
        const int slot_mask = p.coop_slots - 1;
        auto row_base = [&](const int t) -> LT * {
            if constexpr (COOP) return ring_rows + static_cast<long>(t & slot_mask) * slot_elems;
            else return packets + (t % 2) * PASSES * kWave * 4;
        };
        auto roff = [&](const int r) { return COOP ? wave * (NCHUNK + 1) * 4 + r * K : r * K; };
        const int off_x = roff(SEG_X + dl), off_dt = roff(SEG_DT + dl), off_dy = roff(SEG_DY + dl);
        int off_b[NPL], off_c[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            off_b[k] = roff(SEG_B + g * NPL + k);
            off_c[k] = roff(SEG_C + g * NPL + k);
        }
        // Polls an LDS counter until it reaches `need` (bounded like every wait).
        // A wait that gave up: later waits are skipped, and the decay
        // exponents become NaN, so that every output this strip computes
        // from here on (and, through its carries, the strips after it) is
        // NaN instead of a plausible wrong value.
        auto give_up = [&]() {
            timed_out = true;
            skip = kSkipWaits;
#pragma unroll
            for (int k = 0; k < NPL; ++k) Ap[k] = quiet_nan();
        };
        auto wait_count = [&](const int *c, const int need) {
            long long spins = 0;
            while (__builtin_amdgcn_readfirstlane(lds_peek(c)) < need) {
                if (++spins > p.spin_limit) {
                    give_up();
                    break;
                }
                if (spins > kSpinPolls) sleep_a_bit();
            }
            signal_fence();
        };

        // x and delta of one row: read one row ahead, they start the row's
        // arithmetic. B, C and the skip input are read when the row starts.
        struct Ops {
            float xv[K], dv[K];
        };
        auto read_ops = [&](const LT *pk, Ops &o) {
            read_packet<K, FW>(pk, off_x, o.xv);
            read_packet<K, FW>(pk, off_dt, o.dv);
        };
        // Stage input for row t and issue the reads of this lane's x and delta
        // of row t (their latency hides behind the current row). Per-wave
        // packets: `cb` is row t's packet, written to buffer t % 2.
        // Cooperative: `cb` is this wave's share of row t + XA, written to the
        // row ring; the slot is free because no strip can be more than XA + 1
        // rows behind another (a strip reads row t only after every strip has
        // written its share of it, XA + 1 rows earlier) and the ring holds
        // more than 2 XA + 2 rows. Row t's arrival count is read before its x
        // and delta; confirm() checks it later, off this row's critical path,
        // and reads them again after waiting if the row was not complete.
        auto stage = [&](const Chunk (&cb)[PASSES], const int t, Ops &o) -> int {
            if constexpr (COOP) {
                const int tw = t + XA;
                LT *slot = row_base(tw);
#pragma unroll
                for (int pp = 0; pp < PASSES; ++pp)
                    reinterpret_cast<LChunk *>(slot)[wpos[pp]] = to_packet_ring(cb[pp]);
                signal_fence();
                if (lane == 0)
                    __hip_atomic_fetch_add(&s_arrive[tw & slot_mask], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                signal_fence();
                const int v = lds_peek(&s_arrive[t & slot_mask]);
                signal_fence();
                read_ops(row_base(t), o);
                return v;
            } else {
                LT *pk = row_base(t);
#pragma unroll
                for (int pp = 0; pp < PASSES; ++pp) reinterpret_cast<LChunk *>(pk)[pp * kWave + lane] = to_packet(cb[pp]);
                read_ops(pk, o);
                return 0;
            }
        };
        auto confirm = [&](const int t, const int seen_count, Ops &o) {
            if constexpr (COOP) {
                const int need = nact * ((t >> p.coop_shift) + 1);
                if (max(__builtin_amdgcn_readfirstlane(seen_count), skip) < need) {
                    wait_count(&s_arrive[t & slot_mask], need);
                    read_ops(row_base(t), o);
                }
            }
        };

        // Rows of the strip, with the code for the strip's neighbours fixed at
        // compile time (LEFT: a strip to the left sends carries; RIGHT: one to
        // the right takes them).
        // Carries between workgroups in the courier-free adjoint pass
        // (kModeEdges: its 256-VGPR waves leave no room for couriers next to
        // 8 strips): the workgroup's first strip reads the global ring
        // itself, its last strip writes it. Every row has its own slot there
        // (no reuse, so no back-pressure).
        const unsigned int etag_c = s_epoch << 16;  // (set when chains span workgroups)
        const long gstride_c = static_cast<long>(p.qg) * NPL * kWave;
        const unsigned long long *gin_c =
            p.gring + (static_cast<long>(chain) * (p.groups - 1) + (grp > 0 ? grp - 1 : 0)) * gstride_c + lane;
        unsigned long long *gout_c = p.gring + (static_cast<long>(chain) * (p.groups - 1) + grp) * gstride_c + lane;

        // LK / RK: 0 no neighbour, 1 a strip of this workgroup (LDS ring),
        // 2 a strip of another workgroup reached by this strip itself.
        auto strip_rows = [&](auto left_tag, auto right_tag) {
            constexpr int LK = decltype(left_tag)::value, RK = decltype(right_tag)::value;
            constexpr bool LEFT = LK == 1, RIGHT = RK == 1;
            constexpr bool LEFT_G = LK == 2, RIGHT_G = RK == 2;
            int room = 0;  // rows this wave may publish, as seen

            // Row i from packet buffer i % 2 and operands `o`; row i+1's
            // packet `nb` is staged (and its x, delta read into `on`) first,
            // so that LDS traffic overlaps this row's arithmetic.
            auto do_row = [&](const int i, const Ops &o, const Chunk (&nb)[PASSES], Ops &on, const T (&yo)[KO],
                              const float4 (&hcur)[NPL], const float4 (&hnext)[NPL], const float (&rcur)[NPL]) {
                const LT *pk = row_base(i);
                float Bv[NPL][K], Cv[NPL][K], xo[KO], dyv[K], dyo[KO];
#pragma unroll
                for (int k = 0; k < NPL; ++k) read_packet<K, FW>(pk, off_b[k], Bv[k]);
                const int next_count = stage(nb, i + 1, on);
                if constexpr (BWD) {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) read_packet<K, FW>(pk, off_c[k], Cv[k]);
                }
                read_packet_scalar<KO, FW>(pk, off_x, c_out, xo);
                if constexpr (BWD) {
                    read_packet<K, FW>(pk, off_dy, dyv);
                    read_packet_scalar<KO, FW>(pk, off_dy, c_out, dyo);
                }

                // ---- left carry of row i: the counter and the ring slot are
                // read together (LDS executes a wave's accesses in order, and
                // the producer writes the slot before the counter), before the
                // carry-independent work below, so their latency overlaps it.
                float hh[NPL];
                int seen = 0;
                unsigned long long gw[NPL];
                if constexpr (LEFT) {
                    seen = lds_peek(&s_done[wave]);
                    signal_fence();
                    const float *src_c = ring_in + (static_cast<long>(i & RM) * kWave + lane) * NPL;
#pragma unroll
                    for (int k = 0; k < NPL; ++k) hh[k] = src_c[k];
                } else if constexpr (RC) {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) hh[k] = rcur[k];  // the row's carried state (or 0)
                } else {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) hh[k] = 0.0f;
                }
                if constexpr (LEFT_G) {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) gw[k] = ld_relaxed(gin_c + (static_cast<long>(i) * NPL + k) * kWave);
                }

                // ---- carry-independent work: decay factors and inputs of the row
                float av[K][NPL], bx[K][NPL];
#pragma unroll
                for (int c = 0; c < K; ++c) {
                    const float dx = o.dv[c] * o.xv[c];
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        av[c][k] = __builtin_amdgcn_exp2f(o.dv[c] * Ap[k]);
                        bx[c][k] = dx * Bv[k][c];
                    }
                }
                // Column recurrence first (vertical-first order): it needs no
                // carry, so it joins the carry-independent work, and the row
                // recurrence below runs over its results.
                if constexpr (VF) {
#pragma unroll
                    for (int c = 0; c < K; ++c)
#pragma unroll
                        for (int k = 0; k < NPL; ++k) bx[c][k] = hv[c][k] = __builtin_fmaf(av[c][k], hv[c][k], bx[c][k]);
                }
                // Backward: the adjoint of the vertical scan runs first and
                // needs no carry: g_h = dy C + (Abar g_h) of the row below,
                // kept pre-multiplied in hv. The carried adjoint of the row
                // scan then adds Abar g_hh of the cell to the right.
                float gh[K][NPL];
                if constexpr (BWD) {
#pragma unroll
                    for (int c = 0; c < K; ++c)
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            gh[c][k] = __builtin_fmaf(dyv[c], Cv[k][c], hv[c][k]);
                            hv[c][k] = av[c][k] * gh[c][k];
                            asm volatile("" : "+v"(gh[c][k]), "+v"(hv[c][k]));
                        }
                }
                // Pin that work here, ahead of the wait below: left to itself
                // the compiler sinks it past the wait, onto the carry's
                // critical path.
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int k = 0; k < NPL; ++k) asm volatile("" : "+v"(av[c][k]), "+v"(bx[c][k]));

                // room in the right ring for row i (rarely short; checked here,
                // off the carry's critical path)
                if constexpr (RIGHT) {
                    if (i >= max(room, skip)) {
                        room = wait_counter_above(&s_used[wave + 1], i - p.ring_rows, p.spin_limit, timed_out) +
                               p.ring_rows;
                        if (timed_out) give_up();
                    }
                }

                if constexpr (LEFT) {
                    if (max(__builtin_amdgcn_readfirstlane(seen), skip) <= i) {
                        // Not published yet: poll. Each poll reads the counter
                        // and then the slot, back to back, so the poll that sees
                        // row i published has already fetched its carry (one
                        // LDS round trip per poll). Short waits spin; long ones
                        // sleep between polls.
                        const float *src_c = ring_in + (static_cast<long>(i & RM) * kWave + lane) * NPL;
                        long long spins = 0;
                        while (true) {
                            const int v = lds_peek(&s_done[wave]);
                            signal_fence();
                            float t[NPL];
#pragma unroll
                            for (int k = 0; k < NPL; ++k) t[k] = src_c[k];
                            // issue the slot read with the counter read (left
                            // alone, the compiler reads the slot only after the
                            // check: a second round trip on the carry's path)
#pragma unroll
                            for (int k = 0; k < NPL; ++k) asm volatile("" : "+v"(t[k]));
                            if (__builtin_amdgcn_readfirstlane(v) > i) {
#pragma unroll
                                for (int k = 0; k < NPL; ++k) hh[k] = t[k];
                                break;
                            }
                            if (++spins > p.spin_limit) {
                                give_up();
#pragma unroll
                                for (int k = 0; k < NPL; ++k) hh[k] = quiet_nan();
                                break;
                            }
                            if (spins > kSpinPolls) sleep_a_bit();
                        }
                    }
                }

                if constexpr (LEFT_G) {
                    // the tagged words of row i from the left workgroup's
                    // last strip; polled again until every lane has them
                    const unsigned long long want = static_cast<unsigned long long>(etag_c | static_cast<unsigned>(i)) << 32;
                    long long spins = 0;
                    while (!timed_out) {
                        bool ok = true;
#pragma unroll
                        for (int k = 0; k < NPL; ++k) ok = ok && ((gw[k] & 0xffffffff00000000ull) == want);
                        if (__all(ok)) break;
                        if (++spins > p.spin_limit) {
                            give_up();
                            break;
                        }
                        if (spins > kSpinPolls) sleep_a_bit();
#pragma unroll
                        for (int k = 0; k < NPL; ++k) gw[k] = ld_relaxed(gin_c + (static_cast<long>(i) * NPL + k) * kWave);
                    }
#pragma unroll
                    for (int k = 0; k < NPL; ++k)
                        hh[k] = timed_out ? quiet_nan() : __uint_as_float(static_cast<unsigned>(gw[k] & 0xffffffffu));
                }

                // ---- horizontal recurrence along the row, then hand the carry on
                float hc[K][NPL];
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        if constexpr (BWD) {
                            // g_hh = g_h + carry; carry' = Abar g_hh = Abar g_h + Abar carry
                            hc[c][k] = gh[c][k] + hh[k];
                            hh[k] = __builtin_fmaf(av[c][k], hh[k], hv[c][k]);
                        } else {
                            hh[k] = __builtin_fmaf(av[c][k], hh[k], bx[c][k]);
                            hc[c][k] = hh[k];
                        }
                    }
                if constexpr (RIGHT) {
                    float *dst = ring_out + (static_cast<long>(i & RM) * kWave + lane) * NPL;
#pragma unroll
                    for (int k = 0; k < NPL; ++k) dst[k] = hh[k];
                    signal_fence();
                    lds_poke(&s_done[wave + 1], i + 1);
                    // keep the vertical step below from being scheduled ahead
                    // of the publish: it would sit on the carry's path
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (RIGHT_G) {
                    const unsigned long long tagw = static_cast<unsigned long long>(etag_c | static_cast<unsigned>(i)) << 32;
#pragma unroll
                    for (int k = 0; k < NPL; ++k)
                        st_relaxed(gout_c + (static_cast<long>(i) * NPL + k) * kWave, tagw | __float_as_uint(hh[k]));
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (LEFT) lds_poke(&s_used[wave], i + 1);
                if constexpr (RC && !RIGHT && !RIGHT_G) {
                    if (rc_out && !timed_out) {
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            long idx;
                            if (row_carry_index(i, k, idx)) p.hh_last[idx] = hh[k];
                        }
                    }
                }
                // C of the forward's row: read once the carry is handed on
                // (needed only for the output sum; read with B, it held 16
                // more registers across the carry wait and spilled)
                if constexpr (!BWD) {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) read_packet<K, FW>(pk, off_c[k], Cv[k]);
                }

                if constexpr (BWD) {
                    // ---- local derivatives. With hh = h - Abar h(row above)
                    // and u = Bx, the decay's adjoint times Abar is
                    // g_a Abar = g_hh (hh - u) + g_h (h - hh).
                    float ddp[K], dxp[K], dBv[NPL][K], dCv[NPL][K], dAr[NPL], dDr = 0.0f;
#pragma unroll
                    for (int k = 0; k < NPL; ++k) dAr[k] = 0.0f;
#pragma unroll
                    for (int c = 0; c < K; ++c) {
                        float sdd = 0.0f, sdx = 0.0f;
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            const float hcu = chunk_elem(hcur[k], 3 - c);   // chunks hold cells in memory order
                            const float hab = chunk_elem(hnext[k], 3 - c);
                            const float hhv = __builtin_fmaf(-av[c][k], hab, hcu);
                            const float gaa = hc[c][k] * (hhv - bx[c][k]) + gh[c][k] * (hcu - hhv);
                            const float gb = hc[c][k] * Bv[k][c];
                            sdd = __builtin_fmaf(gaa, At[k], sdd);
                            sdd = __builtin_fmaf(gb, o.xv[c], sdd);
                            sdx = __builtin_fmaf(gb, o.dv[c], sdx);
                            dBv[k][c] = hc[c][k] * (o.dv[c] * o.xv[c]);
                            dCv[k][c] = dyv[c] * hcu;
                            dAr[k] = __builtin_fmaf(gaa, o.dv[c], dAr[k]);
                        }
                        ddp[c] = sdd;
                        dxp[c] = sdx;
                        dDr = __builtin_fmaf(dyv[c], o.xv[c], dDr);
                    }
#pragma unroll
                    for (int k = 0; k < NPL; ++k) dAacc[k] += static_cast<double>(dAr[k]);
                    dDacc += static_cast<double>(dDr);
                    // sums over the state groups; dx takes the skip term's dy D
                    float ddo[KO], dxo[KO];
                    reduce_groups<K, G>(ddp, ddo, g);
                    reduce_groups<K, G>(dxp, dxo, g);
#pragma unroll
                    for (int c = 0; c < KO; ++c) dxo[c] = __builtin_fmaf(Dd, dyo[c], dxo[c]);
                    if (vec_store) {
                        store_row<K, G, FW>(yvec, dxo, vec_lane);
                        store_row<K, G, FW>(yvec + dvoff, ddo, vec_lane);
                        yvec += rs;
                    } else {
#pragma unroll
                        for (int c = 0; c < KO; ++c) {
                            store_elem(ydst[c], dxo[c]);
                            store_elem(ydst[c] + ddoff[c], ddo[c]);
                            ydst[c] += ystep[c];
                        }
                    }
                    // dB and dC: sums over the wave's 8 channels of a state
                    // group (the sum over channel blocks comes later), cells
                    // in memory order
                    const long prow = static_cast<long>(i) * (p.flip_h ? -pld : pld);
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        float sb[K], sc[K];
#pragma unroll
                        for (int c = 0; c < K; ++c) {
                            sb[c] = sum8(dBv[k][c]);
                            sc[c] = sum8(dCv[k][c]);
                        }
                        if (part_lane && hok[k]) {
                            const long off = static_cast<long>(k) * H * pld + prow;
                            if constexpr (FW) {
                                *reinterpret_cast<float4 *>(pbrow + off) = make_float4(sb[3], sb[2], sb[1], sb[0]);
                                *reinterpret_cast<float4 *>(pcrow + off) = make_float4(sc[3], sc[2], sc[1], sc[0]);
                            } else {
                                *reinterpret_cast<float4 *>(pbrow + off) = make_float4(sb[0], sb[1], sb[2], sb[3]);
                                *reinterpret_cast<float4 *>(pcrow + off) = make_float4(sc[0], sc[1], sc[2], sc[3]);
                            }
                        }
                    }
                } else {
                    // ---- vertical recurrence (unless it ran first) and the sum
                    // over this lane's states
                    float part[K];
#pragma unroll
                    for (int c = 0; c < K; ++c) {
                        float acc = 0.0f;
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            if constexpr (VF) {
                                acc = __builtin_fmaf(Cv[k][c], hc[c][k], acc);
                            } else {
                                hv[c][k] = __builtin_fmaf(av[c][k], hv[c][k], hc[c][k]);
                                acc = __builtin_fmaf(Cv[k][c], hv[c][k], acc);
                            }
                        }
                        part[c] = acc;
                    }

                    if constexpr (STATES) {
                        // the wave's tile of this row
#pragma unroll
                        for (int k = 0; k < NPL; ++k)
                            *reinterpret_cast<float4 *>(hrow + static_cast<long>(i) * TILE + k * kWave * 4) =
                                make_float4(hv[0][k], hv[1][k], hv[2][k], hv[3][k]);
                    } else {
                        // ---- sum over the state groups, skip term, store
                        float out[KO];
                        reduce_groups<K, G>(part, out, g);
#pragma unroll
                        for (int c = 0; c < KO; ++c) out[c] += Dd * xo[c];
                        if constexpr (GATE) {
                            // times SiLU(z) = z / (1 + e^-z); z of this row was read with its inputs
#pragma unroll
                            for (int c = 0; c < KO; ++c) {
                                const float zf = elem_value(yo[c]);
                                out[c] *= zf * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zf * kLog2e));
                            }
                        }
                        if constexpr (ACC) {
                            // y of this row was read with the row's inputs
#pragma unroll
                            for (int c = 0; c < KO; ++c) {
                                store_elem(ydst[c], elem_value(yo[c]) + out[c]);
                                ydst[c] += ystep[c];
                            }
                        } else if (vec_store) {
                            store_row<K, G, FW>(yvec, out, vec_lane);
                            yvec += rs;
                        } else {
#pragma unroll
                            for (int c = 0; c < KO; ++c) {
                                store_elem(ydst[c], out[c]);
                                ydst[c] += ystep[c];
                            }
                        }
                    }
                }
                confirm(i + 1, next_count, on);
            };

            // Two prefetch buffers of P rows: while one buffer's rows are
            // computed, the other's loads are in flight. Operands alternate
            // between two register sets, row by row. Full blocks of 2P rows run
            // without per-row guards (a guard would make the compiler copy the
            // register-resident state at every row); the last, partial block
            // runs guarded. Rows past the map's end are never computed; their
            // loads read the last row again.
            // Accumulating into y: each row's y cells are read with its inputs
            // (yoA / yoB, loaded with bufA / bufB), added to the result and
            // written back by the same lane, so no other wave touches them.
            // Gated: yoA / yoB hold z of those cells instead.
            // Backward: each row's stored states (hbA / hbB), read likewise;
            // a row needs its own and the next scan row's.
            Chunk bufA[P][PASSES], bufB[P][PASSES];
            T yoA[P][KO], yoB[P][KO];
            float4 hbA[P][NPL], hbB[P][NPL];
            float rcA[P][NPL], rcB[P][NPL];  // carried row states (kModeRowCarry)
            Ops ops[2];
            auto load_rows = [&](Chunk (&buf)[P][PASSES], T (&yo)[P][KO], float4 (&hb)[P][NPL], float (&rc)[P][NPL],
                                 const int first) {
#pragma unroll
                for (int s = 0; s < P; ++s) {
#pragma unroll
                    for (int pp = 0; pp < PASSES; ++pp)
                        buf[s][pp] = load_chunk<ALIGN>(src[pp], static_cast<long>(min(first + s + (COOP ? XA : 0), H - 1)) * rs);
                    if constexpr (ACC) {
#pragma unroll
                        for (int c = 0; c < KO; ++c) yo[s][c] = ybase[c][static_cast<long>(min(first + s, H - 1)) * ystep[c]];
                    }
                    if constexpr (GATE) {
#pragma unroll
                        for (int c = 0; c < KO; ++c)
                            yo[s][c] = ybase[c][zoff[c] + static_cast<long>(min(first + s, H - 1)) * ystep[c]];
                    }
                    if constexpr (BWD) {
                        const int t = first + s;
#pragma unroll
                        for (int k = 0; k < NPL; ++k)
                            hb[s][k] = *reinterpret_cast<const float4 *>(
                                t <= H ? hlast - static_cast<long>(t) * TILE + k * kWave * 4 : zeros_f);
                    }
                    if constexpr (RC) {
                        // the row's carried horizontal state (0 unless the chain's first strip)
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            long idx;
                            const bool ok = rc_in && row_carry_index(first + s, k, idx);
                            rc[s][k] = ok ? p.hh_init[idx] : 0.0f;
                        }
                    }
                }
            };
            if constexpr (COOP) {
                // shares of rows 0 .. XA-1; row XA's comes from bufA[0] below
                for (int t = 0; t < XA; ++t) {
                    Chunk c0[PASSES];
#pragma unroll
                    for (int pp = 0; pp < PASSES; ++pp)
                        c0[pp] = load_chunk<ALIGN>(src[pp], static_cast<long>(min(t, H - 1)) * rs);
                    LT *slot = row_base(t);
#pragma unroll
                    for (int pp = 0; pp < PASSES; ++pp)
                        reinterpret_cast<LChunk *>(slot)[wpos[pp]] = to_packet_ring(c0[pp]);
                    signal_fence();
                    if (lane == 0)
                        __hip_atomic_fetch_add(&s_arrive[t & slot_mask], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    signal_fence();
                }
            }
            load_rows(bufA, yoA, hbA, rcA, 0);
            load_rows(bufB, yoB, hbB, rcB, P);
            confirm(0, stage(bufA[0], 0, ops[0]), ops[0]);
            int i0 = 0;
            for (; i0 + 2 * P <= H; i0 += 2 * P) {
#pragma unroll
                for (int s = 0; s < P; ++s)
                    do_row(i0 + s, ops[s % 2], s + 1 < P ? bufA[s + 1] : bufB[0], ops[(s + 1) % 2], yoA[s], hbA[s],
                           s + 1 < P ? hbA[s + 1] : hbB[0], rcA[s]);
                load_rows(bufA, yoA, hbA, rcA, i0 + 2 * P);
#pragma unroll
                for (int s = 0; s < P; ++s)
                    do_row(i0 + P + s, ops[(P + s) % 2], s + 1 < P ? bufB[s + 1] : bufA[0], ops[(P + s + 1) % 2], yoB[s],
                           hbB[s], s + 1 < P ? hbB[s + 1] : hbA[0], rcB[s]);
                load_rows(bufB, yoB, hbB, rcB, i0 + 3 * P);
            }
            if (i0 < H) {
#pragma unroll
                for (int s = 0; s < P; ++s)
                    if (i0 + s < H)
                        do_row(i0 + s, ops[s % 2], s + 1 < P ? bufA[s + 1] : bufB[0], ops[(s + 1) % 2], yoA[s], hbA[s],
                               s + 1 < P ? hbA[s + 1] : hbB[0], rcA[s]);
                // (the last slot here is never a map row: i0 + 2P > H)
#pragma unroll
                for (int s = 0; s < P; ++s)
                    if (i0 + P + s < H)
                        do_row(i0 + P + s, ops[(P + s) % 2], s + 1 < P ? bufB[s + 1] : bufB[s], ops[(P + s + 1) % 2], yoB[s],
                               hbB[s], s + 1 < P ? hbB[s + 1] : hbB[s], rcB[s]);
            }
        };
        using N0 = std::integral_constant<int, 0>;
        using N1 = std::integral_constant<int, 1>;
        using N2 = std::integral_constant<int, 2>;
        if constexpr (EDGES) {
            const int lk = !has_left ? 0 : (wave == 0 && grp > 0 ? 2 : 1);
            const int rk = !has_right ? 0 : (wave == nact - 1 ? 2 : 1);
            auto with_right = [&](auto lt) {
                if (rk == 0) strip_rows(lt, N0{});
                else if (rk == 1) strip_rows(lt, N1{});
                else strip_rows(lt, N2{});
            };
            if (lk == 0) with_right(N0{});
            else if (lk == 1) with_right(N1{});
            else with_right(N2{});
        } else if (has_left) {
            if (has_right) strip_rows(N1{}, N1{});
            else strip_rows(N1{}, N0{});
        } else {
            if (has_right) strip_rows(N0{}, N1{});
            else strip_rows(N0{}, N0{});
        }
        if constexpr (!STATES) {
            if (p.h_last && !timed_out) {
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        long idx;
                        if (carry_index(c, k, idx)) p.h_last[idx] = hv[c][k];
                    }
            }
        }
        if constexpr (BWD) {
            // this strip's parts of dA (every state of the lane) and dD (one
            // lane per channel)
#pragma unroll
            for (int k = 0; k < NPL; ++k)
                if (hok[k]) (void)unsafeAtomicAdd(p.dA + d * p.d_state + g * NPL + k, static_cast<float>(dAacc[k]));
            if (d_ok && g == 0) (void)unsafeAtomicAdd(p.dD + d, static_cast<float>(dDacc));
        }
        if (timed_out) report_timeout(p);
    }

    if (p.use_ticket) finish_launch(p, s_epoch, s_last);
}

// ---------------------------------------------------------------- host side

// Buffers of the two backward passes (the stored states and the partial sums
// of dB and dC live in a library workspace; the rest are the caller's).
struct BwdArgs {
    float *states;
    int pad;
    const void *dy;
    void *ddelta;
    float *dBp, *dCp, *dA, *dD;
    long part_stride;
};

struct Plan {
    int G, K, npl, nstrips, s_local, groups, n_dblk, n_chains, total_wg, ring_rows, qg;
    int ovf;         // overflow rows after the bounded ring (Params::ovf)
    int tblk;        // chains per block of tickets (0: n_chains)
    int coop_slots;  // rows of the shared row ring with cooperative loads, 0 = per-wave packets
    int mode;        // kMode* bits
    int flip_h;      // rows bottom to top
    const BwdArgs *bw;  // stored-state and backward passes
    const void *z;   // gate input (kModeGate)
    const float *h_init;  // carried vertical states in / out (may be null)
    float *h_last;
    const float *hh_init;  // carried horizontal states in / out (kModeRowCarry; may be null)
    float *hh_last;
    // Workspace of fixed size to launch in (null: the per-(device, stream)
    // workspace, grown as needed)
    const struct WsEntry *fixed_ws;
};

int env_int(const char *name, int dflt);

constexpr size_t kHeadBytes = 256;   // ticket, done, err, epoch
constexpr size_t kSinkBytes = 4096;  // >= 64 lanes x 8 cells x 4 bytes

// The scan's workspace: head words (ticket, done, err, epoch), the sink, the
// consumer words cons[], the global carry ring and the zero page.
struct WsEntry {
    unsigned int *head = nullptr;          // ticket, done, err, epoch, then the sink and cons[]
    unsigned long long *gring = nullptr;
    void *zeros = nullptr;
    unsigned int *herr = nullptr;          // host-mapped timeout flag (null if unavailable)
    size_t gring_bytes = 0, zero_bytes = 0, cons_count = 0;
};

int hip_fail(hipError_t e);
extern long long g_spin_limit;
int get_ws(int dev, void *stream, size_t gring_bytes, size_t zero_bytes, size_t cons_count, WsEntry **out);
int device_cus(int dev);

// Sizes of the scan workspace a plan needs (the global ring, the zero page,
// the consumer words).
struct WsNeed {
    size_t gring_bytes, zero_bytes, cons_count;
};
// The plan's launch, given its workspace (shared by the allocating entry
// points and the one that runs in a static device array).
template <typename T, int K, int NPL, int ALIGN, int G, bool COOP, int MODE>
int launch_plan(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int batch,
                int d_inner, int d_state, int H, int W, const Plan &pl, const WsEntry &e, void *stream);

// Two courier waves join the strips when a chain spans workgroups (not in
// the courier-free adjoint pass, whose boundary strips reach the global ring
// themselves).
inline int block_threads(const Plan &pl)
{
    return kWave * (pl.s_local + ((pl.groups > 1 && !(pl.mode & kModeEdges)) ? 2 : 0));
}

template <typename T, int K, int NPL, int G, int MODE>
size_t lds_bytes(const Plan &pl)
{
    // the shared row ring keeps the input type; per-wave packets are fp32
    const size_t chunk_bytes = pl.coop_slots > 0 ? sizeof(typename ChunkOf<T>::type) : sizeof(float4);
    const size_t nchunk = static_cast<size_t>(packet_rows<NPL, G, MODE>()) * (K / 4);
    const size_t chunks = pl.coop_slots > 0 ? pl.coop_slots * (nchunk + 1)                                  // ring rows
                                            : 2 * static_cast<size_t>(passes_for<NPL, G, MODE>(K)) * kWave;  // 2 padded packets
    return static_cast<size_t>(pl.s_local) * chunks * chunk_bytes +
           static_cast<size_t>(pl.s_local + 1) * pl.ring_rows * kWave * NPL * sizeof(float);
}

// Global ring between the workgroups of a chain. Where the whole grid fits
// the GPU at once, a bounded ring of qg = 32 rows (SSM2D_RING) with
// back-pressure, followed by a row per map row of overflow: a producer whose
// ring is full waits for its consumer only once the consumer has reported
// progress; before that (the consumer may not have started: other work holds
// the GPU) it moves on to the overflow rows and tells the consumer from which
// row. So no producer waits on a consumer that has not started, and a launch
// drains whatever else holds the GPU. Tickets go strip group by strip group
// (every chain's first tile starts at once). A workspace of fixed size that
// cannot hold the overflow rows takes the ring alone; its producers may then
// wait on consumers that have not started, and tickets are dealt in blocks of
// one chain, so only the started workgroups of the last chain begun (groups -
// 1 at most) can wait so. SSM2D_OVERFLOW=0 leaves the overflow rows out (then
// tblk keeps two launches' waiting workgroups under the GPU's slots, in
// multiples of 8 so that a chain's workgroups share an XCD), =2 makes every
// producer move to them after its first 8 rows (a test of that path). Grids
// larger than the GPU, or SSM2D_RING < 8 or >= H, take a slot a row.
inline void bound_ring(Plan &pl, long resident, int H, int npl)
{
    pl.qg = H;
    pl.tblk = pl.n_chains;
    pl.ovf = 0;
    if (pl.groups <= 1) return;
    const int qg = env_int("SSM2D_RING", 32);
    if (resident < pl.total_wg || qg < 8 || qg >= H) return;
    int ovf = env_int("SSM2D_OVERFLOW", 1);
    ovf = ovf < 0 ? 0 : (ovf > 2 ? 2 : ovf);
    bool one_chain = false;
    if (pl.fixed_ws) {
        const size_t row_bytes = static_cast<size_t>(pl.n_chains) * (pl.groups - 1) * npl * kWave * sizeof(unsigned long long);
        if (ovf && row_bytes * (qg + H) > pl.fixed_ws->gring_bytes) {
            ovf = 0;
            one_chain = true;
        }
    }
    pl.qg = qg;
    pl.ovf = ovf;
    const int forced = env_int("SSM2D_TICKET_BLOCK", 0);
    long tb = pl.n_chains;
    if (forced > 0) {
        tb = forced;
    } else if (!ovf) {
        tb = one_chain ? 1 : (resident - 1) / (2L * (pl.groups - 1));
        if (tb >= 8) tb -= tb % 8;
    }
    pl.tblk = static_cast<int>(tb < 1 ? 1 : (tb < pl.n_chains ? tb : pl.n_chains));
}

template <typename T, int K, int NPL, int ALIGN, int G, bool COOP, int MODE>
void choose_ring(Plan &pl, int dev, int H)
{
    pl.qg = H;
    pl.tblk = pl.n_chains;
    pl.ovf = 0;
    if (pl.groups <= 1 || (pl.mode & kModeEdges)) return;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan2d_fwd_kernel<T, K, NPL, ALIGN, G, COOP, MODE>, block_threads(pl),
                                                     lds_bytes<T, K, NPL, G, MODE>(pl)) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    bound_ring(pl, static_cast<long>(per_cu) * device_cus(dev), H, NPL);
}

template <int NPL>
WsNeed ws_need(const Plan &pl, int d_inner, int H, int W)
{
    const long n_bound = static_cast<long>(pl.n_chains) * (pl.groups - 1);
    WsNeed n{};
    n.gring_bytes = static_cast<size_t>(n_bound) * (pl.qg + (pl.ovf ? H : 0)) * NPL * kWave * sizeof(unsigned long long);
    // zero page: whole rows of any input type, and a zero D (no skip term)
    n.zero_bytes = static_cast<size_t>(H) * W * 4 + 64;
    if (n.zero_bytes < static_cast<size_t>(d_inner) * 4 + 64) n.zero_bytes = static_cast<size_t>(d_inner) * 4 + 64;
    n.cons_count = static_cast<size_t>(n_bound > 0 ? 2 * n_bound : 1);
    return n;
}

template <typename T, int K, int NPL, int ALIGN, int G, bool COOP, int MODE>
int run(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int batch,
        int d_inner, int d_state, int H, int W, Plan pl, int dev, void *stream)
{
    if (!COOP) pl.coop_slots = 0;
    choose_ring<T, K, NPL, ALIGN, G, COOP, MODE>(pl, dev, H);
    const WsNeed need = ws_need<NPL>(pl, d_inner, H, W);
    if (pl.fixed_ws) {
        // a workspace of fixed size (no allocation): the plan must fit it
        if (need.gring_bytes > pl.fixed_ws->gring_bytes || need.zero_bytes > pl.fixed_ws->zero_bytes ||
            need.cons_count > pl.fixed_ws->cons_count)
            return SSM2D_ERR_TOO_LARGE;
        return launch_plan<T, K, NPL, ALIGN, G, COOP, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl,
                                                            *pl.fixed_ws, stream);
    }
    WsEntry *e = nullptr;
    const int st = get_ws(dev, stream, need.gring_bytes, need.zero_bytes, need.cons_count, &e);
    if (st != SSM2D_OK) return st;
    return launch_plan<T, K, NPL, ALIGN, G, COOP, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, *e,
                                                        stream);
}

// Kernel parameters of a plan and its workspace (shared by the kernels).
inline Params make_params(const void *x, const void *delta, const float *A, const void *B, const void *C,
                          const float *D, void *y, int batch, int d_inner, int d_state, int H, int W, const Plan &pl,
                          const WsEntry &ws)
{
    const WsEntry *e = &ws;
    Params prm{};
    prm.x = x; prm.delta = delta;
    prm.B = d_state ? static_cast<const void *>(B) : e->zeros;
    prm.C = d_state ? static_cast<const void *>(C) : e->zeros;
    prm.A = A; prm.D = D ? D : static_cast<const float *>(e->zeros); prm.y = y; prm.zeros = e->zeros;
    prm.ticket = e->head; prm.done = e->head + 1; prm.err = e->head + 2; prm.epoch = e->head + 3;
    prm.herr = e->herr;
    prm.sink = reinterpret_cast<char *>(e->head) + kHeadBytes;
    prm.cons = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(e->head) + kHeadBytes + kSinkBytes);
    prm.gring = e->gring;
    prm.gring_words = static_cast<long>(e->gring_bytes / sizeof(unsigned long long));
    prm.cons_words = static_cast<long>(e->cons_count);
    prm.batch = batch; prm.d_inner = d_inner; prm.d_state = d_state; prm.H = H; prm.W = W;
    prm.nstrips = pl.nstrips; prm.s_local = pl.s_local; prm.groups = pl.groups; prm.n_dblk = pl.n_dblk;
    prm.n_chains = pl.n_chains; prm.total_wg = pl.total_wg; prm.ring_rows = pl.ring_rows; prm.qg = pl.qg;
    prm.ovf = pl.qg < H ? pl.ovf : 0;
    prm.use_ticket = pl.groups > 1 ? 1 : 0;
    prm.tblk = pl.tblk > 0 && pl.tblk < pl.n_chains ? pl.tblk : pl.n_chains;
    prm.xcd_remap = (pl.groups == 1 && pl.total_wg % 8 == 0 && env_int("SSM2D_XCD_REMAP", 1)) ? 1 : 0;
    // Gathered stores pay for 4-column strips (one row swap, two cells a lane).
    // Gathering the eight cells of an 8-column strip costs more VALU work than
    // the scattered stores, which the memory system coalesces anyway.
    prm.vec_store = env_int("SSM2D_VECSTORE", pl.K == 4 ? 1 : 0);
    prm.flip_h = pl.flip_h;
    if (pl.bw) {
        prm.states = pl.bw->states;
        prm.states_pad = pl.bw->pad;
        prm.dy = pl.bw->dy;
        prm.ddelta = pl.bw->ddelta;
        prm.dBp = pl.bw->dBp;
        prm.dCp = pl.bw->dCp;
        prm.dA = pl.bw->dA;
        prm.dD = pl.bw->dD;
        prm.part_stride = pl.bw->part_stride;
    }
    prm.z = pl.z;
    prm.h_init = pl.h_init;
    prm.h_last = pl.h_last;
    prm.hh_init = pl.hh_init;
    prm.hh_last = pl.hh_last;
    prm.coop_slots = pl.coop_slots > 0 ? pl.coop_slots : 2;
    prm.coop_shift = 0;
    while ((1 << prm.coop_shift) < prm.coop_slots) ++prm.coop_shift;
    prm.spin_limit = g_spin_limit > 0 ? g_spin_limit : (1ll << 22);
    return prm;
}

template <typename T, int K, int NPL, int ALIGN, int G, bool COOP, int MODE>
int launch_plan(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int batch,
                int d_inner, int d_state, int H, int W, const Plan &pl, const WsEntry &ws, void *stream)
{
    const Params prm = make_params(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, ws);
    const size_t lds = lds_bytes<T, K, NPL, G, MODE>(pl);
    scan2d_fwd_kernel<T, K, NPL, ALIGN, G, COOP, MODE><<<dim3(pl.total_wg), dim3(block_threads(pl)), lds,
                                   static_cast<hipStream_t>(stream)>>>(prm);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? SSM2D_OK : hip_fail(err);
}

// Launch of a right-to-left, vertical-first, accumulating, gated, stored-state
// or adjoint scan: 8 state groups; 4-column strips (per-wave packets, align 4
// or 1, or the shared row ring) or, for the forward modes, 8-column strips
// (align 4); and for the forward modes 4 state groups with 4 states a lane
// (4-column strips, per-wave packets, align 4 or 2). Instantiated by one
// translation unit per (input type, mode).
template <typename T, int MODE>
int dispatch_mode(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
                  int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream, int align)
{
    if ((MODE & (kModeStates | kModeBackward)) && !pl.bw) return SSM2D_ERR_UNSUPPORTED;
    if ((MODE & kModeGate) && !pl.z) return SSM2D_ERR_UNSUPPORTED;
    if (pl.G == 4) {
        // 4 state groups (16 channels a wave, 4 states a lane) for the forward
        // modes: 4-column strips, per-wave packets, rows of an even length
        if constexpr (!(MODE & (kModeStates | kModeBackward))) {
            if (pl.K == 4 && pl.npl == 4 && pl.coop_slots == 0) {
                if (align == 4) return run<T, 4, 4, 4, 4, false, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
                if (align == 2) return run<T, 4, 4, 2, 4, false, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
            }
        }
        return SSM2D_ERR_UNSUPPORTED;
    }
    if (pl.G != 8 || (pl.K != 4 && pl.K != 8)) return SSM2D_ERR_UNSUPPORTED;
    if (pl.coop_slots != 0) {
        // the shared row ring (tall maps cut into several workgroups per chain;
        // for the adjoint pass, its courier-free kernels)
        if constexpr (!(MODE & kModeBackward) || (MODE & kModeEdges)) {
            if (align != 4) return SSM2D_ERR_UNSUPPORTED;
#define SSM2D_MODE_COOP(NN) \
    if (pl.npl == NN) return run<T, 4, NN, 4, 8, true, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
            SSM2D_MODE_COOP(1) SSM2D_MODE_COOP(2) SSM2D_MODE_COOP(4)
            if constexpr (!(MODE & kModeBackward)) {  // the backward keeps at most 4 states per lane
                SSM2D_MODE_COOP(8)
            }
#undef SSM2D_MODE_COOP
        }
        return SSM2D_ERR_UNSUPPORTED;
    }
    if (pl.K == 8) {
        // 8-column strips: rows of a multiple of 4 columns, at most 4 states a lane
        if constexpr (!(MODE & (kModeStates | kModeBackward))) {
            if (align != 4) return SSM2D_ERR_UNSUPPORTED;
#define SSM2D_MODE_WIDE(NN) \
    if (pl.npl == NN) return run<T, 8, NN, 4, 8, false, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
            SSM2D_MODE_WIDE(1) SSM2D_MODE_WIDE(2) SSM2D_MODE_WIDE(4)
#undef SSM2D_MODE_WIDE
        }
        return SSM2D_ERR_UNSUPPORTED;
    }
    const int al = align == 4 ? 4 : 1;
#define SSM2D_MODE_CASE(NN, AL)    \
    if (pl.npl == NN && al == AL) \
        return run<T, 4, NN, AL, 8, false, MODE>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
    SSM2D_MODE_CASE(1, 4) SSM2D_MODE_CASE(2, 4) SSM2D_MODE_CASE(4, 4)
    SSM2D_MODE_CASE(1, 1) SSM2D_MODE_CASE(2, 1) SSM2D_MODE_CASE(4, 1)
    if constexpr (!(MODE & kModeBackward)) {  // the backward keeps at most 4 states per lane (d_state <= 32)
        SSM2D_MODE_CASE(8, 4) SSM2D_MODE_CASE(8, 1)
    }
#undef SSM2D_MODE_CASE
    return SSM2D_ERR_UNSUPPORTED;
}

// Launch for a plan: one translation unit per (input type, state-group
// layout) instantiates the kernels, so they compile in parallel.
#define SSM2D_DISPATCH_DECL(TT, NAME)                                                                       \
    int NAME(const TT *x, const TT *delta, const float *A, const TT *B, const TT *C, const float *D, TT *y, \
             int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream, int align);
SSM2D_DISPATCH_DECL(float, dispatch_g4)
SSM2D_DISPATCH_DECL(float, dispatch_g8)
SSM2D_DISPATCH_DECL(uint16_t, dispatch_g4)
SSM2D_DISPATCH_DECL(uint16_t, dispatch_g8)
// The plain forward of tall maps, two rows per step (scan2d_fast.h), or
// kNoFastPath when the plan is not of its layout.
constexpr int kNoFastPath = -1;
SSM2D_DISPATCH_DECL(float, dispatch_fast)
SSM2D_DISPATCH_DECL(uint16_t, dispatch_fast)
// The plain forward of narrow maps, one wave a whole row (scan2d_narrow.h):
// rows of at most 16 columns, at most 16 states.
int dispatch_narrow(const float *x, const float *delta, const float *A, const float *B, const float *C,
                    const float *D, float *y, int batch, int d_inner, int d_state, int H, int W, int flip_h,
                    void *stream);
int dispatch_narrow(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C,
                    const float *D, uint16_t *y, int batch, int d_inner, int d_state, int H, int W, int flip_h,
                    void *stream);
// Whether dispatch_fast takes a plan (for inputs of type T; rows of a
// multiple of `align` columns).
template <typename T>
bool fast_path_taken(const Plan &pl, int align);
template <>
bool fast_path_taken<float>(const Plan &pl, int align);
template <>
bool fast_path_taken<uint16_t>(const Plan &pl, int align);
// The other modes (8 state groups; 4-column strips with per-wave packets or
// the shared row ring, align 2 served by the align-1 kernels; 8-column strips
// for the forward modes on rows of a multiple of 4 columns), one translation
// unit per (type, mode).
#define SSM2D_MODE_DECLS(TT)                         \
    SSM2D_DISPATCH_DECL(TT, dispatch_flipw)          \
    SSM2D_DISPATCH_DECL(TT, dispatch_vfirst)         \
    SSM2D_DISPATCH_DECL(TT, dispatch_flipw_vfirst)   \
    SSM2D_DISPATCH_DECL(TT, dispatch_acc)            \
    SSM2D_DISPATCH_DECL(TT, dispatch_flipw_acc)      \
    SSM2D_DISPATCH_DECL(TT, dispatch_vfirst_acc)     \
    SSM2D_DISPATCH_DECL(TT, dispatch_flipw_vfirst_acc) \
    SSM2D_DISPATCH_DECL(TT, dispatch_states)           \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd)              \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_edges)        \
    SSM2D_DISPATCH_DECL(TT, dispatch_states_flipw)     \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_ltr)          \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_ltr_edges)    \
    SSM2D_DISPATCH_DECL(TT, dispatch_gate)             \
    SSM2D_DISPATCH_DECL(TT, dispatch_gate_vfirst)      \
    SSM2D_DISPATCH_DECL(TT, dispatch_gate_flipw)       \
    SSM2D_DISPATCH_DECL(TT, dispatch_gate_flipw_vfirst) \
    SSM2D_DISPATCH_DECL(TT, dispatch_rowc)             \
    SSM2D_DISPATCH_DECL(TT, dispatch_rowc_flipw)       \
    SSM2D_DISPATCH_DECL(TT, dispatch_rowc_vfirst)      \
    SSM2D_DISPATCH_DECL(TT, dispatch_rowc_flipw_vfirst) \
    SSM2D_DISPATCH_DECL(TT, dispatch_states_rowc)       \
    SSM2D_DISPATCH_DECL(TT, dispatch_states_flipw_rowc) \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_rowc)          \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_edges_rowc)    \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_ltr_rowc)      \
    SSM2D_DISPATCH_DECL(TT, dispatch_bwd_ltr_edges_rowc)
SSM2D_MODE_DECLS(float)
SSM2D_MODE_DECLS(uint16_t)
#undef SSM2D_MODE_DECLS
#undef SSM2D_DISPATCH_DECL

}  // namespace ssm2d_impl

// libssm2d: 2DMamba 2D selective scan (forward) for MI355X / gfx950.
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
//     producer is resident or done. A bounded global ring with back-pressure
//     is used only when the whole grid is co-resident; otherwise every row has
//     its own slot and nothing ever waits on a consumer.
//   * The sum over n: each lane holds K partial sums over its NPL states; two
//     permlane swaps (32- and 16-lane) transpose-reduce them across the 4 state
//     groups, leaving each lane with K/4 finished cells.
// No MFMA: the scan is not a dense contraction.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "ssm2d.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxWaves = 10;                  // waves per workgroup (strips + couriers)
// Waves per workgroup: 10 (up to 3 per SIMD) when a lane's register state is
// small (8 state groups, K * NPL <= 16), else 8, which leaves a wave 256 VGPRs.
constexpr int max_waves(int K, int NPL, int G) { return (G == 8 && K * NPL <= 16) ? 10 : 8; }
constexpr int kCourierBatch = 4;               // rows a courier requests per poll
constexpr int kSpinPolls = 64;                  // polls of an LDS counter before sleeping between polls
constexpr float kLog2e = 1.4426950408889634f;

struct Params {
    const void *x, *delta, *B, *C;
    const float *A, *D;
    void *y;
    const void *zeros;                 // zero page, >= H*W*4 bytes
    void *sink;                        // write target of masked-off output lanes
    unsigned int *ticket, *done, *err;
    unsigned long long *gring;         // [n_bound][qg][NPL][64] tagged carries
    unsigned long long *cons;          // [n_bound] consumer progress: epoch<<32 | rows
    int batch, d_inner, d_state, H, W;
    int nstrips, s_local, groups, n_dblk, n_chains, total_wg;
    int ring_rows;                     // LDS ring depth between waves
    int qg;                            // global ring depth (== H: no reuse)
    int use_ticket;                    // chains span workgroups
    int xcd_remap;                     // spread chains over XCDs in contiguous blocks
    int vec_store;                     // gather each channel's cells and store whole chunks
    unsigned int epoch;
    long long spin_limit;
};

template <typename T> struct ChunkOf;
template <> struct ChunkOf<float> { using type = float4; };      // 4 fp32
template <> struct ChunkOf<uint16_t> { using type = uint2; };    // 4 bf16

__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

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
template <int N>
__device__ __forceinline__ void read_packet(const float *pk, int off, float (&v)[N])
{
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        float4 t = *reinterpret_cast<const float4 *>(pk + off + 4 * q);
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
}
template <int N>
__device__ __forceinline__ void read_packet(const uint16_t *pk, int off, float (&v)[N])
{
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        uint2 t = *reinterpret_cast<const uint2 *>(pk + off + 4 * q);
        v[4 * q] = bf16_lo(t.x); v[4 * q + 1] = bf16_hi(t.x);
        v[4 * q + 2] = bf16_lo(t.y); v[4 * q + 3] = bf16_hi(t.y);
    }
}
// N elements one by one.
template <int N>
__device__ __forceinline__ void read_packet_scalar(const float *pk, int off, float (&v)[N])
{
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = pk[off + c];
}
template <int N>
__device__ __forceinline__ void read_packet_scalar(const uint16_t *pk, int off, float (&v)[N])
{
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = __uint_as_float(static_cast<unsigned>(pk[off + c]) << 16);
}

__device__ __forceinline__ void store_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ unsigned bf16_bits(float v);
__device__ __forceinline__ void store_elem(uint16_t *p, float v) { *p = static_cast<uint16_t>(bf16_bits(v)); }

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
template <int K, int G>
__device__ __forceinline__ void store_row(float *p, const float (&v)[(K / G) > 0 ? K / G : 1], bool storer)
{
    constexpr int KO = (K / G) > 0 ? K / G : 1;
    float cells[K];
    if constexpr (G == 4) {
        // row r = group r holds cells [r*KO, (r+1)*KO)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < KO; ++c) cells[r * KO + c] = from_row(v[c], r);
    } else if constexpr (K == 4) {
        // row r holds cell r (twice: groups 2r and 2r+1)
#pragma unroll
        for (int r = 0; r < 4; ++r) cells[r] = from_row(v[0], r);
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
#pragma unroll
        for (int q = 0; q < K / 4; ++q)
            *reinterpret_cast<float4 *>(p + 4 * q) = make_float4(cells[4 * q], cells[4 * q + 1], cells[4 * q + 2], cells[4 * q + 3]);
    }
}
template <int K, int G>
__device__ __forceinline__ void store_row(uint16_t *p, const float (&v)[(K / G) > 0 ? K / G : 1], bool storer)
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
    } else if constexpr (K == 4) {
        // one cell per lane: rows 0..3 hold cells 0..3
        const unsigned h = bf16_bits(v[0]);
        unsigned t[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = row_word(h, r);
        words[0] = t[0] | (t[1] << 16);
        words[1] = t[2] | (t[3] << 16);
    } else {
        static_assert(G == 8 && K == 8, "bf16 row store layouts");
        const unsigned h = bf16_bits(v[0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const unsigned t = row_word(h, r);
            words[r] = t | (__float_as_uint(row_ror8(__uint_as_float(t))) << 16);
        }
    }
    if (storer) {
        if constexpr (K == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(words[0], words[1]);
        else *reinterpret_cast<uint4 *>(p) = make_uint4(words[0], words[1], words[2], words[3]);
    }
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
template <int NPL, int G> constexpr int packet_rows() { return 2 * (kWave / G) + 2 * G * NPL; }
template <int NPL, int G> constexpr int passes_for(int K) { return (packet_rows<NPL, G>() * (K / 4) + kWave - 1) / kWave; }
template <int NPL, int G> constexpr int prefetch_rows(int K) { return passes_for<NPL, G>(K) == 1 ? 4 : 2; }

template <typename T, int K, int NPL, int ALIGN, int G>
__global__ __launch_bounds__(kWave * max_waves(K, NPL, G)) void scan2d_fwd_kernel(Params p)
{
    static_assert(K % 4 == 0, "strip width must be a multiple of 4");
    using Chunk = typename ChunkOf<T>::type;
    constexpr int CPW = kWave / G;                    // channels per wave
    constexpr int KO = K / G > 0 ? K / G : 1;         // finished cells per lane and row
    constexpr int SEG_X = 0, SEG_DT = CPW, SEG_B = 2 * CPW, SEG_C = 2 * CPW + G * NPL;
    constexpr int SEGROWS = packet_rows<NPL, G>();    // packet rows of K elements
    constexpr int CPR = K / 4;                        // chunks per packet row
    constexpr int NCHUNK = SEGROWS * CPR;
    constexpr int PASSES = passes_for<NPL, G>(K);
    constexpr int P = prefetch_rows<NPL, G>(K);       // rows per prefetch buffer

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_done[kMaxWaves + 1];   // rows published into LDS ring b
    __shared__ int s_used[kMaxWaves + 1];   // rows consumed from LDS ring b
    __shared__ unsigned int s_ticket;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    if (p.use_ticket && threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x <= kMaxWaves) {
        s_done[threadIdx.x] = 0;
        s_used[threadIdx.x] = 0;
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
    const int chain = wg % p.n_chains;
    const int grp = wg / p.n_chains;
    const int b = chain / p.n_dblk;
    const int dblk = chain % p.n_dblk;
    const int H = p.H, W = p.W;
    const int RM = p.ring_rows - 1;                   // ring depth is a power of two
    const long ring_floats = static_cast<long>(p.ring_rows) * kWave * NPL;
    float *lring = reinterpret_cast<float *>(smem + static_cast<long>(p.s_local) * 2 * PASSES * kWave * sizeof(Chunk));

    if (wave >= p.s_local) {
        // ---------------- couriers between the global ring and the LDS rings.
        // Wave s_local brings the left workgroup's carries into LDS ring 0;
        // wave s_local + 1 sends LDS ring s_local to the right workgroup. They
        // are separate waves so that waiting for loads never also waits for
        // the write-through of stores (one counter tracks both).
        const long nb_per_chain = p.groups - 1;
        const long gstride = static_cast<long>(p.qg) * NPL * kWave;
        const unsigned int etag = p.epoch << 16;
        const unsigned long long ctag = static_cast<unsigned long long>(p.epoch) << 32;
        long idle = 0;
        bool timed_out = false;
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
                                w[r][k] = ld_relaxed(gin + (static_cast<long>((in_next + r) % p.qg) * NPL + k) * kWave);
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
                    if (p.qg < H) st_relaxed(p.cons + bound_in, ctag | static_cast<unsigned>(in_next));
                    idle = 0;
                } else {
                    if (++idle > p.spin_limit) { timed_out = true; break; }
                    sleep_a_bit();
                }
            }
            if (timed_out) lds_publish(&s_done[0], H);  // let wave 0 run to the end
        } else if (wave == p.s_local + 1 && (grp + 1) * p.s_local < p.nstrips) {
            const long bound_out = chain * nb_per_chain + grp;
            unsigned long long *gout = p.gring + bound_out * gstride + lane;
            const float *ringS = lring + static_cast<long>(p.s_local) * ring_floats;
            int out_next = 0, cons_seen = 0;
            while (out_next < H) {
                const int avail = lds_counter(&s_done[p.s_local]);
                int nb = min(kCourierBatch, avail - out_next);
                if (p.qg < H && nb > 0 && out_next + nb > cons_seen + p.qg) {
                    const unsigned long long c = ld_relaxed(p.cons + bound_out);
                    if ((c & 0xffffffff00000000ull) == ctag) cons_seen = static_cast<int>(c & 0xffffffffu);
                    nb = min(nb, cons_seen + p.qg - out_next);
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
                                st_relaxed(gout + (static_cast<long>(row % p.qg) * NPL + k) * kWave,
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
        if (timed_out) atomicOr(p.err, 1u);
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
        const T *zeros = static_cast<const T *>(p.zeros);
        // Two packet buffers of PASSES x 64 chunks (chunks past NCHUNK are
        // padding, so every lane stores its chunk without a mask): row i is
        // read from buffer i % 2 while row i + 1 is staged into the other.
        T *packets = reinterpret_cast<T *>(smem) + static_cast<long>(wave) * 2 * PASSES * kWave * 4;

        // Chunk sources of this lane: packet row r, chunk q of that row, split
        // into 4/ALIGN sub-loads; a sub-load past the row end reads the zero page.
        constexpr int NSUB = 4 / ALIGN;
        const T *src[PASSES][NSUB];
#pragma unroll
        for (int pp = 0; pp < PASSES; ++pp) {
            const int c = pp * kWave + lane;
            const int r = c / CPR, q = c % CPR;
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
                } else {
                    const int n = r - SEG_C;
                    if (n < p.d_state) base = static_cast<const T *>(p.C) + (static_cast<long>(b) * p.d_state + n) * HW;
                }
            }
#pragma unroll
            for (int e = 0; e < NSUB; ++e) {
                const int col = j0 + 4 * q + e * ALIGN;
                src[pp][e] = ((col + ALIGN <= W) ? base : zeros) + col;
            }
        }

        float Ap[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int n = g * NPL + k;
            Ap[k] = (n < p.d_state && d_ok) ? p.A[d * p.d_state + n] * kLog2e : 0.0f;
        }
        const float Dd = d_ok ? p.D[d] : 0.0f;
        // First of this lane's finished cells (for G = 8 and K = 4 the two
        // lanes of a pair hold the same cell and the odd one does not store).
        const int c_out = (K >= G) ? g * KO : g / 2;
        const bool storer = (K >= G) || (g % 2 == 0);
        // Output cells of this lane; cells outside the map go to the sink.
        // The pointers advance one row per processed row.
        T *ydst[KO];
        int ystep[KO];
#pragma unroll
        for (int c = 0; c < KO; ++c) {
            const bool ok = d_ok && storer && (c_out + c < valid);
            ydst[c] = ok ? static_cast<T *>(p.y) + (static_cast<long>(b) * p.d_inner + d) * HW + j0 + c_out + c
                         : static_cast<T *>(p.sink) + lane * KO + c;
            ystep[c] = ok ? W : 0;
        }
        // Whole-strip stores: with 4-aligned rows and a full strip, each
        // channel's cells are gathered into one lane of row 0 and stored as
        // chunks; other strips store cell by cell.
        const bool vec_store = (ALIGN == 4) && (valid == K) && p.vec_store;
        const bool vec_lane = (lane < CPW) && d_ok;
        T *yvec = static_cast<T *>(p.y) + (static_cast<long>(b) * p.d_inner + (vec_lane ? d : 0)) * HW + j0;

        const bool has_left = strip > 0;
        const bool has_right = strip + 1 < p.nstrips;
        const float *ring_in = lring + static_cast<long>(wave) * ring_floats;
        float *ring_out = lring + static_cast<long>(wave + 1) * ring_floats;
        bool timed_out = false;

        float hv[K][NPL];
#pragma unroll
        for (int c = 0; c < K; ++c)
#pragma unroll
            for (int k = 0; k < NPL; ++k) hv[c][k] = 0.0f;

        // x and delta of one row: read one row ahead, they start the row's
        // arithmetic. B, C and the skip input are read when the row starts.
        struct Ops {
            float xv[K], dv[K];
        };
        // Stage a row's packet in LDS buffer `buf` and issue the reads of this
        // lane's x and delta (their latency hides behind the current row).
        auto stage = [&](const Chunk (&cb)[PASSES], const int buf, Ops &o) {
            T *pk = packets + buf * PASSES * kWave * 4;
#pragma unroll
            for (int pp = 0; pp < PASSES; ++pp) reinterpret_cast<Chunk *>(pk)[pp * kWave + lane] = cb[pp];
            read_packet<K>(pk, (SEG_X + dl) * K, o.xv);
            read_packet<K>(pk, (SEG_DT + dl) * K, o.dv);
        };

        // Rows of the strip, with the code for the strip's neighbours fixed at
        // compile time (LEFT: a strip to the left sends carries; RIGHT: one to
        // the right takes them).
        auto strip_rows = [&](auto left_tag, auto right_tag) {
            constexpr bool LEFT = decltype(left_tag)::value;
            constexpr bool RIGHT = decltype(right_tag)::value;
            int room = 0;  // rows this wave may publish, as seen

            // Row i from packet buffer i % 2 and operands `o`; row i+1's
            // packet `nb` is staged (and its x, delta read into `on`) first,
            // so that LDS traffic overlaps this row's arithmetic.
            auto do_row = [&](const int i, const Ops &o, const Chunk (&nb)[PASSES], Ops &on) {
                const T *pk = packets + (i % 2) * PASSES * kWave * 4;
                float Bv[NPL][K], Cv[NPL][K], xo[KO];
#pragma unroll
                for (int k = 0; k < NPL; ++k) read_packet<K>(pk, (SEG_B + g * NPL + k) * K, Bv[k]);
                stage(nb, (i + 1) % 2, on);
#pragma unroll
                for (int k = 0; k < NPL; ++k) read_packet<K>(pk, (SEG_C + g * NPL + k) * K, Cv[k]);
                read_packet_scalar<KO>(pk, (SEG_X + dl) * K + c_out, xo);

                // ---- left carry of row i: the counter and the ring slot are
                // read together (LDS executes a wave's accesses in order, and
                // the producer writes the slot before the counter), before the
                // carry-independent work below, so their latency overlaps it.
                float hh[NPL];
                int seen = 0;
                if constexpr (LEFT) {
                    seen = lds_peek(&s_done[wave]);
                    signal_fence();
                    const float *src_c = ring_in + (static_cast<long>(i & RM) * kWave + lane) * NPL;
#pragma unroll
                    for (int k = 0; k < NPL; ++k) hh[k] = src_c[k];
                } else {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) hh[k] = 0.0f;
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
                    if (i >= room && !timed_out)
                        room = wait_counter_above(&s_used[wave + 1], i - p.ring_rows, p.spin_limit, timed_out) +
                               p.ring_rows;
                }

                if constexpr (LEFT) {
                    if (__builtin_amdgcn_readfirstlane(seen) <= i && !timed_out) {
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
                            if (__builtin_amdgcn_readfirstlane(v) > i) {
#pragma unroll
                                for (int k = 0; k < NPL; ++k) hh[k] = t[k];
                                break;
                            }
                            if (++spins > p.spin_limit) {
                                timed_out = true;
                                break;
                            }
                            if (spins > kSpinPolls) sleep_a_bit();
                        }
                    }
                }

                // ---- horizontal recurrence along the row, then hand the carry on
                float hc[K][NPL];
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        hh[k] = __builtin_fmaf(av[c][k], hh[k], bx[c][k]);
                        hc[c][k] = hh[k];
                    }
                if constexpr (RIGHT) {
                    float *dst = ring_out + (static_cast<long>(i & RM) * kWave + lane) * NPL;
#pragma unroll
                    for (int k = 0; k < NPL; ++k) dst[k] = hh[k];
                    signal_fence();
                    lds_poke(&s_done[wave + 1], i + 1);
                }
                if constexpr (LEFT) lds_poke(&s_used[wave], i + 1);

                // ---- vertical recurrence and the sum over this lane's states
                float part[K];
#pragma unroll
                for (int c = 0; c < K; ++c) {
                    float acc = 0.0f;
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        hv[c][k] = __builtin_fmaf(av[c][k], hv[c][k], hc[c][k]);
                        acc = __builtin_fmaf(Cv[k][c], hv[c][k], acc);
                    }
                    part[c] = acc;
                }

                // ---- sum over the state groups, skip term, store
                float out[KO];
                reduce_groups<K, G>(part, out, g);
#pragma unroll
                for (int c = 0; c < KO; ++c) out[c] += Dd * xo[c];
                if (vec_store) {
                    store_row<K, G>(yvec, out, vec_lane);
                    yvec += W;
                } else {
#pragma unroll
                    for (int c = 0; c < KO; ++c) {
                        store_elem(ydst[c], out[c]);
                        ydst[c] += ystep[c];
                    }
                }
            };

            // Two prefetch buffers of P rows: while one buffer's rows are
            // computed, the other's loads are in flight. Operands alternate
            // between two register sets, row by row. Full blocks of 2P rows run
            // without per-row guards (a guard would make the compiler copy the
            // register-resident state at every row); the last, partial block
            // runs guarded. Rows past the map's end are never computed; their
            // loads read the last row again.
            Chunk bufA[P][PASSES], bufB[P][PASSES];
            Ops ops[2];
            auto load_rows = [&](Chunk (&buf)[P][PASSES], const int first) {
#pragma unroll
                for (int s = 0; s < P; ++s)
#pragma unroll
                    for (int pp = 0; pp < PASSES; ++pp)
                        buf[s][pp] = load_chunk<ALIGN>(src[pp], static_cast<long>(min(first + s, H - 1)) * W);
            };
            load_rows(bufA, 0);
            load_rows(bufB, P);
            stage(bufA[0], 0, ops[0]);
            int i0 = 0;
            for (; i0 + 2 * P <= H; i0 += 2 * P) {
#pragma unroll
                for (int s = 0; s < P; ++s)
                    do_row(i0 + s, ops[s % 2], s + 1 < P ? bufA[s + 1] : bufB[0], ops[(s + 1) % 2]);
                load_rows(bufA, i0 + 2 * P);
#pragma unroll
                for (int s = 0; s < P; ++s)
                    do_row(i0 + P + s, ops[(P + s) % 2], s + 1 < P ? bufB[s + 1] : bufA[0], ops[(P + s + 1) % 2]);
                load_rows(bufB, i0 + 3 * P);
            }
            if (i0 < H) {
#pragma unroll
                for (int s = 0; s < P; ++s)
                    if (i0 + s < H) do_row(i0 + s, ops[s % 2], s + 1 < P ? bufA[s + 1] : bufB[0], ops[(s + 1) % 2]);
#pragma unroll
                for (int s = 0; s < P; ++s)
                    if (i0 + P + s < H)
                        do_row(i0 + P + s, ops[(P + s) % 2], s + 1 < P ? bufB[s + 1] : bufB[s], ops[(P + s + 1) % 2]);
            }
        };
        if (has_left) {
            if (has_right) strip_rows(std::true_type{}, std::true_type{});
            else strip_rows(std::true_type{}, std::false_type{});
        } else {
            if (has_right) strip_rows(std::false_type{}, std::true_type{});
            else strip_rows(std::false_type{}, std::false_type{});
        }
        if (timed_out) atomicOr(p.err, 1u);
    }

    if (p.use_ticket) {
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned int old = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == static_cast<unsigned int>(p.total_wg)) {
                __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ---------------------------------------------------------------- host side

struct Plan {
    int G, K, npl, nstrips, s_local, groups, n_dblk, n_chains, total_wg, ring_rows, qg;
};

int env_int(const char *name, int dflt)
{
    const char *s = std::getenv(name);
    return (s && *s) ? std::atoi(s) : dflt;
}

Plan make_plan(int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W)
{
    Plan pl{};
    const int want_wg = 256;  // enough workgroups to cover the chip's CUs
    // Layout: 4 state groups per wave (16 channels) unless the map has more
    // than 4 states and too few (batch, channel-block) chains to give every CU
    // a chain of its own. Then 8 groups (8 channels, half the states per lane)
    // double the chains, halve the workgroups each chain spans, and put two
    // compute waves on each SIMD. Above 32 states a lane of a 4-group layout
    // would hold 16 states, more than its registers: 8 groups then too.
    const int64_t chains4 = batch * ((d_inner + 15) / 16);
    int G = (d_state > 32 || (d_state > 4 && chains4 < want_wg)) ? 8 : 4;
    const int genv = env_int("SSM2D_GROUPS", 0);
    if (genv == 8 || (genv == 4 && d_state <= 32)) G = genv;
    pl.G = G;
    int npl = 1;
    while (npl * G < d_state) npl *= 2;
    pl.npl = npl;
    const int cpw = kWave / G;
    pl.n_dblk = static_cast<int>((d_inner + cpw - 1) / cpw);
    pl.n_chains = static_cast<int>(batch) * pl.n_dblk;
    // With that many chains, keep each chain in one workgroup (its carries
    // stay in LDS), widening the strips to 8 columns if that makes the chain
    // fit. Otherwise chains are cut into groups of s_local strips linked by two
    // courier waves (so at most maxw - 2 strips per workgroup).
    const bool wide_ok = npl <= 4 && W % 4 == 0;
    pl.K = 4;
    if (pl.n_chains >= want_wg && (W + 3) / 4 > max_waves(4, npl, G) && wide_ok &&
        (W + 7) / 8 <= max_waves(8, npl, G))
        pl.K = 8;
    const int kenv = env_int("SSM2D_STRIP", 0);
    if (kenv == 4 || (kenv == 8 && wide_ok)) pl.K = kenv;
    const int maxw = max_waves(pl.K, npl, G);
    pl.nstrips = static_cast<int>((W + pl.K - 1) / pl.K);
    int s_local;
    if (pl.n_chains >= want_wg && pl.nstrips <= maxw) {
        s_local = pl.nstrips;
    } else {
        const int groups = (pl.n_chains >= want_wg) ? 1 : (want_wg + pl.n_chains - 1) / pl.n_chains;
        s_local = (pl.nstrips + groups - 1) / groups;
        if (s_local < 4) s_local = 4;
    }
    s_local = env_int("SSM2D_WAVES", s_local);
    if (s_local < 1) s_local = 1;
    if (s_local > pl.nstrips) s_local = pl.nstrips;
    if (s_local > maxw) s_local = maxw;
    if (s_local < pl.nstrips && s_local > maxw - 2) s_local = maxw - 2;  // room for 2 couriers
    pl.s_local = s_local;
    pl.groups = (pl.nstrips + s_local - 1) / s_local;
    pl.total_wg = pl.n_chains * pl.groups;
    // LDS ring depth: a power of two, at least 2 (and at least a courier
    // batch), with all rings of a workgroup within ~48 KB.
    const long row_bytes = static_cast<long>(kWave) * npl * 4;
    const long budget = 48 * 1024;
    int R = 8;
    while (R > 2 && (s_local + 1) * R * row_bytes > budget) R /= 2;
    pl.ring_rows = R;
    pl.qg = static_cast<int>(H);
    return pl;
}

constexpr size_t kHeadBytes = 256;   // ticket, done, err
constexpr size_t kSinkBytes = 4096;  // >= 64 lanes x 8 cells x 4 bytes

struct WsEntry {
    unsigned int *head = nullptr;          // ticket, done, err, then cons[]
    unsigned long long *gring = nullptr;
    void *zeros = nullptr;
    size_t gring_bytes = 0, zero_bytes = 0, cons_count = 0;
    unsigned int epoch = 0;
};

std::mutex g_mutex;
std::atomic<int> g_last_hip_error{hipSuccess};

int hip_fail(hipError_t e)
{
    g_last_hip_error.store(static_cast<int>(e));
    return SSM2D_ERR_HIP;
}

#define SSM2D_HIP_TRY(call)                               \
    do {                                                  \
        const hipError_t e_ = (call);                     \
        if (e_ != hipSuccess) return hip_fail(e_);        \
    } while (0)
std::map<std::pair<int, void *>, WsEntry> g_ws;
long long g_spin_limit = 0;

void free_ws(WsEntry &e)
{
    if (e.head) (void)hipFree(e.head);
    if (e.gring) (void)hipFree(e.gring);
    if (e.zeros) (void)hipFree(e.zeros);
    e = WsEntry{};
}

// Workspace for (device, stream), grown when needed. Growth waits for the
// stream so that no in-flight kernel still uses the old buffers. Fresh
// buffers are zeroed; tags are never zero, so no stale word matches.
int get_ws(int dev, void *stream, size_t gring_bytes, size_t zero_bytes, size_t cons_count, WsEntry **out)
{
    WsEntry &e = g_ws[{dev, stream}];
    if (e.head && gring_bytes <= e.gring_bytes && zero_bytes <= e.zero_bytes && cons_count <= e.cons_count) {
        *out = &e;
        return SSM2D_OK;
    }
    unsigned int epoch = e.epoch;
    if (e.head) {
        SSM2D_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
        free_ws(e);
    }
    size_t gb = gring_bytes < 256 ? 256 : gring_bytes;
    size_t zb = zero_bytes < 256 ? 256 : zero_bytes;
    size_t cc = cons_count < 1 ? 1 : cons_count;
    size_t head = kHeadBytes + kSinkBytes + cc * sizeof(unsigned long long);
    void *h = nullptr, *g = nullptr, *z = nullptr;
    if (hipMalloc(&h, head) != hipSuccess || hipMalloc(&g, gb) != hipSuccess || hipMalloc(&z, zb) != hipSuccess) {
        if (h) (void)hipFree(h);
        if (g) (void)hipFree(g);
        (void)hipGetLastError();
        return SSM2D_ERR_NOMEM;
    }
    SSM2D_HIP_TRY(hipMemset(h, 0, head));
    SSM2D_HIP_TRY(hipMemset(g, 0, gb));
    SSM2D_HIP_TRY(hipMemset(z, 0, zb));
    e.head = static_cast<unsigned int *>(h);
    e.gring = static_cast<unsigned long long *>(g);
    e.zeros = z;
    e.gring_bytes = gb;
    e.zero_bytes = zb;
    e.cons_count = cc;
    e.epoch = epoch;
    *out = &e;
    return SSM2D_OK;
}

int device_cus(int dev)
{
    static std::map<int, int> cache;
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cache[dev] = n;
    return n;
}

int block_threads(const Plan &pl) { return kWave * (pl.s_local + (pl.groups > 1 ? 2 : 0)); }

template <typename T, int K, int NPL, int G>
size_t lds_bytes(const Plan &pl)
{
    using Chunk = typename ChunkOf<T>::type;
    const size_t chunks = 2 * static_cast<size_t>(passes_for<NPL, G>(K)) * kWave;  // per wave: 2 padded buffers
    return static_cast<size_t>(pl.s_local) * chunks * sizeof(Chunk) +
           static_cast<size_t>(pl.s_local + 1) * pl.ring_rows * kWave * NPL * sizeof(float);
}

// Global ring depth: bounded (with back-pressure) only if the whole grid is
// co-resident, so that a producer never waits on a consumer that cannot run.
template <typename T, int K, int NPL, int ALIGN, int G>
int choose_qg(const Plan &pl, int dev, int H)
{
    if (pl.groups <= 1) return H;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan2d_fwd_kernel<T, K, NPL, ALIGN, G>, block_threads(pl),
                                                     lds_bytes<T, K, NPL, G>(pl)) != hipSuccess) {
        (void)hipGetLastError();
        return H;
    }
    const long resident = static_cast<long>(per_cu) * device_cus(dev);
    const int qg = env_int("SSM2D_RING", 32);
    if (resident >= pl.total_wg && qg >= 8 && qg < H) return qg;
    return H;
}

template <typename T, int K, int NPL, int ALIGN, int G>
int run(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int batch,
        int d_inner, int d_state, int H, int W, Plan pl, int dev, void *stream)
{
    pl.qg = choose_qg<T, K, NPL, ALIGN, G>(pl, dev, H);
    const long n_bound = static_cast<long>(pl.n_chains) * (pl.groups - 1);
    const size_t gring_bytes = static_cast<size_t>(n_bound) * pl.qg * NPL * kWave * sizeof(unsigned long long);
    const size_t zero_bytes = static_cast<size_t>(H) * W * 4 + 64;
    WsEntry *e = nullptr;
    int st = get_ws(dev, stream, gring_bytes, zero_bytes, static_cast<size_t>(n_bound > 0 ? n_bound : 1), &e);
    if (st != SSM2D_OK) return st;
    e->epoch = (e->epoch + 1) & 0xffffu;
    if (e->epoch == 0) e->epoch = 1;  // tags are (epoch << 16 | row); zero never matches

    Params prm{};
    prm.x = x; prm.delta = delta;
    prm.B = d_state ? static_cast<const void *>(B) : e->zeros;
    prm.C = d_state ? static_cast<const void *>(C) : e->zeros;
    prm.A = A; prm.D = D; prm.y = y; prm.zeros = e->zeros;
    prm.ticket = e->head; prm.done = e->head + 1; prm.err = e->head + 2;
    prm.sink = reinterpret_cast<char *>(e->head) + kHeadBytes;
    prm.cons = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(e->head) + kHeadBytes + kSinkBytes);
    prm.gring = e->gring;
    prm.batch = batch; prm.d_inner = d_inner; prm.d_state = d_state; prm.H = H; prm.W = W;
    prm.nstrips = pl.nstrips; prm.s_local = pl.s_local; prm.groups = pl.groups; prm.n_dblk = pl.n_dblk;
    prm.n_chains = pl.n_chains; prm.total_wg = pl.total_wg; prm.ring_rows = pl.ring_rows; prm.qg = pl.qg;
    prm.use_ticket = pl.groups > 1 ? 1 : 0;
    prm.xcd_remap = (pl.groups == 1 && pl.total_wg % 8 == 0 && env_int("SSM2D_XCD_REMAP", 1)) ? 1 : 0;
    prm.epoch = e->epoch;
    prm.vec_store = env_int("SSM2D_VECSTORE", 1);
    prm.spin_limit = g_spin_limit > 0 ? g_spin_limit : (1ll << 22);
    const size_t lds = lds_bytes<T, K, NPL, G>(pl);
    scan2d_fwd_kernel<T, K, NPL, ALIGN, G><<<dim3(pl.total_wg), dim3(block_threads(pl)), lds,
                                   static_cast<hipStream_t>(stream)>>>(prm);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? SSM2D_OK : hip_fail(err);
}

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

template <typename T>
int scan_fwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
             int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, void *stream)
{
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (batch == 0 || d_inner == 0 || H == 0 || W == 0) return SSM2D_OK;
    if (d_state > SSM2D_MAX_STATE || H > SSM2D_MAX_SIDE || W > SSM2D_MAX_SIDE) return SSM2D_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t{1} << 31) - 1;
    if (batch * d_inner * H * W > lim || batch * d_state * H * W > lim || d_inner * d_state > lim)
        return SSM2D_ERR_UNSUPPORTED;
    if (!x || !delta || !D || !y || (d_state > 0 && (!A || !B || !C))) return SSM2D_ERR_NULLPTR;
    if (misaligned(x) || misaligned(delta) || misaligned(D) || misaligned(y) ||
        (d_state > 0 && (misaligned(A) || misaligned(B) || misaligned(C))))
        return SSM2D_ERR_MISALIGNED;

    const Plan pl = make_plan(batch, d_inner, d_state, H, W);
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_mutex);
    const int bi = static_cast<int>(batch), di = static_cast<int>(d_inner), ni = static_cast<int>(d_state);
    const int hi = static_cast<int>(H), wi = static_cast<int>(W);
    const int align = (W % 4 == 0) ? 4 : ((W % 2 == 0) ? 2 : 1);
#define SSM2D_CASE(GG, KK, NN, AL) \
    if (pl.G == GG && pl.K == KK && pl.npl == NN && align == AL) \
        return run<T, KK, NN, AL, GG>(x, delta, A, B, C, D, y, bi, di, ni, hi, wi, pl, dev, stream);
    SSM2D_CASE(4, 4, 1, 4) SSM2D_CASE(4, 4, 2, 4) SSM2D_CASE(4, 4, 4, 4) SSM2D_CASE(4, 4, 8, 4)
    SSM2D_CASE(4, 8, 1, 4) SSM2D_CASE(4, 8, 2, 4) SSM2D_CASE(4, 8, 4, 4)
    SSM2D_CASE(4, 4, 1, 2) SSM2D_CASE(4, 4, 2, 2) SSM2D_CASE(4, 4, 4, 2) SSM2D_CASE(4, 4, 8, 2)
    SSM2D_CASE(4, 4, 1, 1) SSM2D_CASE(4, 4, 2, 1) SSM2D_CASE(4, 4, 4, 1) SSM2D_CASE(4, 4, 8, 1)
    SSM2D_CASE(8, 4, 1, 4) SSM2D_CASE(8, 4, 2, 4) SSM2D_CASE(8, 4, 4, 4) SSM2D_CASE(8, 4, 8, 4)
    SSM2D_CASE(8, 8, 1, 4) SSM2D_CASE(8, 8, 2, 4) SSM2D_CASE(8, 8, 4, 4)
    SSM2D_CASE(8, 4, 1, 2) SSM2D_CASE(8, 4, 2, 2) SSM2D_CASE(8, 4, 4, 2) SSM2D_CASE(8, 4, 8, 2)
    SSM2D_CASE(8, 4, 1, 1) SSM2D_CASE(8, 4, 2, 1) SSM2D_CASE(8, 4, 4, 1) SSM2D_CASE(8, 4, 8, 1)
#undef SSM2D_CASE
    return SSM2D_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

int ssm2d_scan_fwd(const float *x, const float *delta, const float *A, const float *B, const float *C,
                   const float *D, float *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                   int64_t W, void *stream)
{
    return scan_fwd<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, stream);
}

int ssm2d_scan_fwd_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                        const uint16_t *C, const float *D, uint16_t *y, int64_t batch, int64_t d_inner,
                        int64_t d_state, int64_t H, int64_t W, void *stream)
{
    return scan_fwd<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, stream);
}

const char *ssm2d_status_string(int status)
{
    switch (status) {
    case SSM2D_OK: return "ok";
    case SSM2D_ERR_NULLPTR: return "null pointer argument";
    case SSM2D_ERR_BAD_DIM: return "negative dimension";
    case SSM2D_ERR_UNSUPPORTED: return "unsupported size (d_state > 64, side > 65535 or tensor >= 2^31 elements)";
    case SSM2D_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case SSM2D_ERR_HIP: return "HIP runtime error";
    case SSM2D_ERR_NOMEM: return "workspace allocation failed";
    case SSM2D_ERR_DEVICE_TIMEOUT: return "kernel timed out waiting for a neighbouring strip's carries";
    default: return "unknown status";
    }
}

int ssm2d_sync_check(void *stream)
{
    SSM2D_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_mutex);
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || !it->second.head) return SSM2D_OK;
    unsigned int v = 0;
    SSM2D_HIP_TRY(hipMemcpy(&v, it->second.head + 2, sizeof(v), hipMemcpyDeviceToHost));
    if (v != 0) {
        unsigned int z = 0;
        SSM2D_HIP_TRY(hipMemcpy(it->second.head + 2, &z, sizeof(z), hipMemcpyHostToDevice));
        return SSM2D_ERR_DEVICE_TIMEOUT;
    }
    return SSM2D_OK;
}

int ssm2d_set_spin_limit(int64_t polls)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    g_spin_limit = polls < 0 ? 0 : polls;
    return SSM2D_OK;
}

int ssm2d_version(void) { return 200; }

const char *ssm2d_last_hip_error(void)
{
    return hipGetErrorString(static_cast<hipError_t>(g_last_hip_error.load()));
}

}  // extern "C"

// libssm2d: the plain forward scan of tall maps whose chains of strips are cut
// into several workgroups (the giga-pixel layout), two rows per step.
//
// Method (juejin.cn "2DMamba 精读", part 四 section 5; papernotes.org "2DMamba" 关键设计):
//   Abar = exp(delta*A), Bx = delta*B*x
//   hh[i,j] = Abar*hh[i,j-1] + Bx         horizontal scan, zero before column 0
//   h[i,j]  = Abar*h[i-1,j]  + hh[i,j]    vertical scan of the horizontal results
//   y = sum_n C*h + D*x                   state dims reduced on chip, only y stored
//
// Same decomposition as the general kernel (scan2d_kernel.h): a wave is 64/G
// channels x G state groups of NPL states, walking a strip of 4 columns down
// the map; the strips of a chain pass the row carry on through LDS rings
// inside a workgroup and through the couriers' tagged global words between
// workgroups; the workgroup's strips load their input rows cooperatively, in
// whole cache lines, into a shared ring of rows in LDS.
//
// What differs is the row loop, whose bookkeeping the general kernel pays
// per row: here one step covers two rows. Both rows' carry-independent work
// (decay factors, inputs) runs first; then one wait covers both rows' left
// carries, the two horizontal chains (independent of each other) run side by
// side, and one publish hands both carries on. The step loop is unrolled over
// the input ring (8 steps, 16 rows) and the carry rings (4 steps), so every
// LDS slot is a compile-time offset; the ring's arrival counts are per step;
// the output stores have one layout (a full strip of 4 aligned columns).
#pragma once

#include "scan2d_kernel.h"

namespace ssm2d_impl {

constexpr int kFastSteps = 8;       // steps of the input ring (two rows each)
constexpr int kFastAhead = 3;       // steps a wave writes its share ahead of processing
#ifndef SSM2D_FAST_PREFETCH
#define SSM2D_FAST_PREFETCH 2
#endif
constexpr int kFastPrefetch = SSM2D_FAST_PREFETCH;    // steps a share's loads are issued ahead of writing it
constexpr int kFastCarryRows = 8;   // rows of each LDS carry ring
constexpr int kFastStrips = 8;      // strips a workgroup of a chain across workgroups holds (with two couriers)
constexpr int kFastStripsWide = 4;  // the same for 8-column strips (one compute wave a SIMD)
constexpr int kFastStripsOne = 16;  // strips a workgroup holding a whole chain can hold (light layouts)

// Input ring: the invariant that keeps a slot from being rewritten while it is
// read. A wave reads step t only after every wave has written its share of
// it, which each wave does kFastAhead steps before processing it: so no wave
// is more than kFastAhead steps ahead of another. The fastest wave (at step f)
// writes step f + kFastAhead; the slowest reads a step >= f - kFastAhead; the
// two are 2 * kFastAhead < kFastSteps steps apart, so never in one slot.
static_assert(2 * kFastAhead < kFastSteps, "input ring too shallow for the staging distance");
static_assert(kFastSteps % kFastPrefetch == 0, "register sets of staged shares rotate with the unrolled steps");

// One chunk (4 elements) as a plain vector, which the compiler keeps in
// registers across the unrolled steps.
template <typename T> struct FastChunkOf;
template <> struct FastChunkOf<float> { using type = float __attribute__((ext_vector_type(4))); };
template <> struct FastChunkOf<uint16_t> { using type = unsigned __attribute__((ext_vector_type(2))); };

// LDS a launch may take (with the kernel's few static words).
constexpr size_t kFastLdsMax = 160 * 1024 - 256;

template <typename T, int G, int NPL, int K>
struct FastShape {
    using Chunk = typename FastChunkOf<T>::type;
    static constexpr int CPW = kWave / G;                       // channels per wave
    static constexpr int CPR = K / 4;                           // chunks per packet row of a strip
    static constexpr int NCHUNK = (2 * CPW + 2 * G * NPL) * CPR;  // packet rows: x, delta, B, C
    static constexpr int PASSES = (NCHUNK + kWave - 1) / kWave;  // chunks a lane loads per row
    static constexpr int PST = NCHUNK + 1;                      // chunks per strip packet (one pad chunk)
    static constexpr int SST = 2 * kFastSteps * PST + 1;        // chunks per strip's ring (its packets of 16 rows)
    // LDS of a workgroup of s strips: the input ring (each strip's packets of
    // 2 kFastSteps rows, strip-major, so that every offset within a strip's
    // ring is a compile-time constant) and s + 1 carry rings.
    static constexpr size_t ring_bytes(int s) { return static_cast<size_t>(s) * SST * sizeof(Chunk); }
    static constexpr size_t carry_bytes(int s)
    {
        return static_cast<size_t>(s + 1) * kFastCarryRows * kWave * NPL * 4;
    }
    static constexpr size_t lds_bytes(int s) { return ring_bytes(s) + carry_bytes(s); }
    // Strips a workgroup can hold: 8 (and two couriers) for chains of
    // 4-column strips across workgroups, 4 for 8-column strips (one compute
    // wave a SIMD, 256 registers a wave); 16 for a whole chain in the layouts light enough in
    // registers for 16 waves a CU (4-column strips with 1 state a lane, or
    // bf16 inputs), else 8.
    static constexpr int max_strips(bool chained)
    {
        if (chained) return K == 8 ? kFastStripsWide : kFastStrips;
        return (K == 4 && (NPL == 1 || sizeof(T) == 2)) ? kFastStripsOne : kFastStrips;
    }
};

// CHAINED: chains cut into several workgroups (tickets, couriers); else one
// workgroup holds a whole chain.
template <typename T, int G, int NPL, int K, bool CHAINED>
__global__ __launch_bounds__(kWave * (FastShape<T, G, NPL, K>::max_strips(CHAINED) + (CHAINED ? 2 : 0)))
void scan2d_fast_kernel(Params p)
{
    static_assert(K == 4 || K == 8, "4- or 8-column strips");
    using Sh = FastShape<T, G, NPL, K>;
    using Chunk = typename Sh::Chunk;
    constexpr int CPW = Sh::CPW, CPR = Sh::CPR, NCHUNK = Sh::NCHUNK, PASSES = Sh::PASSES, PST = Sh::PST,
                  SST = Sh::SST;
    constexpr int MAXS = Sh::max_strips(CHAINED);
    constexpr int SEG_DT = CPW, SEG_B = 2 * CPW, SEG_C = 2 * CPW + G * NPL;
    constexpr int CR = kFastCarryRows;
    constexpr int KO = K / G > 0 ? K / G : 1;  // finished cells per lane and row

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_done[MAXS + 1];   // rows published into LDS carry ring w
    __shared__ int s_used[MAXS + 1];   // rows consumed from LDS carry ring w
    __shared__ int s_arrive[kFastSteps];      // shares written into input-ring step slot
    __shared__ unsigned int s_ticket, s_epoch;
    __shared__ int s_last;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    if (CHAINED && threadIdx.x == 0) {
        s_ticket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_epoch = __hip_atomic_load(p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) % kEpochs + 1;
    }
    if (threadIdx.x <= MAXS) {
        s_done[threadIdx.x] = 0;
        s_used[threadIdx.x] = 0;
    }
    if (threadIdx.x < kFastSteps) s_arrive[threadIdx.x] = 0;
    __syncthreads();

    // Chained: tickets put every producer workgroup before its consumer (a
    // waiting workgroup's producer is resident or done). Otherwise workgroups
    // are dealt to the 8 XCDs round-robin; each XCD takes a contiguous run of
    // chains, so chains sharing a batch entry (and its B, C) share its L2.
    int wg;
    if constexpr (CHAINED) {
        wg = static_cast<int>(s_ticket);
    } else if (p.xcd_remap) {
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
    const long ring_floats = static_cast<long>(CR) * kWave * NPL;
    float *lring = reinterpret_cast<float *>(smem + Sh::ring_bytes(p.s_local));

    if (wave >= p.s_local) {
        if constexpr (CHAINED)
            courier_wave<NPL>(p, wave, lane, chain, grp, lring, s_done, s_used, s_epoch, ring_floats, CR - 1);
    } else if (grp * p.s_local + wave < p.nstrips) {
        // ---------------- compute wave: one strip of K columns
        const int strip = grp * p.s_local + wave;
        const int j0 = strip * K;
        const int valid = min(K, W - j0);  // columns of the strip inside the map
        const int nact = min(p.s_local, p.nstrips - grp * p.s_local);  // strips of this workgroup
        const int g = lane / CPW;
        const int dl = lane % CPW;
        const int d = dblk * CPW + dl;
        const bool d_ok = d < p.d_inner;
        const long HW = static_cast<long>(H) * W;
        // rows in scan order: top to bottom, or bottom to top (row t at row0 + t * rs)
        const int rs = p.flip_h ? -W : W;
        const long row0 = p.flip_h ? HW - W : 0;
        const T *zeros = static_cast<const T *>(p.zeros);
        T *ring = reinterpret_cast<T *>(smem);  // [strip][16 rows][PST chunks of 4 elements] (SST a strip)

        // This lane's chunks of the workgroup's rows: wave w loads chunks
        // [w NCHUNK, (w + 1) NCHUNK) of a row taken in column order (packet row
        // r of strips 0 .. nact-1, then packet row r + 1, ...), so a load
        // instruction reads whole cache lines, and writes each chunk into its
        // strip's packet. Padding lanes, and chunks past the row's end (the
        // second half of a last 8-column strip), read the zero page.
        const T *src[PASSES];
        int wdst[PASSES];
#pragma unroll
        for (int pp = 0; pp < PASSES; ++pp) {
            const int c = pp * kWave + lane;
            const T *base = zeros;
            int dst = wave * SST + NCHUNK;
            long col = 0;
            if (c < NCHUNK) {
                const int cw = wave * NCHUNK + c;
                const int r = cw / (nact * CPR), rem = cw % (nact * CPR);
                const int sj = rem / CPR, q = rem % CPR;
                dst = sj * SST + r * CPR + q;
                col = static_cast<long>(grp * p.s_local + sj) * K + 4 * q;
                if (col + 4 > W) {
                    // past the row's end: zeros
                } else if (r < SEG_DT) {
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
            src[pp] = base + row0 + (base == zeros ? 0 : col);
            wdst[pp] = dst;
        }

        float Ap[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int n = g * NPL + k;
            Ap[k] = (n < p.d_state && d_ok) ? p.A[d * p.d_state + n] * kLog2e : 0.0f;
        }
        const float Dd = d_ok ? p.D[d] : 0.0f;
#pragma unroll
        for (int k = 0; k < NPL; ++k) asm volatile("" ::"v"(Ap[k]));
        asm volatile("" ::"v"(Dd));

        // Operand offsets (elements) of this lane in a ring row.
        const int off_x = (wave * SST + dl * CPR) * 4;
        const int off_dt = (wave * SST + (SEG_DT + dl) * CPR) * 4;
        int off_b[NPL], off_c[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            off_b[k] = (wave * SST + (SEG_B + g * NPL + k) * CPR) * 4;
            off_c[k] = (wave * SST + (SEG_C + g * NPL + k) * CPR) * 4;
        }
        // The first finished cell of this lane after the sum over state
        // groups (for G = 8 and K = 4 the two lanes of a pair hold the same
        // cell). 4-column strips: pair stores (row r of the wave holds cell r;
        // one swap of odd and even rows leaves cells 0, 1 in row 0 and 2, 3 in
        // row 2, whose channel lanes store two cells each). 8-column strips:
        // each lane stores its own KO cells.
        const int c_out = (K >= G) ? g * KO : g / 2;
        const int off_xo = off_x + c_out;
        const bool storer = K == 4 ? (((lane & ~32) < CPW) && d_ok) : d_ok;
        T *yv = static_cast<T *>(p.y) + (static_cast<long>(b) * p.d_inner + (d_ok ? d : 0)) * HW + row0 + j0 +
                (K == 4 ? (((lane >> 5) & 1) ? 2 : 0) : c_out);
        bool cell_ok[KO];
#pragma unroll
        for (int c = 0; c < KO; ++c) cell_ok[c] = d_ok && c_out + c < valid;
        T *const ysink = static_cast<T *>(p.sink) + lane * 2 * KO;  // (8-column strips)

        const bool has_left = strip > 0;
        const bool has_right = strip + 1 < p.nstrips;
        const float *ring_in = lring + static_cast<long>(wave) * ring_floats + lane * NPL;
        float *ring_out = lring + static_cast<long>(wave + 1) * ring_floats + lane * NPL;
        bool timed_out = false;
        int skip = 0;  // kSkipWaits once a wait has given up: later waits pass at once

        // A wait that gave up: later waits are skipped, and the decay
        // exponents become NaN, so that every output this strip computes
        // from here on (and, through its carries, the strips after it) is NaN.
        auto give_up = [&]() __attribute__((always_inline)) {
            timed_out = true;
            skip = kSkipWaits;
#pragma unroll
            for (int k = 0; k < NPL; ++k) Ap[k] = quiet_nan();
        };
        auto wait_count = [&](const int *c, const int need) __attribute__((always_inline)) {
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

        float hv[K][NPL];
#pragma unroll
        for (int c = 0; c < K; ++c)
#pragma unroll
            for (int k = 0; k < NPL; ++k) hv[c][k] = 0.0f;

        // Shares of kFastPrefetch steps in flight: stg[s] holds the share of
        // the step staged kFastPrefetch steps after it was loaded.
        Chunk stg[kFastPrefetch][2][PASSES];
        auto load_step = [&](Chunk (&dst)[2][PASSES], const int first_row) __attribute__((always_inline)) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                for (int pp = 0; pp < PASSES; ++pp) {
                    const long off = static_cast<long>(min(first_row + rr, H - 1)) * rs;
                    dst[rr][pp] = *reinterpret_cast<const Chunk *>(src[pp] + off);
                }
        };
        auto write_step = [&](const Chunk (&sh)[2][PASSES], const int slot) __attribute__((always_inline)) {
            T *r0 = ring + 2 * slot * PST * 4;
#pragma unroll
            for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                for (int pp = 0; pp < PASSES; ++pp)
                    reinterpret_cast<Chunk *>(r0 + rr * PST * 4)[wdst[pp]] = sh[rr][pp];
            signal_fence();
            if (lane == 0) __hip_atomic_fetch_add(&s_arrive[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            signal_fence();
        };

        // Rows of the strip. LEFT: a strip (or the inbound courier) to the
        // left sends carries into LDS ring `wave`; RIGHT: one to the right
        // takes them from ring `wave + 1`.
        auto strip_rows = [&](auto left_tag, auto right_tag) __attribute__((always_inline)) {
            constexpr bool LEFT = decltype(left_tag)::value != 0;
            constexpr bool RIGHT = decltype(right_tag)::value != 0;
            int room = CR;  // rows this wave may publish, as last seen

            // Step of rows i = i0 + 2J and i + 1; J fixes the ring slots.
            // TAIL: the last, partial block of 16 rows (steps past the map
            // are skipped, and a second row past it is not stored).
            auto step = [&](const int i0, auto jt, auto tail_t) __attribute__((always_inline)) {
                constexpr int J = decltype(jt)::value;
                constexpr bool TAIL = decltype(tail_t)::value != 0;
                const int i = i0 + 2 * J;
                if constexpr (TAIL) {
                    if (i >= H) return;
                }
                // ---- stage: this wave's share of step J + kFastAhead, loaded
                // two steps ago; then the loads for two steps further on
                constexpr int JS = (J + kFastAhead) % kFastSteps;
                write_step(stg[J % kFastPrefetch], JS);
                load_step(stg[J % kFastPrefetch], i + 2 * (kFastAhead + kFastPrefetch));

                // ---- this step's rows (their arrival was confirmed at the end
                // of the previous step), and the arrival count of the next
                // step's, confirmed at the end of this one
                const T *r0 = ring + 2 * J * PST * 4;
                const T *r1 = r0 + PST * 4;
                float xv[2][K], dv[2][K], Bv[2][NPL][K], Cv[2][NPL][K], xo[2][KO];
                read_packet<K>(r0, off_x, xv[0]);
                read_packet<K>(r0, off_dt, dv[0]);
                read_packet<K>(r1, off_x, xv[1]);
                read_packet<K>(r1, off_dt, dv[1]);
#pragma unroll
                for (int k = 0; k < NPL; ++k) {
                    read_packet<K>(r0, off_b[k], Bv[0][k]);
                    read_packet<K>(r1, off_b[k], Bv[1][k]);
                    read_packet<K>(r0, off_c[k], Cv[0][k]);
                    read_packet<K>(r1, off_c[k], Cv[1][k]);
                }
#pragma unroll
                for (int c = 0; c < KO; ++c) {
                    xo[0][c] = elem_value(r0[off_xo + c]);
                    xo[1][c] = elem_value(r1[off_xo + c]);
                }
                constexpr int JN = (J + 1) % kFastSteps;
                const int need_next = nact * (((i + 2) >> 4) + 1);
                const int seen_next = lds_peek(&s_arrive[JN]);
                // left carries of both rows (counter, then the two slots)
                constexpr int C0 = (2 * J) % CR;
                int seen_c = 0;
                float hh[2][NPL];
                if constexpr (LEFT) {
                    seen_c = lds_peek(&s_done[wave]);
                    signal_fence();
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        hh[0][k] = ring_in[C0 * kWave * NPL + k];
                        hh[1][k] = ring_in[(C0 + 1) * kWave * NPL + k];
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) hh[0][k] = hh[1][k] = 0.0f;
                }

                // ---- carry-independent work of both rows
                float av[2][K][NPL], bx[2][K][NPL];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                    for (int c = 0; c < K; ++c) {
                        const float dx = dv[rr][c] * xv[rr][c];
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            av[rr][c][k] = __builtin_amdgcn_exp2f(dv[rr][c] * Ap[k]);
                            bx[rr][c][k] = dx * Bv[rr][k][c];
                        }
                    }
                // keep that work ahead of the waits below (the compiler would
                // sink it onto the carries' critical path)
#pragma unroll
                for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                    for (int c = 0; c < K; ++c)
#pragma unroll
                        for (int k = 0; k < NPL; ++k) asm volatile("" : "+v"(av[rr][c][k]), "+v"(bx[rr][c][k]));

                const int pub = TAIL ? min(i + 2, H) : i + 2;  // rows published after this step
                // room in the right ring for both rows (rarely short)
                if constexpr (RIGHT) {
                    if (pub > max(room, skip)) {
                        room = wait_counter_above(&s_used[wave + 1], pub - CR - 1, p.spin_limit, timed_out) + CR;
                        if (timed_out) give_up();
                    }
                }
                if constexpr (LEFT) {
                    if (max(__builtin_amdgcn_readfirstlane(seen_c), skip) < pub) {
                        // not both rows published yet: poll counter and slots
                        // together (one LDS round trip per poll)
                        long long spins = 0;
                        while (true) {
                            const int v = lds_peek(&s_done[wave]);
                            signal_fence();
                            float t0[NPL], t1[NPL];
#pragma unroll
                            for (int k = 0; k < NPL; ++k) {
                                t0[k] = ring_in[C0 * kWave * NPL + k];
                                t1[k] = ring_in[(C0 + 1) * kWave * NPL + k];
                            }
#pragma unroll
                            for (int k = 0; k < NPL; ++k) asm volatile("" : "+v"(t0[k]), "+v"(t1[k]));
                            if (__builtin_amdgcn_readfirstlane(v) >= pub) {
#pragma unroll
                                for (int k = 0; k < NPL; ++k) {
                                    hh[0][k] = t0[k];
                                    hh[1][k] = t1[k];
                                }
                                break;
                            }
                            if (++spins > p.spin_limit) {
                                give_up();
#pragma unroll
                                for (int k = 0; k < NPL; ++k) hh[0][k] = hh[1][k] = quiet_nan();
                                break;
                            }
                            if (spins > kSpinPolls) sleep_a_bit();
                        }
                    }
                }

                // ---- the two horizontal chains, then hand both carries on
                float hc[2][K][NPL];
#pragma unroll
                for (int c = 0; c < K; ++c)
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            hh[rr][k] = __builtin_fmaf(av[rr][c][k], hh[rr][k], bx[rr][c][k]);
                            hc[rr][c][k] = hh[rr][k];
                        }
                if constexpr (RIGHT) {
#pragma unroll
                    for (int k = 0; k < NPL; ++k) {
                        ring_out[C0 * kWave * NPL + k] = hh[0][k];
                        ring_out[(C0 + 1) * kWave * NPL + k] = hh[1][k];
                    }
                    signal_fence();
                    lds_poke(&s_done[wave + 1], pub);
                    // keep the vertical step below from being scheduled ahead
                    // of the publish: it would sit on the carry's path
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (LEFT) lds_poke(&s_used[wave], pub);

                // ---- vertical recurrence, sums over the lane's states and
                // over the state groups, skip term, stores
                float out[2][KO];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    float part[K];
#pragma unroll
                    for (int c = 0; c < K; ++c) {
                        float acc = 0.0f;
#pragma unroll
                        for (int k = 0; k < NPL; ++k) {
                            hv[c][k] = __builtin_fmaf(av[rr][c][k], hv[c][k], hc[rr][c][k]);
                            acc = __builtin_fmaf(Cv[rr][k][c], hv[c][k], acc);
                        }
                        part[c] = acc;
                    }
                    reduce_groups<K, G>(part, out[rr], g);
#pragma unroll
                    for (int c = 0; c < KO; ++c) out[rr][c] = __builtin_fmaf(Dd, xo[rr][c], out[rr][c]);
                }
                // pair stores of both rows (one swap of odd and even 16-lane
                // rows each), under one mask
                const long ro = static_cast<long>(i) * rs;
                const bool second = !TAIL || i + 1 < H;
                if constexpr (K == 8) {
                    // each lane its own cells; cells outside the map go to the
                    // sink, so the stores need no branch (a branch around them
                    // makes the next step's staging wait for their completion)
#pragma unroll
                    for (int c = 0; c < KO; ++c) {
                        store_elem(cell_ok[c] ? yv + ro + c : ysink + c, out[0][c]);
                        if (second) store_elem(cell_ok[c] ? yv + ro + rs + c : ysink + KO + c, out[1][c]);
                    }
                } else if constexpr (std::is_same<T, float>::value) {
                    float lo[2], hi[2];
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(out[rr][0]),
                                                                         __float_as_uint(out[rr][0]), false, false);
                        lo[rr] = __uint_as_float(sw[0]);
                        hi[rr] = __uint_as_float(sw[1]);
                    }
                    if (storer) {
                        *reinterpret_cast<float2 *>(yv + ro) = make_float2(lo[0], hi[0]);
                        if (second) *reinterpret_cast<float2 *>(yv + ro + rs) = make_float2(lo[1], hi[1]);
                    }
                } else {
                    unsigned wv[2];
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const unsigned h = bf16_bits(out[rr][0]);
                        const auto sw = __builtin_amdgcn_permlane16_swap(h, h, false, false);
                        wv[rr] = sw[0] | (sw[1] << 16);
                    }
                    if (storer) {
                        *reinterpret_cast<unsigned *>(yv + ro) = wv[0];
                        if (second) *reinterpret_cast<unsigned *>(yv + ro + rs) = wv[1];
                    }
                }
                // the next step's rows in: every strip's share written
                if (i + 2 < H && max(__builtin_amdgcn_readfirstlane(seen_next), skip) < need_next)
                    wait_count(&s_arrive[JN], need_next);
            };

            // shares of the first kFastAhead steps, and the loads of the next two
#pragma unroll
            for (int s = 0; s < kFastAhead; ++s) {
                load_step(stg[0], 2 * s);
                write_step(stg[0], s);
            }
#pragma unroll
            for (int q = 0; q < kFastPrefetch; ++q) load_step(stg[q], 2 * (kFastAhead + q));
            wait_count(&s_arrive[0], nact);  // the first step's rows
            using I = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            int i0 = 0;
            for (; i0 + 2 * kFastSteps <= H; i0 += 2 * kFastSteps) {
                step(i0, std::integral_constant<int, 0>{}, I{});
                step(i0, std::integral_constant<int, 1>{}, I{});
                step(i0, std::integral_constant<int, 2>{}, I{});
                step(i0, std::integral_constant<int, 3>{}, I{});
                step(i0, std::integral_constant<int, 4>{}, I{});
                step(i0, std::integral_constant<int, 5>{}, I{});
                step(i0, std::integral_constant<int, 6>{}, I{});
                step(i0, std::integral_constant<int, 7>{}, I{});
            }
            if (i0 < H) {
                step(i0, std::integral_constant<int, 0>{}, I1{});
                step(i0, std::integral_constant<int, 1>{}, I1{});
                step(i0, std::integral_constant<int, 2>{}, I1{});
                step(i0, std::integral_constant<int, 3>{}, I1{});
                step(i0, std::integral_constant<int, 4>{}, I1{});
                step(i0, std::integral_constant<int, 5>{}, I1{});
                step(i0, std::integral_constant<int, 6>{}, I1{});
                step(i0, std::integral_constant<int, 7>{}, I1{});
            }
        };
        using N0 = std::integral_constant<int, 0>;
        using N1 = std::integral_constant<int, 1>;
        if (has_left) {
            if (has_right) strip_rows(N1{}, N1{});
            else strip_rows(N1{}, N0{});
        } else {
            if (has_right) strip_rows(N0{}, N1{});
            else strip_rows(N0{}, N0{});
        }
        if (timed_out) report_timeout(p);
    }

    if constexpr (CHAINED) finish_launch(p, s_epoch, s_last);
}

// ---------------------------------------------------------------- host side

// Launch for a plan of one of the shared-row-ring layouts; CHAINED: the
// chains span workgroups (tickets, couriers and the global carry ring).
template <typename T, int G, int NPL, int K, bool CHAINED>
int run_fast(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int batch,
             int d_inner, int d_state, int H, int W, Plan pl, int dev, void *stream)
{
    using Sh = FastShape<T, G, NPL, K>;
    pl.ring_rows = kFastCarryRows;
    const int threads = kWave * (pl.s_local + (CHAINED ? 2 : 0));
    const size_t lds = Sh::lds_bytes(pl.s_local);
    pl.qg = H;
    pl.tblk = pl.n_chains;
    pl.ovf = 0;
    if constexpr (CHAINED) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan2d_fast_kernel<T, G, NPL, K, true>, threads,
                                                         lds) == hipSuccess)
            bound_ring(pl, static_cast<long>(per_cu) * device_cus(dev), H, NPL);
        else
            (void)hipGetLastError();
    }
    const WsNeed need = ws_need<NPL>(pl, d_inner, H, W);
    const WsEntry *e = pl.fixed_ws;
    if (e) {
        if (need.gring_bytes > e->gring_bytes || need.zero_bytes > e->zero_bytes || need.cons_count > e->cons_count)
            return SSM2D_ERR_TOO_LARGE;
    } else {
        WsEntry *w = nullptr;
        const int st = get_ws(dev, stream, need.gring_bytes, need.zero_bytes, need.cons_count, &w);
        if (st != SSM2D_OK) return st;
        e = w;
    }
    const Params prm = make_params(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, *e);
    scan2d_fast_kernel<T, G, NPL, K, CHAINED>
        <<<dim3(pl.total_wg), dim3(threads), lds, static_cast<hipStream_t>(stream)>>>(prm);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? SSM2D_OK : hip_fail(err);
}

// Whether a plan fits a layout's kernel: at most max_strips strips a
// workgroup, LDS within the CU's.
template <typename T, int G, int NPL, int K>
bool fast_layout_ok(const Plan &pl)
{
    using Sh = FastShape<T, G, NPL, K>;
    const bool chained = pl.groups > 1;
    return pl.s_local >= 1 && pl.s_local <= Sh::max_strips(chained) && Sh::lds_bytes(pl.s_local) <= kFastLdsMax;
}

template <typename T, int G, int NPL, int K>
int run_fast_layout(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int batch,
                    int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream)
{
    if (pl.groups > 1)
        return run_fast<T, G, NPL, K, true>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
    return run_fast<T, G, NPL, K, false>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
}

// Whether a plan's launch is the two-rows-per-step kernel: the plain forward
// (no direction or order bits, no carried states) of rows of a multiple of 4
// columns, in a plan with one of its layouts (4 or 8 state groups with 1 or 2
// states a lane, 4- or 8-column strips) that fast_layout_ok accepts.
template <typename T>
bool fast_path_taken_impl(const Plan &pl, int align)
{
    if (pl.mode != 0 || pl.h_init || pl.h_last || align != 4) return false;
#define SSM2D_FAST_CASE(GG, NN, KK) \
    if (pl.G == GG && pl.npl == NN && pl.K == KK) return fast_layout_ok<T, GG, NN, KK>(pl);
    SSM2D_FAST_CASE(8, 1, 4) SSM2D_FAST_CASE(8, 2, 4) SSM2D_FAST_CASE(8, 1, 8) SSM2D_FAST_CASE(8, 2, 8)
    SSM2D_FAST_CASE(4, 1, 4) SSM2D_FAST_CASE(4, 2, 4)
#undef SSM2D_FAST_CASE
    return false;
}

// The two-rows-per-step launch of a plan that fast_path_taken_impl accepts;
// kNoFastPath otherwise (the general kernel then runs it).
template <typename T>
int dispatch_fast_impl(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
                       int batch, int d_inner, int d_state, int H, int W, const Plan &pl, int dev, void *stream,
                       int align)
{
    if (!fast_path_taken_impl<T>(pl, align)) return kNoFastPath;
#define SSM2D_FAST_CASE(GG, NN, KK)                         \
    if (pl.G == GG && pl.npl == NN && pl.K == KK)           \
        return run_fast_layout<T, GG, NN, KK>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, pl, dev, stream);
    SSM2D_FAST_CASE(8, 1, 4) SSM2D_FAST_CASE(8, 2, 4) SSM2D_FAST_CASE(8, 1, 8) SSM2D_FAST_CASE(8, 2, 8)
    SSM2D_FAST_CASE(4, 1, 4) SSM2D_FAST_CASE(4, 2, 4)
#undef SSM2D_FAST_CASE
    return kNoFastPath;
}

}  // namespace ssm2d_impl

// libssm2d: 2DMamba 2D selective scan (forward) for MI355X / gfx950.
//
// Method (juejin.cn "2DMamba 精读" section 5; papernotes.org "2DMamba" 关键设计):
//   Abar = exp(delta*A), Bx = delta*B*x
//   hh[i,j] = Abar*hh[i,j-1] + Bx         horizontal scan, zero before column 0
//   h[i,j]  = Abar*h[i-1,j]  + hh[i,j]    vertical scan of the horizontal results
//   y = sum_n C*h + D*x                   state dims reduced on chip, only y stored
//
// Work decomposition (gfx950-specific; the pages' CUDA tiling is prior art):
//   * One wave = 64 lanes = 16 channels d x 4 state groups g. All lanes of a
//     wave sit on the same cell at the same time, so B and C (shared by all
//     channels) are broadcast loads, and x / delta are 16 contiguous row
//     segments. Each lane keeps NPL states (n = g*NPL + k).
//   * A lane walks a strip of K columns from the top row to the bottom row.
//     Along a row it runs the horizontal recurrence sequentially; the vertical
//     state of its K columns stays in registers. Nothing is padded to the
//     wavefront width: a map needs only ceil(W/K) strips.
//   * The horizontal carry (hh at the strip's right edge, per row) flows to the
//     next strip. Strips of one (batch, channel block) form a chain: waves of a
//     workgroup hand carries on through an LDS ring, workgroups through a
//     global buffer with epoch-tagged progress counters. A strip only waits
//     for the row it is about to process, so the chain runs as a pipeline.
//   * Workgroups take tickets from an atomic counter; ticket order puts every
//     producer before its consumer, so a waiting workgroup's producer is
//     always resident or done.
//   * The sum over n: each lane holds K partial sums over its NPL states; two
//     permlane swaps (32- and 16-lane) transpose-reduce them across the 4 state
//     groups, leaving each lane with K/4 finished cells.
// No MFMA: the scan is not a dense contraction.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "ssm2d.h"

namespace {

constexpr int kWave = 64;
constexpr int kGroups = 4;                 // state groups per wave
constexpr int kChanPerWave = kWave / kGroups;  // channels per wave
constexpr int kMaxStrips = 8;              // waves (strips) per workgroup
constexpr float kLog2e = 1.4426950408889634f;

struct Workspace {
    unsigned int *ticket;        // [1] next ticket
    unsigned int *done;          // [1] finished workgroups (last one resets both)
    unsigned int *err;           // [1] device error word
    unsigned long long *prog;    // [n_chains * groups] epoch<<32 | rows published
    float *carry;                // [n_chains][groups-1][H][NPL][64]
    void *zeros;                 // zero page: max(H*W) elements of 4 bytes
};

struct Params {
    const void *x, *delta, *B, *C;
    const float *A, *D;
    void *y;
    const void *zeros;
    unsigned int *ticket, *done, *err;
    unsigned long long *prog;
    float *carry;
    int batch, d_inner, d_state, H, W;
    int nstrips, s_local, groups, n_dblk, n_chains, total_wg;
    int ring_rows;     // LDS ring depth between waves
    int publish_rows;  // rows between global progress updates
    unsigned int epoch;
    long long spin_limit;
    int vec_ok;        // W % 4 == 0: strips can use vector loads
};

// Load N consecutive elements starting at p (fp32 or bf16 bits) into floats.
// `valid` < N masks the tail with zeros. `vec` allows 16-byte loads (fp32) or
// 8/16-byte loads (bf16), which needs N % 4 == 0 and a 16-byte aligned row.
template <int N> __device__ __forceinline__ void load_row(const float *p, float (&v)[N], int valid, bool vec)
{
    if constexpr (N % 4 == 0) {
        if (vec && valid == N) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                float4 t = reinterpret_cast<const float4 *>(p)[q];
                v[4 * q + 0] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
            }
            return;
        }
    }
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = (c < valid) ? p[c] : 0.0f;
}

template <int N> __device__ __forceinline__ void load_row(const uint16_t *p, float (&v)[N], int valid, bool vec)
{
    if constexpr (N % 4 == 0) {
        if (vec && valid == N) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                uint2 t = reinterpret_cast<const uint2 *>(p)[q];
                v[4 * q + 0] = __uint_as_float(t.x << 16);
                v[4 * q + 1] = __uint_as_float(t.x & 0xffff0000u);
                v[4 * q + 2] = __uint_as_float(t.y << 16);
                v[4 * q + 3] = __uint_as_float(t.y & 0xffff0000u);
            }
            return;
        }
    }
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = (c < valid) ? __uint_as_float(static_cast<unsigned>(p[c]) << 16) : 0.0f;
}

__device__ __forceinline__ void store_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t *p, float v)
{
    unsigned u = __float_as_uint(v);
    unsigned r;
    if ((u & 0x7fffffffu) > 0x7f800000u) r = (u >> 16) | 0x40u;          // quiet NaN
    else r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                       // nearest even
    *p = static_cast<uint16_t>(r);
}

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

template <int K>
__device__ __forceinline__ void reduce_groups(const float (&p)[K], float (&out)[K / 4])
{
    float q[K / 2];
#pragma unroll
    for (int c = 0; c < K / 2; ++c) q[c] = perm_sum32(p[c], p[c + K / 2]);
#pragma unroll
    for (int c = 0; c < K / 4; ++c) out[c] = perm_sum16(q[c], q[c + K / 4]);
}

__device__ __forceinline__ void sleep_a_bit() { __builtin_amdgcn_s_sleep(2); }

template <typename T, int K, int NPL>
__global__ __launch_bounds__(kWave * kMaxStrips) void scan2d_fwd_kernel(Params p)
{
    static_assert(K % kGroups == 0, "strip width must split over the 4 state groups");
    extern __shared__ float ring[];  // [s_local-1][ring_rows][64][NPL]
    __shared__ int s_done[kMaxStrips];
    __shared__ int s_used[kMaxStrips];
    __shared__ unsigned int s_ticket;

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < kMaxStrips) {
        s_done[threadIdx.x] = 0;
        s_used[threadIdx.x] = 0;
    }
    __syncthreads();

    const int ticket = static_cast<int>(s_ticket);
    const int chain = ticket % p.n_chains;
    const int grp = ticket / p.n_chains;
    const int b = chain / p.n_dblk;
    const int dblk = chain % p.n_dblk;
    const int strip = grp * p.s_local + wave;
    const int H = p.H, W = p.W;

    if (strip < p.nstrips) {
        const int j0 = strip * K;
        const int valid = min(K, W - j0);
        const bool vec = p.vec_ok != 0;
        const int g = lane / kChanPerWave;
        const int d = dblk * kChanPerWave + lane % kChanPerWave;
        const bool d_ok = d < p.d_inner;
        const long HW = static_cast<long>(H) * W;
        const T *zeros = static_cast<const T *>(p.zeros);

        // Channel rows (zero page for channels past d_inner).
        const T *xrow = d_ok ? static_cast<const T *>(p.x) + (static_cast<long>(b) * p.d_inner + d) * HW + j0 : zeros;
        const T *drow = d_ok ? static_cast<const T *>(p.delta) + (static_cast<long>(b) * p.d_inner + d) * HW + j0 : zeros;
        T *yrow = static_cast<T *>(p.y) + (static_cast<long>(b) * p.d_inner + (d_ok ? d : 0)) * HW + j0;
        const T *Brow[NPL];
        const T *Crow[NPL];
        float Ap[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
            const int n = g * NPL + k;
            const bool n_ok = n < p.d_state;
            Brow[k] = n_ok ? static_cast<const T *>(p.B) + (static_cast<long>(b) * p.d_state + n) * HW + j0 : zeros;
            Crow[k] = n_ok ? static_cast<const T *>(p.C) + (static_cast<long>(b) * p.d_state + n) * HW + j0 : zeros;
            Ap[k] = (n_ok && d_ok) ? p.A[d * p.d_state + n] * kLog2e : 0.0f;
        }
        const float Dd = d_ok ? p.D[d] : 0.0f;
        // Cells this lane finishes after the group reduction.
        constexpr int KO = K / kGroups;
        const int c_out = g * KO;

        // Neighbours in the chain.
        const bool has_left = strip > 0;
        const bool left_in_lds = has_left && wave > 0;
        const bool has_right = strip + 1 < p.nstrips;
        const bool right_in_lds = has_right && wave + 1 < p.s_local;
        const bool right_global = has_right && !right_in_lds;
        const int R = p.ring_rows;
        float *ring_in = ring + static_cast<long>(wave - 1) * R * kWave * NPL;
        float *ring_out = ring + static_cast<long>(wave) * R * kWave * NPL;
        unsigned long long *prog_in = p.prog + static_cast<long>(chain) * p.groups + (grp - 1);
        unsigned long long *prog_out = p.prog + static_cast<long>(chain) * p.groups + grp;
        const long carry_stride = static_cast<long>(H) * NPL * kWave;  // one boundary
        const float *gin = p.carry + (static_cast<long>(chain) * (p.groups - 1) + (grp - 1)) * carry_stride;
        float *gout = p.carry + (static_cast<long>(chain) * (p.groups - 1) + grp) * carry_stride;
        const unsigned long long tag = static_cast<unsigned long long>(p.epoch) << 32;

        int avail = 0;      // rows the left neighbour has published (as seen)
        int room = R;       // rows this wave may publish before the ring is full
        bool timed_out = false;

        float hv[K][NPL];
#pragma unroll
        for (int c = 0; c < K; ++c)
#pragma unroll
            for (int k = 0; k < NPL; ++k) hv[c][k] = 0.0f;

        for (int i = 0; i < H; ++i) {
            const long roff = static_cast<long>(i) * W;
            // ---- inputs of row i (independent of the carry: issue first)
            float xv[K], dv[K], Bv[NPL][K], Cv[NPL][K], xo[KO];
            load_row<K>(xrow + roff, xv, valid, vec);
            load_row<K>(drow + roff, dv, valid, vec);
#pragma unroll
            for (int k = 0; k < NPL; ++k) {
                load_row<K>(Brow[k] + roff, Bv[k], valid, vec);
                load_row<K>(Crow[k] + roff, Cv[k], valid, vec);
            }
            load_row<KO>(xrow + roff + c_out, xo, valid - c_out, false);

            // ---- left carry of row i
            float hh[NPL];
            if (!has_left) {
#pragma unroll
                for (int k = 0; k < NPL; ++k) hh[k] = 0.0f;
            } else if (left_in_lds) {
                if (i >= avail && !timed_out) {
                    long spins = 0;
                    while ((avail = __hip_atomic_load(&s_done[wave - 1], __ATOMIC_ACQUIRE,
                                                      __HIP_MEMORY_SCOPE_WORKGROUP)) <= i) {
                        if (++spins > p.spin_limit) { timed_out = true; break; }
                        sleep_a_bit();
                    }
                }
                const float *src = ring_in + (static_cast<long>(i % R) * kWave + lane) * NPL;
#pragma unroll
                for (int k = 0; k < NPL; ++k) hh[k] = src[k];
                __hip_atomic_store(&s_used[wave - 1], i + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                if (i >= avail && !timed_out) {
                    long spins = 0;
                    for (;;) {
                        unsigned long long v = __hip_atomic_load(prog_in, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
                        if ((v & 0xffffffff00000000ull) == tag) {
                            avail = static_cast<int>(v & 0xffffffffu);
                            if (avail > i) break;
                        }
                        if (++spins > p.spin_limit) { timed_out = true; break; }
                        sleep_a_bit();
                    }
                }
                const float *src = gin + static_cast<long>(i) * NPL * kWave + lane;
#pragma unroll
                for (int k = 0; k < NPL; ++k) hh[k] = src[k * kWave];
            }

            // ---- the scan over this row's K cells
            float part[K];
#pragma unroll
            for (int c = 0; c < K; ++c) {
                const float dt = dv[c];
                const float dx = dt * xv[c];
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < NPL; ++k) {
                    const float a = __builtin_amdgcn_exp2f(dt * Ap[k]);
                    hh[k] = __builtin_fmaf(a, hh[k], dx * Bv[k][c]);
                    hv[c][k] = __builtin_fmaf(a, hv[c][k], hh[k]);
                    acc = __builtin_fmaf(Cv[k][c], hv[c][k], acc);
                }
                part[c] = acc;
            }

            // ---- hand the right-edge carry on
            if (right_in_lds) {
                if (i >= room && !timed_out) {
                    long spins = 0;
                    int used;
                    while ((used = __hip_atomic_load(&s_used[wave], __ATOMIC_ACQUIRE,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP)) + R <= i) {
                        if (++spins > p.spin_limit) { timed_out = true; break; }
                        sleep_a_bit();
                    }
                    room = used + R;
                }
                float *dst = ring_out + (static_cast<long>(i % R) * kWave + lane) * NPL;
#pragma unroll
                for (int k = 0; k < NPL; ++k) dst[k] = hh[k];
                __hip_atomic_store(&s_done[wave], i + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else if (right_global) {
                float *dst = gout + static_cast<long>(i) * NPL * kWave + lane;
#pragma unroll
                for (int k = 0; k < NPL; ++k) dst[k * kWave] = hh[k];
                if ((i + 1) % p.publish_rows == 0 || i + 1 == H)
                    __hip_atomic_store(prog_out, tag | static_cast<unsigned long long>(i + 1),
                                       __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }

            // ---- sum over the state groups, skip term, store
            float out[KO];
            reduce_groups<K>(part, out);
            if (d_ok) {
#pragma unroll
                for (int c = 0; c < KO; ++c)
                    if (c_out + c < valid) store_elem(yrow + roff + c_out + c, out[c] + Dd * xo[c]);
            }
        }
        if (timed_out) atomicOr(p.err, 1u);
    }

    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned int old = __hip_atomic_fetch_add(p.done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == static_cast<unsigned int>(p.total_wg)) {
            __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- host side

struct Plan {
    int K, npl, nstrips, s_local, groups, n_dblk, n_chains, total_wg, ring_rows, publish_rows;
};

int env_int(const char *name, int dflt)
{
    const char *s = std::getenv(name);
    return (s && *s) ? std::atoi(s) : dflt;
}

Plan make_plan(int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W)
{
    Plan pl{};
    int npl = 1;
    while (npl * kGroups < d_state) npl *= 2;
    pl.npl = npl;
    pl.K = 4;
    pl.K = env_int("SSM2D_STRIP", pl.K);
    if (pl.K != 4 && pl.K != 8) pl.K = 4;
    if (npl == 16) pl.K = 4;
    pl.nstrips = static_cast<int>((W + pl.K - 1) / pl.K);
    pl.n_dblk = static_cast<int>((d_inner + kChanPerWave - 1) / kChanPerWave);
    pl.n_chains = static_cast<int>(batch) * pl.n_dblk;
    // Enough workgroups to cover the chip; otherwise keep a whole chain in
    // one workgroup so the carries stay in LDS.
    int want_wg = 512;
    int groups = (pl.n_chains >= want_wg) ? 1 : (want_wg + pl.n_chains - 1) / pl.n_chains;
    int s_local = (pl.nstrips + groups - 1) / groups;
    if (s_local < 1) s_local = 1;
    if (s_local > kMaxStrips) s_local = kMaxStrips;
    s_local = env_int("SSM2D_WAVES", s_local);
    if (s_local < 1) s_local = 1;
    if (s_local > kMaxStrips) s_local = kMaxStrips;
    if (s_local > pl.nstrips) s_local = pl.nstrips;
    pl.s_local = s_local;
    pl.groups = (pl.nstrips + s_local - 1) / s_local;
    pl.total_wg = pl.n_chains * pl.groups;
    pl.ring_rows = (npl <= 4) ? 8 : (npl == 8 ? 4 : 2);
    pl.publish_rows = env_int("SSM2D_PUBLISH", 2);
    if (pl.publish_rows < 1) pl.publish_rows = 1;
    return pl;
}

struct WsEntry {
    Workspace ws{};
    size_t carry_bytes = 0, zero_bytes = 0, prog_count = 0;
    unsigned int epoch = 0;
};

std::mutex g_mutex;
std::map<std::pair<int, void *>, WsEntry> g_ws;
long long g_spin_limit = 0;

void free_ws(WsEntry &e)
{
    if (e.ws.ticket) (void)hipFree(e.ws.ticket);
    if (e.ws.carry) (void)hipFree(e.ws.carry);
    if (e.ws.zeros) (void)hipFree(e.ws.zeros);
    e = WsEntry{};
}

// Workspace for (device, stream), grown when needed. Growth waits for the
// stream so that no in-flight kernel still uses the old buffers.
int get_ws(int dev, void *stream, size_t carry_bytes, size_t zero_bytes, size_t prog_count, WsEntry **out)
{
    WsEntry &e = g_ws[{dev, stream}];
    if (e.ws.ticket && carry_bytes <= e.carry_bytes && zero_bytes <= e.zero_bytes && prog_count <= e.prog_count) {
        *out = &e;
        return SSM2D_OK;
    }
    if (e.ws.ticket) {
        if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SSM2D_ERR_HIP;
        free_ws(e);
    }
    size_t cb = carry_bytes < 256 ? 256 : carry_bytes;
    size_t zb = zero_bytes < 256 ? 256 : zero_bytes;
    size_t pc = prog_count < 1 ? 1 : prog_count;
    size_t head = 256 + pc * sizeof(unsigned long long);
    void *h = nullptr, *c = nullptr, *z = nullptr;
    if (hipMalloc(&h, head) != hipSuccess || hipMalloc(&c, cb) != hipSuccess || hipMalloc(&z, zb) != hipSuccess) {
        if (h) (void)hipFree(h);
        if (c) (void)hipFree(c);
        (void)hipGetLastError();
        return SSM2D_ERR_NOMEM;
    }
    if (hipMemset(h, 0, head) != hipSuccess || hipMemset(z, 0, zb) != hipSuccess) return SSM2D_ERR_HIP;
    e.ws.ticket = static_cast<unsigned int *>(h);
    e.ws.done = e.ws.ticket + 1;
    e.ws.err = e.ws.ticket + 2;
    e.ws.prog = reinterpret_cast<unsigned long long *>(static_cast<char *>(h) + 256);
    e.ws.carry = static_cast<float *>(c);
    e.ws.zeros = z;
    e.carry_bytes = cb;
    e.zero_bytes = zb;
    e.prog_count = pc;
    e.epoch = 0;
    *out = &e;
    return SSM2D_OK;
}

template <typename T, int K, int NPL>
hipError_t launch(const Params &prm, const Plan &pl, hipStream_t stream)
{
    size_t lds = static_cast<size_t>(pl.s_local > 1 ? pl.s_local - 1 : 0) * pl.ring_rows * kWave * NPL * sizeof(float);
    hipLaunchKernelGGL((scan2d_fwd_kernel<T, K, NPL>), dim3(pl.total_wg), dim3(kWave * pl.s_local), lds, stream, prm);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const Params &prm, const Plan &pl, hipStream_t stream)
{
#define SSM2D_CASE(KK, NN) if (pl.K == KK && pl.npl == NN) return launch<T, KK, NN>(prm, pl, stream);
    SSM2D_CASE(4, 1) SSM2D_CASE(4, 2) SSM2D_CASE(4, 4) SSM2D_CASE(4, 8) SSM2D_CASE(4, 16)
    SSM2D_CASE(8, 1) SSM2D_CASE(8, 2) SSM2D_CASE(8, 4) SSM2D_CASE(8, 8)
#undef SSM2D_CASE
    return hipErrorInvalidValue;
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
    if (hipGetDevice(&dev) != hipSuccess) return SSM2D_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    const size_t carry_bytes = static_cast<size_t>(pl.n_chains) * (pl.groups - 1) * H * pl.npl * kWave * sizeof(float);
    const size_t zero_bytes = static_cast<size_t>(H) * W * 4 + 64;
    WsEntry *e = nullptr;
    int st = get_ws(dev, stream, carry_bytes, zero_bytes, static_cast<size_t>(pl.n_chains) * pl.groups, &e);
    if (st != SSM2D_OK) return st;
    e->epoch += 1;
    if (e->epoch == 0) e->epoch = 1;  // 0 marks never-written progress counters

    Params prm{};
    prm.x = x; prm.delta = delta; prm.B = d_state ? B : e->ws.zeros; prm.C = d_state ? C : e->ws.zeros;
    prm.A = A; prm.D = D; prm.y = y; prm.zeros = e->ws.zeros;
    prm.ticket = e->ws.ticket; prm.done = e->ws.done; prm.err = e->ws.err;
    prm.prog = e->ws.prog; prm.carry = e->ws.carry;
    prm.batch = static_cast<int>(batch); prm.d_inner = static_cast<int>(d_inner);
    prm.d_state = static_cast<int>(d_state); prm.H = static_cast<int>(H); prm.W = static_cast<int>(W);
    prm.nstrips = pl.nstrips; prm.s_local = pl.s_local; prm.groups = pl.groups; prm.n_dblk = pl.n_dblk;
    prm.n_chains = pl.n_chains; prm.total_wg = pl.total_wg; prm.ring_rows = pl.ring_rows;
    prm.publish_rows = pl.publish_rows; prm.epoch = e->epoch;
    prm.spin_limit = g_spin_limit > 0 ? g_spin_limit : (1ll << 22);
    prm.vec_ok = (W % 4 == 0) ? 1 : 0;
    hipError_t err = dispatch<T>(prm, pl, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? SSM2D_OK : SSM2D_ERR_HIP;
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
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SSM2D_ERR_HIP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSM2D_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || !it->second.ws.err) return SSM2D_OK;
    unsigned int v = 0;
    if (hipMemcpy(&v, it->second.ws.err, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return SSM2D_ERR_HIP;
    if (v != 0) {
        unsigned int z = 0;
        if (hipMemcpy(it->second.ws.err, &z, sizeof(z), hipMemcpyHostToDevice) != hipSuccess) return SSM2D_ERR_HIP;
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

int ssm2d_version(void) { return 100; }

}  // extern "C"

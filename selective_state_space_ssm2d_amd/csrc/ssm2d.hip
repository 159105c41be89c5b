// libssm2d: 2DMamba 2D selective scan for MI355X / gfx950 -- host side:
// argument checks, the work plan, per-stream workspaces, the small elementwise
// kernels around the scan (step-size preparation, gating of summed outputs,
// the backward's zeroing and channel sums) and the C ABI declared in
// include/ssm2d.h. The scan kernel is in scan2d_kernel.h; its instances are
// compiled in scan2d_{f32,bf16}_*.hip.
#include "scan2d_kernel.h"

namespace ssm2d_impl {

int env_int(const char *name, int dflt)
{
    const char *s = std::getenv(name);
    return (s && *s) ? std::atoi(s) : dflt;
}

Plan make_plan(int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, int mode)
{
    Plan pl{};
    pl.mode = mode;
    const int want_wg = 256;  // enough workgroups to cover the chip's CUs
    // Layout: 4 state groups per wave (16 channels) unless the map has more
    // than 4 states and too few (batch, channel-block) chains to give every CU
    // two chains. Then 8 groups (8 channels, half the states per lane) double
    // the chains, halve the workgroups each chain spans, and put two compute
    // waves on each SIMD; with between one and two chains per CU they also
    // even out the last round of workgroups (VMamba stage 1: 384 chains of
    // 16 channels, 768 of 8). Above 32 states a lane of a 4-group layout would
    // hold 16 states, more than its registers: 8 groups then too.
    const int64_t chains4 = batch * ((d_inner + 15) / 16);
    int G = (d_state > 32 || (d_state > 4 && chains4 < 2 * want_wg)) ? 8 : 4;
    const int genv = env_int("SSM2D_GROUPS", 0);
    if (genv == 8 || (genv == 4 && d_state <= 32)) G = genv;
    // The other modes use 8 groups, except the forward modes on maps whose
    // chains fit one workgroup of 4-column strips (W <= 32) with 9 to 16
    // states and rows of an even number of columns: there they have 4-group
    // kernels too (4 states a lane, like the forward's).
    if (mode != 0) {
        const bool g4_ok = G == 4 && d_state > 8 && d_state <= 16 && W % 2 == 0 && (W + 3) / 4 <= max_waves(4, 4, 4) &&
                           !(mode & (kModeStates | kModeBackward));
        if (!g4_ok) G = 8;
    }
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
    // 8-column strips: forward scans of any direction and order; the
    // backward's passes keep 4-column strips (one tile layout)
    const bool wide_ok = npl <= 4 && W % 4 == 0 && !(mode & (kModeStates | kModeBackward));
    pl.K = 4;
    if (pl.n_chains >= want_wg && (W + 3) / 4 > max_waves(4, npl, G, mode) && wide_ok &&
        (W + 7) / 8 <= max_waves(8, npl, G, mode))
        pl.K = 8;
    const int kenv = env_int("SSM2D_STRIP", 0);
    if (kenv == 4 || (kenv == 8 && wide_ok)) pl.K = kenv;
    if ((mode & (kModeStates | kModeBackward)) || (mode != 0 && G == 4)) pl.K = 4;
    const int maxw = max_waves(pl.K, npl, G, mode);
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
    if (s_local < pl.nstrips && s_local > maxw - 2 && !(mode & kModeEdges))
        s_local = maxw - 2;  // room for 2 couriers (none in the courier-free adjoint pass)
    pl.s_local = s_local;
    pl.groups = (pl.nstrips + s_local - 1) / s_local;
    pl.total_wg = pl.n_chains * pl.groups;
    // LDS ring depth: a power of two, at least 2 (and at least a courier
    // batch), with all rings of a workgroup within ~48 KB.
    const long row_bytes = static_cast<long>(kWave) * npl * 4;
    const long budget = 48 * 1024;
    int R = 8;
    const int renv = env_int("SSM2D_LDSRING", 0);
    if (renv == 4 || renv == 16 || renv == 32) R = renv;
    while (R > 2 && (s_local + 1) * R * row_bytes > budget * (R > 8 ? 2 : 1)) R /= 2;
    pl.ring_rows = R;
    pl.qg = static_cast<int>(H);
    return pl;
}


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

// ---------------------------------------------------------------- backward

// Backward workspace per (device, stream): the stored states and the
// per-channel-block partial sums of dB and dC. Grown when needed (after
// waiting for the stream); zeroed when allocated.
struct BwdWs {
    void *buf = nullptr;
    size_t bytes = 0;
};
std::map<std::pair<int, void *>, BwdWs> g_bwd_ws;

int get_bwd_ws(int dev, void *stream, size_t bytes, void **out)
{
    BwdWs &e = g_bwd_ws[{dev, stream}];
    if (e.buf && bytes <= e.bytes) {
        *out = e.buf;
        return SSM2D_OK;
    }
    if (e.buf) {
        SSM2D_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
        (void)hipFree(e.buf);
        e = BwdWs{};
    }
    void *b = nullptr;
    if (hipMalloc(&b, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return SSM2D_ERR_NOMEM;
    }
    SSM2D_HIP_TRY(hipMemset(b, 0, bytes));
    e.buf = b;
    e.bytes = bytes;
    *out = b;
    return SSM2D_OK;
}

// Zeroes dA and dD (the backward adds into them).
__global__ void bwd_prepare_kernel(float *dA, long n_a, float *dD, long n_d)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < n_a) dA[t] = 0.0f;
    if (t < n_d) dD[t] = 0.0f;
}

__device__ __forceinline__ void put(float *p, float v) { *p = v; }
__device__ __forceinline__ void put(uint16_t *p, float v) { *p = static_cast<uint16_t>(bf16_bits(v)); }

// dB, dC [batch][d_state][H][W] = sums over the channel blocks of the
// backward's 8-channel sums ([channel block][batch][d_state][H][ld], the map
// starting at column pad of each row).
template <typename T>
__global__ void bwd_reduce_kernel(const float *dBp, const float *dCp, long part_stride, int n_dblk, T *dB, T *dC,
                                  long total, int W, int ld, int pad)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const long row = t / W;
    long idx = row * ld + pad + (t - row * W);
    float sb = 0.0f, sc = 0.0f;
    for (int q = 0; q < n_dblk; ++q, idx += part_stride) {
        sb += dBp[idx];
        sc += dCp[idx];
    }
    put(dB + t, sb);
    put(dC + t, sc);
}

// ---------------------------------------------------------------- Mamba-op options

// Scratch per (device, stream, slot), grown when needed; not zeroed.
std::map<std::pair<std::pair<int, void *>, int>, BwdWs> g_aux_ws;

int get_aux_ws(int dev, void *stream, int slot, size_t bytes, void **out)
{
    BwdWs &e = g_aux_ws[{{dev, stream}, slot}];
    if (e.buf && bytes <= e.bytes) {
        *out = e.buf;
        return SSM2D_OK;
    }
    if (e.buf) {
        SSM2D_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
        (void)hipFree(e.buf);
        e = BwdWs{};
    }
    void *b = nullptr;
    if (hipMalloc(&b, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return SSM2D_ERR_NOMEM;
    }
    e.buf = b;
    e.bytes = bytes;
    *out = b;
    return SSM2D_OK;
}

__device__ __forceinline__ float get(const float *p) { return *p; }
__device__ __forceinline__ float get(const uint16_t *p) { return __uint_as_float(static_cast<unsigned>(*p) << 16); }

// Step size of the scan: delta + bias[d], through softplus if asked, computed
// in fp32 and stored in the input type. softplus(v) = max(v, 0) + log1p(e^-|v|).
template <typename T>
__global__ void delta_prep_kernel(const T *delta, const float *bias, T *out, long total, long hw, int d_inner,
                                  int use_softplus)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    float v = get(delta + t);
    if (bias) v += bias[(t / hw) % d_inner];
    if (use_softplus) v = fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));
    put(out + t, v);
}

// y *= SiLU(z) = z / (1 + e^-z), for outputs summed over several launches.
template <typename T>
__global__ void gate_kernel(T *y, const T *z, long total)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const float zf = get(z + t);
    put(y + t, get(y + t) * (zf / (1.0f + expf(-zf))));
}

// Backward of the gate: dz = dy * y * SiLU'(z), and the scan's upstream
// gradient dy * SiLU(z); SiLU'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z).
template <typename T>
__global__ void gate_bwd_kernel(const T *dy, const T *y, const T *z, T *dz, T *dys, long total)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const float zf = get(z + t), g = get(dy + t);
    const float sg = 1.0f / (1.0f + expf(-zf));
    put(dz + t, g * get(y + t) * sg * (1.0f + zf * (1.0f - sg)));
    put(dys + t, g * zf * sg);
}

// Backward of the step-size preparation, one block per (batch, channel) map:
// d delta = d delta' * sigmoid(delta + bias[d]) with softplus (else
// unchanged), and d bias[d] += the map's sum of d delta.
template <typename T>
__global__ void step_bwd_kernel(T *ddelta, const T *delta, const float *bias, float *dbias, long hw, int d_inner,
                                int use_softplus)
{
    __shared__ float part[256];
    const long map = blockIdx.x;
    const int d = static_cast<int>(map % d_inner);
    const float bd = bias ? bias[d] : 0.0f;
    float acc = 0.0f;
    for (long p = threadIdx.x; p < hw; p += blockDim.x) {
        const long t = map * hw + p;
        float g = get(ddelta + t);
        if (use_softplus) {
            g *= 1.0f / (1.0f + expf(-(get(delta + t) + bd)));
            put(ddelta + t, g);
        }
        acc += g;
    }
    if (!dbias) return;
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w /= 2) {
        if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) (void)unsafeAtomicAdd(dbias + d, part[0]);
}

__global__ void zero_kernel(float *p, long n)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < n) p[t] = 0.0f;
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

}  // namespace ssm2d_impl

namespace {

using namespace ssm2d_impl;

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }  // NULL passes

// Cooperative loads (a shared ring of input rows per workgroup): 8-group
// layouts with 4-column strips and 4-aligned rows, when a workgroup holds part
// of a chain of a tall map (short maps do not repay the ring's start-up), if
// the row ring fits; for the adjoint pass, with its courier-free chains.
template <typename T>
void choose_coop(Plan &pl, int64_t H, int align)
{
    pl.coop_slots = 0;
    if (((pl.mode & kModeBackward) && !(pl.mode & kModeEdges)) || pl.G != 8 || pl.K != 4 || align != 4 ||
        pl.groups <= 1 || H < 128 || !env_int("SSM2D_COOP", 1))
        return;
    using Chunk = typename ChunkOf<T>::type;
    // packet rows: x and delta of 8 channels, B and C of 8 * npl states, and
    // dy of the 8 channels in the adjoint pass
    const size_t nchunk = static_cast<size_t>(16 + 16 * pl.npl + ((pl.mode & kModeBackward) ? 8 : 0));
    const size_t rings = static_cast<size_t>(pl.s_local + 1) * pl.ring_rows * kWave * pl.npl * 4;
    for (int slots = kMaxSlots; slots >= 8 && pl.coop_slots == 0; slots /= 2)
        if (static_cast<size_t>(pl.s_local) * slots * (nchunk + 1) * sizeof(Chunk) + rings <= 144 * 1024)
            pl.coop_slots = slots;
}

template <typename T>
int launch(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int64_t batch,
           int64_t d_inner, int64_t d_state, int64_t H, int64_t W, int mode, int flip_h, int dev, void *stream,
           const T *z = nullptr, const float *h_init = nullptr, float *h_last = nullptr)
{
    Plan pl = make_plan(batch, d_inner, d_state, H, W, mode);
    pl.flip_h = flip_h;
    pl.z = z;
    pl.h_init = h_init;
    pl.h_last = h_last;
    const int bi = static_cast<int>(batch), di = static_cast<int>(d_inner), ni = static_cast<int>(d_state);
    const int hi = static_cast<int>(H), wi = static_cast<int>(W);
    const int align = (W % 4 == 0) ? 4 : ((W % 2 == 0) ? 2 : 1);
    choose_coop<T>(pl, H, align);
#define SSM2D_ARGS x, delta, A, B, C, D, y, bi, di, ni, hi, wi, pl, dev, stream, align
    constexpr int FW = kModeFlipW, VF = kModeVFirst, AC = kModeAccumulate;
    switch (mode) {
    case 0: return pl.G == 8 ? dispatch_g8(SSM2D_ARGS) : dispatch_g4(SSM2D_ARGS);
    case FW: return dispatch_flipw(SSM2D_ARGS);
    case VF: return dispatch_vfirst(SSM2D_ARGS);
    case FW | VF: return dispatch_flipw_vfirst(SSM2D_ARGS);
    case AC: return dispatch_acc(SSM2D_ARGS);
    case FW | AC: return dispatch_flipw_acc(SSM2D_ARGS);
    case VF | AC: return dispatch_vfirst_acc(SSM2D_ARGS);
    case FW | VF | AC: return dispatch_flipw_vfirst_acc(SSM2D_ARGS);
    case kModeGate: return dispatch_gate(SSM2D_ARGS);
    case kModeGate | VF: return dispatch_gate_vfirst(SSM2D_ARGS);
    case kModeGate | FW: return dispatch_gate_flipw(SSM2D_ARGS);
    case kModeGate | FW | VF: return dispatch_gate_flipw_vfirst(SSM2D_ARGS);
    default: return SSM2D_ERR_UNSUPPORTED;
    }
#undef SSM2D_ARGS
}

constexpr unsigned kKnownFlags = SSM2D_FLIP_H | SSM2D_FLIP_W | SSM2D_VERTICAL_FIRST | SSM2D_ACCUMULATE | SSM2D_FOUR_WAY |
                                 SSM2D_DELTA_SOFTPLUS;

// `extended`: the flag-taking entry points, where D may be NULL (no skip term).
// z (gate) and delta_bias come with the Mamba-option entry points only.
template <typename T>
int scan_fwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
             int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, unsigned flags, bool extended,
             void *stream, const T *z = nullptr, const float *delta_bias = nullptr, const float *h_init = nullptr,
             float *h_last = nullptr)
{
    if ((flags & ~kKnownFlags) != 0) return SSM2D_ERR_BAD_FLAGS;
    if ((flags & SSM2D_FOUR_WAY) && (flags & (SSM2D_FLIP_H | SSM2D_FLIP_W))) return SSM2D_ERR_BAD_FLAGS;
    if (z && (flags & SSM2D_ACCUMULATE)) return SSM2D_ERR_BAD_FLAGS;
    if ((h_init || h_last) && (flags & SSM2D_FOUR_WAY)) return SSM2D_ERR_BAD_FLAGS;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (batch == 0 || d_inner == 0 || H == 0 || W == 0) return SSM2D_OK;
    if (d_state > SSM2D_MAX_STATE || H > SSM2D_MAX_SIDE || W > SSM2D_MAX_SIDE) return SSM2D_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t{1} << 31) - 1;
    if (batch * d_inner * H * W > lim || batch * d_state * H * W > lim || d_inner * d_state > lim)
        return SSM2D_ERR_UNSUPPORTED;
    if (!x || !delta || (!D && !extended) || !y || (d_state > 0 && (!A || !B || !C))) return SSM2D_ERR_NULLPTR;
    if (misaligned(x) || misaligned(delta) || misaligned(D) || misaligned(y) || misaligned(z) ||
        misaligned(delta_bias) || misaligned(h_init) || misaligned(h_last) ||
        (d_state > 0 && (misaligned(A) || misaligned(B) || misaligned(C))))
        return SSM2D_ERR_MISALIGNED;

    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_mutex);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long total = batch * d_inner * H * W;
    const unsigned nblk = static_cast<unsigned>((total + 255) / 256);
    if (delta_bias || (flags & SSM2D_DELTA_SOFTPLUS)) {
        // the scan's step size, prepared once (an HBM-bound pass; done inside
        // the scan it would cost every state group of every channel the
        // softplus of its cells)
        void *buf = nullptr;
        const int st = get_aux_ws(dev, stream, 0, static_cast<size_t>(total) * sizeof(T) + 256, &buf);
        if (st != SSM2D_OK) return st;
        delta_prep_kernel<T><<<dim3(nblk), dim3(256), 0, s>>>(delta, delta_bias, static_cast<T *>(buf), total, H * W,
                                                                static_cast<int>(d_inner),
                                                                (flags & SSM2D_DELTA_SOFTPLUS) ? 1 : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
        delta = static_cast<const T *>(buf);
    }
    const int vf = (flags & SSM2D_VERTICAL_FIRST) ? kModeVFirst : 0;
    const int acc = (flags & SSM2D_ACCUMULATE) ? kModeAccumulate : 0;
    if (!(flags & SSM2D_FOUR_WAY)) {
        const int mode = ((flags & SSM2D_FLIP_W) ? kModeFlipW : 0) | vf | acc | (z ? kModeGate : 0);
        return launch(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, mode, (flags & SSM2D_FLIP_H) ? 1 : 0,
                      dev, stream, z, h_init, h_last);
    }
    // Four scans, one per starting corner, summed into y in stream order; the
    // skip term is added once, by the first.
    for (int q = 0; q < 4; ++q) {
        const int mode = ((q & 2) ? kModeFlipW : 0) | vf | (q == 0 ? acc : kModeAccumulate);
        const int st = launch(x, delta, A, B, C, q == 0 ? D : nullptr, y, batch, d_inner, d_state, H, W, mode,
                              q & 1, dev, stream);
        if (st != SSM2D_OK) return st;
    }
    if (z) {
        // the gate is linear in y: applied once to the sum
        gate_kernel<T><<<dim3(nblk), dim3(256), 0, s>>>(y, z, total);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    return SSM2D_OK;
}

// flags: SSM2D_FLIP_H / SSM2D_FLIP_W, the direction of the forward scan.
template <typename T>
int scan_bwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *dy, T *dx,
             T *ddelta, float *dA, T *dB, T *dC, float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
             int64_t W, void *stream, unsigned flags = 0)
{
    if ((flags & ~kKnownFlags) != 0 || (flags & (SSM2D_ACCUMULATE | SSM2D_FOUR_WAY | SSM2D_DELTA_SOFTPLUS)))
        return SSM2D_ERR_BAD_FLAGS;
    if (flags & SSM2D_VERTICAL_FIRST) return SSM2D_ERR_UNSUPPORTED;
    const bool f_h = (flags & SSM2D_FLIP_H) != 0, f_w = (flags & SSM2D_FLIP_W) != 0;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (d_inner == 0) return SSM2D_OK;
    if (d_state > SSM2D_MAX_STATE_BWD || H > SSM2D_MAX_SIDE || W > SSM2D_MAX_SIDE) return SSM2D_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t{1} << 31) - 1;
    const int64_t nstrips = (W + 3) / 4, pad = 4 * nstrips - W;
    const int64_t n_dblk = (d_inner + 7) / 8;
    int64_t npl = 1;
    while (npl * 8 < d_state) npl *= 2;
    const int64_t tiles = batch * n_dblk * nstrips * H;  // (chain, strip, row)
    if (batch * d_inner * H * W > lim || batch * d_state * H * W > lim || d_inner * d_state > lim)
        return SSM2D_ERR_UNSUPPORTED;
    const bool work = batch > 0 && H > 0 && W > 0;
    if ((!dA && d_state > 0) || !dD || (work && (!x || !delta || !D || !dy || !dx || !ddelta)) ||
        (work && d_state > 0 && (!A || !B || !C || !dB || !dC)))
        return SSM2D_ERR_NULLPTR;
    if (misaligned(x) || misaligned(delta) || misaligned(A) || misaligned(B) || misaligned(C) || misaligned(D) ||
        misaligned(dy) || misaligned(dx) || misaligned(ddelta) || misaligned(dA) || misaligned(dB) || misaligned(dC) ||
        misaligned(dD))
        return SSM2D_ERR_MISALIGNED;

    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(g_mutex);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t state_elems = work ? static_cast<size_t>(tiles) * npl * kWave * 4 : 0;
    const long part_stride = batch * d_state * H * 4 * nstrips;  // floats per channel block
    const size_t part_elems = work ? static_cast<size_t>(n_dblk) * part_stride : 0;
    void *ws = nullptr;
    if (work) {
        const int st = get_bwd_ws(dev, stream, (state_elems + 2 * part_elems) * sizeof(float) + 256, &ws);
        if (st != SSM2D_OK) return st;
    }
    float *states = static_cast<float *>(ws);
    {
        const long n = std::max<long>(d_inner * d_state, d_inner);
        bwd_prepare_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(dA, d_inner * d_state,
                                                                                            dD, d_inner);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    if (!work) return SSM2D_OK;

    BwdArgs bw{};
    bw.states = states;
    bw.pad = static_cast<int>(pad);
    bw.dy = dy;
    bw.ddelta = ddelta;
    bw.dBp = states + state_elems;
    bw.dCp = bw.dBp + part_elems;
    bw.dA = dA;
    bw.dD = dD;
    bw.part_stride = part_stride;
    const int bi = static_cast<int>(batch), di = static_cast<int>(d_inner), ni = static_cast<int>(d_state);
    const int hi = static_cast<int>(H), wi = static_cast<int>(W);
    const int align = (W % 4 == 0) ? 4 : ((W % 2 == 0) ? 2 : 1);
    // 1. the forward pass again, in its direction, storing every state
    Plan pf = make_plan(batch, d_inner, d_state, H, W, kModeStates | (f_w ? kModeFlipW : 0));
    pf.bw = &bw;
    pf.flip_h = f_h ? 1 : 0;
    choose_coop<T>(pf, H, align);
    if (pf.npl != npl || pf.n_dblk != n_dblk || pf.nstrips != nstrips) return SSM2D_ERR_UNSUPPORTED;
    int st = f_w ? dispatch_states_flipw(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pf, dev, stream, align)
                 : dispatch_states(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pf, dev, stream, align);
    if (st != SSM2D_OK) return st;
    // 2. the adjoint scans from the opposite corner, with every local
    // derivative (chains cut into several workgroups: the courier-free
    // kernels, which fit 8 strips per workgroup instead of 6)
    const int bmode = kModeBackward | (f_w ? 0 : kModeFlipW);
    Plan pb = make_plan(batch, d_inner, d_state, H, W, bmode);
    const bool edges = pb.groups > 1;
    if (edges) pb = make_plan(batch, d_inner, d_state, H, W, bmode | kModeEdges);
    pb.flip_h = f_h ? 0 : 1;
    pb.bw = &bw;
    choose_coop<T>(pb, H, align);
    if (pb.npl != npl || pb.n_dblk != n_dblk || pb.nstrips != nstrips) return SSM2D_ERR_UNSUPPORTED;
    if (f_w)
        st = edges ? dispatch_bwd_ltr_edges(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align)
                   : dispatch_bwd_ltr(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align);
    else
        st = edges ? dispatch_bwd_edges(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align)
                   : dispatch_bwd(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align);
    if (st != SSM2D_OK) return st;
    // 3. dB and dC: sums over the channel blocks
    if (d_state > 0) {
        const long total = batch * d_state * H * W;
        // (the partial rows start at column pad when the adjoint ran right to
        // left, at 0 when it ran left to right)
        bwd_reduce_kernel<T><<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
            bw.dBp, bw.dCp, part_stride, static_cast<int>(n_dblk), dB, dC, total, wi, static_cast<int>(4 * nstrips),
            f_w ? 0 : static_cast<int>(pad));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    return SSM2D_OK;
}

// Backward of the Mamba-option forward: the chain rule around scan_bwd (the
// gate and the step-size preparation are elementwise).
template <typename T>
int scan_bwd_mamba(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *z,
                   const float *delta_bias, const T *dy, T *dx, T *ddelta, float *dA, T *dB, T *dC, float *dD, T *dz,
                   float *ddelta_bias, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                   unsigned flags, void *stream)
{
    if ((flags & ~SSM2D_DELTA_SOFTPLUS) != 0) return SSM2D_ERR_BAD_FLAGS;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (d_inner == 0) return SSM2D_OK;
    if ((z && !dz) || (ddelta_bias && !delta_bias)) return SSM2D_ERR_NULLPTR;
    if (misaligned(z) || misaligned(dz) || misaligned(delta_bias) || misaligned(ddelta_bias)) return SSM2D_ERR_MISALIGNED;
    const bool prep = delta_bias || (flags & SSM2D_DELTA_SOFTPLUS);
    const long total = batch * d_inner * H * W;
    const unsigned nblk = static_cast<unsigned>((total + 255) / 256);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    if (ddelta_bias) {
        zero_kernel<<<dim3(static_cast<unsigned>((d_inner + 255) / 256)), dim3(256), 0, s>>>(ddelta_bias, d_inner);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    if (total == 0 || d_state > SSM2D_MAX_STATE_BWD)  // the backward reports sizes and zeroes dA, dD
        return scan_bwd<T>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                           stream);
    if (!x || !delta || !dy || !dx || !ddelta) return SSM2D_ERR_NULLPTR;
    void *ws1 = nullptr, *ws2 = nullptr, *ws3 = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        const size_t bytes = static_cast<size_t>(total) * sizeof(T) + 256;
        int st = prep ? get_aux_ws(dev, stream, 0, bytes, &ws1) : SSM2D_OK;
        if (st == SSM2D_OK && z) st = get_aux_ws(dev, stream, 1, bytes, &ws2);
        if (st == SSM2D_OK && z) st = get_aux_ws(dev, stream, 2, bytes, &ws3);
        if (st != SSM2D_OK) return st;
        if (prep) {
            delta_prep_kernel<T><<<dim3(nblk), dim3(256), 0, s>>>(delta, delta_bias, static_cast<T *>(ws1), total,
                                                                    H * W, static_cast<int>(d_inner),
                                                                    (flags & SSM2D_DELTA_SOFTPLUS) ? 1 : 0);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e);
        }
    }
    const T *dstep = prep ? static_cast<const T *>(ws1) : delta;
    const T *g = dy;
    if (z) {
        // the ungated scan output, then dz and the scan's upstream gradient
        T *y0 = static_cast<T *>(ws2);
        int st = scan_fwd<T>(x, dstep, A, B, C, D, y0, batch, d_inner, d_state, H, W, 0u, false, stream);
        if (st != SSM2D_OK) return st;
        gate_bwd_kernel<T><<<dim3(nblk), dim3(256), 0, s>>>(dy, y0, z, dz, static_cast<T *>(ws3), total);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
        g = static_cast<const T *>(ws3);
    }
    int st = scan_bwd<T>(x, dstep, A, B, C, D, g, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W, stream);
    if (st != SSM2D_OK) return st;
    if ((flags & SSM2D_DELTA_SOFTPLUS) || ddelta_bias) {
        step_bwd_kernel<T><<<dim3(static_cast<unsigned>(batch * d_inner)), dim3(256), 0, s>>>(
            ddelta, delta, delta_bias, ddelta_bias, H * W, static_cast<int>(d_inner),
            (flags & SSM2D_DELTA_SOFTPLUS) ? 1 : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    return SSM2D_OK;
}

}  // namespace

extern "C" {

int ssm2d_scan_fwd(const float *x, const float *delta, const float *A, const float *B, const float *C,
                   const float *D, float *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                   int64_t W, void *stream)
{
    return scan_fwd<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, 0u, false, stream);
}

int ssm2d_scan_fwd_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                        const uint16_t *C, const float *D, uint16_t *y, int64_t batch, int64_t d_inner,
                        int64_t d_state, int64_t H, int64_t W, void *stream)
{
    return scan_fwd<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, 0u, false, stream);
}

int ssm2d_scan_fwd_ex(const float *x, const float *delta, const float *A, const float *B, const float *C,
                      const float *D, float *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                      int64_t W, uint32_t flags, void *stream)
{
    return scan_fwd<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, true, stream);
}

int ssm2d_scan_fwd_ex_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                           const uint16_t *C, const float *D, uint16_t *y, int64_t batch, int64_t d_inner,
                           int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_fwd<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, true, stream);
}

int ssm2d_scan_fwd_mamba(const float *x, const float *delta, const float *A, const float *B, const float *C,
                         const float *D, const float *z, const float *delta_bias, const float *h_init,
                         float *h_last, float *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                         int64_t W, uint32_t flags, void *stream)
{
    return scan_fwd<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, true, stream, z, delta_bias,
                           h_init, h_last);
}

int ssm2d_scan_fwd_mamba_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                              const uint16_t *C, const float *D, const uint16_t *z, const float *delta_bias,
                              const float *h_init, float *h_last, uint16_t *y, int64_t batch, int64_t d_inner,
                              int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_fwd<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, true, stream, z,
                              delta_bias, h_init, h_last);
}

int ssm2d_scan_bwd(const float *x, const float *delta, const float *A, const float *B, const float *C,
                   const float *D, const float *dy, float *dx, float *ddelta, float *dA, float *dB, float *dC,
                   float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, void *stream)
{
    return scan_bwd<float>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W, stream);
}

int ssm2d_scan_bwd_ex(const float *x, const float *delta, const float *A, const float *B, const float *C,
                      const float *D, const float *dy, float *dx, float *ddelta, float *dA, float *dB, float *dC,
                      float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, uint32_t flags,
                      void *stream)
{
    return scan_bwd<float>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W, stream,
                           flags);
}

int ssm2d_scan_bwd_ex_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                           const uint16_t *C, const float *D, const uint16_t *dy, uint16_t *dx, uint16_t *ddelta,
                           float *dA, uint16_t *dB, uint16_t *dC, float *dD, int64_t batch, int64_t d_inner,
                           int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_bwd<uint16_t>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                              stream, flags);
}

int ssm2d_scan_bwd_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                        const uint16_t *C, const float *D, const uint16_t *dy, uint16_t *dx, uint16_t *ddelta,
                        float *dA, uint16_t *dB, uint16_t *dC, float *dD, int64_t batch, int64_t d_inner,
                        int64_t d_state, int64_t H, int64_t W, void *stream)
{
    return scan_bwd<uint16_t>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                              stream);
}

int ssm2d_scan_bwd_mamba(const float *x, const float *delta, const float *A, const float *B, const float *C,
                         const float *D, const float *z, const float *delta_bias, const float *dy, float *dx,
                         float *ddelta, float *dA, float *dB, float *dC, float *dD, float *dz, float *ddelta_bias,
                         int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, uint32_t flags,
                         void *stream)
{
    return scan_bwd_mamba<float>(x, delta, A, B, C, D, z, delta_bias, dy, dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                                 batch, d_inner, d_state, H, W, flags, stream);
}

int ssm2d_scan_bwd_mamba_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                              const uint16_t *C, const float *D, const uint16_t *z, const float *delta_bias,
                              const uint16_t *dy, uint16_t *dx, uint16_t *ddelta, float *dA, uint16_t *dB,
                              uint16_t *dC, float *dD, uint16_t *dz, float *ddelta_bias, int64_t batch,
                              int64_t d_inner, int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_bwd_mamba<uint16_t>(x, delta, A, B, C, D, z, delta_bias, dy, dx, ddelta, dA, dB, dC, dD, dz,
                                    ddelta_bias, batch, d_inner, d_state, H, W, flags, stream);
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
    case SSM2D_ERR_BAD_FLAGS:
        return "unknown flag bits, SSM2D_FOUR_WAY with a flip flag or carried states, or a gate with SSM2D_ACCUMULATE";
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

int ssm2d_version(void) { return 300; }

const char *ssm2d_last_hip_error(void)
{
    return hipGetErrorString(static_cast<hipError_t>(g_last_hip_error.load()));
}

}  // extern "C"

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

// k_want = 8: 8-column strips wherever the mode allows them (the plain
// forward's choice for long chains across workgroups, below).
Plan make_plan(int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, int mode, int k_want = 0)
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
    else if (k_want == 8 && wide_ok) pl.K = 8;
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


std::recursive_mutex g_mutex;  // (entry points call one another on the widened bf16 paths)
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

// Zeroes n16 16-byte words (a kernel rather than a memset node, so that a
// caller capturing a graph records nothing the replays could misapply).
__global__ void fill_zero_kernel(uint4 *p, long n16)
{
    for (long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; t < n16;
         t += static_cast<long>(gridDim.x) * blockDim.x)
        p[t] = make_uint4(0u, 0u, 0u, 0u);
}

// dst = src, or zeros where src is null (n floats).
__global__ void copy_or_zero_kernel(const float *src, float *dst, long n)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < n) dst[t] = src ? src[t] : 0.0f;
}

int zero_async(void *p, size_t bytes, hipStream_t s)
{
    const long n16 = static_cast<long>((bytes + 15) / 16);
    if (n16 == 0) return SSM2D_OK;
    const long blocks = std::min<long>((n16 + 255) / 256, 4096);
    fill_zero_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(static_cast<uint4 *>(p), n16);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSM2D_OK : hip_fail(e);
}

// Device memory in stream order: allocated and freed on the caller's stream
// (no host wait; a buffer being replaced is released after the work queued
// before it). Sizes are rounded up to 16 bytes.
int alloc_async(void **p, size_t bytes, hipStream_t s)
{
    *p = nullptr;
    if (hipMallocAsync(p, (bytes + 15) & ~size_t{15}, s) != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        return SSM2D_ERR_NOMEM;
    }
    return SSM2D_OK;
}
void free_async(void *p, hipStream_t s)
{
    if (p) (void)hipFreeAsync(p, s);
}

void free_ws(WsEntry &e, hipStream_t s)
{
    free_async(e.head, s);
    free_async(e.gring, s);
    free_async(e.zeros, s);
    unsigned int *herr = e.herr;
    e = WsEntry{};
    e.herr = herr;  // the flag stays with the (device, stream)
}

// Workspace for (device, stream), grown when needed: the old buffers are
// released in stream order, the new ones zeroed by a kernel on the stream
// (tags are never zero, so no zero word matches). The host-visible timeout
// flag is pinned host memory, mapped for the device, allocated once.
int get_ws(int dev, void *stream, size_t gring_bytes, size_t zero_bytes, size_t cons_count, WsEntry **out)
{
    WsEntry &e = g_ws[{dev, stream}];
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (!e.herr) {
        void *h = nullptr;
        if (hipHostMalloc(&h, 64, hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess && h) {
            std::memset(h, 0, 64);
            e.herr = static_cast<unsigned int *>(h);
        } else {
            (void)hipGetLastError();  // no flag: timeouts are reported by ssm2d_sync_check only
        }
    }
    if (e.head && gring_bytes <= e.gring_bytes && zero_bytes <= e.zero_bytes && cons_count <= e.cons_count) {
        *out = &e;
        return SSM2D_OK;
    }
    if (e.head) free_ws(e, s);
    size_t gb = std::max(gring_bytes, size_t{256});
    size_t zb = std::max(zero_bytes, size_t{256});
    size_t cc = std::max(cons_count, size_t{1});
    size_t head = kHeadBytes + kSinkBytes + cc * sizeof(unsigned long long);
    void *h = nullptr, *g = nullptr, *z = nullptr;
    if (alloc_async(&h, head, s) != SSM2D_OK || alloc_async(&g, gb, s) != SSM2D_OK ||
        alloc_async(&z, zb, s) != SSM2D_OK) {
        free_async(h, s);
        free_async(g, s);
        return SSM2D_ERR_NOMEM;
    }
    int st = zero_async(h, head, s);
    if (st == SSM2D_OK) st = zero_async(g, gb, s);
    if (st == SSM2D_OK) st = zero_async(z, zb, s);
    if (st != SSM2D_OK) {
        free_async(h, s);
        free_async(g, s);
        free_async(z, s);
        return st;
    }
    e.head = static_cast<unsigned int *>(h);
    e.gring = static_cast<unsigned long long *>(g);
    e.zeros = z;
    e.gring_bytes = (gb / 8) * 8;
    e.zero_bytes = zb;
    e.cons_count = cc;
    *out = &e;
    return SSM2D_OK;
}

// A timeout reported by a kernel of an earlier call on (device, stream)
// (the host-mapped flag, read without waiting): consumed, and reported once.
bool take_timeout_flag(int dev, void *stream)
{
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || !it->second.herr) return false;
    unsigned int *f = it->second.herr;
    if (__atomic_load_n(f, __ATOMIC_ACQUIRE) == 0u) return false;
    __atomic_store_n(f, 0u, __ATOMIC_RELEASE);
    return true;
}

// ---------------------------------------------------------------- backward

// Buffers per (device, stream, slot) in stream order, grown when needed
// (the old buffer is released after the work queued before it, the new one
// optionally zeroed by a kernel on the stream). Slots: kSlotBwd holds the
// backward's stored states and channel-block sums; the others are scratch
// tensors of the option and widening passes.
struct Buf {
    void *buf = nullptr;
    size_t bytes = 0;
};
std::map<std::pair<std::pair<int, void *>, int>, Buf> g_bufs;
constexpr int kSlotBwd = -1;

int get_buf(int dev, void *stream, int slot, size_t bytes, bool zero, void **out)
{
    Buf &e = g_bufs[{{dev, stream}, slot}];
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (e.buf && bytes <= e.bytes) {
        *out = e.buf;
        return SSM2D_OK;
    }
    if (e.buf) {
        free_async(e.buf, s);
        e = Buf{};
    }
    void *b = nullptr;
    int st = alloc_async(&b, bytes, s);
    if (st == SSM2D_OK && zero) st = zero_async(b, bytes, s);
    if (st != SSM2D_OK) {
        free_async(b, s);
        return st;
    }
    e.buf = b;
    e.bytes = bytes;
    *out = b;
    return SSM2D_OK;
}
int get_bwd_ws(int dev, void *stream, size_t bytes, void **out) { return get_buf(dev, stream, kSlotBwd, bytes, true, out); }
int get_aux_ws(int dev, void *stream, int slot, size_t bytes, void **out)
{
    return get_buf(dev, stream, slot, bytes, false, out);
}

// Zeroes dA and dD (the backward adds into them).
__global__ void bwd_prepare_kernel(float *dA, long n_a, float *dD, long n_d)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < n_a) dA[t] = 0.0f;
    if (t < n_d) dD[t] = 0.0f;
}

// States [n0, n0 + nc) of an [outer][N][inner] tensor to an [outer][nc][inner]
// one, or back (scatter).
template <typename T>
__global__ void state_slice_kernel(const T *src, T *dst, long outer, long N, long n0, long nc, long inner, int scatter)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= outer * nc * inner) return;
    const long i = t % inner, j = (t / inner) % nc, o = t / (inner * nc);
    const long full = (o * N + n0 + j) * inner + i;
    if (scatter) dst[full] = src[t];
    else dst[t] = src[full];
}

template <typename T>
int state_slice(const T *src, T *dst, long outer, long N, long n0, long nc, long inner, bool scatter, hipStream_t s)
{
    const long n = outer * nc * inner;
    if (n == 0) return SSM2D_OK;
    state_slice_kernel<T><<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(src, dst, outer, N, n0, nc,
                                                                                           inner, scatter ? 1 : 0);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSM2D_OK : hip_fail(e);
}

__global__ void add_into_kernel(float *dst, const float *src, long n)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < n) dst[t] += src[t];
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

__device__ __forceinline__ float get(const float *p) { return *p; }
__device__ __forceinline__ float get(const uint16_t *p) { return __uint_as_float(static_cast<unsigned>(*p) << 16); }

// Step size of the scan: delta + bias[d], through softplus if asked, computed
// in fp32 and stored as TO (the scan's input type, or fp32 for the widened
// bf16 paths). softplus(v) = max(v, 0) + log1p(e^-|v|).
template <typename TI, typename TO>
__global__ void delta_prep_kernel(const TI *delta, const float *bias, TO *out, long total, long hw, int d_inner,
                                  int use_softplus)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    float v = get(delta + t);
    if (bias) v += bias[(t / hw) % d_inner];
    if (use_softplus) v = fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));
    put(out + t, v);
}

// bf16 -> fp32, exact.
__global__ void widen_kernel(const uint16_t *in, float *out, long total)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < total) out[t] = get(in + t);
}

// out = in * SiLU(z) (z may be null: no gate), rounded once to out's type.
template <typename TI, typename TO>
__global__ void gate_kernel(const TI *in, const TO *z, TO *out, long total)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= total) return;
    float v = get(in + t);
    if (z) {
        const float zf = get(z + t);
        v *= zf / (1.0f + expf(-zf));
    }
    put(out + t, v);
}

// Backward of the gate: dz = dy * y * SiLU'(z), and the scan's upstream
// gradient dy * SiLU(z) (held as TY: fp32 on the widened bf16 path);
// SiLU'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z).
template <typename T, typename TY>
__global__ void gate_bwd_kernel(const T *dy, const TY *y, const T *z, T *dz, TY *dys, long total)
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
// unchanged), read from gin (TG) and written to gout (T; may be gin), and
// d bias[d] += the map's sum of d delta.
template <typename TG, typename T>
__global__ void step_bwd_kernel(const TG *gin, T *gout, const T *delta, const float *bias, float *dbias, long hw,
                                int d_inner, int use_softplus)
{
    __shared__ float part[256];
    const long map = blockIdx.x;
    const int d = static_cast<int>(map % d_inner);
    const float bd = bias ? bias[d] : 0.0f;
    float acc = 0.0f;
    for (long p = threadIdx.x; p < hw; p += blockDim.x) {
        const long t = map * hw + p;
        float g = get(gin + t);
        if (use_softplus) g *= 1.0f / (1.0f + expf(-(get(delta + t) + bd)));
        put(gout + t, g);
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

// out[m][j][i] = in[m][i][j] for `maps` maps of H x W cells: 64 x 64 tiles
// through LDS, so that both the reads and the writes run along rows.
template <typename T>
__global__ void transpose_kernel(const T *in, T *out, long maps, int H, int W)
{
    __shared__ T tile[64][65];
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;  // 256 threads: 64 x 4
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    const long hw = static_cast<long>(H) * W;
    for (long m = blockIdx.z; m < maps; m += gridDim.z) {
        const T *src = in + m * hw;
        T *dst = out + m * hw;
        for (int r = ty; r < 64; r += 4) {
            const int i = i0 + r, j = j0 + tx;
            if (i < H && j < W) tile[r][tx] = src[static_cast<long>(i) * W + j];
        }
        __syncthreads();
        for (int r = ty; r < 64; r += 4) {
            const int j = j0 + r, i = i0 + tx;
            if (j < W && i < H) dst[static_cast<long>(j) * H + i] = tile[tx][r];
        }
        __syncthreads();
    }
}

template <typename T>
int transpose_maps(const T *in, T *out, long maps, long H, long W, hipStream_t s)
{
    if (maps == 0 || H == 0 || W == 0) return SSM2D_OK;
    const dim3 grid(static_cast<unsigned>((W + 63) / 64), static_cast<unsigned>((H + 63) / 64),
                    static_cast<unsigned>(std::min<long>(maps, 65535)));
    transpose_kernel<T><<<grid, dim3(256), 0, s>>>(in, out, maps, static_cast<int>(H), static_cast<int>(W));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSM2D_OK : hip_fail(e);
}

int widen(const uint16_t *in, float *out, long total, hipStream_t s)
{
    if (total == 0) return SSM2D_OK;
    widen_kernel<<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(in, out, total);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSM2D_OK : hip_fail(e);
}

template <typename TI, typename TO>
int gate_or_round(const TI *in, const TO *z, TO *out, long total, hipStream_t s)
{
    if (total == 0) return SSM2D_OK;
    gate_kernel<TI, TO><<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(in, z, out, total);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSM2D_OK : hip_fail(e);
}

__global__ void zero_kernel(float *p, long n)
{
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t < n) p[t] = 0.0f;
}

// ---------------------------------------------------------------- static scratch

// Workspace of ssm2d_scan_fwd_noalloc: a static device array (each GPU the
// library runs on holds its own copy until the process ends). Its layout
// follows the scan workspace: head words, sink and up to kScratchCons
// consumer words; the zero page; the global carry ring in the rest.
constexpr size_t kScratchBytes = size_t{16} << 20;
constexpr size_t kScratchHead = size_t{64} << 10;
constexpr size_t kScratchZeros = size_t{1} << 20;
constexpr size_t kScratchCons = (kScratchHead - kHeadBytes - kSinkBytes) / sizeof(unsigned long long);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::map<int, WsEntry> g_scratch;  // per device: views of that device's copy (its address from the runtime)

// The scratch workspace of device `dev` (current). On the first call on a
// device its address is looked up (the array's name is a host-side stand-in,
// not a device address) and the array is zeroed on `s`.
int scratch_ws(int dev, hipStream_t s, const WsEntry **out)
{
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!ptr) return SSM2D_ERR_HIP;
        const int st = zero_async(ptr, kScratchBytes, s);
        if (st != SSM2D_OK) return st;
        WsEntry w{};
        unsigned char *base = static_cast<unsigned char *>(ptr);
        w.head = reinterpret_cast<unsigned int *>(base);
        w.zeros = base + kScratchHead;
        w.gring = reinterpret_cast<unsigned long long *>(base + kScratchHead + kScratchZeros);
        w.gring_bytes = kScratchBytes - kScratchHead - kScratchZeros;
        w.zero_bytes = kScratchZeros;
        w.cons_count = kScratchCons;
        w.herr = nullptr;  // (nothing is allocated: timeouts show as NaN outputs and in ssm2d_sync_check)
        it = g_scratch.emplace(dev, w).first;
    }
    *out = &it->second;
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

// Rows of a multiple of 4, 2 or 1 columns (the widest vector loads a row takes).
inline int row_align(int64_t W)
{
    return (W % 4 == 0) ? 4 : ((W % 2 == 0) ? 2 : 1);
}

// Whether a launch runs in the two-rows-per-step kernel; if so, pl becomes
// its plan. By default that is the plain forward of plans whose chains span
// workgroups (there it beats the general kernel: one handshake per two rows
// against the couriers' and the shared ring's latencies). Chains held in one
// workgroup stay on the general kernel, faster there as measured (VMamba
// stage 1: 159 us against 168 us in 8-column and 174 us in 4-column strips);
// SSM2D_FAST=2 runs them in the two-rows-per-step kernel too, trying first
// a chain of up to 16 4-column strips where the general plan widens the
// strips to 8 columns.
template <typename T>
bool takes_fast(Plan &pl, int64_t W, int align)
{
    const int fast = env_int("SSM2D_FAST", 1);
    if (pl.mode != 0 || fast <= 0) return false;
    if (pl.groups == 1 && fast < 2) return false;
    if (pl.K == 8 && pl.groups == 1 && env_int("SSM2D_STRIP", 0) != 8) {
        Plan p4 = pl;
        p4.K = 4;
        p4.nstrips = static_cast<int>((W + 3) / 4);
        p4.s_local = p4.nstrips;
        p4.total_wg = p4.n_chains;
        if (fast_path_taken<T>(p4, align)) {
            pl = p4;
            return true;
        }
    }
    return fast_path_taken<T>(pl, align);
}

// The plan of a forward launch. For the plain forward of chains cut into
// several workgroups, 8-column strips (4 a workgroup with two couriers, one
// compute wave a SIMD) in the two-rows-per-step kernel where that plan still
// gives the chip 256 workgroups: half the strips a chain, so half the carry
// hops, at the same work a SIMD (giga-pixel map: 270 us against 276-281 us
// for 4-column strips, two compute waves a SIMD). Narrower maps keep 4-column
// strips (with 8-column ones their chains would fill only part of the chip).
// `carries`: a gate or carried states, which the two-rows-per-step kernel
// does not take.
template <typename T>
Plan forward_plan(int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, int mode, bool carries)
{
    Plan pl = make_plan(batch, d_inner, d_state, H, W, mode);
    if (mode != 0 || carries || pl.groups <= 1 || pl.K != 4 || env_int("SSM2D_STRIP", 0) != 0) return pl;
    Plan p8 = make_plan(batch, d_inner, d_state, H, W, mode, 8);
    if (p8.K == 8 && p8.groups > 1 && p8.total_wg >= 256 && fast_path_taken<T>(p8, row_align(W))) return p8;
    return pl;
}

// Whether a launch runs in the whole-row kernel for narrow maps: the plain
// forward (rows in either direction, no gate or carried states) of rows of at
// most 16 columns with at most 16 states. There one wave of 16 channels does
// a whole row, against a chain of up to four strip waves handing the row's
// carry on in the general kernel; taken when the map is short or the batch
// gives at least 256 such waves (one a CU), else the general kernel's strips
// spread a few tall maps over more waves. SSM2D_NARROW=0 never takes it,
// SSM2D_NARROW=2 always where it applies.
inline bool takes_narrow(int mode, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                         bool carries, int elem_bytes)
{
    const int env = env_int("SSM2D_NARROW", 1);
    if (env <= 0 || mode != 0 || carries || W > 16 || d_state > 16) return false;
    // its buffer offsets are 32-bit: every tensor under 2^31 bytes
    const int64_t limit = int64_t{1} << 31;
    if (batch * d_inner * H * W * elem_bytes >= limit || batch * d_state * H * W * elem_bytes >= limit) return false;
    return env >= 2 || H <= 128 || batch * ((d_inner + 15) / 16) >= 256;
}

template <typename T>
int launch(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y, int64_t batch,
           int64_t d_inner, int64_t d_state, int64_t H, int64_t W, int mode, int flip_h, int dev, void *stream,
           const T *z = nullptr, const float *h_init = nullptr, float *h_last = nullptr,
           const WsEntry *fixed_ws = nullptr, const float *hh_init = nullptr, float *hh_last = nullptr)
{
    if (hh_init || hh_last) mode |= kModeRowCarry;
    if (takes_narrow(mode, batch, d_inner, d_state, H, W, z || h_init || h_last, static_cast<int>(sizeof(T))))
        return dispatch_narrow(x, delta, A, B, C, D, y, static_cast<int>(batch), static_cast<int>(d_inner),
                               static_cast<int>(d_state), static_cast<int>(H), static_cast<int>(W), flip_h, stream);
    Plan pl = forward_plan<T>(batch, d_inner, d_state, H, W, mode, z || h_init || h_last || hh_init || hh_last);
    pl.flip_h = flip_h;
    pl.z = z;
    pl.h_init = h_init;
    pl.h_last = h_last;
    pl.hh_init = hh_init;
    pl.hh_last = hh_last;
    pl.fixed_ws = fixed_ws;
    const int bi = static_cast<int>(batch), di = static_cast<int>(d_inner), ni = static_cast<int>(d_state);
    const int hi = static_cast<int>(H), wi = static_cast<int>(W);
    const int align = row_align(W);
    choose_coop<T>(pl, H, align);
#define SSM2D_ARGS x, delta, A, B, C, D, y, bi, di, ni, hi, wi, pl, dev, stream, align
    constexpr int FW = kModeFlipW, VF = kModeVFirst, AC = kModeAccumulate;
    if (takes_fast<T>(pl, W, align)) {
        // the plain forward: two rows per step, where the plan's layout has that kernel
        const int st = dispatch_fast(SSM2D_ARGS);
        if (st != kNoFastPath) return st;
    }
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
    case kModeRowCarry: return dispatch_rowc(SSM2D_ARGS);
    case kModeRowCarry | FW: return dispatch_rowc_flipw(SSM2D_ARGS);
    case kModeRowCarry | VF: return dispatch_rowc_vfirst(SSM2D_ARGS);
    case kModeRowCarry | FW | VF: return dispatch_rowc_flipw_vfirst(SSM2D_ARGS);
    default: return SSM2D_ERR_UNSUPPORTED;
    }
#undef SSM2D_ARGS
}

constexpr unsigned kKnownFlags = SSM2D_FLIP_H | SSM2D_FLIP_W | SSM2D_VERTICAL_FIRST | SSM2D_ACCUMULATE | SSM2D_FOUR_WAY |
                                 SSM2D_DELTA_SOFTPLUS;

// Scratch slots of the widened bf16 paths (tensors shaped like x or B, fp32).
enum : int {
    kSlotStep = 0, kSlotY0 = 1, kSlotG = 2,
    kSlotX32 = 3, kSlotD32 = 4, kSlotB32 = 5, kSlotC32 = 6, kSlotY32 = 7, kSlotG32 = 8,
    kSlotDX32 = 9, kSlotDD32 = 10, kSlotDB32 = 11, kSlotDC32 = 12,
    kSlotT0 = 13,  // 13 .. 21: the transposed tensors of the vertical-first backward
    kSlotK0 = 22   // 22 .. 37: the state chunks of a backward with more than 32 states
};

template <typename T>
int scan_fwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
             int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, unsigned flags, bool extended,
             void *stream, const T *z = nullptr, const float *delta_bias = nullptr, const float *h_init = nullptr,
             float *h_last = nullptr, const float *hh_init = nullptr, float *hh_last = nullptr);

// bf16 calls whose result is more than one scan's rounded output (the
// four-corner sums) or whose scan runs on a computed step size (bias,
// softplus): x, B, C are widened to fp32 (exactly), the step size is computed
// and kept in fp32, the fp32 scans produce the result in an fp32 tensor, and
// that is rounded to bf16 once (times SiLU(z) when gated).
int scan_fwd_widened(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B, const uint16_t *C,
                     const float *D, uint16_t *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                     int64_t W, unsigned flags, void *stream, const uint16_t *z, const float *delta_bias,
                     const float *h_init, float *h_last, int dev,
                     const float *hh_init, float *hh_last)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long total = batch * d_inner * H * W, tb = batch * d_state * H * W;
    void *bx = nullptr, *bd = nullptr, *bb = nullptr, *bc = nullptr, *by = nullptr;
    const size_t ebytes = static_cast<size_t>(total) * 4 + 256, bbytes = static_cast<size_t>(tb) * 4 + 256;
    int st = get_aux_ws(dev, stream, kSlotX32, ebytes, &bx);
    if (st == SSM2D_OK) st = get_aux_ws(dev, stream, kSlotD32, ebytes, &bd);
    if (st == SSM2D_OK) st = get_aux_ws(dev, stream, kSlotB32, bbytes, &bb);
    if (st == SSM2D_OK) st = get_aux_ws(dev, stream, kSlotC32, bbytes, &bc);
    if (st == SSM2D_OK) st = get_aux_ws(dev, stream, kSlotY32, ebytes, &by);
    if (st != SSM2D_OK) return st;
    float *x32 = static_cast<float *>(bx), *d32 = static_cast<float *>(bd), *B32 = static_cast<float *>(bb);
    float *C32 = static_cast<float *>(bc), *y32 = static_cast<float *>(by);
    if ((st = widen(x, x32, total, s)) != SSM2D_OK) return st;
    delta_prep_kernel<uint16_t, float><<<dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s>>>(
        delta, delta_bias, d32, total, H * W, static_cast<int>(d_inner), (flags & SSM2D_DELTA_SOFTPLUS) ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    if (d_state > 0) {
        if ((st = widen(B, B32, tb, s)) != SSM2D_OK) return st;
        if ((st = widen(C, C32, tb, s)) != SSM2D_OK) return st;
    }
    if ((flags & SSM2D_ACCUMULATE) && (st = widen(y, y32, total, s)) != SSM2D_OK) return st;
    st = scan_fwd<float>(x32, d32, A, d_state ? B32 : nullptr, d_state ? C32 : nullptr, D, y32, batch, d_inner,
                         d_state, H, W, flags & ~SSM2D_DELTA_SOFTPLUS, true, stream, nullptr, nullptr, h_init, h_last,
                         hh_init, hh_last);
    if (st != SSM2D_OK) return st;
    return gate_or_round<float, uint16_t>(y32, z, y, total, s);
}

// Argument checks of the forward entry points (`extended`: the flag-taking
// ones, where D may be NULL). SSM2D_OK with *work == false: nothing to do.
template <typename T>
int check_fwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *y,
              int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, unsigned flags, bool extended,
              const T *z, const float *delta_bias, const float *h_init, const float *h_last, bool *work,
              const float *hh_init = nullptr, const float *hh_last = nullptr)
{
    *work = false;
    if ((flags & ~kKnownFlags) != 0) return SSM2D_ERR_BAD_FLAGS;
    if ((flags & SSM2D_FOUR_WAY) && (flags & (SSM2D_FLIP_H | SSM2D_FLIP_W))) return SSM2D_ERR_BAD_FLAGS;
    if (z && (flags & SSM2D_ACCUMULATE)) return SSM2D_ERR_BAD_FLAGS;
    if ((h_init || h_last) && (flags & SSM2D_FOUR_WAY)) return SSM2D_ERR_BAD_FLAGS;
    // carried horizontal states: plain (not accumulated, not gated) single scans
    if ((hh_init || hh_last) && (z || (flags & (SSM2D_FOUR_WAY | SSM2D_ACCUMULATE)))) return SSM2D_ERR_BAD_FLAGS;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (batch == 0 || d_inner == 0 || H == 0 || W == 0) return SSM2D_OK;
    if (d_state > SSM2D_MAX_STATE || H > SSM2D_MAX_SIDE || W > SSM2D_MAX_SIDE) return SSM2D_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t{1} << 31) - 1;
    if (batch * d_inner * H * W > lim || batch * d_state * H * W > lim || d_inner * d_state > lim)
        return SSM2D_ERR_UNSUPPORTED;
    if (!x || !delta || (!D && !extended) || !y || (d_state > 0 && (!A || !B || !C))) return SSM2D_ERR_NULLPTR;
    if (misaligned(x) || misaligned(delta) || misaligned(D) || misaligned(y) || misaligned(z) ||
        misaligned(delta_bias) || misaligned(h_init) || misaligned(h_last) || misaligned(hh_init) ||
        misaligned(hh_last) ||
        (d_state > 0 && (misaligned(A) || misaligned(B) || misaligned(C))))
        return SSM2D_ERR_MISALIGNED;
    *work = true;
    return SSM2D_OK;
}

// `extended`: the flag-taking entry points, where D may be NULL (no skip term).
// z (gate) and delta_bias come with the Mamba-option entry points only.
template <typename T>
int scan_fwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
             int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, unsigned flags, bool extended,
             void *stream, const T *z, const float *delta_bias, const float *h_init, float *h_last,
             const float *hh_init, float *hh_last)
{
    bool work = false;
    const int chk = check_fwd(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, extended, z, delta_bias,
                              h_init, h_last, &work, hh_init, hh_last);
    if (chk != SSM2D_OK || !work) return chk;

    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    if (take_timeout_flag(dev, stream)) return SSM2D_ERR_DEVICE_TIMEOUT;
    if constexpr (std::is_same<T, uint16_t>::value) {
        if ((flags & SSM2D_FOUR_WAY) || delta_bias || (flags & SSM2D_DELTA_SOFTPLUS))
            return scan_fwd_widened(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, stream, z,
                                    delta_bias, h_init, h_last, dev, hh_init, hh_last);
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long total = batch * d_inner * H * W;
    const unsigned nblk = static_cast<unsigned>((total + 255) / 256);
    if (delta_bias || (flags & SSM2D_DELTA_SOFTPLUS)) {
        // (fp32 only, see above) the scan's step size, prepared once (an
        // HBM-bound pass; done inside the scan it would cost every state
        // group of every channel the softplus of its cells)
        void *buf = nullptr;
        const int st = get_aux_ws(dev, stream, kSlotStep, static_cast<size_t>(total) * sizeof(T) + 256, &buf);
        if (st != SSM2D_OK) return st;
        delta_prep_kernel<T, T><<<dim3(nblk), dim3(256), 0, s>>>(delta, delta_bias, static_cast<T *>(buf), total,
                                                                  H * W, static_cast<int>(d_inner),
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
                      dev, stream, z, h_init, h_last, nullptr, hh_init, hh_last);
    }
    // (fp32 only) four scans, one per starting corner, summed into y in
    // stream order; the skip term is added once, by the first.
    for (int q = 0; q < 4; ++q) {
        const int mode = ((q & 2) ? kModeFlipW : 0) | vf | (q == 0 ? acc : kModeAccumulate);
        const int st = launch(x, delta, A, B, C, q == 0 ? D : nullptr, y, batch, d_inner, d_state, H, W, mode,
                              q & 1, dev, stream);
        if (st != SSM2D_OK) return st;
    }
    // the gate is linear in y: applied once to the sum
    if (z) return gate_or_round<T, T>(y, z, y, total, s);
    return SSM2D_OK;
}

template <typename T>
int scan_bwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *dy, T *dx,
             T *ddelta, float *dA, T *dB, T *dC, float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
             int64_t W, void *stream, unsigned flags = 0, const float *h_init = nullptr, const float *dh_last = nullptr,
             float *dh_init = nullptr, const float *hh_init = nullptr, const float *dhh_last = nullptr,
             float *dhh_init = nullptr);

// Backward of the vertical-first order: that scan is the horizontal-first
// scan of the transposed maps (the column recurrence becomes the row
// recurrence), with the two flips trading places, so its gradients are the
// transposed maps' gradients, transposed back. dA and dD need no transpose.
// Carried states trade places there: the vertical-first scan's state carried
// down its columns is the transposed map's row state, and the other way round
// (both arrays keep their layout).
template <typename T>
int scan_bwd_vfirst(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *dy,
                    T *dx, T *ddelta, float *dA, T *dB, T *dC, float *dD, int64_t batch, int64_t d_inner,
                    int64_t d_state, int64_t H, int64_t W, void *stream, unsigned flags, int dev, const float *h_init,
                    const float *dh_last, float *dh_init, const float *hh_init, const float *dhh_last, float *dhh_init)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long me = batch * d_inner, mb = batch * d_state;
    const size_t eb = static_cast<size_t>(me * H * W) * sizeof(T) + 256, bb = static_cast<size_t>(mb * H * W) * sizeof(T) + 256;
    void *buf[9] = {};
    const size_t sizes[9] = {eb, eb, bb, bb, eb, eb, eb, bb, bb};
    for (int k = 0; k < 9; ++k) {
        const int st = get_aux_ws(dev, stream, kSlotT0 + k, sizes[k], &buf[k]);
        if (st != SSM2D_OK) return st;
    }
    T *xt = static_cast<T *>(buf[0]), *dt = static_cast<T *>(buf[1]), *Bt = static_cast<T *>(buf[2]);
    T *Ct = static_cast<T *>(buf[3]), *dyt = static_cast<T *>(buf[4]), *dxt = static_cast<T *>(buf[5]);
    T *ddt = static_cast<T *>(buf[6]), *dBt = static_cast<T *>(buf[7]), *dCt = static_cast<T *>(buf[8]);
    int st = SSM2D_OK;
    if ((st = transpose_maps(x, xt, me, H, W, s)) != SSM2D_OK) return st;
    if ((st = transpose_maps(delta, dt, me, H, W, s)) != SSM2D_OK) return st;
    if ((st = transpose_maps(dy, dyt, me, H, W, s)) != SSM2D_OK) return st;
    if (d_state > 0) {
        if ((st = transpose_maps(B, Bt, mb, H, W, s)) != SSM2D_OK) return st;
        if ((st = transpose_maps(C, Ct, mb, H, W, s)) != SSM2D_OK) return st;
    }
    const unsigned tflags = ((flags & SSM2D_FLIP_H) ? SSM2D_FLIP_W : 0u) | ((flags & SSM2D_FLIP_W) ? SSM2D_FLIP_H : 0u);
    st = scan_bwd<T>(xt, dt, A, d_state ? Bt : nullptr, d_state ? Ct : nullptr, D, dyt, dxt, ddt, dA,
                     d_state ? dBt : nullptr, d_state ? dCt : nullptr, dD, batch, d_inner, d_state, W, H, stream,
                     tflags, hh_init, dhh_last, dhh_init, h_init, dh_last, dh_init);
    if (st != SSM2D_OK) return st;
    if ((st = transpose_maps(dxt, dx, me, W, H, s)) != SSM2D_OK) return st;
    if ((st = transpose_maps(ddt, ddelta, me, W, H, s)) != SSM2D_OK) return st;
    if (d_state > 0) {
        if ((st = transpose_maps(dBt, dB, mb, W, H, s)) != SSM2D_OK) return st;
        if ((st = transpose_maps(dCt, dC, mb, W, H, s)) != SSM2D_OK) return st;
    }
    return SSM2D_OK;
}

// More than SSM2D_MAX_STATE_BWD states (fp32): the states' recurrences are
// independent and y sums over them, so the backward runs on chunks of at most
// that many states, gathered into scratch tensors, and adds the chunks' dx
// and d delta; the skip term's gradients come from the first chunk alone (the
// others get D = 0 and their dD is dropped). dA, dB, dC and the carried
// states' gradients are scattered back by state.
int scan_bwd_chunked(const float *x, const float *delta, const float *A, const float *B, const float *C,
                     const float *D, const float *dy, float *dx, float *ddelta, float *dA, float *dB, float *dC,
                     float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, void *stream,
                     unsigned flags, const float *h_init, const float *dh_last, float *dh_init, const float *hh_init,
                     const float *dhh_last, float *dhh_init, int dev)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const long CH = SSM2D_MAX_STATE_BWD, HW = H * W, BD = batch * d_inner;
    const size_t fs = sizeof(float);
    // scratch: A, B, C, dA, dB, dC of a chunk; dx, d delta of the later
    // chunks; a zero D and a dropped dD; the carried states of a chunk
    const size_t sizes[16] = {static_cast<size_t>(d_inner * CH) * fs, static_cast<size_t>(batch * CH * HW) * fs,
                              static_cast<size_t>(batch * CH * HW) * fs, static_cast<size_t>(d_inner * CH) * fs,
                              static_cast<size_t>(batch * CH * HW) * fs, static_cast<size_t>(batch * CH * HW) * fs,
                              static_cast<size_t>(BD * HW) * fs, static_cast<size_t>(BD * HW) * fs,
                              static_cast<size_t>(d_inner) * fs, static_cast<size_t>(d_inner) * fs,
                              static_cast<size_t>(BD * CH * W) * fs, static_cast<size_t>(BD * CH * W) * fs,
                              static_cast<size_t>(BD * CH * W) * fs, static_cast<size_t>(BD * CH * H) * fs,
                              static_cast<size_t>(BD * CH * H) * fs, static_cast<size_t>(BD * CH * H) * fs};
    float *w[16] = {};
    for (int k = 0; k < 16; ++k) {
        void *v = nullptr;
        const int st = get_aux_ws(dev, stream, kSlotK0 + k, sizes[k] + 256, &v);
        if (st != SSM2D_OK) return st;
        w[k] = static_cast<float *>(v);
    }
    float *Ac = w[0], *Bc = w[1], *Cc = w[2], *dAc = w[3], *dBc = w[4], *dCc = w[5], *dxc = w[6], *ddc = w[7];
    float *zD = w[8], *dDc = w[9], *h0c = w[10], *glc = w[11], *dh0c = w[12], *g0c = w[13], *gglc = w[14];
    float *dg0c = w[15];
    int st = zero_async(zD, static_cast<size_t>(d_inner) * fs, s);
    if (st != SSM2D_OK) return st;
    for (long n0 = 0; n0 < d_state; n0 += CH) {
        const long nc = std::min<long>(CH, d_state - n0);
        const bool first = n0 == 0;
        if ((st = state_slice(A, Ac, d_inner, d_state, n0, nc, 1, false, s)) != SSM2D_OK) return st;
        if ((st = state_slice(B, Bc, batch, d_state, n0, nc, HW, false, s)) != SSM2D_OK) return st;
        if ((st = state_slice(C, Cc, batch, d_state, n0, nc, HW, false, s)) != SSM2D_OK) return st;
        if (h_init && (st = state_slice(h_init, h0c, BD, d_state, n0, nc, W, false, s)) != SSM2D_OK) return st;
        if (dh_last && (st = state_slice(dh_last, glc, BD, d_state, n0, nc, W, false, s)) != SSM2D_OK) return st;
        if (hh_init && (st = state_slice(hh_init, g0c, BD, d_state, n0, nc, H, false, s)) != SSM2D_OK) return st;
        if (dhh_last && (st = state_slice(dhh_last, gglc, BD, d_state, n0, nc, H, false, s)) != SSM2D_OK) return st;
        st = scan_bwd<float>(x, delta, Ac, Bc, Cc, first ? D : zD, dy, first ? dx : dxc, first ? ddelta : ddc, dAc,
                             dBc, dCc, first ? dD : dDc, batch, d_inner, nc, H, W, stream,
                             flags, h_init ? h0c : nullptr, dh_last ? glc : nullptr, dh_init ? dh0c : nullptr,
                             hh_init ? g0c : nullptr, dhh_last ? gglc : nullptr, dhh_init ? dg0c : nullptr);
        if (st != SSM2D_OK) return st;
        if ((st = state_slice(static_cast<const float *>(dAc), dA, d_inner, d_state, n0, nc, 1, true, s)) != SSM2D_OK)
            return st;
        if ((st = state_slice(static_cast<const float *>(dBc), dB, batch, d_state, n0, nc, HW, true, s)) != SSM2D_OK)
            return st;
        if ((st = state_slice(static_cast<const float *>(dCc), dC, batch, d_state, n0, nc, HW, true, s)) != SSM2D_OK)
            return st;
        if (dh_init &&
            (st = state_slice(static_cast<const float *>(dh0c), dh_init, BD, d_state, n0, nc, W, true, s)) != SSM2D_OK)
            return st;
        if (dhh_init &&
            (st = state_slice(static_cast<const float *>(dg0c), dhh_init, BD, d_state, n0, nc, H, true, s)) != SSM2D_OK)
            return st;
        if (!first) {
            const long n = BD * HW;
            const unsigned nb = static_cast<unsigned>((n + 255) / 256);
            add_into_kernel<<<dim3(nb), dim3(256), 0, s>>>(dx, dxc, n);
            add_into_kernel<<<dim3(nb), dim3(256), 0, s>>>(ddelta, ddc, n);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e);
        }
    }
    return SSM2D_OK;
}

// flags: SSM2D_FLIP_H / SSM2D_FLIP_W / SSM2D_VERTICAL_FIRST, the direction
// and order of the forward scan. h_init (may be null): the carried vertical
// state the forward started from; dh_last (may be null): dL/dh_last for the
// state it handed out; dh_init (may be null): receives dL/dh_init (all
// float32 [batch][d_inner][d_state][W]); hh_init, dhh_last, dhh_init: the
// same for the carried row state ([batch][d_inner][d_state][H]).
template <typename T>
int scan_bwd(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *dy, T *dx,
             T *ddelta, float *dA, T *dB, T *dC, float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
             int64_t W, void *stream, unsigned flags, const float *h_init, const float *dh_last, float *dh_init,
             const float *hh_init, const float *dhh_last, float *dhh_init)
{
    if ((flags & ~kKnownFlags) != 0 || (flags & (SSM2D_ACCUMULATE | SSM2D_FOUR_WAY | SSM2D_DELTA_SOFTPLUS)))
        return SSM2D_ERR_BAD_FLAGS;
    const bool f_h = (flags & SSM2D_FLIP_H) != 0, f_w = (flags & SSM2D_FLIP_W) != 0;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (d_inner == 0) return SSM2D_OK;
    if (d_state > SSM2D_MAX_STATE || H > SSM2D_MAX_SIDE || W > SSM2D_MAX_SIDE) return SSM2D_ERR_UNSUPPORTED;
    // more states than the kernels hold: fp32 runs in chunks of states; bf16
    // callers widen first (the chunks' dx and d delta are summed in fp32)
    if (d_state > SSM2D_MAX_STATE_BWD && !std::is_same<T, float>::value) return SSM2D_ERR_UNSUPPORTED;
    const int64_t lim = (int64_t{1} << 31) - 1;
    const int64_t nstrips = (W + 3) / 4, pad = 4 * nstrips - W;
    const int64_t n_dblk = (d_inner + 7) / 8;
    int64_t npl = 1;
    while (npl * 8 < d_state) npl *= 2;
    const int64_t tiles = batch * n_dblk * nstrips * (H + 1);  // (chain, strip, row), rows -1 .. H-1
    if (batch * d_inner * H * W > lim || batch * d_state * H * W > lim || d_inner * d_state > lim)
        return SSM2D_ERR_UNSUPPORTED;
    const bool work = batch > 0 && H > 0 && W > 0;
    if ((!dA && d_state > 0) || !dD || (work && (!x || !delta || !D || !dy || !dx || !ddelta)) ||
        (work && d_state > 0 && (!A || !B || !C || !dB || !dC)))
        return SSM2D_ERR_NULLPTR;
    if (misaligned(x) || misaligned(delta) || misaligned(A) || misaligned(B) || misaligned(C) || misaligned(D) ||
        misaligned(dy) || misaligned(dx) || misaligned(ddelta) || misaligned(dA) || misaligned(dB) || misaligned(dC) ||
        misaligned(dD) || misaligned(h_init) || misaligned(dh_last) || misaligned(dh_init) || misaligned(hh_init) ||
        misaligned(dhh_last) || misaligned(dhh_init))
        return SSM2D_ERR_MISALIGNED;
    const bool rcarry = hh_init || dhh_last || dhh_init;

    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    if (take_timeout_flag(dev, stream)) return SSM2D_ERR_DEVICE_TIMEOUT;
    const hipStream_t s0 = static_cast<hipStream_t>(stream);
    // no rows (no columns): a handed-out state is the carried one itself
    const bool vf = (flags & SSM2D_VERTICAL_FIRST) != 0;
    float *cdst = vf ? dhh_init : dh_init, *rdst = vf ? dh_init : dhh_init;
    const float *csrc = vf ? dhh_last : dh_last, *rsrc = vf ? dh_last : dhh_last;
    const long cn = batch * d_inner * d_state * (vf ? H : W), rn = batch * d_inner * d_state * (vf ? W : H);
    if (cdst && cn > 0 && (vf ? W : H) == 0) {
        copy_or_zero_kernel<<<dim3(static_cast<unsigned>((cn + 255) / 256)), dim3(256), 0, s0>>>(csrc, cdst, cn);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    if (rdst && rn > 0 && (vf ? H : W) == 0) {
        copy_or_zero_kernel<<<dim3(static_cast<unsigned>((rn + 255) / 256)), dim3(256), 0, s0>>>(rsrc, rdst, rn);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    if constexpr (std::is_same<T, float>::value) {
        if (d_state > SSM2D_MAX_STATE_BWD && work)
            return scan_bwd_chunked(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H,
                                    W, stream, flags, h_init, dh_last, dh_init, hh_init, dhh_last, dhh_init, dev);
    }
    if (vf && work)
        return scan_bwd_vfirst<T>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                                  stream, flags, dev, h_init, dh_last, dh_init, hh_init, dhh_last, dhh_init);
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
    const int rc = rcarry ? kModeRowCarry : 0;
    Plan pf = make_plan(batch, d_inner, d_state, H, W, kModeStates | (f_w ? kModeFlipW : 0) | rc);
    pf.bw = &bw;
    pf.flip_h = f_h ? 1 : 0;
    pf.h_init = h_init;
    pf.hh_init = hh_init;
    choose_coop<T>(pf, H, align);
    if (pf.npl != npl || pf.n_dblk != n_dblk || pf.nstrips != nstrips) return SSM2D_ERR_UNSUPPORTED;
    int st;
    if (rcarry)
        st = f_w ? dispatch_states_flipw_rowc(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pf, dev, stream, align)
                 : dispatch_states_rowc(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pf, dev, stream, align);
    else
        st = f_w ? dispatch_states_flipw(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pf, dev, stream, align)
                 : dispatch_states(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pf, dev, stream, align);
    if (st != SSM2D_OK) return st;
    // 2. the adjoint scans from the opposite corner, with every local
    // derivative (chains cut into several workgroups: the courier-free
    // kernels, which fit 8 strips per workgroup instead of 6)
    const int bmode = kModeBackward | (f_w ? 0 : kModeFlipW) | rc;
    Plan pb = make_plan(batch, d_inner, d_state, H, W, bmode);
    const bool edges = pb.groups > 1;
    if (edges) pb = make_plan(batch, d_inner, d_state, H, W, bmode | kModeEdges);
    pb.flip_h = f_h ? 0 : 1;
    pb.bw = &bw;
    pb.h_init = dh_last;   // the vertical adjoint's carry in and out
    pb.h_last = dh_init;
    pb.hh_init = dhh_last;  // the row adjoint's carry in and out
    pb.hh_last = dhh_init;
    choose_coop<T>(pb, H, align);
    if (pb.npl != npl || pb.n_dblk != n_dblk || pb.nstrips != nstrips) return SSM2D_ERR_UNSUPPORTED;
    if (rcarry) {
        if (f_w)
            st = edges ? dispatch_bwd_ltr_edges_rowc(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align)
                       : dispatch_bwd_ltr_rowc(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align);
        else
            st = edges ? dispatch_bwd_edges_rowc(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align)
                       : dispatch_bwd_rowc(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align);
    } else if (f_w) {
        st = edges ? dispatch_bwd_ltr_edges(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align)
                   : dispatch_bwd_ltr(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align);
    } else {
        st = edges ? dispatch_bwd_edges(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align)
                   : dispatch_bwd(x, delta, A, B, C, D, dx, bi, di, ni, hi, wi, pb, dev, stream, align);
    }
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
// gate and the step-size preparation are elementwise). fp32: the prepared
// step size, the recomputed ungated output and the gated upstream gradient
// are fp32 tensors. bf16 with any option: every tensor the chain rule hands
// on is kept in fp32 (x, B, C widened exactly, the fp32 backward), and each
// gradient is rounded to bf16 once.
template <typename T>
int scan_bwd_mamba(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, const T *z,
                   const float *delta_bias, const float *h_init, const float *dh_last, const float *hh_init,
                   const float *dhh_last, const T *dy, T *dx, T *ddelta, float *dA, T *dB, T *dC, float *dD, T *dz,
                   float *ddelta_bias, float *dh_init, float *dhh_init, int64_t batch, int64_t d_inner,
                   int64_t d_state, int64_t H, int64_t W, unsigned flags, void *stream)
{
    constexpr unsigned kDirs = SSM2D_FLIP_H | SSM2D_FLIP_W | SSM2D_VERTICAL_FIRST;
    if ((flags & ~(SSM2D_DELTA_SOFTPLUS | kDirs)) != 0) return SSM2D_ERR_BAD_FLAGS;
    const unsigned dirs = flags & kDirs;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (d_inner == 0) return SSM2D_OK;
    if ((z && !dz) || (ddelta_bias && !delta_bias)) return SSM2D_ERR_NULLPTR;
    if (misaligned(z) || misaligned(dz) || misaligned(delta_bias) || misaligned(ddelta_bias) || misaligned(h_init) ||
        misaligned(dh_last) || misaligned(dh_init) || misaligned(hh_init) || misaligned(dhh_last) || misaligned(dhh_init))
        return SSM2D_ERR_MISALIGNED;
    const bool softplus = (flags & SSM2D_DELTA_SOFTPLUS) != 0;
    const bool prep = delta_bias || softplus;
    const long total = batch * d_inner * H * W;
    const unsigned nblk = static_cast<unsigned>((total + 255) / 256);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    if (ddelta_bias) {
        zero_kernel<<<dim3(static_cast<unsigned>((d_inner + 255) / 256)), dim3(256), 0, s>>>(ddelta_bias, d_inner);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    // (bf16 with more states than the kernels hold: the widened fp32 path,
    // whose backward runs in chunks of states)
    const bool wide_states = std::is_same<T, uint16_t>::value && d_state > SSM2D_MAX_STATE_BWD;
    if (total == 0 || d_state > SSM2D_MAX_STATE || (!prep && !z && !wide_states))  // the backward alone (it also reports sizes)
        return scan_bwd<T>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                           stream, dirs, h_init, dh_last, dh_init, hh_init, dhh_last, dhh_init);
    if (!x || !delta || !dy || !dx || !ddelta || !D || (d_state > 0 && (!A || !B || !C || !dB || !dC || !dA)) || !dD)
        return SSM2D_ERR_NULLPTR;
    if (misaligned(x) || misaligned(delta) || misaligned(dy) || misaligned(dx) || misaligned(ddelta))
        return SSM2D_ERR_MISALIGNED;
    if (take_timeout_flag(dev, stream)) return SSM2D_ERR_DEVICE_TIMEOUT;
    using TW = float;  // the working type of everything the chain rule hands on
    constexpr bool WIDE = std::is_same<T, uint16_t>::value;
    const long tb = batch * d_state * H * W;
    const size_t eb = static_cast<size_t>(total) * 4 + 256, bb = static_cast<size_t>(tb) * 4 + 256;
    auto buf = [&](int slot, size_t bytes, TW **out) {
        void *v = nullptr;
        const int st = get_aux_ws(dev, stream, slot, bytes, &v);
        *out = static_cast<TW *>(v);
        return st;
    };
    // inputs of the scan in the working type
    const TW *xw, *Bw, *Cw;
    TW *dstep = nullptr;
    int st = buf(kSlotStep, eb, &dstep);
    if (st != SSM2D_OK) return st;
    delta_prep_kernel<T, TW><<<dim3(nblk), dim3(256), 0, s>>>(delta, delta_bias, dstep, total, H * W,
                                                               static_cast<int>(d_inner), softplus ? 1 : 0);
    {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    if constexpr (WIDE) {
        TW *x32, *B32, *C32;
        if ((st = buf(kSlotX32, eb, &x32)) != SSM2D_OK || (st = buf(kSlotB32, bb, &B32)) != SSM2D_OK ||
            (st = buf(kSlotC32, bb, &C32)) != SSM2D_OK)
            return st;
        if ((st = widen(x, x32, total, s)) != SSM2D_OK) return st;
        if (d_state > 0 && ((st = widen(B, B32, tb, s)) != SSM2D_OK || (st = widen(C, C32, tb, s)) != SSM2D_OK))
            return st;
        xw = x32; Bw = B32; Cw = C32;
    } else {
        xw = x; Bw = B; Cw = C;
    }
    // upstream gradient of the scan
    TW *g = nullptr;
    if ((st = buf(kSlotG32, eb, &g)) != SSM2D_OK) return st;
    if (z) {
        // the ungated scan output, then dz and dy * SiLU(z)
        TW *y0 = nullptr;
        if ((st = buf(kSlotY0, eb, &y0)) != SSM2D_OK) return st;
        st = scan_fwd<TW>(xw, dstep, A, d_state ? Bw : nullptr, d_state ? Cw : nullptr, D, y0, batch, d_inner,
                          d_state, H, W, dirs, false, stream, nullptr, nullptr, h_init, nullptr, hh_init, nullptr);
        if (st != SSM2D_OK) return st;
        gate_bwd_kernel<T, TW><<<dim3(nblk), dim3(256), 0, s>>>(dy, y0, z, dz, g, total);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    } else if constexpr (WIDE) {
        if ((st = widen(dy, g, total, s)) != SSM2D_OK) return st;
    } else {
        g = const_cast<TW *>(reinterpret_cast<const TW *>(dy));
    }
    // the scan's backward in the working type
    TW *dxw, *ddw, *dBw, *dCw;
    if constexpr (WIDE) {
        if ((st = buf(kSlotDX32, eb, &dxw)) != SSM2D_OK || (st = buf(kSlotDD32, eb, &ddw)) != SSM2D_OK ||
            (st = buf(kSlotDB32, bb, &dBw)) != SSM2D_OK || (st = buf(kSlotDC32, bb, &dCw)) != SSM2D_OK)
            return st;
    } else {
        dxw = reinterpret_cast<TW *>(dx); ddw = reinterpret_cast<TW *>(ddelta);
        dBw = reinterpret_cast<TW *>(dB); dCw = reinterpret_cast<TW *>(dC);
    }
    st = scan_bwd<TW>(xw, dstep, A, d_state ? Bw : nullptr, d_state ? Cw : nullptr, D, g, dxw, ddw, dA,
                      d_state ? dBw : nullptr, d_state ? dCw : nullptr, dD, batch, d_inner, d_state, H, W, stream, dirs,
                      h_init, dh_last, dh_init, hh_init, dhh_last, dhh_init);
    if (st != SSM2D_OK) return st;
    // d delta with respect to the raw step size, d bias (and the rounding)
    if (prep || WIDE) {
        step_bwd_kernel<TW, T><<<dim3(static_cast<unsigned>(batch * d_inner)), dim3(256), 0, s>>>(
            ddw, ddelta, delta, delta_bias, ddelta_bias, H * W, static_cast<int>(d_inner), softplus ? 1 : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e);
    }
    if constexpr (WIDE) {
        if ((st = gate_or_round<TW, T>(dxw, nullptr, dx, total, s)) != SSM2D_OK) return st;
        if (d_state > 0) {
            if ((st = gate_or_round<TW, T>(dBw, nullptr, dB, tb, s)) != SSM2D_OK) return st;
            if ((st = gate_or_round<TW, T>(dCw, nullptr, dC, tb, s)) != SSM2D_OK) return st;
        }
    }
    return SSM2D_OK;
}

// Scan launches of a forward call (no gate, delta bias or carried states) in
// each kernel, as scan_fwd and launch() plan them.
template <typename T>
void count_fwd_launches(int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, unsigned flags,
                        int *two_row, int *general, int *narrow)
{
    const int vf = (flags & SSM2D_VERTICAL_FIRST) ? kModeVFirst : 0;
    const int acc = (flags & SSM2D_ACCUMULATE) ? kModeAccumulate : 0;
    const int n = (flags & SSM2D_FOUR_WAY) ? 4 : 1;
    for (int q = 0; q < n; ++q) {
        const int mode = (flags & SSM2D_FOUR_WAY)
                             ? (((q & 2) ? kModeFlipW : 0) | vf | (q == 0 ? acc : kModeAccumulate))
                             : (((flags & SSM2D_FLIP_W) ? kModeFlipW : 0) | vf | acc);
        if (takes_narrow(mode, batch, d_inner, d_state, H, W, false, static_cast<int>(sizeof(T)))) {
            ++*narrow;
            continue;
        }
        Plan pl = forward_plan<T>(batch, d_inner, d_state, H, W, mode, false);
        const int align = row_align(W);
        choose_coop<T>(pl, H, align);
        ++*(takes_fast<T>(pl, W, align) ? two_row : general);
    }
}

}  // namespace

extern "C" {

int ssm2d_fwd_kernels(int bf16, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                      uint32_t flags, int *two_row, int *general, int *narrow)
{
    if (!two_row || !general || !narrow) return SSM2D_ERR_NULLPTR;
    *two_row = *general = *narrow = 0;
    if ((flags & ~kKnownFlags) != 0 || ((flags & SSM2D_FOUR_WAY) && (flags & (SSM2D_FLIP_H | SSM2D_FLIP_W))))
        return SSM2D_ERR_BAD_FLAGS;
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return SSM2D_ERR_BAD_DIM;
    if (batch == 0 || d_inner == 0 || H == 0 || W == 0) return SSM2D_OK;
    if (d_state > SSM2D_MAX_STATE || H > SSM2D_MAX_SIDE || W > SSM2D_MAX_SIDE) return SSM2D_ERR_UNSUPPORTED;
    // bf16 four-corner sums and softplus step sizes run the fp32 kernels
    if (bf16 && !(flags & (SSM2D_FOUR_WAY | SSM2D_DELTA_SOFTPLUS)))
        count_fwd_launches<uint16_t>(batch, d_inner, d_state, H, W, flags, two_row, general, narrow);
    else
        count_fwd_launches<float>(batch, d_inner, d_state, H, W, flags, two_row, general, narrow);
    return SSM2D_OK;
}

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
                         float *h_last, const float *hh_init, float *hh_last, float *y, int64_t batch,
                         int64_t d_inner, int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_fwd<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, true, stream, z, delta_bias,
                           h_init, h_last, hh_init, hh_last);
}

int ssm2d_scan_fwd_mamba_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                              const uint16_t *C, const float *D, const uint16_t *z, const float *delta_bias,
                              const float *h_init, float *h_last, const float *hh_init, float *hh_last, uint16_t *y,
                              int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W, uint32_t flags,
                              void *stream)
{
    return scan_fwd<uint16_t>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, flags, true, stream, z,
                              delta_bias, h_init, h_last, hh_init, hh_last);
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
    if (d_state > SSM2D_MAX_STATE_BWD && d_state <= SSM2D_MAX_STATE && !(flags & SSM2D_DELTA_SOFTPLUS))
        // (more states than the kernels hold: widened to fp32, in chunks of states)
        return scan_bwd_mamba<uint16_t>(x, delta, A, B, C, D, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dy,
                                        dx, ddelta, dA, dB, dC, dD, nullptr, nullptr, nullptr, nullptr, batch, d_inner,
                                        d_state, H, W, flags, stream);
    return scan_bwd<uint16_t>(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                              stream, flags);
}

int ssm2d_scan_bwd_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                        const uint16_t *C, const float *D, const uint16_t *dy, uint16_t *dx, uint16_t *ddelta,
                        float *dA, uint16_t *dB, uint16_t *dC, float *dD, int64_t batch, int64_t d_inner,
                        int64_t d_state, int64_t H, int64_t W, void *stream)
{
    return ssm2d_scan_bwd_ex_bf16(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                                  0u, stream);
}

int ssm2d_scan_bwd_mamba(const float *x, const float *delta, const float *A, const float *B, const float *C,
                         const float *D, const float *z, const float *delta_bias, const float *h_init,
                         const float *dh_last, const float *hh_init, const float *dhh_last, const float *dy,
                         float *dx, float *ddelta, float *dA, float *dB, float *dC, float *dD, float *dz,
                         float *ddelta_bias, float *dh_init, float *dhh_init, int64_t batch, int64_t d_inner,
                         int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_bwd_mamba<float>(x, delta, A, B, C, D, z, delta_bias, h_init, dh_last, hh_init, dhh_last, dy, dx,
                                 ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh_init, dhh_init, batch, d_inner, d_state,
                                 H, W, flags, stream);
}

int ssm2d_scan_bwd_mamba_bf16(const uint16_t *x, const uint16_t *delta, const float *A, const uint16_t *B,
                              const uint16_t *C, const float *D, const uint16_t *z, const float *delta_bias,
                              const float *h_init, const float *dh_last, const float *hh_init,
                              const float *dhh_last, const uint16_t *dy, uint16_t *dx, uint16_t *ddelta, float *dA,
                              uint16_t *dB, uint16_t *dC, float *dD, uint16_t *dz, float *ddelta_bias,
                              float *dh_init, float *dhh_init, int64_t batch, int64_t d_inner, int64_t d_state,
                              int64_t H, int64_t W, uint32_t flags, void *stream)
{
    return scan_bwd_mamba<uint16_t>(x, delta, A, B, C, D, z, delta_bias, h_init, dh_last, hh_init, dhh_last, dy, dx,
                                    ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh_init, dhh_init, batch, d_inner,
                                    d_state, H, W, flags, stream);
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
    case SSM2D_ERR_TOO_LARGE: return "the call's workspace exceeds the static scratch of ssm2d_scan_fwd_noalloc";
    default: return "unknown status";
    }
}

int ssm2d_scan_fwd_noalloc(const float *x, const float *delta, const float *A, const float *B, const float *C,
                           const float *D, float *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                           int64_t W, void *stream)
{
    bool work = false;
    const int chk = check_fwd<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, 0u, false, nullptr,
                                     nullptr, nullptr, nullptr, &work);
    if (chk != SSM2D_OK || !work) return chk;
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    const WsEntry *ws = nullptr;
    const int st = scratch_ws(dev, static_cast<hipStream_t>(stream), &ws);
    if (st != SSM2D_OK) return st;
    return launch<float>(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, 0, 0, dev, stream, nullptr, nullptr,
                         nullptr, ws);
}

int ssm2d_sync_check(void *stream)
{
    SSM2D_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    bool timeout = take_timeout_flag(dev, stream);
    // device error words, cleared here: the stream's workspace (a timeout
    // counts from there only when the workspace has no host-visible flag,
    // which reports it once by itself), and the static scratch
    unsigned int *words[2] = {nullptr, nullptr};
    bool counts[2] = {false, true};
    auto it = g_ws.find({dev, stream});
    if (it != g_ws.end() && it->second.head) {
        words[0] = it->second.head + 2;
        counts[0] = it->second.herr == nullptr;
    }
    auto sc = g_scratch.find(dev);
    if (sc != g_scratch.end()) words[1] = sc->second.head + 2;
    for (int k = 0; k < 2; ++k) {
        if (!words[k]) continue;
        unsigned int v = 0;
        SSM2D_HIP_TRY(hipMemcpy(&v, words[k], sizeof(v), hipMemcpyDeviceToHost));
        if (v != 0) {
            const unsigned int zero = 0;
            SSM2D_HIP_TRY(hipMemcpy(words[k], &zero, sizeof(zero), hipMemcpyHostToDevice));
            timeout = timeout || counts[k];
        }
    }
    return timeout ? SSM2D_ERR_DEVICE_TIMEOUT : SSM2D_OK;
}

int ssm2d_release_workspaces(void *stream)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    SSM2D_HIP_TRY(hipStreamSynchronize(s));
    const bool timeout = take_timeout_flag(dev, stream);
    auto it = g_ws.find({dev, stream});
    if (it != g_ws.end()) {
        free_ws(it->second, s);
        if (it->second.herr) (void)hipHostFree(it->second.herr);
        g_ws.erase(it);
    }
    for (auto b = g_bufs.begin(); b != g_bufs.end();) {
        if (b->first.first == std::make_pair(dev, stream)) {
            free_async(b->second.buf, s);
            b = g_bufs.erase(b);
        } else {
            ++b;
        }
    }
    SSM2D_HIP_TRY(hipStreamSynchronize(s));
    return timeout ? SSM2D_ERR_DEVICE_TIMEOUT : SSM2D_OK;
}

int ssm2d_test_set_epoch(void *stream, uint32_t epoch)
{
    int dev = 0;
    SSM2D_HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || !it->second.head) return SSM2D_ERR_UNSUPPORTED;
    SSM2D_HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    const unsigned int v = epoch % kEpochs;
    SSM2D_HIP_TRY(hipMemcpy(it->second.head + 3, &v, sizeof(v), hipMemcpyHostToDevice));
    return SSM2D_OK;
}

int ssm2d_set_spin_limit(int64_t polls)
{
    std::lock_guard<std::recursive_mutex> lock(g_mutex);
    g_spin_limit = polls < 0 ? 0 : polls;
    return SSM2D_OK;
}

int ssm2d_version(void) { return 401; }

const char *ssm2d_last_hip_error(void)
{
    return hipGetErrorString(static_cast<hipError_t>(g_last_hip_error.load()));
}

}  // extern "C"

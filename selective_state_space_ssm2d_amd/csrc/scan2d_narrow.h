// libssm2d: the plain forward scan of narrow maps (at most 16 columns and 16
// states), one wave per 16 channels, whole rows at a time.
//
// Method (juejin.cn "2DMamba 精读", part 四 section 5; papernotes.org "2DMamba" 关键设计):
//   Abar = exp(delta*A), Bx = delta*B*x
//   hh[i,j] = Abar*hh[i,j-1] + Bx         horizontal scan, zero before column 0
//   h[i,j]  = Abar*h[i-1,j]  + hh[i,j]    vertical scan of the horizontal results
//   y = sum_n C*h + D*x                   state dims reduced on chip, only y stored
//
// The strip kernels cut a row into strips of 4 or 8 columns, one wave each,
// and pass the row carry from strip to strip; on a map of 14 columns (the
// 14 x 14 patch grid of the pages' padding example) that is a chain of four
// waves handing a carry on at every row, for 14 rows. Here a wave holds the
// whole row: lane (g, ch) of a wave is channel ch of 16 and state group g of
// 4 (NPL states each), keeps the vertical states of all the row's cells in
// registers, runs the horizontal chain over the row itself, and no carry
// leaves the wave. Per row the wave loads the rows of x, delta (its 16
// channels) and B, C (all states) with whole-wave loads, widens them to fp32
// into its own LDS tile, reads back what each lane needs as 16-byte vectors,
// and sums its partial outputs over the 4 state groups with two lane swaps,
// leaving each lane with a quarter of the row's cells. Rows run top to bottom
// or bottom to top (runtime row stride). Columns past the map's width are
// zero-padded: their decay is 1 and their inputs 0, and they are never stored.
// Padded states (B = C = 0) stay exactly 0.
//
// The row loop has no branch: loads and stores go through buffer resources
// (a lane outside the block or the map uses an offset past the buffer's end:
// its load reads 0 and its store is dropped by the hardware), and tile
// writes of such lanes land in spare LDS rows. With branches around them the
// compiler cannot count the memory operations in flight, and each row began
// by waiting for every one of them, the last row's output stores included.
#pragma once

#include "scan2d_kernel.h"

namespace ssm2d_impl {

constexpr int kNarrowMaxW = 16;    // widest row a wave scans whole
constexpr int kNarrowMaxN = 16;    // states (4 groups of at most 4 a lane)
constexpr int kNarrowCh = 16;      // channels a wave
constexpr int kNarrowWaves = 4;    // waves a workgroup (independent of each other)
// elements of one row a wave loads per tensor: x and delta hold 16 channel
// rows, B and C 16 state rows, of at most 16 columns
constexpr int kNarrowLoads = kNarrowCh * kNarrowMaxW / kWave;
// a buffer offset past the end of every buffer the kernel addresses (each
// holds fewer than 2^31 bytes): loads there read 0, stores are dropped
constexpr unsigned kNarrowOff = 0x80000000u;
constexpr int kBufferWord3 = 0x00020000;  // descriptor word 3 of a raw gfx9 buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t narrow_rsrc(const void *base, long bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kBufferWord3);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff, float)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), soff, 0));
}
__device__ __forceinline__ uint16_t buf_load(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff, uint16_t)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), soff, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff, float v, float)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(voff), soff, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff, float v, uint16_t)
{
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(bf16_bits(v)), r, static_cast<int>(voff), soff, 0);
}

struct NarrowParams {
    const void *x, *delta, *B, *C;
    const float *A, *D;
    void *y;
    int batch, d_inner, d_state, H, W, flip_h;
    int n_dblk;  // 16-channel blocks per batch entry
};

// WW: the row padded to 8 or 16 columns; NPL: states a lane (1, 2 or 4).
template <typename T, int NPL, int WW>
__global__ __launch_bounds__(kWave *kNarrowWaves) void scan2d_narrow_kernel(const NarrowParams p)
{
    // one tile per wave: rows of x, delta (16 channels) and B, C (16 states),
    // WW columns each, fp32; then 4 spare rows that take the writes of lanes
    // outside the block
    __shared__ __align__(16) float s_tile[kNarrowWaves][4][kNarrowCh + 4][WW];
    constexpr int KO = WW / 4;  // finished cells a lane holds after the group sum

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wid = blockIdx.x * kNarrowWaves + wave;  // (batch, channel block)
    if (wid >= p.batch * p.n_dblk) return;
    const int b = wid / p.n_dblk;
    const int d0 = (wid % p.n_dblk) * kNarrowCh;
    const int g = lane / kNarrowCh;      // state group
    const int chl = lane % kNarrowCh;    // channel in the block
    const int d = d0 + chl;
    const bool d_ok = d < p.d_inner;
    const int H = p.H, W = p.W;
    const long HW = static_cast<long>(H) * W;
    float(*tile)[kNarrowCh + 4][WW] = s_tile[wave];

    // What each lane loads of a row: element e = lane + 64 j of the 16 x W
    // block, as (row r of the block: channel or state, column c). Byte
    // offsets of the row-0 element in its tensor (x / delta and B / C share
    // them; every tensor has fewer than 2^31 bytes), kNarrowOff where the
    // element is outside the tensor, and the tile position (a spare row
    // outside the block).
    const long xd_bytes = static_cast<long>(p.batch) * p.d_inner * HW * sizeof(T);
    const long bc_bytes = static_cast<long>(p.batch) * p.d_state * HW * sizeof(T);
    const __amdgpu_buffer_rsrc_t rx = narrow_rsrc(p.x, xd_bytes), rd = narrow_rsrc(p.delta, xd_bytes);
    const __amdgpu_buffer_rsrc_t rb = narrow_rsrc(p.B, bc_bytes), rc = narrow_rsrc(p.C, bc_bytes);
    const __amdgpu_buffer_rsrc_t ry = narrow_rsrc(p.y, xd_bytes);
    unsigned off_xd[kNarrowLoads], off_bc[kNarrowLoads];
    int tpos[kNarrowLoads];
#pragma unroll
    for (int j = 0; j < kNarrowLoads; ++j) {
        const int e = lane + kWave * j;
        const int r = e / W, c = e % W;
        const bool in_block = e < kNarrowCh * W;
        tpos[j] = in_block ? r * WW + c : kNarrowCh * WW + (lane & (4 * WW - 1));
        off_xd[j] = (in_block && d0 + r < p.d_inner)
                        ? static_cast<unsigned>(((static_cast<long>(b) * p.d_inner + d0 + r) * HW + c) * sizeof(T))
                        : kNarrowOff;
        off_bc[j] = (in_block && r < p.d_state)
                        ? static_cast<unsigned>(((static_cast<long>(b) * p.d_state + r) * HW + c) * sizeof(T))
                        : kNarrowOff;
    }
    // the padding of every row stays zero
    for (int k = lane; k < 4 * (kNarrowCh + 4) * WW; k += kWave) (&tile[0][0][0])[k] = 0.0f;

    float Ap[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
        const int n = g * NPL + k;
        Ap[k] = (n < p.d_state && d_ok) ? p.A[d * p.d_state + n] * kLog2e : 0.0f;
    }
    const float Dd = (p.D && d_ok) ? p.D[d] : 0.0f;
    float hv[WW][NPL];
#pragma unroll
    for (int c = 0; c < WW; ++c)
#pragma unroll
        for (int k = 0; k < NPL; ++k) hv[c][k] = 0.0f;

    const int rs = p.flip_h ? -W : W;
    const int row0 = p.flip_h ? static_cast<int>(HW) - W : 0;
    // byte offsets of this lane's output cells in row 0 (kNarrowOff: not stored)
    unsigned off_y[KO];
#pragma unroll
    for (int c = 0; c < KO; ++c) {
        const int col = g * KO + c;
        off_y[c] = (d_ok && col < W) ? static_cast<unsigned>(((static_cast<long>(b) * p.d_inner + d) * HW + col) * sizeof(T))
                                     : kNarrowOff;
    }

    // the first row's elements
    T ex[kNarrowLoads], ed[kNarrowLoads], eb[kNarrowLoads], ec[kNarrowLoads];
    auto load_row = [&](int ro) __attribute__((always_inline)) {
        const int so = ro * static_cast<int>(sizeof(T));
#pragma unroll
        for (int j = 0; j < kNarrowLoads; ++j) {
            ex[j] = buf_load(rx, off_xd[j], so, T());
            ed[j] = buf_load(rd, off_xd[j], so, T());
            eb[j] = buf_load(rb, off_bc[j], so, T());
            ec[j] = buf_load(rc, off_bc[j], so, T());
        }
    };
    load_row(row0);

    // a row's outputs are stored at the start of the next row, after that
    // row's loads: the wait at the top of a row (for the loads issued a row
    // earlier) then never waits on stores just issued
    float pend[KO];
#pragma unroll
    for (int c = 0; c < KO; ++c) pend[c] = 0.0f;
    int pend_so = 0;

    for (int t = 0; t < H; ++t) {
        const int ro = row0 + t * rs;
        // this row into the tile (the wave's reads of the last row are done:
        // LDS accesses of one wave complete in order)
#pragma unroll
        for (int j = 0; j < kNarrowLoads; ++j) {
            (&tile[0][0][0])[tpos[j]] = elem_value(ex[j]);
            (&tile[1][0][0])[tpos[j]] = elem_value(ed[j]);
            (&tile[2][0][0])[tpos[j]] = elem_value(eb[j]);
            (&tile[3][0][0])[tpos[j]] = elem_value(ec[j]);
        }
        // the next row's loads (the last row loads itself again), in flight
        // during this row's arithmetic
        load_row(t + 1 < H ? ro + rs : ro);
        // the previous row's outputs (none before the first row)
#pragma unroll
        for (int c = 0; c < KO; ++c) buf_store(ry, t > 0 ? off_y[c] : kNarrowOff, pend_so, pend[c], T());

        float acc[WW];
#pragma unroll
        for (int c = 0; c < WW; ++c) acc[c] = 0.0f;
        float hh[NPL];
#pragma unroll
        for (int k = 0; k < NPL; ++k) hh[k] = 0.0f;
#pragma unroll
        for (int q = 0; q < WW / 4; ++q) {
            const float4 x4 = *reinterpret_cast<const float4 *>(&tile[0][chl][4 * q]);
            const float4 d4 = *reinterpret_cast<const float4 *>(&tile[1][chl][4 * q]);
            const float xq[4] = {x4.x, x4.y, x4.z, x4.w};
            const float dq[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int k = 0; k < NPL; ++k) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&tile[2][g * NPL + k][4 * q]);
                const float4 c4 = *reinterpret_cast<const float4 *>(&tile[3][g * NPL + k][4 * q]);
                const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
                const float cq[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float a = __builtin_amdgcn_exp2f(dq[c] * Ap[k]);
                    hh[k] = __builtin_fmaf(a, hh[k], (dq[c] * xq[c]) * bq[c]);
                    hv[4 * q + c][k] = __builtin_fmaf(a, hv[4 * q + c][k], hh[k]);
                    acc[4 * q + c] = __builtin_fmaf(cq[c], hv[4 * q + c][k], acc[4 * q + c]);
                }
            }
        }
        // sum over the 4 state groups: group g ends with cells [g KO, (g+1) KO)
        float out[KO];
        reduce_groups<WW, 4>(acc, out, g);
        const float *xrow = &tile[0][chl][g * KO];
#pragma unroll
        for (int c = 0; c < KO; ++c) pend[c] = __builtin_fmaf(Dd, xrow[c], out[c]);
        pend_so = ro * static_cast<int>(sizeof(T));
    }
#pragma unroll
    for (int c = 0; c < KO; ++c) buf_store(ry, off_y[c], pend_so, pend[c], T());
}

template <typename T>
int launch_narrow(const T *x, const T *delta, const float *A, const T *B, const T *C, const float *D, T *y,
                  int batch, int d_inner, int d_state, int H, int W, int flip_h, void *stream)
{
    NarrowParams p{};
    p.x = x; p.delta = delta; p.B = B; p.C = C; p.A = A; p.D = D; p.y = y;
    p.batch = batch; p.d_inner = d_inner; p.d_state = d_state; p.H = H; p.W = W; p.flip_h = flip_h;
    p.n_dblk = (d_inner + kNarrowCh - 1) / kNarrowCh;
    const long waves = static_cast<long>(batch) * p.n_dblk;
    const dim3 grid(static_cast<unsigned>((waves + kNarrowWaves - 1) / kNarrowWaves));
    const dim3 block(kWave * kNarrowWaves);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int npl = (d_state + 3) / 4;
    const bool wide = W > 8;
#define SSM2D_NARROW_LAUNCH(NPL_, WW_) \
    hipLaunchKernelGGL((scan2d_narrow_kernel<T, NPL_, WW_>), grid, block, 0, s, p)
    if (npl <= 1) {
        if (wide) SSM2D_NARROW_LAUNCH(1, 16); else SSM2D_NARROW_LAUNCH(1, 8);
    } else if (npl == 2) {
        if (wide) SSM2D_NARROW_LAUNCH(2, 16); else SSM2D_NARROW_LAUNCH(2, 8);
    } else {
        if (wide) SSM2D_NARROW_LAUNCH(4, 16); else SSM2D_NARROW_LAUNCH(4, 8);
    }
#undef SSM2D_NARROW_LAUNCH
    return hipGetLastError() == hipSuccess ? SSM2D_OK : SSM2D_ERR_HIP;
}

}  // namespace ssm2d_impl

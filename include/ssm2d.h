/*
 * ssm2d.h — C ABI of the MI355X (gfx950) 2D selective scan library, libssm2d.so.
 *
 * The operation is the forward pass of the 2DMamba 2D selective scan
 * (arXiv 2412.00678). For batch b, channel d < d_inner, state n < d_state and
 * cell (i, j) of an H x W map:
 *
 *   Abar = exp(delta * A[d,n]),   Bx = delta * B[b,n,i,j] * x[b,d,i,j]
 *   hh[i,j] = Abar * hh[i,j-1] + Bx          (horizontal scan, left to right)
 *   h[i,j]  = Abar * h[i-1,j]  + hh[i,j]     (vertical scan over the horizontal results)
 *   y[b,d,i,j] = sum_n C[b,n,i,j] * h[i,j] + D[d] * x[b,d,i,j]
 *
 * with zero state before the first column and above the first row.
 * Passages: juejin.cn "2DMamba 精读", part 四 section 5 (横向扫描, 纵向扫描, final output
 * y = C h); papernotes.org "2DMamba" 关键设计, items 2D选择性SSM架构 (row scans are
 * 1D Mamba, the vertical scan runs over the horizontal results) and 硬件感知2D并行
 * 扫描算子 (state dims reduced on chip, only the aggregate written back). The
 * pages name Abar and Bbar without defining them: this library uses the
 * zero-order-hold A and Euler B of Mamba. The D x skip term is the Mamba
 * convention (the pages' output is y = C h).
 *
 * Layout: every tensor is dense row-major (C order), W fastest:
 *   x, delta, y : [batch][d_inner][H][W]
 *   B, C        : [batch][d_state][H][W]   (input dependent, shared by all d)
 *   A           : [d_inner][d_state]       float32
 *   D           : [d_inner]                float32
 * All pointers are DEVICE pointers on the current HIP device, allocated and
 * owned by the caller, 16-byte aligned. y must not alias any input. The library
 * keeps no pointer after the call returns.
 *
 * Asynchrony: a call validates its arguments on the host, enqueues its kernels
 * on `stream` (hipStream_t; NULL = the null stream) and returns without waiting.
 * Launch errors are reported as SSM2D_ERR_HIP. The library keeps an internal
 * workspace per (device, stream); calls on the same stream are ordered, calls
 * on different streams use different workspaces. A workspace is allocated and
 * grown in stream order (hipMallocAsync / hipFreeAsync on `stream`, zeroed by
 * a kernel on `stream`): no call waits for the host, and a call whose
 * workspace is already large enough allocates nothing. ssm2d_release_workspaces
 * frees a stream's workspaces.
 *
 * Graph capture: once a call of the same kind and size has run on `stream`
 * (so that nothing is allocated), the calls may be captured into a HIP graph
 * and replayed. The carry words that link the tiles of one map carry a tag
 * epoch kept in device memory and advanced by every launch, so replays and
 * launches never take each other's words.
 *
 * Carry waits: when a map's chain of tiles spans several workgroups, a tile
 * waits for its left neighbour's carries, produced by a workgroup that started
 * earlier (workgroups take tickets in the order they start). The carries go
 * through a bounded ring of rows (32; where the launch's grid fits the GPU at
 * once) followed by overflow rows: a producer waits for room only once its
 * consumer has reported progress, and otherwise writes on into the overflow
 * rows. So no producer waits on a consumer that has not started: kernels of
 * other streams or processes (other ssm2d launches too, any number of them)
 * that hold part of the GPU delay a launch but cannot block it, as long as
 * they release their compute units in time. ssm2d_scan_fwd_noalloc, when its
 * array cannot hold the overflow rows, runs the ring alone; its producers
 * may then wait on consumers that have not started, and its tickets are
 * dealt one chain at a time, so at most one chain's workgroups wait so.
 * A wait gives up after a bound (about a second; ssm2d_set_spin_limit): the
 * outputs from that point on are NaN, the next call on the same (device,
 * stream) returns SSM2D_ERR_DEVICE_TIMEOUT without enqueueing anything (read
 * from a host-visible flag, no wait), and ssm2d_sync_check reports it too.
 *
 * Errors: every function returns a status and never throws or aborts.
 *   batch, d_inner, d_state, H or W < 0          -> SSM2D_ERR_BAD_DIM
 *   batch, d_inner, H or W == 0                  -> SSM2D_OK, nothing is launched
 *   d_state == 0                                 -> valid: y = D x
 *   d_state > SSM2D_MAX_STATE                    -> SSM2D_ERR_UNSUPPORTED
 *   H or W > SSM2D_MAX_SIDE, or a tensor of 2^31 or more elements
 *                                                -> SSM2D_ERR_UNSUPPORTED
 *   any NULL pointer when there is work          -> SSM2D_ERR_NULLPTR
 *   any pointer not 16-byte aligned              -> SSM2D_ERR_MISALIGNED
 *   workspace allocation failure                 -> SSM2D_ERR_NOMEM
 *   a kernel of an earlier call on this (device, stream) timed out
 *                                                -> SSM2D_ERR_DEVICE_TIMEOUT
 *   (ssm2d_scan_fwd_noalloc only) a workspace beyond its static array
 *                                                -> SSM2D_ERR_TOO_LARGE
 * NaN and Inf inputs are not checked; they propagate.
 */
#ifndef SSM2D_H
#define SSM2D_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM2D_MAX_STATE 64
#define SSM2D_MAX_STATE_BWD 32   /* states the backward's kernels hold at once */
#define SSM2D_MAX_SIDE 65535

typedef enum {
    SSM2D_OK = 0,
    SSM2D_ERR_NULLPTR = 1,
    SSM2D_ERR_BAD_DIM = 2,
    SSM2D_ERR_UNSUPPORTED = 3,
    SSM2D_ERR_MISALIGNED = 4,
    SSM2D_ERR_HIP = 5,
    SSM2D_ERR_NOMEM = 6,
    SSM2D_ERR_DEVICE_TIMEOUT = 7,
    SSM2D_ERR_BAD_FLAGS = 8,
    SSM2D_ERR_TOO_LARGE = 9
} ssm2d_status;

/* fp32 forward: x, delta, B, C, y are float32; A, D float32; state fp32. */
int ssm2d_scan_fwd(const float *x, const float *delta, const float *A, const float *B,
                   const float *C, const float *D, float *y, int64_t batch, int64_t d_inner,
                   int64_t d_state, int64_t H, int64_t W, void *stream);

/* bf16 forward: x, delta, B, C, y are bfloat16 (raw uint16 bits); A, D float32;
 * the state and all arithmetic are fp32; y is rounded to bf16 (nearest-even). */
int ssm2d_scan_fwd_bf16(const uint16_t *x, const uint16_t *delta, const float *A,
                        const uint16_t *B, const uint16_t *C, const float *D, uint16_t *y,
                        int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                        void *stream);

/* ---- Scan direction, scan order and multi-direction sums ----------------
 *
 * The scan above starts at the upper-left corner: a cell sees the cells above
 * and to its left. The pages leave other directions and the other order as
 * variants: the papernotes.org page finds the vertical-then-horizontal order
 * about as good (消融实验要点) and notes that full context needs a reverse scan
 * from the lower right (局限与展望); the juejin.cn page (part 七, section 4)
 * lists bidirectional and four-quadrant 2D propagation. Read plainly:
 *
 *   SSM2D_FLIP_H          rows run bottom to top (h[i,j] takes h[i+1,j])
 *   SSM2D_FLIP_W          columns run right to left (hh[i,j] takes hh[i,j+1])
 *   SSM2D_VERTICAL_FIRST  v[i,j] = Abar v[i-1,j] + Bx   (column scan first)
 *                         h[i,j] = Abar h[i,j-1] + v[i,j] (row scan of its results)
 *                         ("i-1", "j-1": the previous cell in scan order)
 *   SSM2D_ACCUMULATE      y += result, instead of y = result
 *   SSM2D_FOUR_WAY        result = the sum of the four scans from the four
 *                         corners (no flip, FLIP_H, FLIP_W, both), each in the
 *                         order VERTICAL_FIRST selects, plus D x once
 *
 * State starts at zero before the first row and column in scan order. */
#define SSM2D_FLIP_H 1u
#define SSM2D_FLIP_W 2u
#define SSM2D_VERTICAL_FIRST 4u
#define SSM2D_ACCUMULATE 8u
#define SSM2D_FOUR_WAY 16u
#define SSM2D_DELTA_SOFTPLUS 32u

/* Forward pass in the direction and order `flags` selects (an OR of the bits
 * above; 0 gives ssm2d_scan_fwd). Arguments, layout, ownership, asynchrony and
 * errors as for ssm2d_scan_fwd, and also:
 *   D may be NULL: no skip term (as D = 0).
 *   SSM2D_ACCUMULATE reads y: y must hold valid values. Each cell of y is
 *     read and rewritten by one thread, so the result is y + result computed
 *     in fp32 and rounded once to y's type; deterministic.
 *   SSM2D_FOUR_WAY enqueues four kernels on `stream`, the last three
 *     accumulating; with SSM2D_ACCUMULATE the first accumulates too.
 *   Unknown bits (SSM2D_DELTA_SOFTPLUS is accepted and applies softplus to
 *   delta), or SSM2D_FOUR_WAY with SSM2D_FLIP_H or SSM2D_FLIP_W
 *                                                -> SSM2D_ERR_BAD_FLAGS
 *     (checked first, before the sizes).
 * Right-to-left and vertical-first scans run 4-column strips with 8 state
 * groups per wave whatever the shape. */
int ssm2d_scan_fwd_ex(const float *x, const float *delta, const float *A, const float *B,
                      const float *C, const float *D, float *y, int64_t batch, int64_t d_inner,
                      int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream);

/* bf16 variant of ssm2d_scan_fwd_ex: types as for ssm2d_scan_fwd_bf16. */
int ssm2d_scan_fwd_ex_bf16(const uint16_t *x, const uint16_t *delta, const float *A,
                           const uint16_t *B, const uint16_t *C, const float *D, uint16_t *y,
                           int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                           uint32_t flags, void *stream);

/* ---- Mamba selective-scan options -----------------------------------------
 *
 * The codewithpapers.app record of the paper lists selective_scan_fn (in the
 * official code's pscan_2d.py) as the code's entry point: Mamba's operator
 * of that name, whose options around the scan are, for the 2D scan:
 *   step size  delta' = delta + delta_bias[d] (delta_bias may be NULL: 0),
 *              then softplus(delta') = log(1 + e^delta') if SSM2D_DELTA_SOFTPLUS;
 *              computed in fp32 by a separate pass and kept in fp32 in a
 *              library workspace of batch*d_inner*H*W elements per
 *              (device, stream); the scan then runs on delta';
 *   gate       y = (sum_n C h + D x) * SiLU(z), SiLU(z) = z / (1 + e^-z), z
 *              shaped like x in x's type (z may be NULL: no gate);
 *   carried    h_init (may be NULL: zeros): per (b, d, n) and column, the
 *   states     vertical state before the first row in scan order (h, or v for
 *              SSM2D_VERTICAL_FIRST); h_last (may be NULL): the same state
 *              after the last row; both float32 [batch][d_inner][d_state][W].
 *              A map scanned in bands of rows, each band passed the previous
 *              band's h_last as h_init, gives the scan of the whole map (Mamba's
 *              last-state return, for maps processed in pieces).
 *   carried    hh_init (may be NULL: zeros): per (b, d, n) and row, the state
 *   row states the row recurrence starts from, before the first column in
 *              scan order (hh, or h for SSM2D_VERTICAL_FIRST); hh_last (may be
 *              NULL): the row recurrence's state after the last column; both
 *              float32 [batch][d_inner][d_state][H], indexed by memory row.
 *              A map scanned in bands of columns, each band passed the
 *              previous band's (in scan order) hh_last as hh_init, gives the
 *              scan of the whole map; with h_init / h_last too, tiles compose
 *              the same way (each tile taking the carries of its upper and
 *              left neighbours in scan order).
 * Arguments otherwise as for ssm2d_scan_fwd_ex, with the same flags (and
 * SSM2D_DELTA_SOFTPLUS). The gate applies to this call's result: with
 * SSM2D_FOUR_WAY it multiplies the four-corner sum (one more pass over y);
 * a gate with SSM2D_ACCUMULATE, carried states with SSM2D_FOUR_WAY, or
 * carried row states with a gate, SSM2D_ACCUMULATE or SSM2D_FOUR_WAY
 * -> SSM2D_ERR_BAD_FLAGS. Gated single scans use 8 state groups and 4-column
 * strips, with the gate fused into the store. h_last and hh_last are written
 * only by kernels that did not time out (see ssm2d_sync_check). */
int ssm2d_scan_fwd_mamba(const float *x, const float *delta, const float *A, const float *B,
                         const float *C, const float *D, const float *z, const float *delta_bias,
                         const float *h_init, float *h_last, const float *hh_init, float *hh_last,
                         float *y, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                         int64_t W, uint32_t flags, void *stream);

/* bf16 variant: x, delta, B, C, z, y bfloat16 bits; A, D, delta_bias, h_init,
 * h_last, hh_init, hh_last float32. With a step-size bias or softplus, and for SSM2D_FOUR_WAY
 * (also through ssm2d_scan_fwd_ex_bf16), x, B and C are widened to fp32
 * (exactly) in library workspaces, the fp32 kernels compute the result in
 * an fp32 workspace (the four scans summed there), and y is rounded to bf16
 * once, after the gate: nothing between the inputs and y is rounded to bf16.
 * A gated single scan without those options rounds once in its kernel. */
int ssm2d_scan_fwd_mamba_bf16(const uint16_t *x, const uint16_t *delta, const float *A,
                              const uint16_t *B, const uint16_t *C, const float *D,
                              const uint16_t *z, const float *delta_bias, const float *h_init,
                              float *h_last, const float *hh_init, float *hh_last, uint16_t *y,
                              int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                              uint32_t flags, void *stream);

/* ---- Backward pass -------------------------------------------------------
 *
 * Gradients of a scalar loss through ssm2d_scan_fwd, given dy = dL/dy. The
 * pages train models built on the scan but do not describe its backward pass;
 * this is the plain derivative of the forward above. Per (b, d, n), with
 * a = Abar, u = Bx, and terms outside the map zero:
 *
 *   g_h[i,j]  = dy[b,d,i,j] C[b,n,i,j] + a[i+1,j] g_h[i+1,j]   (bottom to top)
 *   g_hh[i,j] = g_h[i,j] + a[i,j+1] g_hh[i,j+1]                 (right to left)
 *   g_a       = g_hh[i,j] hh[i,j-1] + g_h[i,j] h[i-1,j]
 *   ddelta = sum_n (g_a A a + g_hh B x)      dx = sum_n g_hh delta B + dy D
 *   dA[d,n] = sum_{b,i,j} g_a delta a        dB[b,n] = sum_d g_hh delta x
 *   dC[b,n] = sum_d dy h                     dD[d] = sum_{b,i,j} dy x
 *
 * Inputs x, delta, A, B, C, D as for ssm2d_scan_fwd; dy like y. Outputs (all
 * overwritten, none may alias an input or another output): dx, ddelta like x;
 * dA like A; dB, dC like B; dD like D. Device pointers, 16-byte aligned.
 * Three kernels are enqueued on `stream`: the forward again, storing every
 * state h; the adjoint scans with the local derivatives; the sums of dB and
 * dC over channel blocks. The library keeps a workspace per (device, stream)
 * of 4 * ceil(d_inner / 8) * batch * 4 * ceil(W / 4) * H * (64 npl + 2 d_state)
 * bytes, npl = d_state / 8 rounded up to a power of two (the stored states, 4
 * bytes per state and cell at d_state = 8 npl, plus the sums over 8-channel
 * blocks for dB and dC; grown when needed, kept until ssm2d_release_workspaces
 * or the end of the process). dA and dD are accumulated with
 * atomics, so their last bits may differ from run to run; every other output
 * is deterministic.
 * More than SSM2D_MAX_STATE_BWD states (up to SSM2D_MAX_STATE): the states'
 * recurrences are independent, so the backward runs on chunks of at most
 * SSM2D_MAX_STATE_BWD states gathered into scratch tensors and sums the
 * chunks' dx and d delta (in fp32; bf16 calls are widened to fp32 first).
 * Errors as for ssm2d_scan_fwd (with d_state == 0, A, B, C, dA, dB and dC
 * are not touched and may be NULL). d_inner == 0: nothing to do. batch, H
 * or W == 0: dA and dD are zeroed, nothing else is touched. */
int ssm2d_scan_bwd(const float *x, const float *delta, const float *A, const float *B,
                   const float *C, const float *D, const float *dy, float *dx, float *ddelta,
                   float *dA, float *dB, float *dC, float *dD, int64_t batch, int64_t d_inner,
                   int64_t d_state, int64_t H, int64_t W, void *stream);

/* Backward of ssm2d_scan_fwd_ex for the scan direction and order `flags`
 * selects (SSM2D_FLIP_H, SSM2D_FLIP_W, SSM2D_VERTICAL_FIRST; 0 gives
 * ssm2d_scan_bwd): the stored-state pass runs in the forward's direction, the
 * adjoint from the opposite corner. The vertical-first scan is the
 * horizontal-first scan of the transposed maps (the flips trading places): its
 * backward transposes x, delta, dy, B and C into library workspaces (five
 * tensors, and four for the transposed gradients), runs the horizontal-first
 * backward and transposes dx, ddelta, dB and dC back. SSM2D_ACCUMULATE,
 * SSM2D_FOUR_WAY, SSM2D_DELTA_SOFTPLUS or unknown bits -> SSM2D_ERR_BAD_FLAGS
 * (a four-corner sum's gradient is the sum of the four directions'). Otherwise
 * as ssm2d_scan_bwd. */
int ssm2d_scan_bwd_ex(const float *x, const float *delta, const float *A, const float *B,
                      const float *C, const float *D, const float *dy, float *dx, float *ddelta,
                      float *dA, float *dB, float *dC, float *dD, int64_t batch, int64_t d_inner,
                      int64_t d_state, int64_t H, int64_t W, uint32_t flags, void *stream);

/* bf16 variant of ssm2d_scan_bwd_ex: types as for ssm2d_scan_bwd_bf16. */
int ssm2d_scan_bwd_ex_bf16(const uint16_t *x, const uint16_t *delta, const float *A,
                           const uint16_t *B, const uint16_t *C, const float *D, const uint16_t *dy,
                           uint16_t *dx, uint16_t *ddelta, float *dA, uint16_t *dB, uint16_t *dC,
                           float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                           int64_t W, uint32_t flags, void *stream);

/* bf16 backward: x, delta, B, C, dy, dx, ddelta, dB, dC are bfloat16 (raw
 * uint16 bits, outputs rounded to nearest even); A, D, dA, dD float32; the
 * stored states and all arithmetic fp32. */
int ssm2d_scan_bwd_bf16(const uint16_t *x, const uint16_t *delta, const float *A,
                        const uint16_t *B, const uint16_t *C, const float *D, const uint16_t *dy,
                        uint16_t *dx, uint16_t *ddelta, float *dA, uint16_t *dB, uint16_t *dC,
                        float *dD, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                        int64_t W, void *stream);

/* Backward of ssm2d_scan_fwd_mamba (a single scan; flags: SSM2D_DELTA_SOFTPLUS
 * and the direction and order flags SSM2D_FLIP_H, SSM2D_FLIP_W,
 * SSM2D_VERTICAL_FIRST of the forward): the gradients of ssm2d_scan_bwd_ex,
 * with ddelta taken with respect to the raw delta, plus dz (shaped like z;
 * required when z is given) and ddelta_bias (float32 [d_inner], may be
 * NULL; requires delta_bias). By the chain rule around the scan's backward:
 * the gate gives dz = dy * y * SiLU'(z) and passes dy * SiLU(z) on (y = the
 * ungated scan, recomputed); the step size passes d delta' back through
 * softplus (times sigmoid(delta + bias)) and sums it over cells for the bias.
 * Carried vertical states: h_init (may be NULL: zeros) the state the forward
 * started from, dh_last (may be NULL: zeros) dL/dh_last for the state it
 * handed out, dh_init (may be NULL: not computed) receives dL/dh_init; all
 * float32 [batch][d_inner][d_state][W]. The vertical adjoint starts from
 * dh_last and hands out dh_init = Abar(first row) g_h(first row); the first
 * row's decay derivative uses h_init. Carried row states likewise: hh_init,
 * dhh_last, dhh_init, float32 [batch][d_inner][d_state][H] (the row
 * adjoint starts from dhh_last and hands out Abar(first column) g_hh(first
 * column)), so a tiled forward has a tiled backward. With
 * SSM2D_VERTICAL_FIRST the two kinds trade places on the transposed map.
 * Elementwise passes run around the backward's three kernels; scratch of
 * up to three tensors shaped like x per (device, stream). ddelta_bias is
 * accumulated with atomics (last bits may vary between runs). Other flags
 * -> SSM2D_ERR_BAD_FLAGS; errors otherwise as for ssm2d_scan_bwd. */
int ssm2d_scan_bwd_mamba(const float *x, const float *delta, const float *A, const float *B,
                         const float *C, const float *D, const float *z, const float *delta_bias,
                         const float *h_init, const float *dh_last, const float *hh_init,
                         const float *dhh_last, const float *dy, float *dx, float *ddelta, float *dA,
                         float *dB, float *dC, float *dD, float *dz, float *ddelta_bias, float *dh_init,
                         float *dhh_init, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                         int64_t W, uint32_t flags, void *stream);

/* bf16 variant: x, delta, B, C, z, dy, dx, ddelta, dB, dC, dz bfloat16 bits.
 * With any option (z, delta_bias or softplus) every tensor the chain rule
 * hands on (the prepared step size, the recomputed scan output, dy * SiLU(z))
 * is kept in fp32, x, B and C are widened to fp32 (exactly) and the fp32
 * backward runs on them; each gradient is rounded to bf16 once. Without
 * options it is ssm2d_scan_bwd_bf16. */
int ssm2d_scan_bwd_mamba_bf16(const uint16_t *x, const uint16_t *delta, const float *A,
                              const uint16_t *B, const uint16_t *C, const float *D, const uint16_t *z,
                              const float *delta_bias, const float *h_init, const float *dh_last,
                              const float *hh_init, const float *dhh_last, const uint16_t *dy,
                              uint16_t *dx, uint16_t *ddelta, float *dA, uint16_t *dB, uint16_t *dC,
                              float *dD, uint16_t *dz, float *ddelta_bias, float *dh_init, float *dhh_init,
                              int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                              uint32_t flags, void *stream);

/* ---- Forward without allocation -------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not record allocations, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, layout, results and errors as
 * ssm2d_scan_fwd (fp32), and the same kernels, but the scan's workspace (head
 * words, carry ring, zero page) is a static device array of 16 MiB that each
 * GPU the library runs on holds until the process ends: this call allocates
 * nothing, on the device or for the timeout flag. On the first call on a
 * device the array's address is looked up (hipGetSymbolAddress) and the array
 * is zeroed by a kernel on `stream`.
 * Limits: the zero page holds 1 MiB (H * W <= 262128 cells) and the carry
 * ring about 15 MiB (chains of tiles that span workgroups need
 * n_chains * (workgroups per chain - 1) * ring rows * 64 lanes * 8 bytes per
 * state a lane, with 32 rows plus a row per map row where that fits, else
 * the 32 rows alone (where the grid fits the GPU at once); the giga-pixel
 * map, 384 x 512 with 128 channels and 16 states, takes the 32 rows alone:
 * 7.5 MiB). A call whose plan exceeds them returns SSM2D_ERR_TOO_LARGE and
 * enqueues nothing.
 * Every call on a GPU shares that GPU's array, whose head words (tickets,
 * tag epoch) carry over from call to call: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * Timeouts show as NaN outputs and in ssm2d_sync_check (there is no
 * host-visible flag). */
int ssm2d_scan_fwd_noalloc(const float *x, const float *delta, const float *A, const float *B,
                           const float *C, const float *D, float *y, int64_t batch, int64_t d_inner,
                           int64_t d_state, int64_t H, int64_t W, void *stream);

/* Static description of a status code. Never NULL. */
const char *ssm2d_status_string(int status);

/* Waits for `stream`, then returns and clears the timeout records of that
 * stream's workspace (the device error word and the host-visible flag), and
 * the error word of the device's ssm2d_scan_fwd_noalloc array: SSM2D_OK,
 * or SSM2D_ERR_DEVICE_TIMEOUT if a kernel gave up waiting for a neighbouring
 * tile's carries (its outputs from that point on are NaN). Returns
 * SSM2D_ERR_HIP if the wait fails. */
int ssm2d_sync_check(void *stream);

/* Waits for `stream`, then frees every workspace the library keeps for
 * (current device, stream): the scan's carry ring and zero page, the
 * backward's stored states, the scratch tensors of the option, widening and
 * transposition passes, and the host-visible timeout flag. A later call
 * allocates them again. Returns SSM2D_OK, SSM2D_ERR_DEVICE_TIMEOUT if a
 * timeout was still unreported (the workspaces are freed anyway), or
 * SSM2D_ERR_HIP. */
int ssm2d_release_workspaces(void *stream);

/* Test hook: waits for `stream` and sets the stored carry-tag epoch of that
 * stream's workspace (value modulo 65535; a launch tags with stored + 1 and
 * advances it). Setting 65534 makes the next launch that uses the carry ring
 * the last before the epoch wraps, when the ring is cleared. Returns
 * SSM2D_ERR_UNSUPPORTED if the stream has no workspace yet. */
int ssm2d_test_set_epoch(void *stream, uint32_t epoch);

/* Test hook: bound on the polls a kernel makes while waiting for carries
 * (0 = default, about one second). A tiny bound forces the timeout path. */
int ssm2d_set_spin_limit(int64_t polls);

/* Text of the last HIP runtime error behind an SSM2D_ERR_HIP status
 * ("no error" if there was none). Static storage; never NULL. */
const char *ssm2d_last_hip_error(void);

/* Which scan kernels a forward call with these sizes and flags (and no
 * gate, delta bias or carried states) launches, as the call itself plans
 * them (same environment, same device): *two_row = launches of the
 * two-rows-per-step forward (the plain scan of rows of a multiple of 4
 * columns whose layout has it), *general = launches of the general kernel,
 * *narrow = launches of the whole-row kernel (the plain scan of rows of at
 * most 16 columns with at most 16 states, on short maps or batches of at
 * least 256 waves of 16 channels).
 * bf16 != 0: the bf16 entry points (their four-corner sums and softplus step
 * sizes run fp32 kernels). No device work. Returns SSM2D_OK (all 0 for an
 * empty call), or the status the call would return for bad flags or sizes,
 * or SSM2D_ERR_NULLPTR for a null output. */
int ssm2d_fwd_kernels(int bf16, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                      uint32_t flags, int *two_row, int *general, int *narrow);

/* Test and tuning hooks (environment variables, read at each call; integers).
 * They change how the work is laid out, never what is computed:
 *   SSM2D_GROUPS=4|8     state groups per wave (default: by shape)
 *   SSM2D_STRIP=4|8      columns per strip (default: by shape)
 *   SSM2D_WAVES=n        strips per workgroup (forces chains across workgroups)
 *   SSM2D_COOP=0         per-wave input packets instead of the shared row ring
 *   SSM2D_VECSTORE=0|1   cell-by-cell output stores, or each channel's cells
 *                        gathered into wider stores (default 1; 4-column
 *                        strips only: 8-column strips always store cell by
 *                        cell)
 *   SSM2D_RING=n         rows of the bounded global carry ring (default 32;
 *                        n < 8 or n >= H: one slot a row)
 *   SSM2D_OVERFLOW=0|1|2 overflow rows after the bounded ring: none (then
 *                        producers may wait on consumers that have not
 *                        started), for consumers that have not started (1,
 *                        default), from every producer's ninth row (2, a test)
 *   SSM2D_TICKET_BLOCK=n chains per block of tickets (default: all chains
 *                        at once; without overflow rows, the most that keeps
 *                        two launches' waiting workgroups under the GPU's
 *                        slots, in 8s)
 *   SSM2D_LDSRING=4|16|32  depth of the LDS carry rings
 *   SSM2D_XCD_REMAP=0    no placement of consecutive chains on one XCD
 *   SSM2D_NARROW=0|1|2   the whole-row kernel for narrow maps: never (0),
 *                        on short maps or large batches (1, default), wherever
 *                        it applies (2)
 *   SSM2D_FAST=0|1|2     the general kernel for every plain forward (0);
 *                        the two-rows-per-step kernel for chains across
 *                        workgroups (1, default); for every layout it has (2) */

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int ssm2d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM2D_H */

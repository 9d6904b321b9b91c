/*
 * eqlinear.h -- C ABI of the group-circulant (EQ-Linear) layer over the cyclic
 * group C_T, evaluated with a group-axis DFT on AMD Instinct gfx950 (MI355X).
 *
 * What the layer computes ("Resumo Tecnico: Flash EQ-Linear", gist.science,
 * sections "Definicao do Problema" and "Insight Central"; the abstract page
 * "Flash EQ-Linear: Accelerating Equivariant Linear Layers via Group-wise
 * Discrete Fourier Transform"): the weight is one set of shared parameters
 * w[D'][C'][T] replicated under cyclic shifts into the dense matrix
 *
 *     W[d*T+g][c*T+h] = w[d][c][(g-h) mod T]
 *
 * and the layer is y = x W^T with x[N][C'*T], y[N][D'*T] (channel-major,
 * group-minor: flat column index c*T+h).  It is a circular convolution along the
 * group axis composed with a channel GEMM.  The library evaluates it exactly
 * through the convolution theorem ("Abordagem Algoritmica"): a real DFT along the
 * group axis keeping the non-redundant half spectrum, one channel GEMM per
 * frequency (real for k = 0 and k = T/2, complex otherwise), and the inverse DFT.
 * For p4 (T = 4) the transforms use only 0, +-1 and +-1/2 and the contraction is
 * six real GEMMs ("Especializacao para o Grupo de Rotacao p4").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers that the caller allocates and owns; the library
 *    allocates nothing and keeps no per-call state.  Every base pointer must be
 *    16-byte aligned (EQL_EALIGN otherwise).  Inputs and outputs must not alias.
 *  - Arrays are dense, row-major, C-contiguous, in the element type `dtype`
 *    (EQL_F32: IEEE binary32, EQL_F16: IEEE binary16).  Products accumulate in
 *    fp32 in every mode; every conversion to the output type rounds to nearest
 *    even.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call is
 *    asynchronous on that stream; the host never synchronises.  Calls are
 *    re-entrant and thread-safe.
 *  - Return value: an eql_status.  Arguments are validated before anything is
 *    launched; on any error nothing is launched and no memory is touched.
 *    N == 0 is valid and launches nothing.
 *  - Sizes: 1 <= T <= EQL_MAX_T, C' >= 1, D' >= 1, 0 <= N <= 2^31 - 2^20 (room
 *    for the kernels' 32-bit row arithmetic), and one
 *    activation row (C'*T or D'*T elements) at most 2^23 bytes; EQL_EINVAL
 *    otherwise, also when a launch would need more than 2^24 - 1 workgroups.
 */
#ifndef EQLINEAR_H
#define EQLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EQL_MAX_T 16

typedef enum { EQL_F32 = 0, EQL_F16 = 1 } eql_dtype;

/* Activation of eqlinear_fwd_fused. */
typedef enum {
    EQL_ACT_NONE = 0,
    EQL_ACT_GELU = 1    /* v * Phi(v), Phi the standard normal CDF (erf form) */
} eql_act;

typedef enum {
    EQL_PACK_FWD = 0,   /* spectrum of w, for eqlinear_fwd                     */
    EQL_PACK_BWDX = 1   /* spectrum of the transposed, group-reversed weight,   */
                        /* for eqlinear_bwd_x                                   */
} eql_pack_mode;

typedef enum {
    EQL_OK = 0,
    EQL_EINVAL = 1,       /* null pointer, size out of range, unknown dtype/mode, */
                          /* workspace too small                                 */
    EQL_EALIGN = 2,       /* a base pointer is not 16-byte aligned               */
    EQL_EUNSUPPORTED = 3, /* T > EQL_MAX_T                                        */
    EQL_EHIP = 4          /* the HIP runtime rejected a launch                    */
} eql_status;

/*
 * Packed half-spectrum weight ("Abordagem Algoritmica", steps 1-2: pointwise
 * products in the Fourier domain over the non-redundant half of the spectrum).
 *
 * For every (out, in) channel pair the packed form holds T real planes:
 *   plane 0                   : sum_t w_t                            (k = 0)
 *   plane 1 (even T > 1 only) : sum_t (-1)^t w_t                     (k = T/2)
 *   then for k = 1 .. ceil(T/2)-1, two planes:
 *                               sum_t w_t cos(2 pi t k / T)          (Re)
 *                              -sum_t w_t sin(2 pi t k / T)          (Im)
 * Each plane is stored divided by its share of the inverse transform's scale:
 * the real planes (k = 0, k = T/2) by T, the Re / Im planes by T/2 (one correctly
 * rounded fp32 division, exact for power-of-two T outside the subnormal range of
 * `dtype`).  The kernels that consume the packing then neither scale the
 * activations' transform nor the inverse; for p4 both are additions only.
 * In EQL_PACK_BWDX mode the weight is w~[c][d][t] = w[d][c][(-t) mod T]
 * (out = c, in = d), whose spectrum is the complex conjugate: the Im planes
 * change sign.
 *
 * Layout: G = 16 / sizeof(element) (8 for fp16, 4 for fp32) input channels form
 * one 16-byte group; Jin = ceil(in / G) rounded up to a multiple of 4.  Element
 * (o, i, plane p) is stored at
 *     ((o * Jin + i / G) * T + p) * G + i % G
 * and entries with i >= in are zero.  Size = out * Jin * G * T elements
 * (out * Jin * 16 * T bytes), given by eqlinear_packed_weight_bytes(out, in, T,
 * dtype); it must stay below 2^32 bytes.
 * The transform runs in fp32 and rounds once to `dtype`.
 */
size_t eqlinear_packed_weight_bytes(int64_t out_ch, int64_t in_ch, int T, int dtype);

/*
 * w: [Dp][Cp][T] (dtype), read.  w_packed: written, eqlinear_packed_weight_bytes
 * bytes with (out, in) = (Dp, Cp) for EQL_PACK_FWD, (Cp, Dp) for EQL_PACK_BWDX.
 * Called once per weight update.
 */
int eqlinear_pack_weight(const void* w, void* w_packed, int64_t Dp, int64_t Cp, int T,
                         int dtype, int mode, void* stream);

/*
 * Forward: y = x W^T ("Insight Central").  x: [N][Cp*T] read; w_packed: the
 * EQL_PACK_FWD packing of w[Dp][Cp][T]; y: [N][Dp*T] overwritten.
 * One fused kernel: group DFT of x in the GEMM prologue, per-frequency MFMA
 * GEMMs, inverse DFT (with its 1/T scaling) in the epilogue; no intermediate
 * global writes ("Implementacao": fused data flow, Fourier fragments held in
 * registers and shared memory).
 */
int eqlinear_fwd(const void* x, const void* w_packed, void* y, int64_t N, int64_t Cp,
                 int64_t Dp, int T, int dtype, void* stream);

/*
 * Forward with the epilogue of the transformer MLP blocks the layer is built into
 * ("Nivel de Rede": Flash EQ-ViT and Flash EQ-Swin), in the same single kernel:
 *     y[n][d*T+g] = act( (x W^T)[n][d*T+g] + bias[d] ) + residual[n][d*T+g]
 * x, w_packed, y, sizes and errors as eqlinear_fwd.
 * bias: [Dp] elements of `dtype`, or NULL.  One value per output channel, shared
 *   by its T group elements: a bias that varied over g would not commute with
 *   the group action.  Aligned to its element size, else EQL_EALIGN.
 * act: EQL_ACT_NONE or EQL_ACT_GELU; any other value is EQL_EINVAL.  Pointwise,
 *   so it commutes with the group action.
 * residual: [N][Dp*T] elements of `dtype`, or NULL; 16-byte aligned.  It may be
 *   the same buffer as y (an in-place residual add); any other overlap with y is
 *   undefined.
 * pre_out: [N][Dp*T] elements of `dtype`, or NULL; 16-byte aligned.  When given it
 *   receives x W^T + bias (the activation's input, rounded once), which
 *   eqlinear_fused_epilogue_bwd needs for training.
 * The bias, the activation and the residual are applied in fp32 to the fp32
 * result of the inverse transform; y is rounded once.  bias = residual = NULL
 * with EQL_ACT_NONE gives exactly eqlinear_fwd's result.
 */
int eqlinear_fwd_fused(const void* x, const void* w_packed, const void* bias,
                       const void* residual, void* y, void* pre_out, int64_t N, int64_t Cp,
                       int64_t Dp, int T, int dtype, int act, void* stream);

/*
 * Scratch bytes eqlinear_fused_epilogue_bwd needs for the bias gradient: fp32 column
 * sums of dpre, one row of Dp*T per block of rows (16 to 1024 rows, fewer rows per
 * block for small N); depends only on the arguments (0 when N == 0 or the arguments
 * are invalid).
 */
size_t eqlinear_fused_epilogue_bwd_workspace_bytes(int64_t N, int64_t Dp, int T, int dtype);

/*
 * Backward of eqlinear_fwd_fused's epilogue (the training side of "Nivel de Rede"):
 *     dpre[n][d*T+g] = dy[n][d*T+g] * act'(pre[n][d*T+g])     (act' = 1 for EQL_ACT_NONE)
 *     dbias[d]       = sum_n sum_g dpre[n][d*T+g]
 * GELU'(v) = Phi(v) + v phi(v), phi the standard normal density.  dx and dw of the
 * layer then come from eqlinear_bwd_x and eqlinear_bwd_w applied to dpre; the
 * residual's gradient is dy itself.
 * dy, pre: [N][Dp*T] read (pre only with EQL_ACT_GELU, else it may be NULL);
 * dpre: [N][Dp*T] written, may be the same buffer as dy (with EQL_ACT_NONE it then already
 * holds the result and only dbias is computed); dbias: [Dp] written, or NULL
 * (no bias gradient; zeros when N == 0); workspace: at least
 * eqlinear_fused_epilogue_bwd_workspace_bytes bytes when dbias is given.  All in
 * `dtype`, 16-byte aligned (dbias: element-aligned).  dpre is computed in fp32 and
 * rounded once; dbias adds the unrounded fp32 values: column sums per block of rows,
 * then, for each channel, its T positions in every block, in a fixed order (16
 * interleaved slices of the blocks, each in block order, then the slices in order),
 * so the result is deterministic.  Errors as the other entry points;
 * EQL_EINVAL also for an unknown act, a missing pre with EQL_ACT_GELU or a short
 * workspace.
 */
int eqlinear_fused_epilogue_bwd(const void* dy, const void* pre, void* dpre, void* dbias,
                                void* workspace, size_t ws_bytes, int64_t N, int64_t Dp, int T,
                                int dtype, int act, void* stream);

/*
 * Input gradient: dx = dy W.  dy: [N][Dp*T] read; w_packed_bwdx: the
 * EQL_PACK_BWDX packing of the same w; dx: [N][Cp*T] overwritten.  This is the
 * forward algorithm applied to the transposed, group-reversed weight (the pages'
 * backward pass, "Implementacao").
 */
int eqlinear_bwd_x(const void* dy, const void* w_packed_bwdx, void* dx, int64_t N,
                   int64_t Cp, int64_t Dp, int T, int dtype, void* stream);

/*
 * Scratch bytes eqlinear_bwd_w needs for this shape.  Depends only on the
 * arguments (0 when N == 0 or the arguments are invalid).  The workspace holds the
 * half spectra of dy and x (each about the size of that tensor: T real planes per
 * channel, rows padded to a multiple of 2 * 16 / sizeof(element), channels to a
 * multiple of the GEMM tile width: 256, or 64 where padding to 256 would add more
 * than a third of the channels) followed by fp32 partial spectra of the gradient: whole
 * Dp x Cp planes, one set per row range of the reduction over N (the real
 * frequencies and the complex pairs are split separately).
 */
size_t eqlinear_bwd_w_workspace_bytes(int64_t N, int64_t Cp, int64_t Dp, int T, int dtype);

/*
 * Weight gradient: dw[d][c][t] = sum_n sum_g dy[n][d*T+g] x[n][c*T+((g-t) mod T)],
 * the dense gradient dy^T x summed over the entries tied to w[d][c][t].  Launches:
 * the group transforms of dy and x (fp32, rounded once to `dtype`) into the
 * workspace; per frequency the channel GEMM dY_k^T conj(X_k) (K = N, fp32
 * accumulation, one partial per row range; one launch for the real frequencies and
 * one for the complex pairs); the sum of the partials in a fixed order
 * (deterministic), the inverse transform and the rounding to `dtype`.
 * x: [N][Cp*T], dy: [N][Dp*T] read; dw: [Dp][Cp][T] overwritten (zeros when
 * N == 0, which launches one small kernel); workspace: device memory of at least
 * eqlinear_bwd_w_workspace_bytes bytes, 16-byte aligned (contents on entry
 * ignored, clobbered; EQL_EINVAL if ws_bytes is smaller).
 */
int eqlinear_bwd_w(const void* x, const void* dy, void* dw, void* workspace, size_t ws_bytes,
                   int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* eqlinear_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int eqlinear_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EQLINEAR_H */

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
 *    allocates nothing and keeps no per-call state (one exception:
 *    eqlinear_fused_epilogue_bwd_noalloc's static scratch, below).  Every base pointer must be
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
    EQL_EHIP = 4,         /* the HIP runtime rejected a launch                    */
    EQL_ESCRATCH = 5      /* the shape needs more than EQL_NOALLOC_SCRATCH_BYTES   */
                          /* (eqlinear_fused_epilogue_bwd_noalloc only)           */
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
 * Layout (blocked for the forward kernels' loads): G = 16 / sizeof(element) (8 for
 * fp16, 4 for fp32) input channels form one 16-byte group j = i / G;
 * Jin = ceil(in / G) rounded up to a multiple of 4; S = Jin / 2 stages of two groups;
 * output channels form blocks of 32 (out padded to Opad = 32 * ceil(out / 32)).  With
 * b = o / 32, c = o % 32, the 16-byte unit holding group j of plane p is
 *     u(o, j, p) = ((b * S + j / 2) * T + p) * 64 + 2 c + ((j % 2) XOR ((c / 8) % 2))
 * and element (o, i, p) is stored at u(o, i / G, p) * G + i % G: per block and stage
 * one contiguous run of T * 64 units.  Entries with i >= in or o >= out are zero.
 * Size = Opad * Jin * G * T elements (Opad * Jin * 16 * T bytes), given by
 * eqlinear_packed_weight_bytes(out, in, T, dtype); it must stay below 2^32 bytes.
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
 * Both packings of w in one launch: w_packed receives the EQL_PACK_FWD packing and
 * w_packed_bwdx the EQL_PACK_BWDX one, bit-identical to two eqlinear_pack_weight calls
 * (sizes as there; all three pointers device memory, 16-byte aligned, no overlap).  For a
 * training step, which needs both.
 */
int eqlinear_pack_weight_both(const void* w, void* w_packed, void* w_packed_bwdx, int64_t Dp, int64_t Cp, int T,
                              int dtype, void* stream);

/*
 * Forward: y = x W^T ("Insight Central").  x: [N][Cp*T] read; w_packed: the
 * EQL_PACK_FWD packing of w[Dp][Cp][T]; y: [N][Dp*T] overwritten.
 * One fused kernel: group DFT of x in the GEMM prologue, per-frequency MFMA
 * GEMMs, inverse DFT (with its 1/T scaling) in the epilogue; no intermediate
 * global writes ("Implementacao": fused data flow, Fourier fragments held in
 * registers and shared memory).  The output tile width (32, 64 or 128 channels) is
 * chosen per shape; the environment variable EQL_FWD_NB=1|2|4, read once per process,
 * forces it where the shape allows (for measurement; it applies to every forward-kernel
 * launch, the input gradient's included).
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
 * eqlinear_fused_epilogue_bwd without a workspace, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc.  Same arguments, results and
 * errors as eqlinear_fused_epilogue_bwd (bit-identical outputs), minus workspace
 * and ws_bytes.  The bias gradient's row-block partials go to a static device array
 * of EQL_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends (its address is looked up on a device's first call, with
 * that device current).  Nothing is allocated per call, and nothing needs clearing:
 * every partial is written before it is read.  EQL_ESCRATCH (before anything is
 * launched) when dbias is given and the partials would not fit:
 * eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, dtype) above
 * EQL_NOALLOC_SCRATCH_BYTES (about N <= 2^20 rows at Dp * T = 4096); without
 * dbias the scratch is not used and any size is accepted.  Calls that overlap on
 * one device (on different streams, or from different threads without ordering)
 * share that scratch and race: the caller must order them.
 */
#define EQL_NOALLOC_SCRATCH_BYTES (16u << 20)
int eqlinear_fused_epilogue_bwd_noalloc(const void* dy, const void* pre, void* dpre, void* dbias, int64_t N,
                                        int64_t Dp, int T, int dtype, int act, void* stream);

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
 * arguments (0 when N == 0 or the arguments are invalid).  The layout follows the
 * path the shape takes (see eqlinear_bwd_w).  Separate path: the half spectra of dy
 * and x (each about the size of that tensor: T real planes per channel, rows padded
 * to a multiple of 2 * 16 / sizeof(element), channels to a multiple of the GEMM tile
 * width: 256, or 64 where padding to 256 would add more than a third of the
 * channels).  Fused path: x's half spectrum only, channels padded to a column tile
 * of 32 nb channels (nb in {4, 3, 2} with T nb a multiple of 4; the least padding,
 * ties to the wider tile).  Both then hold fp32 partial spectra of the gradient:
 * whole Dp x Cp planes, one set per row range of the reduction over N (on the
 * separate path the real frequencies and the complex pairs are split separately).
 */
size_t eqlinear_bwd_w_workspace_bytes(int64_t N, int64_t Cp, int64_t Dp, int T, int dtype);

/*
 * Weight gradient: dw[d][c][t] = sum_n sum_g dy[n][d*T+g] x[n][c*T+((g-t) mod T)],
 * the dense gradient dy^T x summed over the entries tied to w[d][c][t]
 * ("Resumo Tecnico: Flash EQ-Linear", "Implementacao": the gradient of the compressed weight is
 * the per-frequency product of the output-gradient spectrum with the conjugate
 * input spectrum).  Two paths compute the same sums:
 *  - separate: the group transforms of dy and x (fp32, rounded once to `dtype`) into
 *    the workspace, then per frequency the channel GEMM dY_k^T conj(X_k) (K = N,
 *    fp32 accumulation; one launch for the real frequencies, one for the complex
 *    pairs);
 *  - fused (T in {1, 2, 4}, Dp T sizeof(element) a multiple of 16, and fewer than
 *    400 real-product FLOPs per byte of x and dy, i.e. memory-bound shapes): only
 *    x's transform goes to the workspace; the GEMM reads dy's raw rows and forms
 *    their spectrum as it goes (p4 fp16: with the forward's packed fp16 butterflies,
 *    which round the two real frequencies twice; otherwise in fp32, rounded once).
 *    The environment variable EQL_BWDW_PATH=fused|separate, read once per process,
 *    overrides the choice among shapes the fused path accepts (for measurement), and
 *    EQL_BWDW_WAVES=4|8 (or <real>,<pair>, e.g. 4,8) the waves per workgroup of the
 *    separate path's GEMMs on 256-channel tiles (default 8 for both).
 * Both write one fp32 partial per row range of N, then sum the partials in a fixed
 * order (deterministic for a given shape and path), apply the inverse transform and
 * round to `dtype`.  x: [N][Cp*T], dy: [N][Dp*T] read; dw: [Dp][Cp][T] overwritten
 * (zeros when N == 0, which launches one small kernel); workspace: device memory of
 * at least eqlinear_bwd_w_workspace_bytes bytes, 16-byte aligned (contents on entry
 * ignored, clobbered; EQL_EINVAL if ws_bytes is smaller).
 */
int eqlinear_bwd_w(const void* x, const void* dy, void* dw, void* workspace, size_t ws_bytes,
                   int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream);

/*
 * A training step's three passes sharing one weight-gradient workspace, so that the
 * group transforms of x and dy are taken where the forward and the input gradient
 * already compute them, instead of by a separate pass over x and dy in the weight
 * gradient ("Resumo Tecnico: Flash EQ-Linear", "Implementacao": fused data flows with
 * no intermediate re-reads of the activations).  Arguments, results and errors as
 * eqlinear_fwd, eqlinear_bwd_x and eqlinear_bwd_w, plus `workspace` of at least
 * eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, dtype) bytes, 16-byte aligned
 * (EQL_EINVAL if ws_bytes is smaller or workspace is NULL with N > 0):
 *  - eqlinear_fwd_train writes y exactly as eqlinear_fwd, and x's half spectrum into
 *    the workspace (the operand units of the weight-gradient GEMM).  At p4 fp16 with
 *    16-byte rows the forward kernel stores the transform it has formed for its MFMAs
 *    (packed fp16 butterflies: X0 and X2 rounded twice, as in the forward); otherwise,
 *    after the forward, the weight gradient's own transform (fp32, rounded once).
 *  - eqlinear_bwd_x_train writes dx exactly as eqlinear_bwd_x and, when the shape takes
 *    the separate weight-gradient path, dy's half spectrum likewise; on the fused path
 *    (which reads dy itself) it only computes dx.
 *  - eqlinear_bwd_w_train writes dw from those spectra: the weight gradient's GEMMs and
 *    reduce without its transforms.  dy is read on the fused path only (it may be NULL
 *    on the separate path); x is not needed.
 * Contract: eqlinear_bwd_w_train's workspace must hold what eqlinear_fwd_train (for
 * this x) and eqlinear_bwd_x_train (for this dy) wrote there, for the same N, Cp, Dp,
 * T and dtype, ordered before it on the stream, with nothing else writing that memory
 * in between; the library cannot check this.  Like every entry point these only enqueue
 * work on the stream: outputs are complete when that work is.  The spectra cover every row and
 * every channel of the layer; padding units past the channel count may hold stale
 * values and only reach gradient entries that are discarded.
 */
int eqlinear_fwd_train(const void* x, const void* w_packed, void* y, void* workspace, size_t ws_bytes,
                       int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream);
int eqlinear_bwd_x_train(const void* dy, const void* w_packed_bwdx, void* dx, void* workspace, size_t ws_bytes,
                         int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream);

/*
 * eqlinear_fwd_fused with the training forward's side output: y and pre_out exactly as
 * eqlinear_fwd_fused (arguments, results and errors as there), and x's half spectrum in
 * the weight-gradient workspace as eqlinear_fwd_train leaves it (workspace and ws_bytes
 * as there).  For a layer with the fused epilogue the training step is then this call,
 * eqlinear_fused_epilogue_bwd (dpre), and eqlinear_bwd_x_train / eqlinear_bwd_w_train on
 * dpre, with the same contract as above.
 */
int eqlinear_fwd_fused_train(const void* x, const void* w_packed, const void* bias, const void* residual, void* y,
                             void* pre_out, void* workspace, size_t ws_bytes, int64_t N, int64_t Cp, int64_t Dp, int T,
                             int dtype, int act, void* stream);
int eqlinear_bwd_w_train(const void* dy, void* dw, void* workspace, size_t ws_bytes, int64_t N, int64_t Cp,
                         int64_t Dp, int T, int dtype, void* stream);

/*
 * The layer over p4m's point group (dihedral D4: four rotations r^a and four
 * reflections r^a s; r^4 = s^2 = e, s r s = r^-1).  "Resumo Tecnico: Flash EQ-Linear",
 * "Limitacoes e Trabalho Futuro", names other groups, reflection groups among them, as
 * the method's next step; the construction is kept: shared parameters w[Dp][Cp][8]
 * replicated into W[(d,g),(c,h)] = w[d][c][g h^-1].  The group axis of x, y and w lists
 * r^0, r^1, r^2, r^3, then the reflections r^-m s for m = 0..3 (s, r^3 s, r^2 s, r s):
 * x: [N][Cp*8], y: [N][Dp*8], flat index c*8 + j.
 *
 * With this order the p4m layer is exactly the C_4 layer (T = 4) with 2*Cp input and
 * 2*Dp output channels, on the same memory of x and y, whose weight w4[2*Dp][2*Cp][4]
 * is tied to w (the rotation half and the reflection half of a channel are C_4
 * channels 2c and 2c+1; the four half-to-half blocks are circular convolutions with the
 * kernels w(r^k), w(r^k s), w(r^-k s), w(r^-k)).  A p4m layer is therefore run as:
 *   forward       eqlinear_p4m_expand_weight(w -> w4), eqlinear_pack_weight(w4, ..., 2Dp,
 *                 2Cp, 4, dtype, EQL_PACK_FWD), eqlinear_fwd(x, .., y, N, 2Cp, 2Dp, 4, dtype)
 *   input grad    the EQL_PACK_BWDX packing of w4, eqlinear_bwd_x(.., N, 2Cp, 2Dp, 4, ..)
 *   weight grad   eqlinear_bwd_w(x, dy, dw4, ..., N, 2Cp, 2Dp, 4, dtype) into a
 *                 [2Dp][2Cp][4] buffer, then eqlinear_p4m_fold_weight_grad(dw4 -> dw).
 * The C_4 evaluation costs 24 real multiply-adds per (row, d, c) against 64 for the
 * dense p4m layer.
 *
 * eqlinear_p4m_expand_weight: w [Dp][Cp][8] read; w_c4 [2Dp][2Cp][4] overwritten (a
 * gather: values copied, no arithmetic).  eqlinear_p4m_fold_weight_grad: dw_c4
 * [2Dp][2Cp][4] read; dw [Dp][Cp][8] overwritten, each entry the sum of the two entries of
 * dw_c4 it is tied into, added in fp32 and rounded once to `dtype`.  Both: device
 * pointers, 16-byte aligned, in `dtype`; the sizes of the C_4 view must be valid (as for
 * the other entry points with C' = 2Cp, D' = 2Dp, T = 4); errors as there.
 */
int eqlinear_p4m_expand_weight(const void* w, void* w_c4, int64_t Dp, int64_t Cp, int dtype, void* stream);
int eqlinear_p4m_fold_weight_grad(const void* dw_c4, void* dw, int64_t Dp, int64_t Cp, int dtype, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* eqlinear_status_string(int status);

/* ABI version of this header (major * 100 + minor).  2.00: the blocked packed-weight
 * layout above (1.xx stored ((o * Jin + i / G) * T + p) * G + i % G).  2.01:
 * eqlinear_fused_epilogue_bwd_noalloc and EQL_ESCRATCH.  2.02: the p4m entry points.
 * 2.03: the training-step entry points (eqlinear_fwd_train, eqlinear_bwd_x_train,
 * eqlinear_bwd_w_train).  2.04: eqlinear_fwd_fused_train.  2.05: eqlinear_pack_weight_both. */
int eqlinear_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EQLINEAR_H */

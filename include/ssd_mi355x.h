/*
 * ssd_mi355x.h -- C ABI of the Mamba-2 SSD chunked forward for MI355X (gfx950).
 *
 * The operation (page "ops-transformer MambaV2 算子套件", §1.1 and §1.3; tensor
 * semantics of page "Mamba-2 SSD for Ascend NPU", section "Implementation"):
 * for each batch row b and head h, with group g = h / (H/G),
 *
 *   delta_t = clamp(softplus(dt[b,t,h] + dt_bias[h]), dt_min, dt_max)
 *   S_t     = exp(delta_t A[h]) S_{t-1} + delta_t x[b,t,h,:] (outer) B[b,t,g,:]
 *   out[b,t,h,:] = (S_t . C[b,t,g,:] + D[h] x[b,t,h,:]) * silu(z[b,t,h,:])
 *   final_state[b,h] = S_{L-1}
 *
 * computed chunk by chunk the way that page's §2 and §4.2-§4.5 chain it:
 * in-chunk cumulative decay (chunk_cumsum), per-chunk states (chunk_state),
 * the sequential inter-chunk recurrence (chunk_state_passing), and the
 * intra-chunk masked C.B^T product plus the inter-chunk term (chunk_scan).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, dense and
 *     row-major with the shapes given below, 16-byte aligned.  The library
 *     never allocates, frees or keeps them after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream) and the call returns without synchronising.
 *     Device faults therefore surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid or unsupported call returns an error and launches nothing.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  No exception or abort ever crosses this ABI. */
typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1,  /* NULL required pointer, dim < 1, H % G != 0,
                               misaligned pointer (cu_seqlens, and dt of
                               ssd_fwd: 4 bytes),
                               bad dtype/mma code, final_state NULL
                               while requested, a token stride below its
                               dense value or not a multiple of 16 bytes */
  SSD_ERR_UNSUPPORTED = 2,  /* valid but not compiled: headdim != 64,
                               dstate not in {64,128}, chunk not in
                               {64,128,256}, fp16 storage, or one batch
                               row of x/z/out or of B/C reaching 2 GiB
                               (rows are addressed with 32-bit offsets) */
  SSD_ERR_WORKSPACE = 3,    /* the plan needs a workspace and it is NULL,
                               smaller than required or not 16-byte
                               aligned                                */
  SSD_ERR_LAUNCH = 4        /* the HIP runtime rejected a launch       */
} ssd_status;

/* Storage dtypes. */
typedef enum { SSD_F32 = 0, SSD_F16 = 1, SSD_BF16 = 2 } ssd_dtype;

/* Matrix-core operand precision.  SSD_MMA_F16: x, B, C, the masked C.B^T
 * weights, the decay-weighted B and the carried state are rounded to fp16
 * for the MFMA products, accumulating in fp32 (the mixed precision the page
 * "Mamba-2 SSD for Ascend NPU" describes for its Cube units); every operand
 * must then lie in fp16's range (|v| <= 65504; magnitudes below about 6e-5
 * lose precision and below 6e-8 flush to zero), so fp32 or bf16 inputs
 * outside it overflow to inf or vanish.  SSD_MMA_BF16: the same operands
 * rounded to bf16 (fp32's exponent range, 8 significant bits), the precision
 * that page lists as its next extension ("Limitations and roadmap").
 * SSD_MMA_F32: every operand stays fp32 (a slower check path). */
typedef enum { SSD_MMA_F16 = 0, SSD_MMA_BF16 = 1, SSD_MMA_F32 = 2 } ssd_mma;

/* Shape, dtypes and optional inputs of one call. */
typedef struct ssd_desc {
  int64_t batch;     /* B  >= 1 */
  int64_t seqlen;    /* L  >= 1 (any length; a ragged last chunk is masked) */
  int64_t nheads;    /* H  >= 1 */
  int64_t headdim;   /* P  == 64 */
  int64_t dstate;    /* N  in {64, 128} */
  int64_t ngroups;   /* G  >= 1, H % G == 0; head h reads B/C group h/(H/G) */
  int32_t x_dtype;   /* dtype of x: SSD_F32 or SSD_BF16 */
  int32_t z_dtype;   /* dtype of z: SSD_F32 or SSD_BF16 (ignored when z NULL) */
  int32_t out_dtype; /* dtype of out: SSD_F32 or SSD_BF16 */
  int32_t mma;       /* ssd_mma */
  float dt_min;      /* dt_limit lower bound (0 for none) */
  float dt_max;      /* dt_limit upper bound (+INFINITY for none) */
  const void *z;             /* [B,L,H,P] gate, or NULL (no gate)            */
  const float *dt_bias;      /* [H] fp32, or NULL (zero)                      */
  const float *initial_state;/* [B,H,P,N] fp32, or NULL (zero state)          */
  void *workspace;           /* device scratch owned by the caller (NULL when
                                ssd_fwd_workspace_size reports 0).  Its
                                contents need no initialisation and mean
                                nothing after the call; calls that may run
                                at the same time must not share it           */
  size_t workspace_bytes;    /* its size; see ssd_fwd_workspace_size          */
  int32_t chunks_per_wg;     /* chunks one workgroup walks in sequence; 0 picks
                                automatically (see ssd_fwd_plan)              */
  int32_t bc_dtype;          /* dtype of B and C: SSD_F32 or SSD_BF16       */
  void *ev_main_begin;       /* optional hipEvent_t (as void*) recorded on the
                                stream right before the main-pass kernel, for
                                measurement; NULL records nothing             */
  void *ev_main_end;         /* optional hipEvent_t recorded right after it   */
  const int32_t *cu_seqlens; /* packed variable-length sequences, or NULL.
                                When set, `batch` sequences of different
                                lengths share one token axis: x, z, out are
                                [T,H,P], dt [T,H], B and C [T,G,N], where
                                sequence s holds tokens cu_seqlens[s] ..
                                cu_seqlens[s+1]-1 (DEVICE array of batch+1
                                int32, cu_seqlens[0] = 0, non-decreasing,
                                T = cu_seqlens[batch]).  The state starts
                                from initial_state[s] (or zero) at each
                                sequence and final_state[s] is the state
                                after its last token; initial_state and
                                final_state stay [batch,H,P,N].  `seqlen`
                                is then the longest sequence: the plan is
                                made for it.  A call whose offsets break
                                that contract (a sequence longer than
                                `seqlen`, decreasing offsets, or an offset
                                past packed_tokens when that is given)
                                leaves those sequences' results undefined
                                and sets *error_flag (below).
                                Readings of page "Mamba-2 SSD for Ascend
                                NPU", "Limitations and roadmap" (varlen,
                                cu_seqlens) and page "ops-transformer
                                MambaV2 算子套件" §1.4 (packed batches
                                delimited by cumulative offsets)          */
  int64_t packed_tokens;     /* with cu_seqlens: T, the packed token count
                                (cu_seqlens[batch]), which the plan uses to
                                spread the work of uneven lengths; 0 plans
                                as if every sequence had `seqlen` tokens.
                                Ignored for dense calls                   */
  int32_t *error_flag;       /* optional DEVICE int32, or NULL.  With
                                cu_seqlens, the kernels store 1 into it
                                when the offsets break the contract above
                                (the offsets live on the device, so this is
                                the only place such an error can surface
                                without a synchronisation); a fused-norm
                                call (norm_weight below, dense or packed)
                                stores 2 into it when its exchange timed
                                out.  The library never clears it: the
                                caller zeroes it and reads it after
                                synchronising                             */
  /* Token strides, in elements: the distance between consecutive tokens of
     x, of B (and C, the same), of z and of dt.  0 means the dense layout
     (H*P, G*N, H*P and H).  A larger stride reads these tensors as views of
     wider token-major rows in place -- for example x, B and C as column
     ranges of one conv output [B, L, H*P + 2*G*N], or z and dt inside a
     projection's output -- while out stays dense [B, L, H, P].  Batch row b
     starts b*L tokens after row 0 (for packed calls, the offsets count
     tokens).  Strides of x, B/C and z must be multiples of 16 bytes; each
     batch row's span (seqlen * stride * element size) must stay below 2 GiB.
     dt is read one element at a time: its pointer needs 4-byte alignment
     only, so it may start at any column of a wider fp32 row. */
  int64_t x_stride;
  int64_t bc_stride;
  int64_t z_stride;
  int64_t dt_stride;
  /* Fused gated RMSNorm epilogue (page "ops-transformer MambaV2 算子套件",
     §4.6 mamba2_rmsnormgated, which follows the scan in the chain of its §2):
     with norm_weight set, each token's output y (after D and the z gate,
     y * silu(z) when z is given) is normalised over groups of
     H*P/norm_groups consecutive channels and scaled per channel,
       out[t, c] = y[t, c] / sqrt(mean_{c' in group(c)} y[t, c']^2 + norm_eps)
                   * norm_weight[c],
     before its single store, so `out` is never written unnormalised.  A
     group spans k = H/norm_groups heads (k <= 32, and k <= 16 for 256-token
     chunks); when k > 1 their workgroups exchange per-token partial sums
     through the workspace, as records tagged with a per-call epoch that the
     workspace also holds.  That part of the workspace must be zero before
     the first fused call on it, and again whenever the shape or plan of the
     fused calls that use it changes (calls of one shape leave it ready for
     the next).  A fused call whose exchange does not complete within about
     20 ms stores 2 into *error_flag (when given) and leaves those rows of
     `out` undefined.  ssd_fwd_noalloc keeps this part in its own
     zero-initialised region of the scratch, which no other call touches. */
  const float *norm_weight;  /* [H*P] fp32, or NULL (no fused norm)        */
  float norm_eps;            /* > 0 and finite when norm_weight is set      */
  int32_t norm_groups;       /* >= 1, H % norm_groups == 0                  */
} ssd_desc;

/* Fills `d` with defaults for the given shape: fp32 storage (x, B, C, z,
 * out), fp16 MMA, no optional inputs, no dt_limit, automatic plan, no
 * workspace. */
void ssd_desc_init(ssd_desc *d, int64_t batch, int64_t seqlen, int64_t nheads,
                   int64_t headdim, int64_t dstate, int64_t ngroups);

/* Bytes of device workspace ssd_fwd needs for this descriptor and chunk size
 * (0 when one workgroup walks the whole sequence).  Errors as ssd_fwd's
 * validation of shapes and codes (pointers are not looked at). */
ssd_status ssd_fwd_workspace_size(const ssd_desc *d, int64_t chunk,
                                  size_t *bytes);

/* The plan ssd_fwd will use: chunks walked by one workgroup and the number
 * of such chunk groups per (b, h).  With more than one group, the states of
 * all but the last group are summed in a first pass, chained across groups
 * (page "ops-transformer MambaV2 算子套件", §4.4) and fed to the main pass. */
ssd_status ssd_fwd_plan(const ssd_desc *d, int64_t chunk,
                        int64_t *chunks_per_wg, int64_t *n_chunk_groups);

/* SSD chunked forward.
 *   x      [B,L,H,P]  x_dtype          dt  [B,L,H]  fp32 (raw step)
 *   A      [H]        fp32             B,C [B,L,G,N] x_dtype
 *   D      [H]        fp32 or NULL     chunk: 64, 128 or 256 tokens
 *   dt_softplus: nonzero applies softplus to dt + dt_bias before the clamp
 *   return_final_state: nonzero writes final_state [B,H,P,N] fp32
 *   out    [B,L,H,P]  out_dtype, fully overwritten (never accumulated)
 * The tensor semantics follow page "Mamba-2 SSD for Ascend NPU", section
 * "Implementation" (x, dt, A, B, C, initial_states, out, final_state; D, z,
 * dt_bias, dt_softplus, dt_limit, return_final_state). */
ssd_status ssd_fwd(const void *x, const float *dt, const float *A,
                   const void *B, const void *C, const float *D,
                   int64_t chunk, int dt_softplus, int return_final_state,
                   void *out, float *final_state, void *stream,
                   const ssd_desc *d);

/* Largest workspace, in bytes, that ssd_fwd_noalloc serves from its static
 * scratch (compare ssd_fwd_workspace_size against it).  The first
 * SSD_FWD_NOALLOC_SYNC_BYTES of the scratch are kept for the fused norm's
 * exchange (256 bytes plus 8 bytes per head and token of the call), the rest
 * for everything else the plan needs. */
#define SSD_FWD_NOALLOC_MAX_SCRATCH ((size_t)64 << 20)
#define SSD_FWD_NOALLOC_SYNC_BYTES ((size_t)24 << 20)

/* ssd_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and results as ssd_fwd, but the plan's
 * workspace is a static device array inside the library (one per GPU, held
 * until the process ends) instead of desc->workspace, which is ignored.  The
 * call allocates and frees nothing; on its first call on a device it looks
 * up that device's scratch address (hipGetSymbolAddress), so that device
 * must be current and the stream must belong to it.
 * Limits and errors as ssd_fwd, plus: SSD_ERR_WORKSPACE when the plan needs
 * more than SSD_FWD_NOALLOC_MAX_SCRATCH bytes (checked before any device
 * call); SSD_ERR_INVALID_ARG when the stream is not on the current device;
 * SSD_ERR_LAUNCH when the runtime cannot give the scratch address.  Every
 * call on one GPU shares its scratch, so calls that overlap on one GPU (on
 * different streams) race and must be serialised by the caller.  Only the
 * fused norm's region needs a known start: it is zero when the library
 * loads and holds nothing but tagged records and the epoch afterwards. */
ssd_status ssd_fwd_noalloc(const void *x, const float *dt, const float *A,
                           const void *B, const void *C, const float *D,
                           int64_t chunk, int dt_softplus, int return_final_state,
                           void *out, float *final_state, void *stream,
                           const ssd_desc *d);

/* Bytes of device workspace ssd_bwd needs for this descriptor (the state
 * entering every chunk, per-head dB and dC, per-row partial sums).  Errors as
 * ssd_bwd's validation of shapes and codes. */
ssd_status ssd_bwd_workspace_size(const ssd_desc *d, int64_t chunk, size_t *bytes);

/* SSD backward: gradients of L = <dout, out> + <dfinal_state, final_state>
 * (dense tensors only: the descriptor's token strides must be 0)
 * for the forward ssd_fwd computes, in fp32.  The scope is the
 * one the page "Mamba-2 SSD for Ascend NPU" gives its first backward
 * ("AscendC training", "Limitations and roadmap"): contiguous
 * P = N = chunk = 64, fp32 storage.  The descriptor gives the shape,
 * dt_bias, dt_limit, initial_state, the gate z (fp32; out = y * silu(z))
 * and the workspace (ssd_bwd_workspace_size bytes, no initialisation
 * needed); cu_seqlens must be NULL and x_dtype SSD_F32 (mma is ignored: all
 * arithmetic is fp32).
 *   inputs  x, dout [B,L,H,P]; dt [B,L,H]; A [H]; B, C [B,L,G,N]; D [H] or
 *           NULL; dfinal_state [B,H,P,N] or NULL (zero)
 *   outputs dx [B,L,H,P]; ddt [B,L,H]; dA [H]; dB, dC [B,L,G,N]; dD [H]
 *           (required when D is given); dz [B,L,H,P] (required when z is
 *           given); ddt_bias [H] (required when dt_bias is given);
 *           dinitial_state [B,H,P,N] or NULL (not written)
 * Every output is overwritten.  dA, dD and ddt_bias sum over the batch, dB
 * and dC over the heads of each group.  Results are deterministic.  The
 * descriptor's ev_main_begin/ev_main_end bracket the main backward kernel.
 * Errors:
 * SSD_ERR_INVALID_ARG for NULL required pointers or pointers not 4-byte
 * aligned; SSD_ERR_UNSUPPORTED outside the scope above; SSD_ERR_WORKSPACE
 * for a missing or short workspace. */
ssd_status ssd_bwd(const float *x, const float *dt, const float *A, const float *B,
                   const float *C, const float *D, int64_t chunk, int dt_softplus,
                   const float *dout, const float *dfinal_state, float *dx, float *ddt,
                   float *dA, float *dB, float *dC, float *dD, float *dz,
                   float *ddt_bias, float *dinitial_state, void *stream,
                   const ssd_desc *d);

/* Gated grouped RMSNorm, the operator that closes the SSD chain (page
 * "ops-transformer MambaV2 算子套件", §4.6, mamba2_rmsnormgated):
 *
 *   g   = x * silu(z)                  (g = x when z is NULL)
 *   out = g / sqrt(mean(g^2 over its group) + eps) * w
 *
 * where each row of `dim` elements splits into `ngroups` contiguous groups
 * of dim/ngroups elements, and silu(v) = v / (1 + exp(-v)).
 *   x, z, out  [rows, dim]  fp32     w [dim] fp32     eps >= 0, finite
 * rows is any product of leading dimensions (B*S for the page's [B,S,D]).
 * out may be x or z itself (in-place); w must not overlap out.  Errors:
 * SSD_ERR_INVALID_ARG for a NULL x/w/out, rows/dim/ngroups < 1, ngroups not
 * dividing dim, a negative or non-finite eps or a pointer not 16-byte
 * aligned; SSD_ERR_UNSUPPORTED when dim/ngroups is not a multiple of 4 or
 * above 4096, rows*dim reaches 2^40 elements or ceil(rows/4)*ngroups
 * reaches 2^31 (one workgroup per four rows of one group). */
ssd_status ssd_rmsnorm_gated(const float *x, const float *z, const float *w,
                             int64_t rows, int64_t dim, int64_t ngroups,
                             float eps, float *out, void *stream);

/* Depthwise causal conv1d with bias and SiLU, the step before the SSD (page
 * "ops-transformer MambaV2 算子套件", §1.4 and §4.1, mamba2_causal_conv1d):
 *
 *   out[b,d,t] = act(bias[d] + sum_{k<W} w[d,k] * xx[b,d,t-(W-1)+k])
 *
 * with act = SiLU (activation 1) or none (0), and xx = x preceded by the
 * W-1 steps of the conv state x_prev (zeros when x_prev is NULL): tap W-1
 * weighs the current step, as in a conv1d padded by W-1 and cut to S steps.
 *   x, out      [B, D, S] fp32     w [D, W] fp32     bias [D] fp32 or NULL
 *   x_prev      [B, D, W-1] fp32 or NULL (the steps before t = 0)
 *   final_state [B, D, W-1] fp32 or NULL: receives the last W-1 steps of
 *               xx (the state for the next call); it may be x_prev itself
 *               (an in-place state update) when S <= 1024.
 * Any S >= 1; S % 4 == 0 with 16-byte aligned x and out takes the vector
 * path.  out must not overlap x.  Errors: SSD_ERR_INVALID_ARG for a NULL
 * x/w/out, a dim < 1, activation not 0/1, a pointer not 4-byte aligned or a
 * forbidden overlap; SSD_ERR_UNSUPPORTED for W outside 2..4, S*4 reaching
 * 2^31 bytes, B*D*S reaching 2^40 or ceil(B*D/4)*ceil(S/1024) reaching
 * 2^31 workgroups. */
ssd_status ssd_causal_conv1d(const float *x, const float *w, const float *bias,
                             const float *x_prev, int64_t batch, int64_t dim,
                             int64_t seqlen, int64_t width, int activation,
                             float *out, float *final_state, void *stream);

/* The same convolution over token-major tensors, the layout the input
 * projection writes (page "ops-transformer MambaV2 算子套件", §1.4: x, B and
 * C leave the projection as [B, S, channels] before the conv):
 *
 *   out[b,t,d] = act(bias[d] + sum_{k<W} w[d,k] * xx[b,t-(W-1)+k,d])
 *
 *   x           [B, S, *] fp32: token (b, t) holds channels 0..D-1 at
 *               x + (b*S + t)*x_stride (x_stride >= D), so x may be a column
 *               range of a wider token-major row; 16-byte aligned
 *   out         [B, S, D] fp32 dense, 16-byte aligned
 *   w [D, W], bias [D] or NULL, x_prev / final_state [B, D, W-1] or NULL as
 *   for ssd_causal_conv1d; final_state may be x_prev itself when S <= 32.
 * Errors: SSD_ERR_INVALID_ARG for a NULL x/w/out, a size < 1, x_stride < D,
 * activation not 0/1, x or out not 16-byte aligned, another pointer not
 * 4-byte aligned or a forbidden overlap (out with x or final_state,
 * final_state with x, or with x_prev beyond the in-place case);
 * SSD_ERR_UNSUPPORTED for W outside 2..4, D or x_stride not a multiple of
 * 4, one batch's x or out reaching 2^31 bytes or 2^31 workgroups
 * (B * ceil(D/256) * ceil(S/128)). */
ssd_status ssd_causal_conv1d_tokmajor(const float *x, int64_t x_stride, const float *w,
                                      const float *bias, const float *x_prev, int64_t batch,
                                      int64_t dim, int64_t seqlen, int64_t width,
                                      int activation, float *out, float *final_state,
                                      void *stream);

/* Static, human-readable name of a status code. */
const char *ssd_status_str(int status);

/* ABI version of this header (bumped on any incompatible change). */
int ssd_abi_version(void);

#define SSD_ABI_VERSION 6

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */

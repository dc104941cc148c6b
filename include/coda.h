/*
 * coda.h -- C ABI of libcoda, the MI355X (gfx950) GEMM-epilogue hot path.
 *
 * Source of the method: the news page "CODA: New Research Optimizes
 * Transformer Training with GEMM-Epilogue Programming" (KuCoin news flash,
 * Vietnamese / Indonesian / Hindi editions).  Section "CODA: the secret in the
 * epilogue" states the problem these calls solve: in the pattern GEMM ->
 * residual add -> RMSNorm -> GEMM, the RMS row scale r is one scalar per row,
 * so it commutes with the second GEMM and can be applied at the end of it; the
 * first GEMM's epilogue then only needs partial RMS statistics, which a light
 * reduction kernel combines, and the separate RMSNorm pass disappears.  The
 * same re-parameterisation covers SwiGLU, RoPE and the cross-entropy loss.
 * Section "Five building blocks and a LEGO language" lists the epilogue
 * primitives used here: elementwise transforms (residual add, activation,
 * RoPE), vector loads (per-row / per-column broadcasts), block reductions
 * (local RMS, block log-sum-exp) and stateful max / sum-exp statistics.
 *
 * Conventions for every call below
 *   - Matrices are row-major.  Weights are stored [N, K] (row n = output
 *     feature n, K contiguous), so a linear layer computes X . W^T.
 *   - bf16 tensors are passed as raw 16-bit patterns; e4m3 tensors are OCP
 *     E4M3FN byte codes.  Accumulation is fp32.  Stores round to nearest even.
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises; each call enqueues its
 *     kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     returns.  Results are visible after the caller synchronises the stream.
 *   - Return value: CODA_OK (0) or a negative coda_status.  Arguments are
 *     validated BEFORE any HIP runtime call, so a bad argument never launches
 *     anything.  NaN / Inf inputs are not detected: they propagate as NaN
 *     into the affected rows only.  A label outside [0, V) marks a row that
 *     carries no loss (loss 0) in both cross-entropy calls.
 *   - Matrix pointers must be 16-byte aligned, float / int vectors 4-byte
 *     aligned.  Outputs must not alias inputs.
 *   - Calls keep no global mutable state and are thread-safe; calls on
 *     different streams may overlap.  The one exception is
 *     coda_gemm_block_lse_noalloc, whose partials live in a static scratch
 *     array that every call on one GPU shares: such calls must not overlap.
 */
#ifndef CODA_H
#define CODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CODA_OK = 0,
  CODA_ERR_NULL = -1,    /* a required pointer is NULL */
  CODA_ERR_SHAPE = -2,   /* a size is out of range or not a required multiple */
  CODA_ERR_DTYPE = -3,   /* unknown or unsupported number format */
  CODA_ERR_ALIGN = -4,   /* a pointer is not aligned as required */
  CODA_ERR_DEVICE = -5,  /* current device is not gfx950 or cannot be queried */
  CODA_ERR_LAUNCH = -6   /* the HIP runtime reported an error at launch */
} coda_status;

typedef enum {
  CODA_BF16 = 0,     /* bfloat16 operands */
  CODA_FP8_E4M3 = 1  /* OCP E4M3FN operands with one fp32 scale per tensor */
} coda_dtype;

/* Library version of this ABI (increases on incompatible change). */
int coda_abi_version(void);

/* Static description of a status code (never NULL). */
const char* coda_status_string(int status);

/* Width, in output features, of one partial sum-of-squares tile. */
int coda_rms_tile_width(void);
/* T = number of partial sum-of-squares tiles per row for N features. */
int coda_rms_tiles(int N);
/* Width, in vocabulary entries, of one log-sum-exp tile. */
int coda_lse_tile_width(void);
/* T_v = number of log-sum-exp tiles per row for a vocabulary of V. */
int coda_lse_tiles(int V);

/*
 * GEMM1 with the residual / partial-RMS epilogue.
 * Page section "CODA: the secret in the epilogue" (first GEMM of
 * GEMM-RMSNorm-GEMM computes only a partial RMS in its epilogue) and section
 * "Five building blocks and a LEGO language" (elementwise residual add; block
 * reduction "local RMS").
 *
 *   h[m,n]            = residual[m,n] + (A[m,:] . W[n,:]) * sa * sw   (stored bf16)
 *   partial_sumsq[t*M+m] = sum over n in tile t of h[m,n]^2, from the fp32
 *                        value before rounding; tile t covers features
 *                        [t*w, t*w+w), w = coda_rms_tile_width()
 * bf16:  A [M,K] bf16, W [N,K] bf16; a_scale, w_scale, h8_scale, h8 and
 *        partial_amax must be NULL (sa = sw = 1).
 * fp8:   A [M,K] e4m3, W [N,K] e4m3, *a_scale / *w_scale their fp32 scales
 *        (device scalars).  Additionally, if h8 != NULL:
 *          h8[m,n] = E4M3(h[m,n] / *h8_scale), rounded to nearest even and
 *                    saturated to +-448 (h8_scale: device scalar, typically the
 *                    h8_scale_out of the previous coda_rms_reduce -- delayed
 *                    scaling), and, if partial_amax != NULL,
 *          partial_amax[t*M+m] = max over n in tile t of |h[m,n]|.
 * residual, h: [M,N] bf16.  partial_sumsq: [T,M] fp32, T = coda_rms_tiles(N).
 * Sizes: M >= 1; N >= 16, N % 16 == 0; K >= 64, K % 64 == 0 (fp8: K % 128);
 *        M*K, N*K, M*N element counts below 2^30.
 */
int coda_gemm_residual_partialrms(int dtype, const void* A, const void* W,
                                  const float* a_scale, const float* w_scale,
                                  const void* residual, void* h, float* partial_sumsq,
                                  const float* h8_scale, void* h8, float* partial_amax,
                                  int M, int N, int K, void* stream);

/*
 * The light reduction kernel that combines the partial RMS statistics
 * (page section "CODA: the secret in the epilogue").
 *   r[m] = 1 / sqrt( (sum_t partial_sumsq[t*M+m]) / N + eps )
 * If partial_amax != NULL (fp8 path), also
 *   *h_amax       = max over all t, m of partial_amax[t*M+m]
 *   *h8_scale_out = *h_amax / 448            (both device scalars; required)
 * partial_sumsq: [T,M] fp32 as written by coda_gemm_residual_partialrms.
 * Sizes: T >= 1, M >= 1, N >= 1; eps >= 0.
 */
int coda_rms_reduce(const float* partial_sumsq, const float* partial_amax, int T, int M, int N,
                    float eps, float* r, float* h_amax, float* h8_scale_out, void* stream);

/*
 * GEMM2 with the row-scale + SwiGLU epilogue (page section "CODA: the secret
 * in the epilogue": r moved from before the second GEMM to its end; SwiGLU
 * re-parameterised the same way).  The RMSNorm gain gamma is folded into the
 * weights' columns beforehand (coda_fold_gamma), since it lies along K.
 *   g[m,n] = r[m] * (X[m,:] . Wg[n,:]) * sx * sg
 *   u[m,n] = r[m] * (X[m,:] . Wu[n,:]) * sx * su
 *   out[m,n] = silu(g) * u,  silu(z) = z / (1 + e^-z)      (stored bf16)
 * g and u are never stored.
 * bf16: X [M,K] bf16 (the stored h), Wg, Wu [N,K] bf16; scales NULL.
 * fp8:  X [M,K] e4m3 (h8), Wg, Wu e4m3; x_scale, wg_scale, wu_scale device
 *       fp32 scalars (x_scale = the h8_scale used to write X).
 * r: [M] fp32.  out: [M,N] bf16.
 * Sizes: M >= 1; N >= 16, N % 16 == 0; K >= 64, K % 64 == 0 (fp8: K % 128).
 */
int coda_gemm_rowscale_swiglu(int dtype, const void* X, const float* x_scale, const void* Wg,
                              const void* Wu, const float* wg_scale, const float* wu_scale,
                              const float* r, void* out, int M, int N, int K, void* stream);

/*
 * QKV GEMM with the row-scale + RoPE epilogue (page section "CODA: the
 * secret in the epilogue": RoPE re-parameterised into the epilogue; section
 * "Five building blocks and a LEGO language": RoPE as an elementwise
 * transform).
 *   y[m,c]   = r[m] * (h[m,:] . Wqkv[c,:]),  c in [0, (nq + 2 nkv) * hd)
 *   columns are q heads | k heads | v heads, hd columns per head;
 *   for every q and k head and i < hd/2 (rotate-half pairs (i, i + hd/2)),
 *   with p = pos[m], c = rope_cos[p*(hd/2) + i], s = rope_sin[p*(hd/2) + i]:
 *     qkv[.., i]        = y_i c - y_{i+hd/2} s
 *     qkv[.., i + hd/2] = y_{i+hd/2} c + y_i s
 *   v heads are stored unrotated.                           (stored bf16)
 * h [M,K] bf16, Wqkv [(nq+2nkv)hd, K] bf16 (gamma folded in), r [M] fp32,
 * rope_cos / rope_sin [max_pos, hd/2] fp32 (coda_rope_tables; 16-byte aligned),
 * pos [M] int32 in [0, max_pos) (a position outside is clamped into the table),
 * qkv [M, (nq+2nkv)hd] bf16.
 * Sizes: head_dim 64 or 128; nq, nkv >= 1; K % 64 == 0; M >= 1.
 */
int coda_gemm_rope(const void* h, const void* Wqkv, const float* r, const float* rope_cos,
                   const float* rope_sin, const int32_t* pos, int max_pos, void* qkv, int M,
                   int K, int n_q_heads, int n_kv_heads, int head_dim, void* stream);

/*
 * LM-head GEMM with the block log-sum-exp epilogue and the merge (page
 * section "CODA: the secret in the epilogue": cross-entropy re-parameterised;
 * section "Five building blocks and a LEGO language": block log-sum-exp
 * reduction and the running max / sum-exp statistics).
 *   z[m,v] = r[m] * (X[m,:] . W[v,:])   (r == NULL means r = 1; r > 0, as an
 *            RMS scale is: the tile max is taken before scaling); z never stored
 *   per tile t of w = coda_lse_tile_width() vocabulary entries:
 *     tile_max[t*M+m]    = max over v in tile of z[m,v]
 *     tile_sumexp[t*M+m] = sum over v in tile of exp(z[m,v] - tile_max)
 *   label_logit[m] = z[m, labels[m]], from the fp32 accumulator
 *   lse[m]  = M_m + ln sum_t tile_sumexp * exp(tile_max - M_m), M_m = max_t tile_max
 *   loss[m] = lse[m] - label_logit[m]        (natural log, one value per row)
 *   a label outside [0,V) (e.g. an ignore index such as -100) marks a row that
 *   carries no loss: loss[m] = 0, lse[m] is still written and label_logit[m]
 *   is neither written nor read
 * X [M,K] bf16, W [V,K] bf16, labels [M] int32,
 * tile_max, tile_sumexp [T_v, M] fp32 workspace (T_v = coda_lse_tiles(V)),
 * label_logit, loss [M] fp32, lse [M] fp32 or NULL.
 * Sizes: M >= 1; V >= 16, V % 16 == 0; K % 64 == 0.
 */
int coda_gemm_block_lse(const void* X, const void* W, const float* r, const int32_t* labels,
                        float* tile_max, float* tile_sumexp, float* label_logit, float* lse,
                        float* loss, int M, int V, int K, void* stream);

/* coda_gemm_block_lse for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results (lse, loss), with the per-tile (max, sum-exp) partials
 * and the label logits kept in a scratch array of the library instead of
 * caller workspace.  The array is a static device global of
 * coda_lse_noalloc_max_bytes() bytes (64 MiB) that each GPU the library runs
 * on holds until the process ends; the call allocates and frees nothing.
 * Needs 2 * round256(4 T_v M) + round256(4 M) bytes of it (T_v =
 * coda_lse_tiles(V)); larger sizes return CODA_ERR_SHAPE (M = 8192 at
 * V = 128256 fits).  Nothing in the scratch needs clearing: every entry a
 * call reads is written by that call.  All calls on one GPU share its
 * scratch, so calls that overlap on one GPU (e.g. on two streams) race;
 * order them on one stream.  Other arguments as coda_gemm_block_lse. */
size_t coda_lse_noalloc_max_bytes(void);
int coda_gemm_block_lse_noalloc(const void* X, const void* W, const float* r,
                                const int32_t* labels, float* lse, float* loss, int M, int V,
                                int K, void* stream);

/* Causal grouped-query attention forward, the attention core between the
 * QKV+RoPE GEMM and the output-projection GEMM of a full layer (page section
 * "What CODA can do": the method re-parameterises every operator but
 * attention; this is the plain attention the layer needs):
 *   o[m, h hd + e] = sum_{j <= i} softmax_j( q_i . k_j / sqrt(hd) ) v_j[e]
 * for query m = s L + i of sequence s (rows [s L, (s+1) L) form a sequence),
 * q = qkv[m, h hd ..], k, v of kv head h / (n_q / n_kv) from the k and v
 * parts of qkv (the layout coda_gemm_rope writes: q | k | v).  fp32 scores
 * and statistics, P rounded to bf16 for the P V product, bf16 output.
 * qkv [M, (n_q + 2 n_kv) hd] bf16, o [M, n_q hd] bf16, 16-byte aligned.
 * Sizes: head_dim 64 or 128; n_q % n_kv == 0; seq_len % 128 == 0;
 * M % seq_len == 0. */
int coda_attention_fwd(const void* qkv, void* o, int M, int seq_len, int n_q_heads,
                       int n_kv_heads, int head_dim, void* stream);

/* ---- backward of the MLP sub-layer ----
 *
 * Page section "CODA: the secret in the epilogue": when the forward tail is
 * block-local the backward pass inherits the same structure; section
 * "Experimental results": backward kernels of SwiGLU and of GEMM-Residual-PartialRMS-GEMM.
 * The page prints no formulas; these calls compute the chain rule of
 *   h = res + x Wo^T,  z = [g | u] = r h W'^T,  W' = [Wg; Wu] diag(gamma),
 *   out = silu(g) u,   next = h + out Wd^T
 * given dY = dL/dnext [M, d] (bf16).  Weights enter transposed copies (the
 * GEMMs read K-contiguous rows): WdT = Wd^T [ffn, d], W2T = W'^T [d, 2 ffn].
 * The sequence is
 *   coda_gemm_rowscale_swiglu_save  (forward, keeps z)
 *   coda_gemm_swiglu_bwd -> coda_rms_bwd_reduce -> coda_gemm_rmsnorm_bwd
 * and then dx = dh Wo is a plain GEMM with Wo^T (coda_gemm_bf16).  The weight
 * gradients reduce over the tokens and have no epilogue: token-major copies
 * (coda_transpose_bf16; the row scale r is applied while copying h) and plain
 * GEMMs (coda_gemm_bf16, or coda_gemm_bf16_splitk where the output has too few
 * tiles) give dWd = dY^T out, dW' = dz^T (r h) and dWo = dh^T x.
 */

/* coda_gemm_rowscale_swiglu (bf16) that also stores the pre-activations for
 * the backward pass (section "Five building blocks and a LEGO language": tile
 * stores that keep intermediate activations):
 *   gu[m, n] = bf16(g[m,n]),  gu[m, N + n] = bf16(u[m,n])
 * X [M,K], Wg, Wu [N,K] bf16 (gamma folded), r [M] fp32, out [M,N] bf16,
 * gu [M, 2N] bf16.  Sizes as coda_gemm_rowscale_swiglu (bf16). */
int coda_gemm_rowscale_swiglu_save(const void* X, const void* Wg, const void* Wu, const float* r,
                                   void* out, void* gu, int M, int N, int K, void* stream);

/* SwiGLU backward as the epilogue of the GEMM that forms dout = dY Wd:
 *   dout[m,n] = dY[m,:] . WdT[n,:]                    (fp32, never stored)
 *   s = 1/(1+e^-g),  du = dout silu(g),  dg = dout u (s + silu(g)(1 - s))
 *   dz[m, n] = bf16(dg),  dz[m, N + n] = bf16(du)     (g, u read from gu)
 *   partial_dot[t*M + m] = sum over n in tile t of (dg g + du u)   (fp32)
 * with tiles of coda_rms_tile_width() features, T = coda_rms_tiles(N).
 * dY [M,K] bf16 (K = d), WdT [N,K] bf16 (N = ffn), gu [M,2N] bf16 (from
 * coda_gemm_rowscale_swiglu_save), dz [M,2N] bf16, partial_dot [T,M] fp32.
 * Sizes: M >= 1; N >= 16, N % 16 == 0; K >= 64, K % 64 == 0. */
int coda_gemm_swiglu_bwd(const void* dY, const void* WdT, const void* gu, void* dz,
                         float* partial_dot, int M, int N, int K, void* stream);

/* Row coefficient of the RMSNorm backward, the light reduction of the
 * SwiGLU-backward partial sums:
 *   c[m] = r[m]^2 / N * sum_{t < T} partial_dot[t*M + m]
 * which equals (r^3 / N) sum_j h_j G_j with G = dz W' (sum_j h_j G_j =
 * sum_n dz_n z_n / r).  N = d, the normalised width; r [M] the forward row
 * scale; partial_dot [T,M], c [M] fp32.  Sizes: T, M, N >= 1. */
int coda_rms_bwd_reduce(const float* partial_dot, int T, int M, const float* r, int N, float* c,
                        void* stream);

/* RMSNorm backward and skip connection as the epilogue of the GEMM that forms
 * G = dz W':
 *   dh[m,n] = bf16( r[m] (dz[m,:] . W2T[n,:]) - c[m] h[m,n] + dY[m,n] )
 * dh is also dres, and dy for the GEMM before (dx = dh Wo).
 * dz [M,K] bf16 (K = 2 ffn), W2T [N,K] bf16 (N = d, gamma folded), h [M,N]
 * bf16 (the forward h), dY [M,N] bf16, r, c [M] fp32, dh [M,N] bf16.
 * Sizes: M >= 1; N >= 16, N % 16 == 0; K >= 64, K % 64 == 0. */
int coda_gemm_rmsnorm_bwd(const void* dz, const void* W2T, const void* h, const void* dY,
                          const float* r, const float* c, void* dh, int M, int N, int K,
                          void* stream);

/* Weight gradient of the gamma-folded gate|up weight W' = W diag(gamma), with
 * the gradient of the RMSNorm gain as its epilogue (section "What CODA can
 * do": RMSNorm gradients; section "Five building blocks and a LEGO language":
 * block reduction).  The GEMM reduces over the tokens:
 *   G[n,k] = A[n,:] . B[k,:]            (fp32, never stored; G = dW' = dz^T (r h))
 *   dW[n,k] = bf16( G[n,k] * gamma[k] )  (the gradient of the unfolded W)
 *   partial_dgamma[p*N + k] = sum over n in [128 p, 128 p + 128) of G[n,k] W[n,k]
 * A [M,K] bf16 = dz^T (M = 2 ffn rows, K = tokens), B [N,K] bf16 = (r h)^T
 * (N = d), W [M,N] bf16 = the unfolded [Wg; Wu], gamma [N] fp32, dW [M,N]
 * bf16, partial_dgamma [P,N] fp32 with P = coda_dgamma_slices(M).  Then
 * coda_dgamma_reduce(partial_dgamma, P, N, NULL, dgamma) gives
 * dgamma[k] = sum_n G[n,k] W[n,k] (W'[n,k] = W[n,k] gamma[k]).
 * Sizes as coda_gemm_bf16; partial_dgamma 16-byte aligned. */
int coda_dgamma_slices(int M);
int coda_gemm_wgrad_gamma(const void* A, const void* B, const void* W, const float* gamma,
                          void* dW, float* partial_dgamma, int M, int N, int K, void* stream);

/* dgamma[k] = sum_{p < P} partial[p*N + k], summed in slice order
 * (deterministic), divided by gamma_div[k] when gamma_div is not NULL (the
 * unfused form, whose partial sums hold dW * W with dW = dW' gamma; gamma_div
 * must then have no zero entry).  partial [P,N], dgamma, gamma_div [N] fp32.
 * Sizes: P, N >= 1. */
int coda_dgamma_reduce(const float* partial, int P, int N, const float* gamma_div, float* dgamma,
                       void* stream);

/* ---- weight preparation (run once per weight update, not per token) ---- */

/* W_out[n,k] = bf16( W[n,k] * gamma[k] ): folds the RMSNorm gain, which lies
 * along GEMM2's K axis, into the weight columns.  W, W_out [N,K] bf16,
 * gamma [K] fp32.  Sizes: N, K >= 1, K % 8 == 0. */
int coda_fold_gamma(const void* W, const float* gamma, void* W_out, int N, int K, void* stream);

/* dst[c * ld_dst + r] = src[r * cols + c]: bf16 transpose of src [rows, cols]
 * into the first `rows` columns of dst [cols, ld_dst] (ld_dst >= rows).  With
 * row_scale [rows] fp32 (else NULL) each row is scaled first and rounded once:
 * dst[c * ld_dst + r] = bf16(src[r * cols + c] * row_scale[r]).
 * Used for the transposed weight copies the backward GEMMs read (Wd^T, W'^T,
 * Wo^T) and for the token-major operands of the weight gradients, which are
 * plain GEMMs reducing over the tokens (coda_gemm_bf16):
 *   dWd = dY^T out,  dW' = dz^T (r h) (row_scale = r: the RMS row scale moves
 *   onto the reduction axis),  dWo = dh^T x.
 * Sizes: rows, cols >= 1; rows * cols and cols * ld_dst below 2^31. */
int coda_transpose_bf16(const void* src, const float* row_scale, int rows, int cols, void* dst,
                        int ld_dst, void* stream);

/* The plain GEMM of coda_gemm_bf16 with its reduction split in `parts`
 * ranges, for the weight gradients, whose outputs (d x d at d = 2048: 64
 * tiles of 256 x 256) are too small to occupy every compute unit while the
 * reduction runs over all tokens:
 *   workspace[p, m, n] = sum over k in [p K/parts, (p+1) K/parts) of
 *                        A[m,k] W[n,k]                         (fp32)
 *   C[m, n] = bf16( ((workspace[0,m,n] + workspace[1,m,n]) + ...) )
 * summed in part order for every element (deterministic; equal to
 * coda_gemm_bf16 up to the rounding of the fp32 sums).  A [M,K], W [N,K],
 * C [M,N] bf16; workspace [parts, M, N] fp32, owned by the caller, written
 * whole before it is read (no clearing needed), left holding the partial
 * products.  Two kernels on `stream`; calls that share a workspace must be
 * ordered on one stream.  Sizes as coda_gemm_bf16 with 1 <= parts <= 16,
 * K % (64 parts) == 0 and min(M, 256) * N * 4 below 2^31; 16-byte aligned
 * pointers. */
int coda_gemm_bf16_splitk(const void* A, const void* W, void* C, float* workspace, int M, int N,
                          int K, int parts, void* stream);

/* rope_cos/rope_sin[p*(hd/2)+i] = cos/sin(p * theta^(-2i/hd)), angles and
 * trigonometry in fp64, stored fp32.  Sizes: max_pos >= 1, head_dim even. */
int coda_rope_tables(double theta, int max_pos, int head_dim, float* rope_cos, float* rope_sin,
                     void* stream);

/* ---- the unfused sequence: one HBM round trip per op (speed baseline) ---- */

/* C[m,n] = bf16( A[m,:] . W[n,:] ) -- the same mainloop, plain store.
 * Sizes as coda_gemm_residual_partialrms (bf16). */
int coda_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, void* stream);
/* partial[p*N + k] = sum over rows n in [128 p, 128 p + 128) of X[n,k] Y[n,k]
 * (fp32 sums of bf16 products), P = coda_dgamma_slices(M) slices: the
 * unfused counterpart of the coda_gemm_wgrad_gamma epilogue (X = a stored
 * weight gradient, Y = the weight).  X, Y [M,N] bf16; N % 8 == 0. */
int coda_col_dot_partial(const void* X, const void* Y, int M, int N, float* partial, void* stream);
/* h = bf16(y + res), all [count] bf16; count % 8 == 0. */
int coda_residual_add(const void* y, const void* res, void* h, int64_t count, void* stream);
/* out[m,n] = bf16( h[m,n] * r_m * gamma[n] ), r_m = 1/sqrt(mean_n h^2 + eps).
 * h, out [M,N] bf16; gamma [N] fp32; N % 8 == 0. */
int coda_rmsnorm(const void* h, const float* gamma, float eps, void* out, int M, int N,
                 void* stream);
/* out[m,n] = bf16( silu(gu[m,n]) * gu[m,N+n] ); gu [M,2N], out [M,N] bf16; N % 8 == 0. */
int coda_swiglu(const void* gu, void* out, int M, int N, void* stream);
/* SwiGLU backward from a stored dout [M,N] bf16 and gu [M,2N]: dz [M,2N] as
 * coda_gemm_swiglu_bwd writes it (no partial sums).  N % 8 == 0. */
int coda_swiglu_bwd(const void* dout, const void* gu, void* dz, int M, int N, void* stream);
/* RMSNorm backward from a stored G = dz W' [M,N] bf16, one pass per row that
 * also recomputes the row scale from h:  r = 1/sqrt(mean_n h^2 + eps),
 *   dh = bf16( r G - (r^3 / N) (sum_j h_j G_j) h + dY )
 * G, h, dY, dh [M,N] bf16.  N % 8 == 0, N <= 16384. */
int coda_rmsnorm_bwd(const void* G, const void* h, const void* dY, float eps, void* dh, int M,
                     int N, void* stream);
/* C[m, n] = bf16( A[m,:] . W[n,:] * a_scale * w_scale ), e4m3 operands A [M,K], W [N,K],
 * device fp32 scalars a_scale, w_scale; C rows ldc elements apart (ldc >= N, ldc % 8 == 0).
 * Sizes as coda_gemm_residual_partialrms (fp8: K % 128). */
int coda_gemm_fp8(const void* A, const void* W, const float* a_scale, const float* w_scale,
                  void* C, int ldc, int M, int N, int K, void* stream);
/* out[i] = E4M3_sat( x[i] / *s_in ) (x bf16, out e4m3 bytes, count elements, count % 8 == 0);
 * *amax = max |x|, *s_out = *amax / 448 (1 if amax is 0): delayed scaling, the next call's s_in. */
int coda_quantize_e4m3(const void* x, int64_t count, const float* s_in, void* out, float* amax,
                       float* s_out, void* stream);
/* In place on a stored qkv [M, (nq+2nkv)*hd] bf16 (as a plain GEMM writes it): the
 * rotate-half RoPE of coda_gemm_rope on the q and k heads, each pair rounded to bf16
 * again.  Tables, positions and sizes as coda_gemm_rope (head_dim 64 or 128). */
int coda_rope_apply(void* qkv, const float* rope_cos, const float* rope_sin, const int32_t* pos,
                    int max_pos, int M, int n_q_heads, int n_kv_heads, int head_dim, void* stream);
/* Cross entropy of stored bf16 logits z [M,V] (as a plain GEMM writes them):
 *   lse[m] = ln sum_v exp z[m,v],  loss[m] = lse[m] - z[m, labels[m]]
 * labels [M] int32; a label outside [0,V) gives loss[m] = 0 (as coda_gemm_block_lse);
 * lse, loss [M] fp32; V % 8 == 0. */
int coda_cross_entropy_rows(const void* logits, const int32_t* labels, float* lse, float* loss,
                            int M, int V, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H */

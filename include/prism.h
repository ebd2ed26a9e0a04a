/*
 * prism.h -- C ABI of libprism.so: Prism's dynamic block-sparse video self-attention for
 * one layer and one group of heads, on AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2610.05416, "Prism: Dynamic Sparse Attention for Native 2K Joint
 * Video-Audio Generation Model Training"), as described by the nanless audio-paper-digest
 * post and the xyznot.com review:
 *   1. the T x H x W video token grid is cut into 8 x 8 x 8 macro-zones (digest, pipeline
 *      section and Fig. 2);
 *   2. per zone and head, a variation indicator g_d = r_{v,d} + a_bar * v_hat_{a,d} + eps
 *      from the channel variance of axis-pooled V and from the audio-to-video
 *      cross-attention norm field (digest, guidance section, Eq. g_d; review, "Метод"
 *      item 1);
 *   3. a block volume B in {64, 128, 256} from the normalised information density rho
 *      (thresholds 0.5 and 0.25) and the candidate shape nearest in log2 space to the
 *      closed-form optimum of the shape loss J (digest, density section, Eq. rho_raw and
 *      Eq. J; review item 2);
 *   4. a permutation making every block contiguous (shared by Q, K, V), mean-pooled block
 *      representatives, block scores, and Top-k union Top-p key-block selection per query
 *      block (digest, selection section; review item 3);
 *   5. exact attention over the selected key blocks with an online softmax, forward and
 *      backward, the plan held constant for the gradient (digest, selection and training
 *      sections), and the inverse permutation of the outputs.
 *
 * Conventions shared by every entry point
 *   - Token order is raster over (t, h, w) with w fastest: n = (t*H + h)*W + w.
 *   - Token tensors (q, k, v, o, dout, dq, dk, dv) are dense row-major [N][heads][D] in the
 *     configured dtype (float32 or bfloat16); lse is float32 [heads][N]; the A2V norm
 *     field is float32 [N] shared by all heads.
 *   - All pointers are device pointers.  The caller owns every buffer, including the
 *     workspace; the library allocates no device memory.
 *   - Calls are asynchronous on the caller's HIP stream (a hipStream_t passed as void*,
 *     NULL = the null stream) and never synchronise the host, except prism_check_flags.
 *   - Arguments are checked before any launch; a rejected call launches nothing and
 *     returns a negative status.  No exception crosses this boundary.
 *   - A call is thread-safe as long as concurrent calls use distinct workspaces.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PRISM_OK = 0,
    PRISM_ERR_ARG = -1,          /* null pointer, bad size, inconsistent configuration */
    PRISM_ERR_UNSUPPORTED = -2,  /* grid not a multiple of 8, head_dim / dtype not built */
    PRISM_ERR_WORKSPACE = -3,    /* workspace smaller than prism_workspace_bytes() */
    PRISM_ERR_HIP = -4,          /* a HIP launch failed; see prism_last_error() */
    PRISM_ERR_STATE = -5,        /* call out of order for this workspace: a forward with no
                                    prism_plan of the same configuration on it, or a
                                    backward with no forward since its last plan */
    PRISM_ERR_RANGE = -6         /* prism_check_flags: some head's flags are set (inputs
                                    outside the float16 operand range, or more selected
                                    block pairs than max_pairs); its outputs are NaN */
} prism_status;

typedef enum { PRISM_F32 = 0, PRISM_BF16 = 1 } prism_dtype;

typedef struct prism_config {
    int T, H, W;          /* video latent grid; each a positive multiple of 8 (zone edge) */
    int num_heads;        /* heads handled by one call, each with its own plan */
    int head_dim;         /* D: 64 or 128, both dtypes */
    int dtype;            /* prism_dtype of every token tensor */
    int min_edge_log2;    /* 1: edges {2,4,8}, 16 candidate shapes (the pages' pool);
                             0: edges {1,2,4,8}, 19 shapes */
    int top_k;            /* Top-k in key blocks (>= number of blocks keeps all) */
    float top_p;          /* Top-p cumulative block relevance; 0 leaves Top-k alone */
    float tau128;         /* rho >= tau128 -> B = 64 (pages: 0.5) */
    float tau256;         /* tau256 <= rho < tau128 -> B = 128, else 256 (pages: 0.25) */
    double eps;           /* epsilon in g_d (pages give no value; default 1e-6) */
    float score_scale;    /* block-score logit scale; <= 0 selects 1/sqrt(D) */
    float softmax_scale;  /* attention logit scale; <= 0 selects 1/sqrt(D) */
    /* Operating-point and ablation settings (digest, selection section and the sparsity,
     * shape, density and mapping ablations).  All-zero values keep the method as above. */
    float top_k_frac;     /* > 0: Top-k = ceil(top_k_frac * Nb) key blocks for each head
                             (Nb = that head's block count), replacing top_k; Top-k at the
                             pages' 95% sparsity is 0.05.  Range [0, 1] */
    int fixed_shape;      /* > 0: every zone takes this packed shape (lT*16 + lH*4 + lW;
                             each log2 edge in [min_edge_log2, 3], volume 64, 128 or 256)
                             instead of the adaptive one: the fixed-shape baseline */
    float map_exponent;   /* exponent a of the shape mapping b_d ~ g_d^-a (the Lagrange
                             optimum of J is 1/2); <= 0 selects 1/2 */
    int density_mode;     /* information density driving the volume tier: 0 spatial plus
                             temporal terms of rho_raw (the method), 1 spatial term only,
                             2 temporal term only, 3 the normalised A2V intensity a_bar */
    /* Capacity of the selection lists. */
    long long max_pairs;  /* selected (query block, key block) pairs one head may hold in
                             its CSR and CSC lists; 0 = Nb_max^2, which always suffices.
                             A head that selects more keeps a truncated selection, gets
                             PRISM_FLAG_SELECTION_OVERFLOW and NaN outputs. */
} prism_config;

/* Per-head status flags, written on the device by prism_plan (bits 0-1) and prism_attn_bwd
 * (bits 2-3), read with prism_check_flags.  A flagged head's outputs (o and lse for bits
 * 0-1; dq, dk, dv for any bit) are NaN, never silently wrong numbers. */
enum {
    PRISM_FLAG_QKV_RANGE = 1,          /* a q, k or v value outside +-65504, the float16
                                          range of the attention operands (or not finite) */
    PRISM_FLAG_SELECTION_OVERFLOW = 2, /* more selected pairs than max_pairs */
    PRISM_FLAG_DOUT_RANGE = 4,         /* a dout value outside +-65504 (or not finite) */
    PRISM_FLAG_DS_RANGE = 8            /* the bound |dout_x| (max_y |v_y| + |o_x|) on dS =
                                          P (dP - delta) reaches 65504 for some row */
};

/* Offsets (bytes from the workspace base) and element types of the plan's arrays, for
 * inspection.  Nb_max = N / 64; Cap = max_pairs (Nb_max^2 when 0).  Per head h:
 *   zone_stats  double [heads][Z][4]: sigma2_T, sigma2_H, sigma2_W, rho_raw (Z = N / 512)
 *   audio_stats double [Z][4]: zone mean of a, sigma2_T, sigma2_H, sigma2_W
 *   zone_diag   double [heads][Z][4]: rho, tier margin, shape margin, best distance
 *   zone_shape  int32  [heads][Z]: log2 edges packed as lT*16 + lH*4 + lW
 *   zone_block  int32  [heads][Z+1]: first block of each zone; [Z] = block count Nb
 *   block_start int32  [heads][Nb_max]: permuted offset of each block (multiple of 64)
 *   block_size  int32  [heads][Nb_max]: 64, 128 or 256
 *   unit_block  int32  [heads][N/64]: block holding each 64-token unit
 *   perm        int32  [heads][N]: permuted position -> token
 *   inv_perm    int32  [heads][N]: token -> permuted position
 *   qbar, kbar  float  [heads][Nb_max][D]: block means of Q and K
 *   sel_count   int32  [heads][Nb_max]: selected key blocks per query block
 *   csr_ptr     int32  [heads][Nb_max+1]: row i of the CSR starts at csr_ptr[i]
 *   csr_col     int32  [heads][Cap]: row i holds sel_count[i] key blocks, ascending
 *   csc_count, csc_ptr, csc_row: the transpose, in the same form (query blocks selecting
 *                      each key block, ascending)
 *   scores      float  [Nb_max][Nb_max]: block logits of the last head planned
 *   flags       uint32 [heads]: PRISM_FLAG_* bits */
typedef struct prism_layout {
    size_t zone_stats, audio_stats, zone_diag, zone_shape, zone_block, block_start,
        block_size, unit_block, perm, inv_perm, qbar, kbar, sel_count, csr_ptr, csr_col,
        csc_count, csc_ptr, csc_row, scores, flags, total;
    int N, Z, nb_max;
    long long pair_cap;   /* Cap */
} prism_layout;

/* Bytes of workspace a configuration needs (0 if the configuration is rejected). */
size_t prism_workspace_bytes(const prism_config *cfg);

/* Fills *out with the workspace layout of cfg.  PRISM_ERR_ARG / _UNSUPPORTED on a
 * rejected configuration. */
prism_status prism_plan_layout(const prism_config *cfg, prism_layout *out);

/* The same, for a planned workspace: *out holds byte offsets into workspace of the plan's
 * arrays (zone shapes, permutation, block table, CSR and CSC lists, ...), for viewing
 * them.  PRISM_ERR_ARG on a null workspace or output. */
prism_status prism_plan_view(const prism_config *cfg, const void *workspace,
                             prism_layout *out);

/* Plans every head: zone statistics of V and of the A2V norm field, shapes, permutation,
 * permuted copies of Q, K, V, block means, block scores and the Top-k union Top-p
 * selection (steps 1-4 above).  q, k, v: element (token n, head h, channel c) at
 * n * tok_stride + h * head_stride + c, in elements, the same strides for the three (0
 * selects the dense [N][heads][D] value: heads * D, respectively D), so q, k, v may be
 * views into a fused QKV projection; they must be 16-byte aligned and the strides
 * multiples of 16 bytes (PRISM_ERR_ARG otherwise).  a2v_norm: [N] float32, or NULL for a
 * layer with no cached A2V norm (the first layer: video guidance only).  The plan is
 * written into workspace (256-byte aligned, PRISM_ERR_ARG otherwise), which must stay
 * untouched until the last fwd/bwd using it. */
prism_status prism_plan(const prism_config *cfg, const void *q, const void *k, const void *v,
                        int64_t tok_stride, int64_t head_stride, const float *a2v_norm,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Sparse attention forward over the plan in workspace (step 5): o [N][heads][D] in token
 * order, lse [heads][N] float32 (natural-log sum of exp of the scaled logits).  Also keeps
 * a float32 copy of o and the lse in workspace for prism_attn_bwd.  o must be 16-byte
 * aligned, lse 4-byte, workspace 256-byte (PRISM_ERR_ARG otherwise).  PRISM_ERR_STATE,
 * with nothing launched, when no prism_plan with the same configuration has been issued
 * on this workspace (the library records the last plan of each workspace address). */
prism_status prism_attn_fwd(const prism_config *cfg, void *workspace, size_t workspace_bytes,
                            void *o, float *lse, void *stream);

/* The A2V norm field a later layer's prism_plan consumes (digest, guidance section: the
 * audio injection strength of a video position is the vector length of its output of the
 * audio-to-video cross-attention, cached from the previous layer):
 *   a2v_norm[n] = sqrt(sum_c x[n][c]^2), c < channels,
 * x: n_tokens rows of `channels` values in dtype (prism_dtype), row n starting at element
 * n * ld (ld >= channels; x 16-byte aligned and ld * element size a multiple of 16);
 * a2v_norm: [n_tokens] float32 (overwritten).  Sums in float64.  PRISM_ERR_ARG on null
 * pointers or bad sizes, PRISM_ERR_UNSUPPORTED on an unknown dtype. */
prism_status prism_a2v_norm(const void *x, int64_t n_tokens, int channels, int64_t ld,
                            int dtype, float *a2v_norm, void *stream);

/* Sparse attention backward with the plan held constant (digest, training section): given
 * dout [N][heads][D], writes dq, dk, dv [N][heads][D] (overwritten, token order).  Reads
 * the float32 copy of the output and the lse that prism_attn_fwd left in workspace, so
 * prism_attn_fwd must have run on this workspace since the last prism_plan: otherwise the
 * call returns PRISM_ERR_STATE and launches nothing.  dout, dq, dk, dv must be 16-byte
 * aligned, workspace 256-byte (PRISM_ERR_ARG otherwise). */
prism_status prism_attn_bwd(const prism_config *cfg, void *workspace, size_t workspace_bytes,
                            const void *dout, void *dq, void *dk, void *dv, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): prism_plan followed by prism_attn_fwd,
 * with the workspace taken from a static scratch array of 128 MiB that the library holds
 * on each GPU it runs on until the process ends.  Arguments as in prism_plan (q, k, v,
 * strides, a2v_norm) and prism_attn_fwd (o, lse); allocates nothing (no hipMalloc, no
 * allocating library call).  Configurations whose workspace (prism_workspace_bytes)
 * exceeds 128 MiB are refused with PRISM_ERR_WORKSPACE before any launch.  Every call on
 * one GPU shares that GPU's scratch and leaves its plan there: calls that overlap on one
 * GPU (from several threads or streams) race; a prism_attn_bwd cannot follow. */
prism_status prism_forward_static(const prism_config *cfg, const void *q, const void *k,
                                  const void *v, int64_t tok_stride, int64_t head_stride,
                                  const float *a2v_norm, void *o, float *lse, void *stream);

/* Waits for the work queued on stream, then copies the per-head status flags of
 * workspace into flags[heads] (host memory; may be NULL) and returns PRISM_ERR_RANGE if any
 * head has a flag set, PRISM_OK otherwise.  This is the one entry point that synchronises
 * the host; call it after prism_plan or prism_attn_bwd when inputs may leave the float16
 * range or the selection may exceed max_pairs. */
prism_status prism_check_flags(const prism_config *cfg, const void *workspace,
                               uint32_t *flags, void *stream);

/* Per-stage tracing with HIP events (for benchmarks and profiles; off by default).  While
 * enabled, every entry point records a HIP event pair on the caller's stream around the
 * kernel launches of each stage it runs; prism_trace_read waits for the recorded events,
 * writes the summed milliseconds and the number of traced launches per stage into
 * ms[PRISM_STAGE_COUNT] and calls[PRISM_STAGE_COUNT] (either may be NULL) and forgets
 * them.  Enabling or disabling also forgets pending records.  Tracing state is
 * process-wide; the stage names are those of prism_stage_name. */
typedef enum {
    PRISM_STAGE_AUDIO_STATS = 0, /* zone statistics of the A2V norm field */
    PRISM_STAGE_ZONE_STATS,      /* zone statistics of V */
    PRISM_STAGE_QUANTIZE,        /* g_d, tier, shape, block table */
    PRISM_STAGE_GATHER,          /* permutation, permuted Q/K/V, block means */
    PRISM_STAGE_TILES,           /* attention tile list */
    PRISM_STAGE_SCORES,          /* block-score GEMM (per head) */
    PRISM_STAGE_SELECT,          /* Top-k union Top-p, CSR and CSC lists (per head) */
    PRISM_STAGE_ATTN_FWD,        /* sparse attention forward */
    PRISM_STAGE_BWD_PREP,        /* dO gather and rowsum(dO * O) */
    PRISM_STAGE_BWD_DKDV,        /* dK, dV */
    PRISM_STAGE_BWD_DQ,          /* dQ */
    PRISM_STAGE_COUNT
} prism_stage;

prism_status prism_trace_enable(int on);
prism_status prism_trace_read(double *ms, int *calls);
const char *prism_stage_name(int stage);

/* Text of a status code. */
const char *prism_status_string(int status);

/* Message of the last failed call on the calling thread ("" if none). */
const char *prism_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PRISM_H */

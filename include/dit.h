/*
 * dit.h - C ABI of libdit.so: one FLUX.2-[klein]-style diffusion-transformer
 * denoise step on an AMD Instinct MI355X (gfx950), in hand-written HIP.
 *
 * What is computed (sources are the pages this follows):
 *   - "flux2-klein-p100a" model card, Tasks table: each of the 4 sampling
 *     steps is one DiT call (distilled, no CFG); the scheduler stays on the
 *     host (card header). Caveats: all 512 padded text rows enter the DiT
 *     unmasked, as the concatenation of three encoder layers ([512, 7680]);
 *     one modulation result per step serves every block.
 *   - "tt_flux2_klein - Python reference", Modules: the DiT is 5 dual-stream
 *     blocks then 20 single-stream blocks; host maths builds token ids and
 *     RoPE. "Things that are easy to get wrong": one modulation per step
 *     for all blocks, unmasked text rows, RoPE of 32 dims per axis with
 *     theta 2000 on adjacent pairs, reference image i at t = 10 + 10 i.
 *   - Readings where the pages are open (hidden 3072 = 24 heads x 128,
 *     SwiGLU MLP of ratio 3, QK-RMSNorm before RoPE, no biases, AdaLN with
 *     (1 + scale) and shift, gated residuals, RMS pre-norm by default) are
 *     stated at each entry point.
 *
 * Conventions for every entry point:
 *   - Device pointers ("dev") are HIP device memory owned by the caller; the
 *     library borrows them for the stream-ordered duration of the call and
 *     never allocates, frees or keeps them. Host pointers ("host") are read
 *     before the call returns.
 *   - "bf16" buffers hold bfloat16 bit patterns (uint16 per element).
 *   - Matrices are row-major. Weights use the [out_features, in_features]
 *     layout of a linear layer, i.e. y = x W^T.
 *   - A token sequence for one sample is: text rows [0, n_txt), image rows
 *     (row-major over the patch grid), then reference rows. B samples are
 *     stacked: x[B, S, D].
 *   - Every check happens before the first launch: on an error nothing has
 *     been written or enqueued. The return value is DIT_OK (0) or a negative
 *     dit_status; dit_last_error() then holds a message (thread-local).
 *   - Kernels are enqueued on `stream` (a hipStream_t; 0 is the null
 *     stream) and the call returns without synchronising. Launch failures
 *     return DIT_E_HIP; faults inside kernels surface at the caller's next
 *     synchronisation. Calls that share one workspace must not overlap.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dit_stream_t; /* same type as hipStream_t */

typedef enum dit_status {
  DIT_OK = 0,
  DIT_E_NULL = -1,        /* a required pointer is NULL */
  DIT_E_SHAPE = -2,       /* sizes are inconsistent or out of range */
  DIT_E_UNSUPPORTED = -3, /* valid but not implemented (e.g. head_dim != 128) */
  DIT_E_WORKSPACE = -4,   /* workspace too small or misaligned */
  DIT_E_HIP = -5,         /* a HIP launch or runtime call failed */
  DIT_E_VALUE = -6        /* a scalar argument is not finite / out of range */
} dit_status;

enum { DIT_PRENORM_RMS = 0, DIT_PRENORM_LAYER = 1 };

/* Model hyper-parameters. FLUX.2 [klein] 4B values in brackets. */
typedef struct dit_config {
  int32_t hidden;        /* D = heads * head_dim                       [3072] */
  int32_t heads;         /* H                                             [24] */
  int32_t head_dim;      /* d; only 128 is supported                     [128] */
  int32_t mlp_hidden;    /* F, SwiGLU inner width                       [9216] */
  int32_t n_dual;        /* dual-stream blocks                             [5] */
  int32_t n_single;      /* single-stream blocks                          [20] */
  int32_t in_channels;   /* latent token width (2x2 patches)             [128] */
  int32_t txt_channels;  /* prompt embedding width                      [7680] */
  int32_t time_channels; /* sinusoidal timestep features                 [256] */
  int32_t axes_dim[4];   /* RoPE dims per axis (t, h, w, l)     [32,32,32,32] */
  int32_t prenorm;       /* DIT_PRENORM_RMS or DIT_PRENORM_LAYER           [RMS] */
  float theta;           /* RoPE base                                   [2000] */
  float eps;             /* every norm: x / sqrt(mean + eps)            [1e-6] */
} dit_config;

/* One dual-stream block. Index [0] = text stream, [1] = image stream. */
typedef struct dit_dual_weights {
  const void* qkv[2];     /* dev bf16 [3D, D]: q rows, k rows, v rows; head j
                             is rows 128j..128j+127 of each third           */
  const void* out[2];     /* dev bf16 [D, D]                                 */
  const void* mlp_in[2];  /* dev bf16 [2F, D]: gate rows, then up rows       */
  const void* mlp_out[2]; /* dev bf16 [D, F]                                 */
  const float* q_gain[2]; /* dev fp32 [head_dim] QK-RMSNorm gains            */
  const float* k_gain[2];
} dit_dual_weights;

/* One single-stream block. */
typedef struct dit_single_weights {
  const void* w_in;     /* dev bf16 [3D + 2F, D] = [Wq; Wk; Wv; Wgate; Wup] */
  const void* w_out;    /* dev bf16 [D, D + F]; input = [attention | SwiGLU] */
  const float* q_gain;  /* dev fp32 [head_dim] */
  const float* k_gain;
} dit_single_weights;

/* Whole model. */
typedef struct dit_model_weights {
  const void* t_in;          /* dev bf16 [D, time_channels] */
  const void* t_out;         /* dev bf16 [D, D] */
  const void* mod_dual_img;  /* dev bf16 [6D, D] */
  const void* mod_dual_txt;  /* dev bf16 [6D, D] */
  const void* mod_single;    /* dev bf16 [3D, D] */
  const void* mod_final;     /* dev bf16 [2D, D] */
  const void* x_embed;       /* dev bf16 [D, in_channels] */
  const void* ctx_embed;     /* dev bf16 [D, txt_channels] */
  const void* proj_out;      /* dev bf16 [in_channels, D] */
  const dit_dual_weights* dual;     /* host array [n_dual] */
  const dit_single_weights* single; /* host array [n_single] */
} dit_model_weights;

/* Rows of the per-step modulation buffer mod[B, 17, D] (fp32):
 *   [0, 6)   dual image stream: shift1, scale1, gate1, shift2, scale2, gate2
 *   [6, 12)  dual text stream: same order
 *   [12, 15) single blocks: shift, scale, gate
 *   [15, 17) final layer: shift, scale                                      */
enum { DIT_MOD_DUAL_IMG = 0, DIT_MOD_DUAL_TXT = 6, DIT_MOD_SINGLE = 12,
       DIT_MOD_FINAL = 15, DIT_MOD_ROWS = 17 };

/* Workspace kinds for dit_workspace_bytes. */
enum { DIT_WS_DUAL = 0, DIT_WS_SINGLE = 1, DIT_WS_STEP = 2, DIT_WS_MOD = 3,
       DIT_WS_DENOISE = 4 };

/* Largest batch a call accepts (sigma values travel as kernel arguments). */
enum { DIT_MAX_BATCH = 64 };

/* Largest number of steps of one dit_denoise_forward call. */
enum { DIT_MAX_STEPS = 64 };

/* ------------------------------------------------------------------ host */

/* Token ids (t, h, w, l) of one sample into out[cap_rows][4] (host int32).
 * "tt_flux2_klein - Python reference", Modules (host.py: token ids) and
 * "Things that are easy to get wrong" (reference i at t = 10 + 10 i).
 * Reading: text row l -> (0, 0, 0, l); image patch (r, c) of the hp x wp
 * grid, row-major -> (0, r, c, 0); reference i (0-based) patch (r, c) of its
 * ref_hp[i] x ref_wp[i] grid -> (10 + 10 i, r, c, 0). n_ref <= 3 ("flux2-
 * klein-p100a", Tasks table: 1-3 reference images).
 * Returns the row count S (>= 0) or a negative dit_status
 * (DIT_E_SHAPE if S > cap_rows or a size is negative). */
int64_t dit_position_ids(int64_t n_txt, int32_t hp, int32_t wp, int32_t n_ref,
                         const int32_t* ref_hp, const int32_t* ref_wp,
                         int32_t* out, int64_t cap_rows);

/* Bytes of device workspace a call needs (0 on invalid arguments, with
 * dit_last_error set). kind: DIT_WS_DUAL / DIT_WS_SINGLE for one block call
 * on B samples of S tokens, DIT_WS_STEP for dit_step_forward (S = n_txt +
 * n_img + n_ref), DIT_WS_MOD for dit_modulation_forward, DIT_WS_DENOISE
 * for dit_denoise_forward (S = n_txt + n_img + n_ref). */
size_t dit_workspace_bytes(const dit_config* cfg, int32_t kind, int32_t B, int64_t S);

const char* dit_status_string(int status);
const char* dit_last_error(void);

/* Validates a configuration; DIT_OK or a negative status. */
int dit_config_check(const dit_config* cfg);

/* ---------------------------------------------------------------- device */

/* RoPE tables for S tokens: cos_dev/sin_dev fp32 [S, head_dim/2], one entry
 * per adjacent pair. Pair j of axis a (head dims 32a + 2j, 32a + 2j + 1)
 * turns by pos[s][a] * theta^(-2j / axes_dim[a]) ("tt_flux2_klein - Python
 * reference", Things that are easy to get wrong: 32 dims per axis, theta
 * 2000, adjacent pairs). Angles and their cos/sin are evaluated in double
 * precision and rounded to fp32. pos_dev: dev int32 [S, 4] (t, h, w, l).
 * Tables depend only on the positions, so one build serves every block,
 * every step and every batch row of that shape. */
int dit_rope_tables_build(const dit_config* cfg, const int32_t* pos_dev, int64_t S,
                          float* cos_dev, float* sin_dev, dit_stream_t stream);

/* Global AdaLN modulation for one step ("flux2-klein-p100a", Caveats, and
 * "tt_flux2_klein - Python reference", Things that are easy to get wrong:
 * computed once per step, shared by every block).
 * Reading: tau = 1000 sigma; e = [cos(tau f_k) | sin(tau f_k)],
 * f_k = 10000^(-k / (time_channels/2)); m = SiLU(W_t_out SiLU(W_t_in e));
 * mod[b] = [W_mod_dual_img m; W_mod_dual_txt m; W_mod_single m;
 * W_mod_final m] -> mod_dev fp32 [B, 17, D] (row order above).
 * sigma_host: host fp32 [B], finite; 1 <= B <= DIT_MAX_BATCH.
 * ws: dev workspace of dit_workspace_bytes(cfg, DIT_WS_MOD, B, 0) bytes. */
int dit_modulation_forward(const dit_config* cfg, const dit_model_weights* w,
                           const float* sigma_host, int32_t B, float* mod_dev,
                           void* ws, size_t ws_bytes, dit_stream_t stream);

/* dit_modulation_forward without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * and harnesses that forbid allocation). The intermediate vectors live in a
 * fixed device array inside the library of DIT_NOALLOC_SCRATCH_BYTES (3 MiB
 * and 768 bytes: DIT_MAX_BATCH rows at time_channels and hidden up to 4096),
 * which each GPU the library runs on holds until the process ends; its
 * address is looked up on the first call on each device (the current device
 * is the one the stream belongs to). The call allocates nothing. Every call
 * on one GPU shares that array and leaves its last contents there (every
 * value is written before it is read, so nothing needs clearing): calls that
 * overlap on one GPU (different streams, or threads) race and must be
 * serialised by the caller. Returns DIT_E_UNSUPPORTED if B rows of this
 * configuration need more scratch than the array holds; other arguments and
 * results as for dit_modulation_forward. */
enum { DIT_NOALLOC_SCRATCH_BYTES = 64 * (4096 + 2 * 4096) * 4 + 3 * 256 };
int dit_modulation_forward_noalloc(const dit_config* cfg, const dit_model_weights* w,
                                   const float* sigma_host, int32_t B, float* mod_dev,
                                   dit_stream_t stream);

/* One dual-stream block, in place on x ("tt_flux2_klein - Python reference",
 * Modules: the first 5 blocks). x: dev fp32 [B, S, D]. Text rows [0, n_txt)
 * use stream-0 weights and mod_txt; image+reference rows [n_txt, S) use
 * stream-1 weights and mod_img; mod_txt / mod_img point at six D-vectors
 * (shift1, scale1, gate1, shift2, scale2, gate2) of batch row 0, and
 * mod_batch_stride floats separate batch rows (17 D inside the step's
 * modulation buffer). Per stream s:
 *   h = N(x) (1 + scale1) + shift1;  [q|k|v] = h Wqkv_s^T;
 *   q, k per head <- RoPE(RMSNorm(.) * gain_s); joint attention of both
 *   streams over all S rows, no mask; x += gate1 * (o Wout_s^T);
 *   h2 = N(x) (1 + scale2) + shift2; a = SiLU(h2 Wg^T) * (h2 Wu^T);
 *   x += gate2 * (a Wmlp_out_s^T).
 * cos/sin: tables from dit_rope_tables_build for these S positions.
 * ws: dit_workspace_bytes(cfg, DIT_WS_DUAL, B, S) bytes, 256-byte aligned. */
int dit_dual_block_forward(const dit_config* cfg, const dit_dual_weights* w, float* x,
                           int32_t B, int64_t S, int64_t n_txt,
                           const float* mod_txt, const float* mod_img,
                           int64_t mod_batch_stride, const float* cos_dev,
                           const float* sin_dev, void* ws, size_t ws_bytes,
                           dit_stream_t stream);

/* One single-stream block, in place on x ("tt_flux2_klein - Python
 * reference", Modules: the last 20 blocks). mod: shift, scale, gate (three
 * D-vectors of batch row 0; mod_batch_stride floats between batch rows).
 *   h = N(x) (1 + scale) + shift; u = h W_in^T;
 *   q, k, v = u[:, :3D] with QK-RMSNorm + RoPE; o = attention (no mask);
 *   a = SiLU(u_gate) * u_up; x += gate * ([o | a] W_out^T).
 * ws: dit_workspace_bytes(cfg, DIT_WS_SINGLE, B, S) bytes, 256-byte aligned. */
int dit_single_block_forward(const dit_config* cfg, const dit_single_weights* w,
                             float* x, int32_t B, int64_t S, const float* mod,
                             int64_t mod_batch_stride, const float* cos_dev,
                             const float* sin_dev, void* ws, size_t ws_bytes,
                             dit_stream_t stream);

/* One denoise step ("flux2-klein-p100a", Tasks table: one DiT call per
 * step): global modulation from sigma, embeddings, n_dual dual-stream
 * blocks, n_single single-stream blocks, final AdaLN + projection of the
 * image rows.
 *   txt: dev bf16 [B, n_txt, txt_channels] prompt embedding (the pages'
 *        [512, 7680], all rows, unmasked);
 *   latents: dev bf16 [B, n_img + n_ref, in_channels] image tokens then
 *        reference tokens (2x2-patchified latents);
 *   sigma_host: host fp32 [B];
 *   cos/sin: tables for the S = n_txt + n_img + n_ref positions;
 *   v_out: dev fp32 [B, n_img, in_channels] velocity of the image tokens
 *        (text and reference rows are dropped).
 * ws: dit_workspace_bytes(cfg, DIT_WS_STEP, B, S) bytes, 256-byte aligned. */
int dit_step_forward(const dit_config* cfg, const dit_model_weights* w,
                     const void* txt, const void* latents, const float* sigma_host,
                     int32_t B, int64_t n_txt, int64_t n_img, int64_t n_ref,
                     const float* cos_dev, const float* sin_dev, float* v_out,
                     void* ws, size_t ws_bytes, dit_stream_t stream);

/* The sampling loop on the device: n_steps denoise steps with the flow-
 * matching Euler update between them ("flux2-klein-p100a", Tasks table:
 * 4 steps, one DiT call each, no CFG; the card's header puts the scheduler
 * on the host, so the sigma schedule is an input here). For i < n_steps and
 * every batch row b:
 *   v = dit_step(txt, [bf16(z) ; ref], sigma[b][i]);
 *   z += (sigma[b][i + 1] - sigma[b][i]) * v        (fp32, one fma).
 *   z: dev fp32 [B, n_img, in_channels], in place: the starting latent (the
 *      noise) in, the latent after the last update out;
 *   ref: dev bf16 [B, n_ref, in_channels] reference tokens (never updated;
 *      NULL when n_ref = 0);
 *   sigmas_host: host fp32 [B, n_steps + 1], finite; 1 <= n_steps <=
 *      DIT_MAX_STEPS;
 *   txt, cos/sin, B, n_txt, n_img, n_ref: as for dit_step_forward.
 * The step's latent operand is bf16(z) (the GEMM rounds its operands). The
 * modulation vectors of up to four steps come from one pass over the
 * modulation weights (each step's still depends on its own sigma only), and
 * the text rows' embedding, which depends on the prompt only, is computed by
 * the first step and reused by the others.
 * The sigmas travel as kernel arguments, so the enqueued work for one shape
 * and schedule can be captured once in a HIP graph and replayed.
 * ws: dit_workspace_bytes(cfg, DIT_WS_DENOISE, B, S) bytes, 256-byte aligned. */
int dit_denoise_forward(const dit_config* cfg, const dit_model_weights* w,
                        const void* txt, float* z, const void* ref,
                        const float* sigmas_host, int32_t n_steps, int32_t B,
                        int64_t n_txt, int64_t n_img, int64_t n_ref,
                        const float* cos_dev, const float* sin_dev, void* ws,
                        size_t ws_bytes, dit_stream_t stream);

/* One bias-free linear layer, y = a w^T, through the GEMM every projection of
 * the step uses (the input embeddings, each block's projections and the
 * final projection of "tt_flux2_klein - Python reference", Modules), with its
 * fp32 output epilogue and no K chunking.
 *   a: dev bf16 [M, K] row-major; w: dev bf16 [N, K] row-major (a layer's
 *   weight as stored: out_features rows); y: dev fp32 [M, N] row-major,
 *   overwritten; a, w, y 16-byte aligned and y not overlapping a or w.
 *   0 <= M < 2^31; N a positive multiple of 4; K a positive multiple of 64;
 *   M K and N K bf16 elements each addressable with 32-bit byte offsets.
 * Products are accumulated in fp32 over k in increasing 16-deep steps; the
 * tile shape the planner picks for M, N and K (256- or 384-row tiles,
 * 224- or 256-column tiles) never changes an element's result, so a row
 * of y depends on its row of a only. Returns DIT_E_NULL / DIT_E_SHAPE /
 * DIT_E_UNSUPPORTED (sizes) or DIT_E_VALUE (y overlaps a or w) before any
 * launch, DIT_E_HIP if the launch fails; M = 0 launches nothing and
 * accepts NULL pointers. */
int dit_linear_forward(const void* a, const void* w, float* y, int64_t M, int32_t N,
                       int32_t K, dit_stream_t stream);

/* ------------------------------------------------------------- profiling */

/* Kernel families, for dit_kernel_stats.kind. */
enum { DIT_K_GEMM = 0, DIT_K_ATTENTION = 1, DIT_K_MODNORM = 2, DIT_K_QKV_PAD = 3,
       DIT_K_GEMV = 4, DIT_K_ROPE_TABLES = 5, DIT_K_TIME = 6, DIT_K_SPLIT_SUM = 7,
       DIT_K_LATENT = 8, DIT_K_ATTN_GEMM = 9 /* attention fused with GEMM tiles */,
       /* latent decoder (dit_vae.h) */
       DIT_K_CONV = 10 /* implicit-GEMM conv and the attention products */,
       DIT_K_GROUPNORM = 11, DIT_K_SOFTMAX = 12, DIT_K_LATENT_IMAGE = 13,
       DIT_K_CONV_HALO = 14 /* halo-tiled 3x3 conv */, DIT_K_COUNT = 15 };

typedef struct dit_kernel_stats {
  int32_t kind;     /* DIT_K_* */
  int32_t launches; /* launches recorded */
  double total_ms;  /* sum of per-launch durations (HIP events on the launch stream) */
  double flops;     /* algorithmic FLOPs of those launches (2 M N K per GEMM,
                       4 S^2 d per attention head) */
  double bytes;     /* algorithmic HBM bytes (each operand read once, each
                       result written once) */
} dit_kernel_stats;

/* Measurement helper (not on the compute path's contract). Between
 * dit_profile_begin() and dit_profile_end(), every kernel the library
 * launches (from any thread) is bracketed by a pair of HIP events on its
 * stream. dit_profile_end waits for the recorded work, writes DIT_K_COUNT
 * entries into out (host memory, caller-owned) and stops recording.
 * Recording adds event overhead; time headline numbers without it.
 * Returns DIT_OK, DIT_E_NULL, DIT_E_VALUE (end without begin) or DIT_E_HIP. */
int dit_profile_begin(void);
int dit_profile_end(dit_kernel_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
